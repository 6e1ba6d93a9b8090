// Compressed-key scores for any head_dim through byte tables in LDS (gfx950,
// wave64): the route for key codebooks of up to 3 index planes outside the
// head_dim-128 MFMA kernel: Haar rotations at other head dims, the parts of
// a split head vector (with its channel map), other power-of-two dims.
// Same formula as the one-token-per-thread kernel it replaces there (page
// "bitpolar 0.3.3 src/kv_cache.rs", KvCacheCompressor::attention_scores: the
// score from the packed codes without decoding; "turboquant-plus-rs 0.1.0
// README", Architecture steps 1-2):
//   s = scale * ((n/d) sum_j qt_j c[idx_j] + sqrt(pi/2)/m gamma sum_i p_i (2 s_i - 1)),
// qt the rotated query, p = S qt / sqrt(d).
//
// The MSE sum without per-coordinate work: with the index bits v_p of a
// coordinate and any codebook c of L = 2^k levels, the expansion over plane
// subsets P, a_P = (1/L) sum_v c_v (-1)^popc(~v & P), gives
//   sum_j qt_j c[idx_j] = sum_P a_P (-1)^|P| (sum_j qt_j - 2 M_P),
// M_P = sum_j qt_j x_Pj, x_P the XOR of the planes in P (M_{} = 0).  Each
// M_P, and the sign sum sum_i p_i s_i, is a sum of byte-table entries
// T[pos][byte] = sum of the values whose bits the byte sets, over the bytes
// of the mask words.
//
// One workgroup (8 waves) per (b, kv head, chunk of tokens):
//   * the chunk's records go to LDS once (consecutive threads, consecutive
//     words), rows padded to an odd word count;
//   * the query side of up to 4 query heads of the kv head at once, so that R
//     and S are read once per batch: qt (Walsh-Hadamard in LDS, or R q on the
//     matrix cores), p (S qt on the matrix cores), their sums;
//   * per head: the two byte tables, then one token per thread.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

using namespace mf;

constexpr int kLBlock = 512;             // 8 waves
constexpr int kHB = 4;                   // query heads whose query side is built together
constexpr int kU = 8;                    // loads in flight per thread when staging
constexpr size_t kLutLdsMax = 150 * 1024;

struct LutArgs {
  CodebookArgs cb;
  const uint32_t* krec;
  int64_t B, Hkv, T, Hq;
  const void* q;
  int q_dtype;
  int64_t q_row;
  float scale;
  float* scores;
  int32_t* status;
  ChannelMap cm;
  int accumulate;
  int tch;              // tokens per workgroup
  int rwp;              // LDS words per staged record (odd)
  int64_t chunks;       // workgroups per (b, kv head)
};

// Dynamic LDS (bytes): records [tch][rwp] | q table [4W][256] | p table [4Ws][256]
// | nibble sums [4(W + Ws)][2][16] | qt [kHB][32W] | p [kHB][32Ws] | raw queries [kHB][d].
struct LutLds {
  size_t rec, lq, lp, nib, qt, pp, qraw, total;
};

__host__ __device__ inline LutLds lut_lds(int tch, int rwp, int W, int Ws, int d) {
  LutLds o;
  o.rec = 0;
  o.lq = o.rec + (size_t)tch * rwp * 4;
  o.lp = o.lq + (size_t)4 * W * 256 * 4;
  o.nib = o.lp + (size_t)4 * Ws * 256 * 4;
  o.qt = o.nib + (size_t)4 * (W + Ws) * 32 * 4;
  o.pp = o.qt + (size_t)kHB * 32 * W * 4;
  o.qraw = o.pp + (size_t)kHB * 32 * Ws * 4;
  o.total = o.qraw + (size_t)kHB * d * 4;
  return o;
}

// Three bfloat16 terms of 8 float32 values (t0 + t1 + t2 = x exactly: each
// term takes the top 8 significant bits of what remains), packed two per word.
__device__ inline void split3_bf16(const float (&x)[8], u32x4 (&t)[3]) {
  uint32_t w[3][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float r0 = x[2 * q], r1 = x[2 * q + 1];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const uint32_t h0 = __float_as_uint(r0) & 0xFFFF0000u, h1 = __float_as_uint(r1) & 0xFFFF0000u;
      w[p][q] = (h0 >> 16) | h1;
      r0 -= __uint_as_float(h0);
      r1 -= __uint_as_float(h1);
    }
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) t[p] = u32x4{w[p][0], w[p][1], w[p][2], w[p][3]};
}

// sum of the four byte-table entries of a 32-bit mask word at byte positions 4w..4w+3
__device__ inline float table_word(const float* t, int w, uint32_t mw) {
  const float* tw = t + (size_t)w * 1024;
  return (tw[mw & 255u] + tw[256 + ((mw >> 8) & 255u)]) + (tw[512 + ((mw >> 16) & 255u)] + tw[768 + (mw >> 24)]);
}

template <int K>
__global__ __launch_bounds__(kLBlock) void scores_lut_kernel(LutArgs a) {
  constexpr int L = 1 << K;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float sa[L];            // a_P (-1)^|P|
  __shared__ float hsum[kHB][2];     // per head: sum_j qt_j, sum_i p_i
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.cb.d, m = a.cb.m, W = a.cb.plane_words, Ws = a.cb.sign_words, RW = a.cb.rec_words;
  const int dq = 32 * W, mq = 32 * Ws;
  const int64_t g = blockIdx.x / a.chunks, chunk = blockIdx.x % a.chunks;
  const int64_t b = g / a.Hkv, h = g % a.Hkv;
  const int gq = (int)(a.Hq / a.Hkv);
  const LutLds lay = lut_lds(a.tch, a.rwp, W, Ws, d);
  uint32_t* rec = reinterpret_cast<uint32_t*>(smem + lay.rec);
  float* lq = reinterpret_cast<float*>(smem + lay.lq);
  float* lp = reinterpret_cast<float*>(smem + lay.lp);
  float* nib = reinterpret_cast<float*>(smem + lay.nib);
  float* qt = reinterpret_cast<float*>(smem + lay.qt);
  float* pp = reinterpret_cast<float*>(smem + lay.pp);
  float* qraw = reinterpret_cast<float*>(smem + lay.qraw);
  const uint8_t* blob = blob_of(a.cb, g);
  if (tid == 0 && a.status && blob_mismatch(a.cb, blob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  const int64_t t0 = chunk * a.tch;
  const int nt = (int)(a.T - t0 < a.tch ? a.T - t0 : a.tch);

  // the chunk's records: consecutive threads load consecutive words
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.krec + g * a.T * RW), 0, (int)(a.T * RW * 4), kRsrcWord3);
  // (kU loads in flight per thread: a load and its LDS write one at a time would
  // wait a memory round trip per word)
  for (int e0 = tid; e0 < nt * RW; e0 += kU * kLBlock) {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = e0 + u * kLBlock;
      v[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, e < nt * RW ? (uint32_t)((t0 * RW + e) * 4) : 0xC0000000u, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = e0 + u * kLBlock;
      if (e < nt * RW) {
        const int tok = e / RW, w = e - tok * RW;
        rec[tok * a.rwp + w] = v[u];
      }
    }
  }
  if (tid < L) {
    const float* cent = reinterpret_cast<const float*>(blob + a.cb.off_c);
    double acc = 0.0;
    for (int v = 0; v < L; ++v) acc += (__popc(~v & tid) & 1) ? -(double)cent[v] : (double)cent[v];
    sa[tid] = (float)((__popc(tid) & 1) ? -acc / L : acc / L);
  }

  const bool haar = a.cb.rotation == kRotHaar;
  const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d);
  const float* R = reinterpret_cast<const float*>(blob + a.cb.off_d);
  const _Float16* S = reinterpret_cast<const _Float16*>(blob + a.cb.off_s);
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  // vout[hh][r] = scale sum_i M[r][i] vin[hh][i] for the rows r < nrows of a
  // row-major [nrows][d] matrix M (binary16 or float32), zero for nrows <= r <
  // ostride (a multiple of 32), on v_mfma_f32_32x32x16_bf16: rows are the M
  // side (32 per tile, a tile per wave), the heads of the batch the N side.
  // Both operands are split into three bfloat16 terms (24 significant bits
  // and the float32 exponent range; binary16 entries need two), and the
  // products of terms down to about 2^-20 of the sum are kept.  Row pieces of
  // 8 entries are 16-byte buffer loads when d is a multiple of 8 (then no
  // piece crosses a row or the end), else single entries.  Ends with a barrier.
  int nh = 0;
  const auto mfma_matvec = [&](auto f16_tag, const void* mat, int nrows, float scale, const float* vin, int istride,
                               float* vout, int ostride) {
    constexpr bool F16 = decltype(f16_tag)::value;
    constexpr int NT = F16 ? 2 : 3;                   // bfloat16 terms of a matrix entry
    const __amdgpu_buffer_rsrc_t ms = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(mat), 0, (int)((int64_t)nrows * d * (F16 ? 2 : 4)), kRsrcWord3);
    const bool pieces = (d & 7) == 0;
    const int nkc = (d + 15) / 16, hcol = lane & 31, hk = lane >> 5;
    for (int M = wave; M < ostride / 32; M += kLBlock / 64) {
      const int row = 32 * M + hcol;
      f32x16 acc = {};
#pragma unroll 8
      for (int c = 0; c < nkc; ++c) {
        const int k0 = 16 * c + 8 * hk;
        float av[8], bv[8];
        const bool rok = row < nrows && k0 < d;
        if (pieces) {
          const uint32_t off = rok ? (uint32_t)(((int64_t)row * d + k0) * (F16 ? 2 : 4)) : 0xC0000000u;
          if constexpr (F16) {
            const uint4 w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ms, off, 0, 0));
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              av[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)((ww[e >> 1] >> (16 * (e & 1))) & 0xFFFFu));
          } else {
            const uint4 w0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ms, off, 0, 0));
            const uint4 w1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ms, off + 16u, 0, 0));
            const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) av[e] = __uint_as_float(ww[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool ok = row < nrows && k0 + e < d;
            const uint32_t off = ok ? (uint32_t)(((int64_t)row * d + k0 + e) * (F16 ? 2 : 4)) : 0xC0000000u;
            if constexpr (F16)
              av[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(ms, off, 0, 0));
            else
              av[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ms, off, 0, 0));
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (k0 + e >= d) av[e] = 0.0f;
          bv[e] = hcol < nh && k0 + e < d ? vin[hcol * istride + k0 + e] : 0.0f;
        }
        u32x4 at[3], bt[3];
        split3_bf16(av, at);
        split3_bf16(bv, bt);
        // term pairs (i, j) with i + j <= 2
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(at[0]), as<bf16x8>(bt[0]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(at[0]), as<bf16x8>(bt[1]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(at[1]), as<bf16x8>(bt[0]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(at[0]), as<bf16x8>(bt[2]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(at[1]), as<bf16x8>(bt[1]), acc, 0, 0, 0);
        if constexpr (NT == 3)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(at[2]), as<bf16x8>(bt[0]), acc, 0, 0, 0);
      }
      // register k of lane half hk holds row 32M + 8(k >> 2) + 4hk + (k & 3), column (head) hcol
      if (hcol < nh) {
#pragma unroll
        for (int k = 0; k < 16; ++k) vout[hcol * ostride + 32 * M + 8 * (k >> 2) + 4 * hk + (k & 3)] = acc[k] * scale;
      }
    }
    __syncthreads();
  };
  for (int hb = 0; hb < gq; hb += kHB) {
    nh = gq - hb < kHB ? gq - hb : kHB;
    __syncthreads();                                  // the previous batch's vectors and tables are read
    // raw queries through the channel map (Walsh-Hadamard: with the signs of D)
    for (int e = tid; e < nh * d; e += kLBlock) {
      const int hh = e / d, j = e - hh * d;
      const int64_t hq = h * gq + hb + hh;
      float v = load_elem(a.q, a.q_dtype, (b * a.Hq + hq) * a.q_row + a.cm.channel(g, j, a.status));
      if (!haar && ((dbits[j >> 5] >> (j & 31)) & 1u)) v = -v;
      qraw[hh * d + j] = v;
    }
    __syncthreads();
    if (haar) {
      // qt = R q, R streamed through LDS in row tiles (zero past d)
      mfma_matvec(std::false_type{}, R, d, 1.0f, qraw, d, qt, dq);
    } else {
      // qt = H (D q): butterflies in LDS (d a power of two), zero past d
      for (int e = tid; e < nh * dq; e += kLBlock) {
        const int hh = e / dq, j = e - hh * dq;
        qt[e] = j < d ? qraw[hh * d + j] : 0.0f;
      }
      __syncthreads();
      for (int hs = 1; hs < d; hs <<= 1) {
        for (int e = tid; e < nh * (d / 2); e += kLBlock) {
          const int hh = e / (d / 2), pr = e - hh * (d / 2);
          const int i = (pr / hs) * 2 * hs + (pr % hs);
          float* row = qt + hh * dq;
          const float x0 = row[i], x1 = row[i + hs];
          row[i] = x0 + x1;
          row[i + hs] = x0 - x1;
        }
        __syncthreads();
      }
    }
    __syncthreads();
    // p = S qt / sqrt(d), S streamed through LDS in row tiles (zero past m)
    mfma_matvec(std::true_type{}, S, m, inv_sqrt_d, qt, dq, pp, mq);
    __syncthreads();
    if (wave < nh) {
      float s1 = 0.0f, s2 = 0.0f;
      for (int j = lane; j < d; j += 64) s1 += qt[wave * dq + j];
      for (int i = lane; i < m; i += 64) s2 += pp[wave * mq + i];
      s1 = wave_sum_f32(s1);
      s2 = wave_sum_f32(s2);
      if (lane == 0) {
        hsum[wave][0] = s1;
        hsum[wave][1] = s2;
      }
    }
    for (int hh = 0; hh < nh; ++hh) {
      __syncthreads();                                // sums visible; the previous head's tables are read
      // byte tables: entry (pos, v) = sum of the values 8 pos + b whose bit b is
      // set in v; first the sums over each nibble value of each half-byte
      // (positions of qt, then of p), then one add per entry
      for (int e = tid; e < 4 * (W + Ws) * 32; e += kLBlock) {
        const int pos = e >> 5, half = (e >> 4) & 1, v = e & 15;
        const float* src = (pos < 4 * W ? qt + hh * dq + 8 * pos : pp + hh * mq + 8 * (pos - 4 * W)) + 4 * half;
        float sum = 0.0f;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) sum += ((v >> bb) & 1) ? src[bb] : 0.0f;
        nib[e] = sum;
      }
      __syncthreads();
      for (int e = tid; e < 4 * (W + Ws) * 256; e += kLBlock) {
        const int pos = e >> 8, v = e & 255;
        lq[e] = nib[pos * 32 + (v & 15)] + nib[pos * 32 + 16 + (v >> 4)];   // lp follows lq in LDS
      }
      __syncthreads();
      const float sq = hsum[hh][0], sp = hsum[hh][1];
      float c0 = 0.0f, fp[L];
#pragma unroll
      for (int P = 0; P < L; ++P) {
        c0 += sa[P];                                  // the sum_j qt_j terms of every subset
        fp[P] = -2.0f * sa[P];
      }
      const int64_t hq = h * gq + hb + hh;
      float* out = a.scores + (b * a.Hq + hq) * a.T + t0;
      for (int tl = tid; tl < nt; tl += kLBlock) {
        const uint32_t* r = rec + tl * a.rwp;
        float mp[L];
#pragma unroll
        for (int P = 0; P < L; ++P) mp[P] = 0.0f;
        for (int w = 0; w < W; ++w) {
          uint32_t pl[K];
#pragma unroll
          for (int p = 0; p < K; ++p) pl[p] = r[p * W + w];
#pragma unroll
          for (int P = 1; P < L; ++P) {
            uint32_t mw = 0;
#pragma unroll
            for (int p = 0; p < K; ++p)
              if ((P >> p) & 1) mw ^= pl[p];
            mp[P] += table_word(lq, w, mw);
          }
        }
        float mse = c0 * sq;
#pragma unroll
        for (int P = 1; P < L; ++P) mse = fmaf(fp[P], mp[P], mse);
        float ps = 0.0f;
        for (int w = 0; w < Ws; ++w) ps += table_word(lp, w, r[K * W + w]);
        const float qjl = 2.0f * ps - sp;
        const float n = __uint_as_float(r[K * W + Ws]);
        const float gam = __uint_as_float(r[K * W + Ws + 1]);
        const float s = (n / (float)d) * mse + (kQjlConst / (float)m) * gam * qjl;
        out[tl] = a.accumulate ? out[tl] + a.scale * s : a.scale * s;
      }
    }
  }
}

template <int K>
int launch_k(const LutArgs& a, size_t lds, hipStream_t s) {
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&scores_lut_kernel<K>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLutLdsMax) != hipSuccess)
      return -10;
    attr_set = true;
  }
  hipLaunchKernelGGL(scores_lut_kernel<K>, dim3((unsigned)(a.B * a.Hkv * a.chunks)), dim3(kLBlock), lds, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

// Tokens per workgroup: 512 (one per thread) while the tables and records fit,
// fewer for wide records or tables; 0 when not even 64 tokens fit.
int lut_tokens(const CodebookArgs& cb) {
  const int rwp = cb.rec_words | 1;
  for (int tch = 512; tch >= 64; tch >>= 1)
    if (lut_lds(tch, rwp, cb.plane_words, cb.sign_words, cb.d).total <= kLutLdsMax) return tch;
  return 0;
}

}  // namespace

bool lut_scores_supported(const CodebookArgs& cb, int64_t T) {
  if (cb.role != TQ_ROLE_KEY || cb.k < 1 || cb.k > 3 || cb.m < 1) return false;
  if (cb.rotation != kRotHaar && (cb.d & (cb.d - 1))) return false;
  if (T * cb.rec_words * 4 >= (int64_t(1) << 31)) return false;   // 32-bit buffer offsets per group
  return lut_tokens(cb) > 0;
}

int launch_scores_lut(const CodebookArgs& cb, const uint32_t* krec, int64_t B, int64_t Hkv, int64_t T,
                      const void* q, int q_dtype, int64_t Hq, float scale, float* scores, int32_t* status,
                      hipStream_t s, int64_t q_row, const ChannelMap& cm, bool accumulate) {
  if (B * Hq * T == 0) return 0;
  LutArgs a;
  a.cb = cb;
  a.krec = krec;
  a.B = B; a.Hkv = Hkv; a.T = T; a.Hq = Hq;
  a.q = q; a.q_dtype = q_dtype; a.q_row = q_row > 0 ? q_row : cb.d;
  a.scale = scale;
  a.scores = scores;
  a.status = status;
  a.cm = cm;
  a.accumulate = accumulate ? 1 : 0;
  a.tch = lut_tokens(cb);
  a.rwp = cb.rec_words | 1;
  a.chunks = (T + a.tch - 1) / a.tch;
  const size_t lds = lut_lds(a.tch, a.rwp, cb.plane_words, cb.sign_words, cb.d).total;
  switch (cb.k) {
    case 1: return launch_k<1>(a, lds, s);
    case 2: return launch_k<2>(a, lds, s);
    case 3: return launch_k<3>(a, lds, s);
  }
  return TQ_ERR_UNSUPPORTED;
}

}  // namespace tq
