// Attention output over compressed keys and values for one decode step, split
// over the token axis (page "bitpolar 0.3.3 src/kv_cache.rs",
// attention_scores: pre-softmax scores q.k/sqrt(d); the weighted sum of
// decoded values follows the page's decode_values).
//
// x^_t = (n_t/d) D H c[idx_t], so sum_t w_t x^_t = (1/d) D H (sum_t w_t n_t c[idx_t]):
// the weighted sum is accumulated in the rotated domain and transformed once.
//
// Stage 1 (one workgroup per (b, hq, chunk of tokens)): chunk max m_c of the
//   scores, l_c = sum_t exp(s_t - m_c), a_c[j] = sum_t exp(s_t - m_c) n_t c[idx_tj].
// Stage 2 (one workgroup per (b, hq)): m = max_c m_c, l = sum_c l_c e^(m_c - m),
//   a = sum_c a_c e^(m_c - m), o = D H a / (d l)  (o = 0 when T = 0).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_score_core.h"

namespace tq {
namespace {

constexpr int kBlock = 256;
constexpr int64_t kChunk = 1024;

struct PartArgs {
  CodebookArgs vcb;
  const uint32_t* vrec;
  const float* scores;   // [B][Hq][T]
  int64_t Hkv, T, Hq, chunks;
  float* part;           // [B*Hq][chunks][d + 2]: a[0..d), m, l
};

// Lanes per token = d/8: lane `sub` of a token owns coordinates 8 sub .. 8 sub + 7,
// i.e. one byte of each bit-plane word.
template <int K>
__global__ __launch_bounds__(kBlock) void attend_part_kernel(PartArgs a) {
  __shared__ float lut[1 << K];
  __shared__ float red[kBlock];
  __shared__ float acc_s[kMaxHeadDim];
  const int tid = threadIdx.x;
  const int d = a.vcb.d, W = a.vcb.plane_words;
  const int64_t bh = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
  const int64_t b = bh / a.Hq, hq = bh % a.Hq;
  const int64_t g = b * a.Hkv + hq * a.Hkv / a.Hq;
  const uint8_t* blob = blob_of(a.vcb, g);
  const float* cent = reinterpret_cast<const float*>(blob + a.vcb.off_c);
  for (int i = tid; i < (1 << K); i += kBlock) lut[i] = cent[i];
  const int64_t t0 = c * kChunk;
  const int64_t t1 = t0 + kChunk < a.T ? t0 + kChunk : a.T;
  const float* s = a.scores + bh * a.T;

  float mx = -INFINITY;
  for (int64_t t = t0 + tid; t < t1; t += kBlock) mx = fmaxf(mx, s[t]);
  mx = wave_max_f32(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  const int lpt = d >> 3;                 // lanes per token
  const int slots = kBlock / lpt;         // threads past slots * lpt (d not dividing 2048) take no token
  const int slot = tid / lpt, sub = tid % lpt;
  const int word = sub >> 2, shift = (sub & 3) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float esum = 0.0f;
  // the next token's plane words, norm and score are loaded while this one is
  // accumulated (one token in flight per lane group is latency-bound)
  const uint32_t* rv = a.vrec + g * a.T * a.vcb.rec_words;
  uint32_t nw[K];
  float nn = 0.0f, ns = 0.0f;
  const auto load_tok = [&](int64_t t) {
    const uint32_t* r = rv + t * a.vcb.rec_words;
#pragma unroll
    for (int p = 0; p < K; ++p) nw[p] = r[p * W + word];
    nn = __uint_as_float(r[K * W]);
    ns = s[t];
  };
  const int64_t tbeg = slot < slots ? t0 + slot : t1;
  if (tbeg < t1) load_tok(tbeg);
  for (int64_t t = tbeg; t < t1; t += slots) {
    uint32_t by[K];
#pragma unroll
    for (int p = 0; p < K; ++p) by[p] = nw[p] >> shift;
    const float e = expf(ns - mx);
    const float w = e * nn;
    if (t + slots < t1) load_tok(t + slots);
    esum += e;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t idx = 0;
#pragma unroll
      for (int p = 0; p < K; ++p) idx |= ((by[p] >> i) & 1u) << p;
      acc[i] = fmaf(w, lut[idx], acc[i]);
    }
  }
  // sum over the token slots: coordinates 8 sub + i
  for (int j = tid; j < d; j += kBlock) acc_s[j] = 0.0f;
  red[tid] = sub == 0 ? esum : 0.0f;
  __syncthreads();
  for (int sl = 0; sl < slots; ++sl) {
    if (slot == sl) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc_s[8 * sub + i] += acc[i];
    }
    __syncthreads();
  }
  float* out = a.part + (bh * a.chunks + c) * (d + 2);
  for (int j = tid; j < d; j += kBlock) out[j] = acc_s[j];
  if (tid < 64) {
    float l = 0.0f;
    for (int i = tid; i < kBlock; i += 64) l += red[i];
    l = wave_sum_f32(l);
    if (tid == 0) {
      out[d] = mx;
      out[d + 1] = l;
    }
  }
}

// ---- the same chunk partials on int8 MFMA (value codebooks of k <= 3 bits)
//
// With the symmetric codebook written in the sign basis (as in the score
// kernel), c[idx_tj] = sum over odd plane subsets P of a_P (2 mask_P,tj - 1),
// mask_P = XOR of the planes in P.  With weights w_t = exp(s_t - m_c) n_t:
//   a_c[j] = sum_P a_P (2 M_P[j] - W),  M_P[j] = sum_t w_t mask_P,tj,  W = sum_t w_t.
// M_P is a product over the token axis, [heads x tokens] x [tokens x coordinates],
// run as v_mfma_i32_32x32x32_i8 per 32 tokens and 32 coordinates:
//  * A: w_t in 27-bit fixed point (unit = chunk max / 2^27), four 7-bit digits;
//    rows 8q + 4hc + l = digit l of query head 2q + hc of the GQA group.
//  * B: lane (column n = coordinate 32w + n, token half) takes byte n/8 of the
//    mask word of 16 tokens, from a byte-transposed copy of the records in LDS,
//    AND bit n%8: values {0, 2^(n%8)} (-128 for bit 7), undone after the sum.
// Integer sums are exact; only the fixed-point rounding of w_t (2^-28 of the
// chunk's largest weight) enters the result.
constexpr int kSub = 256;                  // tokens per staged sub-chunk
constexpr double kFix = 134217728.0;       // 2^27

struct MfmaPartArgs {
  CodebookArgs vcb;
  const uint32_t* vrec;
  const float* scores;   // [B][Hq][T]
  int64_t Hkv, T, Hq, chunks;
  int gq;                // query heads per kv head (<= 8)
  float* part;
};

// LDS carve-up (bytes) of attend_mfma_kernel, shared with its launcher.
constexpr int kRecStride = kSub + 4;       // words per record-word row (16-byte aligned, bank offset 4)
constexpr int kTbStride = kSub + 32;       // bytes per transposed mask-byte row: the 4 rows read by one
                                           // MFMA operand fall in different banks
constexpr int kAfGroup = 66;               // fragment entries per 32-token group: 2 halves of 33

struct AttendLds {
  size_t wq, rec, tb, af, total;
};

__host__ __device__ inline size_t a16(size_t x) { return (x + 15) / 16 * 16; }

__host__ __device__ inline AttendLds attend_lds(int gq, int rec_words, int masks, int W) {
  AttendLds o;
  o.wq = 0;                                                   // float weights, then digit bytes [gq][kChunk]
  o.rec = a16((size_t)gq * kChunk * 4);                       // uint32 [rec_words][kRecStride]
  o.tb = o.rec + a16((size_t)rec_words * kRecStride * 4);     // bytes [masks][W][4][kTbStride]
  o.af = o.tb + (size_t)masks * W * 4 * kTbStride;            // i32x4 [kSub/32][2][33]
  o.total = o.af + (size_t)(kSub / 32) * kAfGroup * 16;
  return o;
}

typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef int i32x16v __attribute__((ext_vector_type(16)));

template <int K>
__device__ __host__ constexpr int odd_subset(int s) {
  return K == 1 ? 1 : K == 2 ? (1 << s) : (s < 3 ? (1 << s) : 7);
}

// Block-wide reductions over 256 threads (4 waves) through `red` (4 slots).
__device__ inline float block_max(float v, float* red) {
  v = wave_max_f32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ inline float block_sum(float v, float* red) {
  v = wave_sum_f32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ inline double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// 4 x 4 byte transpose: y[b] = byte b of x[0], x[1], x[2], x[3] (in that order).
__device__ inline void transpose4x4(const uint32_t* x, uint32_t* y) {
  const uint32_t p01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
  const uint32_t p23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t q01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
  const uint32_t q23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  y[0] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
  y[1] = __builtin_amdgcn_perm(p23, p01, 0x07060302u);
  y[2] = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
  y[3] = __builtin_amdgcn_perm(q23, q01, 0x07060302u);
}

// One workgroup per (b, kv head, chunk of kChunk tokens), all gq query heads.
// Wave v owns record words w = v, v + 4, ... (WPW of them) and every mask of each.
template <int K, int WPW>
__global__ __launch_bounds__(kBlock) void attend_mfma_kernel(MfmaPartArgs a) {
  constexpr int NM = 1 << (K - 1);          // odd plane subsets
  constexpr int RWMAX = K * 4 * WPW + 1;    // record words (planes + norm)
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float red[4];
  __shared__ double redd[4];
  __shared__ double coef[NM];
  __shared__ float hm[8], hl[8], hunit[8];
  __shared__ double homega[8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches on it stay scalar
  const int d = a.vcb.d, W = a.vcb.plane_words, RW = a.vcb.rec_words, gq = a.gq;
  const AttendLds lay = attend_lds(gq, RW, NM, W);
  float* wf = reinterpret_cast<float*>(smem + lay.wq);
  uint32_t* wd = reinterpret_cast<uint32_t*>(smem + lay.wq);   // digit bytes of the codes
  uint32_t* rec = reinterpret_cast<uint32_t*>(smem + lay.rec);
  uint8_t* tb = smem + lay.tb;
  i32x4v* af = reinterpret_cast<i32x4v*>(smem + lay.af);

  const int64_t g = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
  const int64_t b = g / a.Hkv, hkv = g % a.Hkv;
  const uint8_t* blob = blob_of(a.vcb, g);
  const int64_t t0 = c * kChunk;
  const int nt = (int)(a.T - t0 < kChunk ? a.T - t0 : kChunk);
  const uint32_t* rv = a.vrec + (g * a.T + t0) * RW;

  // records of sub-chunk 0 in flight (thread = token) while the weights are formed
  uint32_t pre[RWMAX];
  const auto load_sub = [&](int s0) {
    const bool ok = s0 + tid < nt;
    const uint32_t* r = rv + (int64_t)(ok ? s0 + tid : 0) * RW;
#pragma unroll
    for (int i = 0; i < RWMAX; ++i)
      if (i < RW) pre[i] = ok ? r[i] : 0u;
  };
  load_sub(0);

  if (tid < NM) {
    // a_P = (1/L) sum_v c_v prod_{p in P} sigma_p(v)
    const float* cent = reinterpret_cast<const float*>(blob + a.vcb.off_c);
    const int sb = odd_subset<K>(tid);
    double acc = 0.0;
    for (int v = 0; v < (1 << K); ++v) acc += (__popc(~v & sb) & 1) ? -(double)cent[v] : (double)cent[v];
    coef[tid] = acc / (1 << K);
  }
  for (int e = tid; e < (kSub / 32) * kAfGroup; e += kBlock) af[e] = i32x4v{0, 0, 0, 0};   // rows of absent heads

  // ---- weights: per head, chunk max, exp, sum, and the fixed-point codes
  constexpr int kPer = kChunk / kBlock;
  float nrm[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = tid + i * kBlock;
    nrm[i] = t < nt ? __uint_as_float(rv[(int64_t)t * RW + K * W]) : 0.0f;
  }
  for (int h = 0; h < gq; ++h) {
    const float* sc = a.scores + ((b * a.Hq + hkv * gq + h) * a.T + t0);
    float sv[kPer], mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int t = tid + i * kBlock;
      sv[i] = t < nt ? sc[t] : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = block_max(mx, red);
    float es = 0.0f, om = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int t = tid + i * kBlock;
      const float e = t < nt ? expf(sv[i] - mx) : 0.0f;
      es += e;
      const float w = e * nrm[i];
      om = fmaxf(om, w);
      wf[h * kChunk + t] = w;
    }
    es = block_sum(es, red);
    om = block_max(om, red);
    const double fs = kFix / (double)(om > 0.0f ? om : 1.0f);
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int t = tid + i * kBlock;
      const uint32_t v = (uint32_t)rint((double)wf[h * kChunk + t] * fs);   // <= 2^27
      tot += (double)v;                           // integers: exact in any order
      // 7-bit digits of v in the four bytes
      wd[h * kChunk + t] = (v & 0x7Fu) | ((v << 1) & 0x7F00u) | ((v << 2) & 0x7F0000u) | ((v << 3) & 0x7F000000u);
    }
    tot = block_sum_f64(tot, redd);
    if (tid == 0) {
      hm[h] = mx;
      hl[h] = es;
      hunit[h] = om > 0.0f ? om : 1.0f;
      homega[h] = tot;
    }
  }

  i32x16v acc[WPW][NM];
#pragma unroll
  for (int x = 0; x < WPW; ++x)
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[x][m] = i32x16v{};
  const int col = lane & 31, kh = lane >> 5;

  for (int s0 = 0; s0 < nt; s0 += kSub) {
    const int ns = nt - s0 < kSub ? nt - s0 : kSub;
    // record words of this sub-chunk, word-major; then the next sub-chunk's loads
#pragma unroll
    for (int i = 0; i < RWMAX; ++i)
      if (i < RW) rec[i * kRecStride + tid] = pre[i];
    if (s0 + kSub < nt) load_sub(s0 + kSub);
    __syncthreads();                              // records, codes in; last sub-chunk's fragments consumed
    // A fragments: head hh, tokens 4 qd .. 4 qd + 3 -> dword q of lanes (row 8(hh/2) + 4(hh%2) + l, half)
    for (int e = tid; e < gq * (kSub / 4); e += kBlock) {
      const int hh = e / (kSub / 4), qd = e % (kSub / 4);
      const int gi = qd >> 3, half = (qd >> 2) & 1, q = qd & 3;
      const uint4 x4 = *reinterpret_cast<const uint4*>(wd + hh * kChunk + s0 + 4 * qd);
      const uint32_t x[4] = {x4.x, x4.y, x4.z, x4.w};
      uint32_t y[4];
      transpose4x4(x, y);
      const int row0 = 8 * (hh >> 1) + 4 * (hh & 1);
#pragma unroll
      for (int l = 0; l < 4; ++l) reinterpret_cast<uint32_t*>(af + gi * kAfGroup + 33 * half + row0 + l)[q] = y[l];
    }
    // byte transpose of the mask words: tb[m][w][byte][token]
    for (int e = tid; e < NM * W * (kSub / 4); e += kBlock) {
      const int tq = e % (kSub / 4), mw = e / (kSub / 4), w = mw % W, m = mw / W;
      const int sb = odd_subset<K>(m);
      uint32_t x[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int p = 0; p < K; ++p)
        if ((sb >> p) & 1) {
          const uint4 r4 = *reinterpret_cast<const uint4*>(rec + (p * W + w) * kRecStride + 4 * tq);
          x[0] ^= r4.x; x[1] ^= r4.y; x[2] ^= r4.z; x[3] ^= r4.w;
        }
      uint32_t y[4];
      transpose4x4(x, y);
      uint32_t* dst = reinterpret_cast<uint32_t*>(tb + (size_t)(m * W + w) * 4 * kTbStride) + tq;
#pragma unroll
      for (int by = 0; by < 4; ++by) dst[by * (kTbStride / 4)] = y[by];
    }
    __syncthreads();
    const uint32_t bit = 0x01010101u << (col & 7);
    for (int gi = 0; gi < (ns + 31) / 32; ++gi) {
      const i32x4v av = af[gi * kAfGroup + 33 * kh + col];
#pragma unroll
      for (int x = 0; x < WPW; ++x) {
        const int w = wave + 4 * x;
        if (w < W) {
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const uint4 r4 = *reinterpret_cast<const uint4*>(
                tb + ((size_t)(m * W + w) * 4 + (col >> 3)) * kTbStride + 32 * gi + 16 * kh);
            const i32x4v bv = {(int)(r4.x & bit), (int)(r4.y & bit), (int)(r4.z & bit), (int)(r4.w & bit)};
            acc[x][m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc[x][m], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- a[j] = unit * sum_P a_P (2 M_P[j] - W) for this lane's coordinate and heads
  const int e7 = col & 7;
#pragma unroll
  for (int x = 0; x < WPW; ++x) {
    const int w = wave + 4 * x;
    if (w >= W) continue;
    const int j = 32 * w + col;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int hh = 2 * q + kh;
      if (hh >= gq) continue;
      double tot = 0.0;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        int64_t mv = 0;
#pragma unroll
        for (int l = 3; l >= 0; --l) mv = mv * 128 + (int64_t)acc[x][m][4 * q + l];
        mv = e7 == 7 ? -(mv >> 7) : (mv >> e7);
        tot += coef[m] * (double)(2 * mv - (int64_t)homega[hh]);
      }
      const double unit = (double)hunit[hh] / kFix;
      a.part[((b * a.Hq + hkv * gq + hh) * a.chunks + c) * (d + 2) + j] = (float)(tot * unit);
    }
  }
  if (tid < gq) {
    float* out = a.part + ((b * a.Hq + hkv * gq + tid) * a.chunks + c) * (d + 2);
    out[d] = hm[tid];
    out[d + 1] = hl[tid];
  }
}

// ---- fused decode attention at head_dim 128 (keys and values, k <= 3 planes
// each).  A small kernel prepares the query side of every (sequence, kv head)
// once (the score kernel's fixed-point MFMA fragments, tq_score_core.h) into
// the workspace; then one workgroup per (sequence, kv head, chunk of kFChunk
// tokens) issues all of its loads at once (fragments, key tiles, value norms
// and records), scores the chunk's keys straight into LDS, and runs the chunk
// softmax and the value MFMA above on them, writing the same per-chunk partials
// for attend_merge_kernel.  No score reaches memory.
// Small workgroups (4 waves, 512 tokens) so that four share a CU: the phases of
// a chunk (loads, scores, softmax, values) then overlap across workgroups
// (with one workgroup per CU the step took 1.45x as long as with two).
constexpr int64_t kFChunk = 512;           // tokens per fused workgroup
constexpr int kFBlock = 256;               // 4 waves
constexpr int kFWaves = kFBlock / 64;
constexpr int kQBlock = 512;               // query-side workgroup (8 waves)
constexpr size_t kQprepBytes = 20 * 1024 + 256;   // per group: fragments (<= 20 MFMAs x 1 KB), constants
constexpr int kFSub = 256;                 // tokens per value sub-chunk (two per chunk)
constexpr int kFRecStride = kFSub + 4;     // as kRecStride and kTbStride, for kFSub tokens
constexpr int kFTbStride = kFSub + 32;

struct QprepArgs {
  CodebookArgs kcb;
  const void* q;
  int q_dtype;
  int64_t Hkv, Hq;
  int gq;
  uint8_t* qws;          // [groups][kQprepBytes]: i32x4 fragments [NMF][64], then float consts [4][4]
  int32_t* status;
};

template <int KK>
__global__ __launch_bounds__(kQBlock) void attend_qprep_kernel(QprepArgs a) {
  constexpr int NMF = sc128::Masks<KK>::kMfma;
  __shared__ sc128::QueryLds<KK> qs;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.x, b = g / a.Hkv, hkv = g % a.Hkv;
  const uint8_t* kblob = blob_of(a.kcb, g);
  if (tid == 0 && a.status && blob_mismatch(a.kcb, kblob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  const sc128::QuerySrc src{reinterpret_cast<const float*>(kblob + a.kcb.off_c),
                            reinterpret_cast<const uint32_t*>(kblob + a.kcb.off_d),
                            reinterpret_cast<const _Float16*>(kblob + a.kcb.off_s),
                            a.q, a.q_dtype, ((b * a.Hq) + hkv * a.gq) * sc128::kD, a.gq,
                            a.kcb.rotation == kRotHaar ? reinterpret_cast<const float*>(kblob + a.kcb.off_d)
                                                       : nullptr};
  sc128::QueryRegs<KK> qr;
  sc128::query_load<KK>(src, qr, tid, wave, lane);
  sc128::query_build<KK, kQBlock>(qs, qr, a.gq, tid, wave, lane);
  uint8_t* out = a.qws + g * kQprepBytes;
  for (int e = tid; e < NMF * 64; e += kQBlock) reinterpret_cast<sc128::i32x4*>(out)[e] = qs.afrag[e];
  if (tid < 16) reinterpret_cast<float*>(out + NMF * 1024)[tid] = qs.consts[tid >> 2][tid & 3];
}

struct FusedArgs {
  CodebookArgs kcb, vcb;
  const uint32_t* krec;
  const uint32_t* vrec;
  const uint8_t* qws;
  float scale;
  int64_t Hkv, T, Hq, chunks;
  int gq;                // query heads per kv head (1, 2 or 4)
  float* part;
  int32_t* status;
};

// Dynamic LDS of attend_fused_kernel (bytes), shared with its launcher.
struct FusedLds {
  size_t wq, rec, tb, af, kst, total;
};

__host__ __device__ inline FusedLds fused_lds(int gq, int kv_planes, int kk_planes) {
  const int rwv = 4 * kv_planes + 1, nm = 1 << (kv_planes - 1);
  const int nch = (16 * (4 * kk_planes + 6) + 63) / 64;
  FusedLds o;
  o.wq = 0;                                                   // scores, weights, digit bytes [gq][kFChunk]
  o.rec = a16((size_t)gq * kFChunk * 4);                      // value words [rwv][kFRecStride]
  o.tb = o.rec + a16((size_t)rwv * kFRecStride * 4);          // bytes [nm][4][4][kFTbStride]
  o.af = o.tb + (size_t)nm * 4 * 4 * kFTbStride;              // i32x4 [kFSub/32][2][33]
  o.kst = o.af + (size_t)(kFSub / 32) * kAfGroup * 16;        // key tiles: uint2 [kFWaves][64 nch]
  o.total = o.kst + (size_t)kFWaves * 64 * nch * 8;
  return o;
}

template <int KK, int KV>
__global__ __launch_bounds__(kFBlock) void attend_fused_kernel(FusedArgs a) {
  using sc128::i32x4;
  constexpr int NMF = sc128::Masks<KK>::kMfma;
  constexpr int RWK = sc128::key_words<KK>();
  constexpr int NCH = (16 * RWK + 63) / 64;       // 8-byte chunks per lane per key tile
  constexpr int NM = 1 << (KV - 1);               // odd value-plane subsets
  constexpr int W = 4;                            // value plane words (d = 128)
  constexpr int RWV = KV * W + 1;                 // value record words
  constexpr int kTiles = kFChunk / 32 / kFWaves;   // key tiles per wave
  constexpr int kPer = kFChunk / kFBlock;          // tokens per thread in the softmax
  constexpr int kVH = kFBlock / kFSub;            // staging threads per value token
  constexpr int kVW = (RWV + kVH - 1) / kVH;      // value words per staging thread and sub-chunk
  constexpr int kNS = kFChunk / kFSub;             // value sub-chunks
  constexpr int d = sc128::kD;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float consts[4][4];
  __shared__ float wred[kFWaves][4][3];           // per wave and head: max score, sum exp, max weight
  __shared__ double womega[kFWaves][4];           // per wave and head: sum of the fixed-point weights
  __shared__ double vcoef[NM];
  __shared__ float hm[4], hl[4], hunit[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches on it stay scalar
  const int gq = a.gq;
  const FusedLds lay = fused_lds(gq, KV, KK);
  float* wf = reinterpret_cast<float*>(smem + lay.wq);
  uint32_t* wd = reinterpret_cast<uint32_t*>(smem + lay.wq);   // digit bytes of the codes
  uint32_t* rec = reinterpret_cast<uint32_t*>(smem + lay.rec);
  uint8_t* tb = smem + lay.tb;
  i32x4v* af = reinterpret_cast<i32x4v*>(smem + lay.af);
  uint2* kst = reinterpret_cast<uint2*>(smem + lay.kst);

  const int64_t g = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
  const int64_t b = g / a.Hkv, hkv = g % a.Hkv;
  const int64_t t0 = c * kFChunk;
  const int nt = (int)(a.T - t0 < kFChunk ? a.T - t0 : kFChunk);
  const uint8_t* vblob = blob_of(a.vcb, g);
  if (tid == 0 && a.status && blob_mismatch(a.vcb, vblob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  const int h = lane >> 5, col = lane & 31, kh = lane >> 5;

  // ---- every load at once, in the order of use; past T the buffer loads
  // return zero (such tokens get no weight), so all are issued unconditionally
  // and each wait counts exactly the loads still needed
  const uint8_t* qw = a.qws + g * kQprepBytes;
  i32x4 A[NMF];
#pragma unroll
  for (int f = 0; f < NMF; ++f) A[f] = reinterpret_cast<const i32x4*>(qw)[f * 64 + lane];
  float cst = 0.0f;
  if (tid < 16) cst = reinterpret_cast<const float*>(qw + NMF * 1024)[tid];
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.krec + g * a.T * RWK), 0, (int)(a.T * RWK * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.vrec + g * a.T * RWV), 0, (int)(a.T * RWV * 4), kRsrcWord3);
  uint2 raw[kTiles][NCH];                         // wave w: tiles w, w + 8, ... of the chunk
#pragma unroll
  for (int k = 0; k < kTiles; ++k) {
    const uint32_t base = (uint32_t)((t0 + (int64_t)(wave + kFWaves * k) * 32) * RWK * 4) + 8u * lane;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      raw[k][i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(krs, base + 512u * i, 0, 0));
  }
  float nrm[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    nrm[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        vrs, (uint32_t)((t0 + tid + i * kFBlock) * RWV * 4) + 4u * (KV * W), 0, 0));
  const int vtok = tid % kFSub, vhalf = tid / kFSub;   // value staging: token, first word
  uint32_t vr[kNS][kVW];
#pragma unroll
  for (int sc = 0; sc < kNS; ++sc) {
    const uint32_t tok_off = (uint32_t)((t0 + sc * kFSub + vtok) * RWV * 4);
#pragma unroll
    for (int i = 0; i < kVW; ++i) {
      const int wi = vhalf + kVH * i;
      vr[sc][i] = __builtin_amdgcn_raw_buffer_load_b32(vrs, wi < RWV ? tok_off + 4u * wi : 0xC0000000u, 0, 0);
    }
  }
  if (tid < NM) {
    // value codebook in the sign basis: a_P = (1/L) sum_v c_v prod_{p in P} sigma_p(v)
    const float* cent = reinterpret_cast<const float*>(vblob + a.vcb.off_c);
    const int sb = odd_subset<KV>(tid);
    double acc = 0.0;
    for (int v = 0; v < (1 << KV); ++v) acc += (__popc(~v & sb) & 1) ? -(double)cent[v] : (double)cent[v];
    vcoef[tid] = acc / (1 << KV);
  }
  for (int e = tid; e < (kFSub / 32) * kAfGroup; e += kFBlock) af[e] = i32x4v{0, 0, 0, 0};   // rows of absent heads
  if (tid < 16) consts[tid >> 2][tid & 3] = cst;
  __syncthreads();

  // ---- (S) scores of the chunk's keys into wf[head][token]
  uint2* st2 = kst + wave * 64 * NCH;
  const uint32_t* st = reinterpret_cast<const uint32_t*>(st2) + col * RWK;
#pragma unroll
  for (int k = 0; k < kTiles; ++k) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) st2[lane + 64 * i] = raw[k][i];
    float sa, sb;
    sc128::score_tile<KK>(A, st, consts, a.scale, h, sa, sb);
    const int tt = (wave + kFWaves * k) * 32 + col;
    if (2 * h < gq) wf[(2 * h) * kFChunk + tt] = sa;
    if (2 * h + 1 < gq) wf[(2 * h + 1) * kFChunk + tt] = sb;
  }
  __syncthreads();

  // ---- (W) weights of all heads at once, two barriers: chunk max; then exp,
  // sum and the largest weight; then the fixed-point codes, whose sum stays in
  // per-wave partials until the finalize
  {
    float sv[4][kPer], mloc[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      mloc[hh] = -INFINITY;
      if (hh < gq) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int t = tid + i * kFBlock;
          sv[hh][i] = t < nt ? wf[hh * kFChunk + t] : -INFINITY;
          mloc[hh] = fmaxf(mloc[hh], sv[hh][i]);
        }
        mloc[hh] = wave_max_f32(mloc[hh]);
        if (lane == 0) wred[wave][hh][0] = mloc[hh];
      }
    }
    __syncthreads();
    float mx[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      if (hh >= gq) continue;
      mx[hh] = wred[0][hh][0];
#pragma unroll
      for (int w = 1; w < kFWaves; ++w) mx[hh] = fmaxf(mx[hh], wred[w][hh][0]);
      float esl = 0.0f, oml = 0.0f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int t = tid + i * kFBlock;
        const float e = t < nt ? expf(sv[hh][i] - mx[hh]) : 0.0f;
        esl += e;
        sv[hh][i] = e * nrm[i];                     // the weight
        oml = fmaxf(oml, sv[hh][i]);
      }
      esl = wave_sum_f32(esl);
      oml = wave_max_f32(oml);
      if (lane == 0) {
        wred[wave][hh][1] = esl;
        wred[wave][hh][2] = oml;
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      if (hh >= gq) continue;
      float es = 0.0f, om = 0.0f;
#pragma unroll
      for (int w = 0; w < kFWaves; ++w) {
        es += wred[w][hh][1];
        om = fmaxf(om, wred[w][hh][2]);
      }
      const double fs = kFix / (double)(om > 0.0f ? om : 1.0f);
      double tot = 0.0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int t = tid + i * kFBlock;
        const uint32_t v = (uint32_t)rint((double)sv[hh][i] * fs);   // <= 2^27
        tot += (double)v;                           // integers: exact in any order
        wd[hh * kFChunk + t] = (v & 0x7Fu) | ((v << 1) & 0x7F00u) | ((v << 2) & 0x7F0000u) | ((v << 3) & 0x7F000000u);
      }
      tot = wave_sum_f64(tot);
      if (lane == 0) womega[wave][hh] = tot;
      if (tid == 0) {
        hm[hh] = mx[hh];
        hl[hh] = es;
        hunit[hh] = om > 0.0f ? om : 1.0f;
      }
    }
  }

  // ---- (V) value MFMA over sub-chunks of kFSub tokens; all 8 waves: wave w
  // takes word w % 4 and the 32-token groups of parity w / 4
  i32x16v acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = i32x16v{};
  constexpr int kVPar = kFWaves / 4;              // waves per value word
  const int vw = wave & 3, vpar = wave >> 2;
#pragma unroll
  for (int sc = 0; sc < kNS; ++sc) {
    const int s0 = sc * kFSub;
    if (s0 >= nt) break;
    const int ns = nt - s0 < kFSub ? nt - s0 : kFSub;
#pragma unroll
    for (int i = 0; i < kVW; ++i) {
      const int wi = vhalf + kVH * i;
      if (wi < RWV) rec[wi * kFRecStride + vtok] = vr[sc][i];
    }
    __syncthreads();                              // records, codes in; last sub-chunk's fragments consumed
    // A fragments: head hh, tokens 4 qd .. 4 qd + 3 -> dword q of lanes (row 8(hh/2) + 4(hh%2) + l, half)
    for (int e = tid; e < gq * (kFSub / 4); e += kFBlock) {
      const int hh = e / (kFSub / 4), qd = e % (kFSub / 4);
      const int gi = qd >> 3, half = (qd >> 2) & 1, q = qd & 3;
      const uint4 x4 = *reinterpret_cast<const uint4*>(wd + hh * kFChunk + s0 + 4 * qd);
      const uint32_t x[4] = {x4.x, x4.y, x4.z, x4.w};
      uint32_t y[4];
      transpose4x4(x, y);
      const int row0 = 8 * (hh >> 1) + 4 * (hh & 1);
#pragma unroll
      for (int l = 0; l < 4; ++l) reinterpret_cast<uint32_t*>(af + gi * kAfGroup + 33 * half + row0 + l)[q] = y[l];
    }
    // byte transpose of the mask words: tb[m][w][byte][token]
    for (int e = tid; e < NM * W * (kFSub / 4); e += kFBlock) {
      const int tq = e % (kFSub / 4), mw = e / (kFSub / 4), w = mw % W, m = mw / W;
      const int sb = odd_subset<KV>(m);
      uint32_t x[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int p = 0; p < KV; ++p)
        if ((sb >> p) & 1) {
          const uint4 r4 = *reinterpret_cast<const uint4*>(rec + (p * W + w) * kFRecStride + 4 * tq);
          x[0] ^= r4.x; x[1] ^= r4.y; x[2] ^= r4.z; x[3] ^= r4.w;
        }
      uint32_t y[4];
      transpose4x4(x, y);
      uint32_t* dst = reinterpret_cast<uint32_t*>(tb + (size_t)(m * W + w) * 4 * kFTbStride) + tq;
#pragma unroll
      for (int by = 0; by < 4; ++by) dst[by * (kFTbStride / 4)] = y[by];
    }
    __syncthreads();
    const uint32_t bit = 0x01010101u << (col & 7);
    for (int gi = vpar; gi < (ns + 31) / 32; gi += kVPar) {
      const i32x4v av = af[gi * kAfGroup + 33 * kh + col];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 r4 = *reinterpret_cast<const uint4*>(
            tb + ((size_t)(m * W + vw) * 4 + (col >> 3)) * kFTbStride + 32 * gi + 16 * kh);
        const i32x4v bv = {(int)(r4.x & bit), (int)(r4.y & bit), (int)(r4.z & bit), (int)(r4.w & bit)};
        acc[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc[m], 0, 0, 0);
      }
    }
  }

  // ---- (F) waves 4-7 hand their sums to waves 0-3 through LDS (from the
  // value records' area on, free now); a[j] = unit * sum_P a_P (2 M_P[j] - W)
  __syncthreads();
  int* xch = reinterpret_cast<int*>(smem + lay.rec);   // [4 waves][NM][8 regs][64 lanes]
  if (kVPar > 1 && wave >= 4) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int r = 0; r < 8; ++r) xch[((vw * NM + m) * 8 + r) * 64 + lane] = acc[m][r];
  }
  __syncthreads();
  if (wave < 4) {
    const int e7 = col & 7;
    const int j = 32 * vw + col;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int hh = 2 * q + kh;
      if (hh >= gq) continue;
      double omega = 0.0;
#pragma unroll
      for (int w = 0; w < kFWaves; ++w) omega += womega[w][hh];
      double tot = 0.0;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        int64_t mv = 0;
#pragma unroll
        for (int l = 3; l >= 0; --l)
          mv = mv * 128 + (int64_t)acc[m][4 * q + l] +
               (kVPar > 1 ? (int64_t)xch[((vw * NM + m) * 8 + 4 * q + l) * 64 + lane] : 0);
        mv = e7 == 7 ? -(mv >> 7) : (mv >> e7);
        tot += vcoef[m] * (double)(2 * mv - (int64_t)omega);
      }
      const double unit = (double)hunit[hh] / kFix;
      a.part[((b * a.Hq + hkv * gq + hh) * a.chunks + c) * (d + 2) + j] = (float)(tot * unit);
    }
  }
  if (tid < gq) {
    float* out = a.part + ((b * a.Hq + hkv * gq + tid) * a.chunks + c) * (d + 2);
    out[d] = hm[tid];
    out[d + 1] = hl[tid];
  }
}

struct MergeArgs {
  CodebookArgs vcb;
  const float* part;
  int64_t Hkv, Hq, chunks;
  float* out;            // [B][Hq][d]
};

// One workgroup per (b, query head) merges that row's chunk partials.  Its
// 16 waves hold kU chunk rows per thread in flight; the first batch is issued
// before the pass over the chunk maxima (the rows do not depend on the
// weights), so at 256 chunks per row and d = 128 every load of the row is in
// flight at once and the kernel waits about one memory round trip.
constexpr int kMBlock = 1024;

__global__ __launch_bounds__(kMBlock) void attend_merge_kernel(MergeArgs a) {
  constexpr int kWTile = 2048;             // chunk weights held in LDS at a time
  constexpr int kU = 16;                   // chunk rows in flight per thread
  constexpr int kMWaves = kMBlock / 64;
  __shared__ float v[kMaxHeadDim];
  __shared__ float wsh[kWTile];
  __shared__ float lsh[kWTile];
  __shared__ float part[2 * kMBlock];      // [row class][d]: rp * d = 2 * kMBlock floats
  __shared__ float red[kMWaves];
  const int tid = threadIdx.x;
  const int d = a.vcb.d;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.Hq, hq = bh % a.Hq;
  const int64_t g = b * a.Hkv + hq * a.Hkv / a.Hq;
  const uint8_t* blob = blob_of(a.vcb, g);
  const float* p = a.part + bh * a.chunks * (d + 2);
  // thread = (coordinate pair jp, row class cg): rows c = cg, cg + rp, ... of each
  // tile are summed in order, then the rp classes in order through LDS (threads
  // past rp classes, where d does not divide 2 kMBlock, take no rows)
  const int tpr = d / 2, rp = kMBlock / tpr;
  const int jp = tid % tpr, cg = tid / tpr < rp ? tid / tpr : kWTile;
  const auto load_rows = [&](float2* pv, int64_t c0, int c, int nc) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int cc = c + rp * u;
      pv[u] = cc < nc ? *reinterpret_cast<const float2*>(p + (c0 + cc) * (d + 2) + 2 * jp) : float2{0.0f, 0.0f};
    }
  };
  float2 pv[kU];
  load_rows(pv, 0, cg, (int)(a.chunks < kWTile ? a.chunks : kWTile));
  // chunk maxima (and, for the first tile, the maxima and sums kept in LDS)
  float mx = -INFINITY;
  for (int64_t c = tid; c < a.chunks; c += kMBlock) {
    const float2 ml = *reinterpret_cast<const float2*>(p + c * (d + 2) + d);
    mx = fmaxf(mx, ml.x);
    if (c < kWTile) {
      wsh[c] = ml.x;
      lsh[c] = ml.y;
    }
  }
  mx = wave_max_f32(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < kMWaves; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float l = 0.0f;
  float2 aj = {0.0f, 0.0f};
  for (int64_t c0 = 0; c0 < a.chunks; c0 += kWTile) {
    const int nc = (int)(a.chunks - c0 < kWTile ? a.chunks - c0 : kWTile);
    // rescale factor of each chunk, once
    for (int c = tid; c < nc; c += kMBlock) {
      float m_c, l_c;
      if (c0 == 0) {
        m_c = wsh[c];
        l_c = lsh[c];
      } else {
        const float2 ml = *reinterpret_cast<const float2*>(p + (c0 + c) * (d + 2) + d);
        m_c = ml.x;
        l_c = ml.y;
      }
      const float wc = expf(m_c - mx);
      wsh[c] = wc;
      l = fmaf(l_c, wc, l);
    }
    __syncthreads();
    for (int c = cg; c < nc; c += rp * kU) {
      if (c0 != 0 || c != cg) load_rows(pv, c0, c, nc);   // the first batch is already in flight
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int cc = c + rp * u;
        const float wc = cc < nc ? wsh[cc] : 0.0f;
        aj.x = fmaf(pv[u].x, wc, aj.x);
        aj.y = fmaf(pv[u].y, wc, aj.y);
      }
    }
    __syncthreads();
  }
  if (cg < rp) {
    part[cg * d + 2 * jp] = aj.x;
    part[cg * d + 2 * jp + 1] = aj.y;
  }
  l = wave_sum_f32(l);
  if ((tid & 63) == 0) red[tid >> 6] = l;
  __syncthreads();
  for (int j = tid; j < d; j += kMBlock) {
    float t = 0.0f;
    for (int q = 0; q < rp; ++q) t += part[q * d + j];
    v[j] = t;
  }
  __syncthreads();
  l = 0.0f;
#pragma unroll
  for (int w = 0; w < kMWaves; ++w) l += red[w];
  const float norm = l > 0.0f ? 1.0f / ((float)d * l) : 0.0f;
  if (a.vcb.rotation == kRotHaar) {
    // x^ = (n/d) R^T c: o_j = sum_i R[i][j] a_i / (d l), R row-major at off_d
    const float* R = reinterpret_cast<const float*>(blob + a.vcb.off_d);
    for (int j = tid; j < d; j += kMBlock) {
      float o = 0.0f;
      for (int i = 0; i < d; ++i) o = fmaf(R[i * d + j], v[i], o);
      a.out[bh * d + j] = o * norm;
    }
    return;
  }
  const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.vcb.off_d);
  for (int h = 1; h < d; h <<= 1) {
    for (int q = tid; q < d / 2; q += kMBlock) {
      int i = (q / h) * 2 * h + (q % h);
      float x0 = v[i], x1 = v[i + h];
      v[i] = x0 + x1;
      v[i + h] = x0 - x1;
    }
    __syncthreads();
  }
  for (int j = tid; j < d; j += kMBlock) {
    const float o = v[j] * norm;
    a.out[bh * d + j] = ((dbits[j >> 5] >> (j & 31)) & 1u) ? -o : o;
  }
}

}  // namespace

int64_t attend_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }
int64_t attend_fused_chunks(int64_t T) { return (T + kFChunk - 1) / kFChunk; }

namespace {

template <int K, int WPW>
int launch_attend_mfma(const MfmaPartArgs& pa, int64_t blocks, hipStream_t s) {
  const size_t lds = attend_lds(pa.gq, pa.vcb.rec_words, 1 << (K - 1), pa.vcb.plane_words).total;
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_mfma_kernel<K, WPW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024) != hipSuccess)
      return -10;
    attr_set = true;
  }
  hipLaunchKernelGGL((attend_mfma_kernel<K, WPW>), dim3((unsigned)blocks), dim3(kBlock), lds, s, pa);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

// MFMA partials (in the rotated domain, so for either rotation): values with
// k <= 3, head_dim a multiple of 32, an even GQA grouping of at most 8 query
// heads, and the LDS plan within 150 KB.
bool attend_mfma_supported(const CodebookArgs& vcb, int64_t Hkv, int64_t Hq) {
  if (vcb.k < 1 || vcb.k > 3 || vcb.d < 32 || (vcb.d & 31) != 0) return false;
  if (Hkv <= 0 || Hq % Hkv != 0 || Hq / Hkv > 8) return false;
  const int W = vcb.plane_words, masks = 1 << (vcb.k - 1);
  const int wpw = (W + 3) / 4;
  if (wpw != 1 && wpw != 2 && wpw != 4) return false;
  if (masks * wpw > 8) return false;
  return attend_lds((int)(Hq / Hkv), vcb.rec_words, masks, W).total <= 150 * 1024;
}

int launch_attend_mfma_k(const MfmaPartArgs& pa, int64_t blocks, hipStream_t s) {
  const int wpw = (pa.vcb.plane_words + 3) / 4;
  switch (pa.vcb.k * 8 + wpw) {
    case 8 + 1: return launch_attend_mfma<1, 1>(pa, blocks, s);
    case 8 + 2: return launch_attend_mfma<1, 2>(pa, blocks, s);
    case 8 + 4: return launch_attend_mfma<1, 4>(pa, blocks, s);
    case 16 + 1: return launch_attend_mfma<2, 1>(pa, blocks, s);
    case 16 + 2: return launch_attend_mfma<2, 2>(pa, blocks, s);
    case 16 + 4: return launch_attend_mfma<2, 4>(pa, blocks, s);
    case 24 + 1: return launch_attend_mfma<3, 1>(pa, blocks, s);
    case 24 + 2: return launch_attend_mfma<3, 2>(pa, blocks, s);
  }
  return -10;
}

}  // namespace

namespace {

template <int KK, int KV>
int launch_fused(const FusedArgs& fa, int64_t blocks, hipStream_t s) {
  const size_t lds = fused_lds(fa.gq, KV, KK).total;
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_fused_kernel<KK, KV>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 120 * 1024) != hipSuccess)
      return -10;
    attr_set = true;
  }
  hipLaunchKernelGGL((attend_fused_kernel<KK, KV>), dim3((unsigned)blocks), dim3(kFBlock), lds, s, fa);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace

size_t attend_qprep_bytes(int64_t groups) { return (size_t)groups * kQprepBytes; }

// Fused path: head_dim 128, 128 projections, Walsh-Hadamard or Haar rotations, key and
// value codebooks of k <= 3 planes, 1, 2 or 4 query heads per kv head, 8-byte
// aligned key records, and a group's key and value records under 2^30 bytes
// (32-bit buffer offsets).
bool attend_fused_supported(const CodebookArgs& kcb, const CodebookArgs& vcb, int64_t Hkv, int64_t Hq, int64_t T,
                            const void* krec) {
  const auto rot_ok = [](int r) { return r == kRotHadamard || r == kRotHaar; };
  if (kcb.d != 128 || kcb.m != 128 || !rot_ok(kcb.rotation) || kcb.k < 1 || kcb.k > 3) return false;
  if (vcb.d != 128 || !rot_ok(vcb.rotation) || vcb.k < 1 || vcb.k > 3) return false;
  if (reinterpret_cast<uintptr_t>(krec) & 7) return false;
  if (T + kChunk > (int64_t(1) << 30) / (4 * (kcb.rec_words > vcb.rec_words ? kcb.rec_words : vcb.rec_words)))
    return false;
  if (Hkv <= 0 || Hq % Hkv != 0) return false;
  const int64_t gq = Hq / Hkv;
  if (gq != 1 && gq != 2 && gq != 4) return false;
  const FusedLds lay = fused_lds((int)gq, vcb.k, kcb.k);
  // the finalize hands partial sums over through the LDS from the value records on
  const size_t xch = (size_t)4 * (1 << (vcb.k - 1)) * 8 * 64 * 4;
  return lay.total <= 120 * 1024 && lay.total - lay.rec >= xch;
}

int launch_attend_fused(const CodebookArgs& kcb, const CodebookArgs& vcb, const uint32_t* krec,
                        const uint32_t* vrec, int64_t B, int64_t Hkv, int64_t T, const void* q, int q_dtype,
                        int64_t Hq, float scale, uint8_t* qws, float* part, float* out, int32_t* status,
                        hipStream_t s) {
  if (B * Hq == 0) return 0;
  const int64_t chunks = attend_fused_chunks(T);
  const int64_t groups = B * Hkv;
  const int gq = (int)(Hq / Hkv);
  if (chunks > 0) {
    QprepArgs qa{kcb, q, q_dtype, Hkv, Hq, gq, qws, status};
    switch (kcb.k) {
      case 1: hipLaunchKernelGGL(attend_qprep_kernel<1>, dim3((unsigned)groups), dim3(kQBlock), 0, s, qa); break;
      case 2: hipLaunchKernelGGL(attend_qprep_kernel<2>, dim3((unsigned)groups), dim3(kQBlock), 0, s, qa); break;
      case 3: hipLaunchKernelGGL(attend_qprep_kernel<3>, dim3((unsigned)groups), dim3(kQBlock), 0, s, qa); break;
      default: return -13;
    }
    if (hipGetLastError() != hipSuccess) return -10;
    FusedArgs fa;
    fa.kcb = kcb;
    fa.vcb = vcb;
    fa.krec = krec;
    fa.vrec = vrec;
    fa.qws = qws;
    fa.scale = scale;
    fa.Hkv = Hkv; fa.T = T; fa.Hq = Hq;
    fa.chunks = chunks;
    fa.gq = gq;
    fa.part = part;
    fa.status = status;
    const int64_t blocks = groups * chunks;       // one workgroup per (sequence, kv head, chunk)
    int rc;
    switch (kcb.k * 4 + vcb.k) {
      case 4 + 1: rc = launch_fused<1, 1>(fa, blocks, s); break;
      case 4 + 2: rc = launch_fused<1, 2>(fa, blocks, s); break;
      case 4 + 3: rc = launch_fused<1, 3>(fa, blocks, s); break;
      case 8 + 1: rc = launch_fused<2, 1>(fa, blocks, s); break;
      case 8 + 2: rc = launch_fused<2, 2>(fa, blocks, s); break;
      case 8 + 3: rc = launch_fused<2, 3>(fa, blocks, s); break;
      case 12 + 1: rc = launch_fused<3, 1>(fa, blocks, s); break;
      case 12 + 2: rc = launch_fused<3, 2>(fa, blocks, s); break;
      case 12 + 3: rc = launch_fused<3, 3>(fa, blocks, s); break;
      default: rc = -13;
    }
    if (rc) return rc;
  }
  MergeArgs ma{vcb, part, Hkv, Hq, chunks, out};
  hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)(B * Hq)), dim3(kMBlock), 0, s, ma);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

// Chunk partials and merge: eight coordinates per lane in the partials, pairs
// in the merge, so head_dim a multiple of 8 (any power of two from 8 for the
// Walsh-Hadamard rotation).
bool attend_split_supported(const CodebookArgs& vcb) {
  return (vcb.rotation == kRotHadamard || vcb.rotation == kRotHaar) && vcb.d >= 8 && vcb.d % 8 == 0 &&
         vcb.d <= kMaxHeadDim && vcb.k >= 1 && vcb.k <= 8;
}

int launch_attend_split(const CodebookArgs& vcb, const uint32_t* vrec, const float* scores, int64_t B,
                        int64_t Hkv, int64_t T, int64_t Hq, float* part, float* out, hipStream_t s) {
  if (B * Hq == 0) return 0;
  const int64_t chunks = attend_chunks(T);
  if (chunks > 0 && attend_mfma_supported(vcb, Hkv, Hq)) {
    const MfmaPartArgs pa{vcb, vrec, scores, Hkv, T, Hq, chunks, (int)(Hq / Hkv), part};
    if (launch_attend_mfma_k(pa, B * Hkv * chunks, s) != 0) return -10;
  } else if (chunks > 0) {
    PartArgs pa{vcb, vrec, scores, Hkv, T, Hq, chunks, part};
    const dim3 grid((unsigned)(B * Hq * chunks));
    switch (vcb.k) {
      case 1: hipLaunchKernelGGL(attend_part_kernel<1>, grid, dim3(kBlock), 0, s, pa); break;
      case 2: hipLaunchKernelGGL(attend_part_kernel<2>, grid, dim3(kBlock), 0, s, pa); break;
      case 3: hipLaunchKernelGGL(attend_part_kernel<3>, grid, dim3(kBlock), 0, s, pa); break;
      case 4: hipLaunchKernelGGL(attend_part_kernel<4>, grid, dim3(kBlock), 0, s, pa); break;
      case 5: hipLaunchKernelGGL(attend_part_kernel<5>, grid, dim3(kBlock), 0, s, pa); break;
      case 6: hipLaunchKernelGGL(attend_part_kernel<6>, grid, dim3(kBlock), 0, s, pa); break;
      case 7: hipLaunchKernelGGL(attend_part_kernel<7>, grid, dim3(kBlock), 0, s, pa); break;
      default: hipLaunchKernelGGL(attend_part_kernel<8>, grid, dim3(kBlock), 0, s, pa); break;
    }
    if (hipGetLastError() != hipSuccess) return -10;
  }
  MergeArgs ma{vcb, part, Hkv, Hq, chunks, out};
  hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)(B * Hq)), dim3(kMBlock), 0, s, ma);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace tq
