// head_dim-128 scoring from compressed keys for gfx950 (CDNA4, wave64).
//
// Score of query head hq against key t (page "bitpolar 0.3.3
// src/kv_cache.rs", attention_scores: inner-product estimate times
// 1/sqrt(head_dim); page "turboquant-plus-rs 0.1.0 README", "Architecture":
// MSE stage + QJL residual correction):
//   s = scale * ( (n_t/d) sum_j qt_j c[idx_tj] + sqrt(pi/2)/m gamma_t sum_i p_i (2 s_ti - 1) ),
//   qt = H(D q), p = S qt / sqrt(d).
// No key is decoded.  The Lloyd-Max codebook is symmetric, so with
// sigma_p = 2 b_p - 1 (b_p = bit-plane p of idx)
//   c[idx] = sum over odd subsets P of planes of a_P * prod_{p in P} sigma_p,
// and prod_{p in P} sigma_p = 2 (XOR of the planes in P) - 1.  Both sums
// are then subset sums over bit masks of the record:
//   sum_j qt_j c[idx_j] = sum_P sum_{j in mask_P} 2 a_P qt_j - c_max sum_j qt_j
//   sum_i p_i (2 s_i - 1) = sum_{i in signs} 2 p_i - sum_i p_i.
// They run as int8 MFMA (v_mfma_i32_32x32x32_i8): B = mask bits expanded by
// one AND per dword (bytes in {0, 2^e}, e = bit offset in the byte), A = the
// query-side values 2 a_P qt_j and 2 p_i in 32-bit fixed point, split into 4
// signed int8 limbs and pre-divided by 2^e.  A rows: 4 query heads x
// {mse part, qjl part} x 4 limbs.  Integer accumulation is exact; only the
// fixed-point rounding of the query side (2^-23 of its largest entry, or
// less) enters the score.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_fast.h"

namespace tq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kM = 128;
// Workgroup size: 16 waves (one workgroup per CU) while the A fragments fit in
// 128 VGPRs; 8 waves for the 3-plane codebook, whose fragments need more.
template <int K>
constexpr int block_threads() { return K <= 2 ? 1024 : 512; }

struct Score128Args {
  const uint8_t* cbs;
  int64_t stride, n_cb;
  const uint32_t* krec;
  int64_t B, Hkv, T, Hq;
  const void* q;
  int q_dtype;
  float scale;
  float* scores;
  int32_t* status;
  int bits, rec_words, gq;   // gq = query heads per kv head (1, 2 or 4)
  uint32_t off_c, off_d, off_s;
  int64_t tiles, tiles_per_block, blocks_per_group;
};

// Number of odd subsets of k planes = 2^(k-1) mask words sets; plus signs.
template <int K>
struct Masks {
  static constexpr int kPlaneMasks = 1 << (K - 1);
  static constexpr int kMasks = kPlaneMasks + 1;
  static constexpr int kWords = 4 * kMasks;      // 32-bit words per key fed to MFMA
  static constexpr int kMfma = 2 * kWords / 2;   // each word feeds 2 MFMAs, 2 words per MFMA
};

// Odd subsets of {0..K-1} in a fixed order: for K=1 {0}; K=2 {0},{1};
// K=3 {0},{1},{2},{0,1,2}.
template <int K>
__device__ __host__ constexpr int subset_bits(int s) {
  return K == 1 ? 1 : K == 2 ? (1 << s) : (s < 3 ? (1 << s) : 7);
}

template <int K>
__global__ __launch_bounds__(block_threads<K>()) void score128_kernel(Score128Args a) {
  using Mk = Masks<K>;
  constexpr int kBlock = block_threads<K>();
  constexpr int kWaves = kBlock / 64;
  constexpr int L = 1 << K;
  constexpr int NMF = Mk::kMfma;                 // MFMAs per tile
  constexpr int kPWaves = 4 * kM / 64;           // waves of the projection step
  __shared__ float qt[4][kD];
  __shared__ float pp[4][kM];
  __shared__ float qstat[4][2];                  // per head: max |qt_j|, sum qt_j
  __shared__ float pstat[kPWaves][4][2];         // per projection wave and head: max |p_i|, sum p_i
  __shared__ float consts[4][4];                 // per head: delta_mse, delta_qjl, C_mse, C_qjl
  __shared__ float coef[8];                      // a_P
  __shared__ float cmax;                         // largest centroid
  __shared__ __align__(16) i32x4 afrag[NMF * 64];
  constexpr int kStage = 64 * ((16 * (4 * K + 6) + 63) / 64);   // 8-byte chunks per wave: one tile, rounded up
  __shared__ uint2 stage[kWaves * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches on it stay scalar
  const int64_t grp = blockIdx.x / a.blocks_per_group;      // (b, kv head)
  const int64_t chunk = blockIdx.x % a.blocks_per_group;
  const int64_t b = grp / a.Hkv, hkv = grp % a.Hkv;
  const uint8_t* blob = a.cbs + (grp % a.n_cb) * a.stride;
  if (tid == 0 && a.status) {
    const BlobHeader* hd = reinterpret_cast<const BlobHeader*>(blob);
    if (hd->magic != kBlobMagic || hd->version != kBlobVersion || hd->head_dim != kD || hd->bits != a.bits ||
        hd->role != TQ_ROLE_KEY || hd->projections != kM)
      atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  }
  const float* cent = reinterpret_cast<const float*>(blob + a.off_c);
  const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.off_d);
  const _Float16* S = reinterpret_cast<const _Float16*>(blob + a.off_s);

  // ---- query-side loads first: waves 0-3 take head `wave` (coordinates lane
  // and lane + 64), the projection waves a quarter row of S each, wave 0 the
  // centroids
  float q0 = 0.0f, q1 = 0.0f;
  uint32_t d0 = 0, d1 = 0;
  if (wave < 4 && wave < a.gq) {
    const int64_t off = ((b * a.Hq) + hkv * a.gq + wave) * kD + lane;
    q0 = load_elem(a.q, a.q_dtype, off);
    q1 = load_elem(a.q, a.q_dtype, off + 64);
    d0 = dbits[lane >> 5];
    d1 = dbits[2 + (lane >> 5)];
  }
  const int prow = tid >> 2, qtr = tid & 3;      // projection step: row prow, quarter qtr
  uint4 srow[4];
  if (wave < kPWaves) {
    const uint4* row = reinterpret_cast<const uint4*>(S + prow * kD + 32 * qtr);
#pragma unroll
    for (int v = 0; v < 4; ++v) srow[v] = row[v];
  }
  float cv[L];
  if (tid < Mk::kPlaneMasks) {
#pragma unroll
    for (int v = 0; v < L; ++v) cv[v] = cent[v];
  }
  __builtin_amdgcn_sched_barrier(0);

  const int h = lane >> 5, col = lane & 31;
  const float kqjl = kQjlConst / (float)kM;
  const float inv_d = 1.0f / (float)kD;
  const int64_t tile0 = chunk * a.tiles_per_block;
  const int64_t tile_end = min(tile0 + a.tiles_per_block, a.tiles);
  // A tile's 32 records are contiguous: they are loaded as 8-byte chunks by
  // consecutive lanes (RW even, so every record is 8-byte aligned and a ragged
  // tile ends on a chunk boundary), kPrefetch tiles ahead in a register ring,
  // then passed through this wave's LDS row so that lane (col, h) reads the
  // words it feeds: words h and h+2 of every bit plane and of the sign mask,
  // then n and gamma.
  // The loads go through a buffer resource that ends at this workgroup's last
  // record: past it (the ragged tail, prefetches beyond the range) they return
  // zero without a memory access, so every load is issued unconditionally and
  // the waits before each tile count exactly the loads and stores still needed
  // in flight (predicated loads make the compiler drain everything instead).
  // A zero record scores 0 and is never stored.
  constexpr int RW = 4 * K + 6;                          // record words (d = m = 128 keys)
  constexpr int NCH = (16 * RW + 63) / 64;               // 8-byte chunks per lane per tile
  constexpr int kPrefetch = 2;
  uint2 raw[kPrefetch][NCH];
  const int64_t rec_end = min(tile_end * 32, a.T);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.krec + grp * a.T * RW), 0, (int)(rec_end * RW * 4), kRsrcWord3);
  const auto load_raw = [&](int64_t t, uint2* rw) {
    const uint32_t base = (uint32_t)(t * 32 * RW * 4) + 8u * lane;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      rw[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(krs, base + 512u * i, 0, 0));
  };
  // scores of this (b, kv head): [gq][T]; stores past the end are dropped
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      a.scores + (b * a.Hq + hkv * a.gq) * a.T, 0, (int)(a.gq * a.T * 4), kRsrcWord3);
  uint2* st2 = stage + wave * kStage;
  const uint32_t* st = reinterpret_cast<const uint32_t*>(st2) + col * RW;
  // The first tiles' records are in flight while the query side is prepared.
  // Issued in slot order, each followed by two stores past the end of the
  // scores (dropped by the hardware): on entry the memory operations then stand
  // in the same order as in the loop (a slot's loads, its two score stores), so
  // the wait before each slot leaves the later slots' loads in flight.
#pragma unroll
  for (int sl = 0; sl < kPrefetch; ++sl) {
    load_raw(tile0 + wave + sl * kWaves, raw[sl]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_raw_buffer_store_b32(0u, srs, 0xC0000000u, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(0u, srs, 0xC0000040u, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- query side, three barriers
  // (1) a_P = (1/L) sum_v c_v prod_{p in P} sigma_p(v); qt = H D q per head in
  //     registers (butterflies of span 1..32 across lanes, then 64 within the
  //     lane), with max |qt_j| and sum qt_j
  if (tid < Mk::kPlaneMasks) {
    const int sb = subset_bits<K>(tid);
    double acc = 0.0;
#pragma unroll
    for (int v = 0; v < L; ++v) {
      const int par = __popc(~v & sb) & 1;       // number of -1 factors
      acc += par ? -(double)cv[v] : (double)cv[v];
    }
    coef[tid] = (float)(acc / L);
    if (tid == 0) cmax = cv[L - 1];
  }
  if (wave < 4) {
    float x0 = ((d0 >> (lane & 31)) & 1u) ? -q0 : q0;
    float x1 = ((d1 >> (lane & 31)) & 1u) ? -q1 : q1;
#pragma unroll
    for (int hs = 1; hs < 64; hs <<= 1) {
      const float o0 = __shfl_xor(x0, hs, 64), o1 = __shfl_xor(x1, hs, 64);
      x0 = (lane & hs) ? o0 - x0 : x0 + o0;
      x1 = (lane & hs) ? o1 - x1 : x1 + o1;
    }
    const float y0 = x0 + x1, y1 = x0 - x1;
    qt[wave][lane] = y0;
    qt[wave][lane + 64] = y1;
    const float m1 = wave_max_f32(fmaxf(fabsf(y0), fabsf(y1)));
    const float s1 = wave_sum_f32(y0 + y1);
    if (lane == 0) {
      qstat[wave][0] = m1;
      qstat[wave][1] = s1;
    }
  }
  __syncthreads();
  // (2) p = S qt / sqrt(d): threads 4i .. 4i+3 own row i, a quarter of it each,
  //     all four heads, then a 4-lane reduction; per wave, max |p_i| and sum p_i
  if (wave < kPWaves) {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t ww[4] = {srow[v].x, srow[v].y, srow[v].z, srow[v].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 pr = __builtin_bit_cast(f16x2, ww[e]);
        const int j = 32 * qtr + 8 * v + 2 * e;
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          acc[hh] = fmaf((float)pr[0], qt[hh][j], acc[hh]);
          acc[hh] = fmaf((float)pr[1], qt[hh][j + 1], acc[hh]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      acc[hh] += __shfl_xor(acc[hh], 1, 64);
      acc[hh] += __shfl_xor(acc[hh], 2, 64);
      acc[hh] *= 0.08838834764831845f;          // 1/sqrt(128)
    }
    pp[qtr][prow] = acc[qtr];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float pm = wave_max_f32(fabsf(acc[hh]));
      const float ps = wave_sum_f32(qtr == 0 ? acc[hh] : 0.0f);
      if (lane == 0) {
        pstat[wave][hh][0] = pm;
        pstat[wave][hh][1] = ps;
      }
    }
  }
  __syncthreads();
  // (3) per head, the value of one fixed-point unit (2^30 units for the largest
  //     |2 a_P qt_j| or |2 p_i|) and the constant terms; then the A fragments.
  // A fragment of MFMA f = 2*w2 + g, lane l: row m = l%32, K = 16(l/32) + 4q + byte.
  // Lane half hl of MFMA (w2, g) carries list word 2*w2 + hl; bit (8*byte + 4g + q)
  // of that word.  Row m = 8 hh + 4 part + limb holds signed int8 limb `limb` of
  // the value (zero where the mask belongs to the other part): the value V of
  // coordinate j is 2 a_P qt_j (plane masks) or 2 p_j (sign mask) in units,
  // pre-divided by 2^(j mod 8) (-128 for j mod 8 == 7: the top bit of a byte),
  // and its signed base-256 digits are the bytes of V + 0x80808080, each minus 128.
  // A thread's entries all share one row m (kBlock is a multiple of 128).
  const auto unit_of = [&](int hh, int part) {
    float vm;
    if (part == 0) {
      float amax = 0.0f;
      for (int s = 0; s < Mk::kPlaneMasks; ++s) amax = fmaxf(amax, fabsf(coef[s]));
      vm = 2.0f * amax * qstat[hh][0];
    } else {
      float m2 = 0.0f;
      for (int w = 0; w < kPWaves; ++w) m2 = fmaxf(m2, pstat[w][hh][0]);
      vm = 2.0f * m2;
    }
    return vm > 0.0f ? vm * (1.0f / 1073741824.0f) : 1.0f;
  };
  if (tid < 16) {
    const int hh = tid >> 2, c = tid & 3;
    float v;
    if (c < 2) {
      v = unit_of(hh, c);
    } else if (c == 2) {
      v = cmax * qstat[hh][1];                   // c_max * sum qt
    } else {
      v = 0.0f;
      for (int w = 0; w < kPWaves; ++w) v += pstat[w][hh][1];   // sum p
    }
    consts[hh][c] = v;
  }
  {
    const int m = (tid >> 2) & 31;
    const int hh = m >> 3, part = (m >> 2) & 1, limb = m & 3;
    const double inv_unit = 1.0 / (double)unit_of(hh, part);
    for (int idx = tid; idx < NMF * 64 * 4; idx += kBlock) {
      const int q = idx & 3, ln = (idx >> 2) & 63, f = idx >> 8;
      const int w2 = f >> 1, g = f & 1;
      const int li = 2 * w2 + (ln >> 5);        // list word: mask li/4, word li%4
      const int mask = li >> 2, ww = li & 3;
      const bool is_sign_mask = mask == Mk::kPlaneMasks;
      uint32_t packed = 0;
      if (hh < a.gq && part == (is_sign_mask ? 1 : 0)) {
#pragma unroll
        for (int byt = 0; byt < 4; ++byt) {
          const int jj = 32 * ww + 8 * byt + 4 * g + q;
          const float val = is_sign_mask ? 2.0f * pp[hh][jj] : 2.0f * coef[mask] * qt[hh][jj];
          const int sh = jj & 7;
          const double inv_div = sh == 7 ? -1.0 / 128.0 : 1.0 / (double)(1 << sh);
          const int V = (int)rint((double)val * inv_unit * inv_div);
          const uint32_t digit = (((uint32_t)V + 0x80808080u) >> (8 * limb)) & 0xFFu;
          packed |= (digit ^ 0x80u) << (8 * byt);
        }
      }
      reinterpret_cast<uint32_t*>(afrag)[(f * 64 + ln) * 4 + q] = packed;
    }
  }
  __syncthreads();

  i32x4 A[NMF];
#pragma unroll
  for (int f = 0; f < NMF; ++f) A[f] = afrag[f * 64 + lane];

  for (int64_t tile_base = tile0 + wave; tile_base < tile_end; tile_base += kPrefetch * kWaves) {
#pragma unroll
   for (int sl = 0; sl < kPrefetch; ++sl) {
    const int64_t tile = tile_base + sl * kWaves;
    const int64_t tok = tile * 32 + col;
    const bool valid = tok < rec_end;   // a tile past the range reads zeros and stores nothing
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      st2[c] = raw[sl][i];
    }
    load_raw(tile + kPrefetch * kWaves, raw[sl]);
    uint32_t wv[Mk::kWords / 2];
#pragma unroll
    for (int w2 = 0; w2 < Mk::kWords / 2; ++w2) {
      const int li = 2 * w2 + h, mask = li >> 2, s2 = (li & 3) >> 1;
      uint32_t word;
      if (mask == Mk::kPlaneMasks) {
        word = st[K * 4 + h + 2 * s2];
      } else {
        const int sb = subset_bits<K>(mask);
        word = 0;
#pragma unroll
        for (int p = 0; p < K; ++p)
          if ((sb >> p) & 1) word ^= st[p * 4 + h + 2 * s2];
      }
      wv[w2] = word;
    }
    const float nrm = __uint_as_float(st[K * 4 + 4]);
    const float gam = __uint_as_float(st[K * 4 + 5]);

    // one accumulation chain (registers are the occupancy limit; the other waves of
    // the SIMD fill the MFMA latency)
    i32x16 acc = {};
#pragma unroll
    for (int w2 = 0; w2 < Mk::kWords / 2; ++w2) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        i32x4 bv;
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[q] = (int)(wv[w2] & (0x01010101u << (4 * g + q)));
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[2 * w2 + g], bv, acc, 0, 0, 0);
      }
    }
    // rows 8*hh + 4*h + limb: this lane holds part h (0: mse, 1: qjl) of heads 0..3
    float part[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
      part[hh] = (float)acc[4 * hh] + 256.0f * (float)acc[4 * hh + 1] + 65536.0f * (float)acc[4 * hh + 2] +
                 16777216.0f * (float)acc[4 * hh + 3];
    // lane half 0 finishes heads 0,1; half 1 heads 2,3 (swap the parts they lack)
    // permlane32_swap(x, y): lanes 0-31 get x of lanes 32-63 in [1]; lanes 32-63 get y of lanes 0-31 in [0]
    auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
    auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
    // after the swap: half 0 holds (mse0, mse1) own + (qjl0, qjl1) received;
    //                 half 1 holds (qjl2, qjl3) own + (mse2, mse3) received
    float mse_a, mse_b, qjl_a, qjl_b;
    if (h == 0) {
      mse_a = part[0]; mse_b = part[1];
      qjl_a = __uint_as_float(s0[1]); qjl_b = __uint_as_float(s1[1]);
    } else {
      qjl_a = part[2]; qjl_b = part[3];
      mse_a = __uint_as_float(s0[0]); mse_b = __uint_as_float(s1[0]);
    }
    const int ha = 2 * h, hb = 2 * h + 1;
    // per-head constants stay in LDS (registers are the occupancy limit here)
    const float sa = a.scale * ((nrm * inv_d) * (consts[ha][0] * mse_a - consts[ha][2]) +
                                kqjl * gam * (consts[ha][1] * qjl_a - consts[ha][3]));
    const float sb2 = a.scale * ((nrm * inv_d) * (consts[hb][0] * mse_b - consts[hb][2]) +
                                 kqjl * gam * (consts[hb][1] * qjl_b - consts[hb][3]));
    // heads ha, hb >= gq land past the end of the resource, as does an invalid token
    const uint32_t so = valid ? (uint32_t)tok * 4u : 0xC0000000u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sa), srs, so + (uint32_t)(ha * a.T * 4), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sb2), srs, so + (uint32_t)(hb * a.T * 4), 0, 0);
   }
  }
}

template <int K>
int launch_k(Score128Args a, hipStream_t s) {
  constexpr int kWaves = block_threads<K>() / 64;
  // about one workgroup of 16 waves per CU, at least 16 tiles per wave
  const int64_t groups = a.B * a.Hkv;
  int64_t per_block = (a.tiles * groups + 256 * (16 / kWaves) - 1) / (256 * (16 / kWaves));
  if (per_block < 16 * kWaves) per_block = 16 * kWaves;
  if (per_block > a.tiles) per_block = a.tiles;
  a.tiles_per_block = per_block;
  a.blocks_per_group = (a.tiles + per_block - 1) / per_block;
  const int64_t blocks = groups * a.blocks_per_group;
  hipLaunchKernelGGL(score128_kernel<K>, dim3((unsigned)blocks), dim3(block_threads<K>()), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace

bool fast128_scores_supported(const Layout& L, int64_t Hkv, int64_t Hq, int64_t T, const void* krec) {
  if (L.d != kD || L.m != kM || L.k < 1 || L.k > 3) return false;
  if (reinterpret_cast<uintptr_t>(krec) & 7) return false;   // records read as 8-byte chunks
  // 32-bit buffer offsets: a group's records and its [gq][T] scores stay below 2^30 bytes
  if (T > (int64_t(1) << 30) / (4 * L.rec_words) || T > (int64_t(1) << 30) / 16) return false;
  const int64_t gq = Hq / Hkv;
  return gq == 1 || gq == 2 || gq == 4;
}

int launch_scores_fast128(const Layout& L, const void* cbs, int64_t n_cb, const uint32_t* krec, int64_t B,
                          int64_t Hkv, int64_t T, const void* q, int q_dtype, int64_t Hq, float scale,
                          float* scores, int32_t* status, hipStream_t s) {
  Score128Args a;
  a.cbs = static_cast<const uint8_t*>(cbs);
  a.stride = L.total;
  a.n_cb = n_cb;
  a.krec = krec;
  a.B = B; a.Hkv = Hkv; a.T = T; a.Hq = Hq;
  a.q = q; a.q_dtype = q_dtype;
  a.scale = scale;
  a.scores = scores;
  a.status = status;
  a.bits = L.bits; a.rec_words = L.rec_words; a.gq = (int)(Hq / Hkv);
  a.off_c = L.off_c; a.off_d = L.off_d; a.off_s = L.off_s;
  a.tiles = (T + 31) / 32;
  switch (L.k) {
    case 1: return launch_k<1>(a, s);
    case 2: return launch_k<2>(a, s);
    case 3: return launch_k<3>(a, s);
    default: return -13;
  }
}

}  // namespace tq
