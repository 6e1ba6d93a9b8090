// Compressed-key scoring at head_dim 128 (gfx950, wave64), shared by the score
// kernel and the fused attention kernel: the query side as int8 MFMA
// fragments, and the scores of one staged tile of 32 keys.
//
// Score of query head hq against key t (page "bitpolar 0.3.3
// src/kv_cache.rs", attention_scores: inner-product estimate times
// 1/sqrt(head_dim); page "turboquant-plus-rs 0.1.0 README", "Architecture":
// MSE stage + QJL residual correction):
//   s = scale * ( (n_t/d) sum_j qt_j c[idx_tj] + sqrt(pi/2)/m gamma_t sum_i p_i (2 s_ti - 1) ),
//   qt = H(D q) (Haar codebooks: qt = R q), p = S qt / sqrt(d).
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
#pragma once

#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace sc128 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kM = 128;
constexpr int kPWaves = 4 * kM / 64;   // waves of the projection step; workgroups have at least this many

// Odd subsets of the K planes (2^(K-1) plane masks) plus the sign mask; 4
// words of each per key feed the MFMA, two words per MFMA.
template <int K>
struct Masks {
  static constexpr int kPlaneMasks = 1 << (K - 1);
  static constexpr int kMasks = kPlaneMasks + 1;
  static constexpr int kWords = 4 * kMasks;      // 32-bit words per key fed to MFMA
  static constexpr int kMfma = kWords;           // each word feeds 2 MFMAs, 2 words per MFMA
};

// Odd subsets of {0..K-1} in a fixed order: for K=1 {0}; K=2 {0},{1};
// K=3 {0},{1},{2},{0,1,2}.
template <int K>
__device__ __host__ constexpr int subset_bits(int s) {
  return K == 1 ? 1 : K == 2 ? (1 << s) : (s < 3 ? (1 << s) : 7);
}

// Record words of a key (d = m = 128): K planes of 4 words, 4 sign words, n, gamma.
template <int K>
constexpr int key_words() { return 4 * K + 6; }

// qt rows in LDS carry 8 floats of padding after every 32 coordinates: the
// projection step's four quarter-row threads of a row then read different banks.
__device__ __host__ constexpr int qt_pad(int j) { return j + 8 * (j >> 5); }
constexpr int kQtRow = kD + 8 * (kD / 32);

// Query side of one (sequence, kv head): up to 4 query heads.
template <int K>
struct QueryLds {
  float qt[4][kQtRow];                 // qt[hh][qt_pad(j)]
  float pp[4][kM];
  int vt[4][Masks<K>::kMasks][kD];     // fixed-point values V per head, mask and coordinate
  float qstat[4][2];                   // per head: max |qt_j|, sum qt_j
  float pstat[kPWaves][4][2];          // per projection wave and head: max |p_i|, sum p_i
  float consts[4][4];                  // per head: delta_mse, delta_qjl, C_mse, C_qjl
  float coef[8];                       // a_P
  float cmax;                          // largest centroid
  i32x4 afrag[Masks<K>::kMfma * 64];
};

struct QuerySrc {
  const float* cent;                   // 2^K centroids
  const uint32_t* dbits;               // D as sign bits
  const _Float16* S;                   // [m][d]
  const void* q;
  int q_dtype;
  int64_t q_off;                       // element offset of the group's first query head
  int gq;                              // query heads of the group (1, 2 or 4)
  const float* R;                      // Haar codebooks: R = sqrt(d) Q [d][d] (dbits unused); else null
};

// Query-side loads, issued first: waves 0-3 take head `wave` (coordinates lane
// and lane + 64), the projection waves a quarter row of S each, thread 0.. the
// centroids.
template <int K>
struct QueryRegs {
  float q0 = 0.0f, q1 = 0.0f;
  uint32_t d0 = 0, d1 = 0;
  const float* R = nullptr;
  uint4 srow[4];
  float cv[1 << K];
};

template <int K>
__device__ inline void query_load(const QuerySrc& src, QueryRegs<K>& r, int tid, int wave, int lane) {
  if (wave < 4 && wave < src.gq) {
    const int64_t off = src.q_off + (int64_t)wave * kD + lane;
    r.q0 = load_elem(src.q, src.q_dtype, off);
    r.q1 = load_elem(src.q, src.q_dtype, off + 64);
    if (!src.R) {
      r.d0 = src.dbits[lane >> 5];
      r.d1 = src.dbits[2 + (lane >> 5)];
    }
  }
  r.R = src.R;
  if (wave < kPWaves) {
    const int prow = tid >> 2, qtr = tid & 3;
    const uint4* row = reinterpret_cast<const uint4*>(src.S + prow * kD + 32 * qtr);
#pragma unroll
    for (int v = 0; v < 4; ++v) r.srow[v] = row[v];
  }
  if (tid < Masks<K>::kPlaneMasks) {
#pragma unroll
    for (int v = 0; v < (1 << K); ++v) r.cv[v] = src.cent[v];
  }
}

struct NoStep {
  __device__ void operator()() const {}
};

// The query side from the loaded registers, in four barriers; on return
// s.afrag and s.consts are complete and visible to the workgroup.  `after1`
// runs on every thread right after the first barrier, once the query loads
// have landed (a caller issues its own memory traffic there, so that it does
// not queue in front of them).
// kBlock (threads) is a multiple of 128 and at least 64 * kPWaves.
template <int K, int kBlock, typename After1 = NoStep>
__device__ inline void query_build(QueryLds<K>& s, const QueryRegs<K>& r, int gq, int tid, int wave, int lane,
                                   After1 after1 = After1()) {
  using Mk = Masks<K>;
  constexpr int L = 1 << K;
  constexpr int NMF = Mk::kMfma;
  static_assert(kBlock % 128 == 0 && kBlock >= 64 * kPWaves, "workgroup shape");
  // (1) a_P = (1/L) sum_v c_v prod_{p in P} sigma_p(v); qt = H D q per head in
  //     registers (butterflies of span 1..32 across lanes, then 64 within the
  //     lane), with max |qt_j| and sum qt_j
  if (tid < Mk::kPlaneMasks) {
    const int sb = subset_bits<K>(tid);
    double acc = 0.0;
#pragma unroll
    for (int v = 0; v < L; ++v) {
      const int par = __popc(~v & sb) & 1;       // number of -1 factors
      acc += par ? -(double)r.cv[v] : (double)r.cv[v];
    }
    s.coef[tid] = (float)(acc / L);
    if (tid == 0) s.cmax = r.cv[L - 1];
  }
  if (r.R) {
    // Haar: qt = R q as a dense product.  The queries pass through s.pp (free
    // until step 2); threads 4i .. 4i+3 own row i of R, a quarter of it each,
    // all four heads, then a 4-lane reduction as in step 2.
    if (wave < 4) {
      s.pp[wave][lane] = r.q0;
      s.pp[wave][lane + 64] = r.q1;
    }
    const int row = tid >> 2, qtr = tid & 3;
    float4 rv[8];
    if (tid < 4 * kD) {
      const float4* rp = reinterpret_cast<const float4*>(r.R + row * kD + 32 * qtr);
#pragma unroll
      for (int v = 0; v < 8; ++v) rv[v] = rp[v];
    }
    __syncthreads();
    if (tid < 4 * kD) {
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float rr[4] = {rv[v].x, rv[v].y, rv[v].z, rv[v].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int hh = 0; hh < 4; ++hh) acc[hh] = fmaf(rr[e], s.pp[hh][32 * qtr + 4 * v + e], acc[hh]);
      }
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        acc[hh] += xor1_f32(acc[hh]);
        acc[hh] += xor2_f32(acc[hh]);
      }
      s.qt[qtr][qt_pad(row)] = acc[qtr];
    }
    __syncthreads();
    if (wave < 4) {
      const float y0 = s.qt[wave][qt_pad(lane)], y1 = s.qt[wave][qt_pad(lane + 64)];
      const float m1 = wave_max_uniform(fmaxf(fabsf(y0), fabsf(y1)));
      const float s1 = wave_sum_uniform(y0 + y1);
      if (lane == 0) {
        s.qstat[wave][0] = m1;
        s.qstat[wave][1] = s1;
      }
    }
  } else if (wave < 4) {
    float x0 = ((r.d0 >> (lane & 31)) & 1u) ? -r.q0 : r.q0;
    float x1 = ((r.d1 >> (lane & 31)) & 1u) ? -r.q1 : r.q1;
#pragma unroll
    for (int hs = 1; hs < 64; hs <<= 1) {
      // partners xor 1, 2, 8 by DPP and xor 32 by a permlane swap; xor 4 and 16
      // through the LDS crossbar
      float o0, o1;
      if (hs == 1) {
        o0 = xor1_f32(x0), o1 = xor1_f32(x1);
      } else if (hs == 2) {
        o0 = xor2_f32(x0), o1 = xor2_f32(x1);
      } else if (hs == 8) {
        o0 = xor8_f32(x0), o1 = xor8_f32(x1);
      } else if (hs == 32) {
        o0 = xor32_f32(x0, lane), o1 = xor32_f32(x1, lane);
      } else {
        o0 = __shfl_xor(x0, hs, 64), o1 = __shfl_xor(x1, hs, 64);
      }
      x0 = (lane & hs) ? o0 - x0 : x0 + o0;
      x1 = (lane & hs) ? o1 - x1 : x1 + o1;
    }
    const float y0 = x0 + x1, y1 = x0 - x1;
    s.qt[wave][qt_pad(lane)] = y0;
    s.qt[wave][qt_pad(lane + 64)] = y1;
    const float m1 = wave_max_uniform(fmaxf(fabsf(y0), fabsf(y1)));
    const float s1 = wave_sum_uniform(y0 + y1);
    if (lane == 0) {
      s.qstat[wave][0] = m1;
      s.qstat[wave][1] = s1;
    }
  }
  __syncthreads();
  after1();
  // (2) p = S qt / sqrt(d): threads 4i .. 4i+3 own row i, a quarter of it each,
  //     all four heads (qt read as float4, the quarters in different banks),
  //     then a 4-lane reduction; per wave, max |p_i| and sum p_i
  if (wave < kPWaves) {
    const int prow = tid >> 2, qtr = tid & 3;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t ww[4] = {r.srow[v].x, r.srow[v].y, r.srow[v].z, r.srow[v].w};
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const float4 qa = *reinterpret_cast<const float4*>(&s.qt[hh][qt_pad(32 * qtr + 8 * v)]);
        const float4 qb = *reinterpret_cast<const float4*>(&s.qt[hh][qt_pad(32 * qtr + 8 * v + 4)]);
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const h16x2 pr = __builtin_bit_cast(h16x2, ww[e]);
          acc[hh] = fmaf((float)pr[0], qv[2 * e], acc[hh]);
          acc[hh] = fmaf((float)pr[1], qv[2 * e + 1], acc[hh]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      acc[hh] += xor1_f32(acc[hh]);
      acc[hh] += xor2_f32(acc[hh]);
      acc[hh] *= 0.08838834764831845f;          // 1/sqrt(128)
    }
    s.pp[qtr][prow] = acc[qtr];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float pm = wave_max_uniform(fabsf(acc[hh]));
      const float ps = wave_sum_uniform(qtr == 0 ? acc[hh] : 0.0f);
      if (lane == 0) {
        s.pstat[wave][hh][0] = pm;
        s.pstat[wave][hh][1] = ps;
      }
    }
  }
  __syncthreads();
  // (3) per head, the value of one fixed-point unit (2^30 units for the largest
  //     |2 a_P qt_j| or |2 p_i|) and the constant terms; the fixed-point values
  //     V; then the A fragments.
  // A fragment of MFMA f = 2*w2 + g, lane l: row m = l%32, K = 16(l/32) + 4q + byte.
  // Lane half hl of MFMA (w2, g) carries list word 2*w2 + hl; bit (8*byte + 4g + q)
  // of that word.  Row m = 8 hh + 4 part + limb holds signed int8 limb `limb` of
  // the value (zero where the mask belongs to the other part): the value V of
  // coordinate j is 2 a_P qt_j (plane masks) or 2 p_j (sign mask) in units,
  // pre-divided by 2^(j mod 8) (-128 for j mod 8 == 7: the top bit of a byte),
  // and its signed base-256 digits are the bytes of V + 0x80808080, each minus 128.
  // Each V is computed once (step 3a, a table in LDS) and its four limbs read
  // from it (step 3b); a thread's fragment entries all share one row m (kBlock
  // is a multiple of 128).
  const auto unit_of = [&](int hh, int part) {
    float vm;
    if (part == 0) {
      float amax = 0.0f;
      for (int k = 0; k < Mk::kPlaneMasks; ++k) amax = fmaxf(amax, fabsf(s.coef[k]));
      vm = 2.0f * amax * s.qstat[hh][0];
    } else {
      float m2 = 0.0f;
      for (int w = 0; w < kPWaves; ++w) m2 = fmaxf(m2, s.pstat[w][hh][0]);
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
      v = s.cmax * s.qstat[hh][1];               // c_max * sum qt
    } else {
      v = 0.0f;
      for (int w = 0; w < kPWaves; ++w) v += s.pstat[w][hh][1];   // sum p
    }
    s.consts[hh][c] = v;
  }
  for (int e = tid; e < 4 * Mk::kMasks * kD; e += kBlock) {
    const int j = e % kD, mask = (e / kD) % Mk::kMasks, hh = e / (kD * Mk::kMasks);
    const bool is_sign_mask = mask == Mk::kPlaneMasks;
    int V = 0;
    if (hh < gq) {
      const float val = is_sign_mask ? 2.0f * s.pp[hh][j] : 2.0f * s.coef[mask] * s.qt[hh][qt_pad(j)];
      const int sh = j & 7;
      const double inv_div = sh == 7 ? -1.0 / 128.0 : 1.0 / (double)(1 << sh);
      V = (int)rint((double)val * (1.0 / (double)unit_of(hh, is_sign_mask ? 1 : 0)) * inv_div);
    }
    s.vt[hh][mask][j] = V;
  }
  __syncthreads();
  {
    const int m = (tid >> 2) & 31;
    const int hh = m >> 3, part = (m >> 2) & 1, limb = m & 3;
    for (int idx = tid; idx < NMF * 64 * 4; idx += kBlock) {
      const int q = idx & 3, ln = (idx >> 2) & 63, f = idx >> 8;
      const int w2 = f >> 1, g = f & 1;
      const int li = 2 * w2 + (ln >> 5);        // list word: mask li/4, word li%4
      const int mask = li >> 2, ww = li & 3;
      const bool is_sign_mask = mask == Mk::kPlaneMasks;
      uint32_t packed = 0;
      if (hh < gq && part == (is_sign_mask ? 1 : 0)) {
#pragma unroll
        for (int byt = 0; byt < 4; ++byt) {
          const int V = s.vt[hh][mask][32 * ww + 8 * byt + 4 * g + q];
          const uint32_t digit = (((uint32_t)V + 0x80808080u) >> (8 * limb)) & 0xFFu;
          packed |= (digit ^ 0x80u) << (8 * byt);
        }
      }
      reinterpret_cast<uint32_t*>(s.afrag)[(f * 64 + ln) * 4 + q] = packed;
    }
  }
  __syncthreads();
}

// Scores of one tile of 32 keys staged in LDS: `st` points at key `col` of the
// tile (its key_words<K>() words), h = lane / 32.  Returns the scores of query
// heads 2h and 2h+1 of the group for that key; heads past the group's are
// garbage and must not be stored.
template <int K>
__device__ inline void score_tile(const i32x4* A, const uint32_t* st, const float (*consts)[4], float scale, int h,
                                  float& s_a, float& s_b) {
  using Mk = Masks<K>;
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
  const float kqjl = kQjlConst / (float)kM;
  const float inv_d = 1.0f / (float)kD;
  // per-head constants stay in LDS (registers are the occupancy limit here)
  s_a = scale * ((nrm * inv_d) * (consts[ha][0] * mse_a - consts[ha][2]) +
                 kqjl * gam * (consts[ha][1] * qjl_a - consts[ha][3]));
  s_b = scale * ((nrm * inv_d) * (consts[hb][0] * mse_b - consts[hb][2]) +
                 kqjl * gam * (consts[hb][1] * qjl_b - consts[hb][3]));
}

}  // namespace sc128
}  // namespace tq
