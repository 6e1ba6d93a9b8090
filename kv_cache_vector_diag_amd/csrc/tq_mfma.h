// Device helpers shared by the MFMA kernels of libtq (gfx950, wave64): vector
// types, the 32x32 MFMA result layout, and register-only ALU sequences of the
// quantizer, pinned in inline assembly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {
namespace mf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t h_sign(int i, int j) { return __popc(i & j) & 1; }

template <typename V>
__device__ inline V as(u32x4 v) {
  return __builtin_bit_cast(V, v);
}

// Row rho of a 32-row result tile lands in lane half (rho>>2)&1, register
// 4(rho>>3) + (rho&3).  Tile rows are permuted so that lane half h holds the
// 16 consecutive indices 16h .. 16h+15 of its tile in registers 0..15.
__device__ inline int tile_row_index(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

// Coordinate fed by B-operand element e (0..7) of lane half h in projection
// K-chunk c = 2M + p: register 8p + e of tile M, i.e. coordinate 32M + 16h + 8p + e.
__device__ inline int qjl_coord(int c, int h, int e) {
  return 32 * (c >> 1) + 16 * h + 8 * (c & 1) + e;
}

// x0^2 + x1^2 of a packed pair, widened to fp64.
__device__ inline double pair_sumsq_bf16(uint32_t w) {
  s16x2 v = __builtin_bit_cast(s16x2, w);
  return (double)__builtin_amdgcn_fdot2_f32_bf16(v, v, 0.0f, false);
}

// acc + x0^2 + x1^2 of a packed pair (float32, the products exact).
__device__ inline float sumsq2_bf16(uint32_t w, float acc) {
  s16x2 v = __builtin_bit_cast(s16x2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

// Sum of squares of four packed bf16 pairs in float64, exactly: for chunks
// whose float32 pair sums may have lost squares to underflow (|x| < 2^-63).
__device__ inline double sumsq8_bf16_f64(u32x4 w) {
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const double lo = (double)__uint_as_float(w[q] << 16), hi = (double)__uint_as_float(w[q] & 0xFFFF0000u);
    s = fma(lo, lo, s);
    s = fma(hi, hi, s);
  }
  return s;
}

__device__ inline float sumsq2_f16(uint32_t w, float acc) {
  f16x2 v = __builtin_bit_cast(f16x2, w);
  return __builtin_amdgcn_fdot2(v, v, acc, false);
}

// 2 acc + (sign bit of v): shifts the sign bit of v in at bit 0.
__device__ inline uint32_t neg_bit(uint32_t acc, float v) {
  return __builtin_amdgcn_alignbit(acc, __float_as_uint(v), 31);
}


// ---- per-element ALU sequences pinned in inline assembly (register-only,
// no memory access).  Each helper documents the exact operation.

// Scaled two-term half-precision split of a pair: hi = f16(w*sc) (round to
// nearest even), lo = f16(w*sc - hi), packed two per word (element 0 in the low
// half).  w*sc is exact for the power-of-two sc used here, and w*sc - hi is
// exact in fp32, so hi + lo carries 22 significant bits of w*sc.
__device__ inline void split_f16x2(float w0, float w1, float sc, uint32_t& hi, uint32_t& lo) {
  asm("v_fma_mixlo_f16 %[h], %[w0], %[sc], 0\n\t"
      "v_fma_mixhi_f16 %[h], %[w1], %[sc], 0\n\t"
      "v_fma_mixlo_f16 %[l], %[w0], %[sc], -%[h] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %[l], %[w1], %[sc], -%[h] op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : [h] "=&v"(hi), [l] "=&v"(lo)
      : [w0] "v"(w0), [w1] "v"(w1), [sc] "v"(sc));
}

// Squares of a split residual pair, in the scaled domain: hh += hi.hi and
// hl += hi.lo over both halves (binary16 products are exact in float32), so
// that (w sc)^2 = hi^2 + 2 hi lo + lo^2 is summed as hh + 2 hl (lo^2 is below
// 2^-22 of it).  Unlike w^2 it cannot underflow for tiny inputs.
__device__ inline void split_sumsq(uint32_t hi, uint32_t lo, float& hh, float& hl) {
  const f16x2 h = __builtin_bit_cast(f16x2, hi), l = __builtin_bit_cast(f16x2, lo);
  hh = __builtin_amdgcn_fdot2(h, h, hh, false);
  hl = __builtin_amdgcn_fdot2(h, l, hl, false);
}

// First threshold step of the quantizer: above = |u| > tn; acc = 2*acc + above;
// mag = above ? c1 : c0.
__device__ inline float thr_first(uint32_t& acc, float u, float tn, float c0, float c1) {
  uint64_t m, c;
  float mag;
  asm("v_cmp_gt_f32_e64 %[m], |%[u]|, %[t]\n\t"
      "v_addc_co_u32_e64 %[acc], %[c], %[acc], %[acc], %[m]\n\t"
      "v_cndmask_b32_e64 %[mag], %[c0], %[c1], %[m]"
      : [acc] "+v"(acc), [mag] "=v"(mag), [m] "=&s"(m), [c] "=&s"(c)
      : [u] "v"(u), [t] "v"(tn), [c0] "v"(c0), [c1] "v"(c1));
  return mag;
}

// Further threshold steps: above = |u| > tn; acc = 2*acc + above; mag = above ? cnext : mag.
__device__ inline void thr_step(uint32_t& acc, float& mag, float u, float tn, float cnext) {
  uint64_t m, c;
  asm("v_cmp_gt_f32_e64 %[m], |%[u]|, %[t]\n\t"
      "v_addc_co_u32_e64 %[acc], %[c], %[acc], %[acc], %[m]\n\t"
      "v_cndmask_b32_e64 %[mag], %[mag], %[cn], %[m]"
      : [acc] "+v"(acc), [mag] "+v"(mag), [m] "=&s"(m), [c] "=&s"(c)
      : [u] "v"(u), [t] "v"(tn), [cn] "v"(cnext));
}

// Sign half: pos = u > 0 as the top bit of (0 - bits(u)) (exact for every u
// except -0, which the MFMA never produces from a +0 accumulator); acc = 2*acc + pos;
// nsg = pos ? -n : n.
__device__ inline void pos_step(uint32_t& acc, float& nsg, float u, uint32_t nbits, uint32_t signmask) {
  uint32_t t;
  asm("v_sub_u32 %[t], 0, %[u]\n\t"
      "v_alignbit_b32 %[acc], %[acc], %[t], 31\n\t"
      "v_and_or_b32 %[nsg], %[t], %[sm], %[nb]"
      : [acc] "+v"(acc), [nsg] "=&v"(nsg), [t] "=&v"(t)
      : [u] "v"(u), [sm] "s"(signmask), [nb] "v"(nbits));
}

// Value quantizer step of a binary search: above = |u| > t; acc = 2*acc + above;
// returns the lane mask of `above` for choosing the next threshold.
__device__ inline uint64_t thr_bit(uint32_t& acc, float u, float t) {
  uint64_t m, c;
  asm("v_cmp_gt_f32_e64 %[m], |%[u]|, %[t]\n\t"
      "v_addc_co_u32_e64 %[acc], %[c], %[acc], %[acc], %[m]"
      : [acc] "+v"(acc), [m] "=&s"(m), [c] "=&s"(c)
      : [u] "v"(u), [t] "v"(t));
  return m;
}

// m ? if_set : if_clear, per lane, for a mask from thr_bit.
__device__ inline float sel_mask(uint64_t m, float if_set, float if_clear) {
  float r;
  asm("v_cndmask_b32_e64 %[r], %[b], %[a], %[m]" : [r] "=v"(r) : [a] "v"(if_set), [b] "v"(if_clear), [m] "s"(m));
  return r;
}

// Sign half without the signed norm: pos = u > 0 (top bit of 0 - bits(u), as in
// pos_step); acc = 2*acc + pos.
__device__ inline void pos_bit(uint32_t& acc, float u) {
  uint32_t t;
  asm("v_sub_u32 %[t], 0, %[u]\n\t"
      "v_alignbit_b32 %[acc], %[acc], %[t], 31"
      : [acc] "+v"(acc), [t] "=&v"(t)
      : [u] "v"(u));
}

}  // namespace mf
}  // namespace tq
