// Device-side helpers shared by the libtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"
#include "tq_layout.h"

namespace tq {

// Arguments common to every kernel that reads a codebook array.
struct CodebookArgs {
  const uint8_t* cbs;
  int64_t stride;      // bytes between blobs
  int64_t n_cb;
  int d, bits, m, role, k, levels, rotation;
  uint32_t off_c, off_t, off_d, off_s;
  int plane_words, sign_words, rec_words;
};

inline CodebookArgs make_cb_args(const void* cbs, int64_t n_cb, const Layout& L) {
  CodebookArgs a;
  a.cbs = static_cast<const uint8_t*>(cbs);
  a.stride = L.total;
  a.n_cb = n_cb;
  a.d = L.d; a.bits = L.bits; a.m = L.m; a.role = L.role; a.k = L.k; a.levels = L.levels;
  a.rotation = L.rotation;
  a.off_c = L.off_c; a.off_t = L.off_t; a.off_d = L.off_d; a.off_s = L.off_s;
  a.plane_words = L.plane_words; a.sign_words = L.sign_words; a.rec_words = L.rec_words;
  return a;
}

__device__ inline const uint8_t* blob_of(const CodebookArgs& a, int64_t g) {
  return a.cbs + (g % a.n_cb) * a.stride;
}

// True when the blob header disagrees with the call's parameters.
__device__ inline bool blob_mismatch(const CodebookArgs& a, const uint8_t* blob) {
  const BlobHeader* h = reinterpret_cast<const BlobHeader*>(blob);
  return h->magic != kBlobMagic || h->version != kBlobVersion || h->head_dim != a.d ||
         h->bits != a.bits || h->role != a.role || h->projections != a.m || (int)h->rotation != a.rotation;
}

// Optional channel map of a split head vector: coordinate j of group g's part
// is channel map[g*stride + off + j] of the full row (of `full` channels).
// Without a map coordinate j is channel j.  An entry outside [0, full) is
// reported in the status word and replaced by channel 0.
struct ChannelMap {
  const int32_t* map;
  int64_t stride;
  int off;
  int full;
  __device__ inline int channel(int64_t g, int j, int32_t* status) const {
    if (!map) return j;
    int c = map[g * stride + off + j];
    if ((unsigned)c >= (unsigned)full) {
      if (status) atomicOr(status, TQ_STATUS_BAD_CHANNEL);
      c = 0;
    }
    return c;
  }
};

__device__ inline float bf16_bits_to_float(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ inline float load_elem(const void* x, int dtype, int64_t off) {
  if (dtype == 1) {
    return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(x)[off]);
  } else if (dtype == 2) {
    return (float)reinterpret_cast<const _Float16*>(x)[off];
  }
  return reinterpret_cast<const float*>(x)[off];
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Lane exchanges without LDS: DPP within a 16-lane row (xor 1 and xor 2 by
// quad permutation, xor 8 by a rotation of the row by 8), and across the two
// halves of the wave (xor 32) by a permlane swap.
template <int C>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), C, 0xF, 0xF, true));
}
__device__ inline float xor1_f32(float v) { return dpp_f32<0xB1>(v); }
__device__ inline float xor2_f32(float v) { return dpp_f32<0x4E>(v); }
__device__ inline float xor8_f32(float v) { return dpp_f32<0x128>(v); }
__device__ inline float xor32_f32(float v, int lane) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(lane < 32 ? p[1] : p[0]);
}

// Sum and maximum over the 64 lanes, the result uniform: within each 16-lane
// row by DPP (quad permutations, then the half-row and row mirrors), then row 0
// into row 1 and row 2 into row 3 (row broadcast of lane 15), then row 1 into
// rows 2-3 (broadcast of lane 31); lane 63 holds the total.
__device__ inline float wave_sum_uniform(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ inline float wave_max_uniform(float v) {
  constexpr int kNegInf = (int)0xFF800000u;
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// z = u/|x| (float64) rounded toward +infinity.  For every float32 threshold t,
// t < z_up exactly when t < z, the comparison the quantizer's definition asks
// for: if z > t then z_up >= z > t; if z <= t then z_up <= t, because t is a
// float32 value at or above z and z_up is the least such value.
__device__ inline float z_up(double u, double nrm) { return nrm > 0.0 ? __double2float_ru(u / nrm) : 0.0f; }

// Number of thresholds strictly below z (lower_bound over t[0 .. L-2]).
__device__ inline int quantize_index(const float* t, int levels, float z) {
  int lo = 0, n = levels - 1;
  while (n > 0) {
    int half = n >> 1;
    if (t[lo + half] < z) {
      lo += half + 1;
      n -= half + 1;
    } else {
      n = half;
    }
  }
  return lo;
}

constexpr float kQjlConst = 1.2533141373155002512f;  // sqrt(pi/2)

// Word 3 of a raw buffer resource on gfx9-family chips (32-bit data format; no
// swizzle, no stride): offsets at or past the resource size read 0 and drop stores.
constexpr int kRsrcWord3 = 0x00020000;

}  // namespace tq
