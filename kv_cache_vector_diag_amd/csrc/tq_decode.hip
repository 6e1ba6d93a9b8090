// Value decode for the Walsh-Hadamard codec at head_dim 32, 64, 128 or 256,
// any value width up to 8 bits (page "turboquant-plus-rs 0.1.0 README",
// "Architecture": the MSE reconstruction undoes the rotation of the looked-up
// centroids, x^ = (n32 / d) D H c[idx], n32 the stored norm, H the unnormalised
// Walsh-Hadamard matrix, D the random sign diagonal).
//
// A vector takes d/32 lanes; lane x holds rotated coordinates 32x .. 32x + 31,
// i.e. plane word x of every bit plane.
//  * indices: bytes of the k plane words regrouped by byte permutes into one
//    64-bit word per 8 coordinates (byte p = plane p), then an 8x8 bit transpose
//    (byte e = index of coordinate e); centroids from a wave-private LDS table;
//  * H c in float32: the five coordinate bits by butterflies in registers, the
//    lane bits by butterflies whose partner comes through DPP (xor 1 and 2 by
//    quad permutation; at d = 256, xor 7 by the half-row mirror instead of xor
//    4).  Lane x takes the sum or the difference by a fixed linear role of its
//    lane bits, after which it holds output block a(x) (a = identity for up to
//    4 lanes, a fixed relabelling of the three lane bits for 8);
//  * the scale n32/d and the signs of D (a wave-private table of sign bits per
//    coordinate), then the output goes through LDS, half a wave's lanes at a
//    time, so that every global store instruction writes 1 KiB of consecutive
//    floats; the stores are non-temporal (the output is written once and not
//    read back by this kernel).
// A wave decodes 64/(d/32) consecutive vectors per step and prefetches the
// records of its next step; a workgroup of four waves walks one contiguous
// range of vectors.  The wave's two table slots hold the codebooks of the
// group of its first vector and of the next group, so a step may straddle one
// group boundary (needs N >= 64/(d/32)).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

struct DecodeWHArgs {
  CodebookArgs cb;
  const uint32_t* rec;   // [G][N][k d/32 + 1]
  uint32_t G, N, total;  // total = G N
  uint32_t span;         // vectors per workgroup (a multiple of a workgroup step)
  float* out;            // [G][N][d]
  int32_t* status;
};

using LdsF = const float __attribute__((address_space(3)))*;
typedef float F4 __attribute__((ext_vector_type(4)));

__device__ inline int parity(uint32_t v) { return __popc(v) & 1; }

template <int C>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), C, 0xF, 0xF, true));
}

// 8x8 bit transpose of the 64-bit word (lo = bytes 0-3, hi = bytes 4-7): bit p
// of byte j moves to bit j of byte p.
__device__ inline void transpose8x8(uint32_t& lo, uint32_t& hi) {
  uint32_t t;
  t = (lo ^ (lo >> 7)) & 0x00AA00AAu; lo ^= t | (t << 7);
  t = (hi ^ (hi >> 7)) & 0x00AA00AAu; hi ^= t | (t << 7);
  t = (lo ^ (lo >> 14)) & 0x0000CCCCu; lo ^= t | (t << 14);
  t = (hi ^ (hi >> 14)) & 0x0000CCCCu; hi ^= t | (t << 14);
  t = (lo ^ (hi << 4)) & 0xF0F0F0F0u;
  lo ^= t;
  hi ^= t >> 4;
}

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// WIDE: value width above 4 bits (planes 4..7 present).
template <int D, bool WIDE>
__global__ __launch_bounds__(kBlock) void decode_wh_kernel(DecodeWHArgs a) {
  constexpr int L = D / 32;          // lanes per vector
  constexpr int VPW = 64 / L;        // vectors per wave step
  constexpr int VPB = kWaves * VPW;  // vectors per workgroup step
  __shared__ float s_cent[kWaves][2][256];
  __shared__ uint32_t s_sign[kWaves][2][D];
  __shared__ float4 s_stage[kWaves][256];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = lane & (L - 1);
  const int blk = L <= 4 ? x : (parity(x & 5) | parity(x & 6) << 1 | parity(x & 7) << 2);
  const float sg0 = (L <= 4 ? (x & 1) : parity(x & 5)) ? -1.0f : 1.0f;
  const float sg1 = (L <= 4 ? (x & 2) : parity(x & 6)) ? -1.0f : 1.0f;
  const float sg2 = parity(x & 4) ? -1.0f : 1.0f;
  const int k = a.cb.k;
  const int RW = k * L + 1;
  const uint32_t n_cb = (uint32_t)a.cb.n_cb;
  constexpr float kInvD = 1.0f / (float)D;

  const uint32_t start = blockIdx.x * a.span;
  const uint32_t end = min(start + a.span, a.total);
  uint32_t vw = start + wave * VPW;
  if (vw >= end) return;
  // group of the wave's first vector, the next group's first vector, the
  // codebook of that group
  uint32_t gf = vw / a.N;
  uint32_t bnd = (gf + 1) * a.N;
  uint32_t cbf = gf % n_cb;
  uint32_t loaded = 0xFFFFFFFFu;   // codebook of slot 0 in the tables

  float* cent = &s_cent[wave][0][0];
  uint32_t* sign = &s_sign[wave][0][0];
  float4* stage = s_stage[wave];
  // the 32 output floats of this lane are floats 32 piece .. 32 piece + 31 of
  // the wave's step
  const int piece = (lane & ~(L - 1)) + blk;

  uint32_t w[8];
  uint32_t nbits;
  auto load_rec = [&](uint32_t v) {
    const uint32_t* r = a.rec + (uint64_t)v * RW;
#pragma unroll
    for (int p = 0; p < 8; ++p) w[p] = (p < (WIDE ? 8 : 4) && p < k) ? r[p * L + x] : 0u;
    nbits = r[k * L];
  };
  load_rec(min(vw + (uint32_t)(lane / L), end - 1));

  for (; vw < end; vw += VPB) {
    while (vw >= bnd) {
      ++gf;
      bnd += a.N;
      if (++cbf == n_cb) cbf = 0;
    }
    if (cbf != loaded) {
      // tables of the codebooks of groups gf and gf + 1 (the codebook pair
      // repeats whenever the first one does)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (gf + s < a.G) {
          const uint32_t c = s == 0 ? cbf : (cbf + 1 == n_cb ? 0 : cbf + 1);
          const uint8_t* blob = a.cb.cbs + (int64_t)c * a.cb.stride;
          const float* cc = reinterpret_cast<const float*>(blob + a.cb.off_c);
          const uint32_t* db = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d);
          for (int i = lane; i < a.cb.levels; i += 64) cent[s * 256 + i] = cc[i];
#pragma unroll
          for (int j = lane; j < D; j += 64) sign[s * D + j] = ((db[j >> 5] >> (j & 31)) & 1u) << 31;
          if (lane == 0 && a.status && blob_mismatch(a.cb, blob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
        }
      }
      loaded = cbf;
      wave_sync_lds();
    }
    const uint32_t v = vw + (uint32_t)(lane / L);
    const int slot = v >= bnd ? 1 : 0;
    // this step's records; the next step's are loaded meanwhile
    uint32_t c[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) c[p] = w[p];
    const float n32 = __uint_as_float(nbits);
    if (vw + VPB < end) load_rec(min(v + (uint32_t)VPB, end - 1));

    // ---- indices of coordinates 32x + 8q + e (byte e of word pair q)
    float u[32];
    const float* tab = cent + slot * 256;
    {
      const uint32_t t01a = __builtin_amdgcn_perm(c[1], c[0], 0x05010400u);
      const uint32_t t01b = __builtin_amdgcn_perm(c[1], c[0], 0x07030602u);
      const uint32_t t23a = __builtin_amdgcn_perm(c[3], c[2], 0x05010400u);
      const uint32_t t23b = __builtin_amdgcn_perm(c[3], c[2], 0x07030602u);
      uint32_t lo[4] = {__builtin_amdgcn_perm(t23a, t01a, 0x05040100u), __builtin_amdgcn_perm(t23a, t01a, 0x07060302u),
                        __builtin_amdgcn_perm(t23b, t01b, 0x05040100u), __builtin_amdgcn_perm(t23b, t01b, 0x07060302u)};
      uint32_t hi[4] = {0u, 0u, 0u, 0u};
      if (WIDE) {
        const uint32_t t45a = __builtin_amdgcn_perm(c[5], c[4], 0x05010400u);
        const uint32_t t45b = __builtin_amdgcn_perm(c[5], c[4], 0x07030602u);
        const uint32_t t67a = __builtin_amdgcn_perm(c[7], c[6], 0x05010400u);
        const uint32_t t67b = __builtin_amdgcn_perm(c[7], c[6], 0x07030602u);
        hi[0] = __builtin_amdgcn_perm(t67a, t45a, 0x05040100u);
        hi[1] = __builtin_amdgcn_perm(t67a, t45a, 0x07060302u);
        hi[2] = __builtin_amdgcn_perm(t67b, t45b, 0x05040100u);
        hi[3] = __builtin_amdgcn_perm(t67b, t45b, 0x07060302u);
      }
      // LDS byte address of entry idx: base + 4 idx.  Up to 4 bits the whole word
      // is scaled once (4 idx still fits a byte), and each entry is one add of a
      // selected byte.
      const uint32_t tbase = (uint32_t)(uintptr_t)(LdsF)tab;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        transpose8x8(lo[q], hi[q]);
        if (!WIDE) {
          lo[q] <<= 2;
          hi[q] <<= 2;
          asm volatile("" : "+v"(lo[q]), "+v"(hi[q]));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t b = ((e < 4 ? lo[q] : hi[q]) >> (8 * (e & 3))) & 0xFFu;
          const uint32_t addr = WIDE ? tbase + 4u * b : tbase + b;
          u[8 * q + e] = *(LdsF)(uintptr_t)addr;
        }
      }
    }
    // ---- H: coordinate bits in registers, then lane bits
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
      for (int e = 0; e < 32; ++e)
        if ((e & h) == 0) {
          const float x0 = u[e], x1 = u[e + h];
          u[e] = x0 + x1;
          u[e + h] = x0 - x1;
        }
    if (L >= 2) {
#pragma unroll
      for (int e = 0; e < 32; ++e) u[e] = fmaf(u[e], sg0, dpp<0xB1>(u[e]));
    }
    if (L >= 4) {
#pragma unroll
      for (int e = 0; e < 32; ++e) u[e] = fmaf(u[e], sg1, dpp<0x4E>(u[e]));
    }
    if (L >= 8) {
#pragma unroll
      for (int e = 0; e < 32; ++e) u[e] = fmaf(u[e], sg2, dpp<0x141>(u[e]));
    }
    // ---- scale, signs of output coordinates 32 blk + e, stores through LDS
    const float scale = n32 * kInvD;
    const uint4* sg = reinterpret_cast<const uint4*>(sign + slot * D + 32 * blk);
    float* obase = a.out + (uint64_t)vw * D;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // lanes 32 half .. 32 half + 31 hold the output of 1024 consecutive floats
      if ((lane >> 5) == half) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint4 s4 = sg[q];
          const int e = 4 * q;
          float4 t;
          t.x = __uint_as_float(__float_as_uint(u[e] * scale) ^ s4.x);
          t.y = __uint_as_float(__float_as_uint(u[e + 1] * scale) ^ s4.y);
          t.z = __uint_as_float(__float_as_uint(u[e + 2] * scale) ^ s4.z);
          t.w = __uint_as_float(__float_as_uint(u[e + 3] * scale) ^ s4.w);
          stage[8 * (piece & 31) + (q ^ (piece & 7))] = t;
        }
      }
      wave_sync_lds();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = 64 * i + lane;        // float4 f of the 1024 floats: piece f/8, eighth f%8
        const int P = f >> 3;
        const float4 t = stage[8 * P + ((f & 7) ^ (P & 7))];
        if (vw + (uint32_t)((P + 32 * half) / L) < end) {
          const F4 tv = {t.x, t.y, t.z, t.w};
          __builtin_nontemporal_store(tv, reinterpret_cast<F4*>(obase + 1024 * half + 4 * f));
        }
      }
      wave_sync_lds();
    }
  }
}

template <int D, bool WIDE>
int launch_wh(DecodeWHArgs a, hipStream_t s) {
  constexpr int VPB = kWaves * (64 / (D / 32));
  const uint32_t steps = (a.total + VPB - 1) / VPB;
  // up to 16 workgroups per compute unit, each on one contiguous range
  uint32_t blocks = steps < 4096 ? steps : 4096;
  const uint32_t steps_per = (steps + blocks - 1) / blocks;
  a.span = steps_per * VPB;
  blocks = (a.total + a.span - 1) / a.span;
  hipLaunchKernelGGL((decode_wh_kernel<D, WIDE>), dim3(blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : TQ_ERR_HIP;
}

template <int D>
int launch_d(const DecodeWHArgs& a, hipStream_t s) {
  return a.cb.k > 4 ? launch_wh<D, true>(a, s) : launch_wh<D, false>(a, s);
}

}  // namespace

bool decode_wh_supported(const CodebookArgs& cb, int64_t G, int64_t N, const void* out) {
  if (cb.rotation != kRotHadamard || cb.role != TQ_ROLE_VALUE || cb.k > 8) return false;
  if (cb.d != 32 && cb.d != 64 && cb.d != 128 && cb.d != 256) return false;
  const int64_t vpw = 64 / (cb.d / 32);
  return N >= vpw && G * N < (int64_t(1) << 31) && cb.n_cb < (int64_t(1) << 31) &&
         (reinterpret_cast<uintptr_t>(out) & 15) == 0;
}

int launch_decode_wh(const CodebookArgs& cb, const uint32_t* rec, int64_t G, int64_t N, float* out,
                     int32_t* status, hipStream_t s) {
  if (G * N == 0) return 0;
  DecodeWHArgs a;
  a.cb = cb;
  a.rec = rec;
  a.G = (uint32_t)G;
  a.N = (uint32_t)N;
  a.total = (uint32_t)(G * N);
  a.span = 0;
  a.out = out;
  a.status = status;
  switch (cb.d) {
    case 32: return launch_d<32>(a, s);
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    case 256: return launch_d<256>(a, s);
  }
  return TQ_ERR_BAD_DIMENSION;
}

}  // namespace tq
