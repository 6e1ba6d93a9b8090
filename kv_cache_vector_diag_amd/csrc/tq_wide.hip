// Encode at head_dim 256 with wide codebooks (Lloyd-Max indices of up to 8
// bits: 8-bit values, keys of up to 9 bits) on gfx950 (page "turboquant-plus-rs
// 0.1.0 README", "Architecture": Walsh-Hadamard rotation with random signs,
// per-coordinate Lloyd-Max codes, and for keys the QJL signs of a Gaussian
// projection of the residual; record layout as in tq.h).
//
// A workgroup of 16 waves owns a range of 32-vector tiles of one group.
//  * Encoder waves (all 16 for values, waves 0-7 for keys) take 4 vectors
//    each, 16 lanes per vector and 16 coordinates per lane, in float64:
//    - u = H(D x): the four coordinate bits held in registers by plain
//      butterflies; the four held across the 16 lanes by butterflies whose
//      partner comes from a DPP permutation (xor 1, xor 2, xor 8 within the
//      row, mirror within the half row).  Their partners are xor masks
//      1, 2, 8, 7 rather than 1, 2, 4, 8, so each lane takes the sum or the
//      difference by a fixed linear role (parity of lane & 5, 6, 8, 4) and
//      ends up holding block a(lane) = (parity(l&5), parity(l&6), parity(l&7),
//      parity(l&8)) of u: coordinates 16 a + e in register e.
//    - idx = #{t_i < z}, z = u/|x|: v = u * (1/|x|) in float64; cell =
//      floor(128 v + 2048) indexes an LDS table with the count L of
//      thresholds below the cell's left edge; idx = L + [t_L < v].  One
//      comparison is enough because the thresholds, float32 values, lie more
//      than a cell width (1/128) apart, so a cell holds at most one of them,
//      and v carries float64 accuracy, so the cell found is the cell of z
//      except within ~1e-15 of an edge, where the count still agrees (both the
//      edges and the thresholds are dyadic).  A codebook that breaks the
//      spacing is reported as TQ_STATUS_BAD_BLOB.
//    - bit planes: the 16 indices of a lane, bytes in two 64-bit words, go
//      through an 8x8 bit transpose; byte p is then the lane's 16-bit share of
//      plane p, stored as a half word.
//    - keys: residual w = u - n32 c[idx] and gamma in float64; w scaled by a
//      power of two and split into two binary16 terms (22 bits), staged in LDS
//      as MFMA B operands.
//  * Projector waves (keys: waves 8-15) hold rows 32 p .. 32 p + 31 of S in
//    registers (the A operands of all 16 K steps) and compute the signs of
//    S w for the previous tile, C[32 projections][32 vectors] with
//    v_mfma_f32_32x32x16_f16 over the hi and lo terms, while the encoders work
//    on the next tile (double-buffered LDS, one barrier per tile).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

using namespace mf;

constexpr int kD = 256;
constexpr int kThreads = 1024;
constexpr int kEncKey = 8;                 // encoder waves of the key kernel
constexpr int kTileVec = 32;               // vectors of a key tile (MFMA N)
constexpr int kCells = 4097;               // z in [-16, 16] (|z| <= sqrt(256)) at 1/128
constexpr int kChunkPad = 33;              // LDS B-operand row: 32 vectors + 1 (banks)

// LDS carve-up (bytes).
constexpr int kOffLut = 0;                                   // uint8 [kCells]
constexpr int kOffTt = 4112;                                 // double [257]: t_0 .. t_{L-2}, +inf
constexpr int kOffCc = kOffTt + 2064;                        // double [256]: centroids
constexpr int kOffR = kOffCc + 2048;                         // uint4 [2][2][32][kChunkPad]
constexpr int kRBytes = 2 * 2 * 32 * kChunkPad * 16;
constexpr int kLdsKey = kOffR + kRBytes;
constexpr int kLdsValue = kOffCc;

struct WideArgs {
  CodebookArgs cb;
  const void* x;
  int64_t G, N, sx_g, sx_n;
  uint32_t* rec;
  int32_t* status;
  int64_t tiles;             // tiles per group
  int64_t tiles_per_block, blocks_per_group;
};

__device__ inline int parity(int v) { return __popc(v) & 1; }

// Partner value of a float64 across lanes of a 16-lane row (DPP control `C`).
template <int C>
__device__ inline double dpp64(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), C, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), C, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppXor8 = 0x128;   // row_ror:8
constexpr int kDppXor7 = 0x141;   // row_half_mirror

// Sum over the 16 lanes of a row.
__device__ inline double row_sum16(double v) {
  v += dpp64<kDppXor1>(v);
  v += dpp64<kDppXor2>(v);
  v += dpp64<kDppXor8>(v);
  v += dpp64<kDppXor7>(v);
  return v;
}

// 8x8 bit transpose of the 64-bit word (lo, hi): bit p of byte j moves to bit
// j of byte p (three block-swap steps of 1, 2 and 4 bits).
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

// 2^(14 - floor(log2 |w|)) as a float32 power of two (1 for |w| = 0).
__device__ inline float residual_scale(double wn) {
  const float f = (float)wn;
  if (!(f > 0.0f) || !(f < 3.0e38f)) return 1.0f;
  const int e = (int)((__float_as_uint(f) >> 23) & 0xFFu) - 127;
  int se = 14 - (e < -126 ? -126 : e);
  se = se > 127 ? 127 : se;
  return __uint_as_float((uint32_t)(se + 127) << 23);
}

template <int DT, bool KEY>
__global__ __launch_bounds__(kThreads) void encode_wide_kernel(WideArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* lut = smem + kOffLut;
  double* tt = reinterpret_cast<double*>(smem + kOffTt);
  double* cc = reinterpret_cast<double*>(smem + kOffCc);
  uint4* rbuf = reinterpret_cast<uint4*>(smem + kOffR);

  constexpr int kEnc = KEY ? kEncKey : kThreads / 64;   // encoder waves
  constexpr int kStepVec = 4 * kEnc;                     // vectors per step
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.x / a.blocks_per_group;
  const int64_t tile0 = (blockIdx.x % a.blocks_per_group) * a.tiles_per_block;
  const int64_t tile_end = min(tile0 + a.tiles_per_block, a.tiles);
  const int ntiles = (int)(tile_end - tile0);
  const int k = a.cb.k, levels = a.cb.levels, W = a.cb.plane_words, RW = a.cb.rec_words;
  const int n_off = k * W + (KEY ? a.cb.sign_words : 0);
  const uint8_t* blob = blob_of(a.cb, g);

  // ---- codebook tables
  if (tid == 0 && a.status && blob_mismatch(a.cb, blob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  {
    const float* tsrc = reinterpret_cast<const float*>(blob + a.cb.off_t);
    const float* csrc = reinterpret_cast<const float*>(blob + a.cb.off_c);
    for (int i = tid; i < levels; i += kThreads) {
      tt[i] = i < levels - 1 ? (double)tsrc[i] : __longlong_as_double(0x7FF0000000000000ll);
      if (KEY) cc[i] = (double)csrc[i];
    }
  }
  __syncthreads();
  for (int c = tid; c < kCells; c += kThreads) {
    // L = #{t_i < (c - 2048) / 128} over t_0 .. t_{levels-2} (sorted)
    const double edge = ((double)c - 2048.0) * (1.0 / 128.0);
    int lo = 0, n = levels - 1;
    while (n > 0) {
      const int half = n >> 1;
      if (tt[lo + half] < edge) {
        lo += half + 1;
        n -= half + 1;
      } else {
        n = half;
      }
    }
    lut[c] = (uint8_t)lo;
  }
  if (tid + 1 < levels - 1 && !(tt[tid + 1] - tt[tid] > 1.0 / 128.0) && a.status)
    atomicOr(a.status, TQ_STATUS_BAD_BLOB);   // thresholds closer than a cell
  __syncthreads();

  // records of this group: words past the end are dropped
  const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
      a.rec + g * a.N * RW, 0, (int)(a.N * RW * 4), kRsrcWord3);

  if (!KEY || wave < kEncKey) {
    // ================= encoder =================
    const int x16 = lane & 15, vg = lane >> 4;
    const int blk = parity(x16 & 5) | parity(x16 & 6) << 1 | parity(x16 & 7) << 2 | parity(x16 & 8) << 3;
    // D signs of input coordinates 16 x16 .. 16 x16 + 15
    const uint32_t dw = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d)[x16 >> 1] >> (16 * (x16 & 1));
    constexpr int ES = DT == 0 ? 4 : 2;                   // element bytes
    constexpr int NR = 16 * ES / 16;                      // uint4 loads per lane
    const int64_t rows_bytes = (a.N - 1) * a.sx_n * ES + kD * ES;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(a.x) + g * a.sx_g * ES), 0, (int)rows_bytes, kRsrcWord3);
    const int vec_in_step = 4 * wave + vg;
    const auto load_in = [&](int i, u32x4* raw) {
      // tokens past N read zeros (offsets past the resource)
      const int64_t t = (tile0 + i) * kStepVec + vec_in_step;
      const uint32_t off = t < a.N ? (uint32_t)(t * a.sx_n * ES) + (uint32_t)(16 * ES * x16) : 0x80000000u;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        raw[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, off + 16u * r, 0, 0));
    };
    // float32 rows are loaded in the step that uses them (a prefetch would
    // double their 16 registers); 2-byte rows one step ahead
    constexpr bool kAhead = DT != 0;
    u32x4 raw[NR];
    if (kAhead) load_in(0, raw);

    for (int i = 0; i <= ntiles; ++i) {
      if (i < ntiles) {
        u32x4 nxt[NR];
        if (kAhead)
          load_in(i + 1 < ntiles ? i + 1 : i, nxt);   // the last step re-reads itself
        else
          load_in(i, raw);
        const int64_t t = (tile0 + i) * kStepVec + vec_in_step;
        // ---- widen, D signs, squared norm
        double u[16];
        double ss = 0.0;
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {
          const uint32_t b0 = (dw >> (2 * pr)) & 1u, b1 = (dw >> (2 * pr + 1)) & 1u;
          float f0, f1;
          if constexpr (DT == 0) {
            const uint32_t w0 = raw[pr >> 1][2 * (pr & 1)], w1 = raw[pr >> 1][2 * (pr & 1) + 1];
            f0 = __uint_as_float(w0 ^ (b0 << 31));
            f1 = __uint_as_float(w1 ^ (b1 << 31));
          } else {
            const uint32_t w = raw[pr >> 2][pr & 3] ^ ((b0 << 15) | (b1 << 31));
            if constexpr (DT == 1) {
              f0 = __uint_as_float(w << 16);
              f1 = __uint_as_float(w & 0xFFFF0000u);
            } else {
              const f16x2 hv = __builtin_bit_cast(f16x2, w);
              f0 = (float)hv[0];
              f1 = (float)hv[1];
            }
          }
          u[2 * pr] = (double)f0;
          u[2 * pr + 1] = (double)f1;
          ss = fma(u[2 * pr], u[2 * pr], ss);
          ss = fma(u[2 * pr + 1], u[2 * pr + 1], ss);
        }
        if (kAhead)
#pragma unroll
          for (int r = 0; r < NR; ++r) raw[r] = nxt[r];
        // ---- Walsh-Hadamard: register bits, then lane bits
#pragma unroll
        for (int h = 1; h < 16; h <<= 1)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if ((e & h) == 0) {
              const double x0 = u[e], x1 = u[e + h];
              u[e] = x0 + x1;
              u[e + h] = x0 - x1;
            }
        {
          // the role signs are rebuilt per step from an opaque copy of the lane
          // id (hoisted out of the loop they would hold 8 more registers)
          int xr = x16;
          asm volatile("" : "+v"(xr));
          const double sg0 = parity(xr & 5) ? -1.0 : 1.0;
#pragma unroll
          for (int e = 0; e < 16; ++e) u[e] = fma(u[e], sg0, dpp64<kDppXor1>(u[e]));
          const double sg1 = parity(xr & 6) ? -1.0 : 1.0;
#pragma unroll
          for (int e = 0; e < 16; ++e) u[e] = fma(u[e], sg1, dpp64<kDppXor2>(u[e]));
          const double sg2 = parity(xr & 8) ? -1.0 : 1.0;
#pragma unroll
          for (int e = 0; e < 16; ++e) u[e] = fma(u[e], sg2, dpp64<kDppXor8>(u[e]));
          const double sg3 = parity(xr & 4) ? -1.0 : 1.0;
#pragma unroll
          for (int e = 0; e < 16; ++e) u[e] = fma(u[e], sg3, dpp64<kDppXor7>(u[e]));
        }

        // ---- norm
        ss = row_sum16(ss);
        const bool valid = t < a.N;
        const bool finite = ss <= 3.4028234663852886e38;
        if (a.status && __ballot(valid && !finite) != 0 && lane == 0) atomicOr(a.status, TQ_STATUS_NON_FINITE);
        const double nrm = sqrt(ss);
        const float n32 = (float)nrm;
        const double rn = nrm > 0.0 ? 1.0 / nrm : 1.0;   // |x| = 0: u = 0, z = 0
        const double n32d = (double)n32;

        // ---- quantizer (and the residual for keys)
        uint32_t pk[4] = {0u, 0u, 0u, 0u};
        double ws = 0.0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if ((e & 3) == 0) __builtin_amdgcn_sched_barrier(0);   // four coordinates at a time
          const double v = u[e] * rn;
          const int cell = (int)fma(v, 128.0, 2048.0);
          const uint32_t cl = min((uint32_t)cell, (uint32_t)(kCells - 1));
          const int L = lut[cl];
          const int idx = L + (tt[L] < v ? 1 : 0);
          pk[e >> 2] |= (uint32_t)idx << (8 * (e & 3));
          if (KEY) {
            const double r = fma(-n32d, cc[idx], u[e]);
            u[e] = r;
            ws = fma(r, r, ws);
          }
        }
        // ---- bit planes: the lane's 16 bits of each plane
        transpose8x8(pk[0], pk[1]);
        transpose8x8(pk[2], pk[3]);
        const uint32_t rbase = (uint32_t)(t * RW * 4) + (uint32_t)(4 * (blk >> 1) + 2 * (blk & 1));
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          if (p < k) {
            const uint32_t lo8 = (pk[p >> 2] >> (8 * (p & 3))) & 0xFFu;
            const uint32_t hi8 = (pk[2 + (p >> 2)] >> (8 * (p & 3))) & 0xFFu;
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(lo8 | (hi8 << 8)), rrs,
                                                 valid ? rbase + (uint32_t)(p * W * 4) : 0x80000000u, 0, 0);
          }
        }
        if (x16 == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(n32), rrs,
                                                valid ? (uint32_t)((t * RW + n_off) * 4) : 0x80000000u, 0, 0);
        if (KEY) {
          ws = row_sum16(ws);
          const double wn = sqrt(ws);
          if (x16 == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((float)(wn / 16.0)), rrs,
                                                  valid ? (uint32_t)((t * RW + n_off + 1) * 4) : 0x80000000u, 0, 0);
          // hi/lo binary16 terms of w * sc as B operands: chunk (2 blk + e/8) of vector n
          const float sc = residual_scale(wn);
          const int buf = i & 1, n = vec_in_step;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            u32x4 hi, lo;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t hv, lv;
              split_f16x2((float)u[8 * kh + 2 * q], (float)u[8 * kh + 2 * q + 1], sc, hv, lv);
              hi[q] = hv;
              lo[q] = lv;
            }
            const int chunk = 2 * blk + kh;
            rbuf[((buf * 2 + 0) * 32 + chunk) * kChunkPad + n] = __builtin_bit_cast(uint4, hi);
            rbuf[((buf * 2 + 1) * 32 + chunk) * kChunkPad + n] = __builtin_bit_cast(uint4, lo);
          }
        }
      }
      if (KEY) __syncthreads();
    }
  } else {
    // ================= projector (keys) =================
    const int rb = wave - kEncKey;                 // projection block: rows 32 rb .. 32 rb + 31
    const int m = a.cb.m;
    const bool active = 32 * rb < m;
    const int row = lane & 31, kh = lane >> 5;
    u32x4 sreg[16];
    {
      const bool rok = 32 * rb + row < m;
      const _Float16* srow = reinterpret_cast<const _Float16*>(blob + a.cb.off_s) + (int64_t)(rok ? 32 * rb + row : 0) * kD + 8 * kh;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (rok) v = *reinterpret_cast<const u32x4*>(srow + 16 * s);
        sreg[s] = v;
      }
    }
    const uint32_t keep = 32 * rb + 32 <= m ? 0xFFFFFFFFu : ((1u << (m - 32 * rb)) - 1u);
    for (int i = 0; i <= ntiles; ++i) {
      if (i >= 1 && active) {
        const int buf = (i - 1) & 1;
        f32x16 acc = {};
        const uint4* bh = rbuf + ((buf * 2 + 0) * 32 + kh) * kChunkPad + row;
        const uint4* bl = rbuf + ((buf * 2 + 1) * 32 + kh) * kChunkPad + row;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const u32x4 vh = __builtin_bit_cast(u32x4, bh[2 * s * kChunkPad]);
          const u32x4 vl = __builtin_bit_cast(u32x4, bl[2 * s * kChunkPad]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sreg[s]), as<f16x8>(vh), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sreg[s]), as<f16x8>(vl), acc, 0, 0, 0);
        }
        // acc[r] of lane (n, kh) is projection 32 rb + 8(r/4) + 4 kh + r%4 of vector n
        uint32_t bits = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc[r] >= 0.0f) bits |= 1u << (8 * (r >> 2) + 4 * kh + (r & 3));
        bits |= (uint32_t)__shfl_xor((int)bits, 32, 64);
        const int64_t t = (tile0 + i - 1) * kTileVec + row;
        if (kh == 0)
          __builtin_amdgcn_raw_buffer_store_b32(bits & keep, rrs,
                                                t < a.N ? (uint32_t)((t * RW + k * W + rb) * 4) : 0x80000000u, 0,
                                                0);
      }
      __syncthreads();
    }
  }
}

template <int DT, bool KEY>
int launch_wide(WideArgs a, hipStream_t s) {
  const auto kern = encode_wide_kernel<DT, KEY>;
  const int lds = KEY ? kLdsKey : kLdsValue;
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
        hipSuccess)
      return TQ_ERR_HIP;
    attr_set = true;
  }
  constexpr int kStepVec = KEY ? kTileVec : 4 * (kThreads / 64);
  a.tiles = (a.N + kStepVec - 1) / kStepVec;
  // about one workgroup per CU
  int64_t per_block = (a.tiles * a.G + 255) / 256;
  if (per_block < 1) per_block = 1;
  if (per_block > a.tiles) per_block = a.tiles;
  a.tiles_per_block = per_block;
  a.blocks_per_group = (a.tiles + per_block - 1) / per_block;
  const int64_t blocks = a.G * a.blocks_per_group;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), lds, s, a);
  return hipGetLastError() == hipSuccess ? 0 : TQ_ERR_HIP;
}

}  // namespace

bool wide_encode_supported(const CodebookArgs& cb, int dtype, const void* x, int64_t sx_g, int64_t sx_n, int64_t N) {
  if (cb.rotation != kRotHadamard || cb.d != kD || cb.levels > 256) return false;
  if (cb.role == TQ_ROLE_KEY && cb.m > 256) return false;
  const int64_t es = dtype == TQ_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(x) & 15) return false;          // 16-byte loads
  if ((sx_g * es) % 16 || (sx_n * es) % 16 || sx_n < kD) return false;
  // 32-bit buffer offsets within a group's rows and records
  if (N > 0 && ((N - 1) * sx_n + kD) * es >= (int64_t(1) << 31)) return false;
  if (N * cb.rec_words * 4 >= (int64_t(1) << 31)) return false;
  return true;
}

int launch_encode_wide(const CodebookArgs& cb, const void* x, int dtype, int64_t G, int64_t N, int64_t sx_g,
                       int64_t sx_n, uint32_t* rec, int32_t* status, hipStream_t s) {
  if (G * N == 0) return 0;
  WideArgs a{};
  a.cb = cb;
  a.x = x;
  a.G = G; a.N = N; a.sx_g = sx_g; a.sx_n = sx_n;
  a.rec = rec;
  a.status = status;
  const bool key = cb.role == TQ_ROLE_KEY;
  switch (dtype) {
    case TQ_F32: return key ? launch_wide<0, true>(a, s) : launch_wide<0, false>(a, s);
    case TQ_BF16: return key ? launch_wide<1, true>(a, s) : launch_wide<1, false>(a, s);
    case TQ_F16: return key ? launch_wide<2, true>(a, s) : launch_wide<2, false>(a, s);
  }
  return TQ_ERR_UNSUPPORTED;
}

}  // namespace tq
