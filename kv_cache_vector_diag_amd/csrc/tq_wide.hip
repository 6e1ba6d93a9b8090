// Encode at head_dim 256 with wide codebooks (Lloyd-Max indices of up to 8
// bits: 8-bit values, keys of up to 9 bits) on gfx950 (page "turboquant-plus-rs
// 0.1.0 README", "Architecture": Walsh-Hadamard rotation with random signs,
// per-coordinate Lloyd-Max codes, and for keys the QJL signs of a Gaussian
// projection of the residual; record layout as in tq.h).
//
// A workgroup of 16 waves owns a range of 32-vector steps of one group.
//  * Encoder waves (all 16 for values, waves 0-7 for keys) take 4 vectors
//    each, 16 lanes per vector and 16 coordinates per lane, in float64:
//    - u = H(D x) as H16 (x) H16: the four low coordinate bits in registers,
//      then a transpose through the wave's own LDS rows so that the four high
//      bits are in registers, then back (every butterfly is in registers; two
//      LDS round trips replace four cross-lane stages).
//    - idx = #{t_i < z}, z = u/|x|: the cell floor(64 z + 288), computed in
//      float64 and clamped to the 576 cells of z in [-4.5, 4.5) (beyond, the
//      index is 0 or the last one), reads one 16-byte LDS entry: the count L
//      of thresholds below the cell's left edge and the first threshold t_L at
//      or above it (values: t_L as 64 t_L + 288 in float64; keys: t_L, c_L and
//      c_{L+1} in float32, compared against z in float64); idx = L + [t_L < z].
//      One comparison is enough because the thresholds, float32 values, lie
//      more than a cell width (1/64) apart, so a cell holds at most one of
//      them, and z carries float64 accuracy, so the cell found is the cell of
//      z except within ~1e-14 of an edge, where the count still agrees (the
//      edges and the thresholds are both dyadic).  A codebook that breaks the
//      spacing, or has a threshold outside the inner cells, is reported as
//      TQ_STATUS_BAD_BLOB.
//    - bit planes: the 16 indices of a lane, bytes in two 64-bit words, go
//      through an 8x8 bit transpose; byte p is then the lane's 16-bit share of
//      plane p, stored as a half word.
//    - keys: residual w = u - n32 c[idx] (c_L and c_{L+1} read with the
//      threshold) and gamma in float64; w scaled by a power of two and split
//      into two binary16 terms (22 bits), staged in LDS as MFMA B operands.
//  * Projector waves (keys: waves 8-15) hold rows 32 p .. 32 p + 31 of S in
//    registers (the A operands of all 16 K steps) and compute the signs of
//    S w for the previous step, C[32 projections][32 vectors] with
//    v_mfma_f32_32x32x16_f16 over the hi and lo terms, while the encoders work
//    on the next step (double-buffered LDS, one barrier per step).
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
constexpr int kCells = 576;                // z in [-4.5, 4.5) at 1/64
constexpr int kChunkPad = 33;              // LDS B-operand row: 32 vectors + 1 (banks)

// LDS carve-up (bytes): the cell table (16-byte entries), then per encoder
// wave four transpose rows (double [288]: 256
// coordinates + 2 after every 16), then for keys the B operands, uint4
// [2 buffers][hi, lo][32 chunks][kChunkPad].  The setup writes the scaled
// thresholds (double [255]) where the transpose rows go.
constexpr int kXRow = 288;
constexpr int kXWave = 4 * kXRow * 8;
constexpr int kRBytes = 2 * 2 * 32 * kChunkPad * 16;
constexpr int kCellBytes = kCells * 16;
constexpr int lds_bytes(bool key) {
  return kCellBytes + (key ? kEncKey : kThreads / 64) * kXWave + (key ? kRBytes : 0);
}
static_assert(lds_bytes(true) <= 160 * 1024 && lds_bytes(false) <= 160 * 1024, "LDS per workgroup");

struct WideArgs {
  CodebookArgs cb;
  const void* x;
  int64_t G, N, sx_g, sx_n;
  uint32_t* rec;
  int32_t* status;
  int64_t tiles;             // tiles per group
  int64_t tiles_per_block, blocks_per_group;
  double cell_off;           // 288 (a kernel argument, so that it sits in scalar registers)
};

// Partner value of a float64 across lanes of a 16-lane row (DPP control `C`).
template <int C>
__device__ inline double dpp64(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), C, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), C, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

// Sum over the 16 lanes of a row: partners xor 1 and xor 2 (quad_perm), xor 8
// (row_ror:8) and the half-row mirror (xor 7), which together reach every lane.
__device__ inline double row_sum16(double v) {
  v += dpp64<0xB1>(v);
  v += dpp64<0x4E>(v);
  v += dpp64<0x128>(v);
  v += dpp64<0x141>(v);
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
  const double2* cell = reinterpret_cast<const double2*>(smem);

  constexpr int kEnc = KEY ? kEncKey : kThreads / 64;   // encoder waves
  constexpr int kStepVec = 4 * kEnc;                     // vectors per step
  constexpr int kOffX = kCellBytes;
  uint4* rbuf = reinterpret_cast<uint4*>(smem + kOffX + kEnc * kXWave);
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
    double* thr = reinterpret_cast<double*>(smem + kOffX);
    const float* tsrc = reinterpret_cast<const float*>(blob + a.cb.off_t);
    const float* csrc = reinterpret_cast<const float*>(blob + a.cb.off_c);
    // thresholds in units of y = 64 z + 288 (exact: t has 24 bits)
    for (int i = tid; i < levels - 1; i += kThreads) thr[i] = fma((double)tsrc[i], 64.0, 288.0);
    __syncthreads();
    double2* cw = reinterpret_cast<double2*>(smem);
    for (int c = tid; c < kCells; c += kThreads) {
      // L = #{i : 64 t_i + 288 < c}, the thresholds below the cell's left edge
      int lo = 0, n = levels - 1;
      while (n > 0) {
        const int half = n >> 1;
        if (thr[lo + half] < (double)c) {
          lo += half + 1;
          n -= half + 1;
        } else {
          n = half;
        }
      }
      const double tl = lo < levels - 1 ? thr[lo] : __longlong_as_double(0x7FF0000000000000ll);
      if (KEY) {
        const float tz = lo < levels - 1 ? tsrc[lo] : __int_as_float(0x7F800000);
        reinterpret_cast<uint4*>(cw)[c] = make_uint4(__float_as_uint(tz), (uint32_t)lo, __float_as_uint(csrc[lo]),
                                                     __float_as_uint(csrc[lo + 1 < levels ? lo + 1 : lo]));
      } else {
        cw[c] = make_double2(tl, __longlong_as_double((long long)lo));
      }
    }
    // one threshold per cell at most, none in the end cells
    bool bad = tid + 1 < levels - 1 && !(thr[tid + 1] - thr[tid] > 1.0);
    if (tid == 0 && levels > 1) bad |= !(thr[0] >= 1.0) || !(thr[levels - 2] < (double)(kCells - 1));
    if (bad && a.status) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  }
  __syncthreads();

  // records of this group: words past the end are dropped
  const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
      a.rec + g * a.N * RW, 0, (int)(a.N * RW * 4), kRsrcWord3);
  constexpr uint32_t kDrop = 0x80000000u;   // an offset past every resource: the access is dropped

  if (!KEY || wave < kEncKey) {
    // ================= encoder =================
    const int x16 = lane & 15, vg = lane >> 4;
    double* xrow = reinterpret_cast<double*>(smem + kOffX + wave * kXWave) + vg * kXRow;   // this vector's LDS row
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
      const uint32_t off = t < a.N ? (uint32_t)(t * a.sx_n * ES) + (uint32_t)(16 * ES * x16) : kDrop;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        raw[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, off + 16u * r, 0, 0));
    };
    // float32 rows are loaded in the step that uses them (a prefetch would
    // double their 16 registers); 2-byte rows one step ahead
    constexpr bool kAhead = DT != 0;
    u32x4 raw[NR];
    if (kAhead) {
      load_in(0, raw);
      // Wait for the first rows here.  Left pending into the loop, they would
      // make the loop head wait for every earlier memory operation on each
      // step (the counter state at the head merges the entry path, where the
      // rows are the oldest operation, with the back edge, where the previous
      // step's record stores follow them).
#pragma unroll
      for (int r = 0; r < NR; ++r) asm volatile("" ::"v"(raw[r]));
    }

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
        // ---- Walsh-Hadamard, H16 (x) H16: the low four coordinate bits in
        // registers (lane x16 holds coordinates 16 x16 + e), through LDS to the
        // high four (coordinates x16 + 16 e), and back.  Row index of
        // coordinate c: c + 2 (c >> 4) (16-byte rows, padded against conflicts).
        const auto h16 = [&]() {
#pragma unroll
          for (int h = 1; h < 16; h <<= 1)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if ((e & h) == 0) {
                const double x0 = u[e], x1 = u[e + h];
                u[e] = x0 + x1;
                u[e + h] = x0 - x1;
              }
        };
        h16();
#pragma unroll
        for (int e = 0; e < 16; e += 2)
          *reinterpret_cast<double2*>(xrow + 18 * x16 + e) = make_double2(u[e], u[e + 1]);
#pragma unroll
        for (int e = 0; e < 16; ++e) u[e] = xrow[x16 + 18 * e];
        h16();
#pragma unroll
        for (int e = 0; e < 16; ++e) xrow[x16 + 18 * e] = u[e];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const double2 v = *reinterpret_cast<const double2*>(xrow + 18 * x16 + e);
          u[e] = v.x;
          u[e + 1] = v.y;
        }

        // ---- norm
        ss = row_sum16(ss);
        const bool valid = t < a.N;
        const bool finite = ss <= 3.4028234663852886e38;
        if (a.status && __ballot(valid && !finite) != 0 && lane == 0) atomicOr(a.status, TQ_STATUS_NON_FINITE);
        const double nrm = sqrt(ss);
        const float n32 = (float)nrm;
        const double rn64 = nrm > 0.0 ? 64.0 / nrm : 64.0;   // |x| = 0: u = 0, z = 0
        const double rn = nrm > 0.0 ? 1.0 / nrm : 1.0;
        const double n32d = (double)n32;

        // ---- quantizer (and the residual for keys)
        uint32_t pk[4] = {0u, 0u, 0u, 0u};
        double ws = 0.0;
        float rf[KEY ? 16 : 1];                      // residual, float32 (what the split takes)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if constexpr (KEY) {
            const double v = u[e] * rn;
            const int cl = min(max((int)fma(v, 64.0, a.cell_off), 0), kCells - 1);
            const uint4 ce = reinterpret_cast<const uint4*>(cell)[cl];
            const bool up = (double)__uint_as_float(ce.x) < v;
            pk[e >> 2] |= (ce.y + (up ? 1u : 0u)) << (8 * (e & 3));
            const double r = fma(-n32d, (double)__uint_as_float(up ? ce.w : ce.z), u[e]);
            ws = fma(r, r, ws);
            rf[e] = (float)r;
          } else {
            const double y = fma(u[e], rn64, a.cell_off);
            const int cl = min(max((int)y, 0), kCells - 1);
            const double2 tl = cell[cl];
            const bool up = tl.x < y;
            pk[e >> 2] |= (uint32_t)((int)__double_as_longlong(tl.y) + (up ? 1 : 0)) << (8 * (e & 3));
          }
          if ((e & 3) == 3) {
            // four coordinates at a time: their results are consumed here
            // (and the memory clobber keeps the next four's reads below), so
            // at most four table entries are live
            if constexpr (KEY)
              asm volatile("" : "+v"(pk[e >> 2]), "+v"(ws), "+v"(rf[e - 3]), "+v"(rf[e - 2]), "+v"(rf[e - 1]),
                           "+v"(rf[e])::"memory");
            else
              asm volatile("" : "+v"(pk[e >> 2])::"memory");
          }
        }
        // ---- bit planes: the lane's 16 bits of each plane
        transpose8x8(pk[0], pk[1]);
        transpose8x8(pk[2], pk[3]);
        const uint32_t rbase = valid ? (uint32_t)(t * RW * 4) + (uint32_t)(4 * (x16 >> 1) + 2 * (x16 & 1)) : kDrop;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const uint32_t lo8 = (pk[p >> 2] >> (8 * (p & 3))) & 0xFFu;
          const uint32_t hi8 = (pk[2 + (p >> 2)] >> (8 * (p & 3))) & 0xFFu;
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(lo8 | (hi8 << 8)), rrs,
                                               p < k ? rbase + (uint32_t)(p * W * 4) : kDrop, 0, 0);
        }
        const uint32_t nbase = valid && x16 == 0 ? (uint32_t)((t * RW + n_off) * 4) : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(n32), rrs, nbase, 0, 0);
        if (KEY) {
          ws = row_sum16(ws);
          const double wn = sqrt(ws);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((float)(wn / 16.0)), rrs, nbase + 4u, 0, 0);
          // hi/lo binary16 terms of w * sc as B operands: chunk (2 x16 + e/8) of vector n
          const float sc = residual_scale(wn);
          const int buf = i & 1, n = vec_in_step;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            u32x4 hi, lo;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t hv, lv;
              split_f16x2(rf[8 * kh + 2 * q], rf[8 * kh + 2 * q + 1], sc, hv, lv);
              hi[q] = hv;
              lo[q] = lv;
            }
            const int chunk = 2 * x16 + kh;
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
          if (acc[r] >= 0.0f) bits |= 1u << (8 * (r >> 2) + (r & 3));
        bits <<= 4 * kh;
        bits |= (uint32_t)__shfl_xor((int)bits, 32, 64);
        const int64_t t = (tile0 + i - 1) * kTileVec + row;
        __builtin_amdgcn_raw_buffer_store_b32(bits & keep, rrs,
                                              t < a.N && kh == 0 ? (uint32_t)((t * RW + k * W + rb) * 4) : kDrop, 0, 0);
      }
      __syncthreads();
    }
  }
}

template <int DT, bool KEY>
int launch_wide(WideArgs a, hipStream_t s) {
  const auto kern = encode_wide_kernel<DT, KEY>;
  constexpr int lds = lds_bytes(KEY);
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
        hipSuccess)
      return TQ_ERR_HIP;
    attr_set = true;
  }
  constexpr int kStepVec = KEY ? kTileVec : 4 * (kThreads / 64);
  a.tiles = (a.N + kStepVec - 1) / kStepVec;
  a.cell_off = 288.0;
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
