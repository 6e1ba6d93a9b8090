// Outlier/normal split encode on MFMA for head_dim 256 with 32 outlier
// channels and bf16 input (page "turboquant-plus-rs 0.1.0 README", "Modules"
// outlier: channels split into outlier and normal parts, each quantized on its
// own; "Architecture" step 1: Haar-distributed rotation via QR or the
// Walsh-Hadamard transform).  Same device semantics as the generic split path
// (encode_generic_kernel with a channel map), restated for throughput:
//
//  * A prep kernel folds each group's channel map into MFMA A-operand
//    fragments in caller scratch:
//      normal rotation R' = R P_n (224 x 256, R = sqrt(224) Q of the Haar
//        codebook, P_n selects the normal channels), split exactly into three
//        bf16 pieces (24 significant bits);
//      the outlier gather P_o (0/1) and the outlier rotation H_32 D_o (32 x 32,
//        exact +-1) applied to the gathered channels after the contraction;
//      keys: the QJL matrices S_n (224 x 224) and S_o (32 x 32), binary16, their
//        columns permuted to the rotation-result layout.
//  * One workgroup (8 waves) encodes 256 tokens per step, one 32-token tile per
//    wave; the bf16 row is the B operand as it is, in natural channel order.
//    The contraction runs chunk-outer: for each 16-channel chunk, its slice of
//    fragments (all row tiles) is staged in LDS (double buffered) and shared by
//    the 8 waves, and the 7 + 2 row-tile accumulators stay in registers.  The
//    next slice goes straight from memory into LDS (buffer loads to LDS) while
//    the current one feeds the matrix cores; the two buffers are distinct
//    arrays, so reading one never waits for the loads into the other.
//  * Norms: |x|^2 in float64 from pair sums; |x_o|^2 exactly from the gathered
//    outlier channels; |x_n|^2 = |x|^2 - |x_o|^2.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

using namespace mf;

constexpr int kD = 256;              // head_dim
constexpr int kNo = 32;              // outlier channels
constexpr int kDn = kD - kNo;        // normal channels (224)
constexpr int kMT = kDn / 32;        // 32-row tiles of the normal part (7)
constexpr int kKC = kD / 16;         // 16-channel K-chunks of a row (16)
constexpr int kQC = kDn / 16;        // 16-coordinate K-chunks of the normal part (14)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kFragLanes = 64;       // one fragment: 64 lanes x 16 bytes

// fragment offsets within a group's scratch (in fragments)
constexpr int kRPieces = 3;
constexpr int kSliceR = kMT * kRPieces;           // rotation fragments of one K-chunk (21)
constexpr int kOffR = 0;                          // [c][m][piece]
constexpr int kOffOP = kOffR + kKC * kSliceR;     // outlier gather [c]
constexpr int kOffHO = kOffOP + kKC;              // outlier rotation H_32 D_o of the gathered channels [c < 2]
constexpr int kOffSO = kOffHO + 2;                // outlier QJL [c < 2]
constexpr int kOffS = kOffSO + 2;                 // normal QJL [m'][c < 14]
constexpr int kFragsValue = kOffSO;               // 354
constexpr int kFragsKey = kOffS + kMT * kQC;      // 454
constexpr int kSliceS = kQC;                      // fragments per projection slice (14)
constexpr int kOutFrags = kKC + 4;                // outlier fragments kept in LDS (20)

constexpr size_t kLdsOut = (size_t)kOutFrags * kFragLanes * 16;     // 20 KB
constexpr size_t kLdsBytes = kLdsOut + 256;   // the two slice buffers are static arrays

struct PrepArgs {
  const uint8_t* cbn;
  const uint8_t* cbo;
  int64_t stride_n, stride_o, n_cb;
  uint32_t off_dn, off_sn, off_do, off_so;
  const int32_t* chan;
  int frags;
  u32x4* work;
  int32_t* status;
};

// bf16 round-to-nearest-even of a float (bit pattern in the low 16 bits).
__device__ inline uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// One thread per (fragment, lane); blockIdx.y = group.
__global__ __launch_bounds__(256) void split256_prep_kernel(PrepArgs a) {
  __shared__ int inv[kD];   // channel -> position in the map (< 32: outlier, else 32 + normal index)
  const int64_t g = blockIdx.y;
  const int tid = threadIdx.x;
  const int32_t* ch = a.chan + g * kD;
  inv[tid] = -1;
  __syncthreads();
  {
    const int c = ch[tid];
    if ((unsigned)c < (unsigned)kD) {
      inv[c] = tid;
    } else if (a.status) {
      atomicOr(a.status, TQ_STATUS_BAD_CHANNEL);
    }
  }
  __syncthreads();
  const int f = blockIdx.x * 4 + (tid >> 6);
  const int lane = tid & 63;
  if (f >= a.frags) return;
  const uint8_t* bn = a.cbn + (g % a.n_cb) * a.stride_n;
  const uint8_t* bo = a.cbo + (g % a.n_cb) * a.stride_o;
  const float* R = reinterpret_cast<const float*>(bn + a.off_dn);
  const uint16_t* Sn = reinterpret_cast<const uint16_t*>(bn + a.off_sn);
  const uint16_t* So = reinterpret_cast<const uint16_t*>(bo + a.off_so);
  const uint32_t dbits_o = reinterpret_cast<const uint32_t*>(bo + a.off_do)[0];
  const int row = tile_row_index(lane & 31), hl = lane >> 5;
  u32x4 v;
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
    for (int hh = 0; hh < 2; ++hh) {
      const int e = 2 * q + hh;
      uint32_t b16 = 0;
      if (f < kOffOP) {                       // R' piece (c, m, piece): r = p1 + p2 + p3 in bf16
        const int c = f / kSliceR, m = (f % kSliceR) / kRPieces, piece = f % kRPieces;
        const int p = inv[16 * c + 8 * hl + e];
        if (p >= kNo) {
          float r = R[(32 * m + row) * kDn + (p - kNo)];
          uint32_t pb = 0;
          for (int t = 0; t <= piece; ++t) {
            pb = bf16_rne(r);
            r -= __uint_as_float(pb << 16);
          }
          b16 = pb;
        }
      } else if (f < kOffHO) {                // P_o: result row r = channel chan[r]
        if (inv[16 * (f - kOffOP) + 8 * hl + e] == row) b16 = 0x3F80u;
      } else if (f < kOffSO) {                // H_32 D_o, columns in the gather's result order
        const int p = qjl_coord(f - kOffHO, hl, e);
        b16 = 0x3F80u | ((h_sign(row, p) ^ ((dbits_o >> p) & 1u)) << 15);
      } else if (f < kOffS) {                 // S_o, columns in result order
        b16 = So[row * kNo + qjl_coord(f - kOffSO, hl, e)];
      } else {                                // S_n, columns in result order
        const int mp = (f - kOffS) / kQC, c = (f - kOffS) % kQC;
        b16 = Sn[(32 * mp + row) * kDn + qjl_coord(c, hl, e)];
      }
      word |= b16 << (16 * hh);
    }
    v[q] = word;
  }
  a.work[((int64_t)g * a.frags + f) * kFragLanes + lane] = v;
}

struct SplitArgs {
  const u32x4* frag;
  const uint8_t* cbn;
  const uint8_t* cbo;
  int64_t stride_n, stride_o, n_cb;
  uint32_t off_cn, off_tn, off_co, off_to;
  int bits_n, bits_o, role;
  const uint32_t* x;         // bf16 pairs
  int64_t G, N, sx_g, sx_n;  // strides in elements
  uint32_t* rec_n;
  uint32_t* rec_o;
  int32_t* status;
  int frags;
  int64_t tiles_per_group, tiles_per_block, blocks_per_group;
  bool xcd_major;
};

// |w| of a token from the square sums of its two lane halves.  The float32
// squares of a tiny residual can underflow (norms below ~2^-40), so such
// tokens take it from the scaled split terms instead: (w sc)^2 = hi.hi +
// 2 hi.lo (+ lo^2, below 2^-22 of it), square-rooted before unscaling.
__device__ inline float split_gamma(float wsq, float n32, float sc, const u32x4* whi, const u32x4* wlo, int nchunks) {
  float sq = wsq;
  const bool tiny = n32 < 0x1p-40f;
  if (tiny) {
    float hh = 0.0f, hl = 0.0f;
    for (int c = 0; c < nchunks; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) split_sumsq(whi[c][q], wlo[c][q], hh, hl);
    sq = fmaf(2.0f, hl, hh);
  }
  const auto pg = __builtin_amdgcn_permlane32_swap(__float_as_uint(sq), __float_as_uint(sq), false, false);
  const float tot = __uint_as_float(pg[0]) + __uint_as_float(pg[1]);
  return tiny ? sqrtf(tot) / sc : sqrtf(tot);
}

// Quantize one 32-row result tile (lane half h holds coordinates 16h + r in
// register r): sign word, thermometer words, and (keys) the residual, scaled
// by the power of two sc and split into f16 hi/lo pairs (two K-chunks of 4
// words each), plus its (unscaled) square sum.
template <int K, bool KEY>
__device__ inline void quantize_tile(const f32x16& u, float ns, const float* cpos, const float* tn, float sc,
                                     uint32_t& pw, uint32_t* tw, u32x4* whi, u32x4* wlo, float& wsq) {
  constexpr int NT = (1 << K) / 2 - 1;
  const uint32_t nbits = __float_as_uint(ns);
  uint32_t pacc = 0;
  uint32_t tacc[NT > 0 ? NT : 1];
#pragma unroll
  for (int t = 0; t < NT; ++t) tacc[t] = 0;
  float wv[16];
#pragma unroll
  for (int r = 15; r >= 0; --r) {
    const float uu = u[r];
    float nsg;
    pos_step(pacc, nsg, uu, nbits, 0x80000000u);
    float mag = cpos[0];
    if (NT > 0) mag = thr_first(tacc[0], uu, tn[0], cpos[0], cpos[NT > 0 ? 1 : 0]);
#pragma unroll
    for (int t = 1; t < NT; ++t) thr_step(tacc[t], mag, uu, tn[t], cpos[t + 1]);
    if (KEY) {
      const float w = fmaf(nsg, mag, uu);
      wsq = fmaf(w, w, wsq);
      wv[r] = w;
    }
  }
  pw = pacc;
#pragma unroll
  for (int t = 0; t < NT; ++t) tw[t] = tacc[t];
  if (KEY) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t hi, lo;
        split_f16x2(wv[8 * p + 2 * q], wv[8 * p + 2 * q + 1], sc, hi, lo);
        whi[p][q] = hi;
        wlo[p][q] = lo;
      }
  }
}

// Bit plane words of one tile from the sign and thermometer words (16 bits of
// the tile per lane half), as in the head_dim-128 kernel.
template <int K>
__device__ inline void tile_planes(uint32_t pw, const uint32_t* tw, uint32_t* pl) {
  constexpr int NT = (1 << K) / 2 - 1;
  pl[K - 1] = pw;
#pragma unroll
  for (int p = 0; p < K - 1; ++p) {
    uint32_t cb = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (((t + 1) & ((1 << p) - 1)) == 0) cb ^= tw[t];
    pl[p] = ~(cb ^ pw) & 0xFFFFu;
  }
}

__device__ inline uint32_t sign_word(const f32x16& acc) {
  uint32_t a2 = 0;
#pragma unroll
  for (int r = 15; r >= 0; --r) a2 = __builtin_amdgcn_alignbit(a2, __float_as_uint(acc[r]), 31);
  return a2;   // inverted signs of 16 projections (1 = negative)
}

// Store NP 16-bit half words (this lane half's part of NP record words) and the
// trailing float words: pairs of parts are completed by one lane swap.
template <int NP, int NF>
__device__ inline void store_record(const uint32_t* part, const uint32_t* tail, int h, bool valid, uint32_t* out) {
  constexpr int NPP = (NP + 1) / 2 * 2;
  constexpr int R = NP + NF;
  uint32_t words[NPP + NF];
#pragma unroll
  for (int i = 0; i < NPP / 2; ++i) {
    const uint32_t a0 = part[2 * i], a1 = 2 * i + 1 < NP ? part[2 * i + 1] : 0u;
    auto sp = __builtin_amdgcn_permlane32_swap(a0, a1, false, false);
    words[2 * i] = a0 | sp[1];        // complete in half 0
    words[2 * i + 1] = a1 | sp[0];    // complete in half 1
  }
#pragma unroll
  for (int i = 0; i < NF; ++i) words[NP + i] = tail[i];   // same value in both halves
  // half h stores words 2q + h (a plane/sign word 2i is complete in half 0, 2i+1 in half 1)
#pragma unroll
  for (int q = 0; q < (R + 1) / 2; ++q) {
    const int wi = 2 * q + h;
    if (valid && wi < R) out[wi] = h ? words[2 * q + 1 < R ? 2 * q + 1 : 0] : words[2 * q];
  }
}

typedef __attribute__((address_space(3))) uint32_t lds_u32;

template <int KN, int KO, bool KEY>
__global__ __launch_bounds__(kThreads) void split256_kernel(SplitArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  // slice buffers: two distinct arrays, so that a DMA into one never makes the
  // reads of the other wait for it
  __shared__ __align__(16) u32x4 slice_a[kSliceR * kFragLanes];
  __shared__ __align__(16) u32x4 slice_b[kSliceR * kFragLanes];
  u32x4* ofr = reinterpret_cast<u32x4*>(smem);
  float* consts = reinterpret_cast<float*>(smem + kLdsOut);
  constexpr int LN = 1 << KN, LO = 1 << KO;
  constexpr int NTN = LN / 2 - 1, NTO = LO / 2 - 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;
  // group assignment: XCD-major (workgroup b runs on XCD b % 8 under the usual
  // round-robin dispatch; all workgroups of one XCD share a group at a time, so
  // its fragments stay in that XCD's L2), else one group per workgroup range
  const int64_t g_begin = a.xcd_major ? (int64_t)(blockIdx.x % 8) : blockIdx.x / a.blocks_per_group;
  const int64_t chunk = a.xcd_major ? (int64_t)(blockIdx.x / 8) : blockIdx.x % a.blocks_per_group;
  const int64_t g_step = a.xcd_major ? 8 : a.G;
  for (int64_t g = g_begin; g < a.G; g += g_step) {
    __syncthreads();                                   // the previous group is done with LDS
    const uint8_t* bn = a.cbn + (g % a.n_cb) * a.stride_n;
    const uint8_t* bo = a.cbo + (g % a.n_cb) * a.stride_o;
    if (tid == 0 && a.status) {
      const BlobHeader* hn = reinterpret_cast<const BlobHeader*>(bn);
      const BlobHeader* ho = reinterpret_cast<const BlobHeader*>(bo);
      const bool bad = hn->magic != kBlobMagic || hn->version != kBlobVersion || hn->head_dim != kDn ||
                       hn->bits != a.bits_n || hn->role != a.role || hn->rotation != (uint32_t)kRotHaar ||
                       hn->projections != (KEY ? kDn : 0) || ho->magic != kBlobMagic ||
                       ho->version != kBlobVersion || ho->head_dim != kNo || ho->bits != a.bits_o ||
                       ho->role != a.role || ho->rotation != (uint32_t)kRotHadamard ||
                       ho->projections != (KEY ? kNo : 0);
      if (bad) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
    }
    const u32x4* fr = a.frag + (int64_t)g * a.frags * kFragLanes;
    for (int i = tid; i < (KEY ? kOutFrags : kKC + 2) * kFragLanes; i += kThreads) ofr[i] = fr[kOffOP * kFragLanes + i];
    if (tid < LN / 2) consts[tid] = reinterpret_cast<const float*>(bn + a.off_cn)[LN / 2 + tid];
    if (tid < NTN) consts[8 + tid] = reinterpret_cast<const float*>(bn + a.off_tn)[LN / 2 + tid];
    if (tid < LO / 2) consts[16 + tid] = reinterpret_cast<const float*>(bo + a.off_co)[LO / 2 + tid];
    if (tid < NTO) consts[24 + tid] = reinterpret_cast<const float*>(bo + a.off_to)[LO / 2 + tid];
    __syncthreads();
    float cpn[LN / 2], tpn[NTN > 0 ? NTN : 1], cpo[LO / 2], tpo[NTO > 0 ? NTO : 1];
#pragma unroll
    for (int i = 0; i < LN / 2; ++i) cpn[i] = consts[i];
#pragma unroll
    for (int i = 0; i < NTN; ++i) tpn[i] = consts[8 + i];
#pragma unroll
    for (int i = 0; i < LO / 2; ++i) cpo[i] = consts[16 + i];
#pragma unroll
    for (int i = 0; i < NTO; ++i) tpo[i] = consts[24 + i];

    const int64_t tile0 = chunk * a.tiles_per_block;
    const int64_t tile_end = min(tile0 + a.tiles_per_block, a.tiles_per_group);
    constexpr int kSliceEntries = kSliceR * kFragLanes;   // u32x4 per rotation slice
    for (int64_t base = tile0; base < tile_end; base += kWaves) {
      // re-derive the fragment base each step (opaque to the compiler), so that
      // the slice addresses are not hoisted out of the loop into dozens of
      // 64-bit registers; offsets below are 32-bit, from a uniform base
      const uint8_t* frb = reinterpret_cast<const uint8_t*>(fr);
      asm volatile("" : "+s"(frb));
      const __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(frb), 0, a.frags * kFragLanes * 16, kRsrcWord3);
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      // fragments nbase .. nbase + nent of the group straight into an LDS slice
      // buffer, 64 entries (1 KB) per wave and round
      const auto dma = [&](u32x4* dst, uint32_t nbase, int nent) {
#pragma unroll
        for (int i = 0; i < (kSliceEntries + kThreads - 1) / kThreads; ++i) {
          const int e0 = i * kThreads + wv * 64;
          if (e0 < nent)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(frs, (lds_u32*)(dst + e0), 16, (nbase + (uint32_t)(e0 + lane)) * 16u,
                                                     0, 0, 0);
        }
      };
      const int64_t tile = base + wave;
      const int64_t tok = tile * 32 + col;
      const bool valid = tile < tile_end && tok < a.N;

      // ---- x: K-chunk c holds channels 16c + 8h .. +7 of token `col` (bf16 pairs);
      // chunks are loaded kXPre ahead of their use, |x|^2 accumulates as they arrive
      constexpr int kXPre = 4;
      const uint32_t* xr = a.x + (g * a.sx_g + (valid ? tok : 0) * a.sx_n) / 2;
      u32x4 xb[kKC];
#pragma unroll
      for (int c = 0; c < kXPre; ++c) xb[c] = *reinterpret_cast<const u32x4*>(xr + 8 * c + 4 * h);
      double ss = 0.0;
      __syncthreads();                                     // slice buffers free
      dma(slice_a, kOffR * kFragLanes, kSliceEntries);

      // ---- rotation, chunk-outer: u[m] (normal tiles), xo (outlier gather)
      f32x16 u[kMT];
#pragma unroll
      for (int m = 0; m < kMT; ++m) u[m] = f32x16{};
      f32x16 xo = {};
#pragma unroll
      for (int c = 0; c < kKC; ++c) {
        // this wave's slice DMA has landed: it was issued before the one x chunk
        // load of the previous chunk (if any), and loads complete in order
        if (c >= 1 && c - 1 + kXPre < kKC) __builtin_amdgcn_s_waitcnt(0x0F71);   // vmcnt(1)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                                // vmcnt(0)
        __syncthreads();                                   // slice c complete; the other buffer free
        const u32x4* cur = (c & 1) ? slice_b : slice_a;
        u32x4* nxt = (c & 1) ? slice_a : slice_b;
        // next slice: rotation chunk c+1, or (keys, after the last) projection slice 0
        const bool more = c + 1 < kKC || KEY;
        const int nent = (c + 1 < kKC ? kSliceR : kSliceS) * kFragLanes;
        const uint32_t nbase = c + 1 < kKC ? (uint32_t)((kOffR + (c + 1) * kSliceR) * kFragLanes)
                                           : (uint32_t)(kOffS * kFragLanes);
        if (more) dma(nxt, nbase, nent);
        __builtin_amdgcn_sched_barrier(0);                 // the DMA before the x chunk load
        if (c + kXPre < kKC) xb[c + kXPre] = *reinterpret_cast<const u32x4*>(xr + 8 * (c + kXPre) + 4 * h);
        {
          double part = 0.0;
#pragma unroll
          for (int q = 0; q < 4; ++q) part += pair_sumsq_bf16(xb[c][q]);
          // squares below the float32 range: the chunk again, exactly in float64
          ss += part < 0x1p-100 ? sumsq8_bf16_f64(xb[c]) : part;
        }
        const bf16x8 xv = as<bf16x8>(xb[c]);
        // pieces outer, row tiles inner: consecutive MFMAs use different accumulators
#pragma unroll
        for (int pc = 0; pc < kRPieces; ++pc) {
#pragma unroll
          for (int m = 0; m < kMT; ++m)
            u[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(cur[(m * kRPieces + pc) * kFragLanes + lane]), xv,
                                                           u[m], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);               // a few fragments live at a time
        }
        xo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(ofr[c * kFragLanes + lane]), xv, xo, 0, 0, 0);
      }
      // ---- outlier rotation uo = H_32 D_o x_o from the gathered channels (exact
      // bf16 values): lane half h holds channel 16h + r of the map in register r,
      // K-chunk c' takes registers 8c' .. 8c' + 7 (the fragments' column order)
      f32x16 uo = {};
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        u32x4 bx;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          bx[q] = (__float_as_uint(xo[8 * cc + 2 * q]) >> 16) | (__float_as_uint(xo[8 * cc + 2 * q + 1]) & 0xFFFF0000u);
        uo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(ofr[(kKC + cc) * kFragLanes + lane]), as<bf16x8>(bx),
                                                     uo, 0, 0, 0);
      }

      // ---- norms (float64): |x|^2 from pair sums, |x_o|^2 from the exact gather
      double so = 0.0;
#pragma unroll
      for (int r = 0; r < 16; ++r) so = fma((double)xo[r], (double)xo[r], so);
      {
        uint32_t l1 = __double2loint(ss), h1 = __double2hiint(ss), l2 = __double2loint(so), h2 = __double2hiint(so);
        auto p1 = __builtin_amdgcn_permlane32_swap(l1, l1, false, false);
        auto q1 = __builtin_amdgcn_permlane32_swap(h1, h1, false, false);
        auto p2 = __builtin_amdgcn_permlane32_swap(l2, l2, false, false);
        auto q2 = __builtin_amdgcn_permlane32_swap(h2, h2, false, false);
        ss += __hiloint2double((int)(h ? q1[0] : q1[1]), (int)(h ? p1[0] : p1[1]));
        so += __hiloint2double((int)(h ? q2[0] : q2[1]), (int)(h ? p2[0] : p2[1]));
      }
      const bool finite = ss <= 3.4028234663852886e38;
      if (a.status && __ballot(valid && !finite && h == 0) != 0 && lane == 0) atomicOr(a.status, TQ_STATUS_NON_FINITE);
      double sn = ss - so;
      sn = sn > 0.0 ? sn : 0.0;
      const float no32 = (float)sqrt(so), nn32 = (float)sqrt(sn);
      // powers of two bringing each part's residual to O(1) for the f16 split
      const auto pow2_scale = [](float n) {
        const uint32_t e = (__float_as_uint(n) >> 23) & 0xFFu;
        return (n > 0.0f && e < 253u) ? __uint_as_float((254u - e) << 23) : 1.0f;
      };
      const float sco = pow2_scale(no32), scn = pow2_scale(nn32);

      // ---- outlier part: quantize, QJL
      float tno[NTO > 0 ? NTO : 1];
#pragma unroll
      for (int t = 0; t < NTO; ++t) tno[t] = tpo[t] * no32;
      uint32_t pw_o, tw_o[NTO > 0 ? NTO : 1];
      u32x4 who[2], wlo_o[2];
      float wsq_o = 0.0f;
      quantize_tile<KO, KEY>(uo, no32, cpo, tno, sco, pw_o, tw_o, who, wlo_o, wsq_o);
      asm volatile("" : "+v"(pw_o));
#pragma unroll
      for (int t = 0; t < NTO; ++t) asm volatile("" : "+v"(tw_o[t]));
      uint32_t sw_o = 0;
      float gam_o = 0.0f;
      if (KEY) {
        f32x16 acc = {};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 sf = ofr[(kKC + 2 + c) * kFragLanes + lane];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf), as<f16x8>(who[c]), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf), as<f16x8>(wlo_o[c]), acc, 0, 0, 0);
        }
        sw_o = sign_word(acc);
        asm volatile("" : "+v"(sw_o));
        gam_o = split_gamma(wsq_o, no32, sco, who, wlo_o, 2) * 0.17677669529663688f;   // / sqrt(32)
      }

      // ---- normal part: quantize the 7 row tiles
      float tnn[NTN > 0 ? NTN : 1];
#pragma unroll
      for (int t = 0; t < NTN; ++t) tnn[t] = tpn[t] * nn32;
      uint32_t pw_n[kMT], tw_n[NTN > 0 ? NTN : 1][kMT];
      u32x4 whn[KEY ? kQC : 1], wln[KEY ? kQC : 1];
      float wsq_n = 0.0f;
#pragma unroll
      for (int m = 0; m < kMT; ++m) {
        uint32_t twm[NTN > 0 ? NTN : 1];
        quantize_tile<KN, KEY>(u[m], nn32, cpn, tnn, scn, pw_n[m], twm, KEY ? &whn[2 * m] : whn,
                               KEY ? &wln[2 * m] : wln, wsq_n);
#pragma unroll
        for (int t = 0; t < NTN; ++t) {
          tw_n[t][m] = twm[t];
          asm volatile("" : "+v"(tw_n[t][m]));
        }
        asm volatile("" : "+v"(pw_n[m]));
        if (KEY) {
          asm volatile("" : "+v"(whn[2 * m]), "+v"(whn[2 * m + 1]), "+v"(wln[2 * m]), "+v"(wln[2 * m + 1]));
        }
        __builtin_amdgcn_sched_barrier(0);                 // one tile's temporaries at a time
      }

      // ---- keys: QJL of the normal part, one 32-projection slice at a time
      uint32_t sw_n[kMT];
      float gam_n = 0.0f;
      if (KEY) {
#pragma unroll
        for (int mp = 0; mp < kMT; ++mp) {
          __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0): this wave's slice DMA has landed
          __syncthreads();
          const u32x4* cur = ((kKC + mp) & 1) ? slice_b : slice_a;
          u32x4* nxt = ((kKC + mp) & 1) ? slice_a : slice_b;
          const bool more = mp + 1 < kMT;
          const uint32_t nbase = (uint32_t)((kOffS + (mp + 1) * kSliceS) * kFragLanes);
          if (more) dma(nxt, nbase, kSliceS * kFragLanes);
          f32x16 acc = {};
#pragma unroll
          for (int c = 0; c < kQC; ++c) {
            const u32x4 sf = cur[c * kFragLanes + lane];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf), as<f16x8>(whn[c]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf), as<f16x8>(wln[c]), acc, 0, 0, 0);
            if ((c & 3) == 3) __builtin_amdgcn_sched_barrier(0);
          }
          sw_n[mp] = sign_word(acc);
          asm volatile("" : "+v"(sw_n[mp]));   // materialise here (not next to the stores)
        }
        gam_n = split_gamma(wsq_n, nn32, scn, whn, wln, kQC) * 0.06681531047810609f;   // / sqrt(224)
      }

      // ---- records (built in every lane, stored for valid tokens only: keeping
      // the computation unconditional stops the compiler from sinking it into
      // the store branch with all projection accumulators alive)
      {
        const int64_t tk = valid ? tok : 0;
        // normal: KN planes x 7 words, (keys) 7 sign words, n, gamma
        constexpr int NPN = KN * kMT + (KEY ? kMT : 0);
        uint32_t part[NPN];
#pragma unroll
        for (int m = 0; m < kMT; ++m) {
          uint32_t twm[NTN > 0 ? NTN : 1];
#pragma unroll
          for (int t = 0; t < NTN; ++t) twm[t] = tw_n[t][m];
          uint32_t pl[KN];
          tile_planes<KN>(pw_n[m], twm, pl);
#pragma unroll
          for (int p = 0; p < KN; ++p) part[p * kMT + m] = h ? (pl[p] << 16) : (pl[p] & 0xFFFFu);
          if (KEY) part[KN * kMT + m] = h ? ((~sw_n[m]) << 16) : ((~sw_n[m]) & 0xFFFFu);
        }
        const uint32_t tail_n[2] = {__float_as_uint(nn32), __float_as_uint(gam_n)};
        store_record<NPN, KEY ? 2 : 1>(part, tail_n, h, valid, a.rec_n + (g * a.N + tk) * (NPN + (KEY ? 2 : 1)));
        // outlier: KO planes, (keys) 1 sign word, n, gamma
        constexpr int NPO = KO + (KEY ? 1 : 0);
        uint32_t parto[NPO];
        uint32_t plo[KO];
        tile_planes<KO>(pw_o, tw_o, plo);
#pragma unroll
        for (int p = 0; p < KO; ++p) parto[p] = h ? (plo[p] << 16) : (plo[p] & 0xFFFFu);
        if (KEY) parto[KO] = h ? ((~sw_o) << 16) : ((~sw_o) & 0xFFFFu);
        const uint32_t tail_o[2] = {__float_as_uint(no32), __float_as_uint(gam_o)};
        store_record<NPO, KEY ? 2 : 1>(parto, tail_o, h, valid, a.rec_o + (g * a.N + tk) * (NPO + (KEY ? 2 : 1)));
      }
    }
  }
}

template <int KN, int KO, bool KEY>
int launch_split(SplitArgs a, hipStream_t s) {
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&split256_kernel<KN, KO, KEY>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes) != hipSuccess)
      return -10;
    attr_set = true;
  }
  const int64_t grid = a.xcd_major ? 8 * a.blocks_per_group : a.G * a.blocks_per_group;
  hipLaunchKernelGGL((split256_kernel<KN, KO, KEY>), dim3((unsigned)grid), dim3(kThreads),
                     kLdsBytes, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace

bool split256_supported(int role, int head_dim, int n_outlier, int bits, int dtype, const void* x, int64_t sx_g,
                        int64_t sx_n) {
  if (head_dim != kD || n_outlier != kNo || dtype != TQ_BF16) return false;
  if ((reinterpret_cast<uintptr_t>(x) & 15) != 0 || (sx_g & 7) != 0 || (sx_n & 7) != 0) return false;
  if (role == TQ_ROLE_KEY) return bits == 2 || bits == 3;    // normal Lloyd bits 1-2, outlier 2-3
  return bits == 2 || bits == 3;                             // normal 2-3, outlier 3-4
}

size_t split256_workspace_bytes(int role, int64_t G) {
  return (size_t)G * (role == TQ_ROLE_KEY ? kFragsKey : kFragsValue) * kFragLanes * 16;
}

int launch_split256(int role, int bits, const Layout& Ln, const Layout& Lo, const void* cbn, const void* cbo,
                    int64_t n_cb, const void* x, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n,
                    const int32_t* chan, uint32_t* rec_n, uint32_t* rec_o, void* work, int32_t* status,
                    hipStream_t s) {
  const bool key = role == TQ_ROLE_KEY;
  const int frags = key ? kFragsKey : kFragsValue;
  PrepArgs p;
  p.cbn = static_cast<const uint8_t*>(cbn);
  p.cbo = static_cast<const uint8_t*>(cbo);
  p.stride_n = Ln.total;
  p.stride_o = Lo.total;
  p.n_cb = n_cb;
  p.off_dn = Ln.off_d; p.off_sn = Ln.off_s; p.off_do = Lo.off_d; p.off_so = Lo.off_s;
  p.chan = chan;
  p.frags = frags;
  p.work = static_cast<u32x4*>(work);
  p.status = status;
  hipLaunchKernelGGL(split256_prep_kernel, dim3((unsigned)((frags + 3) / 4), (unsigned)G), dim3(256), 0, s, p);
  if (hipGetLastError() != hipSuccess) return -10;

  SplitArgs a;
  a.frag = static_cast<const u32x4*>(work);
  a.cbn = p.cbn; a.cbo = p.cbo;
  a.stride_n = Ln.total; a.stride_o = Lo.total; a.n_cb = n_cb;
  a.off_cn = Ln.off_c; a.off_tn = Ln.off_t; a.off_co = Lo.off_c; a.off_to = Lo.off_t;
  a.bits_n = Ln.bits; a.bits_o = Lo.bits; a.role = role;
  a.x = static_cast<const uint32_t*>(x);
  a.G = G; a.N = N; a.sx_g = sx_g; a.sx_n = sx_n;
  a.rec_n = rec_n; a.rec_o = rec_o;
  a.status = status;
  a.frags = frags;
  a.tiles_per_group = (N + 31) / 32;
  // Many groups: one workgroup per CU (256), XCD-major, each group's tiles split
  // over the 32 workgroups of its XCD.  Few groups: about two workgroups per CU
  // over the launch, each on one group; whole 8-tile steps either way.
  a.xcd_major = G >= 32;
  int64_t bpg = a.xcd_major ? 32 : (512 + G - 1) / G;
  if (bpg > a.tiles_per_group) bpg = a.tiles_per_group;
  if (bpg < 1) bpg = 1;
  int64_t per_block = (a.tiles_per_group + bpg - 1) / bpg;
  per_block = (per_block + kWaves - 1) / kWaves * kWaves;
  a.tiles_per_block = per_block;
  a.blocks_per_group = a.xcd_major ? 32 : (a.tiles_per_group + per_block - 1) / per_block;
  if (key) return bits == 2 ? launch_split<1, 2, true>(a, s) : launch_split<2, 3, true>(a, s);
  return bits == 2 ? launch_split<2, 3, false>(a, s) : launch_split<3, 4, false>(a, s);
}

}  // namespace tq
