// Haar-rotation encode on the matrix cores for head_dim in (128, 256], a
// multiple of 8, bf16 input (page "turboquant-plus-rs 0.1.0 README",
// "Architecture" step 1 and "Modules" rotation: a Haar-distributed rotation
// via QR; then the Lloyd-Max codes and, for keys, the QJL signs of the
// residual and its norm).  Same device semantics as encode_generic_kernel with
// a Haar codebook, restated for throughput:
//
//  * u = R x, R = sqrt(d) Q (float32 in the blob), as bf16 MFMA products: R is
//    split into three bf16 pieces (t0 + t1 + t2 carries 24 bits), and every
//    product with a bf16 input is exact; the sums are float32.  The problem is
//    run as 256 x 256 with zero rows and columns of R past d and zero input
//    coordinates past d.
//  * R does not fit in LDS (384 KB as fragments), so it is streamed: for each
//    16-column K-chunk the workgroup converts R[:, 16c .. 16c+15] into the 24
//    fragments of that chunk (8 row tiles x 3 pieces, one (row tile, lane)
//    per thread) in one of two LDS buffers while the 8 waves run the previous
//    chunk's products, one barrier per chunk.  A wave owns a 32-token tile and
//    keeps the 8 row-tile accumulators (128 registers) in place.
//  * Quantizer and records as in the head_dim-128 encode: lane half h of
//    token col holds coordinates 32M + 16h + r in register r of tile M, so
//    index bits shift straight into 16-bit plane words.  Keys: the residual
//    w = u - n c[idx] (padded coordinates 0), scaled by a power of two and
//    split into binary16 hi + lo, overwrites u in the same registers; S w is
//    two f16 MFMAs per K-chunk with S fragments read straight from the blob
//    (16 bytes per lane, L2-resident), one 32-projection tile at a time.
//  * Records of the codebook's layout (ceil(d/32) plane words, ceil(m/32)
//    sign words, n, gamma) are assembled as half-words in a per-wave LDS row
//    and stored as the tile's contiguous records.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

using namespace mf;

constexpr int kDp = 256;                 // padded head_dim
constexpr int kMT = kDp / 32;            // row tiles (8)
constexpr int kKC = kDp / 16;            // K-chunks (16)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;
constexpr int kSliceFrags = kMT * 3;     // fragments of one K-chunk (24)
constexpr int kRecMax = 3 * 8 + 8 + 2;   // largest record (keys, 3 planes, 256 projections)

struct H256Args {
  const uint8_t* cbs;
  int64_t stride, n_cb;
  const uint16_t* x;                     // bf16
  int64_t G, N, sx_g, sx_n;
  uint32_t* rec;
  int32_t* status;
  int bits, role, rec_words, dv, mv;
  float inv_sqrt_dv;
  uint32_t off_c, off_t, off_d, off_s;
  int64_t tiles_per_group, tiles_per_block, blocks_per_group;
};

// LDS: two slice buffers, the record staging rows, the codebook constants.
constexpr size_t kLdsSlice = (size_t)kSliceFrags * 64 * 16;   // 24 KB
constexpr size_t kLdsStage = (size_t)kWaves * kTile * kRecMax * 4;
constexpr size_t kLdsBytes = 2 * kLdsSlice + kLdsStage + 128;

__device__ inline uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Fragments of K-chunk c into `buf`: thread (M, lane) builds fragments (M, t)
// for the three pieces t: A[rho][k] = t_t of R[32M + tile_row_index(rho)][16c + 8(lane/32) + k'].
__device__ inline void build_slice(u32x4* buf, const float* R, int dv, int c) {
  const int M = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = 32 * M + tile_row_index(lane & 31);
  const int col0 = 16 * c + 8 * (lane >> 5);
  float r[8];
  if (row < dv && col0 < dv) {
    const float4* p = reinterpret_cast<const float4*>(R + (int64_t)row * dv + col0);
    const float4 a = p[0], b = p[1];
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = 0.0f;
  }
  u32x4 v0, v1, v2;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w0 = 0, w1 = 0, w2 = 0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float x = r[2 * q + hh];
      const uint32_t b0 = bf16_rne(x);
      const float e1 = x - __uint_as_float(b0 << 16);
      const uint32_t b1 = bf16_rne(e1);
      const uint32_t b2 = bf16_rne(e1 - __uint_as_float(b1 << 16));
      w0 |= b0 << (16 * hh);
      w1 |= b1 << (16 * hh);
      w2 |= b2 << (16 * hh);
    }
    v0[q] = w0; v1[q] = w1; v2[q] = w2;
  }
  buf[(M * 3 + 0) * 64 + lane] = v0;
  buf[(M * 3 + 1) * 64 + lane] = v1;
  buf[(M * 3 + 2) * 64 + lane] = v2;
}

template <int K, bool KEY>
__global__ __launch_bounds__(kThreads) void haar256_kernel(H256Args a) {
  constexpr int L = 1 << K;
  constexpr int NT = L / 2 - 1;          // positive thresholds
  constexpr int KB = K - 1;              // magnitude bits
  extern __shared__ __align__(16) uint8_t smem[];
  const auto slice = [&](int b) { return reinterpret_cast<u32x4*>(smem + (size_t)b * kLdsSlice); };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem + 2 * kLdsSlice) + wave * kTile * kRecMax * 2;
  float* consts = reinterpret_cast<float*>(smem + 2 * kLdsSlice + kLdsStage);

  const int64_t g = blockIdx.x / a.blocks_per_group;
  const int64_t chunk = blockIdx.x % a.blocks_per_group;
  const uint8_t* blob = a.cbs + (g % a.n_cb) * a.stride;
  if (threadIdx.x == 0 && a.status) {
    const BlobHeader* hd = reinterpret_cast<const BlobHeader*>(blob);
    if (hd->magic != kBlobMagic || hd->version != kBlobVersion || hd->head_dim != a.dv || hd->bits != a.bits ||
        hd->role != a.role || hd->projections != (KEY ? a.mv : 0) || (int)hd->rotation != kRotHaar)
      atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  }
  const float* R = reinterpret_cast<const float*>(blob + a.off_d);
  const uint16_t* S = reinterpret_cast<const uint16_t*>(blob + a.off_s);
  if (threadIdx.x < L / 2) consts[threadIdx.x] = reinterpret_cast<const float*>(blob + a.off_c)[L / 2 + threadIdx.x];
  if (threadIdx.x < NT) consts[16 + threadIdx.x] = reinterpret_cast<const float*>(blob + a.off_t)[L / 2 + threadIdx.x];
  __syncthreads();
  float cpos[L / 2];
#pragma unroll
  for (int i = 0; i < L / 2; ++i) cpos[i] = consts[i];
  float tpos[NT > 0 ? NT : 1];
#pragma unroll
  for (int i = 0; i < NT; ++i) tpos[i] = consts[16 + i];

  const int dv = a.dv, RWo = a.rec_words;
  const int Wv = (dv + 31) / 32, SWv = (a.mv + 31) / 32;
  const int dlim = dv - 16 * h, mlim = a.mv - 16 * h;   // coordinate / projection 32M + 16h + r exists for r < lim - 32M
  const auto live16 = [](int n) -> uint32_t { return n <= 0 ? 0u : (n >= 16 ? 0xFFFFu : (1u << n) - 1u); };
  const __amdgpu_buffer_rsrc_t rrs =
      __builtin_amdgcn_make_buffer_rsrc(a.rec + g * a.N * RWo, 0, (int)(a.N * RWo * 4), kRsrcWord3);
  const int64_t tile0 = chunk * a.tiles_per_block;
  const int64_t tile_end = min(tile0 + a.tiles_per_block, a.tiles_per_group);

  // every wave runs every step (the chunk barriers); a wave past the range
  // encodes row 0 of the group and stores nothing
  for (int64_t tb = tile0; tb < tile_end; tb += kWaves) {
    const int64_t tile = tb + wave;
    const bool tile_ok = tile < tile_end;
    const int64_t tok = tile * kTile + col;
    const bool valid = tile_ok && tok < a.N;
    const uint16_t* xrow = a.x + g * a.sx_g + (valid ? tok : 0) * a.sx_n;
    const auto load_chunk = [&](int c) -> u32x4 {
      const int c0 = 16 * c + 8 * h;
      u32x4 v = *reinterpret_cast<const u32x4*>(xrow + (c0 < dv ? c0 : 0));
      if (c0 >= dv) v = u32x4{0u, 0u, 0u, 0u};
      return v;
    };

    // ---- rotation, chunk by chunk
    f32x16 u[kMT];
#pragma unroll
    for (int M = 0; M < kMT; ++M) u[M] = f32x16{};
    double ss = 0.0;
    build_slice(slice(0), R, dv, 0);
    u32x4 xc = load_chunk(0);
    __syncthreads();
#pragma unroll 1
    for (int c = 0; c < kKC; ++c) {
      u32x4 xn = xc;
      if (c + 1 < kKC) {
        build_slice(slice((c + 1) & 1), R, dv, c + 1);
        xn = load_chunk(c + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      const u32x4* buf = slice(c & 1) + lane;
#pragma unroll
      for (int M = 0; M < kMT; ++M) {
        // three fragment reads, three products: keeps the reads from being
        // hoisted ahead of all 24 products
        const u32x4 f0 = buf[(M * 3 + 0) * 64], f1 = buf[(M * 3 + 1) * 64], f2 = buf[(M * 3 + 2) * 64];
        u[M] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(f0), as<bf16x8>(xc), u[M], 0, 0, 0);
        u[M] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(f1), as<bf16x8>(xc), u[M], 0, 0, 0);
        u[M] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(f2), as<bf16x8>(xc), u[M], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      float part = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) part = sumsq2_bf16(xc[q], part);
      if (part < 0x1p-100f)
        ss += sumsq8_bf16_f64(xc);   // squares below the float32 range: the chunk again in float64
      else
        ss += (double)part;
      __syncthreads();
      xc = xn;
    }

    // ---- norm (both lane halves of the token)
    {
      const uint32_t lo = __double2loint(ss), hi = __double2hiint(ss);
      const auto plo = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      const auto phi = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      ss += __hiloint2double((int)(h ? phi[0] : phi[1]), (int)(h ? plo[0] : plo[1]));
    }
    const bool finite = ss <= 3.4028234663852886e38;
    if (a.status && __ballot(valid && !finite && h == 0) != 0 && lane == 0) atomicOr(a.status, TQ_STATUS_NON_FINITE);
    const float n32 = (float)sqrt(ss);
    const uint32_t nexp = (__float_as_uint(n32) >> 23) & 0xFFu;
    const float sc = (n32 > 0.0f && nexp < 253u) ? __uint_as_float((254u - nexp) << 23) : 1.0f;
    const uint32_t nbits = __float_as_uint(n32);
    float tn[NT > 0 ? NT : 1];
#pragma unroll
    for (int t = 0; t < NT; ++t) tn[t] = tpos[t] * n32;

    // ---- quantize: plane half-words of each tile straight into the staging
    // row (plane p word M < Wv at p Wv + M, half h); keys: residual split in place
    uint16_t* st = stage + col * RWo * 2;
    // the padding limit, opaque per step so that its per-coordinate masks are
    // made where they are used instead of held in registers across the loop
    int dl = dlim;
    asm volatile("" : "+v"(dl));
    const auto put = [&](int p, int M, uint32_t v) {
      if (M < Wv) st[2 * (p * Wv + M) + h] = (uint16_t)v;
    };
    u32x4 whi[KEY ? kMT : 1][2], wlo[KEY ? kMT : 1][2];
    float wsh = 0.0f, wsl = 0.0f;   // (w sc)^2 as hi.hi + 2 hi.lo
#pragma unroll
    for (int M = 0; M < kMT; ++M) {
      const uint32_t vm = live16(dl - 32 * M);
      uint32_t pacc = 0;
      if constexpr (!KEY) {
        uint32_t macc[KB > 0 ? KB : 1];
#pragma unroll
        for (int b = 0; b < KB; ++b) macc[b] = 0;
#pragma unroll
        for (int r = 15; r >= 0; --r) {
          const float uu = u[M][r];
          pos_bit(pacc, uu);
          if constexpr (KB == 1) {
            thr_bit(macc[0], uu, tn[0]);
          } else if constexpr (KB == 2) {
            const uint64_t m1 = thr_bit(macc[1], uu, tn[1]);
            thr_bit(macc[0], uu, sel_mask(m1, tn[2], tn[0]));
          } else if constexpr (KB == 3) {
            const uint64_t m2 = thr_bit(macc[2], uu, tn[3]);
            const uint64_t m1 = thr_bit(macc[1], uu, sel_mask(m2, tn[5], tn[1]));
            const float ta = sel_mask(m2, tn[6], tn[2]), tb = sel_mask(m2, tn[4], tn[0]);
            thr_bit(macc[0], uu, sel_mask(m1, ta, tb));
          }
        }
        put(K - 1, M, pacc & vm);
#pragma unroll
        for (int p = 0; p < KB; ++p) put(p, M, ~(macc[p] ^ pacc) & vm);   // pos ? cnt_p : ~cnt_p
      } else {
        uint32_t tacc[NT > 0 ? NT : 1];
#pragma unroll
        for (int t = 0; t < NT; ++t) tacc[t] = 0;
        float wv[16];
#pragma unroll
        for (int r = 15; r >= 0; --r) {
          const float uu = u[M][r];
          float nsg;
          pos_step(pacc, nsg, uu, nbits, 0x80000000u);      // pos bit; nsg = pos ? -n : n
          float mag = cpos[0];
          if (NT > 0) mag = thr_first(tacc[0], uu, tn[0], cpos[0], cpos[NT > 0 ? 1 : 0]);
#pragma unroll
          for (int t = 1; t < NT; ++t) thr_step(tacc[t], mag, uu, tn[t], cpos[t + 1]);
          // u - n c[idx]; 0 at a padded coordinate (bit r of vm clear)
          const float w = __uint_as_float(__float_as_uint(fmaf(nsg, mag, uu)) & (uint32_t)__builtin_amdgcn_sbfe((int)vm, r, 1));
          wv[r] = w;
          if ((r & 3) == 0) __builtin_amdgcn_sched_barrier(0);   // four coordinates at a time
        }
        put(K - 1, M, pacc & vm);
#pragma unroll
        for (int p = 0; p < K - 1; ++p) {
          // bit p of cnt = XOR of the thermometer bits [cnt >= j] for j a multiple of 2^p
          uint32_t cb = 0;
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (((t + 1) & ((1 << p) - 1)) == 0) cb ^= tacc[t];
          put(p, M, ~(cb ^ pacc) & vm);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t hw, lw;
            split_f16x2(wv[8 * p + 2 * q], wv[8 * p + 2 * q + 1], sc, hw, lw);
            split_sumsq(hw, lw, wsh, wsl);
            whi[KEY ? M : 0][p][q] = hw;
            wlo[KEY ? M : 0][p][q] = lw;
          }
      }
      // one tile at a time: its accumulator dies as its residual is made
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- record staging: signs, n, gamma
    if (KEY) {
      // QJL: one 32-projection tile at a time, S fragments from the blob
      const int npt = SWv;
      for (int Mp = 0; Mp < npt; ++Mp) {
        int dvm = dv;
        asm volatile("" : "+v"(dvm));   // per-chunk S addresses made inside the loop
        const int proj = 32 * Mp + tile_row_index(col);
        const bool pok = proj < a.mv;
        f32x16 acc{};
        const uint16_t* srow = S + (int64_t)(pok ? proj : 0) * dvm;
        // S fragments two K-chunks ahead of their products
        u32x4 sfq[3];
        const auto sload = [&](int c) -> u32x4 {
          const int c0 = qjl_coord(c, h, 0);
          u32x4 v = *reinterpret_cast<const u32x4*>(srow + (c0 < dvm ? c0 : 0));
          if (!pok || c0 >= dvm) v = u32x4{0u, 0u, 0u, 0u};
          return v;
        };
        sfq[0] = sload(0);
        sfq[1] = sload(1);
#pragma unroll
        for (int c = 0; c < kKC; ++c) {
          if (c + 2 < kKC) sfq[(c + 2) % 3] = sload(c + 2);
          const u32x4 sf = sfq[c % 3];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf), as<f16x8>(whi[c >> 1][c & 1]), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf), as<f16x8>(wlo[c >> 1][c & 1]), acc, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        uint32_t sw = 0;   // bit r: projection 32 Mp + 16 h + r negative
#pragma unroll
        for (int r = 15; r >= 0; --r) sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(acc[r]), 31);
        st[2 * (K * Wv + Mp) + h] = (uint16_t)(~sw & live16(mlim - 32 * Mp));
      }
      const float wsq = fmaf(2.0f, wsl, wsh);
      const auto pg = __builtin_amdgcn_permlane32_swap(__float_as_uint(wsq), __float_as_uint(wsq), false, false);
      const float gam = sqrtf(__uint_as_float(pg[0]) + __uint_as_float(pg[1])) / sc * a.inv_sqrt_dv;
      if (h == 0) {
        reinterpret_cast<uint32_t*>(st)[K * Wv + SWv] = nbits;
        reinterpret_cast<uint32_t*>(st)[K * Wv + SWv + 1] = __float_as_uint(gam);
      }
    } else {
      if (h == 0) reinterpret_cast<uint32_t*>(st)[K * Wv] = nbits;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (tile_ok) {
      const int ntok = (int)(a.N - tile * kTile < kTile ? a.N - tile * kTile : kTile);
      const uint32_t base = (uint32_t)(tile * kTile * RWo * 4);
      const uint32_t* st32 = reinterpret_cast<const uint32_t*>(stage);
      for (int e = lane; e < ntok * RWo; e += 64) __builtin_amdgcn_raw_buffer_store_b32(st32[e], rrs, base + 4u * e, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int K, bool KEY>
int launch_k(H256Args a, hipStream_t s) {
  // about two workgroups per CU in total, whole steps of 8 tiles
  int64_t per = (a.tiles_per_group * a.G + 511) / 512;
  per = (per + kWaves - 1) / kWaves * kWaves;
  if (per < kWaves) per = kWaves;
  if (per > a.tiles_per_group) per = (a.tiles_per_group + kWaves - 1) / kWaves * kWaves;
  a.tiles_per_block = per;
  a.blocks_per_group = (a.tiles_per_group + per - 1) / per;
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&haar256_kernel<K, KEY>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes) != hipSuccess)
      return TQ_ERR_HIP;
    attr_set = true;
  }
  hipLaunchKernelGGL((haar256_kernel<K, KEY>), dim3((unsigned)(a.G * a.blocks_per_group)), dim3(kThreads), kLdsBytes,
                     s, a);
  return hipGetLastError() == hipSuccess ? 0 : TQ_ERR_HIP;
}

}  // namespace

bool haar256_supported(const CodebookArgs& cb, int dtype, const void* x, int64_t sx_g, int64_t sx_n, int64_t N) {
  if (cb.rotation != kRotHaar || dtype != TQ_BF16) return false;
  if (cb.d <= 128 || cb.d > kDp || (cb.d & 7)) return false;
  if (cb.role == TQ_ROLE_KEY && (cb.k < 1 || cb.k > 3 || cb.m < 1 || cb.m > kDp)) return false;
  if (cb.role == TQ_ROLE_VALUE && (cb.k < 1 || cb.k > 4)) return false;
  if (cb.rec_words > kRecMax) return false;
  if ((reinterpret_cast<uintptr_t>(x) & 15) || ((sx_g * 2) & 15) || ((sx_n * 2) & 15)) return false;
  if ((cb.off_d & 15) || (cb.off_s & 15) || (cb.stride & 15)) return false;   // 16-byte rows of R and S
  return N <= (int64_t(1) << 30) / (4 * cb.rec_words);                // 32-bit offsets per group
}

int launch_haar256(const CodebookArgs& cb, const void* x, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n,
                   uint32_t* rec, int32_t* status, hipStream_t s) {
  if (G * N == 0) return 0;
  H256Args a;
  a.cbs = cb.cbs; a.stride = cb.stride; a.n_cb = cb.n_cb;
  a.x = static_cast<const uint16_t*>(x);
  a.G = G; a.N = N; a.sx_g = sx_g; a.sx_n = sx_n;
  a.rec = rec; a.status = status;
  a.bits = cb.bits; a.role = cb.role; a.rec_words = cb.rec_words; a.dv = cb.d;
  a.mv = cb.role == TQ_ROLE_KEY ? cb.m : 0;
  a.inv_sqrt_dv = (float)(1.0 / sqrt((double)cb.d));
  a.off_c = cb.off_c; a.off_t = cb.off_t; a.off_d = cb.off_d; a.off_s = cb.off_s;
  a.tiles_per_group = (N + kTile - 1) / kTile;
  a.tiles_per_block = a.blocks_per_group = 0;
  const bool key = cb.role == TQ_ROLE_KEY;
  switch (cb.k * 2 + (key ? 1 : 0)) {
    case 1 * 2 + 1: return launch_k<1, true>(a, s);
    case 2 * 2 + 1: return launch_k<2, true>(a, s);
    case 3 * 2 + 1: return launch_k<3, true>(a, s);
    case 1 * 2: return launch_k<1, false>(a, s);
    case 2 * 2: return launch_k<2, false>(a, s);
    case 3 * 2: return launch_k<3, false>(a, s);
    case 4 * 2: return launch_k<4, false>(a, s);
  }
  return TQ_ERR_UNSUPPORTED;
}

}  // namespace tq
