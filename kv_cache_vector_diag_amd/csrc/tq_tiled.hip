// Encode for any power-of-two head_dim in [32, 512], any bit width and any
// number of projections, 32 vectors per workgroup step (page
// "turboquant-plus-rs 0.1.0 README", "Architecture": PolarQuant codes, then for
// keys the QJL signs of a Gaussian projection of the residual).  Same device
// semantics as encode_generic_kernel, built for wide codebooks (7-8 bit keys,
// 8-bit values) and large projection counts:
//
//  * Phase A (each of the 4 waves, 8 vectors): lane l holds coordinates
//    l + 64e in registers.  u = H(D x) in float64: the lane-bit stages by
//    cross-lane exchange, the e-bit stages in registers, in the same stage
//    order as the one-wave kernel.  Several vectors go through at once so
//    that the exchanges, reductions and codebook searches overlap.  Quantizer
//    from the LDS codebook, bit planes by ballot; keys: residual
//    w = u - n32 c[idx] (float32 copy in LDS) and gamma.
//  * Phase B (keys): S w for the 32 vectors as MFMA tiles, C[32 projections]
//    [32 vectors] += S[32][16] W[16][32].  S is exact in binary16; w is scaled
//    by a power of two (|w| sc in [2^14, 2^15), so every w_j sc fits binary16)
//    and split into two binary16 terms carrying 22 bits, summed in float32.
//    The sign of S w is the sign of the scaled product; the representation and
//    accumulation errors stay near 1e-7 |w|, inside the 1e-6 |w| decision band.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

using namespace mf;

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kVec = 32;                  // vectors per workgroup step (the MFMA tile width)
constexpr int kVecPerWave = kVec / kWaves;

struct TiledArgs {
  CodebookArgs cb;
  const void* x;
  int dtype;
  int64_t G, N, sx_g, sx_n;
  uint32_t* rec;
  int32_t* status;
  int64_t tiles_per_group;
};

// LDS carve-up (bytes), shared by the kernel and its launcher.  w rows are
// padded by 16 bytes so that the 32 vector rows of an MFMA operand read fall
// in different banks.
struct TiledLds {
  size_t wt, words, cb, scl, total;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) / 16 * 16; }

__host__ __device__ inline TiledLds tiled_lds(bool key, int d, int rec_words) {
  TiledLds o;
  o.wt = 0;
  o.words = key ? align16((size_t)kVec * (d + 4) * 4) : 0;
  o.cb = o.words + align16((size_t)kVec * rec_words * 4);
  o.scl = o.cb + 2 * 256 * 4;
  o.total = o.scl + kVec * 4;
  return o;
}

// 2^(14 - floor(log2 |w|)) as a float32 power of two (1 for |w| = 0).
__device__ inline float residual_scale(double wn) {
  const float f = (float)wn;
  if (!(f > 0.0f) || !(f < 3.0e38f)) return 1.0f;
  const int e = (int)((__float_as_uint(f) >> 23) & 0xFFu) - 127;   // floor(log2 f) for normal f
  int se = 14 - (e < -126 ? -126 : e);
  se = se > 127 ? 127 : se;
  return __uint_as_float((uint32_t)(se + 127) << 23);
}

template <int D, bool KEY>
__global__ __launch_bounds__(kThreads) void encode_tiled_kernel(TiledArgs a) {
  constexpr int E = D >= kWave ? D / kWave : 1;     // coordinates per lane
  constexpr int V = E >= 8 ? 1 : 8 / E;             // vectors in flight per wave
  constexpr int LH = D >= kWave ? kWave / 2 : D / 2;  // largest lane-bit stage
  constexpr int SP = D + 4;                         // w row stride (floats)
  static_assert(kVecPerWave % V == 0, "vectors per wave");

  extern __shared__ __align__(16) uint8_t smem[];
  const int W = a.cb.plane_words, RW = a.cb.rec_words;
  const TiledLds lay = tiled_lds(KEY, D, RW);
  float* wt = reinterpret_cast<float*>(smem + lay.wt);          // [kVec][SP]
  uint32_t* words = reinterpret_cast<uint32_t*>(smem + lay.words);   // [kVec][RW]
  float* cent = reinterpret_cast<float*>(smem + lay.cb);
  float* thr = cent + 256;
  float* scl = reinterpret_cast<float*>(smem + lay.scl);        // [kVec]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool live = lane < D;
  const int k = a.cb.k, levels = a.cb.levels;
  const int n_off = k * W + (KEY ? a.cb.sign_words : 0);
  const int64_t total_tiles = a.G * a.tiles_per_group;
  int64_t g_loaded = -1;
  for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    const int64_t g = tile / a.tiles_per_group;
    const int64_t t0 = (tile % a.tiles_per_group) * kVec;
    const uint8_t* blob = blob_of(a.cb, g);
    if (tid == 0 && a.status && blob_mismatch(a.cb, blob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
    __syncthreads();                                   // the previous step is done with every buffer
    if (g % a.cb.n_cb != g_loaded) {
      for (int i = tid; i < levels; i += kThreads) {
        cent[i] = reinterpret_cast<const float*>(blob + a.cb.off_c)[i];
        thr[i] = reinterpret_cast<const float*>(blob + a.cb.off_t)[i];
      }
      g_loaded = g % a.cb.n_cb;
    }
    // sign flips of this lane's coordinates
    const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d);
    uint32_t flip = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane + kWave * e;
      if (live) flip |= ((dbits[j >> 5] >> (j & 31)) & 1u) << e;
    }
    __syncthreads();

    // ---- phase A: this wave encodes vectors wave*8 .. wave*8+7, V at a time
    for (int v0 = wave * kVecPerWave; v0 < (wave + 1) * kVecPerWave; v0 += V) {
      double u[V][E], ss[V];
      bool valid[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int64_t t = t0 + v0 + i;
        valid[i] = t < a.N;
        const int64_t base = g * a.sx_g + (valid[i] ? t : 0) * a.sx_n;
        ss[i] = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const double xv = (valid[i] && live) ? (double)load_elem(a.x, a.dtype, base + lane + kWave * e) : 0.0;
          ss[i] += xv * xv;
          u[i][e] = ((flip >> e) & 1u) ? -xv : xv;
        }
      }
#pragma unroll
      for (int i = 0; i < V; ++i) ss[i] = wave_sum_f64(ss[i]);
      // Walsh-Hadamard stages h = 1, 2, ..., D/2: lane bits, then register bits
#pragma unroll
      for (int h = 1; h <= LH; h <<= 1) {
        const bool upper = (lane & h) != 0;
#pragma unroll
        for (int i = 0; i < V; ++i)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const double p = __shfl_xor(u[i][e], h, kWave);
            u[i][e] = upper ? p - u[i][e] : u[i][e] + p;
          }
      }
#pragma unroll
      for (int he = 1; he < E; he <<= 1)
#pragma unroll
        for (int i = 0; i < V; ++i)
#pragma unroll
          for (int e = 0; e < E; ++e)
            if ((e & he) == 0) {
              const double x0 = u[i][e], x1 = u[i][e + he];
              u[i][e] = x0 + x1;
              u[i][e + he] = x0 - x1;
            }
      int q[V][E];
      double ws[V];
      float n32[V];
      float z[V][E];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double nrm = sqrt(ss[i]);
        n32[i] = (float)nrm;
        ws[i] = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          z[i][e] = z_up(u[i][e], nrm);
          q[i][e] = 0;
        }
      }
      // idx = #{t_i < z} over t[0 .. levels-2]: a branch-free binary search of
      // log2(levels) steps, the V*E searches interleaved step by step
#pragma unroll
      for (int b = 7; b >= 0; --b) {
        const int st = 1 << b;
        if (st < levels) {
#pragma unroll
          for (int i = 0; i < V; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) q[i][e] += thr[q[i][e] + st - 1] < z[i][e] ? st : 0;
        }
      }
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int vl = v0 + i;
        if (KEY) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const double r = u[i][e] - (double)n32[i] * (double)cent[q[i][e]];
            if (live) {
              ws[i] += r * r;
              wt[vl * SP + lane + kWave * e] = (float)r;
            }
          }
        }
        uint32_t* wd = words + vl * RW;
        for (int p = 0; p < k; ++p) {
          // the plane's W words gathered into lanes 0 .. W-1, one store
          uint32_t pw = 0;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const uint64_t bl = __ballot(live && ((q[i][e] >> p) & 1));
            pw = lane == 2 * e ? (uint32_t)bl : pw;
            pw = lane == 2 * e + 1 ? (uint32_t)(bl >> 32) : pw;
          }
          if (lane < W) wd[p * W + lane] = pw;
        }
        if (lane == 0) wd[n_off] = __float_as_uint(n32[i]);
      }
      if (KEY) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          ws[i] = wave_sum_f64(ws[i]);
          if (lane == 0) {
            words[(v0 + i) * RW + n_off + 1] = __float_as_uint((float)(sqrt(ws[i]) / sqrt((double)D)));
            scl[v0 + i] = residual_scale(sqrt(ws[i]));
          }
        }
      }
    }
    __syncthreads();

    if (KEY) {
      // ---- phase B: wave handles projection blocks rb = wave, wave+4, ...
      const int m = a.cb.m, nblk = (m + 31) / 32;
      const _Float16* S = reinterpret_cast<const _Float16*>(blob + a.cb.off_s);
      const int col = lane & 31, h = lane >> 5;          // vector column, lane half
      const float sc = scl[col];
      const float* wrow = wt + col * SP + 8 * h;
      for (int rb = wave; rb < nblk; rb += kWaves) {
        const int row = 32 * rb + col;                   // S row fed by this lane
        const bool rok = row < m;
        const _Float16* srow = S + (int64_t)(rok ? row : 0) * D + 8 * h;
        f32x16 acc = {};
#pragma unroll 4
        for (int c = 0; c < D / 16; ++c) {
          u32x4 sf = {0u, 0u, 0u, 0u};
          if (rok) sf = *reinterpret_cast<const u32x4*>(srow + 16 * c);
          const float4 w0 = *reinterpret_cast<const float4*>(wrow + 16 * c);
          const float4 w1 = *reinterpret_cast<const float4*>(wrow + 16 * c + 4);
          uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
          split_f16x2(w0.x, w0.y, sc, h0, l0);
          split_f16x2(w0.z, w0.w, sc, h1, l1);
          split_f16x2(w1.x, w1.y, sc, h2, l2);
          split_f16x2(w1.z, w1.w, sc, h3, l3);
          const u32x4 hi = {h0, h1, h2, h3}, lo = {l0, l1, l2, l3};
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf), as<f16x8>(hi), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf), as<f16x8>(lo), acc, 0, 0, 0);
        }
        // acc[r] of lane (col, h) is projection 32 rb + 8(r/4) + 4h + (r%4) of vector col
        uint32_t bits = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pr = 8 * (r >> 2) + 4 * h + (r & 3);
          if (acc[r] >= 0.0f && 32 * rb + pr < m) bits |= 1u << pr;
        }
        bits |= (uint32_t)__shfl_xor((int)bits, 32, kWave);
        if (h == 0) words[col * RW + k * W + rb] = bits;
      }
      __syncthreads();
    }

    // ---- records of the step's valid vectors (contiguous in rec)
    const int nv = (int)(a.N - t0 < kVec ? a.N - t0 : kVec);
    uint32_t* out = a.rec + (g * a.N + t0) * RW;
    for (int e = tid; e < nv * RW; e += kThreads) out[e] = words[e];
  }
}

template <int D, bool KEY>
int launch_tiled(const TiledArgs& a, hipStream_t s) {
  const size_t lds = tiled_lds(KEY, D, a.cb.rec_words).total;
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&encode_tiled_kernel<D, KEY>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return TQ_ERR_HIP;
    attr_set = true;
  }
  const int64_t tiles = a.G * a.tiles_per_group;
  const int64_t grid = tiles < 4096 ? tiles : 4096;
  hipLaunchKernelGGL((encode_tiled_kernel<D, KEY>), dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  return hipGetLastError() == hipSuccess ? 0 : TQ_ERR_HIP;
}

template <bool KEY>
int launch_tiled_d(const TiledArgs& a, hipStream_t s) {
  switch (a.cb.d) {
    case 32: return launch_tiled<32, KEY>(a, s);
    case 64: return launch_tiled<64, KEY>(a, s);
    case 128: return launch_tiled<128, KEY>(a, s);
    case 256: return launch_tiled<256, KEY>(a, s);
    case 512: return launch_tiled<512, KEY>(a, s);
  }
  return TQ_ERR_BAD_DIMENSION;
}

}  // namespace

bool tiled_encode_supported(const CodebookArgs& cb) {
  const bool key = cb.role == TQ_ROLE_KEY;
  return cb.rotation == kRotHadamard && cb.d >= 32 && cb.d <= kMaxHeadDim && (cb.d & (cb.d - 1)) == 0 &&
         cb.levels <= 256 && tiled_lds(key, cb.d, cb.rec_words).total <= 160 * 1024;
}

int launch_encode_tiled(const CodebookArgs& cb, const void* x, int dtype, int64_t G, int64_t N, int64_t sx_g,
                        int64_t sx_n, uint32_t* rec, int32_t* status, hipStream_t s) {
  if (G * N == 0) return 0;
  const TiledArgs a{cb, x, dtype, G, N, sx_g, sx_n, rec, status, (N + kVec - 1) / kVec};
  return cb.role == TQ_ROLE_KEY ? launch_tiled_d<true>(a, s) : launch_tiled_d<false>(a, s);
}

}  // namespace tq
