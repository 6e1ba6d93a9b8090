// Value decode for Haar codebooks on the matrix cores (gfx950, wave64), head
// dims up to 256, any value bits, with the channel map of a split head vector
// (also Walsh-Hadamard codebooks under a channel map: there the matrix is the
// +-1 (D H)^T, generated in the fragments)
// (page "turboquant-plus-rs 0.1.0 README", Architecture step 1 and Modules
// rotation: Haar-distributed rotation via QR; "bitpolar 0.3.3
// src/kv_cache.rs", KvCacheCompressor::decode_values).  Same result as the
// one-wave-per-vector kernel it replaces there:
//   x^_i = (n/d) sum_j R[j][i] c[idx_j]   (R = sqrt(d) Q, row-major),
// written to out[v][map(i)].
//
// As a product of matrices, X^ (vectors x columns) = U R with U[v][j] =
// c[idx_vj]; on v_mfma_f32_32x32x16_f16 with both operands split into two
// binary16 terms (hi + lo, 22 significant bits, after an exact scaling by 16
// that keeps the lo terms of small entries normal), three products per step
// (hi.hi, hi.lo, lo.hi; lo.lo is below 2^-22 of the sum).
//   * A wave owns 32 vectors; their U fragments (all K-chunks of 16 rows) are
//     built once in registers from the index planes and the centroids.
//   * The workgroup (4 waves, 128 vectors of one group) walks R in slices of
//     32 columns: the slice's B fragments are built in LDS by all threads (all
//     loads in flight), then each wave runs its MFMAs and writes its 32 x 32
//     outputs, scaled by n/d, through the channel map.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

using namespace mf;

constexpr int kDBlock = 256;          // 4 waves
constexpr int kDVec = 128;            // vectors per workgroup (32 per wave)
constexpr float kPre = 16.0f;         // exact scaling of both operands before the split

struct DecHaarArgs {
  CodebookArgs cb;
  const uint32_t* rec;
  int64_t G, N;
  float* out;
  int64_t out_stride;
  ChannelMap cm;
  int32_t* status;
  int64_t tiles;                      // workgroups per group
};

// hi/lo binary16 terms of 8 scaled values, packed two per word
__device__ inline void split8(const float (&w)[8], u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split_f16x2(w[2 * q], w[2 * q + 1], kPre, h[q], l[q]);
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

template <int KC>   // K-chunks of 16 rows: d <= 16 KC
__global__ __launch_bounds__(kDBlock, 2) void decode_haar_kernel(DecHaarArgs a) {
  __shared__ float cent[256];
  __shared__ float nrm[kDVec];
  __shared__ u32x4 bhi[KC * 64];
  __shared__ u32x4 blo[KC * 64];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.cb.d, W = a.cb.plane_words, RW = a.cb.rec_words, K = a.cb.k;
  const int64_t g = blockIdx.x / a.tiles, v0 = (blockIdx.x % a.tiles) * kDVec;
  const uint8_t* blob = blob_of(a.cb, g);
  if (tid == 0 && a.status && blob_mismatch(a.cb, blob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  const float* cb_cent = reinterpret_cast<const float*>(blob + a.cb.off_c);
  const bool haar = a.cb.rotation == kRotHaar;
  const float* R = reinterpret_cast<const float*>(blob + a.cb.off_d);
  const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d);
  for (int i = tid; i < a.cb.levels; i += kDBlock) cent[i] = cb_cent[i];
  const uint32_t* grec = a.rec + g * a.N * RW;
  if (tid < kDVec) {
    const int64_t v = v0 + tid;
    nrm[tid] = v < a.N ? __uint_as_float(grec[v * RW + K * W]) : 0.0f;
  }
  __syncthreads();

  // U fragments of this wave's vectors: lane (col, h) holds vector v0 + 32 wave + col,
  // rows 16c + 8h .. +7 of K-chunk c
  const int64_t vv = v0 + 32 * wave + col;
  const bool vok = vv < a.N;
  const uint32_t* r = grec + (vok ? vv : 0) * RW;
  u32x4 ahi[KC], alo[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const int j = 16 * c + 8 * h;
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = 0.0f;
    if (vok && j < d) {
      int idx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int p = 0; p < K; ++p) {
        const uint32_t byte = (r[p * W + (j >> 5)] >> (j & 24)) & 0xFFu;
#pragma unroll
        for (int e = 0; e < 8; ++e) idx[e] |= (int)((byte >> e) & 1u) << p;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = j + e < d ? cent[idx[e]] : 0.0f;
    }
    split8(u, ahi[c], alo[c]);
  }

  const float post = 1.0f / ((float)d * kPre * kPre);
  for (int i0 = 0; i0 < d; i0 += 32) {
    __syncthreads();                                  // the previous slice is read
    // B fragments of columns i0 .. i0 + 31: entry (c, l) holds column i0 + (l & 31),
    // rows 16c + 8(l >> 5) .. +7 of R (zero past d)
#pragma unroll
    for (int t = 0; t < (KC * 64 + kDBlock - 1) / kDBlock; ++t) {
      const int e = tid + t * kDBlock;
      if (e >= KC * 64) break;
      const int c = e >> 6, l = e & 63;
      const int i = i0 + (l & 31), j = 16 * c + 8 * (l >> 5);
      float w[8];
      if (haar) {
#pragma unroll
        for (int q = 0; q < 8; ++q) w[q] = (i < d && j + q < d) ? R[(int64_t)(j + q) * d + i] : 0.0f;
      } else {
        // Walsh-Hadamard: entry (j, i) of (D H)^T is D_i (-1)^popc(i & j)
        const uint32_t di = i < d ? (dbits[i >> 5] >> (i & 31)) & 1u : 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q] = (i < d && j + q < d) ? (((__popc(i & (j + q)) & 1) ^ di) ? -1.0f : 1.0f) : 0.0f;
      }
      split8(w, bhi[e], blo[e]);
    }
    __syncthreads();
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 bh = bhi[c * 64 + lane], bl = blo[c * 64 + lane];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(ahi[c]), as<f16x8>(bh), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(ahi[c]), as<f16x8>(bl), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(alo[c]), as<f16x8>(bh), acc, 0, 0, 0);
    }
    // register k of lane half h holds vector row 8(k >> 2) + 4h + (k & 3), column col
    const int i = i0 + col;
    if (i < d) {
      const int ch = a.cm.channel(g, i, a.status);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int rho = 8 * (k >> 2) + 4 * h + (k & 3);
        const int64_t v = v0 + 32 * wave + rho;
        if (v < a.N) a.out[(g * a.N + v) * a.out_stride + ch] = acc[k] * nrm[32 * wave + rho] * post;
      }
    }
  }
}

template <int KC>
int launch_kc(const DecHaarArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_haar_kernel<KC>, dim3((unsigned)(a.G * a.tiles)), dim3(kDBlock), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace

bool haar_decode_mfma_supported(const CodebookArgs& cb, bool mapped) {
  if (cb.role != TQ_ROLE_VALUE || cb.k < 1 || cb.k > 8 || cb.d < 1 || cb.d > 256 || cb.levels > 256) return false;
  // Walsh-Hadamard codebooks come here with a channel map only (the
  // Walsh-Hadamard decode kernel writes whole rows)
  return cb.rotation == kRotHaar || (cb.rotation == kRotHadamard && mapped && !(cb.d & (cb.d - 1)));
}

int launch_decode_haar_mfma(const CodebookArgs& cb, const uint32_t* rec, int64_t G, int64_t N, float* out,
                            int32_t* status, hipStream_t s, int64_t out_stride, const ChannelMap& cm) {
  if (G * N == 0) return 0;
  DecHaarArgs a{cb, rec, G, N, out, out_stride > 0 ? out_stride : cb.d, cm, status, (N + kDVec - 1) / kDVec};
  const int kc = (cb.d + 15) / 16;
  if (kc <= 2) return launch_kc<2>(a, s);
  if (kc <= 4) return launch_kc<4>(a, s);
  if (kc <= 8) return launch_kc<8>(a, s);
  return launch_kc<16>(a, s);
}

}  // namespace tq
