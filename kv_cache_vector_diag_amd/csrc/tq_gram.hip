// Gram-table scoring of block-codebook codes (gfx950, wave64).
//
// Page "fib-quant 0.1.0-beta.4 README": a head vector is cut into blocks and
// each block is replaced by the index of a codeword of a small codebook
// ("What's in the box", Codec; the rotation before it is the fast
// Walsh-Hadamard transform, Rotation).  Inner products with stored codes come
// from the codebook's Gram table G[i][j] = <c_i, c_j> with no decode ("New
// modules", Scoring).  Here:
//   encode: n = |x|, u = H(D x) / (sqrt(d) n); block b (k coordinates) takes
//           the nearest codeword in Euclidean distance, the lowest on ties,
//           decided on u rounded to float32 with float64 squared distances;
//   record: d/k indices of w = log2 N bits, LSB first at bit b w of the
//           little-endian words (an index may straddle two words), then
//           float32 n;
//   score:  s = scale n_q n_t sum_b G[cq_b][ct_b], the query encoded alike.
//
// The score reads 4 (d/k) w / 32 + 4 bytes per key and writes 4 per query
// head, so it is a streaming kernel: per (sequence, kv head) the query heads'
// rows of G, pre-scaled by scale n_q, sit in LDS as T[b][i][h], one 16-byte
// read per block for four heads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace {

__global__ void gram_table_kernel(const float* C, int N, int k, float* G) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N * N) return;
  const int i = e / N, j = e - i * N;
  float acc = 0.0f;
  for (int t = 0; t < k; ++t) acc = fmaf(C[i * k + t], C[j * k + t], acc);
  G[e] = acc;
}

// ---- encode: one wave per vector, four vectors per workgroup step.  Lane l
// holds coordinates l + 64 p (p < P = d/64; for d < 64 lane l < d holds l).
// The transform runs in float64 (exact sums of the float32 inputs): spans
// 1..32 across lanes, larger ones within the lane.  u = y / (sqrt(d) n32) is
// rounded to float32 and goes through LDS so that lanes own blocks; each block's
// squared distances to the codewords (float64, codebook in LDS, read as
// broadcasts) pick the nearest, the lowest index on ties.  With at most 32
// blocks, lanes b and b + 32 search the lower and upper half of the codebook.
constexpr int kEncWaves = 4;
constexpr int kMaxWords = 512 * 8 / 32;   // d/k indices of up to 8 bits: at most 128 words

template <int K, int P>
__global__ __launch_bounds__(64 * kEncWaves) void gram_encode_kernel(GramEncArgs a) {
  __shared__ double cb[256 * K];
  __shared__ float ub[kEncWaves][64 * P];
  __shared__ uint32_t wb[kEncWaves][kMaxWords];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < a.N * K; e += blockDim.x) cb[e] = (double)a.C[e];
  const int nw = a.rw - 1;
  const int nb = a.d / K;
  const bool halves = nb <= 32;
  const int hb = lane & 31, half = lane >> 5;
  const int i_lo = halves ? half * (a.N >> 1) : 0;
  const int i_hi = halves ? i_lo + (a.N >> 1) : a.N;
  const int64_t total = a.G * a.Nv;
  const double rsd = 1.0 / sqrt((double)a.d);
  // every wave runs the same number of steps, so the workgroup barriers match
  for (int64_t v0 = (int64_t)blockIdx.x * kEncWaves; v0 < total; v0 += (int64_t)gridDim.x * kEncWaves) {
    const int64_t v = v0 + wave;
    const bool live = v < total;
    const int64_t g = live ? v / a.Nv : 0, t = live ? v - g * a.Nv : 0;
    const int64_t base = g * a.sx_g + t * a.sx_n;
    double y[P];
    double ss = 0.0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int j = lane + 64 * p;
      double xv = 0.0;
      if (live && j < a.d) {
        xv = (double)load_elem(a.x, a.dtype, base + j);
        ss = fma(xv, xv, ss);
        if ((a.signs[j >> 5] >> (j & 31)) & 1u) xv = -xv;
      }
      y[p] = xv;
    }
    ss = wave_sum_f64(ss);
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
      if (h < a.d) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const double o = __shfl_xor(y[p], h, 64);
          y[p] = (lane & h) ? o - y[p] : y[p] + o;
        }
      }
    }
#pragma unroll
    for (int h2 = 1; h2 < P; h2 <<= 1) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (!(p & h2)) {
          const double a0 = y[p], b0 = y[p + h2];
          y[p] = a0 + b0;
          y[p + h2] = a0 - b0;
        }
      }
    }
    const bool finite = ss <= 3.4028234663852886e38;
    if (live && !finite && lane == 0 && a.status) atomicOr(a.status, TQ_STATUS_NON_FINITE);
    const float n32 = (float)sqrt(ss);
    const double sc = (finite && n32 > 0.0f) ? rsd / (double)n32 : 0.0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int j = lane + 64 * p;
      if (j < a.d) ub[wave][j] = (float)(y[p] * sc);
    }
    for (int w = lane; w < nw; w += 64) wb[wave][w] = 0u;
    __syncthreads();
    for (int b0 = 0; b0 < nb; b0 += halves ? 32 : 64) {
      const int b = b0 + (halves ? hb : lane);
      const bool own = b < nb;
      double u[K];
#pragma unroll
      for (int e = 0; e < K; ++e) u[e] = own ? (double)ub[wave][b * K + e] : 0.0;
      int best = i_lo;
      double bd = __builtin_inf();
      for (int i = i_lo; i < i_hi; ++i) {
        double dd = 0.0;
#pragma unroll
        for (int e = 0; e < K; ++e) {
          const double df = u[e] - cb[i * K + e];
          dd = fma(df, df, dd);
        }
        if (dd < bd) {
          bd = dd;
          best = i;
        }
      }
      if (halves) {
        // the upper half wins only when strictly nearer: ties keep the lower index
        const double od = __shfl_xor(bd, 32, 64);
        const int oi = __shfl_xor(best, 32, 64);
        if (od < bd) best = oi;
      }
      if (own && (!halves || half == 0)) {
        const int pos = b * a.W, wi = pos >> 5, sh = pos & 31;
        atomicOr(&wb[wave][wi], (uint32_t)best << sh);
        if (sh + a.W > 32) atomicOr(&wb[wave][wi + 1], (uint32_t)best >> (32 - sh));
      }
    }
    __syncthreads();
    if (live) {
      uint32_t* r = a.rec + v * a.rw;
      for (int w = lane; w < nw; w += 64) r[w] = wb[wave][w];
      if (lane == 0) r[nw] = __float_as_uint(n32);
    }
    __syncthreads();   // ub and wb are rewritten by the next step
  }
}

template <int K, int P>
int launch_encode_kp(const GramEncArgs& a, hipStream_t s) {
  const int64_t steps = (a.G * a.Nv + kEncWaves - 1) / kEncWaves;
  const int64_t blocks = steps < 8192 ? steps : 8192;
  hipLaunchKernelGGL((gram_encode_kernel<K, P>), dim3((unsigned)blocks), dim3(64 * kEncWaves), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : TQ_ERR_HIP;
}

template <int K>
int launch_encode_k(const GramEncArgs& a, hipStream_t s) {
  switch (a.d <= 64 ? 1 : a.d / 64) {
    case 1: return launch_encode_kp<K, 1>(a, s);
    case 2: return launch_encode_kp<K, 2>(a, s);
    case 4: return launch_encode_kp<K, 4>(a, s);
    case 8: return launch_encode_kp<K, 8>(a, s);
    default: return TQ_ERR_UNSUPPORTED;
  }
}

// ---- scores, fixed (w, d/k): one workgroup per (sequence, kv head, 1024 keys),
// one key per thread and pass.  The table T[b][i][h] = scale n_q G[cq_hb][i]
// (h < GQ) is built in the prologue; a key costs d/k LDS reads of GQ floats.
constexpr int kScoreThreads = 256;
constexpr int kScorePasses = 4;
constexpr int kKeysPerBlock = kScoreThreads * kScorePasses;

template <int W, int NB, int GQ>
__global__ __launch_bounds__(kScoreThreads) void gram_scores_fast_kernel(GramScoreArgs a) {
  constexpr int N = 1 << W;
  constexpr int RW = (NB * W + 31) / 32 + 1;
  __shared__ __align__(16) float tab[NB * N * GQ];
  const int tid = threadIdx.x;
  const int64_t grp = blockIdx.x / a.chunks, chunk = blockIdx.x - grp * a.chunks;
  const int64_t b = grp / a.Hkv, hkv = grp - b * a.Hkv;
  for (int e = tid; e < NB * N; e += kScoreThreads) {
    const int blk = e / N, i = e & (N - 1);
    const int pos = blk * W, wi = pos >> 5, sh = pos & 31;
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const uint32_t* qr = a.qrec + ((b * a.Hq) + hkv * GQ + h) * RW;
      const uint32_t lo = qr[wi], hi = (wi + 1 < RW - 1) ? qr[wi + 1] : 0u;
      const uint32_t cq = (uint32_t)((((uint64_t)hi << 32) | lo) >> sh) & (N - 1);
      tab[e * GQ + h] = a.scale * __uint_as_float(qr[RW - 1]) * a.G[cq * N + i];
    }
  }
  __syncthreads();
  // the group's records through a buffer resource: keys past T read as zero
  const uint32_t* kbase = a.krec + grp * a.T * RW;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(kbase), 0,
                                                          (int)(a.T * RW * 4), kRsrcWord3);
  const int64_t t0 = chunk * kKeysPerBlock + tid;
  uint32_t w[kScorePasses][RW];
#pragma unroll
  for (int r = 0; r < kScorePasses; ++r) {
    const uint32_t off = (uint32_t)((t0 + r * kScoreThreads) * RW * 4);
#pragma unroll
    for (int q = 0; q < RW; ++q) w[r][q] = __builtin_amdgcn_raw_buffer_load_b32(krs, off + 4 * q, 0, 0);
  }
  float* srow = a.scores + (b * a.Hq + hkv * GQ) * a.T;
#pragma unroll
  for (int r = 0; r < kScorePasses; ++r) {
    float acc[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      constexpr int kMask = N - 1;
      const int pos = blk * W, wi = pos >> 5, sh = pos & 31;
      const uint32_t idx = (sh + W <= 32 ? (w[r][wi] >> sh) : __builtin_amdgcn_alignbit(w[r][wi + 1], w[r][wi], sh)) &
                           kMask;
      const float* te = tab + (blk * N + idx) * GQ;
      if constexpr (GQ == 4) {
        const float4 tv = *reinterpret_cast<const float4*>(te);
        acc[0] += tv.x; acc[1] += tv.y; acc[2] += tv.z; acc[3] += tv.w;
      } else if constexpr (GQ == 2) {
        const float2 tv = *reinterpret_cast<const float2*>(te);
        acc[0] += tv.x; acc[1] += tv.y;
      } else {
        acc[0] += te[0];
      }
    }
    const int64_t t = t0 + r * kScoreThreads;
    if (t < a.T) {
      const float nt = __uint_as_float(w[r][RW - 1]);
#pragma unroll
      for (int h = 0; h < GQ; ++h) srow[h * a.T + t] = acc[h] * nt;
    }
  }
}

// ---- scores, any shape: one thread per (query head, key), G from memory.
__global__ __launch_bounds__(256) void gram_scores_generic_kernel(GramScoreArgs a, int W, int nb, int rw,
                                                                  int64_t tblocks) {
  const int64_t row = blockIdx.x / tblocks;            // b * Hq + hq
  const int64_t t = (blockIdx.x - row * tblocks) * 256 + threadIdx.x;
  if (t >= a.T) return;
  const int64_t b = row / a.Hq, hq = row - b * a.Hq, h = hq * a.Hkv / a.Hq;
  const uint32_t* qr = a.qrec + row * rw;
  const uint32_t* kr = a.krec + ((b * a.Hkv + h) * a.T + t) * rw;
  const uint32_t mask = (1u << W) - 1u;
  const int N = 1 << W;
  float acc = 0.0f;
  for (int blk = 0; blk < nb; ++blk) {
    const int pos = blk * W, wi = pos >> 5, sh = pos & 31;
    const bool two = sh + W > 32;
    const uint32_t cq = (uint32_t)((((uint64_t)(two ? qr[wi + 1] : 0u) << 32) | qr[wi]) >> sh) & mask;
    const uint32_t ct = (uint32_t)((((uint64_t)(two ? kr[wi + 1] : 0u) << 32) | kr[wi]) >> sh) & mask;
    acc += a.G[cq * N + ct];
  }
  a.scores[row * a.T + t] = a.scale * __uint_as_float(qr[rw - 1]) * __uint_as_float(kr[rw - 1]) * acc;
}

template <int W, int NB, int GQ>
int launch_fast(const GramScoreArgs& a, int64_t blocks, hipStream_t s) {
  hipLaunchKernelGGL((gram_scores_fast_kernel<W, NB, GQ>), dim3((unsigned)blocks), dim3(kScoreThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : TQ_ERR_HIP;
}

template <int W, int NB>
int launch_fast_gq(const GramScoreArgs& a, int gq, int64_t blocks, hipStream_t s) {
  switch (gq) {
    case 1: return launch_fast<W, NB, 1>(a, blocks, s);
    case 2: return launch_fast<W, NB, 2>(a, blocks, s);
    case 4: return launch_fast<W, NB, 4>(a, blocks, s);
    default: return TQ_ERR_UNSUPPORTED;
  }
}

// (w, d/k) pairs with a compiled fast kernel: N = 32 at d/k = 16, 32, 64 (head
// dims 64, 128, 256 with blocks of 4), and N = 16, 64 at d/k = 32.
bool fast_shape(int W, int nb) {
  return (W == 5 && (nb == 16 || nb == 32 || nb == 64)) || ((W == 4 || W == 6) && nb == 32);
}

}  // namespace

int launch_gram_table(const float* C, int N, int k, float* G, hipStream_t s) {
  const int n = N * N;
  hipLaunchKernelGGL(gram_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, C, N, k, G);
  return hipGetLastError() == hipSuccess ? 0 : TQ_ERR_HIP;
}

int launch_gram_encode(const GramEncArgs& a, hipStream_t s) {
  switch (a.k) {
    case 1: return launch_encode_k<1>(a, s);
    case 2: return launch_encode_k<2>(a, s);
    case 4: return launch_encode_k<4>(a, s);
    case 8: return launch_encode_k<8>(a, s);
    default: return TQ_ERR_UNSUPPORTED;
  }
}

int launch_gram_scores(GramScoreArgs a, int W, int nb, int rw, hipStream_t s) {
  const int64_t gq = a.Hq / a.Hkv;
  const int64_t groups = a.B * a.Hkv;
  // the fast kernel addresses a group's records with 32-bit offsets
  if (fast_shape(W, nb) && (gq == 1 || gq == 2 || gq == 4) && a.T * rw * 4 + kKeysPerBlock * rw * 4 < (1ll << 31)) {
    a.chunks = (a.T + kKeysPerBlock - 1) / kKeysPerBlock;
    const int64_t blocks = groups * a.chunks;
    if (W == 5 && nb == 16) return launch_fast_gq<5, 16>(a, (int)gq, blocks, s);
    if (W == 5 && nb == 32) return launch_fast_gq<5, 32>(a, (int)gq, blocks, s);
    if (W == 5 && nb == 64) return launch_fast_gq<5, 64>(a, (int)gq, blocks, s);
    if (W == 4) return launch_fast_gq<4, 32>(a, (int)gq, blocks, s);
    return launch_fast_gq<6, 32>(a, (int)gq, blocks, s);
  }
  const int64_t tblocks = (a.T + 255) / 256;
  if (a.B * a.Hq * tblocks > 0x7FFFFFFF) return TQ_ERR_UNSUPPORTED;   // one-dimensional grid
  hipLaunchKernelGGL(gram_scores_generic_kernel, dim3((unsigned)(a.B * a.Hq * tblocks)), dim3(256), 0, s, a, W, nb,
                     rw, tblocks);
  return hipGetLastError() == hipSuccess ? 0 : TQ_ERR_HIP;
}

}  // namespace tq
