// Outlier channel selection for the outlier/normal split of mixed-precision
// layers (page "turboquant-plus-rs 0.1.0 README", "Modules" outlier: channels
// split into outlier and normal parts for non-integer bit rates).
//
// Per group (layer, kv-head) the n_out channels with the largest population
// variance over the group's N vectors become the outlier part; ties go to the
// lower channel index.  Stage 1 reduces float64 sums of x and x^2 per channel
// over chunks of tokens (deterministic: fixed chunking, no atomics); stage 2
// adds the chunks in order, forms var = E[x^2] - E[x]^2 and ranks.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kStatBlock = 256;
constexpr int64_t kRowsPerChunk = 512;
constexpr int64_t kMaxChunks = 64;

struct StatArgs {
  const void* x;
  int dtype;
  int64_t G, N, sx_g, sx_n;
  int d;
  int64_t chunks, rows;
  double* work;   // [G][chunks][d][2]
};

// One workgroup per (group, chunk).  Thread t owns channels t, t + 256 (d <= 512);
// each row is read contiguously across the workgroup.
__global__ __launch_bounds__(kStatBlock) void channel_stats_kernel(StatArgs a) {
  const int64_t g = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
  const int64_t r0 = c * a.rows;
  const int64_t r1 = r0 + a.rows < a.N ? r0 + a.rows : a.N;
  const int tid = threadIdx.x;
  double s1[2] = {0.0, 0.0}, s2[2] = {0.0, 0.0};
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t base = g * a.sx_g + r * a.sx_n;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = tid + k * kStatBlock;
      if (j < a.d) {
        const double v = (double)load_elem(a.x, a.dtype, base + j);
        s1[k] += v;
        s2[k] = fma(v, v, s2[k]);
      }
    }
  }
  double* out = a.work + ((g * a.chunks + c) * a.d) * 2;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int j = tid + k * kStatBlock;
    if (j < a.d) {
      out[2 * j] = s1[k];
      out[2 * j + 1] = s2[k];
    }
  }
}

// Same sums with four channels per 8- or 16-byte load: thread t reads channels
// 4(t % tpr) .. +3 of rows r0 + t / tpr, r0 + t / tpr + rp, ... (tpr = d / 4
// threads per row, rp = 256 / tpr rows per pass, four passes in flight); the
// rp partial sums of each channel are then added in row-group order.
template <int DT>
__global__ __launch_bounds__(kStatBlock) void channel_stats_vec_kernel(StatArgs a) {
  __shared__ double part[kStatBlock][4][2];
  const int64_t g = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
  const int64_t r0 = c * a.rows;
  const int64_t r1 = r0 + a.rows < a.N ? r0 + a.rows : a.N;
  const int tid = threadIdx.x;
  const int tpr = a.d / 4, rp = kStatBlock / tpr;
  const int cq = tid % tpr, rg = tid / tpr;
  double s1[4] = {0.0, 0.0, 0.0, 0.0}, s2[4] = {0.0, 0.0, 0.0, 0.0};
  if (rg < rp) {
    constexpr int kUnroll = 4;
    for (int64_t rb = r0 + rg; rb < r1; rb += (int64_t)kUnroll * rp) {
      float v[kUnroll][4];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t r = rb + (int64_t)u * rp;
        const int64_t off = g * a.sx_g + (r < r1 ? r : r0) * a.sx_n + 4 * cq;
        if (DT == 0) {
          const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + off);
          v[u][0] = f.x; v[u][1] = f.y; v[u][2] = f.z; v[u][3] = f.w;
        } else {
          const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + off);
          const uint32_t w[2] = {b.x, b.y};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t hb = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            v[u][e] = DT == 1 ? bf16_bits_to_float(hb) : (float)__builtin_bit_cast(_Float16, (uint16_t)hb);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (rb + (int64_t)u * rp < r1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const double x = (double)v[u][e];
            s1[e] += x;
            s2[e] = fma(x, x, s2[e]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    part[tid][e][0] = s1[e];
    part[tid][e][1] = s2[e];
  }
  __syncthreads();
  double* out = a.work + ((g * a.chunks + c) * a.d) * 2;
  for (int j = tid; j < a.d; j += kStatBlock) {
    double t1 = 0.0, t2 = 0.0;
    for (int q = 0; q < rp; ++q) {
      const int src = q * tpr + j / 4;
      t1 += part[src][j & 3][0];
      t2 += part[src][j & 3][1];
    }
    out[2 * j] = t1;
    out[2 * j + 1] = t2;
  }
}

struct SelectArgs {
  const double* work;
  int64_t G, N, chunks;
  int d, n_out;
  int32_t* chan;   // [G][d]
};

// One workgroup per group: variance per channel, rank, then the channel map
// [outliers ascending, normal channels ascending].
__global__ __launch_bounds__(kStatBlock) void select_outliers_kernel(SelectArgs a) {
  __shared__ double var[kMaxHeadDim];
  __shared__ int is_out[kMaxHeadDim];
  const int64_t g = blockIdx.x;
  const int tid = threadIdx.x;
  const double inv_n = a.N > 0 ? 1.0 / (double)a.N : 0.0;
  for (int j = tid; j < a.d; j += kStatBlock) {
    double s1 = 0.0, s2 = 0.0;
    for (int64_t c = 0; c < a.chunks; ++c) {
      const double* p = a.work + ((g * a.chunks + c) * a.d + j) * 2;
      s1 += p[0];
      s2 += p[1];
    }
    const double mean = s1 * inv_n;
    var[j] = a.N > 0 ? s2 * inv_n - mean * mean : 0.0;
  }
  __syncthreads();
  for (int j = tid; j < a.d; j += kStatBlock) {
    const double vj = var[j];
    int rank = 0;
    for (int i = 0; i < a.d; ++i) {
      const double vi = var[i];
      rank += (vi > vj || (vi == vj && i < j)) ? 1 : 0;
    }
    is_out[j] = rank < a.n_out ? 1 : 0;
  }
  __syncthreads();
  for (int j = tid; j < a.d; j += kStatBlock) {
    int before_out = 0;
    for (int i = 0; i < j; ++i) before_out += is_out[i];
    const int pos = is_out[j] ? before_out : a.n_out + (j - before_out);
    a.chan[g * a.d + pos] = j;
  }
}

}  // namespace

int64_t outlier_chunks(int64_t N) {
  int64_t c = (N + kRowsPerChunk - 1) / kRowsPerChunk;
  return c < 1 ? 1 : (c > kMaxChunks ? kMaxChunks : c);
}

int launch_outlier_channels(const void* x, int dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, int d,
                            int n_out, int32_t* chan, double* work, hipStream_t s) {
  if (G == 0) return 0;
  const int64_t chunks = outlier_chunks(N);
  const int64_t rows = (N + chunks - 1) / chunks;
  StatArgs sa{x, dtype, G, N, sx_g, sx_n, d, chunks, rows, work};
  const int esz = dtype == TQ_F32 ? 4 : 2;
  const bool vec = d % 4 == 0 && d / 4 <= kStatBlock && N > 0 &&
                   (reinterpret_cast<uintptr_t>(x) % (4 * esz)) == 0 && (sx_g * esz) % (4 * esz) == 0 &&
                   (sx_n * esz) % (4 * esz) == 0;
  const dim3 grid((unsigned)(G * chunks));
  if (!vec)
    hipLaunchKernelGGL(channel_stats_kernel, grid, dim3(kStatBlock), 0, s, sa);
  else if (dtype == TQ_F32)
    hipLaunchKernelGGL(channel_stats_vec_kernel<0>, grid, dim3(kStatBlock), 0, s, sa);
  else if (dtype == TQ_BF16)
    hipLaunchKernelGGL(channel_stats_vec_kernel<1>, grid, dim3(kStatBlock), 0, s, sa);
  else
    hipLaunchKernelGGL(channel_stats_vec_kernel<2>, grid, dim3(kStatBlock), 0, s, sa);
  if (hipGetLastError() != hipSuccess) return -10;
  SelectArgs la{work, G, N, chunks, d, n_out, chan};
  hipLaunchKernelGGL(select_outliers_kernel, dim3((unsigned)G), dim3(kStatBlock), 0, s, la);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace tq
