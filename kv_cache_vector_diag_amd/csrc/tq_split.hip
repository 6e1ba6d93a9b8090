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
  hipLaunchKernelGGL(channel_stats_kernel, dim3((unsigned)(G * chunks)), dim3(kStatBlock), 0, s, sa);
  if (hipGetLastError() != hipSuccess) return -10;
  SelectArgs la{work, G, N, chunks, d, n_out, chan};
  hipLaunchKernelGGL(select_outliers_kernel, dim3((unsigned)G), dim3(kStatBlock), 0, s, la);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace tq
