// Paged compressed cache (gfx950): the records of one new token per
// (sequence, kv head), encoded together into a staging area, are written to
// their pool pages (page "fib-quant 0.1.0-beta.4 README", "Streaming KV
// encoder": token-by-token construction into pages of tokens_per_page tokens;
// page "bitpolar 0.3.3 src/kv_cache.rs", MultiHeadKvCache::push_token).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kScatterBlock = 256;

struct ScatterArgs {
  const uint32_t* staged;      // record (b, h) at staged[(h * sb + b) * rw] (head-major) or [(b*Hkv + h) * rw]
  int head_major;
  int64_t B, Hkv, sb;
  int rw;                      // record words
  const int32_t* pos;
  const int32_t* page_table;
  int64_t max_pages, num_pages;
  int tpp;                     // tokens per page
  uint32_t* pool;              // [num_pages][Hkv][tpp][rw]
  int32_t* status;
};

// One thread per record word; consecutive threads take consecutive words of a
// record, so a record's store is one contiguous run.
__global__ __launch_bounds__(kScatterBlock) void page_scatter_kernel(ScatterArgs a) {
  const int64_t e = (int64_t)blockIdx.x * kScatterBlock + threadIdx.x;
  if (e >= a.B * a.Hkv * a.rw) return;
  const int w = (int)(e % a.rw);
  const int64_t bh = e / a.rw, b = bh / a.Hkv, h = bh % a.Hkv;
  const int64_t p = a.pos[b];
  const int64_t pi = p >= 0 ? p / a.tpp : -1;
  const int64_t page = pi >= 0 && pi < a.max_pages ? a.page_table[b * a.max_pages + pi] : -1;
  if (page < 0 || page >= a.num_pages) {
    if (w == 0 && h == 0 && a.status) atomicOr(a.status, TQ_STATUS_BAD_PAGE);
    return;
  }
  const int64_t src = a.head_major ? (h * a.sb + b) : (b * a.Hkv + h);
  a.pool[((page * a.Hkv + h) * a.tpp + p % a.tpp) * a.rw + w] = a.staged[src * a.rw + w];
}

}  // namespace

int launch_page_scatter(const uint32_t* staged, bool head_major, int64_t B, int64_t Hkv, int rw,
                        const int32_t* pos, const int32_t* page_table, int64_t max_pages, int tpp,
                        int64_t num_pages, uint32_t* pool, int32_t* status, hipStream_t s) {
  const int64_t n = B * Hkv * rw;
  if (n == 0) return 0;
  ScatterArgs a{staged, head_major ? 1 : 0, B, Hkv, B, rw, pos, page_table, max_pages, num_pages, tpp, pool, status};
  hipLaunchKernelGGL(page_scatter_kernel, dim3((unsigned)((n + kScatterBlock - 1) / kScatterBlock)),
                     dim3(kScatterBlock), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace tq
