// Allocation-free attention entry point: tq_attend with its scratch in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  Contract: include/tq.h.
//
// Each device the library runs on holds its own copy of `scratch` for the
// life of the process.  In host code the array's name is only a host-side
// stand-in, never a device address: its address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that pointer reaches kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/tq.h"
#include "tq_layout.h"

static __device__ __align__(256) uint8_t scratch[TQ_ATTEND_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = size_t(TQ_ATTEND_STATIC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, or null when it
// cannot be had (the caller reports TQ_ERR_HIP).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t tq_attend_static_scratch_bytes(void) { return kScratchBytes; }

int tq_attend_static(int head_dim, int k_bits, int v_bits, int projections, int rotation, const void* kcbs,
                     int64_t n_kcb, const void* vcbs, int64_t n_vcb, const void* krec, const void* vrec, int64_t B,
                     int64_t H_kv, int64_t T, const void* q, int q_dtype, int64_t H_q, float scale, float* out,
                     int32_t* status, void* stream) {
  // argument errors first, as tq_attend_ex reports them (nothing enqueued)
  tq::Layout L;
  int rc = tq::make_layout(head_dim, k_bits, projections, TQ_ROLE_KEY, &L, rotation);
  if (rc) return rc;
  rc = tq::make_layout(head_dim, v_bits, 0, TQ_ROLE_VALUE, &L, rotation);
  if (rc) return rc;
  if (B < 0 || T < 0 || H_q <= 0) return TQ_ERR_EMPTY_INPUT;
  const size_t need = tq_attend_workspace_bytes(head_dim, B, H_q, T);
  if (need > kScratchBytes) return TQ_ERR_SCRATCH_LIMIT;
  void* work = scratch_on_current_device();
  if (!work) return TQ_ERR_HIP;
  return tq_attend_ex(head_dim, k_bits, v_bits, projections, rotation, kcbs, n_kcb, vcbs, n_vcb, krec, vrec, B,
                      H_kv, T, q, q_dtype, H_q, scale, out, work, kScratchBytes, status, stream);
}

}  // extern "C"
