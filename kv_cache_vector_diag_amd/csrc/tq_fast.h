// Specialised (head_dim 128) kernels of libtq and their applicability tests.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_layout.h"

namespace tq {

// Encode with the MFMA kernel: head_dim 128; keys with 128 projections and
// 1..3 Lloyd bits; values with 1..4 bits; 16-byte aligned rows; a group's
// records under 2^30 bytes (32-bit buffer offsets).
// With `po` (paged output, Walsh-Hadamard codebooks), rec is a pool
// [num_pages][Hkv][tpp][rec_words]: the record of token t of group g goes to page
// page_table[b][pos[b] / tpp], slot pos[b] % tpp, kv head h, where (b, h) =
// (t, g) when head_major (groups are kv heads, tokens are sequences), else
// (g / Hkv, g % Hkv); a position or page outside the table or pool stores
// nothing and sets TQ_STATUS_BAD_PAGE.
struct PagedOut {
  const int32_t* page_table;
  const int32_t* pos;
  int64_t max_pages, num_pages, Hkv;
  int tpp;
  bool head_major;
};
bool fast128_encode_supported(const Layout& L, int dtype, const void* x, int64_t sx_g, int64_t sx_n, int64_t N);
int launch_encode_fast128(const Layout& L, const void* cbs, int64_t n_cb, const void* x, int dtype, int64_t G,
                          int64_t N, int64_t sx_g, int64_t sx_n, uint32_t* rec, int32_t* status, hipStream_t s,
                          const PagedOut* po = nullptr);
// The keys and values of a paged append in one launch (the value encode runs
// with the keys' workgroup shape) for bf16 inputs with 1 or 2 key planes and
// f16 with 1; returns 1, with nothing enqueued, for other shapes.
int launch_append_fast128(const Layout& K, const Layout& V, const void* kcbs, int64_t n_kcb, const void* vcbs,
                          int64_t n_vcb, const void* k, const void* v, int dtype, int64_t G, int64_t N, int64_t sx_g,
                          int64_t sx_n, uint32_t* kpool, uint32_t* vpool, int32_t* status, hipStream_t s,
                          const PagedOut& po);

// Keys and values of the same tokens in one launch (contiguous records): turbo3
// keys (2 planes) with 2- or 3-bit values, Walsh-Hadamard, f32 or bf16 inputs,
// both sides passing fast128_encode_supported.  Returns 1 (nothing launched)
// for other shapes.
int launch_encode_pair_fast128(const Layout& K, const Layout& V, const void* kcbs, int64_t n_kcb, const void* vcbs,
                               int64_t n_vcb, const void* k, const void* v, int dtype, int64_t G, int64_t N,
                               int64_t sx_g, int64_t sx_n, uint32_t* krec, uint32_t* vrec, int32_t* status,
                               hipStream_t s);

// Scores with the int8-MFMA kernel: head_dim 128, 128 projections, key bits
// 2..4, 1, 2 or 4 query heads per kv head, 8-byte aligned records, and a
// group's records and scores each under 2^30 bytes (32-bit buffer offsets).
bool fast128_scores_supported(const Layout& L, int64_t Hkv, int64_t Hq, int64_t T, const void* krec);
int launch_scores_fast128(const Layout& L, const void* cbs, int64_t n_cb, const uint32_t* krec, int64_t B,
                          int64_t Hkv, int64_t T, const void* q, int q_dtype, int64_t Hq, float scale,
                          float* scores, int32_t* status, hipStream_t s, const int32_t* page_table = nullptr,
                          int64_t max_pages = 0, int tpp = 0, int64_t num_pages = 0);

}  // namespace tq
