// extern "C" entry points of libtq that touch the device: host-side argument
// validation (synchronous, nothing enqueued on error), then dispatch to the
// kernel launchers.  Contract: include/tq.h.
#include <hip/hip_runtime.h>

#include "../../include/tq.h"
#include "tq_fast.h"
#include "tq_kernels.h"
#include "tq_layout.h"

using namespace tq;

namespace {

bool dtype_ok(int dt) { return dt == TQ_F32 || dt == TQ_BF16 || dt == TQ_F16; }

// Checks shared by the encode/rotate entry points.
int check_input(const Layout& L, const void* cbs, int64_t n_cb, const void* x, int dtype, int64_t G,
                int64_t N, int64_t sx_g, int64_t sx_n) {
  if (n_cb <= 0 || G < 0 || N < 0) return TQ_ERR_EMPTY_INPUT;
  if (G == 0 || N == 0) return TQ_OK;
  if (!cbs || !x) return TQ_ERR_NULL;
  if (!dtype_ok(dtype)) return TQ_ERR_UNSUPPORTED;
  if ((N > 1 && sx_n < L.d) || (G > 1 && sx_g < L.d) || sx_n < 0 || sx_g < 0) return TQ_ERR_DIMENSION_MISMATCH;
  return TQ_OK;
}

// Layouts of the two parts of a split head vector: normal part (Haar, bits),
// outlier part (Walsh-Hadamard, bits + 1); keys project each part onto as many
// signs as it has coordinates.
int split_layouts(int role, int head_dim, int n_outlier, int bits, Layout* Ln, Layout* Lo) {
  if (role != TQ_ROLE_KEY && role != TQ_ROLE_VALUE) return TQ_ERR_INVALID_ROLE;
  if (head_dim == 0) return TQ_ERR_ZERO_DIMENSION;
  if (head_dim < 2 || head_dim > kMaxHeadDim) return TQ_ERR_BAD_DIMENSION;
  if (n_outlier <= 0 || n_outlier >= head_dim) return TQ_ERR_DIMENSION_MISMATCH;
  const int dn = head_dim - n_outlier;
  const bool key = role == TQ_ROLE_KEY;
  int rc = make_layout(dn, bits, key ? dn : 0, role, Ln, kRotHaar);
  if (rc) return rc;
  return make_layout(n_outlier, bits + 1, key ? n_outlier : 0, role, Lo, kRotHadamard);
}

int encode_common(int role, int head_dim, int bits, int projections, int rotation, const void* cbs, int64_t n_cb,
                  const void* x, int x_dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, void* rec,
                  int32_t* status, void* stream) {
  Layout L;
  int rc = make_layout(head_dim, bits, projections, role, &L, rotation);
  if (rc) return rc;
  rc = check_input(L, cbs, n_cb, x, x_dtype, G, N, sx_g, sx_n);
  if (rc || G * N == 0) return rc;
  if (!rec) return TQ_ERR_NULL;
  if (fast128_encode_supported(L, x_dtype, x, sx_g, sx_n, N))
    return launch_encode_fast128(L, cbs, n_cb, x, x_dtype, G, N, sx_g, sx_n, static_cast<uint32_t*>(rec), status,
                                 static_cast<hipStream_t>(stream));
  CodebookArgs cb = make_cb_args(cbs, n_cb, L);
  if (haar256_supported(cb, x_dtype, x, sx_g, sx_n, N))
    return launch_haar256(cb, x, G, N, sx_g, sx_n, static_cast<uint32_t*>(rec), status,
                          static_cast<hipStream_t>(stream));
  if (wide_encode_supported(cb, x_dtype, x, sx_g, sx_n, N))
    return launch_encode_wide(cb, x, x_dtype, G, N, sx_g, sx_n, static_cast<uint32_t*>(rec), status,
                              static_cast<hipStream_t>(stream));
  if (tiled_encode_supported(cb))
    return launch_encode_tiled(cb, x, x_dtype, G, N, sx_g, sx_n, static_cast<uint32_t*>(rec), status,
                               static_cast<hipStream_t>(stream));
  return launch_encode_generic(cb, x, x_dtype, G, N, sx_g, sx_n, static_cast<uint32_t*>(rec), status,
                               static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int tq_encode_keys_ex(int head_dim, int bits, int projections, int rotation, const void* cbs, int64_t n_cb,
                      const void* x, int x_dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, void* rec,
                      int32_t* status, void* stream) {
  return encode_common(TQ_ROLE_KEY, head_dim, bits, projections, rotation, cbs, n_cb, x, x_dtype, G, N, sx_g, sx_n,
                       rec, status, stream);
}

int tq_encode_keys(int head_dim, int bits, int projections, const void* cbs, int64_t n_cb, const void* x,
                   int x_dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, void* rec, int32_t* status,
                   void* stream) {
  return tq_encode_keys_ex(head_dim, bits, projections, kRotHadamard, cbs, n_cb, x, x_dtype, G, N, sx_g, sx_n, rec,
                           status, stream);
}

int tq_encode_values_ex(int head_dim, int bits, int rotation, const void* cbs, int64_t n_cb, const void* x,
                        int x_dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, void* rec, int32_t* status,
                        void* stream) {
  return encode_common(TQ_ROLE_VALUE, head_dim, bits, 0, rotation, cbs, n_cb, x, x_dtype, G, N, sx_g, sx_n, rec,
                       status, stream);
}

int tq_encode_values(int head_dim, int bits, const void* cbs, int64_t n_cb, const void* x, int x_dtype,
                     int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, void* rec, int32_t* status,
                     void* stream) {
  return tq_encode_values_ex(head_dim, bits, kRotHadamard, cbs, n_cb, x, x_dtype, G, N, sx_g, sx_n, rec, status,
                             stream);
}

int tq_decode_values(int head_dim, int bits, const void* cbs, int64_t n_cb, const void* rec, int64_t G,
                     int64_t N, float* out, int32_t* status, void* stream) {
  return tq_decode_values_ex(head_dim, bits, kRotHadamard, cbs, n_cb, rec, G, N, out, status, stream);
}

int tq_decode_values_ex(int head_dim, int bits, int rotation, const void* cbs, int64_t n_cb, const void* rec,
                        int64_t G, int64_t N, float* out, int32_t* status, void* stream) {
  Layout L;
  int rc = make_layout(head_dim, bits, 0, TQ_ROLE_VALUE, &L, rotation);
  if (rc) return rc;
  if (n_cb <= 0 || G < 0 || N < 0) return TQ_ERR_EMPTY_INPUT;
  if (G * N == 0) return TQ_OK;
  if (!cbs || !rec || !out) return TQ_ERR_NULL;
  CodebookArgs cb = make_cb_args(cbs, n_cb, L);
  if (decode_wh_supported(cb, G, N, out))
    return launch_decode_wh(cb, static_cast<const uint32_t*>(rec), G, N, out, status,
                            static_cast<hipStream_t>(stream));
  return launch_decode_generic(cb, static_cast<const uint32_t*>(rec), G, N, out, status,
                               static_cast<hipStream_t>(stream));
}

int tq_encode_kv(int head_dim, int k_bits, int v_bits, int projections, const void* kcbs, int64_t n_kcb,
                 const void* vcbs, int64_t n_vcb, const void* k, const void* v, int x_dtype, int64_t G, int64_t N,
                 int64_t sx_g, int64_t sx_n, void* krec, void* vrec, int32_t* status, void* stream) {
  Layout K, V;
  int rc = make_layout(head_dim, k_bits, projections, TQ_ROLE_KEY, &K, kRotHadamard);
  if (rc) return rc;
  rc = make_layout(head_dim, v_bits, 0, TQ_ROLE_VALUE, &V, kRotHadamard);
  if (rc) return rc;
  rc = check_input(K, kcbs, n_kcb, k, x_dtype, G, N, sx_g, sx_n);
  if (rc || G * N == 0) return rc;
  rc = check_input(V, vcbs, n_vcb, v, x_dtype, G, N, sx_g, sx_n);
  if (rc) return rc;
  if (!krec || !vrec) return TQ_ERR_NULL;
  if (fast128_encode_supported(K, x_dtype, k, sx_g, sx_n, N) && fast128_encode_supported(V, x_dtype, v, sx_g, sx_n, N)) {
    rc = launch_encode_pair_fast128(K, V, kcbs, n_kcb, vcbs, n_vcb, k, v, x_dtype, G, N, sx_g, sx_n,
                                    static_cast<uint32_t*>(krec), static_cast<uint32_t*>(vrec), status,
                                    static_cast<hipStream_t>(stream));
    if (rc != 1) return rc;
  }
  // other shapes: the two encodes one after the other
  rc = tq_encode_keys(head_dim, k_bits, projections, kcbs, n_kcb, k, x_dtype, G, N, sx_g, sx_n, krec, status, stream);
  if (rc) return rc;
  return tq_encode_values(head_dim, v_bits, vcbs, n_vcb, v, x_dtype, G, N, sx_g, sx_n, vrec, status, stream);
}

int tq_scores(int head_dim, int bits, int projections, const void* cbs, int64_t n_cb, const void* krec,
              int64_t B, int64_t H_kv, int64_t T, const void* q, int q_dtype, int64_t H_q, float scale,
              float* scores, int32_t* status, void* stream) {
  return tq_scores_ex(head_dim, bits, projections, kRotHadamard, cbs, n_cb, krec, B, H_kv, T, q, q_dtype, H_q, scale,
                      scores, status, stream);
}

int tq_scores_ex(int head_dim, int bits, int projections, int rotation, const void* cbs, int64_t n_cb,
                 const void* krec, int64_t B, int64_t H_kv, int64_t T, const void* q, int q_dtype, int64_t H_q,
                 float scale, float* scores, int32_t* status, void* stream) {
  Layout L;
  int rc = make_layout(head_dim, bits, projections, TQ_ROLE_KEY, &L, rotation);
  if (rc) return rc;
  if (n_cb <= 0 || B < 0 || H_kv <= 0 || T < 0 || H_q <= 0) return TQ_ERR_EMPTY_INPUT;
  if (H_q % H_kv) return TQ_ERR_DIMENSION_MISMATCH;
  if (B * T == 0) return TQ_OK;
  if (!cbs || !krec || !q || !scores) return TQ_ERR_NULL;
  if (!dtype_ok(q_dtype)) return TQ_ERR_UNSUPPORTED;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf((float)head_dim);
  if (fast128_scores_supported(L, H_kv, H_q, T, krec))
    return launch_scores_fast128(L, cbs, n_cb, static_cast<const uint32_t*>(krec), B, H_kv, T, q, q_dtype, H_q,
                                 scale, scores, status, static_cast<hipStream_t>(stream));
  CodebookArgs cb = make_cb_args(cbs, n_cb, L);
  return launch_scores_generic(cb, static_cast<const uint32_t*>(krec), B, H_kv, T, q, q_dtype, H_q, scale,
                               scores, status, static_cast<hipStream_t>(stream));
}

// Scratch of tq_attend: the scores [B][H_q][T] or, on the fused path, the
// prepared query side of each (b, kv head) (at most B*H_q of them), then
// (256-byte aligned) the per-chunk partials [B*H_q][ceil(T/512)][head_dim + 2]
// of the split softmax.
static size_t attend_scores_bytes(int64_t B, int64_t H_q, int64_t T) {
  const size_t sc = (size_t)(B * H_q * T) * sizeof(float), qp = attend_qprep_bytes(B * H_q);
  return ((sc > qp ? sc : qp) + 255) / 256 * 256;
}

size_t tq_attend_workspace_bytes(int head_dim, int64_t B, int64_t H_q, int64_t T) {
  if (head_dim < 2 || head_dim > kMaxHeadDim || B < 0 || H_q < 0 || T < 0) return 0;
  // partials of the finer of the two chunkings (the fused pass's)
  const int64_t chunks = attend_fused_chunks(T) > attend_chunks(T) ? attend_fused_chunks(T) : attend_chunks(T);
  return attend_scores_bytes(B, H_q, T) + (size_t)(B * H_q * chunks * (head_dim + 2)) * sizeof(float) +
         256;
}

int tq_attend(int head_dim, int k_bits, int v_bits, int projections, const void* kcbs, int64_t n_kcb,
              const void* vcbs, int64_t n_vcb, const void* krec, const void* vrec, int64_t B, int64_t H_kv,
              int64_t T, const void* q, int q_dtype, int64_t H_q, float scale, float* out, void* work,
              size_t work_bytes, int32_t* status, void* stream) {
  return tq_attend_ex(head_dim, k_bits, v_bits, projections, kRotHadamard, kcbs, n_kcb, vcbs, n_vcb, krec, vrec, B,
                      H_kv, T, q, q_dtype, H_q, scale, out, work, work_bytes, status, stream);
}

int tq_attend_ex(int head_dim, int k_bits, int v_bits, int projections, int rotation, const void* kcbs,
                 int64_t n_kcb, const void* vcbs, int64_t n_vcb, const void* krec, const void* vrec, int64_t B,
                 int64_t H_kv, int64_t T, const void* q, int q_dtype, int64_t H_q, float scale, float* out,
                 void* work, size_t work_bytes, int32_t* status, void* stream) {
  Layout K, V;
  int rc = make_layout(head_dim, k_bits, projections, TQ_ROLE_KEY, &K, rotation);
  if (rc) return rc;
  rc = make_layout(head_dim, v_bits, 0, TQ_ROLE_VALUE, &V, rotation);
  if (rc) return rc;
  if (n_kcb <= 0 || n_vcb <= 0 || B < 0 || H_kv <= 0 || T < 0 || H_q <= 0) return TQ_ERR_EMPTY_INPUT;
  if (H_q % H_kv) return TQ_ERR_DIMENSION_MISMATCH;
  if (B == 0) return TQ_OK;
  if (!kcbs || !vcbs || !q || !out || (T > 0 && (!krec || !vrec || !work))) return TQ_ERR_NULL;
  if (!dtype_ok(q_dtype)) return TQ_ERR_UNSUPPORTED;
  if (work_bytes < tq_attend_workspace_bytes(head_dim, B, H_q, T)) return TQ_ERR_DIMENSION_MISMATCH;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf((float)head_dim);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* sc = static_cast<float*>(work);
  CodebookArgs kcb = make_cb_args(kcbs, n_kcb, K);
  CodebookArgs vcb = make_cb_args(vcbs, n_vcb, V);
  if (T > 0 && attend_fused_supported(kcb, vcb, H_kv, H_q, T, krec)) {
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(work) + attend_scores_bytes(B, H_q, T));
    return launch_attend_fused(kcb, vcb, static_cast<const uint32_t*>(krec), static_cast<const uint32_t*>(vrec), B,
                               H_kv, T, q, q_dtype, H_q, scale, static_cast<uint8_t*>(work), part, out, status, s);
  }
  if (T > 0) {
    rc = fast128_scores_supported(K, H_kv, H_q, T, krec)
             ? launch_scores_fast128(K, kcbs, n_kcb, static_cast<const uint32_t*>(krec), B, H_kv, T, q, q_dtype,
                                     H_q, scale, sc, status, s)
             : launch_scores_generic(kcb, static_cast<const uint32_t*>(krec), B, H_kv, T, q, q_dtype, H_q, scale,
                                     sc, status, s);
    if (rc) return rc;
  }
  if (attend_split_supported(vcb)) {
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(work) + attend_scores_bytes(B, H_q, T));
    return launch_attend_split(vcb, static_cast<const uint32_t*>(vrec), sc, B, H_kv, T, H_q, part, out, s);
  }
  return launch_attend_generic(vcb, static_cast<const uint32_t*>(vrec), sc, B, H_kv, T, H_q, out, s);
}

int tq_scores_paged(int head_dim, int bits, int projections, const void* cbs, int64_t n_cb, const void* kpool,
                    const int32_t* page_table, int64_t max_pages, int tokens_per_page, int64_t num_pages, int64_t B,
                    int64_t H_kv, int64_t T, const void* q, int q_dtype, int64_t H_q, float scale, float* scores,
                    int32_t* status, void* stream) {
  Layout L;
  int rc = make_layout(head_dim, bits, projections, TQ_ROLE_KEY, &L);
  if (rc) return rc;
  if (n_cb <= 0 || B < 0 || H_kv <= 0 || T < 0 || H_q <= 0 || num_pages < 0) return TQ_ERR_EMPTY_INPUT;
  if (H_q % H_kv) return TQ_ERR_DIMENSION_MISMATCH;
  if (B * T == 0) return TQ_OK;
  if (tokens_per_page <= 0 || tokens_per_page % 32 || max_pages <= 0) return TQ_ERR_DIMENSION_MISMATCH;
  if (!cbs || !kpool || !page_table || !q || !scores) return TQ_ERR_NULL;
  if (!dtype_ok(q_dtype)) return TQ_ERR_UNSUPPORTED;
  if (!fast128_scores_supported(L, H_kv, H_q, T, kpool)) return TQ_ERR_UNSUPPORTED;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf((float)head_dim);
  return launch_scores_fast128(L, cbs, n_cb, static_cast<const uint32_t*>(kpool), B, H_kv, T, q, q_dtype, H_q, scale,
                               scores, status, static_cast<hipStream_t>(stream), page_table, max_pages,
                               tokens_per_page, num_pages);
}

// Scratch of tq_append_kv: the new keys' records, then (256-byte aligned) the
// new values' records, B*H_kv of each.
static size_t append_stage_bytes(const Layout& L, int64_t B, int64_t H_kv) {
  return ((size_t)(B * H_kv * L.rec_words) * 4 + 255) / 256 * 256;
}

size_t tq_append_workspace_bytes(int head_dim, int k_bits, int v_bits, int projections, int64_t B, int64_t H_kv) {
  Layout K, V;
  if (make_layout(head_dim, k_bits, projections, TQ_ROLE_KEY, &K) ||
      make_layout(head_dim, v_bits, 0, TQ_ROLE_VALUE, &V) || B < 0 || H_kv < 0)
    return 0;
  return append_stage_bytes(K, B, H_kv) + append_stage_bytes(V, B, H_kv);
}

int tq_append_kv(int head_dim, int k_bits, int v_bits, int projections, const void* kcbs, int64_t n_kcb,
                 const void* vcbs, int64_t n_vcb, const void* k_new, const void* v_new, int x_dtype, int64_t B,
                 int64_t H_kv, const int32_t* pos, const int32_t* page_table, int64_t max_pages,
                 int tokens_per_page, int64_t num_pages, void* kpool, void* vpool, void* work, size_t work_bytes,
                 int32_t* status, void* stream) {
  Layout K, V;
  int rc = make_layout(head_dim, k_bits, projections, TQ_ROLE_KEY, &K);
  if (rc) return rc;
  rc = make_layout(head_dim, v_bits, 0, TQ_ROLE_VALUE, &V);
  if (rc) return rc;
  if (n_kcb <= 0 || n_vcb <= 0 || B < 0 || H_kv <= 0 || num_pages < 0) return TQ_ERR_EMPTY_INPUT;
  if (B == 0) return TQ_OK;
  if (tokens_per_page <= 0 || max_pages <= 0) return TQ_ERR_DIMENSION_MISMATCH;
  if (!kcbs || !vcbs || !k_new || !v_new || !pos || !page_table || !kpool || !vpool || !work) return TQ_ERR_NULL;
  if (!dtype_ok(x_dtype)) return TQ_ERR_UNSUPPORTED;
  if (work_bytes < tq_append_workspace_bytes(head_dim, k_bits, v_bits, projections, B, H_kv))
    return TQ_ERR_DIMENSION_MISMATCH;
  uint32_t* kst = static_cast<uint32_t*>(work);
  uint32_t* vst = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(work) + append_stage_bytes(K, B, H_kv));
  // When the codebook of (b, h) is that of h for every b (n_cb divides H_kv),
  // the new vectors are encoded as H_kv groups of B tokens (head-major), so the
  // batch of sequences fills the encode kernel's tiles; else one group per vector.
  const bool head_major = H_kv % n_kcb == 0 && H_kv % n_vcb == 0;
  const int64_t G = head_major ? H_kv : B * H_kv, N = head_major ? B : 1;
  const int64_t sx_g = head_dim, sx_n = head_major ? H_kv * head_dim : head_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The MFMA encode writes each record straight into its page slot (head_dim 128).
  if (head_dim == 128 && fast128_encode_supported(K, x_dtype, k_new, sx_g, sx_n, N) &&
      fast128_encode_supported(V, x_dtype, v_new, sx_g, sx_n, N)) {
    const PagedOut po{page_table, pos, max_pages, num_pages, H_kv, tokens_per_page, head_major};
    rc = launch_append_fast128(K, V, kcbs, n_kcb, vcbs, n_vcb, k_new, v_new, x_dtype, G, N, sx_g, sx_n,
                               static_cast<uint32_t*>(kpool), static_cast<uint32_t*>(vpool), status, s, po);
    if (rc != 1) return rc;
    rc = launch_encode_fast128(K, kcbs, n_kcb, k_new, x_dtype, G, N, sx_g, sx_n, static_cast<uint32_t*>(kpool),
                               status, s, &po);
    if (rc) return rc;
    return launch_encode_fast128(V, vcbs, n_vcb, v_new, x_dtype, G, N, sx_g, sx_n, static_cast<uint32_t*>(vpool),
                                 status, s, &po);
  }
  rc = encode_common(TQ_ROLE_KEY, head_dim, k_bits, projections, kRotHadamard, kcbs, n_kcb, k_new, x_dtype, G, N,
                     sx_g, sx_n, kst, status, stream);
  if (rc) return rc;
  rc = encode_common(TQ_ROLE_VALUE, head_dim, v_bits, 0, kRotHadamard, vcbs, n_vcb, v_new, x_dtype, G, N, sx_g,
                     sx_n, vst, status, stream);
  if (rc) return rc;
  rc = launch_page_scatter(kst, head_major, B, H_kv, K.rec_words, pos, page_table, max_pages, tokens_per_page,
                           num_pages, static_cast<uint32_t*>(kpool), status, s);
  if (rc) return rc;
  return launch_page_scatter(vst, head_major, B, H_kv, V.rec_words, pos, page_table, max_pages, tokens_per_page,
                             num_pages, static_cast<uint32_t*>(vpool), status, s);
}

int tq_rotate(int head_dim, int bits, int projections, int role, const void* cbs, int64_t n_cb, const void* x,
              int x_dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, float* u, float* norms,
              void* stream) {
  Layout L;
  int rc = make_layout(head_dim, bits, projections, role, &L);
  if (rc) return rc;
  rc = check_input(L, cbs, n_cb, x, x_dtype, G, N, sx_g, sx_n);
  if (rc || G * N == 0) return rc;
  if (!u || !norms) return TQ_ERR_NULL;
  CodebookArgs cb = make_cb_args(cbs, n_cb, L);
  return launch_rotate_generic(cb, x, x_dtype, G, N, sx_g, sx_n, u, norms, static_cast<hipStream_t>(stream));
}

size_t tq_outlier_workspace_bytes(int head_dim, int64_t G, int64_t N) {
  if (head_dim < 2 || head_dim > kMaxHeadDim || G < 0 || N < 0) return 0;
  return (size_t)(G * outlier_chunks(N) * head_dim) * 16 + 256;
}

int tq_outlier_channels(int head_dim, int n_outlier, const void* x, int x_dtype, int64_t G, int64_t N,
                        int64_t sx_g, int64_t sx_n, int32_t* chan, void* work, size_t work_bytes,
                        void* stream) {
  if (head_dim == 0) return TQ_ERR_ZERO_DIMENSION;
  if (head_dim < 2 || head_dim > kMaxHeadDim) return TQ_ERR_BAD_DIMENSION;
  if (n_outlier <= 0 || n_outlier >= head_dim) return TQ_ERR_DIMENSION_MISMATCH;
  if (G < 0 || N < 0) return TQ_ERR_EMPTY_INPUT;
  if (G == 0) return TQ_OK;
  if (!chan || !work || (N > 0 && !x)) return TQ_ERR_NULL;
  if (!dtype_ok(x_dtype)) return TQ_ERR_UNSUPPORTED;
  if ((N > 1 && sx_n < head_dim) || (G > 1 && sx_g < head_dim) || sx_n < 0 || sx_g < 0)
    return TQ_ERR_DIMENSION_MISMATCH;
  if (work_bytes < tq_outlier_workspace_bytes(head_dim, G, N)) return TQ_ERR_DIMENSION_MISMATCH;
  return launch_outlier_channels(x, x_dtype, G, N, sx_g, sx_n, head_dim, n_outlier, chan,
                                 static_cast<double*>(work), static_cast<hipStream_t>(stream));
}

size_t tq_encode_split_workspace_bytes(int role, int head_dim, int n_outlier, int bits, int64_t G) {
  Layout Ln, Lo;
  if (split_layouts(role, head_dim, n_outlier, bits, &Ln, &Lo) || G < 0) return 0;
  if (!split256_supported(role, head_dim, n_outlier, bits, TQ_BF16, nullptr, 0, 0)) return 0;
  return split256_workspace_bytes(role, G);
}

int tq_encode_split(int role, int head_dim, int n_outlier, int bits, const void* cbs_normal,
                    const void* cbs_outlier, int64_t n_cb, const void* x, int x_dtype, int64_t G, int64_t N,
                    int64_t sx_g, int64_t sx_n, const int32_t* chan, void* rec_normal, void* rec_outlier,
                    void* work, size_t work_bytes, int32_t* status, void* stream) {
  Layout Ln, Lo;
  int rc = split_layouts(role, head_dim, n_outlier, bits, &Ln, &Lo);
  if (rc) return rc;
  if (n_cb <= 0 || G < 0 || N < 0) return TQ_ERR_EMPTY_INPUT;
  if (G == 0 || N == 0) return TQ_OK;
  if (!cbs_normal || !cbs_outlier || !x || !chan || !rec_normal || !rec_outlier) return TQ_ERR_NULL;
  if (!dtype_ok(x_dtype)) return TQ_ERR_UNSUPPORTED;
  if ((N > 1 && sx_n < head_dim) || (G > 1 && sx_g < head_dim) || sx_n < 0 || sx_g < 0)
    return TQ_ERR_DIMENSION_MISMATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (work && work_bytes >= split256_workspace_bytes(role, G) &&
      split256_supported(role, head_dim, n_outlier, bits, x_dtype, x, sx_g, sx_n))
    return launch_split256(role, bits, Ln, Lo, cbs_normal, cbs_outlier, n_cb, x, G, N, sx_g, sx_n, chan,
                           static_cast<uint32_t*>(rec_normal), static_cast<uint32_t*>(rec_outlier), work, status, s);
  rc = launch_encode_generic(make_cb_args(cbs_normal, n_cb, Ln), x, x_dtype, G, N, sx_g, sx_n,
                             static_cast<uint32_t*>(rec_normal), status, s,
                             ChannelMap{chan, head_dim, n_outlier, head_dim});
  if (rc) return rc;
  return launch_encode_generic(make_cb_args(cbs_outlier, n_cb, Lo), x, x_dtype, G, N, sx_g, sx_n,
                               static_cast<uint32_t*>(rec_outlier), status, s,
                               ChannelMap{chan, head_dim, 0, head_dim});
}

int tq_scores_split(int head_dim, int n_outlier, int bits, const void* cbs_normal, const void* cbs_outlier,
                    int64_t n_cb, const int32_t* chan, const void* krec_normal, const void* krec_outlier,
                    int64_t B, int64_t H_kv, int64_t T, const void* q, int q_dtype, int64_t H_q, float scale,
                    float* scores, int32_t* status, void* stream) {
  Layout Ln, Lo;
  int rc = split_layouts(TQ_ROLE_KEY, head_dim, n_outlier, bits, &Ln, &Lo);
  if (rc) return rc;
  if (n_cb <= 0 || B < 0 || H_kv <= 0 || T < 0 || H_q <= 0) return TQ_ERR_EMPTY_INPUT;
  if (H_q % H_kv) return TQ_ERR_DIMENSION_MISMATCH;
  if (B * T == 0) return TQ_OK;
  if (!cbs_normal || !cbs_outlier || !chan || !krec_normal || !krec_outlier || !q || !scores) return TQ_ERR_NULL;
  if (!dtype_ok(q_dtype)) return TQ_ERR_UNSUPPORTED;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf((float)head_dim);
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launch_scores_generic(make_cb_args(cbs_normal, n_cb, Ln), static_cast<const uint32_t*>(krec_normal), B,
                             H_kv, T, q, q_dtype, H_q, scale, scores, status, s, head_dim,
                             ChannelMap{chan, head_dim, n_outlier, head_dim}, false);
  if (rc) return rc;
  return launch_scores_generic(make_cb_args(cbs_outlier, n_cb, Lo), static_cast<const uint32_t*>(krec_outlier), B,
                               H_kv, T, q, q_dtype, H_q, scale, scores, status, s, head_dim,
                               ChannelMap{chan, head_dim, 0, head_dim}, true);
}

int tq_decode_values_split(int head_dim, int n_outlier, int bits, const void* cbs_normal, const void* cbs_outlier,
                           int64_t n_cb, const int32_t* chan, const void* rec_normal, const void* rec_outlier,
                           int64_t G, int64_t N, float* out, int32_t* status, void* stream) {
  Layout Ln, Lo;
  int rc = split_layouts(TQ_ROLE_VALUE, head_dim, n_outlier, bits, &Ln, &Lo);
  if (rc) return rc;
  if (n_cb <= 0 || G < 0 || N < 0) return TQ_ERR_EMPTY_INPUT;
  if (G * N == 0) return TQ_OK;
  if (!cbs_normal || !cbs_outlier || !chan || !rec_normal || !rec_outlier || !out) return TQ_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launch_decode_generic(make_cb_args(cbs_normal, n_cb, Ln), static_cast<const uint32_t*>(rec_normal), G, N,
                             out, status, s, head_dim, ChannelMap{chan, head_dim, n_outlier, head_dim});
  if (rc) return rc;
  return launch_decode_generic(make_cb_args(cbs_outlier, n_cb, Lo), static_cast<const uint32_t*>(rec_outlier), G,
                               N, out, status, s, head_dim, ChannelMap{chan, head_dim, 0, head_dim});
}

// ---- Gram-table scoring of block-codebook codes

static int gram_check(int head_dim, int block_dim, int codebook_size, int* W) {
  if (head_dim == 0) return TQ_ERR_ZERO_DIMENSION;
  if (head_dim < 2 || head_dim > kMaxHeadDim || (head_dim & (head_dim - 1))) return TQ_ERR_BAD_DIMENSION;
  if ((block_dim != 1 && block_dim != 2 && block_dim != 4 && block_dim != 8) || block_dim > head_dim)
    return TQ_ERR_BAD_DIMENSION;
  if (codebook_size < 2 || codebook_size > 256 || (codebook_size & (codebook_size - 1)))
    return TQ_ERR_INVALID_CODEBOOK;
  int w = 0;
  while ((1 << w) < codebook_size) ++w;
  *W = w;
  return TQ_OK;
}

static int gram_words(int head_dim, int block_dim, int W) { return ((head_dim / block_dim) * W + 31) / 32 + 1; }

size_t tq_gram_record_bytes(int head_dim, int block_dim, int codebook_size) {
  int W;
  if (gram_check(head_dim, block_dim, codebook_size, &W)) return 0;
  return (size_t)gram_words(head_dim, block_dim, W) * 4;
}

int tq_gram_table(int block_dim, int codebook_size, const float* codebook, float* table, void* stream) {
  int W;
  int rc = gram_check(kMaxHeadDim, block_dim, codebook_size, &W);
  if (rc) return rc;
  if (!codebook || !table) return TQ_ERR_NULL;
  return launch_gram_table(codebook, codebook_size, block_dim, table, static_cast<hipStream_t>(stream));
}

int tq_gram_encode(int head_dim, int block_dim, int codebook_size, const float* codebook, const uint32_t* signs,
                   const void* x, int x_dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, void* rec,
                   int32_t* status, void* stream) {
  int W;
  int rc = gram_check(head_dim, block_dim, codebook_size, &W);
  if (rc) return rc;
  if (G < 0 || N < 0) return TQ_ERR_EMPTY_INPUT;
  if (G * N == 0) return TQ_OK;
  if (!codebook || !signs || !x || !rec) return TQ_ERR_NULL;
  if (!dtype_ok(x_dtype)) return TQ_ERR_UNSUPPORTED;
  if ((N > 1 && sx_n < head_dim) || (G > 1 && sx_g < head_dim) || sx_n < 0 || sx_g < 0)
    return TQ_ERR_DIMENSION_MISMATCH;
  GramEncArgs a;
  a.C = codebook;
  a.N = codebook_size; a.k = block_dim; a.W = W; a.d = head_dim; a.nb = head_dim / block_dim;
  a.rw = gram_words(head_dim, block_dim, W);
  a.signs = signs;
  a.x = x; a.dtype = x_dtype;
  a.G = G; a.Nv = N; a.sx_g = sx_g; a.sx_n = sx_n;
  a.rec = static_cast<uint32_t*>(rec);
  a.status = status;
  return launch_gram_encode(a, static_cast<hipStream_t>(stream));
}

int tq_gram_scores(int head_dim, int block_dim, int codebook_size, const float* table, const void* qrec,
                   const void* krec, int64_t B, int64_t H_kv, int64_t T, int64_t H_q, float scale, float* scores,
                   void* stream) {
  int W;
  int rc = gram_check(head_dim, block_dim, codebook_size, &W);
  if (rc) return rc;
  if (B < 0 || H_kv <= 0 || T < 0 || H_q <= 0) return TQ_ERR_EMPTY_INPUT;
  if (H_q % H_kv) return TQ_ERR_DIMENSION_MISMATCH;
  if (B * T == 0) return TQ_OK;
  if (!table || !qrec || !krec || !scores) return TQ_ERR_NULL;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf((float)head_dim);
  GramScoreArgs a;
  a.G = table;
  a.qrec = static_cast<const uint32_t*>(qrec);
  a.krec = static_cast<const uint32_t*>(krec);
  a.B = B; a.Hkv = H_kv; a.T = T; a.Hq = H_q;
  a.scale = scale;
  a.scores = scores;
  a.chunks = 0;
  return launch_gram_scores(a, W, head_dim / block_dim, gram_words(head_dim, block_dim, W),
                            static_cast<hipStream_t>(stream));
}

}  // extern "C"
