// Kernel launchers of libtq (host functions defined next to their kernels).
// Each returns 0 or TQ_ERR_HIP after enqueueing on stream `s`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"
#include "tq_layout.h"

namespace tq {

int launch_encode_generic(const CodebookArgs& cb, const void* x, int dtype, int64_t G, int64_t N,
                          int64_t sx_g, int64_t sx_n, uint32_t* rec, int32_t* status, hipStream_t s,
                          const ChannelMap& cm = ChannelMap{});
// Hadamard encode, 32 vectors per workgroup step (power-of-two d in [32, 512]):
// the projection matrix is staged through LDS once per step.
bool tiled_encode_supported(const CodebookArgs& cb);
int launch_encode_tiled(const CodebookArgs& cb, const void* x, int dtype, int64_t G, int64_t N, int64_t sx_g,
                        int64_t sx_n, uint32_t* rec, int32_t* status, hipStream_t s);
// Hadamard encode at head_dim 256 with up to 256 levels (keys: up to 256
// projections); 16-byte aligned rows of at least head_dim elements.
bool wide_encode_supported(const CodebookArgs& cb, int dtype, const void* x, int64_t sx_g, int64_t sx_n, int64_t N);
int launch_encode_wide(const CodebookArgs& cb, const void* x, int dtype, int64_t G, int64_t N, int64_t sx_g,
                       int64_t sx_n, uint32_t* rec, int32_t* status, hipStream_t s);
// Value decode of the Walsh-Hadamard codec at d in {32, 64, 128, 256}, k <= 8,
// into a 16-byte aligned [G][N][d] output; needs N >= 2048 / d.
bool decode_wh_supported(const CodebookArgs& cb, int64_t G, int64_t N, const void* out);
int launch_decode_wh(const CodebookArgs& cb, const uint32_t* rec, int64_t G, int64_t N, float* out,
                     int32_t* status, hipStream_t s);
// Haar encode on MFMA for head_dim in (128, 256], a multiple of 8, bf16 input
// (keys up to 4 bits with up to 256 projections, values up to 4 bits).
bool haar256_supported(const CodebookArgs& cb, int dtype, const void* x, int64_t sx_g, int64_t sx_n, int64_t N);
int launch_haar256(const CodebookArgs& cb, const void* x, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n,
                   uint32_t* rec, int32_t* status, hipStream_t s);
int launch_decode_generic(const CodebookArgs& cb, const uint32_t* rec, int64_t G, int64_t N, float* out,
                          int32_t* status, hipStream_t s, int64_t out_stride = 0,
                          const ChannelMap& cm = ChannelMap{});
// Value decode on the matrix cores (tq_decode_haar.hip): Haar codebooks, and
// Walsh-Hadamard ones under a channel map; d <= 256, any value bits.
// launch_decode_generic takes this route whenever it is supported.
bool haar_decode_mfma_supported(const CodebookArgs& cb, bool mapped);
int launch_decode_haar_mfma(const CodebookArgs& cb, const uint32_t* rec, int64_t G, int64_t N, float* out,
                            int32_t* status, hipStream_t s, int64_t out_stride, const ChannelMap& cm);
int launch_rotate_generic(const CodebookArgs& cb, const void* x, int dtype, int64_t G, int64_t N,
                          int64_t sx_g, int64_t sx_n, float* u, float* norms, hipStream_t s);
int launch_scores_generic(const CodebookArgs& cb, const uint32_t* krec, int64_t B, int64_t Hkv, int64_t T,
                          const void* q, int q_dtype, int64_t Hq, float scale, float* scores,
                          int32_t* status, hipStream_t s, int64_t q_row = 0,
                          const ChannelMap& cm = ChannelMap{}, bool accumulate = false);
// Scores through byte tables in LDS (tq_score_lut.hip): keys with k <= 3 index
// planes, any head_dim (Walsh-Hadamard: a power of two); launch_scores_generic
// takes this route whenever it is supported.
bool lut_scores_supported(const CodebookArgs& cb, int64_t T);
int launch_scores_lut(const CodebookArgs& cb, const uint32_t* krec, int64_t B, int64_t Hkv, int64_t T,
                      const void* q, int q_dtype, int64_t Hq, float scale, float* scores, int32_t* status,
                      hipStream_t s, int64_t q_row, const ChannelMap& cm, bool accumulate);
// Split-token attention output (any power-of-two d in [8, 512], value k <= 8):
// per-chunk partials in `part` ([B*Hq][attend_chunks(T)][d + 2] floats), then a merge.
int64_t attend_chunks(int64_t T);
// Chunks of the fused pass (512 tokens): it writes partials [B*Hq][attend_fused_chunks(T)][d + 2].
int64_t attend_fused_chunks(int64_t T);
// Fused attention (d = m = 128, k <= 3 for keys and values): the query side of
// each (b, kv head) into `qws` (attend_qprep_bytes(B * Hkv) bytes), then scores
// straight from the key records into the chunk partials, then the merge; `part`
// as above.
size_t attend_qprep_bytes(int64_t groups);
// Paged pools: record (b, h) of `staged` ([Hkv][B] records when head_major, else
// [B][Hkv]) to page page_table[b][pos[b] / tpp], slot pos[b] % tpp of
// pool [num_pages][Hkv][tpp][rw]; bad positions or pages set TQ_STATUS_BAD_PAGE.
int launch_page_scatter(const uint32_t* staged, bool head_major, int64_t B, int64_t Hkv, int rw,
                        const int32_t* pos, const int32_t* page_table, int64_t max_pages, int tpp,
                        int64_t num_pages, uint32_t* pool, int32_t* status, hipStream_t s);
bool attend_fused_supported(const CodebookArgs& kcb, const CodebookArgs& vcb, int64_t Hkv, int64_t Hq, int64_t T,
                            const void* krec);
int launch_attend_fused(const CodebookArgs& kcb, const CodebookArgs& vcb, const uint32_t* krec,
                        const uint32_t* vrec, int64_t B, int64_t Hkv, int64_t T, const void* q, int q_dtype,
                        int64_t Hq, float scale, uint8_t* qws, float* part, float* out, int32_t* status,
                        hipStream_t s);
bool attend_split_supported(const CodebookArgs& vcb);
int launch_attend_split(const CodebookArgs& vcb, const uint32_t* vrec, const float* scores, int64_t B,
                        int64_t Hkv, int64_t T, int64_t Hq, float* part, float* out, hipStream_t s);
// Split encode on MFMA (head_dim 256, 32 outlier channels, bf16 input): a prep
// kernel writes the per-group fragments into `work`, then the encode kernel.
bool split256_supported(int role, int head_dim, int n_outlier, int bits, int dtype, const void* x, int64_t sx_g,
                        int64_t sx_n);
size_t split256_workspace_bytes(int role, int64_t G);
int launch_split256(int role, int bits, const Layout& Ln, const Layout& Lo, const void* cbn, const void* cbo,
                    int64_t n_cb, const void* x, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n,
                    const int32_t* chan, uint32_t* rec_n, uint32_t* rec_o, void* work, int32_t* status,
                    hipStream_t s);
// Outlier channel selection: float64 channel sums over token chunks, then a
// per-group ranking into the channel map.
int64_t outlier_chunks(int64_t N);
int launch_outlier_channels(const void* x, int dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n, int d,
                            int n_out, int32_t* chan, double* work, hipStream_t s);
int launch_attend_generic(const CodebookArgs& vcb, const uint32_t* vrec, const float* scores, int64_t B,
                          int64_t Hkv, int64_t T, int64_t Hq, float* out, hipStream_t s);

// Gram-table scoring of block-codebook codes (tq_gram.hip).  Shapes are
// validated by the caller: d a power of two in [2, 512], k in {1, 2, 4, 8},
// N = 2^W in [2, 256]; records of rw = ceil(d W / (k 32)) + 1 words.
struct GramEncArgs {
  const float* C;            // [N][k] codebook
  int N, k, W, d, nb, rw;    // nb = d / k
  const uint32_t* signs;     // ceil(d/32) words, bit j set: coordinate j negated
  const void* x;
  int dtype;
  int64_t G, Nv, sx_g, sx_n;
  uint32_t* rec;             // [G][Nv][rw]
  int32_t* status;
};
struct GramScoreArgs {
  const float* G;            // [N][N] Gram table
  const uint32_t* qrec;      // [B][Hq][rw]
  const uint32_t* krec;      // [B][Hkv][T][rw]
  int64_t B, Hkv, T, Hq;
  float scale;
  float* scores;             // [B][Hq][T]
  int64_t chunks;            // set by the launcher
};
int launch_gram_table(const float* C, int N, int k, float* G, hipStream_t s);
int launch_gram_encode(const GramEncArgs& a, hipStream_t s);
int launch_gram_scores(GramScoreArgs a, int W, int nb, int rw, hipStream_t s);

}  // namespace tq
