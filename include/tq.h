/*
 * tq.h -- C ABI of libtq: TurboQuant KV-cache compression and compressed-key
 * attention scoring on AMD Instinct MI355X (gfx950).
 *
 * The method (page "turboquant-plus-rs 0.1.0 README", section "Architecture"):
 *   keys   : rotate each head vector by a random sign diagonal D followed by a
 *            Walsh-Hadamard transform H, store the norm, quantize every rotated
 *            coordinate with the (bits-1)-bit Lloyd-Max quantizer of N(0,1),
 *            then store the 1-bit signs of a Gaussian projection S of the
 *            residual together with the residual norm (QJL);
 *   values : the same rotation and a bits-bit Lloyd-Max quantizer only (MSE).
 * A quantizer is fully determined by (head_dim, bits, projections, seed)
 * (page "bitpolar 0.3.3 src/kv_cache.rs", KvCacheConfig).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Ownership: the caller owns all memory.  The library allocates nothing
 *    and keeps no state between calls; calls are thread-safe.
 *  - Device calls take device pointers and a `stream` (a hipStream_t; NULL is
 *    the null stream).  They enqueue work and return; argument validation is
 *    done on the host before anything is enqueued.  A non-zero return means
 *    nothing was enqueued.
 *  - Data errors found by kernels are OR-ed into an optional device int32
 *    status word (`status`, may be NULL): TQ_STATUS_NON_FINITE when an input
 *    vector holds NaN/Inf or its squared norm exceeds the float32 range (the
 *    pages' NonFiniteInput), TQ_STATUS_BAD_BLOB when a codebook header does
 *    not match the call's parameters.  The caller clears it and reads it after
 *    synchronising.
 *  - Layouts are dense and row-major unless a stride is given:
 *      inputs   x   [G][N][head_dim]   (element (g,t,j) at x + g*sx_g + t*sx_n + j)
 *      records      [G][N][record_bytes/4] uint32 words
 *      queries  q   [B][H_q][head_dim]
 *      scores       [B][H_q][T] float32
 *    Group g uses codebook (g mod n_cb); codebooks are stored back to back with
 *    stride tq_codebook_bytes().  For a cache [B][H_kv][T] with one codebook
 *    per kv head, n_cb = H_kv; for [L][H_kv][T] with one per (layer, head),
 *    n_cb = L*H_kv.
 *  - Query head hq attends kv head floor(hq * H_kv / H_q) (grouped queries).
 *
 * Record layout (canonical, what parity is checked on), little-endian uint32:
 *   k planes of W = ceil(head_dim/32) words: bit (j mod 32) of word p*W + j/32
 *     is bit p of the quantizer index of coordinate j   (k = bits-1 for keys,
 *     k = bits for values);
 *   keys: ceil(projections/32) sign words, bit i = [(S rho)_i >= 0], unused
 *     high bits zero;
 *   float32 norm |x|; keys: float32 residual norm |rho|.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 1

/* Return codes (host side).  Names follow the pages' error enum where one exists
 * (bitpolar: ZeroDimension, OddDimension, InvalidBitWidth, ZeroProjections,
 * DimensionMismatch, NonFiniteInput, EmptyInput). */
enum tq_status {
  TQ_OK = 0,
  TQ_ERR_ZERO_DIMENSION = -1,      /* head_dim == 0                                   */
  TQ_ERR_BAD_DIMENSION = -2,       /* head_dim not a power of two in [2, 512]         */
  TQ_ERR_INVALID_BIT_WIDTH = -3,   /* keys: bits not in [2, 9]; values: not in [1, 8] */
  TQ_ERR_ZERO_PROJECTIONS = -4,    /* keys with projections == 0                      */
  TQ_ERR_DIMENSION_MISMATCH = -5,  /* sizes/strides inconsistent (e.g. H_q % H_kv)   */
  TQ_ERR_NON_FINITE_INPUT = -6,    /* reserved: non-finite data is reported on device */
  TQ_ERR_EMPTY_INPUT = -7,         /* n_cb == 0 or a size < 0                         */
  TQ_ERR_NULL = -8,                /* a required pointer is NULL                      */
  TQ_ERR_BAD_BLOB = -9,            /* blob buffer too small                            */
  TQ_ERR_HIP = -10,                /* a HIP launch failed                              */
  TQ_ERR_INVALID_ROLE = -11,       /* role not TQ_ROLE_KEY / TQ_ROLE_VALUE             */
  TQ_ERR_INVALID_PROJECTIONS = -12,/* projections > 1024                               */
  TQ_ERR_UNSUPPORTED = -13,        /* dtype or alignment not supported                 */
  TQ_ERR_INVALID_ROTATION = -14,   /* rotation not TQ_ROT_HADAMARD / TQ_ROT_HAAR       */
  TQ_ERR_INVALID_CODEBOOK = -15,   /* Gram codec: codebook size not a power of two in [2, 256] */
  TQ_ERR_SCRATCH_LIMIT = -16,      /* tq_attend_static: the call needs more than the static scratch */
};

/* Device status bits (OR-ed into *status). */
#define TQ_STATUS_NON_FINITE 1
#define TQ_STATUS_BAD_BLOB 2
#define TQ_STATUS_BAD_CHANNEL 4   /* a channel map entry outside [0, head_dim) */
#define TQ_STATUS_BAD_PAGE 8      /* a position or page-table entry outside the pool */

enum tq_role {
  TQ_ROLE_KEY = 0,    /* TurboQuant: (bits-1)-bit Lloyd-Max + 1-bit QJL of the residual */
  TQ_ROLE_VALUE = 1,  /* MSE only: bits-bit Lloyd-Max                                  */
};

enum tq_dtype { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 };

/* Byte size of one codebook blob (multiple of 256; also the stride between
 * blobs): the quantizer state that (head_dim, bits, projections, seed) fixes
 * (page "bitpolar 0.3.3 src/kv_cache.rs", KvCacheConfig; page
 * "turboquant-plus-rs 0.1.0 README", "Modules" codebook, rotation and qjl).
 * 0 when the parameters are invalid.  Host only. */
size_t tq_codebook_bytes(int head_dim, int bits, int projections, int role);

/* Byte size of one record (multiple of 4): the bit-packed indices, signs and
 * norms of one head vector (README "Modules" utils, bit packing and the
 * memory-footprint calculation; "Compression formats" gives the bits per
 * value, e.g. 56 bytes = 3.5 bits/value for turbo3 keys at head_dim 128).
 * 0 when the parameters are invalid.  Host only. */
size_t tq_record_bytes(int head_dim, int bits, int projections, int role);

/* Build the quantizer state for (head_dim, bits, projections, seed, role) into
 * the caller's HOST buffer `blob` of `blob_bytes` >= tq_codebook_bytes():
 *   64-byte header (magic "TQCB", version, parameters, section offsets),
 *   float32 Lloyd-Max centroids c[2^k] and thresholds t[2^k - 1] of N(0,1)
 *     ("Modules" codebook: Lloyd's algorithm, closed form at 1 bit),
 *   sign-diagonal bits D (bit j set: D_j = -1),
 *   keys only: S, projections x head_dim binary16, row-major.
 * D and S come from SplitMix64 counters seeded by `seed` (Box-Muller for S).
 * For several heads use seed + h, as MultiHeadKvCache::new does.  The caller
 * uploads the blob.  Host only; deterministic. */
int tq_make_codebook(int head_dim, int bits, int projections, uint64_t seed, int role,
                     void* blob, size_t blob_bytes);

/* Rotation of a codebook (README "Architecture" step 1 and "Modules" rotation:
 * the random rotation is Haar-distributed via QR, or the fast Walsh-Hadamard
 * transform).  TQ_ROT_HADAMARD: Pi = H D / sqrt(head_dim), head_dim a power of
 * two; the blob section at off_d holds the bits of D.  TQ_ROT_HAAR: Pi = Q, the
 * orthogonal QR factor (Householder, float64) of the head_dim x head_dim Gaussian
 * matrix drawn from SplitMix64 counters 2^33 + e (Box-Muller, row-major entry e),
 * columns signed so the triangular factor has a positive diagonal; the blob
 * section at off_d holds float32 R = sqrt(head_dim) Q, row-major, which takes the
 * place of H D everywhere (u = R x, x^ = (n/head_dim) R^T c[idx], qt = R q).  Any
 * head_dim in [2, 512]. */
enum tq_rotation { TQ_ROT_HADAMARD = 0, TQ_ROT_HAAR = 1 };

/* As tq_codebook_bytes / tq_record_bytes / tq_make_codebook, with the rotation
 * named.  Host only. */
size_t tq_codebook_bytes_ex(int head_dim, int bits, int projections, int role, int rotation);
size_t tq_record_bytes_ex(int head_dim, int bits, int projections, int role, int rotation);
int tq_make_codebook_ex(int head_dim, int bits, int projections, uint64_t seed, int role, int rotation,
                        void* blob, size_t blob_bytes);

/* Encode keys: x [G][N][head_dim] (dtype TQ_F32/TQ_BF16/TQ_F16, strides in
 * elements; head_dim contiguous) -> records [G][N][tq_record_bytes/4] at `rec`.
 * (page "bitpolar 0.3.3 src/kv_cache.rs", KvCacheCompressor::push; README
 * "Architecture" steps 1-2.)  cbs: n_cb key blobs back to back. */
int tq_encode_keys(int head_dim, int bits, int projections,
                   const void* cbs, int64_t n_cb,
                   const void* x, int x_dtype, int64_t G, int64_t N,
                   int64_t sx_g, int64_t sx_n,
                   void* rec, int32_t* status, void* stream);

/* Encode values (MSE-only path, README "Architecture", last paragraph). */
int tq_encode_values(int head_dim, int bits,
                     const void* cbs, int64_t n_cb,
                     const void* x, int x_dtype, int64_t G, int64_t N,
                     int64_t sx_g, int64_t sx_n,
                     void* rec, int32_t* status, void* stream);

/* Keys and values of the same tokens in one call: tq_encode_keys on k into
 * krec and tq_encode_values on v into vrec (README "Architecture": keys take
 * the MSE stage and the QJL residual, values the MSE stage only), with the
 * same group count, token count, strides and input dtype for k and v; each
 * side has its own codebooks.  Records are bit for bit those of the two
 * calls.  With turbo3 keys, 2- or 3-bit values, head_dim 128 and f32 or bf16
 * inputs the two encodes share one launch (workgroups take key or value
 * ranges); other shapes run the two encodes one after the other.  Errors as
 * for the two calls, checked for both before anything is enqueued. */
int tq_encode_kv(int head_dim, int k_bits, int v_bits, int projections,
                 const void* kcbs, int64_t n_kcb, const void* vcbs, int64_t n_vcb,
                 const void* k, const void* v, int x_dtype, int64_t G, int64_t N,
                 int64_t sx_g, int64_t sx_n,
                 void* krec, void* vrec, int32_t* status, void* stream);

/* Decode value records [G][N] -> out [G][N][head_dim] float32:
 * x^ = (n/head_dim) * D (H c[idx])  (bitpolar decode_values). */
int tq_decode_values(int head_dim, int bits,
                     const void* cbs, int64_t n_cb,
                     const void* rec, int64_t G, int64_t N,
                     float* out, int32_t* status, void* stream);

/* Pre-softmax attention scores from compressed keys, without decoding
 * (bitpolar KvCacheCompressor::attention_scores: estimate(q, k) * scale):
 *   scores[b][hq][t] = scale * ( (n_t/d) sum_j qt_j c[idx_tj]
 *                     + sqrt(pi/2)/m * gamma_t * sum_i p_i (2 s_ti - 1) ),
 * qt = H(D q), p = S qt / sqrt(d), for the kv head of hq.  krec [B][H_kv][T]
 * records; q [B][H_q][head_dim] (TQ_F32/TQ_BF16/TQ_F16); scale <= 0 means
 * 1/sqrt(head_dim).  Group (b, h) uses codebook (b*H_kv + h) mod n_cb. */
int tq_scores(int head_dim, int bits, int projections,
              const void* cbs, int64_t n_cb,
              const void* krec, int64_t B, int64_t H_kv, int64_t T,
              const void* q, int q_dtype, int64_t H_q, float scale,
              float* scores, int32_t* status, void* stream);

/* Attention output over compressed K and V for one decode step:
 * o[b][hq] = sum_t softmax_t(scores[b][hq][t]) * x^_t, the values decoded on
 * the fly (never materialised) and summed in the rotated domain, one inverse
 * transform per (b, hq); the softmax is split over chunks of 1024 tokens (512
 * on the fused path below) and merged by log-sum-exp.  `work` is caller scratch of
 * tq_attend_workspace_bytes(...) bytes: the scores (or, where the scores are
 * computed inside the chunk pass, the prepared query side of each (b, kv head)),
 * then the per-chunk partials.  At head_dim 128 with 128 projections, key and
 * value bits giving at most 3 planes each, and 1, 2 or 4 query heads per kv
 * head, no score is written: one pass per chunk scores the keys on chip.  Key
 * and value codebooks are separate arrays (kcbs, vcbs) with their own n_cb.
 * T == 0 gives o = 0. */
size_t tq_attend_workspace_bytes(int head_dim, int64_t B, int64_t H_q, int64_t T);
int tq_attend(int head_dim, int k_bits, int v_bits, int projections,
              const void* kcbs, int64_t n_kcb, const void* vcbs, int64_t n_vcb,
              const void* krec, const void* vrec, int64_t B, int64_t H_kv, int64_t T,
              const void* q, int q_dtype, int64_t H_q, float scale,
              float* out, void* work, size_t work_bytes, int32_t* status, void* stream);

/* Allocation-free form of tq_attend_ex, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results and errors as tq_attend_ex
 * (rotation as there; TQ_ROT_HADAMARD gives tq_attend), without `work`: the
 * scratch is a library-owned device array of TQ_ATTEND_STATIC_SCRATCH_BYTES
 * (32 MiB) per GPU, held until the process ends.  A call whose
 * tq_attend_workspace_bytes(head_dim, B, H_q, T) exceeds it returns
 * TQ_ERR_SCRATCH_LIMIT with nothing enqueued (e.g. the long-context step of 4
 * sequences x 8 query heads x 131072 tokens needs 18.9 MB).  The call itself allocates nothing (no hipMalloc,
 * no hipFree).  Every call on one GPU shares that GPU's array and leaves its
 * contents behind; nothing in it needs to start at zero.  Calls that overlap on
 * one GPU (two streams, or two host threads) race on the array and give
 * undefined results: serialise them.  The first call on a device looks up the
 * array's device address (hipGetSymbolAddress), so make one such call outside
 * any graph capture first.  tq_attend_static_scratch_bytes() returns the
 * array's size. */
#define TQ_ATTEND_STATIC_SCRATCH_BYTES (32u << 20)
size_t tq_attend_static_scratch_bytes(void);
int tq_attend_static(int head_dim, int k_bits, int v_bits, int projections, int rotation,
                     const void* kcbs, int64_t n_kcb, const void* vcbs, int64_t n_vcb,
                     const void* krec, const void* vrec, int64_t B, int64_t H_kv, int64_t T,
                     const void* q, int q_dtype, int64_t H_q, float scale,
                     float* out, int32_t* status, void* stream);

/* Rotation-named forms of the five compute calls above (README "Architecture"
 * step 1 and "Modules" rotation: the random rotation is Haar via QR, or the fast
 * Walsh-Hadamard transform).  Arguments, layouts and errors as in the plain
 * forms, which are these with rotation = TQ_ROT_HADAMARD; `rotation` names the
 * rotation the codebooks were made with (tq_make_codebook_ex) and must match
 * the blob headers (else the status word gets the blob-mismatch bit).  With
 * TQ_ROT_HAAR, head_dim is any value in [2, 512]; R = sqrt(head_dim) Q takes the
 * place of H D everywhere (u = R x, x^ = (n/head_dim) R^T c[idx], qt = R q), and
 * attention applies R^T once per (b, hq) to the rotated-domain sum.  Encodes
 * of bf16/f16 inputs run R x on the matrix cores (R in three exact 16-bit
 * terms) at head_dim 128 and, padded to 128, at head_dims below 128 that are
 * multiples of 8 (keys of up to 4 bits with up to 128 projections, values of
 * up to 4 bits, 16-byte aligned rows); bf16 encodes at head_dims in (128, 256]
 * that are multiples of 8 stream R through the matrix cores in 16-column
 * chunks (keys of up to 4 bits with up to 256 projections, values of up to 4
 * bits).  At head_dim 128 the scores and the fused attention (128
 * projections) rotate the query by R; scores at other head dims of keys with
 * up to 4 bits run a table-driven kernel (byte tables of the rotated query and
 * its projection in LDS, R q and S q on the matrix cores); value decodes at
 * head dims up to 256 run x^ = U R on the matrix cores (both in two-term
 * binary16); other Haar encodes, scores and decodes run on the float64
 * per-vector kernels.  The attention's value partials run on the same MFMA
 * kernels as for Walsh-Hadamard codebooks when head_dim is a multiple of 32. */
int tq_encode_keys_ex(int head_dim, int bits, int projections, int rotation,
                      const void* cbs, int64_t n_cb,
                      const void* x, int x_dtype, int64_t G, int64_t N,
                      int64_t sx_g, int64_t sx_n,
                      void* rec, int32_t* status, void* stream);
int tq_encode_values_ex(int head_dim, int bits, int rotation,
                        const void* cbs, int64_t n_cb,
                        const void* x, int x_dtype, int64_t G, int64_t N,
                        int64_t sx_g, int64_t sx_n,
                        void* rec, int32_t* status, void* stream);
int tq_decode_values_ex(int head_dim, int bits, int rotation,
                        const void* cbs, int64_t n_cb,
                        const void* rec, int64_t G, int64_t N,
                        float* out, int32_t* status, void* stream);
int tq_scores_ex(int head_dim, int bits, int projections, int rotation,
                 const void* cbs, int64_t n_cb,
                 const void* krec, int64_t B, int64_t H_kv, int64_t T,
                 const void* q, int q_dtype, int64_t H_q, float scale,
                 float* scores, int32_t* status, void* stream);
int tq_attend_ex(int head_dim, int k_bits, int v_bits, int projections, int rotation,
                 const void* kcbs, int64_t n_kcb, const void* vcbs, int64_t n_vcb,
                 const void* krec, const void* vrec, int64_t B, int64_t H_kv, int64_t T,
                 const void* q, int q_dtype, int64_t H_q, float scale,
                 float* out, void* work, size_t work_bytes, int32_t* status, void* stream);

/* ---- Streaming append into a paged compressed cache ----------------------
 * page "fib-quant 0.1.0-beta.4 README", "Streaming KV encoder": the encoded KV
 * tensor is built one token at a time, pages are complete when they reach
 * tokens_per_page, and the result equals the batch encode of the same input;
 * page "bitpolar 0.3.3 src/kv_cache.rs", MultiHeadKvCache::push_token: one
 * token's key and value for every head at once.
 *
 * Pools hold pages of tokens_per_page tokens of one sequence, all H_kv heads:
 *   kpool [num_pages][H_kv][tokens_per_page][key record words]   (uint32)
 *   vpool [num_pages][H_kv][tokens_per_page][value record words]
 * so that one (sequence, kv head) has its records of a page contiguous.
 * page_table [B][max_pages] (int32, device): the pool page of each page index
 * of sequence b; the caller maps a fresh page whenever a sequence's length
 * reaches a multiple of tokens_per_page.  pos [B] (int32, device): the position
 * the new token takes in sequence b.
 *
 * tq_append_kv encodes k_new and v_new [B][H_kv][head_dim] (contiguous; dtype
 * as for tq_encode_keys) and writes record (b, h) to page
 * page_table[b][pos[b] / tokens_per_page], slot pos[b] % tokens_per_page.  The
 * records are bit-identical to tq_encode_keys / tq_encode_values on the same
 * vectors (same kernels); codebook of (b, h) as there: (b*H_kv + h) mod n_cb.
 * A negative position, one at or past max_pages * tokens_per_page, or a page
 * outside [0, num_pages) writes nothing for that sequence and sets
 * TQ_STATUS_BAD_PAGE.  `work`: caller scratch of tq_append_workspace_bytes(...)
 * bytes (staging for shapes the head_dim-128 kernels do not take; at head_dim
 * 128 the records go straight to their page slots).  Walsh-Hadamard codebooks. */
size_t tq_append_workspace_bytes(int head_dim, int k_bits, int v_bits, int projections, int64_t B, int64_t H_kv);
int tq_append_kv(int head_dim, int k_bits, int v_bits, int projections,
                 const void* kcbs, int64_t n_kcb, const void* vcbs, int64_t n_vcb,
                 const void* k_new, const void* v_new, int x_dtype, int64_t B, int64_t H_kv,
                 const int32_t* pos, const int32_t* page_table, int64_t max_pages,
                 int tokens_per_page, int64_t num_pages,
                 void* kpool, void* vpool, void* work, size_t work_bytes,
                 int32_t* status, void* stream);

/* Scores (as tq_scores) from a paged key pool filled by tq_append_kv: token t
 * of sequence b, kv head h, is record (page_table[b][t / tokens_per_page], h,
 * t % tokens_per_page) of kpool; every sequence has T tokens.  Scores equal
 * tq_scores on the same records gathered in token order.  Needs head_dim 128,
 * 128 projections, bits 2..4, 1, 2 or 4 query heads per kv head, and
 * tokens_per_page a multiple of 32 (else TQ_ERR_UNSUPPORTED /
 * TQ_ERR_DIMENSION_MISMATCH).  A page outside [0, num_pages) reads as zero
 * records and sets TQ_STATUS_BAD_PAGE. */
int tq_scores_paged(int head_dim, int bits, int projections,
                    const void* cbs, int64_t n_cb,
                    const void* kpool, const int32_t* page_table, int64_t max_pages,
                    int tokens_per_page, int64_t num_pages,
                    int64_t B, int64_t H_kv, int64_t T,
                    const void* q, int q_dtype, int64_t H_q, float scale,
                    float* scores, int32_t* status, void* stream);

/* Test hook: the first half of README "Architecture" step 1 (random rotation,
 * with "Modules" polar_quant's norm extraction): u = H(D x) (unnormalised
 * rotation) and n = |x| for every vector, with the D of the group's codebook.
 * u [G][N][head_dim] f32, norms [G][N] f32 (caller-owned); argument errors as
 * for tq_encode_keys. */
int tq_rotate(int head_dim, int bits, int projections, int role,
              const void* cbs, int64_t n_cb,
              const void* x, int x_dtype, int64_t G, int64_t N,
              int64_t sx_g, int64_t sx_n,
              float* u, float* norms, void* stream);

/* ---- Outlier/normal channel split (mixed-precision layers) ----------------
 * README "Modules" outlier (non-integer bit rates by splitting the channels of a
 * head vector into outlier and normal parts); "Key ideas" 3 (boundary layers at
 * higher precision are plain calls at a higher `bits`).
 * A channel map chan [G][head_dim] int32 lists, for group g, the n_outlier
 * outlier channels ascending, then the other head_dim - n_outlier channels
 * ascending.  Coordinate j of a part is channel chan[g][offset + j] of x.
 *   normal part : head_dim - n_outlier coordinates, TQ_ROT_HAAR codebooks at
 *                 `bits` (keys: projections = head_dim - n_outlier);
 *   outlier part: n_outlier coordinates (a power of two), TQ_ROT_HADAMARD
 *                 codebooks at bits + 1 (keys: projections = n_outlier).
 * Each part has its own records ([G][N][tq_record_bytes_ex(part)/4]) and its own
 * codebook array (n_cb blobs each, group g uses blob g mod n_cb).  Keys: bits in
 * [2, 8]; values: bits in [1, 7].  A map entry outside [0, head_dim) sets
 * TQ_STATUS_BAD_CHANNEL and reads channel 0. */

/* Codebooks of the two parts of one (layer, kv-head) group whose head seed is
 * `seed` (the seed tq_make_codebook would take for the unsplit head):
 *   part 0, normal : head_dim - n_outlier coordinates, TQ_ROT_HAAR, `bits`,
 *                    seeded `seed`;
 *   part 1, outlier: n_outlier coordinates, TQ_ROT_HADAMARD, bits + 1, seeded
 *                    seed XOR 0x9E3779B97F4A7C15 (the 64-bit golden-ratio
 *                    constant), so that the parts draw independent D and S;
 *   keys project each part onto as many signs as it has coordinates.
 * The pages give one seed per head and no rule for sub-quantizers; this is the
 * rule every split call assumes.  tq_split_codebook_bytes gives the byte size
 * (and blob stride) of part 0 or 1, 0 on invalid parameters; blobs are written
 * to the caller's HOST buffers as by tq_make_codebook_ex.  Host only. */
size_t tq_split_codebook_bytes(int role, int head_dim, int n_outlier, int bits, int part);
int tq_make_split_codebooks(int role, int head_dim, int n_outlier, int bits, uint64_t seed,
                            void* normal_blob, size_t normal_bytes, void* outlier_blob, size_t outlier_bytes);

/* Scratch for tq_outlier_channels: G * chunks * head_dim * 16 bytes, chunks =
 * clamp(ceil(N/512), 1, 64).  0 on invalid sizes. */
size_t tq_outlier_workspace_bytes(int head_dim, int64_t G, int64_t N);

/* chan[g] for every group of x [G][N][head_dim] (strides in elements): the
 * n_outlier channels with the largest population variance over the N vectors
 * (float64 sums; ties to the lower channel index), ascending, then the rest
 * ascending.  N == 0 gives channels 0 .. n_outlier-1 as outliers.  `work` is
 * caller scratch of tq_outlier_workspace_bytes.  head_dim in [2, 512],
 * 0 < n_outlier < head_dim. */
int tq_outlier_channels(int head_dim, int n_outlier, const void* x, int x_dtype, int64_t G, int64_t N,
                        int64_t sx_g, int64_t sx_n, int32_t* chan, void* work, size_t work_bytes,
                        void* stream);

/* Scratch for the MFMA path of tq_encode_split (per-group rotation and
 * projection fragments built from the channel map): G * 356 KiB for keys,
 * G * 256 KiB for values.  Non-zero only for the shapes that path serves
 * (head_dim 256, 32 outliers, bits 2 or 3); 0 otherwise. */
size_t tq_encode_split_workspace_bytes(int role, int head_dim, int n_outlier, int bits, int64_t G);

/* Encode both parts of every vector (role TQ_ROLE_KEY or TQ_ROLE_VALUE).
 * `work` (caller scratch of tq_encode_split_workspace_bytes, may be NULL)
 * enables the MFMA path for bf16 input with 16-byte aligned rows; without it,
 * or for other shapes, the generic kernels run.  Both give the same records up
 * to the parity tolerances. */
int tq_encode_split(int role, int head_dim, int n_outlier, int bits,
                    const void* cbs_normal, const void* cbs_outlier, int64_t n_cb,
                    const void* x, int x_dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n,
                    const int32_t* chan, void* rec_normal, void* rec_outlier, void* work, size_t work_bytes,
                    int32_t* status, void* stream);

/* Scores from split key records: scores[b][hq][t] = scale * (estimate of the
 * normal part + estimate of the outlier part), each part scored from its records
 * against the query channels the map selects; scale <= 0 means 1/sqrt(head_dim).
 * chan has one row per (b, kv head) group, b*H_kv + h.  Parts of keys with up to
 * 4 bits run the table-driven score kernel (the outlier part adding into the
 * normal part's scores), larger codebooks the per-token kernel. */
int tq_scores_split(int head_dim, int n_outlier, int bits,
                    const void* cbs_normal, const void* cbs_outlier, int64_t n_cb, const int32_t* chan,
                    const void* krec_normal, const void* krec_outlier, int64_t B, int64_t H_kv, int64_t T,
                    const void* q, int q_dtype, int64_t H_q, float scale, float* scores, int32_t* status,
                    void* stream);

/* Decode split value records to out [G][N][head_dim] float32 (both parts
 * decoded and scattered back to their channels; parts of up to 256 channels run
 * x^ = U M on the matrix cores, M = R or the +-1 (D H)^T, written through the
 * channel map). */
int tq_decode_values_split(int head_dim, int n_outlier, int bits,
                           const void* cbs_normal, const void* cbs_outlier, int64_t n_cb, const int32_t* chan,
                           const void* rec_normal, const void* rec_outlier, int64_t G, int64_t N,
                           float* out, int32_t* status, void* stream);

/* Memory footprint of a K+V cache of seq_len x layers x kv_heads vectors
 * (README "Modules" utils; "Compression formats").  out[0] = fp16 bytes,
 * out[1] = f32 bytes, out[2] = compressed bytes, out[3] = ratio vs fp16
 * (1.0 when empty).  Host only. */
int tq_memory_stats(int head_dim, int k_bits, int v_bits, int projections,
                    int64_t seq_len, int64_t layers, int64_t kv_heads, double out[4]);

/* ---- Gram-table scoring of block-codebook codes --------------------------
 * Page "fib-quant 0.1.0-beta.4 README": a vector is cut into blocks, each
 * block is stored as the index of a codeword of a small codebook ("What's in
 * the box", Codec; rotated first by the fast Walsh-Hadamard transform,
 * Rotation), and inner products with stored codes are estimated from the Gram
 * table G[i][j] = <c_i, c_j> without decoding them ("New modules", Scoring).
 *   head_dim d  : a power of two in [2, 512] (else TQ_ERR_BAD_DIMENSION);
 *   block_dim k : 1, 2, 4 or 8, at most d (else TQ_ERR_BAD_DIMENSION);
 *   codebook_size N : a power of two in [2, 256], w = log2 N bits per index
 *                 (else TQ_ERR_INVALID_CODEBOOK);
 *   codebook    : float32 [N][k], device, caller-made (any contents);
 *   signs       : ceil(d/32) uint32 words, device; bit j set negates
 *                 coordinate j before the transform (the diagonal D).
 * Record: the d/k indices, index b at bits [b w, (b+1) w) of the little-endian
 * words (LSB first; an index may straddle two words), ceil(d w / (k 32))
 * words, then float32 |x|.  Encode: n = |x| (float64, stored as float32),
 * u = H(D x) / (sqrt(d) n) (u = 0 for a zero vector), block b = u[b k, b k + k)
 * takes the nearest codeword (Euclidean; the lowest index on ties).  The
 * kernel decides on u rounded to float32 from a float64 transform, with
 * float64 squared distances to the float32 codewords, so it can differ from
 * the nearest codeword of the exact u only for a block lying within that
 * rounding of the boundary between two codewords.  Scores (the query encoded
 * alike):
 *   s[b][hq][t] = scale * n_q * n_t * sum_blocks G[cq_blk][ct_blk]
 * with query head hq reading kv head floor(hq * H_kv / H_q); scale <= 0 means
 * 1/sqrt(d).  No data errors exist for scores (indices are masked to w bits). */
size_t tq_gram_record_bytes(int head_dim, int block_dim, int codebook_size);

/* G[i][j] = <c_i, c_j>, float32 [N][N] (device), summed in float32 by fma. */
int tq_gram_table(int block_dim, int codebook_size, const float* codebook, float* table, void* stream);

/* Records [G][N][tq_gram_record_bytes/4] of x [G][N][head_dim] (strides as for
 * tq_encode_keys; TQ_F32/TQ_BF16/TQ_F16).  Non-finite input, or a squared
 * norm past the float32 range, sets TQ_STATUS_NON_FINITE (record unspecified). */
int tq_gram_encode(int head_dim, int block_dim, int codebook_size, const float* codebook, const uint32_t* signs,
                   const void* x, int x_dtype, int64_t G, int64_t N, int64_t sx_g, int64_t sx_n,
                   void* rec, int32_t* status, void* stream);

/* scores [B][H_q][T] float32 from query records qrec [B][H_q][words] and key
 * records krec [B][H_kv][T][words], with the table of tq_gram_table. */
int tq_gram_scores(int head_dim, int block_dim, int codebook_size, const float* table,
                   const void* qrec, const void* krec, int64_t B, int64_t H_kv, int64_t T, int64_t H_q,
                   float scale, float* scores, void* stream);

/* Human-readable name of a return code; the names follow the error enum of
 * page "bitpolar 0.3.3 src/kv_cache.rs" where one exists.  A static string,
 * never NULL ("unknown status" for codes outside enum tq_status). */
const char* tq_status_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
