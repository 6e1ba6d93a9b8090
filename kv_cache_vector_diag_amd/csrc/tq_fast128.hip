// head_dim-128 encode kernels for gfx950 (CDNA4, wave64).
//
// Method (page "turboquant-plus-rs 0.1.0 README", "Architecture"): rotate
// each head vector by D then the Walsh-Hadamard matrix H, quantize every
// rotated coordinate with the Lloyd-Max quantizer of N(0,1) (keys: bits-1,
// values: bits), keys additionally keep the signs of a Gaussian projection S
// of the residual and the residual norm (QJL).  Same device semantics as
// encode_generic_kernel, restated for throughput:
//
//  * One wave encodes a tile of 32 vectors.  Lane l owns vector l%32 and, in
//    every 32x32 MFMA result, the 16 rows 8i + 4(l/32) + j of each 32-row
//    tile.
//  * The rotation u = H (D x) is a dense +-1 contraction: MFMA
//    v_mfma_f32_32x32x16_bf16 with A = (H D) fragments (exact +-1 in bf16)
//    and B = the bf16 input itself, so products are exact and only the fp32
//    accumulation rounds.  (Float32 inputs are split exactly into three bf16
//    pieces; float16 inputs use the f16 MFMA.)
//  * |x|^2 is accumulated in float64 from exact pair sums so that the stored
//    float32 norm is the correctly rounded one (the residual depends on it).
//  * Quantizer: symmetric codebook, so idx is the sign of u plus the count of
//    positive thresholds below |u|/|x|; bits are packed in registers.
//  * Keys: residual w = u - n c[idx] (one fma, then the half's sign), scaled by a
//    power of two and split into binary16 hi + lo; the QJL projection S w is
//    two f16 MFMA passes.  The rotation's result layout is used directly as
//    the projection's B operand: the contraction index is permuted and S's
//    columns are permuted to match when its fragments are built in LDS.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_fast.h"
#include "tq_mfma.h"

namespace tq {
namespace {

using namespace mf;

constexpr int kD = 128;
constexpr int kM = 128;
// Waves per workgroup (one workgroup per CU): 12 (three per SIMD) where the
// kernel fits in 168 VGPRs, else 8 (two per SIMD, up to 256 VGPRs).  Keys take
// 8: the four projection accumulators stay live across the slices; so do the
// padded Haar kernels (their masks and record staging).
template <int K, bool KEY, int DT, bool HAAR, bool PAD = false>
constexpr int waves_for() {
  return (KEY || DT == 0 || (HAAR && DT == 2) || PAD) ? 8 : 12;
}
constexpr int kTile = 32;

struct Enc128Args {
  const uint8_t* cbs;
  int64_t stride;
  int64_t n_cb;
  const void* x;
  int64_t G, N, sx_g, sx_n;
  uint32_t* rec;
  int32_t* status;
  int bits, role, rec_words;
  uint32_t off_c, off_t, off_d, off_s;
  int64_t tiles_per_group;   // ceil(N / 32)
  int64_t tiles_per_block;
  int64_t blocks_per_group;
  PagedOut po;               // paged output (the PAGED kernels): rec is the pool
  // head_dim and projections of the codebook: 128 and 128, except for the
  // padded Haar kernels (PAD), which run a smaller head_dim as 128 with zero
  // rows and columns of R and S and zero input coordinates
  int dv, mv;
  float inv_sqrt_dv;         // 1 / sqrt(dv)
};

// Rotation u = H (D x) with H = H_128 in Sylvester order, split as
// H_128 = H_{128/NS} (x) H_NS: with row r = NS a + r', column c = NS b + c',
// H[r][c] = (-1)^popc(a & b) H_NS[r'][c'].  The NS-point transforms of the
// blocks of D x run on MFMA (NS/32 row tiles x NS/16 K-chunks per block), the
// remaining 128/NS-point butterfly across blocks on the VALU:
//   NS = 32 : 8 MFMAs and a 4-point butterfly (2 add/sub per coordinate);
//   NS = 64 : 16 MFMAs and a 2-point butterfly (1 per coordinate);
//   NS = 128: 32 MFMAs, no butterfly.
// NS = 32 is used: at the 32K-context key encode NS = 64 measured the same and
// NS = 128 6% slower (the matrix work lowers the clock more than the VALU
// work it saves).
// The fragments hold -H D (exact in 16 bits), so the products give v = -u:
// then u > 0 is exactly the sign bit of v (v is never -0: every MFMA sum
// starts from a +0 accumulator, and the butterfly adds and subtracts nonzero
// or +0 operands), one instruction per coordinate.
// Fragment (Mi, c) for output row tile Mi < NS/32 of the block and K-chunk c of
// x, lane l: A[rho = l%32][k = 8(l/32) + e] =
//   -H_NS[32 Mi + tile_row_index(rho)][(16 c + k) mod NS] * D[16 c + k].
constexpr int kNS = 32;
constexpr int kRotFrags = (kNS / 32) * 8;
static_assert(kNS == 32 || kNS == 64 || kNS == 128, "sub-transform size");
template <bool F16>
// dv: the codebook's head_dim (its D holds dv bits; columns past it multiply
// zero inputs and take no sign).
__device__ void build_hfrag(u32x4* hfrag, const uint32_t* dbits, int dv) {
  for (int f = threadIdx.x; f < kRotFrags * 64; f += blockDim.x) {
    const int lane = f & 63, c = (f >> 6) & 7, Mi = f >> 9;
    const int row = 32 * Mi + tile_row_index(lane & 31);
    u32x4 v;
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 16 * c + 8 * (lane >> 5) + 2 * q + hh;     // coordinate of x
        const uint32_t dsg = col < dv ? (dbits[col >> 5] >> (col & 31)) & 1u : 0u;
        const uint32_t neg = 1u ^ h_sign(row, col & (kNS - 1)) ^ dsg;
        const uint32_t one = F16 ? 0x3C00u : 0x3F80u;
        word |= (one | (neg << 15)) << (16 * hh);
      }
      v[q] = word;
    }
    hfrag[f] = v;
  }
}

// bf16 round-to-nearest-even of a float (bit pattern in the low 16 bits).
__device__ inline uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Haar rotation (R = sqrt(d) Q, float32 in the blob): u = R x as 96 MFMA products
// per 32-key tile.  R is split into three 16-bit terms so that every product
// with an exact 16-bit input is exact and the fp32 sums carry R to 24 bits or
// more.  bf16 (bf16 inputs): R = t0 + t1 + t2, each term the bf16 rounding of
// what is left.  f16 (f16 inputs): R = t0 + 2^-12 (t1 + t2), the two low terms
// scaled up by 2^12 to stay clear of the f16 subnormals; their products go to
// a second accumulator that is scaled back once per output block.
// Fragment (t, M, c), lane l: A[rho][k] = t_t of R[32M + tile_row_index(rho)][16c + 8(l/32) + e].
template <bool F16>
__device__ uint32_t r_term(float r, int t) {
  if (F16) {
    const _Float16 h0 = (_Float16)r;
    const float e1 = r - (float)h0;                        // exact
    const _Float16 h1 = (_Float16)(e1 * 4096.0f);
    const float e2 = e1 - (float)h1 * (1.0f / 4096.0f);    // exact
    const _Float16 h2 = (_Float16)(e2 * 4096.0f);
    const _Float16 hv = t == 0 ? h0 : (t == 1 ? h1 : h2);
    return __builtin_bit_cast(uint16_t, hv);
  }
  const uint32_t b0 = f32_to_bf16_rne(r);
  const float e1 = r - __uint_as_float(b0 << 16);
  const uint32_t b1 = f32_to_bf16_rne(e1);
  const uint32_t b2 = f32_to_bf16_rne(e1 - __uint_as_float(b1 << 16));
  return t == 0 ? b0 : (t == 1 ? b1 : b2);
}

// R is dv x dv (row-major); rows and columns past dv are zero.
template <bool F16>
__device__ void build_rfrag(u32x4* rfrag, const float* R, int dv) {
  for (int f = threadIdx.x; f < 96 * 64; f += blockDim.x) {
    const int lane = f & 63, c = (f >> 6) & 7, M = (f >> 9) & 3, t = f >> 11;
    const int row = 32 * M + tile_row_index(lane & 31);
    u32x4 v;
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 16 * c + 8 * (lane >> 5) + 2 * q + hh;
        // -R: the products give v = -u
        const float r = (row < dv && col < dv) ? -R[row * dv + col] : 0.0f;
        word |= r_term<F16>(r, t) << (16 * hh);
      }
      v[q] = word;
    }
    rfrag[f] = v;
  }
}

// S fragments (A operand of MFMA#2), negated: the residual is formed as
// w' = -w (from v = -u), so that (-S) w' = S w.  Fragment (Mp, c), lane l: row
// rho = l%32 is projection 32Mp + tile_row_index(rho); element e:
// -S[proj][qjl_coord(c, l/32, e)].
// S is mv x dv (row-major); rows past mv and columns past dv are zero.
__device__ void build_sfrag(u32x4* sfrag, const uint16_t* S, int dv, int mv) {
  for (int f = threadIdx.x; f < 4 * 8 * 64; f += blockDim.x) {
    const int lane = f & 63, c = (f >> 6) & 7, Mp = f >> 9;
    const int row = 32 * Mp + tile_row_index(lane & 31);
    u32x4 v;
    for (int q = 0; q < 4; ++q) {
      const int c0 = qjl_coord(c, lane >> 5, 2 * q), c1 = qjl_coord(c, lane >> 5, 2 * q + 1);
      const uint32_t lo = (row < mv && c0 < dv) ? S[row * dv + c0] : 0u;
      const uint32_t hi = (row < mv && c1 < dv) ? S[row * dv + c1] : 0u;
      v[q] = (lo | (hi << 16)) ^ 0x80008000u;
    }
    sfrag[f] = v;
  }
}


// LDS of encode128_kernel: rotation fragments, S fragments (keys), constants,
// and for the padded kernels a record staging row per wave (32 records of up
// to 18 words, 8 waves).
constexpr int kPadRecMax = 18;
constexpr size_t kPadStageBytes = 8 * 32 * kPadRecMax * 4;
template <bool KEY, bool HAAR, bool PAD = false>
constexpr size_t enc_lds_bytes() {
  return (HAAR ? 98304 : 32768) + (KEY ? 32768 : 0) + 128 + (PAD ? kPadStageBytes : 0);
}

// The page slot of token tok of group g for paged output, or null (the status
// word flagged) when the position or its page lies outside the table or pool.
__device__ inline uint32_t* paged_slot(const Enc128Args& a, int64_t g, int64_t tok, int rw) {
  const PagedOut& po = a.po;
  const int64_t b = po.head_major ? tok : g / po.Hkv, hd = po.head_major ? g : g % po.Hkv;
  const int32_t p = po.pos[b];
  const int64_t pi = p >= 0 ? p / po.tpp : po.max_pages;
  const int32_t page = pi < po.max_pages ? po.page_table[b * po.max_pages + pi] : -1;
  if (page < 0 || page >= po.num_pages) return nullptr;
  return a.rec + ((page * po.Hkv + hd) * po.tpp + p % po.tpp) * rw;
}

// The encode of workgroup `bid` of a launch over a's groups (the kernels below
// run it for their own workgroup index).
template <int K, bool KEY, int DT, bool HAAR, bool PAGED, int kWaves, bool PAD = false>
__device__ __forceinline__ void encode128_body(const Enc128Args& a, int64_t bid) {
  constexpr int kRotBytes = HAAR ? 98304 : 32768;
  static_assert(!HAAR || DT != 0, "the Haar rotation takes 16-bit inputs");
  static_assert(!PAD || (DT != 0 && !PAGED), "padding takes 16-bit inputs and contiguous records");
  extern __shared__ __align__(16) uint8_t smem[];
  u32x4* hfrag = reinterpret_cast<u32x4*>(smem);                // rotation: 8 (Hadamard) or 96 (Haar) fragments
  u32x4* sfrag = reinterpret_cast<u32x4*>(smem + kRotBytes);    // 32 KB (keys)
  float* consts = reinterpret_cast<float*>(smem + kRotBytes + (KEY ? 32768 : 0));

  constexpr int L = 1 << K;
  constexpr int NT = L / 2 - 1;  // positive thresholds
  const int64_t g = bid / a.blocks_per_group;
  const int64_t chunk = bid % a.blocks_per_group;
  const uint8_t* blob = a.cbs + (g % a.n_cb) * a.stride;
  if (threadIdx.x == 0 && a.status) {
    const BlobHeader* hd = reinterpret_cast<const BlobHeader*>(blob);
    if (hd->magic != kBlobMagic || hd->version != kBlobVersion || hd->head_dim != a.dv || hd->bits != a.bits ||
        hd->role != a.role || hd->projections != (KEY ? a.mv : 0) ||
        (int)hd->rotation != (HAAR ? kRotHaar : kRotHadamard))
      atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  }
  if constexpr (HAAR)
    build_rfrag<DT == 2>(hfrag, reinterpret_cast<const float*>(blob + a.off_d), PAD ? a.dv : kD);
  else
    build_hfrag<DT == 2>(hfrag, reinterpret_cast<const uint32_t*>(blob + a.off_d), PAD ? a.dv : kD);
  if (KEY) build_sfrag(sfrag, reinterpret_cast<const uint16_t*>(blob + a.off_s), PAD ? a.dv : kD, PAD ? a.mv : kM);
  if (threadIdx.x < L / 2) consts[threadIdx.x] = reinterpret_cast<const float*>(blob + a.off_c)[L / 2 + threadIdx.x];
  if (threadIdx.x < NT) consts[16 + threadIdx.x] = reinterpret_cast<const float*>(blob + a.off_t)[L / 2 + threadIdx.x];
  __syncthreads();

  float cpos[L / 2];
#pragma unroll
  for (int i = 0; i < L / 2; ++i) cpos[i] = consts[i];
  float tpos[NT > 0 ? NT : 1];
#pragma unroll
  for (int i = 0; i < NT; ++i) tpos[i] = consts[16 + i];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int64_t tile0 = chunk * a.tiles_per_block;
  const int64_t tile_end = min(tile0 + a.tiles_per_block, a.tiles_per_group);
  const uint32_t* xb16 = reinterpret_cast<const uint32_t*>(a.x);
  constexpr int RW = KEY ? (K * 4 + 4 + 2) : (K * 4 + 1);
  // (paged output stores through per-lane page slots; its resource is empty)
  const int RWo = PAD ? a.rec_words : RW;   // record words in memory
  const __amdgpu_buffer_rsrc_t rrs =
      __builtin_amdgcn_make_buffer_rsrc(PAGED ? a.rec : a.rec + g * a.N * RWo, 0, PAGED ? 0 : (int)(a.N * RWo * 4),
                                        kRsrcWord3);
  // padded kernels: plane words and sign words of the smaller record, this
  // wave's record staging row
  const int Wv = (a.dv + 31) / 32, SWv = (a.mv + 31) / 32;
  uint32_t* stage = reinterpret_cast<uint32_t*>(smem + kRotBytes + (KEY ? 32768 : 0) + 128) + wave * 32 * kPadRecMax;
  // coordinates (and projections) 32 M + 16 h + r exist for r < lim - 32 M
  const int dlim = a.dv - 16 * h, mlim = a.mv - 16 * h;
  const auto live16 = [](int n) -> uint32_t { return n <= 0 ? 0u : (n >= 16 ? 0xFFFFu : (1u << n) - 1u); };

  // bf16/f16 inputs: the next tile's rows are loaded while this tile is encoded
  const auto row_ptr = [&](int64_t t) {
    const int64_t tk = t * kTile + col;
    return reinterpret_cast<const u32x4*>(xb16 + (g * a.sx_g + (tk < a.N ? tk : 0) * a.sx_n) / 2);
  };
  u32x4 xr[8];
  if (DT != 0) {
    const u32x4* xp = row_ptr(tile0 + wave);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // tail lanes read row 0, never stored; padded chunks read the row start and are zeroed
      const bool in = !PAD || 16 * c + 8 * h < a.dv;
      xr[c] = xp[in ? 2 * c + h : 0];
      if (!in) xr[c] = u32x4{0u, 0u, 0u, 0u};
    }
    // as many dropped stores as a tile stores, so that on entry the memory
    // operations stand in the loop's order and its first wait is the same
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < (RW + 1) / 2; ++q) __builtin_amdgcn_raw_buffer_store_b32(0u, rrs, 0xC0000000u + 64u * q, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int64_t tile = tile0 + wave; tile < tile_end; tile += kWaves) {
    const int64_t tok = tile * kTile + col;
    const bool valid = tok < a.N;
    const int64_t xoff = g * a.sx_g + (valid ? tok : 0) * a.sx_n;

    // ---- x as the B operand of the rotation, K-chunk c: coords 16c + 8h .. +7
    u32x4 xb[8];
    u32x4 xb2[DT == 0 ? 8 : 1], xb3[DT == 0 ? 8 : 1];
    double ss = 0.0;
    if (DT == 0) {
      const float4* xp = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + xoff);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 v0 = xp[4 * c + 2 * h];   // tail lanes read row 0; their results are never stored
        const float4 v1 = xp[4 * c + 2 * h + 1];
        float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        u32x4 p1, p2, p3;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            float xv = f[2 * q + hh];
            ss = fma((double)xv, (double)xv, ss);
            uint32_t b1 = f32_to_bf16_rne(xv);
            float r1 = xv - __uint_as_float(b1 << 16);
            uint32_t b2 = f32_to_bf16_rne(r1);
            float r2 = r1 - __uint_as_float(b2 << 16);
            uint32_t b3 = f32_to_bf16_rne(r2);
            w1 |= b1 << (16 * hh);
            w2 |= b2 << (16 * hh);
            w3 |= b3 << (16 * hh);
          }
          p1[q] = w1; p2[q] = w2; p3[q] = w3;
        }
        xb[c] = p1; xb2[c] = p2; xb3[c] = p3;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) xb[c] = xr[c];
      // |x|^2: the 8 squares of a chunk summed in float32 by dot2 (exact
      // products), the chunk sums in float64
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float part = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) part = DT == 1 ? sumsq2_bf16(xb[c][q], part) : sumsq2_f16(xb[c][q], part);
        if (DT == 1 && part < 0x1p-100f)
          ss += sumsq8_bf16_f64(xb[c]);   // squares below the float32 range: the chunk again in float64
        else
          ss += (double)part;
      }
    }

    // ---- rotation: t_p = H_32 (D_p x_p) on MFMA (four independent accumulation
    // chains), then the H_4 butterfly across blocks gives u = H (D x)
    f32x16 u[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) u[p] = f32x16{};
    if constexpr (HAAR) {
      // u[M] = sum over K-chunks c and terms t of fragment (t, M, c) x chunk c
#pragma unroll
      for (int M = 0; M < 4; ++M) {
        f32x16 lo{};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
#pragma unroll
          for (int t = 0; t < 3; ++t) {
            const u32x4 rf = hfrag[((t * 4 + M) * 8 + c) * 64 + lane];
            if (DT == 2) {
              if (t == 0)
                u[M] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(rf), as<f16x8>(xb[c]), u[M], 0, 0, 0);
              else
                lo = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(rf), as<f16x8>(xb[c]), lo, 0, 0, 0);
            } else {
              u[M] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(rf), as<bf16x8>(xb[c]), u[M], 0, 0, 0);
            }
          }
          // keep the compiler from hoisting all fragment reads ahead of the products
          __builtin_amdgcn_sched_barrier(0);
        }
        if (DT == 2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) u[M][r] = fmaf(lo[r], 1.0f / 4096.0f, u[M][r]);
        }
      }
    }
    // Walsh-Hadamard: accumulator slot (block b, row tile Mi) = b * NS/32 + Mi
    // collects the NS-point transform of block b (K-chunks of that block)
#pragma unroll
    for (int cc = 0; cc < (HAAR ? 0 : kNS / 16); ++cc) {
#pragma unroll
      for (int b = 0; b < 128 / kNS; ++b) {
#pragma unroll
        for (int Mi = 0; Mi < kNS / 32; ++Mi) {
          const int c = b * (kNS / 16) + cc, slot = b * (kNS / 32) + Mi;
          const u32x4 hf = hfrag[(Mi * 8 + c) * 64 + lane];
          if (DT == 2) {
            u[slot] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(hf), as<f16x8>(xb[c]), u[slot], 0, 0, 0);
          } else {
            u[slot] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(hf), as<bf16x8>(xb[c]), u[slot], 0, 0, 0);
            if (DT == 0) {
              u[slot] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(hf), as<bf16x8>(xb2[c]), u[slot], 0, 0, 0);
              u[slot] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as<bf16x8>(hf), as<bf16x8>(xb3[c]), u[slot], 0, 0, 0);
            }
          }
        }
      }
    }
    if constexpr (!HAAR && kNS == 32) {
      // 4-point butterfly across the blocks: tile M = sum_b (-1)^popc(M & b) block b
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a0 = u[0][r] + u[1][r], b0 = u[0][r] - u[1][r];
        const float a1 = u[2][r] + u[3][r], b1 = u[2][r] - u[3][r];
        u[0][r] = a0 + a1;    // M = 0: + + + +
        u[1][r] = b0 + b1;    // M = 1: + - + -
        u[2][r] = a0 - a1;    // M = 2: + + - -
        u[3][r] = b0 - b1;    // M = 3: + - - +
      }
    } else if constexpr (!HAAR && kNS == 64) {
      // 2-point butterfly across the halves: tiles Mi and 2 + Mi
#pragma unroll
      for (int Mi = 0; Mi < 2; ++Mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float a = u[Mi][r], b = u[2 + Mi][r];
          u[Mi][r] = a + b;
          u[2 + Mi][r] = a - b;
        }
    }
    if (DT != 0) {
      // the last tile re-reads itself (a cache hit) so that the prefetch
      // registers are written on every iteration
      const u32x4* xp = row_ptr(tile + kWaves < tile_end ? tile + kWaves : tile);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bool in = !PAD || 16 * c + 8 * h < a.dv;
        xr[c] = xp[in ? 2 * c + h : 0];
        if (!in) xr[c] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    // ---- norm (float64, both halves of the vector)
    {
      uint32_t lo = __double2loint(ss), hi = __double2hiint(ss);
      auto plo = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      auto phi = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      const uint32_t olo = h ? plo[0] : plo[1], ohi = h ? phi[0] : phi[1];
      ss += __hiloint2double((int)ohi, (int)olo);
    }
    const bool finite = ss <= 3.4028234663852886e38;
    if (a.status && __ballot(valid && !finite && h == 0) != 0 && lane == 0) atomicOr(a.status, TQ_STATUS_NON_FINITE);
    const float n32 = (float)sqrt(ss);
    // A norm below 2^-40 would leave the residual's float32 squares to
    // underflow: such a token is quantized with u and n scaled by 2^64 (exact;
    // z = u / n and the signs are unchanged), gamma scaled back at the end.
    const bool tiny = n32 < 0x1p-40f;
    const float uscale_inv = tiny ? 0x1p-64f : 1.0f;
    if (__ballot(tiny) != 0) {
      const float f = tiny ? 0x1p64f : 1.0f;
#pragma unroll
      for (int M = 0; M < 4; ++M)
#pragma unroll
        for (int r = 0; r < 16; ++r) u[M][r] *= f;
    }
    const float nq = tiny ? n32 * 0x1p64f : n32;   // the norm in the units of u
    // power-of-two scale that brings the residual to O(1) for the f16 split
    const uint32_t nexp = (__float_as_uint(nq) >> 23) & 0xFFu;
    const float sc = (nq > 0.0f && nexp < 253u) ? __uint_as_float((254u - nexp) << 23) : 1.0f;

    // ---- quantize, pack planes, residual.  Lane half h holds coordinates
    // 32M + 16h + r in register r of tile M; bits are shifted in from r = 15 down
    // to 0 so that bit r of the 16-bit partial word is coordinate 32M + 16h + r.
    float tn[NT > 0 ? NT : 1];
#pragma unroll
    for (int t = 0; t < NT; ++t) tn[t] = tpos[t] * nq;   // thresholds in units of u
    const uint32_t nbits = __float_as_uint(nq);
    uint32_t pw[4], tw[NT > 0 ? NT : 1][4];                // sign-half words, thermometer words
    constexpr int KB = K - 1;                              // magnitude bits
    uint32_t mw[KB > 0 ? KB : 1][4];                       // values: magnitude index bits
    // keys: the four projection row tiles of S w accumulate slice by slice.  The
    // 16 products of slice M-1 are issued inside slice M's quantization, one
    // between every 4 VALU instructions, so that they run on the matrix core
    // while the same wave quantizes instead of in one block of 64 (2-3% faster
    // at the 32K-context encode, with far fewer waves waiting to issue).
    f32x16 acc[KEY ? 4 : 1];
#pragma unroll
    for (int j = 0; j < (KEY ? 4 : 1); ++j) acc[j] = f32x16{};
    u32x4 whi[KEY ? 2 : 1], wlo[KEY ? 2 : 1];     // split residual of the previous slice
    const auto qjl_slice = [&](int Ms) {
      // (-S) (w'_hi + w'_lo) over chunks 2Ms, 2Ms+1, four row tiles; the two
      // products on one accumulator are four MFMAs apart
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x4 sf[4];
#pragma unroll
        for (int Mp = 0; Mp < 4; ++Mp) sf[Mp] = sfrag[(Mp * 8 + 2 * Ms + p) * 64 + lane];
#pragma unroll
        for (int Mp = 0; Mp < 4; ++Mp)
          acc[Mp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf[Mp]), as<f16x8>(whi[p]), acc[Mp], 0, 0, 0);
#pragma unroll
        for (int Mp = 0; Mp < 4; ++Mp)
          acc[Mp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as<f16x8>(sf[Mp]), as<f16x8>(wlo[p]), acc[Mp], 0, 0, 0);
      }
    };
    float wsq = 0.0f;
#pragma unroll
    for (int M = 0; M < 4; ++M) {
      uint32_t pacc = 0;
      uint32_t tacc[NT > 0 ? NT : 1];
#pragma unroll
      for (int t = 0; t < NT; ++t) tacc[t] = 0;
      if constexpr (!KEY && KB >= 1 && KB <= 3) {
        // values need no magnitude for a residual: the magnitude index
        // m = #{t : |u| > tn_t} by binary search over the sorted thresholds,
        // its bits shifted straight into words (KB compares instead of 2^KB - 1)
        uint32_t macc[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) macc[b] = 0;
#pragma unroll
        for (int r = 15; r >= 0; --r) {
          const float uu = u[M][r];
          pacc = neg_bit(pacc, uu);
          if constexpr (KB == 1) {
            thr_bit(macc[0], uu, tn[0]);
          } else if constexpr (KB == 2) {
            const uint64_t m1 = thr_bit(macc[1], uu, tn[1]);
            thr_bit(macc[0], uu, sel_mask(m1, tn[2], tn[0]));
          } else {
            const uint64_t m2 = thr_bit(macc[2], uu, tn[3]);
            const uint64_t m1 = thr_bit(macc[1], uu, sel_mask(m2, tn[5], tn[1]));
            const float ta = sel_mask(m2, tn[6], tn[2]), tb = sel_mask(m2, tn[4], tn[0]);
            thr_bit(macc[0], uu, sel_mask(m1, ta, tb));
          }
        }
        pw[M] = pacc;
#pragma unroll
        for (int b = 0; b < KB; ++b) mw[b][M] = macc[b];
        continue;
      }
      float wv[16];
      uint32_t macc2[2] = {0u, 0u};               // keys with three thresholds: magnitude index bits
#pragma unroll
      for (int r = 15; r >= 0; --r) {
        const float uu = u[M][r];                 // -u
        pacc = neg_bit(pacc, uu);                 // bit: u > 0
        // +n where u > 0, -n elsewhere: w' = -w = -u + (+-n) c_mag
        const float nsg = __uint_as_float((~__float_as_uint(uu) & 0x80000000u) | nbits);
        float mag = cpos[0];
        if constexpr (KEY && NT == 3) {
          // three thresholds: the magnitude index by binary search (the same
          // |u| > tn compares), its bits shifted into words, and the centroid
          // chosen pairwise: 8 instructions instead of 3 x 3
          const uint64_t m1 = thr_bit(macc2[1], uu, tn[1]);
          const uint64_t m0 = thr_bit(macc2[0], uu, sel_mask(m1, tn[2], tn[0]));
          mag = sel_mask(m0, sel_mask(m1, cpos[3], cpos[1]), sel_mask(m1, cpos[2], cpos[0]));
        } else {
          if (NT > 0) mag = thr_first(tacc[0], uu, tn[0], cpos[0], cpos[NT > 0 ? 1 : 0]);
#pragma unroll
          for (int t = 1; t < NT; ++t) thr_step(tacc[t], mag, uu, tn[t], cpos[t + 1]);
        }
        if (KEY) {
          // w' = -(u - n c[idx]) with c[idx] = +-mag: fma(+-n, mag, -u), +n on the positive half
          float w = fmaf(nsg, mag, uu);
          if (PAD && r >= dlim - 32 * M) w = 0.0f;   // no residual at padded coordinates
          wsq = fmaf(w, w, wsq);
          wv[r] = w;
        }
      }
      pw[M] = pacc;
#pragma unroll
      for (int t = 0; t < NT; ++t) tw[t][M] = tacc[t];
      if constexpr (KEY && NT == 3) {
        mw[0][M] = macc2[0];
        mw[1][M] = macc2[1];
      }
      if constexpr (KEY) {
        if (M > 0) qjl_slice(M - 1);
        // B operand of projection chunk c = 2M + p: element e = register 8p + e
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t h, l;
            split_f16x2(wv[8 * p + 2 * q], wv[8 * p + 2 * q + 1], sc, h, l);
            whi[p][q] = h;
            wlo[p][q] = l;
          }
        if (M > 0) {
          // the region's order: the 8 fragment reads, then the 16 products of
          // slice M-1 each followed by 4 VALU instructions of slice M
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (KEY) qjl_slice(3);

    // ---- QJL signs of S w (keys), one alignbit each
    uint32_t sw[4] = {0, 0, 0, 0};   // inverted sign bits (1 = negative)
    float gam = 0.0f;
    if (KEY) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t a2 = 0;
#pragma unroll
        for (int r = 15; r >= 0; --r) a2 = __builtin_amdgcn_alignbit(a2, __float_as_uint(acc[j][r]), 31);
        sw[j] = a2;
      }
      auto pg = __builtin_amdgcn_permlane32_swap(__float_as_uint(wsq), __float_as_uint(wsq), false, false);
      const float tot = __uint_as_float(pg[0]) + __uint_as_float(pg[1]);
      gam = sqrtf(tot) * uscale_inv * (PAD ? a.inv_sqrt_dv : 0.08838834764831845f);   // |w| / sqrt(d)
    }

    // ---- plane words: MSB plane = [z > 0]; the lower planes hold cnt on the
    // positive half and its complement (L/2 - 1 - cnt) on the other half, cnt
    // being the number of positive thresholds below |z| (thermometer -> binary)
    constexpr int R = KEY ? (K * 4 + 4 + 2) : (K * 4 + 1);
    uint32_t words[R];
    uint32_t part[KEY ? K * 4 + 4 : K * 4];
#pragma unroll
    for (int M = 0; M < 4; ++M) {
      uint32_t pl[K];
      pl[K - 1] = pw[M] & (PAD ? live16(dlim - 32 * M) : 0xFFFFu);
#pragma unroll
      for (int p = 0; p < K - 1; ++p) {
        uint32_t cb = 0;
        if constexpr ((!KEY && KB <= 3) || (KEY && NT == 3)) {
          cb = mw[p][M];                   // bit p of cnt from the binary search
        } else {
          // bit p of cnt = XOR of the thermometer bits [cnt >= j] for j a multiple of 2^p
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (((t + 1) & ((1 << p) - 1)) == 0) cb ^= tw[t][M];
        }
        pl[p] = ~(cb ^ pw[M]) & (PAD ? live16(dlim - 32 * M) : 0xFFFFu);   // pos ? cnt_p : ~cnt_p
      }
      for (int p = 0; p < K; ++p) part[p * 4 + M] = h ? (pl[p] << 16) : (pl[p] & 0xFFFFu);
    }
    if (KEY) {
#pragma unroll
      for (int Mp = 0; Mp < 4; ++Mp) {
        const uint32_t sv = ~sw[Mp] & (PAD ? live16(mlim - 32 * Mp) : 0xFFFFu);
        part[K * 4 + Mp] = h ? (sv << 16) : sv;
      }
    }
    // complete two words per swap: half 0 finishes word 2i (and stores it), half 1 word 2i+1
    constexpr int NP = KEY ? K * 4 + 4 : K * 4;
#pragma unroll
    for (int i = 0; i < NP / 2; ++i) {
      auto sp = __builtin_amdgcn_permlane32_swap(part[2 * i], part[2 * i + 1], false, false);
      words[2 * i] = part[2 * i] | sp[1];          // valid in half 0
      words[2 * i + 1] = part[2 * i + 1] | sp[0];  // valid in half 1
    }
    if (KEY) {
      words[K * 4 + 4] = __float_as_uint(n32);
      words[K * 4 + 5] = __float_as_uint(gam);
    } else {
      words[K * 4] = __float_as_uint(n32);
    }
    // every store is issued: one past the group's records (a ragged tail's
    // token, the odd word of a value record) is dropped by the buffer bounds,
    // so the next tile's loads never wait for this tile's stores
    if constexpr (PAGED) {
      uint32_t* dst = valid ? paged_slot(a, g, tok, R) : nullptr;
      if (valid && !dst && h == 0 && a.status) atomicOr(a.status, TQ_STATUS_BAD_PAGE);
      if (dst) {
#pragma unroll
        for (int q = 0; q < (R + 1) / 2; ++q) {
          const int wi = 2 * q + h;
          if (wi < R) dst[wi] = h ? words[(2 * q + 1) < R ? 2 * q + 1 : 0] : words[2 * q];
        }
      }
    } else if constexpr (PAD) {
      // the record of a smaller head_dim: plane p word M < Wv at p Wv + M, sign
      // word Mp < SWv after the planes, then n32 (and gamma); through this
      // wave's staging row, then stored as the tile's contiguous records
#pragma unroll
      for (int q = 0; q < (R + 1) / 2; ++q) {
        const int wi = 2 * q + h;
        if (wi >= R) continue;
        const uint32_t v = h ? words[(2 * q + 1) < R ? 2 * q + 1 : 0] : words[2 * q];
        int t;
        if (wi < K * 4) {
          t = (wi & 3) < Wv ? (wi >> 2) * Wv + (wi & 3) : -1;
        } else if (KEY && wi < K * 4 + 4) {
          t = wi - K * 4 < SWv ? K * Wv + (wi - K * 4) : -1;
        } else {
          t = K * Wv + (KEY ? SWv : 0) + (wi - (KEY ? K * 4 + 4 : K * 4));
        }
        if (t >= 0) stage[col * RWo + t] = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int ntok = (int)(a.N - tile * kTile < kTile ? a.N - tile * kTile : kTile);
      const uint32_t base = (uint32_t)(tile * kTile * RWo * 4);
      for (int e = lane; e < ntok * RWo; e += 64) __builtin_amdgcn_raw_buffer_store_b32(stage[e], rrs, base + 4u * e, 0, 0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      const uint32_t ro = valid ? (uint32_t)(tok * R * 4) : 0xC0000000u;
#pragma unroll
      for (int q = 0; q < (R + 1) / 2; ++q) {
        const int wi = 2 * q + h;
        const uint32_t v = h ? words[(2 * q + 1) < R ? 2 * q + 1 : 0] : words[2 * q];
        __builtin_amdgcn_raw_buffer_store_b32(v, rrs, wi < R ? ro + 4u * wi : 0xC0000000u, 0, 0);
      }
    }
  }
}

template <int K, bool KEY, int DT, bool HAAR, bool PAGED, bool PAD = false>
__global__ __launch_bounds__((64 * waves_for<K, KEY, DT, HAAR, PAD>())) void encode128_kernel(Enc128Args a) {
  encode128_body<K, KEY, DT, HAAR, PAGED, waves_for<K, KEY, DT, HAAR, PAD>(), PAD>(a, blockIdx.x);
}

// Keys and values of an append in one launch (paged output): the first
// ka.G * ka.blocks_per_group workgroups encode the keys, the rest the values.
// Both roles run the keys' wave count, and the LDS is the keys' (the larger).
template <int KK, int KV, int DT, bool PAGED = true>
__global__ __launch_bounds__((64 * waves_for<KK, true, DT, false>())) void encode128_pair_kernel(Enc128Args ka,
                                                                                                 Enc128Args va) {
  constexpr int W = waves_for<KK, true, DT, false>();
  const int64_t nk = ka.G * ka.blocks_per_group;
  if ((int64_t)blockIdx.x < nk)
    encode128_body<KK, true, DT, false, PAGED, W>(ka, blockIdx.x);
  else
    encode128_body<KV, false, DT, false, PAGED, W>(va, (int64_t)blockIdx.x - nk);
}

// ~256 workgroups (one per CU) in total, never more tiles than the group
// holds; a multiple of the wave count.
inline void split_tiles(Enc128Args& a, int waves) {
  // tiles per wave: the launch spread over ~256 workgroups, at least one (a
  // small launch takes more workgroups rather than more tiles per wave)
  const int64_t total = a.tiles_per_group * a.G;
  const int64_t tpw = (total + 256 * waves - 1) / (256 * waves);
  int64_t per_block = (tpw < 1 ? 1 : tpw) * waves;
  if (per_block > a.tiles_per_group) per_block = (a.tiles_per_group + waves - 1) / waves * waves;
  a.tiles_per_block = per_block;
  a.blocks_per_group = (a.tiles_per_group + per_block - 1) / per_block;
}

template <int K, bool KEY, int DT, bool HAAR, bool PAGED, bool PAD = false>
int launch_one(Enc128Args a, hipStream_t s) {
  split_tiles(a, waves_for<K, KEY, DT, HAAR, PAD>());
  const size_t lds = enc_lds_bytes<KEY, HAAR, PAD>();
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&encode128_kernel<K, KEY, DT, HAAR, PAGED, PAD>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return -10;
    attr_set = true;
  }
  const int64_t blocks = a.G * a.blocks_per_group;
  hipLaunchKernelGGL((encode128_kernel<K, KEY, DT, HAAR, PAGED, PAD>), dim3((unsigned)blocks),
                     dim3(64 * waves_for<K, KEY, DT, HAAR, PAD>()), lds, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

template <int K, bool KEY>
int launch_dt(const Enc128Args& a, int dt, bool haar, bool paged, hipStream_t s) {
  if (paged) {
    if (haar || a.dv != kD) return -13;
    if (dt == TQ_BF16) return launch_one<K, KEY, 1, false, true>(a, s);
    if (dt == TQ_F16) return launch_one<K, KEY, 2, false, true>(a, s);
    return launch_one<K, KEY, 0, false, true>(a, s);
  }
  if (haar && a.dv < kD)
    return dt == TQ_F16 ? launch_one<K, KEY, 2, true, false, true>(a, s) : launch_one<K, KEY, 1, true, false, true>(a, s);
  if (a.dv < kD)
    return dt == TQ_F16 ? launch_one<K, KEY, 2, false, false, true>(a, s) : launch_one<K, KEY, 1, false, false, true>(a, s);
  if (haar) return dt == TQ_F16 ? launch_one<K, KEY, 2, true, false>(a, s) : launch_one<K, KEY, 1, true, false>(a, s);
  if (dt == TQ_BF16) return launch_one<K, KEY, 1, false, false>(a, s);
  if (dt == TQ_F16) return launch_one<K, KEY, 2, false, false>(a, s);
  return launch_one<K, KEY, 0, false, false>(a, s);
}

}  // namespace

bool fast128_encode_supported(const Layout& L, int dtype, const void* x, int64_t sx_g, int64_t sx_n, int64_t N) {
  // Haar: 16-bit inputs (their products with 16-bit terms of R are exact).  A
  // smaller head_dim runs padded to 128 with 16-bit inputs and up to 128
  // projections: for Haar any multiple of 8; for Walsh-Hadamard a power of two
  // (zero inputs past d: the first d rows of H_128 D x are then H_d D x)
  const bool haar = L.rotation == kRotHaar && dtype != TQ_F32;
  if (L.rotation != kRotHadamard && !haar) return false;
  const bool pad = dtype != TQ_F32 && L.d < kD && L.d >= 8 && L.d % 8 == 0 &&
                   (haar || (L.d & (L.d - 1)) == 0);
  if (L.d != kD && !pad) return false;
  if (N > (int64_t(1) << 30) / (4 * L.rec_words)) return false;   // 32-bit buffer offsets per group
  if (L.role == TQ_ROLE_KEY && (L.k < 1 || L.k > 3)) return false;
  if (L.role == TQ_ROLE_KEY && (pad ? (L.m < 1 || L.m > kM) : L.m != kM)) return false;
  if (L.role == TQ_ROLE_VALUE && (L.k < 1 || L.k > 4)) return false;
  const int esz = dtype == TQ_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(x) & 15) || ((sx_g * esz) & 15) || ((sx_n * esz) & 15)) return false;
  return true;
}

namespace {

Enc128Args make_args(const Layout& L, const void* cbs, int64_t n_cb, const void* x, int64_t G, int64_t N,
                     int64_t sx_g, int64_t sx_n, uint32_t* rec, int32_t* status, const PagedOut* po) {
  Enc128Args a;
  a.po = po ? *po : PagedOut{};
  a.cbs = static_cast<const uint8_t*>(cbs);
  a.stride = L.total;
  a.n_cb = n_cb;
  a.x = x;
  a.G = G; a.N = N; a.sx_g = sx_g; a.sx_n = sx_n;
  a.rec = rec;
  a.status = status;
  a.bits = L.bits; a.role = L.role; a.rec_words = L.rec_words;
  a.off_c = L.off_c; a.off_t = L.off_t; a.off_d = L.off_d; a.off_s = L.off_s;
  a.tiles_per_group = (N + kTile - 1) / kTile;
  a.dv = L.d;
  a.mv = L.role == TQ_ROLE_KEY ? L.m : 0;
  a.inv_sqrt_dv = (float)(1.0 / sqrt((double)L.d));
  return a;
}

template <int KK, int KV, int DT, bool PAGED = true>
int launch_pair(Enc128Args ka, Enc128Args va, hipStream_t s) {
  constexpr int W = waves_for<KK, true, DT, false>();
  split_tiles(ka, W);
  split_tiles(va, W);
  const size_t lds = enc_lds_bytes<true, false>();
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&encode128_pair_kernel<KK, KV, DT, PAGED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return -10;
    attr_set = true;
  }
  const int64_t blocks = ka.G * ka.blocks_per_group + va.G * va.blocks_per_group;
  hipLaunchKernelGGL((encode128_pair_kernel<KK, KV, DT, PAGED>), dim3((unsigned)blocks), dim3(64 * W), lds, s, ka,
                     va);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

template <int KK, int DT>
int launch_pair_v(const Enc128Args& ka, const Enc128Args& va, int kv, hipStream_t s) {
  switch (kv) {
    case 1: return launch_pair<KK, 1, DT>(ka, va, s);
    case 2: return launch_pair<KK, 2, DT>(ka, va, s);
    case 3: return launch_pair<KK, 3, DT>(ka, va, s);
    case 4: return launch_pair<KK, 4, DT>(ka, va, s);
    default: return 1;
  }
}

}  // namespace

int launch_append_fast128(const Layout& K, const Layout& V, const void* kcbs, int64_t n_kcb, const void* vcbs,
                          int64_t n_vcb, const void* k, const void* v, int dtype, int64_t G, int64_t N, int64_t sx_g,
                          int64_t sx_n, uint32_t* kpool, uint32_t* vpool, int32_t* status, hipStream_t s,
                          const PagedOut& po) {
  if (K.rotation != kRotHadamard || V.rotation != kRotHadamard) return 1;
  const Enc128Args ka = make_args(K, kcbs, n_kcb, k, G, N, sx_g, sx_n, kpool, status, &po);
  const Enc128Args va = make_args(V, vcbs, n_vcb, v, G, N, sx_g, sx_n, vpool, status, &po);
  // the pairs whose key and value kernels take the same workgroup shape
  if (dtype == TQ_BF16 && K.k == 1) return launch_pair_v<1, 1>(ka, va, V.k, s);
  if (dtype == TQ_BF16 && K.k == 2) return launch_pair_v<2, 1>(ka, va, V.k, s);
  if (dtype == TQ_F16 && K.k == 1) return launch_pair_v<1, 2>(ka, va, V.k, s);
  return 1;
}

int launch_encode_pair_fast128(const Layout& K, const Layout& V, const void* kcbs, int64_t n_kcb, const void* vcbs,
                               int64_t n_vcb, const void* k, const void* v, int dtype, int64_t G, int64_t N,
                               int64_t sx_g, int64_t sx_n, uint32_t* krec, uint32_t* vrec, int32_t* status,
                               hipStream_t s) {
  // head_dim 128 only: the padded bodies of smaller head dims are not paired
  if (K.d != kD || V.d != kD || K.rotation != kRotHadamard || V.rotation != kRotHadamard || K.k != 2 || V.k < 2 ||
      V.k > 3)
    return 1;
  const Enc128Args ka = make_args(K, kcbs, n_kcb, k, G, N, sx_g, sx_n, krec, status, nullptr);
  const Enc128Args va = make_args(V, vcbs, n_vcb, v, G, N, sx_g, sx_n, vrec, status, nullptr);
  // turbo3 keys with 2- or 3-bit values, 32-bit or bfloat16 inputs: both
  // encodes in one launch, each workgroup taking a key or a value range
  if (dtype == TQ_F32) return V.k == 2 ? launch_pair<2, 2, 0, false>(ka, va, s) : launch_pair<2, 3, 0, false>(ka, va, s);
  if (dtype == TQ_BF16) return V.k == 2 ? launch_pair<2, 2, 1, false>(ka, va, s) : launch_pair<2, 3, 1, false>(ka, va, s);
  return 1;
}

int launch_encode_fast128(const Layout& L, const void* cbs, int64_t n_cb, const void* x, int dtype, int64_t G,
                          int64_t N, int64_t sx_g, int64_t sx_n, uint32_t* rec, int32_t* status, hipStream_t s,
                          const PagedOut* po) {
  const Enc128Args a = make_args(L, cbs, n_cb, x, G, N, sx_g, sx_n, rec, status, po);
  const bool key = L.role == TQ_ROLE_KEY;
  const bool haar = L.rotation == kRotHaar;
  switch (L.k * 2 + (key ? 1 : 0)) {
    case 1 * 2 + 1: return launch_dt<1, true>(a, dtype, haar, po != nullptr, s);
    case 2 * 2 + 1: return launch_dt<2, true>(a, dtype, haar, po != nullptr, s);
    case 3 * 2 + 1: return launch_dt<3, true>(a, dtype, haar, po != nullptr, s);
    case 1 * 2: return launch_dt<1, false>(a, dtype, haar, po != nullptr, s);
    case 2 * 2: return launch_dt<2, false>(a, dtype, haar, po != nullptr, s);
    case 3 * 2: return launch_dt<3, false>(a, dtype, haar, po != nullptr, s);
    case 4 * 2: return launch_dt<4, false>(a, dtype, haar, po != nullptr, s);
    default: return -13;
  }
}

}  // namespace tq
