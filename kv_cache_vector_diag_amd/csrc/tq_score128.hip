// head_dim-128 scoring from compressed keys for gfx950 (CDNA4, wave64): the
// score kernel streams the key records of (sequence, kv head) ranges through
// the shared query-side preparation and tile scoring of tq_score_core.h (the
// formula and its int8-MFMA evaluation are stated there).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_fast.h"
#include "tq_score_core.h"

namespace tq {

// Scalar load through a buffer resource (s_buffer_load_dword): the page id of a
// wave's tile is uniform, and a scalar load keeps it out of the vector memory
// counter that orders the record loads.
typedef int i32x4r __attribute__((ext_vector_type(4)));
__device__ int32_t s_buffer_load_i32(i32x4r rsrc, int32_t offset, int32_t aux) __asm("llvm.amdgcn.s.buffer.load.i32");

namespace {

using sc128::i32x4;
using sc128::kD;
using sc128::kM;
using sc128::Masks;

// Workgroup size: 16 waves (one workgroup per CU) while the A fragments fit in
// 128 VGPRs; 8 waves for the 3-plane codebook, whose fragments need more.
template <int K>
constexpr int block_threads() { return K <= 2 ? 1024 : 512; }

struct Score128Args {
  const uint8_t* cbs;
  int64_t stride, n_cb;
  const uint32_t* krec;
  int64_t B, Hkv, T, Hq;
  const void* q;
  int q_dtype;
  float scale;
  float* scores;
  int32_t* status;
  int bits, rec_words, gq;   // gq = query heads per kv head (1, 2 or 4)
  int rotation;              // kRotHadamard or kRotHaar
  uint32_t off_c, off_d, off_s;
  int64_t tiles, tiles_per_block, blocks_per_group;
  // paged keys (page_table not null): krec is the pool [num_pages][Hkv][tpp][rec],
  // token t of (b, h) in page page_table[b * max_pages + t / tpp], slot t % tpp
  const int32_t* page_table;
  int64_t max_pages, num_pages;
  int tpp;
};

template <int K, bool PAGED>
__global__ __launch_bounds__(block_threads<K>()) void score128_kernel(Score128Args a) {
  using Mk = Masks<K>;
  constexpr int kBlock = block_threads<K>();
  constexpr int kWaves = kBlock / 64;
  constexpr int NMF = Mk::kMfma;                 // MFMAs per tile
  constexpr int RW = sc128::key_words<K>();      // record words
  __shared__ sc128::QueryLds<K> qs;
  constexpr int kStage = 64 * ((16 * RW + 63) / 64);   // 8-byte chunks per wave: one tile, rounded up
  __shared__ uint2 stage[kWaves * kStage];
  __shared__ uint32_t next_tile;                         // the workgroup's tile counter

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches on it stay scalar
  const int64_t grp = blockIdx.x / a.blocks_per_group;      // (b, kv head)
  const int64_t chunk = blockIdx.x % a.blocks_per_group;
  const int64_t b = grp / a.Hkv, hkv = grp % a.Hkv;
  const uint8_t* blob = a.cbs + (grp % a.n_cb) * a.stride;
  if (tid == 0 && a.status) {
    const BlobHeader* hd = reinterpret_cast<const BlobHeader*>(blob);
    if (hd->magic != kBlobMagic || hd->version != kBlobVersion || hd->head_dim != kD || hd->bits != a.bits ||
        hd->role != TQ_ROLE_KEY || hd->projections != kM || (int)hd->rotation != a.rotation)
      atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  }
  const sc128::QuerySrc src{reinterpret_cast<const float*>(blob + a.off_c),
                            reinterpret_cast<const uint32_t*>(blob + a.off_d),
                            reinterpret_cast<const _Float16*>(blob + a.off_s),
                            a.q, a.q_dtype, ((b * a.Hq) + hkv * a.gq) * kD, a.gq,
                            a.rotation == kRotHaar ? reinterpret_cast<const float*>(blob + a.off_d) : nullptr};
  sc128::QueryRegs<K> qr;
  sc128::query_load<K>(src, qr, tid, wave, lane);
  __builtin_amdgcn_sched_barrier(0);

  const int h = lane >> 5, col = lane & 31;
  const int64_t tile0 = chunk * a.tiles_per_block;
  const int64_t tile_end = min(tile0 + a.tiles_per_block, a.tiles);
  // A tile's 32 records are contiguous: they are loaded as 8-byte chunks by
  // consecutive lanes (RW even, so every record is 8-byte aligned and a ragged
  // tile ends on a chunk boundary), kPrefetch tiles ahead in a register ring,
  // then passed through this wave's LDS row so that lane (col, h) reads the
  // words it feeds: words h and h+2 of every bit plane and of the sign mask,
  // then n and gamma.
  // The loads go through a buffer resource that ends at this workgroup's last
  // record: past it (the ragged tail, prefetches beyond the range) they return
  // zero without a memory access, so every load is issued unconditionally and
  // the waits before each tile count exactly the loads and stores still needed
  // in flight (predicated loads make the compiler drain everything instead).
  // A zero record scores 0 and is never stored.
  constexpr int NCH = (16 * RW + 63) / 64;               // 8-byte chunks per lane per tile
  constexpr int kPrefetch = 2;
  uint2 raw[kPrefetch][NCH];
  const int64_t rec_end = min(tile_end * 32, a.T);
  bool bad_page = false;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.krec + grp * a.T * RW), 0, (int)(rec_end * RW * 4), kRsrcWord3);
  // paged: this sequence's row of the page table as a scalar buffer
  const uint64_t ptab = reinterpret_cast<uint64_t>(a.page_table + b * a.max_pages);
  const i32x4r prow = {(int)(uint32_t)ptab, (int)((uint32_t)(ptab >> 32) & 0xFFFFu), (int)(a.max_pages * 4),
                       kRsrcWord3};
  const auto load_raw = [&](int64_t t, uint2* rw) {
    if constexpr (PAGED) {
      // a tile lies in one page (tpp a multiple of 32): a resource per tile,
      // ending at the tile's last valid record; a bad page reads nothing
      const int64_t tok = t * 32;
      const int64_t nrec = rec_end - tok < 0 ? 0 : (rec_end - tok < 32 ? rec_end - tok : 32);
      const int64_t pi = tok / a.tpp;
      const int64_t page = nrec > 0 && pi < a.max_pages ? s_buffer_load_i32(prow, (int)(pi * 4), 0) : 0;
      const bool ok = page >= 0 && page < a.num_pages;
      bad_page |= !ok && nrec > 0;                 // reported once, at the end
      const uint32_t* base = a.krec + ((ok ? page : 0) * a.Hkv + hkv) * a.tpp * RW + (tok % a.tpp) * RW;
      const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint32_t*>(base), 0, ok ? (int)(nrec * RW * 4) : 0, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        rw[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(prs, 8u * lane + 512u * i, 0, 0));
      return;
    }
    const uint32_t base = (uint32_t)(t * 32 * RW * 4) + 8u * lane;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      rw[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(krs, base + 512u * i, 0, 0));
  };
  // scores of this (b, kv head): [gq][T]; stores past the end are dropped
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      a.scores + (b * a.Hq + hkv * a.gq) * a.T, 0, (int)(a.gq * a.T * 4), kRsrcWord3);
  uint2* st2 = stage + wave * kStage;
  const uint32_t* st = reinterpret_cast<const uint32_t*>(st2) + col * RW;
  // Tiles are handed out one at a time from the workgroup's counter: the waves
  // of a SIMD get unequal shares of its issue slots, and with a fixed split
  // the favoured ones finished ~20 us before the last (at the 32K-context
  // shape), leaving the tail of the kernel to a few waves and HBM underused.
  // A wave's first kPrefetch tiles are fixed (wave + sl * kWaves).
  int64_t slot_tile[kPrefetch];
#pragma unroll
  for (int sl = 0; sl < kPrefetch; ++sl) slot_tile[sl] = tile0 + wave + sl * kWaves;
  if (tid == 0) next_tile = kPrefetch * kWaves;          // visible after the query side's barriers
  const auto grab = [&]() -> int64_t {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(&next_tile, 1u);
    return tile0 + (int64_t)__builtin_amdgcn_readfirstlane(v);
  };
  // The first tiles' records are in flight while the query side is prepared,
  // issued once the query loads have landed (at kernel start every workgroup
  // loads at once, and the small query loads would otherwise wait behind the
  // records).  Issued in slot order, each followed by two stores past the end
  // of the scores (dropped by the hardware): on entry the memory operations
  // then stand in the same order as in the loop (a slot's loads, its two score
  // stores), so the wait before each slot leaves the later slots' loads in
  // flight.
  const auto prefetch = [&]() {
#pragma unroll
    for (int sl = 0; sl < kPrefetch; ++sl) {
      load_raw(slot_tile[sl], raw[sl]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_raw_buffer_store_b32(0u, srs, 0xC0000000u, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(0u, srs, 0xC0000040u, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  sc128::query_build<K, kBlock>(qs, qr, a.gq, tid, wave, lane, prefetch);
  i32x4 A[NMF];
#pragma unroll
  for (int f = 0; f < NMF; ++f) A[f] = qs.afrag[f * 64 + lane];

  // A wave's tiles come in increasing order, slot after slot, so the loop ends
  // when slot 0 holds a tile past the range.  The slots after it in the same
  // pass may hold one too: such a tile reads zeros and stores nothing (one
  // exit per pass keeps the compiler's waits at one slot's loads).
  while (slot_tile[0] < tile_end) {
#pragma unroll
    for (int sl = 0; sl < kPrefetch; ++sl) {
      const int64_t tile = slot_tile[sl];
      const int64_t tok = tile * 32 + col;
      const bool valid = tok < rec_end;   // tokens past the range store nothing
#pragma unroll
      for (int i = 0; i < NCH; ++i) st2[lane + 64 * i] = raw[sl][i];
      slot_tile[sl] = grab();
      load_raw(slot_tile[sl], raw[sl]);
      float sa, sb2;
      sc128::score_tile<K>(A, st, qs.consts, a.scale, h, sa, sb2);
      // heads ha, hb >= gq land past the end of the resource, as does an invalid token
      const int ha = 2 * h, hb = 2 * h + 1;
      const uint32_t so = valid ? (uint32_t)tok * 4u : 0xC0000000u;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sa), srs, so + (uint32_t)(ha * a.T * 4), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sb2), srs, so + (uint32_t)(hb * a.T * 4), 0, 0);
    }
  }
  if (bad_page && lane == 0 && a.status) atomicOr(a.status, TQ_STATUS_BAD_PAGE);
}

template <int K>
int launch_k(Score128Args a, hipStream_t s) {
  const auto kern = a.page_table ? score128_kernel<K, true> : score128_kernel<K, false>;
  constexpr int kWaves = block_threads<K>() / 64;
  // about one workgroup of 16 waves per CU, at least 16 tiles per wave
  const int64_t groups = a.B * a.Hkv;
  int64_t per_block = (a.tiles * groups + 256 * (16 / kWaves) - 1) / (256 * (16 / kWaves));
  if (per_block < 16 * kWaves) per_block = 16 * kWaves;
  if (per_block > a.tiles) per_block = a.tiles;
  a.tiles_per_block = per_block;
  a.blocks_per_group = (a.tiles + per_block - 1) / per_block;
  const int64_t blocks = groups * a.blocks_per_group;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(block_threads<K>()), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace

bool fast128_scores_supported(const Layout& L, int64_t Hkv, int64_t Hq, int64_t T, const void* krec) {
  if (L.d != kD || L.m != kM || L.k < 1 || L.k > 3) return false;
  if (L.rotation != kRotHadamard && L.rotation != kRotHaar) return false;
  if (reinterpret_cast<uintptr_t>(krec) & 7) return false;   // records read as 8-byte chunks
  // 32-bit buffer offsets: a group's records and its [gq][T] scores stay below 2^30 bytes
  if (T > (int64_t(1) << 30) / (4 * L.rec_words) || T > (int64_t(1) << 30) / 16) return false;
  const int64_t gq = Hq / Hkv;
  return gq == 1 || gq == 2 || gq == 4;
}

int launch_scores_fast128(const Layout& L, const void* cbs, int64_t n_cb, const uint32_t* krec, int64_t B,
                          int64_t Hkv, int64_t T, const void* q, int q_dtype, int64_t Hq, float scale,
                          float* scores, int32_t* status, hipStream_t s, const int32_t* page_table, int64_t max_pages,
                          int tpp, int64_t num_pages) {
  Score128Args a;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.tpp = tpp;
  a.cbs = static_cast<const uint8_t*>(cbs);
  a.stride = L.total;
  a.n_cb = n_cb;
  a.krec = krec;
  a.B = B; a.Hkv = Hkv; a.T = T; a.Hq = Hq;
  a.q = q; a.q_dtype = q_dtype;
  a.scale = scale;
  a.scores = scores;
  a.status = status;
  a.bits = L.bits; a.rec_words = L.rec_words; a.gq = (int)(Hq / Hkv);
  a.off_c = L.off_c; a.off_d = L.off_d; a.off_s = L.off_s;
  a.rotation = L.rotation;
  a.tiles = (T + 31) / 32;
  switch (L.k) {
    case 1: return launch_k<1>(a, s);
    case 2: return launch_k<2>(a, s);
    case 3: return launch_k<3>(a, s);
    default: return -13;
  }
}

}  // namespace tq
