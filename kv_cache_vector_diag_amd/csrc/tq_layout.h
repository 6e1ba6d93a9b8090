// Internal layout of codebook blobs and records, shared by the host core and
// the kernel launchers of libtq.  Public contract: include/tq.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace tq {

constexpr uint32_t kBlobMagic = 0x42435154u;  // "TQCB" little-endian
constexpr uint32_t kBlobVersion = 1;
constexpr int kMaxHeadDim = 512;
constexpr int kMaxProjections = 1024;
constexpr int kRotHadamard = 0;
constexpr int kRotHaar = 1;
// Seed of the outlier part of a split head vector: the head's seed XOR this
// (the 64-bit golden-ratio constant), so that the two parts draw independent
// D and S from one per-head seed.
constexpr uint64_t kOutlierSeedXor = 0x9E3779B97F4A7C15ull;

// 64-byte header at the start of every blob.
struct BlobHeader {
  uint32_t magic;
  uint32_t version;
  int32_t head_dim;
  int32_t bits;
  int32_t projections;
  int32_t role;
  int32_t k;        // Lloyd-Max bits: bits-1 for keys, bits for values
  int32_t levels;   // 2^k
  uint64_t seed;
  uint32_t off_c;   // float32 centroids [levels]
  uint32_t off_t;   // float32 thresholds [levels-1] (+ one +inf pad)
  uint32_t off_d;   // Walsh-Hadamard: uint32 sign bits [ceil(d/32)];
                    // Haar: float32 R = sqrt(d) Q [d][d], row-major
  uint32_t off_s;   // binary16 S [projections][head_dim] (keys), else 0
  uint32_t total_bytes;
  uint32_t rotation;  // kRotHadamard or kRotHaar
};
static_assert(sizeof(BlobHeader) == 64, "blob header is 64 bytes");

struct Layout {
  int d, bits, m, role, k, levels, rotation;
  uint32_t off_c, off_t, off_d, off_s, total;  // bytes
  int plane_words;   // W = ceil(d/32)
  int sign_words;    // keys: ceil(m/32), else 0
  int rec_words;     // k*W + sign_words + 1 (+1 for keys)
};

inline uint32_t align_up(uint32_t x, uint32_t a) { return (x + a - 1) / a * a; }

// Validates parameters; returns 0 or a negative tq_status code.  The
// Walsh-Hadamard rotation needs a power-of-two head_dim; the dense Haar
// rotation takes any head_dim in [2, 512].
inline int check_params(int d, int bits, int m, int role, int rotation = kRotHadamard) {
  if (role != 0 && role != 1) return -11;
  if (rotation != kRotHadamard && rotation != kRotHaar) return -14;
  if (d == 0) return -1;
  if (d < 2 || d > kMaxHeadDim) return -2;
  if (rotation == kRotHadamard && (d & (d - 1)) != 0) return -2;
  if (role == 0) {
    if (bits < 2 || bits > 9) return -3;
    if (m <= 0) return -4;
    if (m > kMaxProjections) return -12;
  } else {
    if (bits < 1 || bits > 8) return -3;
  }
  return 0;
}

inline int make_layout(int d, int bits, int m, int role, Layout* L, int rotation = kRotHadamard) {
  int rc = check_params(d, bits, m, role, rotation);
  if (rc) return rc;
  L->rotation = rotation;
  L->d = d;
  L->bits = bits;
  L->role = role;
  L->m = role == 0 ? m : 0;
  L->k = role == 0 ? bits - 1 : bits;
  L->levels = 1 << L->k;
  L->plane_words = (d + 31) / 32;
  L->sign_words = role == 0 ? (m + 31) / 32 : 0;
  L->rec_words = L->k * L->plane_words + L->sign_words + 1 + (role == 0 ? 1 : 0);
  uint32_t off = 64;
  L->off_c = off;
  off = align_up(off + 4u * L->levels, 16);
  L->off_t = off;
  off = align_up(off + 4u * L->levels, 16);
  L->off_d = off;
  off = align_up(off + (rotation == kRotHaar ? 4u * (uint32_t)d * (uint32_t)d : 4u * L->plane_words), 16);
  if (role == 0) {
    L->off_s = off;
    off = align_up(off + 2u * (uint32_t)L->m * (uint32_t)d, 16);
  } else {
    L->off_s = 0;
  }
  L->total = align_up(off, 256);
  return 0;
}

}  // namespace tq
