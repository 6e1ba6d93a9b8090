// Host core of libtq: quantizer state (Lloyd-Max codebook, seeded D and S),
// blob and record sizes, footprint.  No device code.
//
// Page "turboquant-plus-rs 0.1.0 README": "Modules" codebook (Lloyd-Max
// centroids of the post-rotation Gaussian, closed form at 1 bit), rotation
// (random sign diagonal + Walsh-Hadamard), qjl (Gaussian sign projection),
// utils (memory footprint).  Page "bitpolar 0.3.3 src/kv_cache.rs":
// KvCacheConfig (head_dim, bits, projections, seed) fully determines a
// quantizer.
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/tq.h"
#include "tq_layout.h"

namespace tq {
namespace {

// ---------------------------------------------------------------------------
// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014; finaliser of Vigna's public
// splitmix64.c).  Counter form: output i of the stream started at `seed`.
// ---------------------------------------------------------------------------
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kStreamS = 1ull << 32;
constexpr uint64_t kStreamHaar = 2ull << 32;

inline uint64_t splitmix64(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * kGamma;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Nearest binary16 to a double, ties to even (IEEE 754 binary16: 10 stored
// fraction bits, exponent bias 15, subnormal quantum 2^-24).
uint16_t double_to_half(double x) {
  uint64_t b;
  std::memcpy(&b, &x, 8);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int ex = (int)((b >> 52) & 0x7FF);
  const uint64_t frac = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return sign | 0x7C00u | (frac ? 0x200u : 0u);
  if (ex == 0) return sign;  // double subnormals are far below half's range
  int e = ex - 1023;         // |x| = 1.frac * 2^e
  if (e > 15) return sign | 0x7C00u;
  const uint64_t full = (1ull << 52) | frac;
  int shift;                 // right shift that leaves the half's significand
  int biased;
  if (e >= -14) {
    shift = 42;
    biased = e + 15;
  } else {
    shift = 42 + (-14 - e);  // subnormal: quantum 2^-24
    biased = 0;
    if (shift > 63) return sign;
  }
  uint64_t q = full >> shift;
  const uint64_t rem = full & ((1ull << shift) - 1);
  const uint64_t halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (q & 1))) q++;
  if (biased == 0) return sign | (uint16_t)q;  // q may reach 1024 = smallest normal
  // normal: q in [1024, 2048]
  if (q == 2048) {
    q = 1024;
    biased++;
  }
  if (biased >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)(biased << 10) | (uint16_t)(q - 1024);
}

// ---------------------------------------------------------------------------
// Lloyd-Max quantizer of N(0,1) with L = 2^k cells.  Fixed point of
//   t_i = (c_i + c_{i+1}) / 2,   c_i = (phi(t_{i-1}) - phi(t_i)) / (Phi(t_i) - Phi(t_{i-1})),
// reached by Lloyd steps from the quantile start until the largest move is
// below 1e-6, then Newton steps on the same equations (tridiagonal Jacobian).
// Iterates are kept exactly antisymmetric (the law is symmetric), so the
// middle threshold is exactly 0.
// ---------------------------------------------------------------------------
const double kInvSqrt2Pi = 0.3989422804014326779399460599343819;

double pdf(double x) { return std::isinf(x) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * x * x); }
double upper(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }  // 1 - Phi(x)
double mass(double a, double b) {                                     // Phi(b) - Phi(a)
  if (a >= 0.0) return upper(a) - upper(b);
  if (b <= 0.0) return upper(-b) - upper(-a);
  return 1.0 - upper(b) - upper(-a);
}

// Phi^{-1}(p) by bisection on the upper tail (start values only).
double inv_cdf(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    double mid = 0.5 * (lo + hi);
    if (1.0 - upper(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

void antisym(std::vector<double>& c) {
  const int L = (int)c.size();
  std::vector<double> r(L);
  for (int i = 0; i < L; ++i) r[i] = 0.5 * (c[i] - c[L - 1 - i]);
  c.swap(r);
}

struct Step {
  std::vector<double> g, a, b, w;  // new centroids, cell edges, cell mass
};

void lloyd_step(const std::vector<double>& c, Step* s) {
  const int L = (int)c.size();
  s->g.resize(L); s->a.resize(L); s->b.resize(L); s->w.resize(L);
  for (int i = 0; i < L; ++i) {
    double a = i == 0 ? -INFINITY : 0.5 * (c[i - 1] + c[i]);
    double b = i == L - 1 ? INFINITY : 0.5 * (c[i] + c[i + 1]);
    double w = mass(a, b);
    s->a[i] = a; s->b[i] = b; s->w[i] = w;
    s->g[i] = (pdf(a) - pdf(b)) / w;
  }
}

void lloyd_max(int k, std::vector<double>* cent, std::vector<double>* thr) {
  const int L = 1 << k;
  std::vector<double> c(L);
  if (L == 1) {
    cent->assign(1, 0.0);
    thr->clear();
    return;
  }
  for (int i = 0; i < L; ++i) c[i] = inv_cdf((i + 0.5) / L);
  antisym(c);
  Step s;
  for (int it = 0; it < 1000000; ++it) {
    lloyd_step(c, &s);
    std::vector<double> n = s.g;
    antisym(n);
    double move = 0.0;
    for (int i = 0; i < L; ++i) move = std::fmax(move, std::fabs(n[i] - c[i]));
    c.swap(n);
    if (move < 1e-6) break;
  }
  std::vector<double> best = c;
  double best_res = INFINITY;
  std::vector<double> lo(L), di(L), up(L), rhs(L);
  for (int it = 0; it < 40; ++it) {
    lloyd_step(c, &s);
    double res = 0.0;
    for (int i = 0; i < L; ++i) res = std::fmax(res, std::fabs(s.g[i] - c[i]));
    if (res < best_res) { best = c; best_res = res; }
    if (res == 0.0) break;
    // Jacobian of (g - c): d g_i / d(edge) from the conditional-mean formula.
    for (int i = 0; i < L; ++i) {
      double fa = std::isinf(s.a[i]) ? 0.0 : s.a[i];
      double fb = std::isinf(s.b[i]) ? 0.0 : s.b[i];
      double dlo = pdf(s.a[i]) * (s.g[i] - fa) / s.w[i];
      double dhi = pdf(s.b[i]) * (fb - s.g[i]) / s.w[i];
      di[i] = 0.5 * (dlo + dhi) - 1.0;
      lo[i] = 0.5 * dlo;   // coefficient of c_{i-1}
      up[i] = 0.5 * dhi;   // coefficient of c_{i+1}
      rhs[i] = -(s.g[i] - c[i]);
    }
    // Thomas algorithm
    for (int i = 1; i < L; ++i) {
      double f = lo[i] / di[i - 1];
      di[i] -= f * up[i - 1];
      rhs[i] -= f * rhs[i - 1];
    }
    std::vector<double> x(L);
    x[L - 1] = rhs[L - 1] / di[L - 1];
    for (int i = L - 2; i >= 0; --i) x[i] = (rhs[i] - up[i] * x[i + 1]) / di[i];
    for (int i = 0; i < L; ++i) c[i] += x[i];
    antisym(c);
  }
  *cent = best;
  thr->resize(L - 1);
  for (int i = 0; i < L - 1; ++i) (*thr)[i] = 0.5 * (best[i] + best[i + 1]);
}

// Standard normals from stream `base`: entry e is the cos (even e) or sin (odd
// e) member of the Box-Muller pair on outputs base + 2*(e/2) and base + 2*(e/2) + 1,
// u1 = ((x1 >> 11) + 1) 2^-53 in (0, 1], u2 = (x2 >> 11) 2^-53, in float64.
void gaussians(uint64_t seed, uint64_t base, uint64_t count, double* out) {
  const double two_pi = 6.283185307179586476925286766559;
  const double two_m53 = 1.0 / 9007199254740992.0;
  for (uint64_t e = 0; e < count; e += 2) {
    uint64_t x1 = splitmix64(seed, base + e);
    uint64_t x2 = splitmix64(seed, base + e + 1);
    double u1 = (double)((x1 >> 11) + 1) * two_m53;
    double u2 = (double)(x2 >> 11) * two_m53;
    double r = std::sqrt(-2.0 * std::log(u1));
    double ang = two_pi * u2;
    out[e] = r * std::cos(ang);
    if (e + 1 < count) out[e + 1] = r * std::sin(ang);
  }
}

// Haar-distributed rotation (README "Modules" rotation: Haar via QR).  G is
// the d x d Gaussian matrix of the Haar stream (row-major); its QR
// factorisation by Householder reflections gives Q, whose columns are then
// signed so that the triangular factor has a positive diagonal (the unique
// factor with that property, Haar-distributed for Gaussian G).  Output
// R = float32(sqrt(d) Q), row-major.
void haar_rotation(uint64_t seed, int d, float* R) {
  const size_t n = (size_t)d;
  std::vector<double> A(n * n), Q(n * n, 0.0), V(n * n, 0.0), diag(n);
  gaussians(seed, kStreamHaar, (uint64_t)n * n, A.data());
  for (size_t k = 0; k < n; ++k) {
    // reflector v (unit) with (I - 2 v v^T) A[k:, k] = alpha e_k
    double nrm = 0.0;
    for (size_t i = k; i < n; ++i) nrm += A[i * n + k] * A[i * n + k];
    nrm = std::sqrt(nrm);
    const double x0 = A[k * n + k];
    const double alpha = x0 >= 0.0 ? -nrm : nrm;
    double* v = &V[k * n];
    for (size_t i = k; i < n; ++i) v[i] = A[i * n + k];
    v[k] -= alpha;
    double vn = 0.0;
    for (size_t i = k; i < n; ++i) vn += v[i] * v[i];
    vn = std::sqrt(vn);
    if (vn > 0.0)
      for (size_t i = k; i < n; ++i) v[i] /= vn;
    for (size_t j = k; j < n; ++j) {
      double dot = 0.0;
      for (size_t i = k; i < n; ++i) dot += v[i] * A[i * n + j];
      for (size_t i = k; i < n; ++i) A[i * n + j] -= 2.0 * v[i] * dot;
    }
    diag[k] = A[k * n + k];
  }
  // Q = H_0 H_1 ... H_{n-1}: apply the reflectors to I from the last one
  for (size_t i = 0; i < n; ++i) Q[i * n + i] = 1.0;
  for (size_t kk = n; kk-- > 0;) {
    const double* v = &V[kk * n];
    for (size_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (size_t i = kk; i < n; ++i) dot += v[i] * Q[i * n + j];
      for (size_t i = kk; i < n; ++i) Q[i * n + j] -= 2.0 * v[i] * dot;
    }
  }
  const double sd = std::sqrt((double)d);
  for (size_t i = 0; i < n; ++i)
    for (size_t j = 0; j < n; ++j) R[i * n + j] = (float)(sd * (diag[j] < 0.0 ? -Q[i * n + j] : Q[i * n + j]));
}

int make_codebook(int head_dim, int bits, int projections, uint64_t seed, int role, int rotation, void* blob,
                  size_t blob_bytes);

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" {

size_t tq_codebook_bytes(int head_dim, int bits, int projections, int role) {
  return tq_codebook_bytes_ex(head_dim, bits, projections, role, TQ_ROT_HADAMARD);
}

size_t tq_codebook_bytes_ex(int head_dim, int bits, int projections, int role, int rotation) {
  Layout L;
  if (make_layout(head_dim, bits, projections, role, &L, rotation)) return 0;
  return L.total;
}

size_t tq_record_bytes(int head_dim, int bits, int projections, int role) {
  return tq_record_bytes_ex(head_dim, bits, projections, role, TQ_ROT_HADAMARD);
}

size_t tq_record_bytes_ex(int head_dim, int bits, int projections, int role, int rotation) {
  Layout L;
  if (make_layout(head_dim, bits, projections, role, &L, rotation)) return 0;
  return 4u * (size_t)L.rec_words;
}

int tq_make_codebook(int head_dim, int bits, int projections, uint64_t seed, int role,
                     void* blob, size_t blob_bytes) {
  return make_codebook(head_dim, bits, projections, seed, role, TQ_ROT_HADAMARD, blob, blob_bytes);
}

int tq_make_codebook_ex(int head_dim, int bits, int projections, uint64_t seed, int role, int rotation,
                        void* blob, size_t blob_bytes) {
  return make_codebook(head_dim, bits, projections, seed, role, rotation, blob, blob_bytes);
}

// The two parts of a split head vector: normal part of head_dim - n_outlier
// channels (Haar, bits), outlier part of n_outlier channels (Walsh-Hadamard,
// bits + 1); keys project each part onto as many signs as it has coordinates.
static int split_part(int role, int head_dim, int n_outlier, int bits, int part, int* d, int* b, int* m, int* rot) {
  if (role != TQ_ROLE_KEY && role != TQ_ROLE_VALUE) return TQ_ERR_INVALID_ROLE;
  if (head_dim == 0) return TQ_ERR_ZERO_DIMENSION;
  if (head_dim < 2 || head_dim > kMaxHeadDim) return TQ_ERR_BAD_DIMENSION;
  if (n_outlier <= 0 || n_outlier >= head_dim || (part != 0 && part != 1)) return TQ_ERR_DIMENSION_MISMATCH;
  *d = part == 0 ? head_dim - n_outlier : n_outlier;
  *b = part == 0 ? bits : bits + 1;
  *m = role == TQ_ROLE_KEY ? *d : 0;
  *rot = part == 0 ? TQ_ROT_HAAR : TQ_ROT_HADAMARD;
  return TQ_OK;
}

size_t tq_split_codebook_bytes(int role, int head_dim, int n_outlier, int bits, int part) {
  int d, b, m, rot;
  if (split_part(role, head_dim, n_outlier, bits, part, &d, &b, &m, &rot)) return 0;
  return tq_codebook_bytes_ex(d, b, m, role, rot);
}

int tq_make_split_codebooks(int role, int head_dim, int n_outlier, int bits, uint64_t seed, void* normal_blob,
                            size_t normal_bytes, void* outlier_blob, size_t outlier_bytes) {
  int d, b, m, rot;
  int rc = split_part(role, head_dim, n_outlier, bits, 0, &d, &b, &m, &rot);
  if (rc) return rc;
  rc = make_codebook(d, b, m, seed, role, rot, normal_blob, normal_bytes);
  if (rc) return rc;
  split_part(role, head_dim, n_outlier, bits, 1, &d, &b, &m, &rot);
  return make_codebook(d, b, m, seed ^ kOutlierSeedXor, role, rot, outlier_blob, outlier_bytes);
}

}  // extern "C"

namespace tq {
namespace {

int make_codebook(int head_dim, int bits, int projections, uint64_t seed, int role, int rotation, void* blob,
                  size_t blob_bytes) {
  Layout L;
  int rc = make_layout(head_dim, bits, projections, role, &L, rotation);
  if (rc) return rc;
  if (!blob) return TQ_ERR_NULL;
  if (blob_bytes < L.total) return TQ_ERR_BAD_BLOB;
  uint8_t* p = static_cast<uint8_t*>(blob);
  std::memset(p, 0, L.total);

  BlobHeader h{};
  h.magic = kBlobMagic;
  h.version = kBlobVersion;
  h.head_dim = head_dim;
  h.bits = bits;
  h.projections = L.m;
  h.role = role;
  h.k = L.k;
  h.levels = L.levels;
  h.seed = seed;
  h.off_c = L.off_c;
  h.off_t = L.off_t;
  h.off_d = L.off_d;
  h.off_s = L.off_s;
  h.total_bytes = L.total;
  h.rotation = (uint32_t)rotation;
  std::memcpy(p, &h, sizeof h);

  std::vector<double> c, t;
  lloyd_max(L.k, &c, &t);
  float* cf = reinterpret_cast<float*>(p + L.off_c);
  float* tf = reinterpret_cast<float*>(p + L.off_t);
  for (int i = 0; i < L.levels; ++i) cf[i] = (float)c[i];
  for (int i = 0; i < L.levels - 1; ++i) tf[i] = (float)t[i];
  tf[L.levels - 1] = INFINITY;

  if (rotation == TQ_ROT_HAAR) {
    haar_rotation(seed, head_dim, reinterpret_cast<float*>(p + L.off_d));
  } else {
    uint32_t* dw = reinterpret_cast<uint32_t*>(p + L.off_d);
    for (int j = 0; j < head_dim; ++j) {
      uint64_t word = splitmix64(seed, (uint64_t)(j / 64));
      if ((word >> (j % 64)) & 1) dw[j / 32] |= 1u << (j % 32);
    }
  }

  if (role == TQ_ROLE_KEY) {
    uint16_t* s = reinterpret_cast<uint16_t*>(p + L.off_s);
    const uint64_t count = (uint64_t)L.m * (uint64_t)head_dim;
    std::vector<double> g(count);
    gaussians(seed, kStreamS, count, g.data());
    for (uint64_t e = 0; e < count; ++e) s[e] = double_to_half(g[e]);
  }
  return TQ_OK;
}

}  // namespace
}  // namespace tq

extern "C" {

int tq_memory_stats(int head_dim, int k_bits, int v_bits, int projections, int64_t seq_len,
                    int64_t layers, int64_t kv_heads, double out[4]) {
  if (!out) return TQ_ERR_NULL;
  Layout K, V;
  int rc = make_layout(head_dim, k_bits, projections, TQ_ROLE_KEY, &K);
  if (rc) return rc;
  rc = make_layout(head_dim, v_bits, projections, TQ_ROLE_VALUE, &V);
  if (rc) return rc;
  if (seq_len < 0 || layers < 0 || kv_heads < 0) return TQ_ERR_EMPTY_INPUT;
  const double vecs = (double)seq_len * (double)layers * (double)kv_heads;
  out[0] = 2.0 * vecs * head_dim * 2.0;
  out[1] = 2.0 * vecs * head_dim * 4.0;
  out[2] = vecs * 4.0 * (K.rec_words + V.rec_words);
  out[3] = out[2] > 0 ? out[0] / out[2] : 1.0;
  return TQ_OK;
}

const char* tq_status_string(int code) {
  switch (code) {
    case TQ_OK: return "ok";
    case TQ_ERR_ZERO_DIMENSION: return "ZeroDimension: head_dim is 0";
    case TQ_ERR_BAD_DIMENSION: return "BadDimension: head_dim must be in [2, 512] (a power of two for Walsh-Hadamard)";
    case TQ_ERR_INVALID_BIT_WIDTH: return "InvalidBitWidth: keys need bits in [2, 9], values in [1, 8]";
    case TQ_ERR_ZERO_PROJECTIONS: return "ZeroProjections: keys need projections >= 1";
    case TQ_ERR_DIMENSION_MISMATCH: return "DimensionMismatch: sizes or strides are inconsistent";
    case TQ_ERR_NON_FINITE_INPUT: return "NonFiniteInput";
    case TQ_ERR_EMPTY_INPUT: return "EmptyInput: n_cb must be > 0 and sizes >= 0";
    case TQ_ERR_NULL: return "Null: a required pointer is NULL";
    case TQ_ERR_BAD_BLOB: return "BadBlob: blob buffer too small";
    case TQ_ERR_HIP: return "HIP launch failed";
    case TQ_ERR_INVALID_ROLE: return "InvalidRole";
    case TQ_ERR_INVALID_PROJECTIONS: return "InvalidProjections: projections must be <= 1024";
    case TQ_ERR_UNSUPPORTED: return "Unsupported dtype or alignment";
    case TQ_ERR_INVALID_ROTATION: return "InvalidRotation: rotation must be TQ_ROT_HADAMARD or TQ_ROT_HAAR";
    case TQ_ERR_INVALID_CODEBOOK: return "InvalidCodebook: codebook size must be a power of two in [2, 256]";
    case TQ_ERR_SCRATCH_LIMIT: return "ScratchLimit: the call needs more than the 32 MiB static scratch of tq_attend_static";
    default: return "unknown status";
  }
}

}  // extern "C"
