// Generic libtq kernels: any power-of-two head_dim in [2, 512], any bit width,
// any number of projections.  One wave (64 lanes, one workgroup) per vector,
// the Walsh-Hadamard transform done in LDS stage by stage.  These kernels
// define the device semantics that the specialised head_dim-128 kernels
// reproduce bit for bit on codes and signs.
//
// Method: page "turboquant-plus-rs 0.1.0 README", "Architecture" (PolarQuant
// b-1 bits + QJL 1 bit for keys, MSE-only for values) and "Modules"
// (rotation, codebook, polar_quant, qjl); page "bitpolar 0.3.3
// src/kv_cache.rs" (push, attention_scores, decode_values).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kWave = 64;
constexpr int kMaxWords = 8 * 16 + 32 + 2;  // planes (k<=8, W<=16) + signs (m<=1024) + n, gamma

struct EncodeArgs {
  CodebookArgs cb;
  const void* x;
  int dtype;
  int64_t G, N, sx_g, sx_n;
  uint32_t* rec;
  int32_t* status;
  ChannelMap cm;
};

// Encode one vector per workgroup (64 lanes).  Steps, in the README's order:
// norm; u = H(D x) (rotation without the 1/sqrt(d), so z = u/|x| ~ N(0,1)),
// or u = R x with the stored dense Haar matrix R = sqrt(d) Q;
// idx_j = #{t_i < z_j}; keys only: residual w = u - n32 c[idx] (sqrt(d) times
// the rotated residual), gamma = |w|/sqrt(d), signs of S w.
// This kernel works in float64 (full rate on CDNA4): the rotation of
// float32/bf16/f16 inputs is then exact to ~1e-16, the quantizer decision is
// taken on float32(u/|x|), and the QJL signs stay exact even for 7-8 bit
// codebooks whose residual is ~1% of the vector.
__global__ __launch_bounds__(64) void encode_generic_kernel(EncodeArgs a) {
  __shared__ double u[kMaxHeadDim];
  __shared__ double w[kMaxHeadDim];
  __shared__ int idx[kMaxHeadDim];
  __shared__ uint32_t words[kMaxWords];
  __shared__ float cent[256];
  __shared__ float thr[256];
  const int lane = threadIdx.x;
  const int d = a.cb.d;
  const int64_t total = a.G * a.N;
  int64_t g_loaded = -1;
  for (int64_t v = blockIdx.x; v < total; v += gridDim.x) {
    const int64_t g = v / a.N, t = v % a.N;
    const uint8_t* blob = blob_of(a.cb, g);
    if (lane == 0 && a.status && blob_mismatch(a.cb, blob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
    if (g % a.cb.n_cb != g_loaded) {
      // centroids and thresholds in LDS: the quantizer's binary search then
      // costs LDS latency, not a chain of dependent global loads
      for (int i = lane; i < a.cb.levels; i += kWave) {
        cent[i] = reinterpret_cast<const float*>(blob + a.cb.off_c)[i];
        thr[i] = reinterpret_cast<const float*>(blob + a.cb.off_t)[i];
      }
      g_loaded = g % a.cb.n_cb;
    }
    const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d);
    const int64_t base = g * a.sx_g + t * a.sx_n;

    const bool haar = a.cb.rotation == kRotHaar;
    double ss = 0.0;
    for (int j = lane; j < d; j += kWave) {
      double xv = (double)load_elem(a.x, a.dtype, base + a.cm.channel(g, j, a.status));
      ss += xv * xv;
      if (haar) w[j] = xv;
      else u[j] = ((dbits[j >> 5] >> (j & 31)) & 1u) ? -xv : xv;
    }
    ss = wave_sum_f64(ss);
    const bool finite = ss <= 3.4028234663852886e38;
    if (lane == 0 && a.status && !finite) atomicOr(a.status, TQ_STATUS_NON_FINITE);
    __syncthreads();
    if (haar) {
      // u_j = sum_i R[j][i] x_i: float32 R times float32/bf16/f16 x is exact in float64
      const float* R = reinterpret_cast<const float*>(blob + a.cb.off_d);
      for (int j = lane; j < d; j += kWave) {
        const float* row = R + (int64_t)j * d;
        double acc = 0.0;
        if ((d & 3) == 0) {
          // 16-byte row reads; four independent partial sums (not one chain of
          // dependent FMAs)
          double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
          for (int i = 0; i < d; i += 4) {
            const float4 r4 = *reinterpret_cast<const float4*>(row + i);
            a0 = fma((double)r4.x, w[i], a0);
            a1 = fma((double)r4.y, w[i + 1], a1);
            a2 = fma((double)r4.z, w[i + 2], a2);
            a3 = fma((double)r4.w, w[i + 3], a3);
          }
          acc = (a0 + a1) + (a2 + a3);
        } else {
          for (int i = 0; i < d; ++i) acc = fma((double)row[i], w[i], acc);
        }
        u[j] = acc;
      }
      __syncthreads();
    } else {
      for (int h = 1; h < d; h <<= 1) {
        for (int p = lane; p < d / 2; p += kWave) {
          int i = (p / h) * 2 * h + (p % h);
          double x0 = u[i], x1 = u[i + h];
          u[i] = x0 + x1;
          u[i + h] = x0 - x1;
        }
        __syncthreads();
      }
    }
    const double nrm = sqrt(ss);
    const float n32 = (float)nrm;
    double ws = 0.0;
    for (int j = lane; j < d; j += kWave) {
      double uj = u[j];
      const float z = z_up(uj, nrm);
      int q = quantize_index(thr, a.cb.levels, z);
      idx[j] = q;
      if (a.cb.role == TQ_ROLE_KEY) {
        double r = uj - (double)n32 * (double)cent[q];
        w[j] = r;
        ws += r * r;
      }
    }
    __syncthreads();
    // bit planes: 64 coordinates per ballot -> two words
    const int W = a.cb.plane_words;
    for (int p = 0; p < a.cb.k; ++p) {
      for (int j0 = 0; j0 < d; j0 += kWave) {
        int j = j0 + lane;
        uint64_t b = __ballot(j < d && ((idx[j < d ? j : 0] >> p) & 1));
        if (lane == 0) {
          words[p * W + j0 / 32] = (uint32_t)b;
          if (j0 / 32 + 1 < W) words[p * W + j0 / 32 + 1] = (uint32_t)(b >> 32);
        }
      }
    }
    int off = a.cb.k * W;
    if (a.cb.role == TQ_ROLE_KEY) {
      const _Float16* S = reinterpret_cast<const _Float16*>(blob + a.cb.off_s);
      const int m = a.cb.m;
      for (int i0 = 0; i0 < m; i0 += kWave) {
        int i = i0 + lane;
        double acc = 0.0;
        if (i < m) {
          const _Float16* row = S + (int64_t)i * d;
          if ((d & 7) == 0) {
            // 16-byte row reads; four independent partial sums
            double pa[4] = {0.0, 0.0, 0.0, 0.0};
            for (int j = 0; j < d; j += 8) {
              const uint4 q4 = *reinterpret_cast<const uint4*>(row + j);
              const uint32_t qw[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(qw[e] & 0xFFFFu));
                const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(qw[e] >> 16));
                pa[e] = fma((double)lo, w[j + 2 * e], pa[e]);
                pa[e] = fma((double)hi, w[j + 2 * e + 1], pa[e]);
              }
            }
            acc = (pa[0] + pa[1]) + (pa[2] + pa[3]);
          } else {
            for (int j = 0; j < d; ++j) acc = fma((double)row[j], w[j], acc);
          }
        }
        uint64_t b = __ballot(i < m && acc >= 0.0);
        if (lane == 0) {
          words[off + i0 / 32] = (uint32_t)b;
          if (i0 / 32 + 1 < a.cb.sign_words) words[off + i0 / 32 + 1] = (uint32_t)(b >> 32);
        }
      }
      off += a.cb.sign_words;
      ws = wave_sum_f64(ws);
      if (lane == 0) {
        words[off] = __float_as_uint(n32);
        words[off + 1] = __float_as_uint((float)(sqrt(ws) / sqrt((double)d)));
      }
    } else if (lane == 0) {
      words[off] = __float_as_uint(n32);
    }
    __syncthreads();
    uint32_t* out = a.rec + v * a.cb.rec_words;
    for (int i = lane; i < a.cb.rec_words; i += kWave) out[i] = words[i];
    __syncthreads();
  }
}

struct DecodeArgs {
  CodebookArgs cb;
  const uint32_t* rec;
  int64_t G, N;
  float* out;
  int32_t* status;
  int64_t out_stride;   // floats between output rows
  ChannelMap cm;        // output channel of coordinate j (scatter)
};

// x^ = (n32/d) D (H c[idx]) per vector; Haar: x^ = (n32/d) R^T c[idx].
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeArgs a) {
  __shared__ float u[kMaxHeadDim];
  const int lane = threadIdx.x;
  const int d = a.cb.d, W = a.cb.plane_words;
  const int64_t total = a.G * a.N;
  for (int64_t v = blockIdx.x; v < total; v += gridDim.x) {
    const int64_t g = v / a.N;
    const uint8_t* blob = blob_of(a.cb, g);
    if (lane == 0 && a.status && blob_mismatch(a.cb, blob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
    const float* cent = reinterpret_cast<const float*>(blob + a.cb.off_c);
    const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d);
    const uint32_t* r = a.rec + v * a.cb.rec_words;
    for (int j = lane; j < d; j += kWave) {
      int q = 0;
      for (int p = 0; p < a.cb.k; ++p) q |= ((r[p * W + (j >> 5)] >> (j & 31)) & 1u) << p;
      u[j] = cent[q];
    }
    __syncthreads();
    const float scale = __uint_as_float(r[a.cb.k * W]) / (float)d;
    float* o = a.out + v * a.out_stride;
    if (a.cb.rotation == kRotHaar) {
      const float* R = reinterpret_cast<const float*>(blob + a.cb.off_d);
      for (int i = lane; i < d; i += kWave) {
        float acc = 0.0f;
        for (int j = 0; j < d; ++j) acc = fmaf(R[(int64_t)j * d + i], u[j], acc);
        o[a.cm.channel(g, i, a.status)] = acc * scale;
      }
    } else {
      for (int h = 1; h < d; h <<= 1) {
        for (int p = lane; p < d / 2; p += kWave) {
          int i = (p / h) * 2 * h + (p % h);
          float x0 = u[i], x1 = u[i + h];
          u[i] = x0 + x1;
          u[i + h] = x0 - x1;
        }
        __syncthreads();
      }
      for (int j = lane; j < d; j += kWave) {
        float val = u[j] * scale;
        o[a.cm.channel(g, j, a.status)] = ((dbits[j >> 5] >> (j & 31)) & 1u) ? -val : val;
      }
    }
    __syncthreads();
  }
}

struct RotateArgs {
  CodebookArgs cb;
  const void* x;
  int dtype;
  int64_t G, N, sx_g, sx_n;
  float* u;
  float* norms;
};

__global__ __launch_bounds__(64) void rotate_generic_kernel(RotateArgs a) {
  __shared__ double u[kMaxHeadDim];
  const int lane = threadIdx.x;
  const int d = a.cb.d;
  const int64_t total = a.G * a.N;
  for (int64_t v = blockIdx.x; v < total; v += gridDim.x) {
    const int64_t g = v / a.N, t = v % a.N;
    const uint8_t* blob = blob_of(a.cb, g);
    const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d);
    const int64_t base = g * a.sx_g + t * a.sx_n;
    double ss = 0.0;
    for (int j = lane; j < d; j += kWave) {
      double xv = (double)load_elem(a.x, a.dtype, base + j);
      ss += xv * xv;
      u[j] = ((dbits[j >> 5] >> (j & 31)) & 1u) ? -xv : xv;
    }
    ss = wave_sum_f64(ss);
    __syncthreads();
    for (int h = 1; h < d; h <<= 1) {
      for (int p = lane; p < d / 2; p += kWave) {
        int i = (p / h) * 2 * h + (p % h);
        double x0 = u[i], x1 = u[i + h];
        u[i] = x0 + x1;
        u[i + h] = x0 - x1;
      }
      __syncthreads();
    }
    for (int j = lane; j < d; j += kWave) a.u[v * d + j] = (float)u[j];
    if (lane == 0) a.norms[v] = (float)sqrt(ss);
    __syncthreads();
  }
}

struct ScoreArgs {
  CodebookArgs cb;
  const uint32_t* krec;
  int64_t B, Hkv, T;
  const void* q;
  int q_dtype;
  int64_t Hq;
  float scale;
  float* scores;
  int32_t* status;
  int64_t q_row;        // elements between query rows
  ChannelMap cm;        // query channel of coordinate j (gather)
  int accumulate;       // add into scores instead of overwriting
};

constexpr int kScoreBlock = 256;

// One workgroup per (b, hq, chunk of 256 tokens).  Prologue: qt = H(D q) (Haar:
// qt = R q) in LDS, p = S qt / sqrt(d); then one token per thread:
//   s = scale * ((n/d) sum_j qt_j c[idx_j] + sqrt(pi/2)/m gamma sum_i p_i (2 s_i - 1)).
__global__ __launch_bounds__(kScoreBlock) void scores_generic_kernel(ScoreArgs a) {
  __shared__ float qt[kMaxHeadDim];
  __shared__ float qraw[kMaxHeadDim];
  __shared__ float p[kMaxProjections];
  __shared__ float cent_s[256];
  const int tid = threadIdx.x;
  const int d = a.cb.d, m = a.cb.m, W = a.cb.plane_words;
  const int64_t chunks = (a.T + kScoreBlock - 1) / kScoreBlock;
  const int64_t bh = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x % chunks;
  const int64_t b = bh / a.Hq, hq = bh % a.Hq;
  const int64_t h = hq * a.Hkv / a.Hq;
  const int64_t g = b * a.Hkv + h;
  const uint8_t* blob = blob_of(a.cb, g);
  if (tid == 0 && a.status && blob_mismatch(a.cb, blob)) atomicOr(a.status, TQ_STATUS_BAD_BLOB);
  const float* cent = reinterpret_cast<const float*>(blob + a.cb.off_c);
  const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.cb.off_d);
  const _Float16* S = reinterpret_cast<const _Float16*>(blob + a.cb.off_s);
  for (int i = tid; i < a.cb.levels; i += kScoreBlock) cent_s[i] = cent[i];
  const bool haar = a.cb.rotation == kRotHaar;
  for (int j = tid; j < d; j += kScoreBlock) {
    float qv = load_elem(a.q, a.q_dtype, (b * a.Hq + hq) * a.q_row + a.cm.channel(g, j, a.status));
    if (haar) qraw[j] = qv;
    else qt[j] = ((dbits[j >> 5] >> (j & 31)) & 1u) ? -qv : qv;
  }
  __syncthreads();
  if (haar) {
    const float* R = reinterpret_cast<const float*>(blob + a.cb.off_d);
    for (int j = tid; j < d; j += kScoreBlock) {
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) acc = fmaf(R[(int64_t)j * d + i], qraw[i], acc);
      qt[j] = acc;
    }
    __syncthreads();
  } else {
    for (int hh = 1; hh < d; hh <<= 1) {
      for (int pp = tid; pp < d / 2; pp += kScoreBlock) {
        int i = (pp / hh) * 2 * hh + (pp % hh);
        float x0 = qt[i], x1 = qt[i + hh];
        qt[i] = x0 + x1;
        qt[i + hh] = x0 - x1;
      }
      __syncthreads();
    }
  }
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  for (int i = tid; i < m; i += kScoreBlock) {
    float acc = 0.0f;
    const _Float16* row = S + (int64_t)i * d;
    for (int j = 0; j < d; ++j) acc = fmaf((float)row[j], qt[j], acc);
    p[i] = acc * inv_sqrt_d;
  }
  __syncthreads();
  const int64_t t = chunk * kScoreBlock + tid;
  if (t >= a.T) return;
  const uint32_t* r = a.krec + (g * a.T + t) * a.cb.rec_words;
  float mse = 0.0f;
  for (int j = 0; j < d; ++j) {
    int q = 0;
    for (int pl = 0; pl < a.cb.k; ++pl) q |= ((r[pl * W + (j >> 5)] >> (j & 31)) & 1u) << pl;
    mse = fmaf(qt[j], cent_s[q], mse);
  }
  const int off = a.cb.k * W;
  float qjl = 0.0f;
  for (int i = 0; i < m; ++i) {
    float pi = p[i];
    qjl += ((r[off + (i >> 5)] >> (i & 31)) & 1u) ? pi : -pi;
  }
  const float n = __uint_as_float(r[off + a.cb.sign_words]);
  const float gam = __uint_as_float(r[off + a.cb.sign_words + 1]);
  const float s = (n / (float)d) * mse + (kQjlConst / (float)m) * gam * qjl;
  float* o = a.scores + (b * a.Hq + hq) * a.T + t;
  *o = a.accumulate ? *o + a.scale * s : a.scale * s;
}

struct AttendArgs {
  CodebookArgs vcb;
  const uint32_t* vrec;
  const float* scores;   // [B][Hq][T]
  int64_t B, Hkv, T, Hq;
  float* out;            // [B][Hq][d]
};

constexpr int kAttendBlock = 256;

// o = sum_t softmax(s)_t x^_t with x^_t = (n_t/d) D H c[idx_t]: accumulate
// a_j = sum_t e_t n_t c[idx_tj] in the rotated domain, then one transform:
// o = D H a / (d sum_t e_t).
__global__ __launch_bounds__(kAttendBlock) void attend_generic_kernel(AttendArgs a) {
  __shared__ float acc[kMaxHeadDim];
  __shared__ float red[kAttendBlock / 64];
  __shared__ float cent_s[256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int d = a.vcb.d, W = a.vcb.plane_words;
  const int64_t b = blockIdx.x / a.Hq, hq = blockIdx.x % a.Hq;
  const int64_t h = hq * a.Hkv / a.Hq;
  const int64_t g = b * a.Hkv + h;
  const uint8_t* blob = blob_of(a.vcb, g);
  const float* cent = reinterpret_cast<const float*>(blob + a.vcb.off_c);
  const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob + a.vcb.off_d);
  for (int i = tid; i < a.vcb.levels; i += kAttendBlock) cent_s[i] = cent[i];
  const float* s = a.scores + (b * a.Hq + hq) * a.T;
  float mx = -INFINITY;
  for (int64_t t = tid; t < a.T; t += kAttendBlock) mx = fmaxf(mx, s[t]);
  mx = wave_max_f32(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = red[0];
  for (int i = 1; i < kAttendBlock / 64; ++i) mx = fmaxf(mx, red[i]);
  __syncthreads();
  float esum = 0.0f;
  for (int64_t t = tid; t < a.T; t += kAttendBlock) esum += expf(s[t] - mx);
  esum = wave_sum_f32(esum);
  if (lane == 0) red[wv] = esum;
  __syncthreads();
  esum = 0.0f;
  for (int i = 0; i < kAttendBlock / 64; ++i) esum += red[i];
  for (int j = tid; j < d; j += kAttendBlock) {
    float aj = 0.0f;
    for (int64_t t = 0; t < a.T; ++t) {
      const uint32_t* r = a.vrec + (g * a.T + t) * a.vcb.rec_words;
      int q = 0;
      for (int pl = 0; pl < a.vcb.k; ++pl) q |= ((r[pl * W + (j >> 5)] >> (j & 31)) & 1u) << pl;
      float n = __uint_as_float(r[a.vcb.k * W]);
      aj = fmaf(expf(s[t] - mx) * n, cent_s[q], aj);
    }
    acc[j] = aj;
  }
  __syncthreads();
  const float norm = esum > 0.0f ? 1.0f / ((float)d * esum) : 0.0f;  // T == 0 gives 0
  if (a.vcb.rotation == kRotHaar) {
    // x^ = (n/d) R^T c: o_j = sum_i R[i][j] acc_i / (d esum), R row-major at off_d
    const float* R = reinterpret_cast<const float*>(blob + a.vcb.off_d);
    for (int j = tid; j < d; j += kAttendBlock) {
      float o = 0.0f;
      for (int i = 0; i < d; ++i) o = fmaf(R[i * d + j], acc[i], o);
      a.out[(b * a.Hq + hq) * d + j] = o * norm;
    }
    return;
  }
  for (int hh = 1; hh < d; hh <<= 1) {
    for (int pp = tid; pp < d / 2; pp += kAttendBlock) {
      int i = (pp / hh) * 2 * hh + (pp % hh);
      float x0 = acc[i], x1 = acc[i + hh];
      acc[i] = x0 + x1;
      acc[i + hh] = x0 - x1;
    }
    __syncthreads();
  }
  for (int j = tid; j < d; j += kAttendBlock) {
    float v = acc[j] * norm;
    a.out[(b * a.Hq + hq) * d + j] = ((dbits[j >> 5] >> (j & 31)) & 1u) ? -v : v;
  }
}

inline int grid_for(int64_t items, int64_t cap) { return (int)(items < cap ? (items > 0 ? items : 1) : cap); }

}  // namespace

int launch_encode_generic(const CodebookArgs& cb, const void* x, int dtype, int64_t G, int64_t N,
                          int64_t sx_g, int64_t sx_n, uint32_t* rec, int32_t* status, hipStream_t s,
                          const ChannelMap& cm) {
  if (G * N == 0) return 0;
  EncodeArgs a{cb, x, dtype, G, N, sx_g, sx_n, rec, status, cm};
  hipLaunchKernelGGL(encode_generic_kernel, dim3(grid_for(G * N, 1 << 16)), dim3(64), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

int launch_decode_generic(const CodebookArgs& cb, const uint32_t* rec, int64_t G, int64_t N, float* out,
                          int32_t* status, hipStream_t s, int64_t out_stride, const ChannelMap& cm) {
  if (G * N == 0) return 0;
  if (haar_decode_mfma_supported(cb, cm.map != nullptr))
    return launch_decode_haar_mfma(cb, rec, G, N, out, status, s, out_stride, cm);
  DecodeArgs a{cb, rec, G, N, out, status, out_stride > 0 ? out_stride : cb.d, cm};
  hipLaunchKernelGGL(decode_generic_kernel, dim3(grid_for(G * N, 1 << 16)), dim3(64), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

int launch_rotate_generic(const CodebookArgs& cb, const void* x, int dtype, int64_t G, int64_t N,
                          int64_t sx_g, int64_t sx_n, float* u, float* norms, hipStream_t s) {
  if (G * N == 0) return 0;
  RotateArgs a{cb, x, dtype, G, N, sx_g, sx_n, u, norms};
  hipLaunchKernelGGL(rotate_generic_kernel, dim3(grid_for(G * N, 1 << 16)), dim3(64), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

int launch_scores_generic(const CodebookArgs& cb, const uint32_t* krec, int64_t B, int64_t Hkv, int64_t T,
                          const void* q, int q_dtype, int64_t Hq, float scale, float* scores,
                          int32_t* status, hipStream_t s, int64_t q_row, const ChannelMap& cm, bool accumulate) {
  if (B * Hq * T == 0) return 0;
  if (lut_scores_supported(cb, T))
    return launch_scores_lut(cb, krec, B, Hkv, T, q, q_dtype, Hq, scale, scores, status, s, q_row, cm, accumulate);
  ScoreArgs a{cb, krec, B, Hkv, T, q, q_dtype, Hq, scale, scores, status, q_row > 0 ? q_row : cb.d, cm,
              accumulate ? 1 : 0};
  const int64_t chunks = (T + kScoreBlock - 1) / kScoreBlock;
  hipLaunchKernelGGL(scores_generic_kernel, dim3((unsigned)(B * Hq * chunks)), dim3(kScoreBlock), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

int launch_attend_generic(const CodebookArgs& vcb, const uint32_t* vrec, const float* scores, int64_t B,
                          int64_t Hkv, int64_t T, int64_t Hq, float* out, hipStream_t s) {
  if (B * Hq == 0) return 0;
  AttendArgs a{vcb, vrec, scores, B, Hkv, T, Hq, out};
  hipLaunchKernelGGL(attend_generic_kernel, dim3((unsigned)(B * Hq)), dim3(kAttendBlock), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace tq
