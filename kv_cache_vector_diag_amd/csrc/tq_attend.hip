// Attention output over compressed keys and values for one decode step, split
// over the token axis (page "bitpolar 0.3.3 src/kv_cache.rs",
// attention_scores: pre-softmax scores q.k/sqrt(d); the weighted sum of
// decoded values follows the page's decode_values).
//
// x^_t = (n_t/d) D H c[idx_t], so sum_t w_t x^_t = (1/d) D H (sum_t w_t n_t c[idx_t]):
// the weighted sum is accumulated in the rotated domain and transformed once.
//
// Stage 1 (one workgroup per (b, hq, chunk of tokens)): chunk max m_c of the
//   scores, l_c = sum_t exp(s_t - m_c), a_c[j] = sum_t exp(s_t - m_c) n_t c[idx_tj].
// Stage 2 (one workgroup per (b, hq)): m = max_c m_c, l = sum_c l_c e^(m_c - m),
//   a = sum_c a_c e^(m_c - m), o = D H a / (d l)  (o = 0 when T = 0).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kBlock = 256;
constexpr int64_t kChunk = 1024;

struct PartArgs {
  CodebookArgs vcb;
  const uint32_t* vrec;
  const float* scores;   // [B][Hq][T]
  int64_t Hkv, T, Hq, chunks;
  float* part;           // [B*Hq][chunks][d + 2]: a[0..d), m, l
};

// Lanes per token = d/8: lane `sub` of a token owns coordinates 8 sub .. 8 sub + 7,
// i.e. one byte of each bit-plane word.
template <int K>
__global__ __launch_bounds__(kBlock) void attend_part_kernel(PartArgs a) {
  __shared__ float lut[1 << K];
  __shared__ float red[kBlock];
  __shared__ float acc_s[kMaxHeadDim];
  const int tid = threadIdx.x;
  const int d = a.vcb.d, W = a.vcb.plane_words;
  const int64_t bh = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
  const int64_t b = bh / a.Hq, hq = bh % a.Hq;
  const int64_t g = b * a.Hkv + hq * a.Hkv / a.Hq;
  const uint8_t* blob = blob_of(a.vcb, g);
  const float* cent = reinterpret_cast<const float*>(blob + a.vcb.off_c);
  for (int i = tid; i < (1 << K); i += kBlock) lut[i] = cent[i];
  const int64_t t0 = c * kChunk;
  const int64_t t1 = t0 + kChunk < a.T ? t0 + kChunk : a.T;
  const float* s = a.scores + bh * a.T;

  float mx = -INFINITY;
  for (int64_t t = t0 + tid; t < t1; t += kBlock) mx = fmaxf(mx, s[t]);
  mx = wave_max_f32(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  const int lpt = d >> 3;                 // lanes per token
  const int slots = kBlock / lpt;
  const int slot = tid / lpt, sub = tid % lpt;
  const int word = sub >> 2, shift = (sub & 3) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float esum = 0.0f;
  // the next token's plane words, norm and score are loaded while this one is
  // accumulated (one token in flight per lane group is latency-bound)
  const uint32_t* rv = a.vrec + g * a.T * a.vcb.rec_words;
  uint32_t nw[K];
  float nn = 0.0f, ns = 0.0f;
  const auto load_tok = [&](int64_t t) {
    const uint32_t* r = rv + t * a.vcb.rec_words;
#pragma unroll
    for (int p = 0; p < K; ++p) nw[p] = r[p * W + word];
    nn = __uint_as_float(r[K * W]);
    ns = s[t];
  };
  if (t0 + slot < t1) load_tok(t0 + slot);
  for (int64_t t = t0 + slot; t < t1; t += slots) {
    uint32_t by[K];
#pragma unroll
    for (int p = 0; p < K; ++p) by[p] = nw[p] >> shift;
    const float e = expf(ns - mx);
    const float w = e * nn;
    if (t + slots < t1) load_tok(t + slots);
    esum += e;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t idx = 0;
#pragma unroll
      for (int p = 0; p < K; ++p) idx |= ((by[p] >> i) & 1u) << p;
      acc[i] = fmaf(w, lut[idx], acc[i]);
    }
  }
  // sum over the token slots: coordinates 8 sub + i
  for (int j = tid; j < d; j += kBlock) acc_s[j] = 0.0f;
  red[tid] = sub == 0 ? esum : 0.0f;
  __syncthreads();
  for (int sl = 0; sl < slots; ++sl) {
    if (slot == sl) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc_s[8 * sub + i] += acc[i];
    }
    __syncthreads();
  }
  float* out = a.part + (bh * a.chunks + c) * (d + 2);
  for (int j = tid; j < d; j += kBlock) out[j] = acc_s[j];
  if (tid < 64) {
    float l = 0.0f;
    for (int i = tid; i < kBlock; i += 64) l += red[i];
    l = wave_sum_f32(l);
    if (tid == 0) {
      out[d] = mx;
      out[d + 1] = l;
    }
  }
}

struct MergeArgs {
  CodebookArgs vcb;
  const float* part;
  int64_t Hkv, Hq, chunks;
  float* out;            // [B][Hq][d]
};

__global__ __launch_bounds__(kBlock) void attend_merge_kernel(MergeArgs a) {
  constexpr int kWTile = 2048;             // chunk weights held in LDS at a time
  __shared__ float v[kMaxHeadDim];
  __shared__ float wsh[kWTile];
  __shared__ float red[kBlock / 64];
  const int tid = threadIdx.x;
  const int d = a.vcb.d;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.Hq, hq = bh % a.Hq;
  const int64_t g = b * a.Hkv + hq * a.Hkv / a.Hq;
  const uint32_t* dbits = reinterpret_cast<const uint32_t*>(blob_of(a.vcb, g) + a.vcb.off_d);
  const float* p = a.part + bh * a.chunks * (d + 2);
  float mx = -INFINITY;
  for (int64_t c = tid; c < a.chunks; c += kBlock) mx = fmaxf(mx, p[c * (d + 2) + d]);
  mx = wave_max_f32(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float l = 0.0f;
  float aj[kMaxHeadDim / kBlock > 0 ? kMaxHeadDim / kBlock : 1] = {};
  for (int64_t c0 = 0; c0 < a.chunks; c0 += kWTile) {
    const int nc = (int)(a.chunks - c0 < kWTile ? a.chunks - c0 : kWTile);
    // rescale factor of each chunk, once
    for (int c = tid; c < nc; c += kBlock) {
      const float wc = expf(p[(c0 + c) * (d + 2) + d] - mx);
      wsh[c] = wc;
      l = fmaf(p[(c0 + c) * (d + 2) + d + 1], wc, l);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxHeadDim / kBlock; ++k) {
      const int j = tid + k * kBlock;
      if (j < d) {
        const float* pj = p + c0 * (d + 2) + j;
        float s0 = 0.0f, s1 = 0.0f;
        int c = 0;
        for (; c + 1 < nc; c += 2) {
          s0 = fmaf(pj[c * (d + 2)], wsh[c], s0);
          s1 = fmaf(pj[(c + 1) * (d + 2)], wsh[c + 1], s1);
        }
        if (c < nc) s0 = fmaf(pj[c * (d + 2)], wsh[c], s0);
        aj[k] += s0 + s1;
      }
    }
    __syncthreads();
  }
  l = wave_sum_f32(l);
  if ((tid & 63) == 0) red[tid >> 6] = l;
#pragma unroll
  for (int k = 0; k < kMaxHeadDim / kBlock; ++k)
    if (tid + k * kBlock < d) v[tid + k * kBlock] = aj[k];
  __syncthreads();
  l = red[0] + red[1] + red[2] + red[3];
  for (int h = 1; h < d; h <<= 1) {
    for (int q = tid; q < d / 2; q += kBlock) {
      int i = (q / h) * 2 * h + (q % h);
      float x0 = v[i], x1 = v[i + h];
      v[i] = x0 + x1;
      v[i + h] = x0 - x1;
    }
    __syncthreads();
  }
  const float norm = l > 0.0f ? 1.0f / ((float)d * l) : 0.0f;
  for (int j = tid; j < d; j += kBlock) {
    const float o = v[j] * norm;
    a.out[bh * d + j] = ((dbits[j >> 5] >> (j & 31)) & 1u) ? -o : o;
  }
}

}  // namespace

int64_t attend_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }

bool attend_split_supported(const CodebookArgs& vcb) {
  return vcb.rotation == kRotHadamard && vcb.d >= 8 && vcb.d <= kMaxHeadDim && vcb.k >= 1 && vcb.k <= 8;
}

int launch_attend_split(const CodebookArgs& vcb, const uint32_t* vrec, const float* scores, int64_t B,
                        int64_t Hkv, int64_t T, int64_t Hq, float* part, float* out, hipStream_t s) {
  if (B * Hq == 0) return 0;
  const int64_t chunks = attend_chunks(T);
  if (chunks > 0) {
    PartArgs pa{vcb, vrec, scores, Hkv, T, Hq, chunks, part};
    const dim3 grid((unsigned)(B * Hq * chunks));
    switch (vcb.k) {
      case 1: hipLaunchKernelGGL(attend_part_kernel<1>, grid, dim3(kBlock), 0, s, pa); break;
      case 2: hipLaunchKernelGGL(attend_part_kernel<2>, grid, dim3(kBlock), 0, s, pa); break;
      case 3: hipLaunchKernelGGL(attend_part_kernel<3>, grid, dim3(kBlock), 0, s, pa); break;
      case 4: hipLaunchKernelGGL(attend_part_kernel<4>, grid, dim3(kBlock), 0, s, pa); break;
      case 5: hipLaunchKernelGGL(attend_part_kernel<5>, grid, dim3(kBlock), 0, s, pa); break;
      case 6: hipLaunchKernelGGL(attend_part_kernel<6>, grid, dim3(kBlock), 0, s, pa); break;
      case 7: hipLaunchKernelGGL(attend_part_kernel<7>, grid, dim3(kBlock), 0, s, pa); break;
      default: hipLaunchKernelGGL(attend_part_kernel<8>, grid, dim3(kBlock), 0, s, pa); break;
    }
    if (hipGetLastError() != hipSuccess) return -10;
  }
  MergeArgs ma{vcb, part, Hkv, Hq, chunks, out};
  hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)(B * Hq)), dim3(kBlock), 0, s, ma);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}

}  // namespace tq
