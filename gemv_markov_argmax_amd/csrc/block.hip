// The rest of the draft block forward at small M: RMSNorm, the SiLU gate and
// multi-head attention of the drafted positions over a short ragged context.
//
// SharpInference #441, "Observation": besides its projections (the GEMVs of
// gemv.hip), the draft block runs an attention over a short context
// (AttentionBatchedRagged). The pages name no norm or activation; RMSNorm
// and a SiLU-gated MLP are the plainest reading of a Qwen3-derived drafter.
//
// All three are small at M = 7 (tens of KB) and latency-bound; each sum runs
// in a fixed order, so results are deterministic.
#include "dspark_internal.h"

#include <algorithm>

namespace dspark {
namespace {

constexpr int kNormThreads = 256;

// y[m, :] = x[m, :] / sqrt(mean(x[m, :]^2) + eps) * gamma. One workgroup per
// row; thread t sums t, t + 256, ... in order, then a fixed butterfly per
// wave and the four wave totals in wave order.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const float* __restrict__ x, int D,
                                                               const uint16_t* __restrict__ gamma, float eps,
                                                               float* __restrict__ y) {
  __shared__ float part[kNormThreads / kWave];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* xr = x + static_cast<size_t>(m) * D;
  float ss = 0.f;
  for (int t = tid; t < D; t += kNormThreads) ss = __builtin_fmaf(xr[t], xr[t], ss);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) part[w] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(D) + eps);
  float* yr = y + static_cast<size_t>(m) * D;
  for (int t = tid; t < D; t += kNormThreads) yr[t] = xr[t] * inv * __uint_as_float(static_cast<uint32_t>(gamma[t]) << 16);
}

// a[m, j] = g / (1 + exp(-g)) * u with g = gu[m, j], u = gu[m, F + j].
__global__ __launch_bounds__(256) void silu_gate_kernel(const float* __restrict__ gu, int M, int F,
                                                        float* __restrict__ a) {
  const size_t n = static_cast<size_t>(M) * F;
  for (size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; e < n; e += static_cast<size_t>(gridDim.x) * 256) {
    const size_t m = e / F, j = e - m * F;
    const float g = gu[m * 2 * F + j], u = gu[m * 2 * F + F + j];
    a[e] = g / (1.0f + expf(-g)) * u;
  }
}

struct AttnParams {
  const float* q;      // [R * B, ld] (head h at columns h * Dh)
  const float* kb;     // [R * B, ld] block keys
  const float* vb;     // [R * B, ld] block values
  int ld;
  int R, B, H, Dh;
  const uint16_t* kc;  // [R, Lmax, H * Dh] context keys (bf16)
  const uint16_t* vc;  // [R, Lmax, H * Dh] context values (bf16)
  int Lmax;
  const int32_t* ctx_len;  // [R]
  int causal;
  float* out;  // [R * B, H * Dh]
};

constexpr int kAttnThreads = 256;
constexpr int kAttnMaxB = 16;
constexpr int kAttnMaxDh = 256;
constexpr size_t kAttnScoreBytes = 96 * 1024;  // LDS for the scores of a (request, head)

// One workgroup per (request, head). Keys: the request's first L context
// positions, then its B block positions (key L + j is block position j).
//  1. q of the B positions into LDS; thread t scores keys t, t + 256, ...
//     against every position (the key's Dh values from memory, q broadcast
//     from LDS), scores into LDS [B][L + B].
//  2. Softmax per position: wave w handles positions w, w + 4, ...; max and
//     sum over its keys in lane order, then a fixed butterfly; the
//     probabilities replace the scores (keys a causal position does not see
//     get 0).
//  3. out[i, d] = sum_j p[i, j] v[j, d]: thread d (of Dh) over all keys in
//     order, for every position.
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(AttnParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* qs = reinterpret_cast<float*>(smem);               // [B][Dh]
  float* S = qs + kAttnMaxB * kAttnMaxDh;                   // [B][Lk]
  const int r = blockIdx.x / p.H, h = blockIdx.x - r * p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int B = p.B, Dh = p.Dh, HD = p.H * Dh;
  const int L = min(max(p.ctx_len[r], 0), p.Lmax);
  const int Lk = L + B;
  const float scale = 1.0f / sqrtf(static_cast<float>(Dh));

  for (int e = tid; e < B * Dh; e += kAttnThreads) {
    const int i = e / Dh, d = e - i * Dh;
    qs[i * Dh + d] = p.q[static_cast<size_t>(r * B + i) * p.ld + h * Dh + d];
  }
  __syncthreads();

  for (int j = tid; j < Lk; j += kAttnThreads) {
    float s[kAttnMaxB];
#pragma unroll
    for (int i = 0; i < kAttnMaxB; ++i) s[i] = 0.f;
    if (j < L) {
      const uint16_t* kr = p.kc + (static_cast<size_t>(r) * p.Lmax + j) * HD + h * Dh;
      for (int d = 0; d < Dh; d += 8) {
        const u32x4 kw = load16(kr + d);
        const float kv[8] = {__uint_as_float(kw.x << 16), __uint_as_float(kw.x & 0xffff0000u),
                             __uint_as_float(kw.y << 16), __uint_as_float(kw.y & 0xffff0000u),
                             __uint_as_float(kw.z << 16), __uint_as_float(kw.z & 0xffff0000u),
                             __uint_as_float(kw.w << 16), __uint_as_float(kw.w & 0xffff0000u)};
#pragma unroll
        for (int i = 0; i < kAttnMaxB; ++i) {
          if (i >= B) break;
#pragma unroll
          for (int u = 0; u < 8; ++u) s[i] = __builtin_fmaf(qs[i * Dh + d + u], kv[u], s[i]);
        }
      }
    } else {
      const float* kr = p.kb + static_cast<size_t>(r * B + (j - L)) * p.ld + h * Dh;
      for (int d = 0; d < Dh; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(kr + d);
#pragma unroll
        for (int i = 0; i < kAttnMaxB; ++i) {
          if (i >= B) break;
          s[i] = __builtin_fmaf(qs[i * Dh + d], kv.x, s[i]);
          s[i] = __builtin_fmaf(qs[i * Dh + d + 1], kv.y, s[i]);
          s[i] = __builtin_fmaf(qs[i * Dh + d + 2], kv.z, s[i]);
          s[i] = __builtin_fmaf(qs[i * Dh + d + 3], kv.w, s[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kAttnMaxB; ++i) {
      if (i >= B) break;
      S[i * Lk + j] = s[i] * scale;
    }
  }
  __syncthreads();

  for (int i = w; i < B; i += kAttnThreads / kWave) {
    float* Si = S + i * Lk;
    const int nk = p.causal ? L + i + 1 : Lk;  // keys position i sees
    float mx = -INFINITY;
    for (int j = lane; j < nk; j += kWave) mx = fmaxf(mx, Si[j]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float sum = 0.f;
    for (int j = lane; j < nk; j += kWave) {
      const float e = expf(Si[j] - mx);
      Si[j] = e;
      sum += e;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    const float inv = 1.0f / sum;
    for (int j = lane; j < Lk; j += kWave) Si[j] = j < nk ? Si[j] * inv : 0.f;
  }
  __syncthreads();

  for (int d = tid; d < Dh; d += kAttnThreads) {
    float o[kAttnMaxB];
#pragma unroll
    for (int i = 0; i < kAttnMaxB; ++i) o[i] = 0.f;
    for (int j = 0; j < Lk; ++j) {
      const float v = j < L ? __uint_as_float(static_cast<uint32_t>(p.vc[(static_cast<size_t>(r) * p.Lmax + j) * HD + h * Dh + d]) << 16)
                            : p.vb[static_cast<size_t>(r * B + (j - L)) * p.ld + h * Dh + d];
#pragma unroll
      for (int i = 0; i < kAttnMaxB; ++i) {
        if (i >= B) break;
        o[i] = __builtin_fmaf(S[i * Lk + j], v, o[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kAttnMaxB; ++i) {
      if (i >= B) break;
      p.out[static_cast<size_t>(r * B + i) * HD + h * Dh + d] = o[i];
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm(const float* x, int M, int D, const uint16_t* gamma, float eps, float* y, hipStream_t st) {
  void* args[] = {&x, &D, &gamma, &eps, &y};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rmsnorm_kernel), dim3(M), dim3(kNormThreads), args, 0, st);
}

hipError_t launch_silu_gate(const float* gu, int M, int F, float* a, hipStream_t st) {
  const long long n = static_cast<long long>(M) * F;
  const int grid = static_cast<int>(std::max(1LL, std::min(4096LL, (n + 255) / 256)));
  void* args[] = {&gu, &M, &F, &a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&silu_gate_kernel), dim3(grid), dim3(256), args, 0, st);
}

size_t attention_lds_bytes(int B, int Lmax) {
  return static_cast<size_t>(kAttnMaxB) * kAttnMaxDh * 4 + static_cast<size_t>(B) * (Lmax + B) * 4;
}

bool attention_shape_fits(int B, int H, int Dh, int Lmax) {
  return B >= 1 && B <= kAttnMaxB && H >= 1 && Dh >= 8 && Dh <= kAttnMaxDh && Dh % 8 == 0 && Lmax >= 0 &&
         static_cast<size_t>(B) * (Lmax + B) * 4 <= kAttnScoreBytes;
}

hipError_t launch_attention(const float* q, const float* kb, const float* vb, int ld, int R, int B, int H, int Dh,
                            const uint16_t* kc, const uint16_t* vc, int Lmax, const int32_t* ctx_len, int causal,
                            float* out, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&attention_kernel);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(160 * 1024));
  if (attr != hipSuccess) return attr;
  AttnParams a{q, kb, vb, ld, R, B, H, Dh, kc, vc, Lmax, ctx_len, causal, out};
  void* args[] = {&a};
  return hipLaunchKernel(fn, dim3(R * H), dim3(kAttnThreads), args, attention_lds_bytes(B, Lmax), st);
}

}  // namespace dspark
