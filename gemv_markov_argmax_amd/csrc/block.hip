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

constexpr int kNormPer = 16;  // values per thread kept in registers (rows up to 4096)

// y[m, :] = x[m, :] / sqrt(mean(x[m, :]^2) + eps) * gamma. One workgroup per
// row; thread t sums t, t + 256, ... in order, then a fixed butterfly per
// wave and the four wave totals in wave order. A row of up to 4096 values is
// read once into registers, x and gamma together, every load in flight.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const float* __restrict__ x, int D,
                                                               const uint16_t* __restrict__ gamma, float eps,
                                                               float* __restrict__ y) {
  __shared__ float part[kNormThreads / kWave];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* xr = x + static_cast<size_t>(m) * D;
  float* yr = y + static_cast<size_t>(m) * D;
  if (D <= kNormThreads * kNormPer) {
    float v[kNormPer];
    uint32_t g[kNormPer];
#pragma unroll
    for (int u = 0; u < kNormPer; ++u) {
      const int t = tid + u * kNormThreads, tc = t < D ? t : 0;
      v[u] = xr[tc];
      g[u] = gamma[tc];
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < kNormPer; ++u)
      if (tid + u * kNormThreads < D) ss = __builtin_fmaf(v[u], v[u], ss);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) part[w] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(D) + eps);
#pragma unroll
    for (int u = 0; u < kNormPer; ++u) {
      const int t = tid + u * kNormThreads;
      if (t < D) yr[t] = v[u] * inv * __uint_as_float(g[u] << 16);
    }
    return;
  }
  float ss = 0.f;
#pragma unroll 4
  for (int t = tid; t < D; t += kNormThreads) ss = __builtin_fmaf(xr[t], xr[t], ss);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) part[w] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(D) + eps);
#pragma unroll 4
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

constexpr int kAttnThreads = 256;                     // merge kernel
constexpr int kChunkWaves = 8;                        // chunk kernel: eight waves share a chunk's work
constexpr int kChunkThreads = kChunkWaves * 64;
constexpr int kAttnMaxB = 16;
constexpr int kAttnMaxDh = 256;
constexpr int kAttnChunk = 64;  // keys per workgroup: one per lane of a wave

// The keys of request r are its first L = ctx_len[r] context positions, then
// its B block positions (key L + j is block position j): Lk = L + B keys.
// They are split into chunks of 64 keys; the softmax is taken per chunk with
// the chunk's own maximum, and the chunks are merged afterwards (the
// rescaling by exp(m_c - M) makes the merge exact up to rounding):
//   m_c[i] = max_{j in c} s[i, j],  l_c[i] = sum_{j in c} exp(s[i, j] - m_c[i]),
//   o_c[i, :] = sum_{j in c} exp(s[i, j] - m_c[i]) v[j, :],
//   out[i, :] = sum_c w_c o_c,  w_c = exp(m_c - M) / sum_c' exp(m_c' - M) l_c',  M = max_c m_c.
// Workspace per (request, head, chunk): m [B], l [B], o [B][Dh] (fp32).
__device__ __forceinline__ size_t attn_ws_index(int r, int h, int c, int H, int NC, int B, int Dh) {
  return ((static_cast<size_t>(r) * H + h) * NC + c) * static_cast<size_t>(B) * (Dh + 2);
}

// The raw bytes behind dims 8g .. 8g + 7 of key j: 16 bytes of the bf16
// context cache for j < L (the second load repeats the first), 32 bytes of
// the fp32 block projections otherwise; a lane that is not live reads row 0
// of q (a valid address). Addresses are selected, not branched on, so that a
// batch of these stays in flight until its first use.
struct Raw8 {
  u32x4 a, b;
};

__device__ __forceinline__ Raw8 issue_kv8(const uint16_t* cache, const float* blk, const AttnParams& p, int r, int h,
                                          int L, int j, int g, bool live) {
  const int HD = p.H * p.Dh;
  const bool ctx = j < L;
  const uint16_t* pc = cache + (static_cast<size_t>(r) * p.Lmax + (ctx ? j : 0)) * HD + h * p.Dh + 8 * g;
  const float* pf = blk + static_cast<size_t>(r * p.B + (ctx ? 0 : j - L)) * p.ld + h * p.Dh + 8 * g;
  const char* pa = !live ? reinterpret_cast<const char*>(p.q)
                   : ctx ? reinterpret_cast<const char*>(pc)
                         : reinterpret_cast<const char*>(pf);
  const char* pb = live && !ctx ? pa + 16 : pa;
  Raw8 raw;
  raw.a = load16(pa);
  raw.b = load16(pb);
  return raw;
}

// The eight values of issue_kv8's bytes (0 for a lane that is not live).
__device__ __forceinline__ void convert_kv8(const Raw8& raw, bool ctx, bool live, float* f) {
  const uint32_t w[8] = {raw.a.x, raw.a.y, raw.a.z, raw.a.w, raw.b.x, raw.b.y, raw.b.z, raw.b.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t bf = (k & 1) ? (w[k >> 1] & 0xffff0000u) : (w[k >> 1] << 16);
    f[k] = live ? __uint_as_float(ctx ? bf : w[k]) : 0.f;
  }
}

// One workgroup per (request, head, chunk of 64 keys); chunks past the
// request's Lk exit at once.
//  1. The chunk's keys and values and q are loaded first, all in flight
//     together and coalesced: unit e = tid + 256 u is (key e / (Dh / 8),
//     8-dim group e % (Dh / 8)), so consecutive lanes read consecutive bytes
//     of a key's row. q and the keys go to LDS (key rows padded by 4 floats).
//  2. Scores: lane l of wave w (eight waves) takes key 64c + l and sums the
//     dims of groups w, w + 8, ... (8 dims each, in order) against every
//     position (q broadcast from LDS); the wave partials are added pairwise,
//     ((w0 + w1) + (w2 + w3)) + ((w4 + w5) + (w6 + w7)). The values then
//     replace the keys in LDS.
//  3. Per position (wave w takes positions w, w + 8): chunk maximum and the
//     sum of exp over visible keys, a fixed butterfly over the lanes.
//  4. o_c: thread (d, kg) sums keys kg, kg + KG, ... in order (KG = 512 / Dh
//     key groups), the groups then in kg order.
__global__ __launch_bounds__(kChunkThreads) void attention_chunk_kernel(AttnParams p, float* __restrict__ ws, int NC) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int B = p.B, Dh = p.Dh, NG = Dh / 8, KS = Dh + 4;
  float* qs = reinterpret_cast<float*>(smem);   // [B][Dh]
  float* Sp = qs + B * Dh;                      // [8][B][64] score partials, later [KG][B][Dh]
  float* Pt = Sp + kChunkWaves * B * kAttnChunk;  // [64][16]: probabilities, key-major
  float* KV = Pt + kAttnChunk * kAttnMaxB;      // [64][Dh + 4]: keys, then values
  const int c = blockIdx.x % NC, rh = blockIdx.x / NC, r = rh / p.H, h = rh - r * p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = min(max(p.ctx_len[r], 0), p.Lmax);
  const int Lk = L + B, j0 = c * kAttnChunk;
  if (j0 >= Lk) return;  // uniform over the workgroup
  const int nj = min(kAttnChunk, Lk - j0);

  // 1. loads: keys and values (all in flight together), then q into LDS
  constexpr int kU = kAttnChunk * kAttnMaxDh / 8 / kChunkThreads;  // units per thread, at most
  Raw8 kraw[kU], vraw[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int e = tid + u * kChunkThreads, jj = e / NG, g = e - jj * NG;
    kraw[u] = issue_kv8(p.kc, p.kb, p, r, h, L, j0 + jj, g, jj < nj);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int e = tid + u * kChunkThreads, jj = e / NG, g = e - jj * NG;
    vraw[u] = issue_kv8(p.vc, p.vb, p, r, h, L, j0 + jj, g, jj < nj);
  }
  const int D4 = Dh / 4;
  for (int e0 = 0; e0 < B * D4; e0 += kChunkThreads) {  // one pass per 512 float4 units of q
    const int e = e0 + tid;
    if (e < B * D4) {
      const int i = e / D4, d4 = e - i * D4;
      *reinterpret_cast<float4*>(qs + 4 * e) =
          *reinterpret_cast<const float4*>(p.q + static_cast<size_t>(r * B + i) * p.ld + h * Dh + 4 * d4);
    }
  }
  auto stage = [&](const Raw8* raw) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = tid + u * kChunkThreads, jj = e / NG, g = e - jj * NG;
      if (jj < kAttnChunk) {
        float f[8];
        convert_kv8(raw[u], j0 + jj < L, jj < nj, f);
        float* dst = KV + jj * KS + 8 * g;
        *reinterpret_cast<float4*>(dst) = float4{f[0], f[1], f[2], f[3]};
        *reinterpret_cast<float4*>(dst + 4) = float4{f[4], f[5], f[6], f[7]};
      }
    }
  };
  stage(kraw);
  __syncthreads();

  // 2. score partials
  {
    float s[kAttnMaxB];
#pragma unroll
    for (int i = 0; i < kAttnMaxB; ++i) s[i] = 0.f;
    const float* kr = KV + lane * KS;
    for (int g = w; g < NG; g += kChunkWaves) {
      const float4 ka = *reinterpret_cast<const float4*>(kr + 8 * g);
      const float4 kb = *reinterpret_cast<const float4*>(kr + 8 * g + 4);
      // Positions in batches of four: one uniform branch per batch, whose
      // eight LDS reads are issued together, and s[] in fixed registers.
      // Slots past B in the last batch read past q (still inside this
      // workgroup's LDS) and are never stored.
#pragma unroll
      for (int i0 = 0; i0 < kAttnMaxB; i0 += 4) {
        if (i0 < B) {
          float4 qa[4], qb[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            qa[u] = *reinterpret_cast<const float4*>(qs + (i0 + u) * Dh + 8 * g);
            qb[u] = *reinterpret_cast<const float4*>(qs + (i0 + u) * Dh + 8 * g + 4);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float t = s[i0 + u];
            t = __builtin_fmaf(qa[u].x, ka.x, t);
            t = __builtin_fmaf(qa[u].y, ka.y, t);
            t = __builtin_fmaf(qa[u].z, ka.z, t);
            t = __builtin_fmaf(qa[u].w, ka.w, t);
            t = __builtin_fmaf(qb[u].x, kb.x, t);
            t = __builtin_fmaf(qb[u].y, kb.y, t);
            t = __builtin_fmaf(qb[u].z, kb.z, t);
            t = __builtin_fmaf(qb[u].w, kb.w, t);
            s[i0 + u] = t;
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kAttnMaxB; ++i)
      if (i < B) Sp[(w * B + i) * kAttnChunk + lane] = s[i];
  }
  __syncthreads();  // the keys are consumed
  stage(vraw);

  // 3. chunk softmax statistics
  const float scale = 1.0f / sqrtf(static_cast<float>(Dh));
  const size_t wbase = attn_ws_index(r, h, c, p.H, NC, B, Dh);
  for (int i = w; i < B; i += kChunkThreads / kWave) {
    const int jj = lane, j = j0 + jj;
    const bool vis = jj < nj && (!p.causal || j <= L + i);
    const float* si = Sp + i * kAttnChunk + jj;
    const int wstride = B * kAttnChunk;
    const float sc = (((si[0] + si[wstride]) + (si[2 * wstride] + si[3 * wstride])) +
                      ((si[4 * wstride] + si[5 * wstride]) + (si[6 * wstride] + si[7 * wstride]))) * scale;
    float mx = vis ? sc : -INFINITY;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float e = vis ? expf(sc - mx) : 0.f;
    float sum = e;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    Pt[jj * kAttnMaxB + i] = e;
    if (lane == 0) {
      ws[wbase + i] = mx;
      ws[wbase + B + i] = sum;
    }
  }
  __syncthreads();

  // 4. o_c
  const int KG = kChunkThreads / Dh;
  float* Op = Sp;  // [KG][B][Dh]: KG * Dh <= 512, so it fits the partials' space
  if (tid < KG * Dh) {
    const int d = tid % Dh, kg = tid / Dh;
    float o[kAttnMaxB];
#pragma unroll
    for (int i = 0; i < kAttnMaxB; ++i) o[i] = 0.f;
#pragma unroll 4
    for (int jj = kg; jj < nj; jj += KG) {
      const float v = KV[jj * KS + d];
      const float* pj = Pt + jj * kAttnMaxB;  // the key's probabilities, read 4 positions at a time
#pragma unroll
      for (int i4 = 0; i4 < kAttnMaxB; i4 += 4) {  // all 16 slots, no branch; slots past B are never stored
        const float4 pv = *reinterpret_cast<const float4*>(pj + i4);
        o[i4] = __builtin_fmaf(pv.x, v, o[i4]);
        o[i4 + 1] = __builtin_fmaf(pv.y, v, o[i4 + 1]);
        o[i4 + 2] = __builtin_fmaf(pv.z, v, o[i4 + 2]);
        o[i4 + 3] = __builtin_fmaf(pv.w, v, o[i4 + 3]);
      }
    }
#pragma unroll
    for (int i = 0; i < kAttnMaxB; ++i)
      if (i < B) Op[(kg * B + i) * Dh + d] = o[i];
  }
  __syncthreads();
  for (int e = tid; e < B * Dh; e += kChunkThreads) {
    float t = Op[e];
    for (int kg = 1; kg < KG; ++kg) t += Op[kg * B * Dh + e];
    ws[wbase + 2 * B + e] = t;
  }
}

// Thread per output element (request, head, position i, dim d); a workgroup
// covers 256 consecutive elements of one (request, head). It reads the m_c of
// every chunk of the request (M), then l_c and o_c, the chunks in order.
__global__ __launch_bounds__(kAttnThreads) void attention_merge_kernel(AttnParams p, const float* __restrict__ ws,
                                                                       int NC) {
  const int B = p.B, Dh = p.Dh;
  const int EB = (B * Dh + kAttnThreads - 1) / kAttnThreads;
  const int rh = blockIdx.x / EB, r = rh / p.H, h = rh - r * p.H;
  const int e = (blockIdx.x - rh * EB) * kAttnThreads + threadIdx.x;
  if (e >= B * Dh) return;
  const int i = e / Dh;
  const int L = min(max(p.ctx_len[r], 0), p.Lmax);
  const int nc = (L + B + kAttnChunk - 1) / kAttnChunk;
  const float* base = ws + attn_ws_index(r, h, 0, p.H, NC, B, Dh);
  const size_t stride = static_cast<size_t>(B) * (Dh + 2);
  float M = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < nc; ++c) M = fmaxf(M, base[c * stride + i]);
  float l = 0.f, t = 0.f;
  for (int c0 = 0; c0 < nc; c0 += 8) {
    float m[8], lc[8], oc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // clamped indexes: the batch's loads are issued together
      const float* b = base + min(c0 + u, nc - 1) * stride;
      m[u] = b[i];
      lc[u] = b[B + i];
      oc[u] = b[2 * B + e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c0 + u < nc) {
        const float a = m[u] == -INFINITY ? 0.f : expf(m[u] - M);  // a chunk with no visible key adds nothing
        l = __builtin_fmaf(lc[u], a, l);
        t = __builtin_fmaf(oc[u], a, t);
      }
    }
  }
  p.out[static_cast<size_t>(r * B + i) * p.H * Dh + h * Dh + (e - i * Dh)] = t / l;
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

int attention_chunks(int B, int Lmax) { return (Lmax + B + kAttnChunk - 1) / kAttnChunk; }

size_t attention_lds_bytes(int B, int Dh) {
  return static_cast<size_t>(B * Dh + kChunkWaves * B * kAttnChunk + kAttnChunk * kAttnMaxB + kAttnChunk * (Dh + 4)) * 4;
}

bool attention_shape_fits(int R, int B, int H, int Dh, int Lmax) {
  return R >= 1 && B >= 1 && B <= kAttnMaxB && H >= 1 && Dh >= 8 && Dh <= kAttnMaxDh && Dh % 8 == 0 && Lmax >= 0 &&
         Lmax <= (1 << 30) && static_cast<long long>(R) * H * attention_chunks(B, Lmax) <= 0x7fffffffLL &&
         static_cast<long long>(R) * H * ((B * Dh + kAttnThreads - 1) / kAttnThreads) <= 0x7fffffffLL;
}

size_t attention_workspace_bytes(int R, int B, int H, int Dh, int Lmax) {
  return static_cast<size_t>(R) * H * attention_chunks(B, Lmax) * B * (Dh + 2) * 4;
}

hipError_t launch_attention(const float* q, const float* kb, const float* vb, int ld, int R, int B, int H, int Dh,
                            const uint16_t* kc, const uint16_t* vc, int Lmax, const int32_t* ctx_len, int causal,
                            float* out, float* ws, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&attention_chunk_kernel);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(160 * 1024));
  if (attr != hipSuccess) return attr;
  AttnParams a{q, kb, vb, ld, R, B, H, Dh, kc, vc, Lmax, ctx_len, causal, out};
  int NC = attention_chunks(B, Lmax);
  void* args[] = {&a, &ws, &NC};
  const long long grid = static_cast<long long>(R) * H * NC;
  hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(kChunkThreads), args,
                                 attention_lds_bytes(B, Dh), st);
  if (e != hipSuccess) return e;
  const long long mgrid = static_cast<long long>(R) * H * ((B * Dh + kAttnThreads - 1) / kAttnThreads);
  return hipLaunchKernel(reinterpret_cast<const void*>(&attention_merge_kernel), dim3(static_cast<unsigned>(mgrid)),
                         dim3(kAttnThreads), args, 0, st);
}

}  // namespace dspark
