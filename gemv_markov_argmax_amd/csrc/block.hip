// The rest of the draft block forward at small M: RMSNorm, the SiLU gate and
// multi-head attention of the drafted positions over a short ragged context.
//
// SharpInference #441, "Observation": besides its projections (the GEMVs of
// gemv.hip), the draft block runs an attention over a short context
// (AttentionBatchedRagged). The pages name no norm or activation; RMSNorm
// and a SiLU-gated MLP are the plainest reading of a Qwen3-derived drafter.
//
// At M = 7 the norm and the gate touch tens of KB; the attention reads the
// context cache (8.4 MB for 512 positions of 32 heads of 128, keys and values).
// All three are latency-bound; every sum runs in a fixed order, so results are
// deterministic.
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

// LDS row strides (floats) of the chunk kernel, chosen so that the MFMA
// operand reads below hit 64 distinct banks: q and the keys are read with
// 16 lanes on 16 rows (stride = 4 mod 64), the values with 4 lanes groups on
// 4 rows of 16 columns (stride = 16 mod 64, whole 16-column tiles).
__host__ __device__ constexpr int attn_ks(int Dh) { return Dh + ((4 - Dh) % 64 + 64) % 64; }
__host__ __device__ constexpr int attn_vs(int Dh) {
  return (Dh + 15) / 16 * 16 + ((16 - (Dh + 15) / 16 * 16) % 64 + 64) % 64;
}

// Reductions over a wave on DPP moves (no LDS round trip): pairs, quads, half
// rows and rows through lane permutes within a row of 16 (every lane of a
// row then holds the row's result), then row 0 into row 1 and row 2 into
// row 3, then rows 0-1 into rows 2-3; lane 63 holds the result, which is
// read back as a scalar. The order is fixed, so the result is deterministic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float x, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
  const float id = MAX ? -INFINITY : 0.f;
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_move<0xb1, 0xf>(v, id));   // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_move<0x4e, 0xf>(v, id));   // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_move<0x141, 0xf>(v, id));  // row_half_mirror
  v = op(v, dpp_move<0x140, 0xf>(v, id));  // row_mirror
  v = op(v, dpp_move<0x142, 0xa>(v, id));  // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_move<0x143, 0xc>(v, id));  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One workgroup of eight waves per (request, head, chunk of 64 keys); chunks
// past the request's Lk exit at once. The chunk's two products run on
// v_mfma_f32_16x16x4f32 (fp32 operands and accumulation; positions padded to
// 16 rows, rows past B never stored):
//  1. The chunk's keys and values and q are loaded first, all in flight
//     together and coalesced: unit e = tid + 512 u is (key e / (Dh / 8),
//     8-dim group e % (Dh / 8)), so consecutive lanes read consecutive bytes
//     of a key's row. q and the keys go to LDS.
//  2. Scores S[16 x 64] = q k^T: wave w takes the 16 keys of tile w % 4 and
//     half of the dims (w / 4), Dh / 8 MFMA steps of 4 dims in order; the two
//     halves are added in step 3. The values then replace the keys in LDS.
//  3. Per position (wave w takes positions w, w + 8): s = (half 0 + half 1)
//     / sqrt(Dh), the chunk maximum and the sum of exp over visible keys
//     (wave_reduce); the probabilities go to LDS.
//  4. o_c[16 x Dh] = P V: wave w takes the 16-column tiles w, w + 8, ..., 16
//     MFMA steps of 4 keys in order, stored straight to the workspace.
__global__ __launch_bounds__(kChunkThreads) void attention_chunk_kernel(AttnParams p, float* __restrict__ ws, int NC) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int B = p.B, Dh = p.Dh, NG = Dh / 8, KS = attn_ks(Dh), VS = attn_vs(Dh);
  float* qs = reinterpret_cast<float*>(smem);      // [16][KS]: q rows (rows past B unused)
  float* Sp = qs + kAttnMaxB * KS;                 // [2][16][64] score halves
  float* Pt = Sp + 2 * kAttnMaxB * kAttnChunk;     // [64][16]: probabilities, key-major
  float* KV = Pt + kAttnChunk * kAttnMaxB;         // [64][KS] keys, then [64][VS] values
  const int c = blockIdx.x % NC, rh = blockIdx.x / NC, r = rh / p.H, h = rh - r * p.H;
  // the wave index as a scalar, so that the loops over a wave's share are
  // uniform (scalar-controlled and unrolled, not exec-masked)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
      *reinterpret_cast<float4*>(qs + i * KS + 4 * d4) =
          *reinterpret_cast<const float4*>(p.q + static_cast<size_t>(r * B + i) * p.ld + h * Dh + 4 * d4);
    }
  }
  auto stage = [&](const Raw8* raw, int stride) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = tid + u * kChunkThreads, jj = e / NG, g = e - jj * NG;
      if (jj < kAttnChunk) {
        float f[8];
        convert_kv8(raw[u], j0 + jj < L, jj < nj, f);
        float* dst = KV + jj * stride + 8 * g;
        *reinterpret_cast<float4*>(dst) = float4{f[0], f[1], f[2], f[3]};
        *reinterpret_cast<float4*>(dst + 4) = float4{f[4], f[5], f[6], f[7]};
      }
    }
  };
  stage(kraw, KS);
  __syncthreads();

  // 2. scores: A = q [16 x 4] (lane: row l % 16, dim l / 16), B = k^T [4 x 16]
  //    (lane: dim l / 16, key l % 16); D rows 4 (l / 16) + v, key l % 16
  const int li = lane & 15, lk = lane >> 4;
  {
    const int t = w & 3, half = w >> 2, steps = Dh / 8, s0 = half * steps;
    const float* qa = qs + li * KS + lk;
    const float* kb = KV + (16 * t + li) * KS + lk;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int st = s0;
    for (; st + 4 <= s0 + steps; st += 4) {  // four steps' operands read before their MFMAs
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = qa[4 * (st + u)];
        b[u] = kb[4 * (st + u)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[u], acc, 0, 0, 0);
    }
    for (; st < s0 + steps; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * st], kb[4 * st], acc, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) Sp[(half * kAttnMaxB + 4 * lk + v) * kAttnChunk + 16 * t + li] = acc[v];
  }
  __syncthreads();  // the keys are consumed
  stage(vraw, VS);

  // 3. chunk softmax statistics
  const float scale = 1.0f / sqrtf(static_cast<float>(Dh));
  const size_t wbase = attn_ws_index(r, h, c, p.H, NC, B, Dh);
  for (int i = w; i < B; i += kChunkWaves) {
    const int jj = lane, j = j0 + jj;
    const bool vis = jj < nj && (!p.causal || j <= L + i);
    const float sc = (Sp[i * kAttnChunk + jj] + Sp[(kAttnMaxB + i) * kAttnChunk + jj]) * scale;
    const float mx = wave_reduce<true>(vis ? sc : -INFINITY);
    const float e = vis ? expf(sc - mx) : 0.f;
    const float sum = wave_reduce<false>(e);
    Pt[jj * kAttnMaxB + i] = e;
    if (lane == 0) {
      ws[wbase + i] = mx;
      ws[wbase + B + i] = sum;
    }
  }
  __syncthreads();

  // 4. o_c = P V: A = P [16 x 4] (lane: row l % 16, key l / 16: Pt[64 st + l]),
  //    B = V [4 x 16] (lane: key l / 16, column l % 16)
  const int NT = (Dh + 15) / 16;
  for (int t = w; t < NT; t += kChunkWaves) {
    const float* pa = Pt + lane;
    const float* vb = KV + lk * VS + 16 * t + li;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kAttnChunk / 4; ++st)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[64 * st], vb[4 * st * VS], acc, 0, 0, 0);
    const int col = 16 * t + li;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = 4 * lk + v;
      if (i < B && col < Dh) ws[wbase + 2 * B + i * Dh + col] = acc[v];
    }
  }
}

// Thread per output element (request, head, position i, dim d); a workgroup
// covers 256 consecutive elements of one (request, head). The request's chunks
// are read 16 at a time (m, l and o together, one memory round trip per
// batch) and merged in chunk order; a later batch with a larger maximum
// rescales what is summed so far by exp(M_old - M_new). With at most 16
// chunks this is exactly out = sum_c w_c o_c as defined above.
__global__ __launch_bounds__(kAttnThreads) void attention_merge_kernel(AttnParams p, const float* __restrict__ ws,
                                                                       int NC) {
  constexpr int kBatch = 16;
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
  float M = -INFINITY, l = 0.f, t = 0.f;
  for (int c0 = 0; c0 < nc; c0 += kBatch) {
    float m[kBatch], lc[kBatch], oc[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // clamped indexes: the batch's loads are issued together
      const float* bp = base + min(c0 + u, nc - 1) * stride;
      m[u] = bp[i];
      lc[u] = bp[B + i];
      oc[u] = bp[2 * B + e];
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (c0 + u < nc) Mb = fmaxf(Mb, m[u]);
    if (Mb != M && M != -INFINITY) {  // rescale the earlier batches
      const float sc = expf(M - Mb);
      l *= sc;
      t *= sc;
    }
    M = Mb;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
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

size_t attention_lds_bytes(int Dh) {  // q rows and score halves sized for 16 positions
  const int ks = attn_ks(Dh), vs = attn_vs(Dh);
  return static_cast<size_t>(kAttnMaxB * ks + 2 * kAttnMaxB * kAttnChunk + kAttnChunk * kAttnMaxB +
                             kAttnChunk * (ks > vs ? ks : vs)) * 4;
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
                                 attention_lds_bytes(Dh), st);
  if (e != hipSuccess) return e;
  const long long mgrid = static_cast<long long>(R) * H * ((B * Dh + kAttnThreads - 1) / kAttnThreads);
  return hipLaunchKernel(reinterpret_cast<const void*>(&attention_merge_kernel), dim3(static_cast<unsigned>(mgrid)),
                         dim3(kAttnThreads), args, 0, st);
}

}  // namespace dspark
