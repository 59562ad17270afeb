// The k-step Markov-biased greedy sampling loop, kept on the device.
//
// vllm.cpp #436 "SPEC-DSPARK W7", section "The fix": each step gathers the
// markov_w1 row of the previous token, multiplies markov_w2 by it, adds the
// step's base-logit row, takes the argmax with the lowest index winning
// ties, maps it through d2t, and the previous token never leaves the device;
// only the final [num_reqs, k] ids are read back. Section "W7 LANDED":
// markov_w2 is [draft_vocab, markov_rank] bf16 and each step's bias GEMV
// reads all of it, so a step costs one pass over markov_w2.
//
// Design on gfx950 (one kernel per step, all on the caller's stream):
//  * Step kernel: each workgroup owns a contiguous range of 16-row tiles of
//    markov_w2. A wave streams a tile with 16-byte loads straight into the
//    B operand of v_mfma_f32_16x16x32_bf16; the A operand holds the gathered
//    markov_w1 rows of up to 16 requests (exact bf16, so no splitting is
//    needed), giving bias[request][vocab] for a whole tile in r/32 MFMAs.
//    The score add and a running (score, index) maximum are fused into the
//    same pass; s never reaches memory.
//  * Argmax: every candidate is packed into a 64-bit key whose unsigned
//    order is (score, then lower index), so the reduction is a plain max:
//    lanes, then waves through LDS, then one key per workgroup written to
//    the workspace. No atomics; the result is independent of scheduling.
//  * prev: the next step's kernel reduces the previous step's per-workgroup
//    keys itself (a few KB from cache) while its first markov_w2 loads are
//    already in flight. A last tiny kernel turns every step's keys into ids.
#include "dspark_internal.h"

#include <algorithm>

namespace dspark {
namespace {

constexpr int kMarkovThreads = 256;           // 4 waves
constexpr int kMarkovWaves = kMarkovThreads / kWave;
constexpr int kMaxGroups = 1024;              // upper bound of the step grid
constexpr int kMaxReqs = 16;

struct MarkovParams {
  const float* base;       // [R, B, V]
  const uint16_t* w1;      // [V, r]
  const uint16_t* w2;      // [V, r]
  const int64_t* prev0;    // [R]
  const int64_t* d2t;      // [V] or null
  int64_t* ids;            // [R, k]
  uint64_t* part;          // [k][R][G] per-workgroup best keys
  int R, B, V, r, k, G, tiles;
};

__device__ __forceinline__ bool prev0_ok(const MarkovParams& p, int m) {
  const int64_t v = p.prev0[m];
  return v >= 0 && v < p.V;
}

// Reduce the G per-workgroup keys of (step, request) with one wave.
__device__ __forceinline__ uint64_t wave_reduce_keys(const uint64_t* keys, int G, int lane) {
  uint64_t best = 0;
  for (int j = lane; j < G; j += kWave) best = umax64(best, keys[j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) best = umax64(best, __shfl_xor(best, off));
  return best;
}

template <int KBMAX>
__global__ __launch_bounds__(kMarkovThreads) void markov_step_kernel(MarkovParams p, int step) {
  __shared__ uint64_t red[kMarkovWaves][kMaxReqs];
  __shared__ int prev_s[kMaxReqs];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int R = p.R, V = p.V, r = p.r;
  const int KB = (r + 31) / 32;

  const int t0 = static_cast<int>((static_cast<long long>(blockIdx.x) * p.tiles) / gridDim.x);
  const int t1 = static_cast<int>((static_cast<long long>(blockIdx.x + 1) * p.tiles) / gridDim.x);

  // First tile of this wave: issue its markov_w2 loads before resolving prev.
  int t = t0 + w;
  u32x4 bcur[KBMAX];
  auto load_tile = [&](u32x4 (&b)[KBMAX], int tt) {
    const int row = min(tt * 16 + i, V - 1);
    const uint16_t* src = p.w2 + static_cast<size_t>(row) * r + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KBMAX; ++kb) {
      const bool ok = kb < KB && (kb * 32 + 8 * g) < r && tt < t1;
      b[kb] = ok ? load16(src + kb * 32) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  load_tile(bcur, t);

  // prev of every request for this step.
  for (int m = w; m < R; m += kMarkovWaves) {
    int pv;
    if (step == 0) {
      pv = prev0_ok(p, m) ? static_cast<int>(p.prev0[m]) : 0;
    } else {
      const uint64_t key = wave_reduce_keys(p.part + (static_cast<size_t>(step - 1) * R + m) * p.G, p.G, lane);
      pv = static_cast<int>(key_index(key));
      if (pv < 0 || pv >= V) pv = 0;  // defensive: keys always hold an index < V
    }
    if (lane == 0) prev_s[m] = pv;
  }
  __syncthreads();

  // A operand: markov_w1[prev of request i], zero for absent requests.
  u32x4 afr[KBMAX];
  {
    const bool live = i < R && prev0_ok(p, i < R ? i : 0);
    const int pv = live ? prev_s[i] : 0;
    const uint16_t* src = p.w1 + static_cast<size_t>(pv) * r + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KBMAX; ++kb) {
      const bool ok = live && kb < KB && (kb * 32 + 8 * g) < r;
      afr[kb] = ok ? load16(src + kb * 32) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  uint64_t best[4] = {0, 0, 0, 0};
  const size_t row_stride = static_cast<size_t>(p.B) * V;
  const float* base_step = p.base + static_cast<size_t>(step) * V;

  auto score_tile = [&](u32x4 (&b)[KBMAX], int tt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBMAX; ++kb)
      if (kb < KB) acc = mfma_16x16x32(afr[kb], b[kb], acc);
    const int n = tt * 16 + i;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < R && n < V) {
        const float sc = base_step[m * row_stride + n] + acc[v];
        best[v] = umax64(best[v], score_key(sc, static_cast<uint32_t>(n)));
      }
    }
  };

  u32x4 bnext[KBMAX];
  for (; t < t1; t += 2 * kMarkovWaves) {
    load_tile(bnext, t + kMarkovWaves);
    score_tile(bcur, t);
    if (t + kMarkovWaves >= t1) break;
    load_tile(bcur, t + 2 * kMarkovWaves);
    score_tile(bnext, t + kMarkovWaves);
  }

  // Lanes of one 16-lane group hold the same requests: reduce across them.
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) best[v] = umax64(best[v], __shfl_xor(best[v], off));
  if (i == 0)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][4 * g + v] = best[v];
  __syncthreads();
  if (tid < R) {
    uint64_t k = red[0][tid];
#pragma unroll
    for (int ww = 1; ww < kMarkovWaves; ++ww) k = umax64(k, red[ww][tid]);
    p.part[(static_cast<size_t>(step) * R + tid) * p.G + blockIdx.x] = k;
  }
}

// One wave per (request, step): reduce the step's keys, map through d2t.
__global__ __launch_bounds__(kWave) void markov_ids_kernel(MarkovParams p) {
  const int m = blockIdx.x / p.k, step = blockIdx.x % p.k, lane = threadIdx.x;
  const uint64_t key = wave_reduce_keys(p.part + (static_cast<size_t>(step) * p.R + m) * p.G, p.G, lane);
  if (lane == 0) {
    int64_t id = -1;
    if (prev0_ok(p, m)) {
      const int64_t tok = static_cast<int64_t>(key_index(key));
      id = p.d2t ? p.d2t[tok] : tok;
    }
    p.ids[static_cast<size_t>(m) * p.k + step] = id;
  }
}

int step_grid(int V) {
  const int tiles = (V + 15) / 16;
  const int cus = device_cu_count();
  int G = std::min((tiles + kMarkovWaves - 1) / kMarkovWaves, std::max(1, cus) * 4);
  return std::max(1, std::min(G, kMaxGroups));
}

template <int KBMAX>
hipError_t launch_steps(const MarkovParams& prm, hipStream_t st) {
  for (int step = 0; step < prm.k; ++step) {
    MarkovParams a = prm;
    int sv = step;
    void* args[] = {&a, &sv};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&markov_step_kernel<KBMAX>),
                                         dim3(prm.G), dim3(kMarkovThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t markov_workspace_bytes(int num_reqs, int k, int V) {
  if (num_reqs < 1 || num_reqs > kMaxReqs || k < 1 || V < 1) return 0;
  return static_cast<size_t>(k) * num_reqs * kMaxGroups * sizeof(uint64_t);
}

hipError_t launch_markov(const float* base, int R, int B, int V, const uint16_t* w1,
                         const uint16_t* w2, int r, const int64_t* d2t, const int64_t* prev0,
                         int k, int64_t* ids, void* workspace, hipStream_t stream) {
  MarkovParams prm{};
  prm.base = base;
  prm.w1 = w1;
  prm.w2 = w2;
  prm.prev0 = prev0;
  prm.d2t = d2t;
  prm.ids = ids;
  prm.part = static_cast<uint64_t*>(workspace);
  prm.R = R;
  prm.B = B;
  prm.V = V;
  prm.r = r;
  prm.k = k;
  prm.G = step_grid(V);
  prm.tiles = (V + 15) / 16;
  const int KB = (r + 31) / 32;
  hipError_t e;
  if (KB <= 2) e = launch_steps<2>(prm, stream);
  else if (KB <= 4) e = launch_steps<4>(prm, stream);
  else if (KB <= 8) e = launch_steps<8>(prm, stream);
  else if (KB <= 16) e = launch_steps<16>(prm, stream);
  else e = launch_steps<32>(prm, stream);
  if (e != hipSuccess) return e;
  MarkovParams a = prm;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&markov_ids_kernel), dim3(R * k), dim3(kWave),
                         args, 0, stream);
}

}  // namespace dspark
