// The k-step Markov-biased greedy sampling loop, kept on the device.
//
// vllm.cpp #436 "SPEC-DSPARK W7", section "The fix": each step gathers the
// markov_w1 row of the previous token, multiplies markov_w2 by it, adds the
// step's base-logit row, takes the argmax with the lowest index winning
// ties, maps it through d2t, and the previous token never leaves the device;
// only the final [num_reqs, k] ids are read back. Section "W7 LANDED":
// markov_w2 is [draft_vocab, markov_rank] bf16 and the bias GEMV of every
// step covers all of it, which the page treats as an irreducible per-step
// re-read.
//
// Design on gfx950: one persistent kernel runs all k steps.
//  * Grid = at most one workgroup per compute unit, and the host checks that
//    the whole grid fits on the device at once, so every workgroup is
//    resident (the steps exchange keys between all of them). Workgroup b owns a contiguous range of 16-row
//    tiles of markov_w2 and loads it ONCE per call into on-chip storage:
//    the first tiles stay in VGPRs (RT tiles per wave, already in MFMA
//    B-operand layout), the next ones in LDS, and only what does not fit
//    (very large vocabularies) is re-read from memory at each step. On
//    MI355X the register files and LDS of 256 CUs hold ~168 MB, so the
//    78 MB markov_w2 of a 151936 x 256 draft vocabulary is read from HBM
//    once per call instead of once per step.
//  * Per step, the A operand of v_mfma_f32_16x16x32_bf16 holds the gathered
//    markov_w1 rows of up to 16 requests (exact bf16), so one tile's bias for
//    every request is r/32 MFMAs; the base-row add and a running maximum of
//    packed (score, index) keys are fused into the same pass. Keys order by
//    score, then by lower index, so a plain max gives the greedy pick with
//    the lowest index winning ties, independent of reduction order.
//  * Steps are separated by a key exchange that doubles as the grid barrier:
//    every workgroup publishes its best key per request into its own slot (a
//    valid key is never zero) and polls the G slots of that step with
//    coherent loads until all are present (bounded spin), taking their
//    maximum as it goes. Every workgroup thus learns prev without a counter
//    or a second round trip. Workgroup 0 writes the ids. The next step's base
//    values are fetched before the exchange, so only the markov_w1 gather
//    follows it.
//  * The key slots must read zero when a call starts, without a clearing
//    launch in front of every call. The workspace holds two slot buffers and
//    a call sequence number whose parity picks the active one; while a call
//    runs, its workgroups clear the entries the previous call used in the
//    other buffer, and workgroup 0, the last to read any slot, advances the
//    sequence number at the end. Only a stream-ordered next call uses that
//    buffer, so it is clean by then. The workspace must therefore be
//    zero-filled once before first use. A poll that gives up (which the
//    residency check rules out on an otherwise idle device) leaves a sticky
//    flag: that call and every later one on the workspace return -2 ids
//    until it is zero-filled again.
//  * Nothing but the exchange sits on the per-step path of workgroup 0: the
//    drafted tokens stay in LDS and the ids (d2t applied) are written once,
//    after the last step.
//  * No floating-point atomics anywhere; results do not depend on timing.
#include "dspark_internal.h"

#include <algorithm>

namespace dspark {
namespace {

constexpr int kMaxReqs = 16;
constexpr int kMaxSteps = 32;
constexpr int kMaxGroups = 256;          // grid cap: one workgroup per CU
constexpr int kLoopWaves = 8;
constexpr int kLoopThreads = kLoopWaves * kWave;
constexpr size_t kCtlBytes = 256;        // control words, then two slot buffers
constexpr size_t kSlotsPerBuffer = static_cast<size_t>(kMaxSteps) * kMaxReqs * kMaxGroups;
// Control words (uint32) at the start of the workspace.
constexpr int kCtlWatchdog = 0;  // nonzero: a poll gave up; sticky until the workspace is zero-filled
constexpr int kCtlSeq = 1;       // call sequence number; its parity selects the active slot buffer
constexpr int kCtlUsed = 4;      // [4 + b]: slots the last call that used buffer b wrote
constexpr size_t kLdsBytes = 160 * 1024;
constexpr uint32_t kSpinLimit = 1u << 18;  // watchdog (~0.3 s of polling): far beyond any legitimate wait

struct MarkovParams {
  const float* base;     // [R, B, V]
  const uint16_t* w1;    // [V, r]
  const uint16_t* w2;    // [V, r]
  const int64_t* prev0;  // [R]
  const int64_t* d2t;    // [V] or null
  int64_t* ids;          // [R, k]
  uint32_t* ctl;         // control words (kCtl*)
  uint64_t* slots;       // [2][kSlotsPerBuffer]; active buffer: [k][R][G] per-workgroup best keys
  int R, B, V, r, k, G, tiles;
  int lds_tiles;         // markov_w2 tiles held in LDS per workgroup
  int bstride;           // floats per request in the LDS base slice (>= 16 * tiles per workgroup)
  int base_in_lds;       // 0: base values are read straight from memory (slice too large)
};

__device__ __forceinline__ bool prev0_ok(const MarkovParams& p, int m) {
  const int64_t v = p.prev0[m];
  return v >= 0 && v < p.V;
}

__device__ __forceinline__ uint64_t load_coherent(const uint64_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_coherent(const uint32_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kMaxPoll = kMaxGroups / kWave;  // slots per lane when polling

template <int KB, int RT>
__global__ __launch_bounds__(kLoopThreads) void markov_loop_kernel(MarkovParams p) {
  constexpr int NW = kLoopWaves;
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4* w2l = reinterpret_cast<u32x4*>(smem);                                         // [lds_tiles][KB][64]
  uint64_t* keys_s = reinterpret_cast<uint64_t*>(smem + static_cast<size_t>(p.lds_tiles) * KB * 1024);  // [NW][16]
  int* prev_s = reinterpret_cast<int*>(keys_s + NW * kMaxReqs);                           // [16]
  int* tok_s = prev_s + kMaxReqs;                                                         // [k][R] drafted tokens
  float* basel = reinterpret_cast<float*>(tok_s + kMaxSteps * kMaxReqs);                  // [R][bstride]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int R = p.R, V = p.V, r = p.r, G = p.G;
  const int t0 = static_cast<int>((static_cast<long long>(blockIdx.x) * p.tiles) / G);
  const int t1 = static_cast<int>((static_cast<long long>(blockIdx.x + 1) * p.tiles) / G);
  const int nt = t1 - t0;
  const int nreg = min(nt, NW * RT);
  const int nheld = nreg + min(nt - nreg, p.lds_tiles);
  // Active slot buffer of this call, and the sticky watchdog flag (issued
  // first: the replies arrive while markov_w2 loads).
  const uint32_t seq = load_coherent(p.ctl + kCtlSeq);
  const uint32_t dead = load_coherent(p.ctl + kCtlWatchdog);

  auto w2_row = [&](int j, int lrow) {
    const int row = min((t0 + j) * 16 + lrow, V - 1);
    return p.w2 + static_cast<size_t>(row) * r;
  };

  // ---- load this workgroup's markov_w2 tiles once: registers, then LDS
  u32x4 wreg[RT > 0 ? RT : 1][KB];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    const int j = w + NW * u;
    const uint16_t* src = w2_row(j, i) + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      wreg[u][kb] = (j < nreg && kb * 32 + 8 * g < r) ? load16(src + kb * 32) : u32x4{0u, 0u, 0u, 0u};
  }
  for (int e = tid; e < (nheld - nreg) * KB * kWave; e += kLoopThreads) {
    const int ln = e & 63, kb = (e >> 6) % KB, jj = (e >> 6) / KB;
    const int gg = ln >> 4;
    w2l[e] = (kb * 32 + 8 * gg < r) ? load16(w2_row(nreg + jj, ln & 15) + kb * 32 + 8 * gg)
                                    : u32x4{0u, 0u, 0u, 0u};
  }
  if (tid < R) prev_s[tid] = prev0_ok(p, tid) ? static_cast<int>(p.prev0[tid]) : 0;

  const int cur = static_cast<int>(seq & 1u);
  uint64_t* part = p.slots + cur * kSlotsPerBuffer;
  const uint32_t used_other = load_coherent(p.ctl + kCtlUsed + (cur ^ 1));
  // Clears what the previous call left in the other buffer (which the next
  // call uses), shared by the workgroups that finish early: all but 0, or 0
  // alone. These stores stay out of the step loop: a store in flight would
  // make a wave drain its outstanding loads before it may use any of them.
  auto clear_other = [&]() {
    uint64_t* other = p.slots + (cur ^ 1) * kSlotsPerBuffer;
    const uint32_t used = min(used_other, static_cast<uint32_t>(kSlotsPerBuffer));
    const uint32_t nwg = G > 1 ? G - 1 : 1, wg = G > 1 ? blockIdx.x - 1 : 0;
    for (uint32_t e = wg * kLoopThreads + tid; e < used; e += nwg * kLoopThreads)
      __hip_atomic_store(other + e, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // Workgroup 0 after the last step (every other workgroup has published
  // every step, so none reads a slot any more): the ids of all steps, the
  // slots used, and the next sequence number. A poll that gave up in this
  // call or an earlier one turns every id into -2.
  auto finish = [&]() {
    if (G == 1) clear_other();
    const bool bad = dead != 0u || load_coherent(p.ctl + kCtlWatchdog) != 0u;
    for (int e = tid; e < R * p.k; e += kLoopThreads) {
      const int m = e / p.k, st = e - m * p.k;
      int64_t id = -1;
      if (dead == 0u && prev0_ok(p, m)) {  // tok_s holds this call's tokens (each in [0, V))
        const int tok = tok_s[st * kMaxReqs + m];
        id = p.d2t ? p.d2t[tok] : static_cast<int64_t>(tok);
      }
      p.ids[e] = bad ? -2 : id;
    }
    if (tid == 0) {
      __hip_atomic_store(p.ctl + kCtlUsed + cur, static_cast<uint32_t>(p.k * R * G), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctl + kCtlSeq, seq + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  const bool bl = p.base_in_lds != 0;
  const int nb = bl ? R * nt * 16 : 0;  // base values of this workgroup staged per step
  constexpr int kPre = 4;               // prefetched base values per thread
  // Entries e = tid + u*threads of the slice: LDS slot and base offset (step 0), fixed for the call.
  int pre_lds[kPre];
  size_t pre_src[kPre];
  bool pre_ok[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int e = tid + u * kLoopThreads;
    const int m = e < nb ? e / (nt * 16) : 0, nl = e - m * (nt * 16);
    const int n = t0 * 16 + nl;
    pre_lds[u] = m * p.bstride + nl;
    pre_src[u] = static_cast<size_t>(m) * p.B * V + n;
    pre_ok[u] = e < nb && n < V;
  }
  float pre[kPre];
  auto fetch_base = [&](int st) {
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      pre[u] = pre_ok[u] ? p.base[pre_src[u] + static_cast<size_t>(st) * V] : 0.f;
  };
  auto stage_base = [&](int st) {  // prefetched values, then any remainder straight from memory
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      if (tid + u * kLoopThreads < nb) basel[pre_lds[u]] = pre[u];
    for (int e = tid + kPre * kLoopThreads; e < nb; e += kLoopThreads) {
      const int m = e / (nt * 16), nl = e - m * (nt * 16);
      const int n = t0 * 16 + nl;
      basel[m * p.bstride + nl] = n < V ? p.base[(static_cast<size_t>(m) * p.B + st) * V + n] : 0.f;
    }
  };
  fetch_base(0);

  if (dead != 0u) {  // an earlier call gave up: report it and touch no slot
    if (blockIdx.x == 0) finish();
    return;
  }

  for (int step = 0; step < p.k; ++step) {
    __syncthreads();  // prev_s written; the previous step is done with basel
    // ---- A operand: markov_w1[prev] of request i (zero for absent or invalid
    // requests); issued first, it is the only load on this step's critical path
    u32x4 afr[KB];
    {
      const bool live = i < R && prev0_ok(p, i < R ? i : 0);
      const uint16_t* src = p.w1 + static_cast<size_t>(live ? prev_s[i] : 0) * r + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        afr[kb] = (live && kb * 32 + 8 * g < r) ? load16(src + kb * 32) : u32x4{0u, 0u, 0u, 0u};
    }
    stage_base(step);
    __syncthreads();  // basel ready

    uint64_t best[4] = {0, 0, 0, 0};
    auto score = [&](int j, f32x4 acc) {
      const int n = (t0 + j) * 16 + i;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < R && n < V) {
          const float bv = bl ? basel[m * p.bstride + j * 16 + i]
                              : p.base[(static_cast<size_t>(m) * p.B + step) * V + n];
          best[v] = umax64(best[v], score_key(bv + acc[v], static_cast<uint32_t>(n)));
        }
      }
    };
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int j = w + NW * u;
      if (j < nreg) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mfma_16x16x32(afr[kb], wreg[u][kb], acc);
        score(j, acc);
      }
    }
    for (int j = nreg + w; j < nt; j += NW) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (j < nheld) {
        const u32x4* src = w2l + static_cast<size_t>(j - nreg) * KB * kWave + lane;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mfma_16x16x32(afr[kb], src[kb * kWave], acc);
      } else {
        const uint16_t* src = w2_row(j, i) + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x4 b = (kb * 32 + 8 * g < r) ? load16(src + kb * 32) : u32x4{0u, 0u, 0u, 0u};
          acc = mfma_16x16x32(afr[kb], b, acc);
        }
      }
      score(j, acc);
    }
    const bool last = step == p.k - 1;
    if (!last) fetch_base(step + 1);  // independent of this step's winner

    // ---- workgroup maximum per request (lanes of a 16-lane group share requests 4g..4g+3)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v >= R) break;
      best[v] = row_max64(best[v]);
    }
    if (i == 0)
#pragma unroll
      for (int v = 0; v < 4; ++v) keys_s[w * kMaxReqs + 4 * g + v] = best[v];
    __syncthreads();

    // ---- publish this workgroup's key of every request
    if (tid < R) {
      uint64_t kk = keys_s[tid];
      for (int ww = 1; ww < NW; ++ww) kk = umax64(kk, keys_s[ww * kMaxReqs + tid]);
      __hip_atomic_store(part + (static_cast<size_t>(step) * R + tid) * G + blockIdx.x, kk, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    if (last && blockIdx.x != 0) {  // only workgroup 0 needs the final step's winner
      clear_other();
      return;
    }

    // ---- exchange: poll the G slots of each request until all are published
    for (int m = w; m < R; m += NW) {
      const uint64_t* src = part + (static_cast<size_t>(step) * R + m) * G;
      uint64_t kk = 0;
      uint32_t spins = 0;
      for (;;) {
        uint64_t slot[kMaxPoll];
        bool have = true;
#pragma unroll
        for (int u = 0; u < kMaxPoll; ++u) {
          const int j = lane + u * kWave;
          slot[u] = j < G ? load_coherent(src + j) : ~0ull;
        }
#pragma unroll
        for (int u = 0; u < kMaxPoll; ++u) have = have && slot[u] != 0ull;
        if (__all(have)) {
#pragma unroll
          for (int u = 0; u < kMaxPoll; ++u) {
            const int j = lane + u * kWave;
            if (j < G) kk = umax64(kk, slot[u]);
          }
          break;
        }
        if (++spins > kSpinLimit) {
          if (lane == 0) __hip_atomic_store(p.ctl + kCtlWatchdog, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int u = 0; u < kMaxPoll; ++u) {
            const int j = lane + u * kWave;
            if (j < G) kk = umax64(kk, slot[u]);
          }
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      kk = row_max64(kk);
      kk = umax64(kk, __shfl_xor(kk, 16));
      kk = umax64(kk, __shfl_xor(kk, 32));
      if (lane == 0) {
        int tok = static_cast<int>(key_index(kk));
        if (tok < 0 || tok >= V) tok = 0;  // only if the watchdog fired
        prev_s[m] = tok;
        tok_s[step * kMaxReqs + m] = tok;
      }
    }
  }
  __syncthreads();  // workgroup 0: every poll of the final step is over, tok_s complete
  finish();
}

struct LoopPlan {
  int G, KB, RT, lds_tiles, bstride, base_in_lds;
  size_t lds;
};

constexpr size_t kBaseLdsMax = 64 * 1024;  // larger base slices are read straight from memory

int reg_tiles(int KB) { return KB <= 4 ? 4 : KB == 8 ? 3 : (KB == 16 ? 1 : 0); }

// Plan for G workgroups (G <= min(tiles, kMaxGroups)).
LoopPlan make_loop_plan(int R, int V, int r, int G) {
  LoopPlan pl{};
  const int tiles = (V + 15) / 16;
  pl.G = G;
  const int kb = (r + 31) / 32;
  pl.KB = kb <= 1 ? 1 : kb <= 2 ? 2 : kb <= 4 ? 4 : kb <= 8 ? 8 : kb <= 16 ? 16 : 32;
  pl.RT = reg_tiles(pl.KB);
  const int ntmax = (tiles + pl.G - 1) / pl.G;
  pl.bstride = ntmax * 16;
  const size_t base_bytes = static_cast<size_t>(R) * pl.bstride * 4;
  pl.base_in_lds = base_bytes <= kBaseLdsMax ? 1 : 0;
  const size_t fixed = static_cast<size_t>(kLoopWaves) * kMaxReqs * 8 + kMaxReqs * 4 +
                       static_cast<size_t>(kMaxSteps) * kMaxReqs * 4 + (pl.base_in_lds ? base_bytes : 0);
  const size_t tile_bytes = static_cast<size_t>(pl.KB) * 1024;
  const int want = std::max(0, ntmax - kLoopWaves * pl.RT);
  const int fit = fixed < kLdsBytes ? static_cast<int>((kLdsBytes - fixed) / tile_bytes) : 0;
  pl.lds_tiles = std::min(want, fit);
  pl.lds = pl.lds_tiles * tile_bytes + fixed;
  return pl;
}

template <int KB>
hipError_t launch_loop(MarkovParams& prm, const LoopPlan& pl, int cus, hipStream_t st) {
  constexpr int RT = KB <= 4 ? 4 : KB == 8 ? 3 : (KB == 16 ? 1 : 0);
  const void* fn = reinterpret_cast<const void*>(&markov_loop_kernel<KB, RT>);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (attr != hipSuccess) return attr;
  // Every workgroup must be resident at once (the steps exchange keys). A
  // cooperative launch would enforce that but costs ~17 us of extra launch
  // latency on MI355X, so the same condition is checked here instead: the
  // grid never exceeds one workgroup per CU times the per-CU occupancy.
  int per_cu = 0;
  const hipError_t oe = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kLoopThreads, pl.lds);
  if (oe != hipSuccess) return oe;
  if (per_cu < 1 || pl.G > per_cu * cus) return hipErrorCooperativeLaunchTooLarge;
  void* args[] = {&prm};
  return hipLaunchKernel(fn, dim3(pl.G), dim3(kLoopThreads), args, pl.lds, st);
}

}  // namespace

size_t markov_workspace_bytes(int num_reqs, int k, int V) {
  if (num_reqs < 1 || num_reqs > kMaxReqs || k < 1 || k > kMaxSteps || V < 1) return 0;
  return kCtlBytes + 2 * kSlotsPerBuffer * sizeof(uint64_t);  // one layout for every size
}

hipError_t launch_markov(const float* base, int R, int B, int V, const uint16_t* w1,
                         const uint16_t* w2, int r, const int64_t* d2t, const int64_t* prev0,
                         int k, int64_t* ids, void* workspace, hipStream_t stream) {
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorNoDevice;
  // Workgroups: one per CU, but at least ~16 tiles each. With fewer tiles a
  // workgroup's step is all latency, and more workgroups only lengthen the
  // exchange (measured: 32000 x 256 with 8 requests 74 -> 67 us per call at
  // 128 instead of 256 workgroups; 4096 x 32 17 -> 14 us at 16).
  const int tiles = (V + 15) / 16;
  const int G = std::max(1, std::min({cus, kMaxGroups, (tiles + 15) / 16}));
  const LoopPlan pl = make_loop_plan(R, V, r, G);
  MarkovParams prm{};
  prm.base = base;
  prm.w1 = w1;
  prm.w2 = w2;
  prm.prev0 = prev0;
  prm.d2t = d2t;
  prm.ids = ids;
  prm.ctl = static_cast<uint32_t*>(workspace);
  prm.slots = reinterpret_cast<uint64_t*>(static_cast<unsigned char*>(workspace) + kCtlBytes);
  prm.R = R;
  prm.B = B;
  prm.V = V;
  prm.r = r;
  prm.k = k;
  prm.G = pl.G;
  prm.tiles = tiles;
  prm.lds_tiles = pl.lds_tiles;
  prm.bstride = pl.bstride;
  prm.base_in_lds = pl.base_in_lds;
  switch (pl.KB) {
    case 1: return launch_loop<1>(prm, pl, cus, stream);
    case 2: return launch_loop<2>(prm, pl, cus, stream);
    case 4: return launch_loop<4>(prm, pl, cus, stream);
    case 8: return launch_loop<8>(prm, pl, cus, stream);
    case 16: return launch_loop<16>(prm, pl, cus, stream);
    default: return launch_loop<32>(prm, pl, cus, stream);
  }
}

}  // namespace dspark
