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
//    zero-filled once before first use.
//  * The polls are bounded. A poll that gives up (all workgroups resident is
//    checked on the host, but another stream's kernels could hold compute
//    units for longer than the bound) marks the workspace: that call's ids
//    are -2, and it leaves the sequence number and the slot counts alone,
//    so that a workgroup of it that starts late still sees the state every
//    other workgroup of the call saw. The next call finds the mark and
//    repairs the workspace instead of sampling: all of its workgroups clear
//    both slot buffers, its ids are -2 too, and workgroup 0 records the
//    repair together with the call's launch number. A workgroup that finds
//    a repair recorded under its own launch number is a late one of the
//    repairing launch (or a replay of the same captured launch): it only
//    clears and leaves. Every call after that samples normally, and the
//    first one that completes removes the repair record. No caller action
//    is needed.
//  * The round's lm_head (dspark_draft_round) takes its rows from a counter
//    word of this workspace and leaves it 0. A nonzero word at the start of
//    the loop means that lm_head started on a dirty counter (a workspace that
//    was never zero-filled) and left base rows out: that call's ids are -2,
//    workgroup 0 stores 0, and the next round is whole again.
//  * Nothing but the exchange sits on the per-step path of workgroup 0: the
//    drafted tokens stay in LDS and the ids (d2t applied) are written once,
//    after the last step.
//  * No floating-point atomics anywhere; results do not depend on timing.
#include "dspark_internal.h"

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

namespace dspark {
namespace {

constexpr int kMaxReqs = 16;
constexpr int kMaxSteps = 32;
constexpr int kMaxGroups = 256;          // grid cap: one workgroup per CU
// Waves per workgroup: 8 (two per SIMD) by default; 4 (one per SIMD, half
// of each SIMD's registers in AGPRs) when eight would leave markov_w2 tiles
// to be re-read from memory at every step: a single wave per SIMD may hold
// 10 tiles of r = 256 instead of 3.
constexpr int kLoopWavesMax = 8;
constexpr size_t kCtlBytes = 256;        // control words, then two slot buffers
constexpr size_t kSlotsPerBuffer = static_cast<size_t>(kMaxSteps) * kMaxReqs * kMaxGroups;
// Copies of every key slot: each workgroup publishes its key into all of
// them and polls the one of its own index modulo the copies, so the 256
// polling waves spread over that many separate memory regions instead of
// all reading the same few lines. A copy takes kCopyStride slots of a
// buffer; calls whose k * R * G slots do not fit use fewer copies.
// Measured on MI355X: 40.1 -> 39.0 us per call at the Qwen3-8B head, 119 ->
// 115 us at the 27B lane (polling two reads in flight, or re-reading only
// the empty slots, or longer sleeps between polls, did not help).
constexpr int kMaxRep = 8;
constexpr size_t kCopyStride = kSlotsPerBuffer / kMaxRep;

// Control words (uint32) at the start of the workspace.
constexpr int kCtlState = 0;       // kStateOk, kStateTimedOut (a poll gave up) or kStateRepaired
constexpr int kCtlSeq = 1;         // call sequence number; its parity selects the active slot buffer
constexpr int kCtlRepairedBy = 2;  // launch number of the call that repaired the workspace
constexpr int kCtlUsed = 4;        // [4 + b]: slots per copy the last call that used buffer b wrote
constexpr int kCtlReps = 6;        // [6 + b]: copies that call wrote
constexpr int kCtlLmCounter = 16;  // not used by the loop: the round's lm_head takes its units from here
constexpr uint32_t kStateOk = 0;
constexpr uint32_t kStateTimedOut = 1;  // any value but kStateOk and kStateRepaired is treated so
constexpr uint32_t kStateRepaired = 2;
constexpr size_t kLdsBytes = 160 * 1024;
constexpr uint32_t kDefaultSpinLimit = 1u << 18;  // ~0.3 s of polling: far beyond any legitimate wait
std::atomic<uint32_t> g_spin_limit{kDefaultSpinLimit};
std::atomic<uint32_t> g_launches{0};

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
  int nrep;              // copies of the key slots this call writes (1..kMaxRep)
  int lds_tiles;         // markov_w2 tiles held in LDS per workgroup
  int bstride;           // floats per request in the LDS base slice (>= 16 * tiles per workgroup)
  int base_in_lds;       // 0: base values are read straight from memory (slice too large)
  int probe_on;          // nonzero: also compute the confidence probe described by `probe`
  uint32_t nonce;        // launch number (never 0): tells a late workgroup of a repairing launch
  uint32_t spin_limit;   // polls before a grid-wide wait gives up
  uint32_t* lm_ticks;    // the round's split lm_head ticket words, set to 0 by every call (or null)
  int n_lm_ticks;
  ProbeArgs probe;
  // Q8_0 weights (the Q8 kernels): quants [V, r] and binary16 block scales [V, r / 32]
  const int8_t* w1q;
  const uint16_t* w1d;
  const int8_t* w2q;
  const uint16_t* w2d;
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

// One k-block (32 entries of the rank) of a lane's MFMA operand: 8 bf16
// values, or 8 int8 quants for Q8_0 weights.
template <bool Q8>
using Frag = std::conditional_t<Q8, uint2, u32x4>;

// Q8_0 block scales are kept in LDS as rows of an even number of halves
// (two per 32-bit word, so every word read is aligned).
constexpr int scale_row(int KB) { return 2 * ((KB + 1) / 2); }
// LDS bytes of one markov_w2 tile held in LDS: the fragments of KB k-blocks
// for 64 lanes, and with Q8_0 weights the 16 rows' block scales.
constexpr size_t lds_tile_bytes(int KB, bool Q8) {
  return static_cast<size_t>(KB) * kWave * (Q8 ? 8 : 16) + (Q8 ? static_cast<size_t>(16) * scale_row(KB) * 2 : 0);
}
// LDS bytes of the A block: R + 1 rows (padded by 16 bytes), then with Q8_0
// weights the rows' block scales (rounded up to 16 bytes).
constexpr size_t a_row_bytes(int KB, bool Q8) { return static_cast<size_t>(KB) * (Q8 ? 32 : 64) + 16; }
constexpr size_t a_block_bytes(int R, int KB, bool Q8) {
  return static_cast<size_t>(R + 1) * a_row_bytes(KB, Q8) +
         (Q8 ? (static_cast<size_t>(R + 1) * scale_row(KB) * 2 + 15) / 16 * 16 : 0);
}

__device__ __forceinline__ float half_lo(uint32_t v) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v))); }
__device__ __forceinline__ float half_hi(uint32_t v) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v >> 16))); }

// NV: request rows a lane's outputs can hold, 1 when there is a single
// request (R = 1), else 4.
template <int NW, int KB, int RT, int LT, bool BL, bool Q8, int NV = 4>
__global__ __launch_bounds__(NW * kWave) void markov_loop_kernel(MarkovParams p) {
  constexpr int kLoopThreads = NW * kWave;
  using BF = Frag<Q8>;
  constexpr int kSH = (KB + 1) / 2;  // packed scale pairs of a row (Q8)
  constexpr int kSR = 2 * kSH;       // halves per LDS scale row (Q8)
  extern __shared__ __align__(16) unsigned char smem[];
  BF* w2l = reinterpret_cast<BF*>(smem);                                               // [lds_tiles][KB][64]
  uint16_t* w2ls = reinterpret_cast<uint16_t*>(smem + static_cast<size_t>(p.lds_tiles) * KB * kWave * sizeof(BF));  // [lds_tiles][16][kSR] (Q8)
  uint64_t* keys_s = reinterpret_cast<uint64_t*>(smem + static_cast<size_t>(p.lds_tiles) * lds_tile_bytes(KB, Q8));  // [NW][16]
  // A block: R rows, then a zero row read by the lanes of absent requests
  // (with Q8_0 weights followed by the rows' block scales).
  constexpr int kARow = static_cast<int>(a_row_bytes(KB, Q8));
  unsigned char* a_lds = reinterpret_cast<unsigned char*>(keys_s + NW * kMaxReqs);       // [R + 1][kARow]
  uint16_t* a_sc = reinterpret_cast<uint16_t*>(a_lds + (p.R + 1) * kARow);              // [R + 1][kSR] (Q8)
  int* prev_s = reinterpret_cast<int*>(a_lds + a_block_bytes(p.R, KB, Q8));            // [16] prev0 (valid or 0)
  int* tok_s = prev_s + kMaxReqs;                                                       // [k][R] drafted tokens
  float* basel = reinterpret_cast<float*>(tok_s + p.k * p.R);                           // [R][bstride]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int R = p.R, V = p.V, r = p.r, G = p.G;
  const int t0 = static_cast<int>((static_cast<long long>(blockIdx.x) * p.tiles) / G);
  const int t1 = static_cast<int>((static_cast<long long>(blockIdx.x + 1) * p.tiles) / G);
  const int nt = t1 - t0;
  const int nreg = min(nt, NW * RT);
  const int nheld = nreg + min(nt - nreg, p.lds_tiles);
  // Active slot buffer of this call and the workspace state (issued first:
  // the replies arrive while markov_w2 loads).
  const uint32_t seq = load_coherent(p.ctl + kCtlSeq);
  const uint32_t state = load_coherent(p.ctl + kCtlState);
  const uint32_t repaired_by = load_coherent(p.ctl + kCtlRepairedBy);
  // The round's lm_head counter (dspark_draft_round): a clean lm_head leaves
  // it 0, so a nonzero word means that lm_head ran on a counter that was not
  // (the workspace was never zero-filled) and some base rows are missing.
  const uint32_t lm_counter = load_coherent(p.ctl + kCtlLmCounter);
  // The round's split lm_head (more than 16 rows) has finished, and the next
  // one starts after this launch: its ticket words are set to 0 here, so a
  // word that was not (a workspace never zero-filled) spoils one round at
  // most. A clean lm_head has already left them 0.
  if (tid == 0)
    for (int e = static_cast<int>(blockIdx.x); e < p.n_lm_ticks; e += G)
      __hip_atomic_store(p.lm_ticks + e, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // kStateRepaired under this launch's number: a late workgroup of the
  // repairing launch, or a replay of that captured launch.
  const bool repair = !(state == kStateOk || (state == kStateRepaired && repaired_by != p.nonce));

  auto w2_row = [&](int j, int lrow) {
    const int row = min((t0 + j) * 16 + lrow, V - 1);
    return p.w2 + static_cast<size_t>(row) * r;
  };
  const int KBr = r / 32;  // Q8_0 blocks per row
  auto w2q_row = [&](int j, int lrow) {
    const int row = min((t0 + j) * 16 + lrow, V - 1);
    return p.w2q + static_cast<size_t>(row) * r;
  };
  auto w2d_row = [&](int j, int lrow) {
    const int row = min((t0 + j) * 16 + lrow, V - 1);
    return p.w2d + static_cast<size_t>(row) * KBr;
  };
  // Lane fragment of k-block kb of tile j (row = 16 (t0 + j) + i, entries
  // 32 kb + 8 g .. + 7), zeros past the rank.
  auto frag_of = [&](int j, int kb, int lrow, int lg) -> BF {
    if constexpr (Q8) {
      return kb * 32 + 8 * lg < r ? *reinterpret_cast<const uint2*>(w2q_row(j, lrow) + kb * 32 + 8 * lg) : uint2{0u, 0u};
    } else {
      return kb * 32 + 8 * lg < r ? load16(w2_row(j, lrow) + kb * 32 + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // Q8_0: the block scales of row lrow of tile j, two per word (zeros past the rank).
  auto scales_of = [&](int j, int lrow, uint32_t (&sc)[kSH]) {
    const uint16_t* sd = w2d_row(j, lrow);
#pragma unroll
    for (int h = 0; h < kSH; ++h) {
      const uint32_t lo = 2 * h < KBr ? sd[2 * h] : 0u, hi = 2 * h + 1 < KBr ? sd[2 * h + 1] : 0u;
      sc[h] = lo | (hi << 16);
    }
  };

  // ---- load this workgroup's markov_w2 tiles once: registers, then LDS
  BF wreg[RT > 0 ? RT : 1][KB];
  uint32_t wsc[Q8 && RT > 0 ? RT : 1][Q8 ? kSH : 1];  // Q8_0: block scales of the register tiles
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    const int j = w + NW * u;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) wreg[u][kb] = j < nreg ? frag_of(j, kb, i, g) : BF{};
    if constexpr (Q8) {
      scales_of(j, i, wsc[u]);
      if (j >= nreg)
#pragma unroll
        for (int h = 0; h < kSH; ++h) wsc[u][h] = 0u;
    }
  }
  // LDS tiles: eight loads per thread in flight at a time, then their LDS
  // writes (one load and write after the other would serialize the latency).
  {
    constexpr int kBatch = 16;
    const int nl = (nheld - nreg) * KB * kWave;
    for (int e0 = 0; e0 < nl; e0 += kBatch * kLoopThreads) {
      BF v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = min(e0 + u * kLoopThreads + tid, nl - 1);
        const int ln = e & 63, kb = (e >> 6) % KB, jj = (e >> 6) / KB;
        const int gg = ln >> 4;
        // (lanes past r read column 0 and store zeros: straight code)
        const bool kok = kb * 32 + 8 * gg < r;
        if constexpr (Q8) {
          v[u] = *reinterpret_cast<const uint2*>(w2q_row(nreg + jj, ln & 15) + (kok ? kb * 32 + 8 * gg : 0));
          v[u] = kok ? v[u] : uint2{0u, 0u};
        } else {
          v[u] = load16(w2_row(nreg + jj, ln & 15) + (kok ? kb * 32 + 8 * gg : 0));
          v[u] = kok ? v[u] : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = e0 + u * kLoopThreads + tid;
        if (e < nl) w2l[e] = v[u];
      }
    }
    if constexpr (Q8) {  // the LDS tiles' block scales: [tile][row][kSR]
      const int ns = (nheld - nreg) * 16 * kSR;
      for (int e = tid; e < ns; e += kLoopThreads) {
        const int kb = e % kSR, row = (e / kSR) % 16, jj = e / (16 * kSR);
        w2ls[e] = kb < KBr ? w2d_row(nreg + jj, row)[kb] : static_cast<uint16_t>(0);
      }
    }
  }
  if (tid < R) prev_s[tid] = prev0_ok(p, tid) ? static_cast<int>(p.prev0[tid]) : 0;

  const int cur = static_cast<int>(seq & 1u);
  uint64_t* part = p.slots + cur * kSlotsPerBuffer;
  const uint32_t used_other = load_coherent(p.ctl + kCtlUsed + (cur ^ 1));
  const uint32_t reps_other = load_coherent(p.ctl + kCtlReps + (cur ^ 1));
  // Clears what the previous call left in the other buffer (which the next
  // call uses), shared by the workgroups that finish early: all but 0, or 0
  // alone. These stores stay out of the step loop: a store in flight would
  // make a wave drain its outstanding loads before it may use any of them.
  auto clear_other = [&]() {
    uint64_t* other = p.slots + (cur ^ 1) * kSlotsPerBuffer;
    const uint32_t reps = min(max(reps_other, 1u), static_cast<uint32_t>(kMaxRep));
    const uint32_t used = min(used_other, static_cast<uint32_t>(reps > 1 ? kCopyStride : kSlotsPerBuffer));
    const uint32_t nwg = G > 1 ? G - 1 : 1, wg = G > 1 ? blockIdx.x - 1 : 0;
    for (uint32_t e = wg * kLoopThreads + tid; e < used * reps; e += nwg * kLoopThreads) {
      const uint32_t c = e / used, o = e - c * used;
      __hip_atomic_store(other + c * kCopyStride + o, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // Workgroup 0 after the last step (every other workgroup has published
  // every step, so none reads a slot any more): the ids of all steps, the
  // slots used, and the next sequence number. When a poll of this call gave
  // up, every id is -2 and the state stays as it is (the next call repairs).
  auto finish = [&]() {
    if (G == 1) clear_other();
    const bool timed_out = load_coherent(p.ctl + kCtlState) == kStateTimedOut;
    const bool bad = timed_out || lm_counter != 0u;
    if (tid == 0 && lm_counter != 0u)  // this call's ids are -2; the next round starts clean
      __hip_atomic_store(p.ctl + kCtlLmCounter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int e = tid; e < R * p.k; e += kLoopThreads) {
      const int m = e / p.k, st = e - m * p.k;
      int64_t id = -1;
      if (prev0_ok(p, m)) {  // tok_s holds this call's tokens (each in [0, V))
        const int tok = tok_s[st * R + m];
        id = p.d2t ? p.d2t[tok] : static_cast<int64_t>(tok);
      }
      p.ids[e] = bad ? -2 : id;
    }
    if (tid == 0 && !timed_out) {
      __hip_atomic_store(p.ctl + kCtlUsed + cur, static_cast<uint32_t>(p.k * R * G), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctl + kCtlReps + cur, static_cast<uint32_t>(p.nrep), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctl + kCtlSeq, seq + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (state == kStateRepaired)
        __hip_atomic_store(p.ctl + kCtlState, kStateOk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // A call that finds the workspace marked: every workgroup clears its
  // share of both slot buffers; workgroup 0 writes -2 ids and records the
  // repair (or, for a late workgroup's launch, drops the record).
  auto repair_workspace = [&]() {
    constexpr size_t kAll = 2 * kSlotsPerBuffer;
    for (size_t e = static_cast<size_t>(blockIdx.x) * kLoopThreads + tid; e < kAll;
         e += static_cast<size_t>(G) * kLoopThreads)
      __hip_atomic_store(p.slots + e, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x != 0) return;
    for (int e = tid; e < R * p.k; e += kLoopThreads) p.ids[e] = -2;
    if (tid == 0) {
      __hip_atomic_store(p.ctl + kCtlLmCounter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (state == kStateRepaired) {
        __hip_atomic_store(p.ctl + kCtlRepairedBy, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        __hip_atomic_store(p.ctl + kCtlUsed + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ctl + kCtlUsed + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ctl + kCtlReps + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ctl + kCtlReps + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ctl + kCtlRepairedBy, p.nonce, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ctl + kCtlState, kStateRepaired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };

  // ---- base values of this workgroup's slice, staged in LDS per step by
  // the stager threads: during the exchange, by the waves that do not poll
  // (w >= R), or after the polls when every wave polls (R >= waves). Loads
  // first, then the LDS writes, so a thread's loads are in flight together.
  const int nb = BL ? R * nt * 16 : 0;
  const int stage_w0 = R < NW ? R : 0;
  const int sthreads = (NW - stage_w0) * kWave;
  const int stid = tid - stage_w0 * kWave;  // < 0: not a stager
  constexpr int kPre = 4;
  float sv[kPre];
  // (the thread index is made opaque per call, so the slice addresses are
  // recomputed here rather than held in registers across the whole step)
  auto stage_fetch = [&](int st) {
    if (!BL || stid < 0) return;
    int so = stid;
    asm volatile("" : "+v"(so));
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int e = so + u * sthreads;
      const int m = e < nb ? e / (nt * 16) : 0, n = t0 * 16 + (e - m * (nt * 16));
      // (always issued, to entry 0 for an unused slot: straight code)
      sv[u] = p.base[e < nb && n < V ? (static_cast<size_t>(m) * p.B + st) * V + n : 0];
    }
  };
  auto stage_store = [&](int st) {
    if (!BL || stid < 0) return;
    int so = stid;
    asm volatile("" : "+v"(so));
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int e = so + u * sthreads;
      const int m = e / (nt * 16);
      if (e < nb) basel[m * p.bstride + (e - m * (nt * 16))] = sv[u];
    }
    for (int e = so + kPre * sthreads; e < nb; e += sthreads) {  // large slices only
      const int m = e / (nt * 16), n = t0 * 16 + (e - m * (nt * 16));
      basel[m * p.bstride + (e - m * (nt * 16))] = n < V ? p.base[(static_cast<size_t>(m) * p.B + st) * V + n] : 0.f;
    }
  };

  // ---- the A operand of the next step, in LDS: row m holds markov_w1[prev]
  // of request m (rows padded by 16 bytes, so the fragment reads of the 16
  // rows fall in different banks). A polling wave gathers its request's row
  // as soon as it knows the token (r <= 1024: at most two 16-byte loads per
  // lane); the LDS writes follow once the stagers' loads are out too.
  // (Q8_0: the row's quants, r bytes, and its r / 32 block scales.)
  constexpr int kRowChunks = Q8 ? 1 : 2;  // 16-byte loads per lane (r <= 1024)
  const int nchunk = Q8 ? r / 16 : r / 8;  // 16-byte chunks of a row
  auto gather_fetch = [&](int tok, u32x4 (&gv)[2], uint32_t& gs) {
    const unsigned char* src = Q8 ? reinterpret_cast<const unsigned char*>(p.w1q + static_cast<size_t>(tok) * r)
                                  : reinterpret_cast<const unsigned char*>(p.w1 + static_cast<size_t>(tok) * r);
#pragma unroll
    for (int q = 0; q < kRowChunks; ++q) {
      const int c = lane + q * kWave;  // 16-byte chunk of the row
      gv[q] = load16(src + 16 * (c < nchunk ? c : 0));
    }
    gs = 0u;
    if constexpr (Q8) gs = p.w1d[static_cast<size_t>(tok) * KBr + (lane < KBr ? lane : 0)];
  };
  auto gather_store = [&](int m, const u32x4 (&gv)[2], uint32_t gs) {
#pragma unroll
    for (int q = 0; q < kRowChunks; ++q) {
      const int c = lane + q * kWave;
      if (c < nchunk) *reinterpret_cast<u32x4*>(a_lds + m * kARow + 16 * c) = gv[q];
    }
    if constexpr (Q8)
      if (lane < KBr) a_sc[m * kSR + lane] = static_cast<uint16_t>(gs);
  };

  // The confidence probe, when asked for: it depends on nothing the loop
  // computes, so it runs on the workgroups that are otherwise idle at the
  // end, those that leave after publishing the last step (all but
  // workgroup 0, or workgroup 0 alone when it is the only one). Each row
  // goes to four waves, which compute its four chains exactly as the
  // standalone probe kernel does, so the logits are the same bits. Called
  // by whole workgroups only (it has barriers); the chain totals go to
  // prev_s, which nothing reads after the prologue.
  auto probe_rows = [&]() {
    if (!p.probe_on) return;
    const ProbeArgs& a = p.probe;
    constexpr int kRowsPerWg = NW / 4;
    const int wg = G > 1 ? static_cast<int>(blockIdx.x) - 1 : 0, nwg = G > 1 ? G - 1 : 1;
    float* ctot = reinterpret_cast<float*>(prev_s);
    __syncthreads();
    for (int m0 = wg * kRowsPerWg; m0 < a.M; m0 += nwg * kRowsPerWg) {
      const int m = m0 + w / 4;
      const float c = m < a.M ? probe_chain<4>(a.x + static_cast<size_t>(m) * a.D, a.D, a.w, lane, w & 3) : 0.f;
      if (lane == 0) ctot[w] = c;
      __syncthreads();
      if (tid < kRowsPerWg && m0 + tid < a.M) {
        const float l = probe_logit(ctot + 4 * tid, a.bias);
        a.logit[m0 + tid] = l;
        if (a.pass) a.pass[m0 + tid] = l >= a.threshold ? 1 : 0;
      }
      __syncthreads();
    }
  };

  if (repair) {  // an earlier call gave up: repair the workspace, sample nothing
    repair_workspace();
    if (blockIdx.x != 0 || G == 1) probe_rows();
    return;
  }

  // Prologue: zero the A block (columns past r stay zero: the markov_w2
  // fragments are zero there too, and uninitialized LDS could hold NaNs),
  // then the rows of step 0 and the base slice of step 0.
  for (int e = tid; e < static_cast<int>(a_block_bytes(R, KB, Q8) / 16); e += kLoopThreads)
    reinterpret_cast<u32x4*>(a_lds)[e] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  for (int m = w; m < R; m += NW) {
    u32x4 gv[2];
    uint32_t gs;
    gather_fetch(prev_s[m], gv, gs);
    gather_store(m, gv, gs);
  }
  stage_fetch(0);
  stage_store(0);
  __syncthreads();

  for (int step = 0; step < p.k; ++step) {
    const bool last = step == p.k - 1;
    // Lane coordinates made opaque once per step, so the compiler recomputes
    // the addresses derived from them (a few VALU ops) instead of keeping
    // dozens of loop-invariant addresses live next to the register tiles.
    int ll = lane;
    asm volatile("" : "+v"(ll));
    const int li = ll & 15, lg = ll >> 4;

    // Scores of tile j: lane (i, g) holds rows m = 4g..4g+3 at column
    // n = 16 (t0 + j) + i. Branch-free: the four base values are read at
    // once (clamped to a valid entry) and a key counts only where the tile,
    // the request and the column exist.
    uint64_t best[4] = {0, 0, 0, 0};
    auto score = [&](int j, bool tile_ok, f32x4 acc) {
      const int jj = tile_ok ? j : 0;
      const int n = (t0 + jj) * 16 + li;
      // (a single request: only row 0 of each lane group exists)
      float bv[4];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int m = min(4 * lg + v, R - 1);
        bv[v] = BL ? basel[m * p.bstride + jj * 16 + li]
                   : p.base[(static_cast<size_t>(m) * p.B + step) * V + min(n, V - 1)];
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint64_t key = score_key(bv[v] + acc[v], static_cast<uint32_t>(n));
        const bool ok = tile_ok && 4 * lg + v < R && n < V;
        best[v] = ok && key > best[v] ? key : best[v];
      }
    };
    // A fragment kb of this lane: k = 32*kb + 8*g + (0..7) of row i, read
    // from LDS where it is needed (it feeds every tile of the k-block).
    const BF* a_frag = reinterpret_cast<const BF*>(a_lds + min(li, R) * kARow + sizeof(BF) * lg);  // + 4*kb
    // Q8_0: the block scales of the A rows of this lane's outputs (rows
    // 4 lg + v; past R the zero row): up to 8 blocks held in registers, two
    // per word, read once per step; longer rows read them per k-block.
    constexpr bool kAscReg = Q8 && KB <= 8;
    uint32_t asc[kAscReg ? NV : 1][kAscReg ? kSH : 1];
    if constexpr (kAscReg) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int h = 0; h < kSH; ++h)
          asc[v][h] = reinterpret_cast<const uint32_t*>(a_sc + min(4 * lg + v, R) * kSR)[h];
    }
    auto a_scales = [&](int kb, float (&s1)[4]) {
      if constexpr (kAscReg) {
#pragma unroll
        for (int v = 0; v < NV; ++v) s1[v] = (kb & 1) ? half_hi(asc[v][kb >> 1]) : half_lo(asc[v][kb >> 1]);
      } else if constexpr (Q8) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
          s1[v] = static_cast<float>(__builtin_bit_cast(_Float16, a_sc[min(4 * lg + v, R) * kSR + kb]));
      }
    };
    // One k-block of a tile into its accumulator. bf16: an MFMA chain.
    // Q8_0: the block's exact integer dot products (int8 MFMA), then scaled
    // by the A row's and the tile row's block scales and added in fp32, for
    // the NV request rows a lane's outputs can hold. The two halves are separate so that a k-block's
    // MFMAs for all tiles go out before any of their results is scaled.
    auto mma8 = [&](BF a, BF b) -> i32x4 {
      if constexpr (Q8) {
        return __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b),
                                                     i32x4{0, 0, 0, 0}, 0, 0, 0);
      } else {
        (void)a;
        (void)b;
        return i32x4{0, 0, 0, 0};
      }
    };
    auto scale_add = [&](f32x4& acc, i32x4 d, const uint32_t* bsc, int kb, const float (&s1)[4]) {
      const float s2 = (kb & 1) ? half_hi(bsc[kb >> 1]) : half_lo(bsc[kb >> 1]);
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = __builtin_fmaf(static_cast<float>(d[v]), s1[v] * s2, acc[v]);
    };
    auto mac = [&](f32x4& acc, BF a, BF b, const uint32_t* bsc, int kb, const float (&s1)[4]) {
      if constexpr (Q8) {
        scale_add(acc, mma8(a, b), bsc, kb, s1);
      } else {
        (void)bsc;
        (void)s1;
        acc = mfma_16x16x32(a, b, acc);
      }
    };

    // The first tile of this wave beyond on-chip capacity, if any (one wave
    // per SIMD only): its fragments are loaded before the on-chip tiles are
    // computed, so their memory round trip overlaps that work (a single
    // request: with four rows per lane the registers spill). (frag_of
    // clamps the row, so a wave without such a tile loads a valid row it
    // never uses.)
    constexpr bool kStreamPre = NW == 4 && !Q8 && NV == 1;
    const int js0 = nheld + (((nreg + w - nheld) % NW) + NW) % NW;
    BF spre[kStreamPre ? KB : 1];
    if constexpr (kStreamPre) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) spre[kb] = frag_of(js0, kb, li, lg);
    }

    // The scores of every tile of this workgroup.
    {
    // Register tiles and the wave's first LT LDS tiles, all accumulation
    // chains interleaved per k-block, so one chain's MFMAs overlap the
    // others' latency and the LDS reads of a k-block go out together. An
    // absent tile computes on zeros (or on LDS tile 0) and is not scored.
    // With many register tiles (one wave per SIMD) they go in two passes,
    // which halves the accumulators held at once; LT LDS tiles ride along
    // with each pass (other tiles in each), so that four waves keep LDS
    // tiles in interleaved chains too.
    constexpr int RG = RT > 6 ? (RT + 1) / 2 : (RT > 0 ? RT : 1);  // register tiles per pass
    constexpr int NPASS = RT > 0 ? (RT + RG - 1) / RG : 1;
#pragma unroll
    for (int u0 = 0; u0 < (RT > 0 ? RT : 1); u0 += RG) {
      constexpr int L1 = LT;
      constexpr int L1A = LT > 0 ? LT : 1;  // (array sizes)
      const int pass = u0 / RG;
      const bool first = true;  // (every pass carries its LDS tiles)
      f32x4 accr[RG], accl[L1A];
      int jl[L1A];
      const BF* srcl[L1A];
      uint32_t lsc[L1A][Q8 ? kSH : 1];  // Q8_0: block scales of those LDS tiles (row li)
#pragma unroll
      for (int t = 0; t < L1; ++t) {
        jl[t] = nreg + w + NW * (LT * pass + t);
        const int lt = jl[t] < nheld ? jl[t] - nreg : 0;
        srcl[t] = w2l + static_cast<size_t>(lt) * KB * kWave + ll;
        accl[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (Q8) {
          if (first)
#pragma unroll
            for (int h = 0; h < kSH; ++h)
              lsc[t][h] = reinterpret_cast<const uint32_t*>(w2ls + (static_cast<size_t>(lt) * 16 + li) * kSR)[h];
        }
      }
#pragma unroll
      for (int u = 0; u < RG; ++u) accr[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const BF a = a_frag[4 * kb];
        float s1[4];
        a_scales(kb, s1);
        BF bl[L1A];
        if (first)
#pragma unroll
          for (int t = 0; t < L1; ++t) bl[t] = srcl[t][kb * kWave];
        if constexpr (Q8) {
          i32x4 dr[RG], dl[L1A];
#pragma unroll
          for (int u = 0; u < RG; ++u)
            if (RT > 0 && u0 + u < RT) dr[u] = mma8(a, wreg[u0 + u < RT ? u0 + u : 0][kb]);
          if (first)
#pragma unroll
            for (int t = 0; t < L1; ++t) dl[t] = mma8(a, bl[t]);
#pragma unroll
          for (int u = 0; u < RG; ++u)
            if (RT > 0 && u0 + u < RT) scale_add(accr[u], dr[u], wsc[u0 + u < RT ? u0 + u : 0], kb, s1);
          if (first)
#pragma unroll
            for (int t = 0; t < L1; ++t) scale_add(accl[t], dl[t], lsc[t], kb, s1);
        } else {
#pragma unroll
          for (int u = 0; u < RG; ++u)
            if (RT > 0 && u0 + u < RT) mac(accr[u], a, wreg[u0 + u < RT ? u0 + u : 0][kb], wsc[0], kb, s1);
          if (first)
#pragma unroll
            for (int t = 0; t < L1; ++t) mac(accl[t], a, bl[t], lsc[t], kb, s1);
        }
        // (one wave per SIMD: keep each k-block's fragment reads next to its
        // MFMAs, so that they do not pile up in registers ahead of them)
        if (NW == 4 && (kb & 1)) __builtin_amdgcn_sched_barrier(0);
        // (Q8_0: one k-block at a time, its MFMAs ahead of their scaling;
        // loads of later k-blocks may not pile up ahead of them)
        if (Q8) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < RG; ++u)
        if (RT > 0 && u0 + u < RT) score(w + NW * (u0 + u), w + NW * (u0 + u) < nreg, accr[u]);
      if (first)
#pragma unroll
        for (int t = 0; t < L1; ++t) score(jl[t], jl[t] < nheld, accl[t]);
    }
    // Further LDS tiles of this wave, if any, FG at a time: their MFMA chains
    // interleaved per k-block (a group's missing tiles compute on LDS tile 0
    // and are not scored). One chain at a time leaves each MFMA waiting on
    // the one before it. Pairs with eight waves (the Q8_0 27B-lane loop:
    // 117 -> 114 us); with four waves and ten register tiles a pair spills
    // (the bf16 27B-lane loop: 112 -> 126 us), so those go one at a time.
    constexpr int FG = NW == 4 ? 1 : 2;
    for (int j0 = nreg + w + NW * LT * NPASS; j0 < nheld; j0 += NW * FG) {
      const BF* srcf[FG];
      uint32_t scf[FG][Q8 ? kSH : 1];
      f32x4 accf[FG];
#pragma unroll
      for (int f = 0; f < FG; ++f) {
        const int j = j0 + NW * f;
        const int lt = j < nheld ? j - nreg : 0;
        srcf[f] = w2l + static_cast<size_t>(lt) * KB * kWave + ll;
        accf[f] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (Q8)
#pragma unroll
          for (int h = 0; h < kSH; ++h)
            scf[f][h] = reinterpret_cast<const uint32_t*>(w2ls + (static_cast<size_t>(lt) * 16 + li) * kSR)[h];
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float s1[4];
        a_scales(kb, s1);
        BF bf[FG];
#pragma unroll
        for (int f = 0; f < FG; ++f) bf[f] = srcf[f][kb * kWave];
#pragma unroll
        for (int f = 0; f < FG; ++f) mac(accf[f], a_frag[4 * kb], bf[f], scf[f], kb, s1);
      }
#pragma unroll
      for (int f = 0; f < FG; ++f) score(j0 + NW * f, j0 + NW * f < nheld, accf[f]);
    }
    // Tiles beyond on-chip capacity are read from memory at every step.
    for (int j = js0; j < nt; j += NW) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      uint32_t sc1[Q8 ? kSH : 1];
      if constexpr (Q8) scales_of(j, li, sc1);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float s1[4];
        a_scales(kb, s1);
        mac(acc, a_frag[4 * kb], kStreamPre && j == js0 ? spre[kStreamPre ? kb : 0] : frag_of(j, kb, li, lg), sc1, kb, s1);
      }
      score(j, true, acc);
    }

    }

    // ---- workgroup maximum per request (lanes of a 16-lane group share requests 4g..4g+3)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v >= R) break;
      best[v] = row_max64(best[v]);
    }
    if (i == 0)
#pragma unroll
      for (int v = 0; v < 4; ++v) keys_s[w * kMaxReqs + 4 * g + v] = best[v];
    __syncthreads();  // keys complete; every wave is done with this step's A block and base slice

    // ---- publish this workgroup's key of every request, into every copy
    if (tid < R * p.nrep) {
      const int m = tid % R, c = tid / R;
      uint64_t kk = keys_s[m];
      for (int ww = 1; ww < NW; ++ww) kk = umax64(kk, keys_s[ww * kMaxReqs + m]);
      __hip_atomic_store(part + c * kCopyStride + (static_cast<size_t>(step) * R + m) * G + blockIdx.x, kk,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (last && blockIdx.x != 0) {  // only workgroup 0 needs the final step's winner
      clear_other();
      probe_rows();
      return;
    }
    // The next step's base slice: waves that do not poll fetch and store it
    // while the pollers wait; when every wave polls, the loads go out before
    // the polls (so they arrive during them) and the stores follow the polls.
    if (!last) stage_fetch(step + 1);
    if (!last && stage_w0 > 0) stage_store(step + 1);

    // ---- exchange: poll the G slots of each request until all are published;
    // the winner's markov_w1 row is the next step's A row (wave w polls
    // request w, and then w + NW, ..., whose rows go to LDS at once)
    u32x4 gv[2];
    uint32_t gs = 0u;
#pragma unroll 1
    for (int h = 0; h < kMaxReqs / NW; ++h) {
      const int m = w + h * NW;
      if (m >= R) break;
      const uint64_t* src = part + (blockIdx.x % p.nrep) * kCopyStride + (static_cast<size_t>(step) * R + m) * G;
      uint64_t kk = 0;
      uint32_t spins = 0;
      uint64_t slot[kMaxPoll];
      for (;;) {
        bool have = true;
#pragma unroll
        for (int u = 0; u < kMaxPoll; ++u) {
          const int j = ll + u * kWave;
          slot[u] = j < G ? load_coherent(src + j) : ~0ull;
        }
#pragma unroll
        for (int u = 0; u < kMaxPoll; ++u) have = have && slot[u] != 0ull;
        if (__all(have)) break;
        if (++spins > p.spin_limit) {
          // Mark the workspace; the fence makes the mark visible before any
          // later key of this workgroup, so workgroup 0, which sees those
          // keys, sees the mark when it writes the ids.
          if (lane == 0)
            __hip_atomic_store(p.ctl + kCtlState, kStateTimedOut, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int u = 0; u < kMaxPoll; ++u) {
        const int j = lane + u * kWave;
        if (j < G) kk = umax64(kk, slot[u]);
      }
      kk = row_max64(kk);
      kk = umax64(kk, __shfl_xor(kk, 16));
      kk = umax64(kk, __shfl_xor(kk, 32));
      int tok = static_cast<int>(key_index(kk));
      if (tok < 0 || tok >= V) tok = 0;  // only if a poll gave up
      if (lane == 0) tok_s[step * R + m] = tok;
      if (!last && h == 0) gather_fetch(tok, gv, gs);
      if (!last && h > 0) {
        u32x4 gv1[2];
        uint32_t gs1;
        gather_fetch(tok, gv1, gs1);
        gather_store(m, gv1, gs1);
      }
    }
    if (!last) {
      if (w < R) gather_store(w, gv, gs);
      if (stage_w0 == 0) stage_store(step + 1);
    }
    __syncthreads();  // the next step's A block and base slice are in LDS (and tok_s complete)
  }
  finish();
  if (G == 1) probe_rows();
}

struct LoopPlan {
  int G, NW, KB, RT, lds_tiles, bstride, base_in_lds;
  size_t lds;
  bool streams;  // some tiles are re-read from memory at every step
};

constexpr size_t kBaseLdsMax = 64 * 1024;  // larger base slices are read straight from memory

// markov_w2 tiles held in registers per wave (the largest counts that leave
// no register spills; one wave per SIMD is built for bf16 at r = 256 only).
// A Q8_0 tile takes half the registers of a bf16 one, plus its scales.
// (One wave per SIMD holds 11 tiles only with the base read straight from
// memory in the scoring, which made the 27B-lane loop 115 -> 167 us; with the
// base slice in LDS the eleventh tile spills.)
constexpr int reg_tiles(int NW, int KB, bool Q8, bool BL = true) {
  if (Q8) return NW != 8 ? 0 : KB <= 2 ? 6 : KB == 4 ? 5 : KB == 8 ? (BL ? 3 : 1) : KB == 16 ? 1 : 0;
  return NW == 4 ? (KB == 8 ? 10 : 0) : KB <= 4 ? 4 : KB == 8 ? 3 : (KB == 16 ? 1 : 0);
}

// Plan for G workgroups (G <= min(tiles, kMaxGroups)) of NW waves.
LoopPlan make_loop_plan(int R, int V, int r, int k, int G, int NW, bool q8) {
  LoopPlan pl{};
  const int tiles = (V + 15) / 16;
  pl.G = G;
  pl.NW = NW;
  const int kb = (r + 31) / 32;
  pl.KB = kb <= 1 ? 1 : kb <= 2 ? 2 : kb <= 4 ? 4 : kb <= 8 ? 8 : kb <= 16 ? 16 : 32;
  const int ntmax = (tiles + pl.G - 1) / pl.G;
  pl.bstride = ntmax * 16;
  const size_t base_bytes = static_cast<size_t>(R) * pl.bstride * 4;
  pl.base_in_lds = base_bytes <= kBaseLdsMax ? 1 : 0;
  pl.RT = reg_tiles(NW, pl.KB, q8, pl.base_in_lds != 0);
  const size_t fixed = static_cast<size_t>(NW) * kMaxReqs * 8 + a_block_bytes(R, pl.KB, q8) + kMaxReqs * 4 +
                       static_cast<size_t>(k) * R * 4 + (pl.base_in_lds ? base_bytes : 0);
  const size_t tile_bytes = lds_tile_bytes(pl.KB, q8);
  const int want = std::max(0, ntmax - NW * pl.RT);
  const int fit = fixed < kLdsBytes ? static_cast<int>((kLdsBytes - fixed) / tile_bytes) : 0;
  pl.lds_tiles = std::min(want, fit);
  pl.lds = pl.lds_tiles * tile_bytes + fixed;
  pl.streams = want > fit;
  return pl;
}

template <int NW, int KB, bool BL, bool Q8, int NV, int LT>
hipError_t launch_loop_lt(MarkovParams& prm, const LoopPlan& pl, int cus, hipStream_t st) {
  constexpr int RT = reg_tiles(NW, KB, Q8, BL);
  constexpr int kLoopThreads = NW * kWave;
  const void* fn = reinterpret_cast<const void*>(&markov_loop_kernel<NW, KB, RT, LT, BL, Q8, NV>);
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

// LT: LDS tiles of a wave that ride in the register tiles' MFMA chains. When
// every tile of a workgroup is in registers (small vocabularies, the batched
// lane) there are none, and LT = 0 drops the two chains that would otherwise
// run on a stand-in tile at every step.
template <int NW, int KB, bool BL, bool Q8, int NV = 4>
hipError_t launch_loop(MarkovParams& prm, const LoopPlan& pl, int cus, hipStream_t st) {
  if (pl.lds_tiles == 0) return launch_loop_lt<NW, KB, BL, Q8, NV, 0>(prm, pl, cus, st);
  return launch_loop_lt<NW, KB, BL, Q8, NV, (KB >= 16 ? 1 : 2)>(prm, pl, cus, st);
}

template <bool Q8>
hipError_t dispatch_loop(MarkovParams& prm, const LoopPlan& pl, int cus, hipStream_t st) {
  const bool bl = pl.base_in_lds != 0;
  if constexpr (Q8) {
    // Q8_0 weights: r <= 256 (at 512 and more the block scales of the A rows
    // and the int8 products do not fit beside the tiles without spills);
    // a single request scales one output row per lane instead of four.
    if (prm.R == 1) {
      switch (pl.KB) {
        case 1: return bl ? launch_loop<8, 1, true, true, 1>(prm, pl, cus, st) : launch_loop<8, 1, false, true, 1>(prm, pl, cus, st);
        case 2: return bl ? launch_loop<8, 2, true, true, 1>(prm, pl, cus, st) : launch_loop<8, 2, false, true, 1>(prm, pl, cus, st);
        case 4: return bl ? launch_loop<8, 4, true, true, 1>(prm, pl, cus, st) : launch_loop<8, 4, false, true, 1>(prm, pl, cus, st);
        case 8: return bl ? launch_loop<8, 8, true, true, 1>(prm, pl, cus, st) : launch_loop<8, 8, false, true, 1>(prm, pl, cus, st);
        default: return hipErrorInvalidValue;
      }
    }
    switch (pl.KB) {
      case 1: return bl ? launch_loop<8, 1, true, true>(prm, pl, cus, st) : launch_loop<8, 1, false, true>(prm, pl, cus, st);
      case 2: return bl ? launch_loop<8, 2, true, true>(prm, pl, cus, st) : launch_loop<8, 2, false, true>(prm, pl, cus, st);
      case 4: return bl ? launch_loop<8, 4, true, true>(prm, pl, cus, st) : launch_loop<8, 4, false, true>(prm, pl, cus, st);
      case 8: return bl ? launch_loop<8, 8, true, true>(prm, pl, cus, st) : launch_loop<8, 8, false, true>(prm, pl, cus, st);
      default: return hipErrorInvalidValue;
    }
  } else {
    if (pl.NW == 4)  // r = 256 only
      return prm.R == 1 ? (bl ? launch_loop<4, 8, true, false, 1>(prm, pl, cus, st)
                              : launch_loop<4, 8, false, false, 1>(prm, pl, cus, st))
                        : (bl ? launch_loop<4, 8, true, false>(prm, pl, cus, st)
                              : launch_loop<4, 8, false, false>(prm, pl, cus, st));
    if (prm.R == 1 && pl.KB == 8)  // the single-request heads at r = 256
      return bl ? launch_loop<8, 8, true, false, 1>(prm, pl, cus, st) : launch_loop<8, 8, false, false, 1>(prm, pl, cus, st);
    switch (pl.KB) {
      case 1: return bl ? launch_loop<8, 1, true, false>(prm, pl, cus, st) : launch_loop<8, 1, false, false>(prm, pl, cus, st);
      case 2: return bl ? launch_loop<8, 2, true, false>(prm, pl, cus, st) : launch_loop<8, 2, false, false>(prm, pl, cus, st);
      case 4: return bl ? launch_loop<8, 4, true, false>(prm, pl, cus, st) : launch_loop<8, 4, false, false>(prm, pl, cus, st);
      case 8: return bl ? launch_loop<8, 8, true, false>(prm, pl, cus, st) : launch_loop<8, 8, false, false>(prm, pl, cus, st);
      case 16: return bl ? launch_loop<8, 16, true, false>(prm, pl, cus, st) : launch_loop<8, 16, false, false>(prm, pl, cus, st);
      default: return bl ? launch_loop<8, 32, true, false>(prm, pl, cus, st) : launch_loop<8, 32, false, false>(prm, pl, cus, st);
    }
  }
}

// Shared by both weight formats: the grid, the plan and the parameters.
hipError_t launch_markov_any(MarkovParams prm, bool q8, const ProbeArgs* probe, hipStream_t stream) {
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorNoDevice;
  // Workgroups: one per CU, but at least ~16 tiles each. With fewer tiles a
  // workgroup's step is all latency, and more workgroups only lengthen the
  // exchange (measured: 32000 x 256 with 8 requests 74 -> 67 us per call at
  // 128 instead of 256 workgroups; 4096 x 32 17 -> 14 us at 16).
  const int R = prm.R, V = prm.V, r = prm.r, k = prm.k;
  const int tiles = (V + 15) / 16;
  const int G = std::max(1, std::min({cus, kMaxGroups, (tiles + 15) / 16}));
  LoopPlan pl = make_loop_plan(R, V, r, k, G, kLoopWavesMax, q8);
  if (!q8 && pl.streams && pl.KB == 8) {  // one wave per SIMD holds more of markov_w2 on chip
    const LoopPlan p4 = make_loop_plan(R, V, r, k, G, 4, false);
    if (p4.lds_tiles + 4 * p4.RT > pl.lds_tiles + kLoopWavesMax * pl.RT) pl = p4;
  }
  prm.G = pl.G;
  prm.tiles = tiles;
  {
    const size_t per_copy = static_cast<size_t>(k) * R * pl.G;
    // Copy c takes slots [c * kCopyStride, c * kCopyStride + per_copy): all
    // kMaxRep copies fit when one call's slots fit in one stride.
    prm.nrep = per_copy <= kCopyStride ? kMaxRep : 1;
  }
  uint32_t nonce = g_launches.fetch_add(1, std::memory_order_relaxed) + 1u;
  if (nonce == 0u) nonce = g_launches.fetch_add(1, std::memory_order_relaxed) + 1u;
  prm.nonce = nonce;
  prm.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  prm.lds_tiles = pl.lds_tiles;
  prm.bstride = pl.bstride;
  prm.base_in_lds = pl.base_in_lds;
  if (probe) {
    prm.probe_on = 1;
    prm.probe = *probe;
  }
  return q8 ? dispatch_loop<true>(prm, pl, cus, stream) : dispatch_loop<false>(prm, pl, cus, stream);
}

MarkovParams common_params(const float* base, int R, int B, int V, int r, const int64_t* d2t, const int64_t* prev0,
                           int k, int64_t* ids, void* workspace) {
  MarkovParams prm{};
  prm.base = base;
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
  return prm;
}

}  // namespace

uint32_t markov_set_spin_limit(uint32_t polls) {
  return g_spin_limit.exchange(polls == 0u ? kDefaultSpinLimit : polls, std::memory_order_relaxed);
}

uint32_t* markov_lm_counter(void* workspace) { return static_cast<uint32_t*>(workspace) + kCtlLmCounter; }

size_t markov_workspace_bytes(int num_reqs, int k, int V) {
  if (num_reqs < 1 || num_reqs > kMaxReqs || k < 1 || k > kMaxSteps || V < 1) return 0;
  return kCtlBytes + 2 * kSlotsPerBuffer * sizeof(uint64_t);  // one layout for every size
}

// ---------------------------------------------------------------------------
// The loop without a caller workspace, for callers that cannot allocate
// (code under graph capture, tight serving loops): its workspace is a
// file-scope device array, one copy per GPU, kept until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory, so
// host code uses only the address hipGetSymbolAddress returns for it.
namespace {

constexpr size_t kScratchBytes = kCtlBytes + 2 * kSlotsPerBuffer * sizeof(uint64_t);  // 2 MiB + 256 B
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* p, size_t n16) {
  for (size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; e < n16; e += static_cast<size_t>(gridDim.x) * 256)
    p[e] = u32x4{0u, 0u, 0u, 0u};
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

size_t markov_scratch_bytes() { return kScratchBytes; }

// Address of this device's copy of `scratch`, set up on the first call per
// device (with that device current): its address from
// hipGetSymbolAddress, then one zero fill, a kernel on `stream` ordered
// before the caller's first loop launch (a kernel rather than a memset, so
// that a first call made under graph capture stays valid).
hipError_t markov_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    static_assert(kScratchBytes % 16 == 0, "the fill kernel writes 16-byte words");
    zero_fill_kernel<<<dim3(64), dim3(256), 0, stream>>>(static_cast<u32x4*>(ptr), kScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_markov(const float* base, int R, int B, int V, const uint16_t* w1,
                         const uint16_t* w2, int r, const int64_t* d2t, const int64_t* prev0,
                         int k, int64_t* ids, void* workspace, const ProbeArgs* probe,
                         hipStream_t stream, uint32_t* lm_ticks, int n_lm_ticks) {
  MarkovParams prm = common_params(base, R, B, V, r, d2t, prev0, k, ids, workspace);
  prm.w1 = w1;
  prm.w2 = w2;
  prm.lm_ticks = lm_ticks;
  prm.n_lm_ticks = lm_ticks ? n_lm_ticks : 0;
  return launch_markov_any(prm, false, probe, stream);
}

hipError_t launch_markov_q8(const float* base, int R, int B, int V, const int8_t* w1q, const uint16_t* w1d,
                            const int8_t* w2q, const uint16_t* w2d, int r, const int64_t* d2t,
                            const int64_t* prev0, int k, int64_t* ids, void* workspace, const ProbeArgs* probe,
                            hipStream_t stream) {
  MarkovParams prm = common_params(base, R, B, V, r, d2t, prev0, k, ids, workspace);
  prm.w1q = w1q;
  prm.w1d = w1d;
  prm.w2q = w2q;
  prm.w2d = w2d;
  return launch_markov_any(prm, true, probe, stream);
}

}  // namespace dspark
