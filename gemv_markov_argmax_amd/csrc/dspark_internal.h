// Internal helpers shared by the gfx950 kernels of libdspark.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// D = A(16x32) * B(32x16) + C on bf16 operands, fp32 accumulate.
// Lane l supplies A[l % 16][8*(l/16) + j] and B[8*(l/16) + j][l % 16]
// (j = 0..7, element j of the 8-wide vector); it receives
// D[4*(l/16) + v][l % 16] in component v. The k index inside a block is
// only ever used to pair A with B, so any fixed bijection works as long as
// both operands use the same one.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Streaming (read-once) 16-byte load: non-temporal hint so a weight stream
// does not evict data that is reused.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Raw buffer resource over [base, base + bytes) (bytes < 2^31). A load whose
// offset is at or past `bytes` returns zeros from the hardware range check
// and touches no memory, so edge lanes need neither a branch nor a clamp.
typedef __amdgpu_buffer_rsrc_t BufRes;
constexpr uint32_t kBufOutOfRange = 0x80000000u;  // an offset past every range used here
constexpr int kBufFlags = 0x00020000;             // word 3 of a raw 32-bit-element resource on gfx9

__device__ __forceinline__ BufRes buf_res(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufFlags);
}

// 16 bytes, non-temporal (read once: a weight stream).
__device__ __forceinline__ u32x4 buf_load16_nt(BufRes r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 2));
}

// 16 bytes with agent scope (cache policy sc1): the load and store that
// relaxed agent-scope atomics compile to on gfx950. A store completes (and
// leaves the wave's vmcnt) once workgroups on any XCD can load its value
// this way.
__device__ __forceinline__ u32x4 buf_load16_coherent(BufRes r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 16));
}
__device__ __forceinline__ void buf_store16_coherent(BufRes r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, 16);
}

__device__ __forceinline__ float4 buf_load_f32x4(BufRes r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}

__device__ __forceinline__ uint2 buf_load_b64(BufRes r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, 0));
}

__device__ __forceinline__ float buf_load_f32(BufRes r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Exact-to-2^-17 split of two fp32 values into bf16 pairs: hi = bf16(x),
// lo = bf16(x - hi), both nearest-even (v_cvt_pk_bf16_f32 on gfx950), so
// x = hi + lo + O(2^-17 |x|). Returns {hi pair, lo pair}, a in the low halves.
__device__ __forceinline__ uint2 split_bf16x2(float a, float b) {
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  const f32x2 r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u)};
  return uint2{hi, __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2))};
}

// The packed A block (M <= 8) holds the hi parts of row m in lane i = m and
// the lo parts in lane i = m + 8 of each 16-lane row, both over the same 8
// activations. Each of the two lanes loads one half of them (lane i >> 3
// picks which) and takes the other half from its partner i ^ 8 through DPP
// row_ror:8, so the activations are read once rather than twice. Returns the
// eight values in k order.
__device__ __forceinline__ void pair_halves(float4 mine, int i, float4& x0, float4& x1) {
  float4 other;
  other.x = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mine.x), 0x128, 0xF, 0xF, false));
  other.y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mine.y), 0x128, 0xF, 0xF, false));
  other.z = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mine.z), 0x128, 0xF, 0xF, false));
  other.w = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mine.w), 0x128, 0xF, 0xF, false));
  const bool upper = (i >> 3) != 0;
  x0 = upper ? other : mine;
  x1 = upper ? mine : other;
}

// Chain h (0..3) of the confidence probe's sum over one row of D entries
// (D % 8 == 0): lane l of a wave accumulates t = 8l + 512h + 2048j,
// j = 0, 1, ..., eight terms at a time in t order, in one fp32 FMA chain;
// the lanes are then combined by a fixed butterfly, so every lane ends with
// the chain's total. A row's sum is (c0 + c1) + (c2 + c3) over its four
// chains, an order fixed by D alone, whichever waves compute the chains.
// Up to NIN iterations' loads are in flight at once (NIN = 4: rows up to
// 8192 entries are a single round trip).
template <int NIN>
__device__ __forceinline__ float probe_chain(const float* __restrict__ x, int D, const uint16_t* __restrict__ w,
                                             int lane, int h) {
  float acc = 0.f;
  for (int t0 = 8 * lane + 512 * h; t0 < D; t0 += NIN * 2048) {
    u32x4 wb[NIN];
    float4 xa[NIN], xb[NIN];
#pragma unroll
    for (int u = 0; u < NIN; ++u) {
      const int t = min(t0 + 2048 * u, D - 8);  // (clamped: a load past D is issued but never used)
      wb[u] = load16(w + t);
      xa[u] = *reinterpret_cast<const float4*>(x + t);
      xb[u] = *reinterpret_cast<const float4*>(x + t + 4);
    }
#pragma unroll
    for (int u = 0; u < NIN; ++u) {
      if (t0 + 2048 * u >= D) break;
      acc = __builtin_fmaf(xa[u].x, __uint_as_float(wb[u].x << 16), acc);
      acc = __builtin_fmaf(xa[u].y, __uint_as_float(wb[u].x & 0xFFFF0000u), acc);
      acc = __builtin_fmaf(xa[u].z, __uint_as_float(wb[u].y << 16), acc);
      acc = __builtin_fmaf(xa[u].w, __uint_as_float(wb[u].y & 0xFFFF0000u), acc);
      acc = __builtin_fmaf(xb[u].x, __uint_as_float(wb[u].z << 16), acc);
      acc = __builtin_fmaf(xb[u].y, __uint_as_float(wb[u].z & 0xFFFF0000u), acc);
      acc = __builtin_fmaf(xb[u].z, __uint_as_float(wb[u].w << 16), acc);
      acc = __builtin_fmaf(xb[u].w, __uint_as_float(wb[u].w & 0xFFFF0000u), acc);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  return acc;
}

// The probe's logit from the four chain totals.
__device__ __forceinline__ float probe_logit(const float* c, float bias) { return ((c[0] + c[1]) + (c[2] + c[3])) + bias; }

// Round a finite float to bf16, nearest-even, returning the 16-bit pattern.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Order-preserving 64-bit key of (score, index): a larger key means a larger
// score, and for equal scores a smaller index. The maximum key over a set is
// therefore the greedy pick with the lowest index winning ties, whatever the
// order in which keys are combined. +0 and -0 map to the same key.
__device__ __forceinline__ uint64_t score_key(float s, uint32_t idx) {
  uint32_t u = __float_as_uint(s);
  if (s == 0.0f) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint64_t>(~idx);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return ~static_cast<uint32_t>(key);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// A 64-bit value moved across lanes by a DPP pattern (both halves).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(v), CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(v >> 32), CTRL, 0xF, 0xF, false);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Maximum over each row of 16 lanes, left in every lane of the row: quad
// swaps (lane ^ 1, lane ^ 2), then the half-row and row mirrors, which
// pair each quad with one in the other half and each half with the other.
__device__ __forceinline__ uint64_t row_max64(uint64_t v) {
  v = umax64(v, dpp64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = umax64(v, dpp64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = umax64(v, dpp64<0x141>(v));  // row_half_mirror
  v = umax64(v, dpp64<0x140>(v));  // row_mirror
  return v;
}

// The unit schedule of the scheduled GEMV (gemv_sched_kernel). Workgroup
// b's units: first S2 static ones, with
// S = chunk >= 2 the contiguous run b*S .. b*S + S - 1 (S*G <= T, set on the
// host), else b and b + G; then D0 + v for each take v of the counter, D0 =
// S2 * G. A take is issued at the start of position S2 - 2 (always) and of
// every later position while the sequence goes on (take_at), and read at the
// end of that position, so the unit after next is known before the next
// unit's loads go out. Every workgroup takes until it gets a unit past the
// last, so the G final takes return max(0, T - D0) .. + G - 1; the one that
// returns the largest is the last take of the launch and stores 0, leaving
// the counter as the launch found it. Takes are atomicInc (an add of 1 below
// 2^32 - 1): an atomicAdd would be turned into a wave-wide reduction whose
// result is waited for at once, which drains the loads in flight.
struct UnitSched {
  uint32_t G, b, S, S2, D0, T, final_take;
  __device__ UnitSched(uint32_t nunits, int chunk)
      : G(gridDim.x), b(blockIdx.x), S(chunk >= 2 ? static_cast<uint32_t>(chunk) : 0u), S2(S >= 2 ? S : 2u),
        D0(S2 * gridDim.x), T(nunits), final_take((nunits > S2 * gridDim.x ? nunits - S2 * gridDim.x : 0u) + gridDim.x - 1) {}
  __device__ uint32_t static_unit(uint32_t k) const { return S >= 2 ? b * S + k : b + k * G; }  // k < S2
  __device__ bool take_at(uint32_t pos, uint32_t unext) const { return pos + 2 == S2 || (pos + 2 > S2 && unext < T); }
  __device__ uint32_t take(uint32_t* counter) const {
    const uint32_t v = atomicInc(counter, 0xffffffffu);
    return v;
  }
  // After a take's value is known: the last take of the launch resets the counter.
  __device__ void settle(uint32_t* counter, uint32_t v) const {
    if (v == final_take) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

// Static units per workgroup of the scheduled GEMV: 90% of an equal share.
inline int sched_static_units(int nunits, int groups) { return 90 * (nunits / groups) / 100; }

// ---------------------------------------------------------------------------
// Host-side launchers (defined next to their kernels).
// ---------------------------------------------------------------------------

// Whether the GEMV kernels can address this shape: every buffer range they
// build (a workgroup's weight rows, the activation rows of a launch) must
// stay below 2^31 bytes.
bool gemv_shape_fits(int N, int K, int M);

// The rest of the draft block: see dspark_rmsnorm, dspark_silu_gate,
// dspark_attention_ragged.
hipError_t launch_rmsnorm(const float* x, int M, int D, const uint16_t* gamma, float eps, float* y, hipStream_t st);
// act = silu(X W_gate^T) * (X W_up^T) for W = [gate rows; up rows] bf16 [2F, K]:
// one GEMV with the gate in its epilogue where the short kernel takes the
// shape, else the GEMV into gu [M, 2F] followed by launch_silu_gate.
hipError_t launch_gemv_gated(const uint16_t* W, int F, int K, const float* X, int M, float* act, float* gu,
                             hipStream_t stream);
hipError_t launch_silu_gate(const float* gu, int M, int F, float* a, hipStream_t st);
// The GEMVs above with the RMSNorm of X fused into them (see
// dspark_proj_smallm_norm): Y = rmsnorm(X; gamma, eps) W^T, and the gated
// form. Only for shapes the short GEMV kernel takes (gemv_norm_fits).
bool gemv_norm_fits(int N, int K, int M);
hipError_t launch_gemv_norm(const uint16_t* W, int N, int K, const float* X, int M, const uint16_t* gamma, float eps,
                            float* Y, hipStream_t stream);
hipError_t launch_gemv_gated_norm(const uint16_t* W, int F, int K, const float* X, int M, const uint16_t* gamma,
                                  float eps, float* act, hipStream_t stream);
bool attention_shape_fits(int R, int B, int H, int Dh, int Lmax);
size_t attention_workspace_bytes(int R, int B, int H, int Dh, int Lmax);
hipError_t launch_attention(const float* q, const float* kb, const float* vb, int ld, int R, int B, int H, int Dh,
                            const uint16_t* kc, const uint16_t* vc, int Lmax, const int32_t* ctx_len, int causal,
                            float* out, float* ws, hipStream_t st);

// Small-M GEMV over Q8_0 weights; see dspark_proj_smallm_q8.
bool gemv_q8_shape_fits(int N, int K, int M);
// ldd: binary16 scales per row of Wd (0: K / 32, the dense layout).
hipError_t launch_gemv_q8(const int8_t* Wq, const uint16_t* Wd, int N, int K, const float* X, int M, float* Y,
                          hipStream_t stream, int ldd = 0);

// Y[m, n] = sum_t X[m, t] W[n, t] for all M rows (any M >= 1).
hipError_t launch_gemv(const uint16_t* W, int N, int K, const float* X, int M, float* Y,
                       hipStream_t stream, const float* res = nullptr);
// The same product for 16 < M with K split in two halves computed by
// different workgroups (half the activations per compute unit), their
// partials added in a caller workspace of gemv_split_workspace_bytes(N, K,
// M) bytes (256-byte aligned, zero-filled once; every launch leaves its
// ticket words 0). Shapes outside gemv_split_fits, or a null workspace, run
// launch_gemv. `dirty`, when given, is set to 1 if a ticket word was found
// not 0 (the outputs of that launch may then be wrong).
bool gemv_split_fits(int N, int K, int M);
size_t gemv_split_workspace_bytes(int N, int K, int M);
int gemv_split_tick_words(int N);  // ticket words at the start of that workspace
hipError_t launch_gemv_split(const uint16_t* W, int N, int K, const float* X, int M, float* Y, void* workspace,
                             hipStream_t stream, const float* res = nullptr, uint32_t* dirty = nullptr);
// The same product with the weight rows handed out to workgroups by a
// counter (see dspark_lm_head_sched) where the shape allows (M <= 8,
// K <= 4096), else launch_gemv. The counter reads 0 before and after.
bool gemv_sched_fits(int N, int K, int M);
hipError_t launch_gemv_sched(const uint16_t* W, int N, int K, const float* X, int M, float* Y, uint32_t* counter,
                             hipStream_t stream);
// The word of the Markov workspace that dspark_draft_round gives its
// lm_head as counter (a control word the loop itself never touches).
uint32_t* markov_lm_counter(void* workspace);

// The confidence probe's arguments (see dspark_conf_probe).
struct ProbeArgs {
  const float* x;  // [M, D]
  int M, D;
  const uint16_t* w;  // [D]
  float bias, threshold;
  float* logit;   // [M]
  int32_t* pass;  // [M] or null
};

// Markov loop; see dspark_markov_sample. With `probe` non-null the same
// launch also computes the confidence probe, bit-identical to launch_probe.
size_t markov_workspace_bytes(int num_reqs, int k, int V);
// Polls before a grid-wide wait of the loop gives up (0: the default);
// returns the previous setting. Applies to launches enqueued afterwards.
uint32_t markov_set_spin_limit(uint32_t polls);
// The per-device static workspace of the allocation-free loop entry point:
// its size, and its device address (set up on the first call per device).
size_t markov_scratch_bytes();
hipError_t markov_scratch(void** out, hipStream_t stream);
// lm_ticks (the round): n_lm_ticks ticket words of the round's split lm_head
// that every call sets to 0.
hipError_t launch_markov(const float* base, int R, int B, int V, const uint16_t* w1,
                         const uint16_t* w2, int r, const int64_t* d2t, const int64_t* prev0,
                         int k, int64_t* ids, void* workspace, const ProbeArgs* probe,
                         hipStream_t stream, uint32_t* lm_ticks = nullptr, int n_lm_ticks = 0);

// The same loop over Q8_0 markov weights (r % 32 == 0); see dspark_markov_sample_q8.
hipError_t launch_markov_q8(const float* base, int R, int B, int V, const int8_t* w1q, const uint16_t* w1d,
                            const int8_t* w2q, const uint16_t* w2d, int r, const int64_t* d2t,
                            const int64_t* prev0, int k, int64_t* ids, void* workspace, const ProbeArgs* probe,
                            hipStream_t stream);
hipError_t launch_probe(const float* x, int M, int D, const uint16_t* w, float bias,
                        float threshold, float* logit, int32_t* pass, hipStream_t stream);

// Streaming read of [buf, buf + bytes) by `groups` workgroups of `threads`
// (256, 512 or 1024), one word per workgroup into sink (a measurement aid).
hipError_t launch_stream_read(const void* buf, size_t bytes, int groups, int threads, uint32_t* sink,
                              hipStream_t stream);
hipError_t launch_stream_read_sched(const void* buf, size_t bytes, int groups, int threads, uint32_t* counter,
                                    uint32_t* sink, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace dspark
