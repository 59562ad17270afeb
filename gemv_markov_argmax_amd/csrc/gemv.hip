// Weight-stationary small-M GEMV on gfx950 matrix cores.
//
// Y[m, n] = sum_t X[m, t] * W[n, t], W bf16 [N, K], X fp32 [M, K], Y fp32.
//
// SharpInference #441 ("Observation", "Proposed work") describes the draft's
// projections and lm_head as tall-skinny products with M = B ~ 7 drafted
// rows, whose cost is reading each weight once; its proposal is a
// weight-stationary matvec that reads every weight row once for all rows.
//
// Design on gfx950:
//  * Every weight byte is read from HBM exactly once, with contiguous 16-byte
//    loads (whole 128-byte lines per row where the shape allows) and the
//    non-temporal hint.
//  * The activations are fp32. Each is split exactly into two bf16 terms,
//    x = hi + lo + O(2^-17 |x|), and both terms enter the A operand of
//    v_mfma_f32_16x16x32_bf16 against the bf16 weights, accumulating in
//    fp32. The expected logit error is ~1e-5. For M <= 8 the hi and lo rows
//    share one 16-row A block (rows 0..7 hi, 8..15 lo): one MFMA per 1 KB of
//    weights.
//  * Four kernels, chosen by shape and entry point:
//      - gemv_short_kernel: M <= 16, at most 16 tiles of 16 rows per workgroup
//        (the projections of a draft layer): the shortest dependency chain.
//        Variants fuse the RMSNorm of X and the gated activation.
//      - gemv_tstream_kernel: M <= 16, many tiles per workgroup (the
//        lm_heads): K split over 16 waves, two tiles of loads in flight,
//        outputs summed in LDS and written once per chunk of tiles.
//      - gemv_sched_kernel: the streaming kernel's work for M <= 8 and
//        K <= 4096 with rows handed out by a counter after a static run per
//        workgroup, which balances the XCDs (dspark_lm_head_sched).
//      - gemv_mrows_kernel: 16 < M <= 80 per launch (batched requests): a
//        small GEMM streaming K chunks of weights and A through LDS; with a
//        caller workspace (dspark_lm_head_split), K is split in two halves
//        taken by different workgroups, whose partials the second to finish
//        adds.
//  * Summation order depends on the shape only (never on timing or on which
//    workgroup took a row; the split sums exactly two partials, whose order
//    does not matter), so reruns are bit-identical; for M <= 16 an
//    output row does not depend on the other rows, and equal weight rows
//    give equal outputs.
#include "dspark_internal.h"

#include <algorithm>
#include <type_traits>

namespace dspark {
namespace {

struct GemvParams {
  const uint16_t* W;
  const float* X;
  float* Y;
  int N, K, M;   // M rows in this launch
  int ldy;       // row stride of Y
  int chunk;     // gemv_tstream_kernel: tiles whose outputs are staged in LDS at once (even)
  int pq, prem;  // row pairs per workgroup: N/2 = pq * gridDim.x + prem (the first prem get one more)
  const float* res;  // null, or [M, N] (row stride ldy) added to the outputs; may be Y itself
  const uint16_t* gamma;  // gemv_short_kernel with NORM: the RMSNorm weights bf16 [K]
  float eps;              // and its epsilon
  // gemv_mrows_kernel with SPLIT: a ticket word per row block (0 between
  // launches), the two halves' partial outputs, and the padded number of
  // row blocks (a multiple of 8).
  uint32_t* tick;
  float* part;
  int nrb;
  uint32_t* dirty;  // or null: set to 1 by a workgroup that draws a ticket past 1 (a word not left 0)
};

// The output value of (m, n), plus the residual when there is one (read and
// written by the same thread, so the residual may be Y itself).
__device__ __forceinline__ float with_res(const GemvParams& p, size_t idx, float y) { return p.res ? p.res[idx] + y : y; }

// Contiguous row range [r0, r1) of workgroup b: a balanced share of the N/2
// row pairs (a load instruction covers 2 rows); the last workgroup also takes
// an odd last row. Plain 32-bit arithmetic (the quotients come from the host).
__device__ __forceinline__ int2 wg_rows(const GemvParams& p) {
  const int b = blockIdx.x;
  const int r0 = 2 * (b * p.pq + min(b, p.prem));
  const int r1 = b + 1 == static_cast<int>(gridDim.x) ? p.N : 2 * ((b + 1) * p.pq + min(b + 1, p.prem));
  return int2{r0, r1};
}

// Rows of the largest workgroup under wg_rows with `grid` workgroups.
inline int wg_rows_max(int N, int grid) {
  const int q = (N / 2) / grid, rem = (N / 2) % grid;
  return std::max(2 * (q + (rem > 0 ? 1 : 0)), 2 * q + (N & 1));
}

// Short variant for M <= 16: at most 16 tiles of 16 rows per workgroup (the
// projections of a draft layer). Little is amortized over a long tile
// stream here, so the order of the first memory round trip decides the
// time: each wave issues its activation loads first (they come from L2),
// then the weight loads of its first tile (from HBM), and splits the
// activations into bf16 hi/lo while the weights are still on their way.
//
// Every 16-row tile is split along K over the 16 waves of a workgroup: wave w
// owns k-blocks [P*16*KBW + w*KBW, +KBW) of phase P (k-block = 32 values),
// so all waves do equal work on every tile and the A fragments of a wave
// (its K slice of X, split into bf16 hi/lo) fit in registers. K longer than
// 16*KBW k-blocks is covered in phases, which add into an LDS copy of the
// outputs; Y is written once, after the last phase. (A global store between
// phases would make the wave drain the next phase's weight loads before it
// could use its activations: loads and stores share one counter on gfx9.)
//
// Weight loads are contiguous runs: each instruction covers 16/KBW rows x
// 64*KBW bytes (whole 128-byte lines for KBW >= 2), which the memory system
// serves noticeably faster than the 16-rows x 64-bytes pattern of loading
// the MFMA B operand directly. The wave transposes its segment through a
// private LDS area (rows padded by 16 bytes: conflict-free writes and B
// reads) and runs the MFMAs from there. All global loads are raw buffer
// loads: lanes past M, K or the workgroup's rows get zeros from the range
// check, so the code is straight and the loads in flight are counted exactly.
//
// M <= 8 (PACK): rows 0..7 of the A block hold the hi parts, rows 8..15 the
// lo parts, one MFMA per k-block; each wave folds lo onto hi. 8 < M <= 16:
// hi and lo are two A blocks with their own accumulators, added per wave.
// The 16 per-wave partial tiles are summed in LDS in wave order (double
// buffered, one barrier per tile).
// GATED (the fused gate/up projection of an MLP, W = [gate rows; up rows],
// N = 2F): output row 2j is gate row j and row 2j + 1 is up row j, so both
// halves of activation j land in the same workgroup (rows come in pairs), and
// the epilogue writes act[m, j] = silu(g) * u, silu(g) = g / (1 + exp(-g)),
// into Y [M, F]; each row's own value is computed exactly as without GATED.
// NORM (the RMSNorm of X fused in front): the A operand is x * gamma[k],
// rounded to fp32 and split as above, and each output is scaled at the end
// by 1 / sqrt(mean_k x[m, k]^2 + eps), the RMSNorm factor of its row m. Each
// lane sums the squares of the activations it loads itself (every one once,
// over the phases, in a fixed order); lanes of the same row are then added
// by a fixed butterfly and the waves in wave order. A row's factor depends on
// that row alone.
template <bool PACK, int KBW, bool MANY, bool GATED = false, bool NORM = false>
__global__ __launch_bounds__(16 * kWave) void gemv_short_kernel(GemvParams p) {
  constexpr int NW = 16, F = PACK ? 1 : 2, ROWS = PACK ? 8 : 16;
  constexpr int SEG = 64 * KBW;                 // bytes of a row segment
  constexpr int RS = SEG + 16;                  // padded LDS row stride
  constexpr int LPR = SEG / 16;                 // lanes per row in a load instruction
  constexpr int RPI = kWave / LPR;              // rows per load instruction
  constexpr int NLD = 16 / RPI;                 // load instructions per tile
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* tr = smem;                                                          // [NW][16][RS]
  float* red = reinterpret_cast<float*>(smem + static_cast<size_t>(NW) * 16 * RS);  // [2][NW][ROWS][16]
  float* ysum = red + 2 * NW * ROWS * 16;                                            // [tiles][ROWS][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int N = p.N, K = p.K, M = p.M;
  const int KB = (K + 31) / 32;
  const int phases = (KB + 16 * KBW - 1) / (16 * KBW);

  // Row range of this workgroup; tiles are 16 rows from r0, the last one
  // masked at r1.
  const int2 rows = wg_rows(p);
  const int r0 = rows.x, r1 = rows.y;
  const int rounds = (r1 - r0 + 15) / 16;
  float* nrm = ysum + rounds * ROWS * 16;  // NORM: [NW][16] per-wave sums of squares
  const int lrow = lane / LPR, lchunk = lane % LPR;
  unsigned char* wtr = tr + w * 16 * RS;
  unsigned char* wr_base = wtr + lrow * RS + 16 * lchunk;  // + RPI*q*RS
  const unsigned char* rd_base = wtr + i * RS + 16 * g;   // + 64*kb

  const uint32_t rowb = static_cast<uint32_t>(K) * 2;  // bytes per weight row
  // Weight rows: this workgroup's range, or (GATED) the whole matrix, lane
  // row lrow of a tile being gate or up row (r0 + lrow) / 2 by its parity
  // (r0, RPI and 16 are even, so the parity is that of lrow); rows past the
  // matrix read zeros, rows past r1 are computed and not stored.
  const BufRes wres = GATED ? buf_res(p.W, static_cast<uint32_t>(N) * rowb)
                            : buf_res(p.W + static_cast<size_t>(r0) * K, static_cast<uint32_t>(r1 - r0) * rowb);
  const BufRes xres = buf_res(p.X, static_cast<uint32_t>(M) * K * 4);
  const BufRes gres = buf_res(NORM ? static_cast<const void*>(p.gamma) : static_cast<const void*>(p.W),
                              NORM ? static_cast<uint32_t>(K) * 2 : 0u);
  const uint32_t row_off = GATED ? static_cast<uint32_t>((lrow & 1) * (N >> 1) + (r0 >> 1) + (lrow >> 1)) * rowb
                                 : static_cast<uint32_t>(lrow) * rowb;
  const uint32_t tile_step = (GATED ? 8u : 16u) * rowb;  // 16 rows further

  auto load = [&](u32x4 (&b)[NLD], uint32_t off) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) b[q] = buf_load16_nt(wres, off + static_cast<uint32_t>(q * (GATED ? RPI / 2 : RPI)) * rowb);
  };
  // A tile's weights into this wave's private LDS area (row-major segments).
  auto stage = [&](const u32x4 (&b)[NLD]) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) *reinterpret_cast<u32x4*>(wr_base + RPI * q * RS) = b[q];
  };
  // B fragments from the staged tile, the MFMAs, and the wave's partial tile
  // into red[buf].
  auto mma_publish = [&](const u32x4 (&afr)[KBW][F], int buf) {
    f32x4 acc[F];
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(rd_base + 64 * kb);
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = mfma_16x16x32(afr[kb][f], bv, acc[f]);
    }
    float* dst = red + (buf * NW + w) * ROWS * 16;
    if (PACK) {
      // lanes 0..31 hold rows 0..7 (hi), lanes 32..63 rows 8..15 (lo) of the same columns
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float lo = __shfl_down(acc[0][v], 32);
        if (g < 2) dst[(4 * g + v) * 16 + i] = acc[0][v] + lo;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[(4 * g + v) * 16 + i] = acc[0][v] + acc[F - 1][v];
    }
  };
  // Wave-order sum of tile t into the LDS outputs (phases add, in order).
  auto reduce = [&](int buf, int t, int ph) {
    if (tid < ROWS * 16) {
      float y = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) y += red[(buf * NW + ww) * ROWS * 16 + tid];
      float* ys = ysum + t * ROWS * 16 + tid;
      *ys = ph == 0 ? y : *ys + y;
    }
  };

  // Activations of phase ph, k-block kb: k = kseg + 32*kb + 8*g + (0..7) of
  // row m (packed rows: each lane of a hi/lo pair loads one half). A phase
  // past the last reads nothing.
  constexpr int XH = PACK ? 1 : 2;
  const int m = PACK ? (i & 7) : i;
  const bool mrow = m < M;
  const uint32_t xrow = static_cast<uint32_t>(m) * K * 4;
  // (the conditions combine with & rather than &&: no short-circuit, so the
  // compiler selects offsets instead of branching around the address math)
  // NORM: gamma of the same entries (8 bytes for a packed lane's half, 16
  // otherwise), per column, so not masked by the row.
  constexpr int GN = NORM ? KBW : 1;
  auto load_x = [&](float4 (&xr)[KBW][XH], u32x4 (&gr)[GN], int ph) {
    const int kseg = 32 * KBW * (ph * NW + w);
    const bool live = (ph < phases) & mrow;
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      const int k = kseg + 32 * kb + 8 * g;
      const uint32_t off = live & (k < K) ? xrow + static_cast<uint32_t>(k) * 4 : kBufOutOfRange;
      if (PACK) {
        xr[kb][0] = buf_load_f32x4(xres, off + 16 * (i >> 3));
      } else {
        xr[kb][0] = buf_load_f32x4(xres, off);
        xr[kb][XH - 1] = buf_load_f32x4(xres, off + 16);
      }
      if constexpr (NORM) {
        const uint32_t goff = (ph < phases) & (k < K) ? static_cast<uint32_t>(k) * 2 : kBufOutOfRange;
        if (PACK) {
          const uint2 v = buf_load_b64(gres, goff + 8 * (i >> 3));
          gr[kb] = u32x4{v.x, v.y, 0u, 0u};
        } else {
          gr[kb] = __builtin_bit_cast(u32x4, buf_load_f32x4(gres, goff));
        }
      }
    }
  };
  // Offset of this lane's first weight load in phase ph (tile 0). A lane
  // whose k lies past K, or a phase past the last, starts out of range (the
  // added row offsets stay below 2^31 and cannot wrap it back).
  auto w_off = [&](int ph) -> uint32_t {
    const int kseg = 32 * KBW * (ph * NW + w);
    return (ph < phases) & (kseg + 8 * lchunk < K) ? row_off + static_cast<uint32_t>(kseg + 8 * lchunk) * 2
                                                   : kBufOutOfRange;
  };
  auto gmul = [](float4 x, uint32_t lo, uint32_t hi) {  // x * four bf16 (entry order)
    return float4{x.x * __uint_as_float(lo << 16), x.y * __uint_as_float(lo & 0xffff0000u),
                  x.z * __uint_as_float(hi << 16), x.w * __uint_as_float(hi & 0xffff0000u)};
  };
  auto sq4 = [](float4 x, float s) {
    s = __builtin_fmaf(x.x, x.x, s);
    s = __builtin_fmaf(x.y, x.y, s);
    s = __builtin_fmaf(x.z, x.z, s);
    return __builtin_fmaf(x.w, x.w, s);
  };
  float ss = 0.f;  // NORM: this lane's sum of squares
  auto split = [&](const float4 (&xr)[KBW][XH], const u32x4 (&gr)[GN], u32x4 (&afr)[KBW][F]) {
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      float4 a0 = xr[kb][0], a1 = xr[kb][XH - 1];
      if constexpr (NORM) {
        ss = sq4(a0, ss);
        if (!PACK) ss = sq4(a1, ss);
        a0 = gmul(a0, gr[kb].x, gr[kb].y);
        if (!PACK) a1 = gmul(a1, gr[kb].z, gr[kb].w);
      }
      float4 x0 = a0, x1 = a1;
      if (PACK) pair_halves(a0, i, x0, x1);
      const uint2 s0 = split_bf16x2(x0.x, x0.y), s1 = split_bf16x2(x0.z, x0.w);
      const uint2 s2 = split_bf16x2(x1.x, x1.y), s3 = split_bf16x2(x1.z, x1.w);
      const u32x4 h = {s0.x, s1.x, s2.x, s3.x}, l = {s0.y, s1.y, s2.y, s3.y};
      if (PACK) {
        afr[kb][0] = (i >> 3) ? l : h;
      } else {
        afr[kb][0] = h;
        afr[kb][F - 1] = l;
      }
    }
  };

  if (!MANY) {
    // One tile per workgroup: the loads of phase ph + 1 go out while phase
    // ph is still being computed (activations before its MFMAs, weights right
    // after them, when their registers are free), so they overlap its
    // reduction and the next split.
    float4 xr[KBW][XH];
    u32x4 b[NLD], afr[KBW][F], gr[GN];
    // (the scheduling barriers keep each step's registers apart: the
    // activations become A fragments, the weights go to LDS, and only then
    // do the next phase's loads reuse those registers; the last phase is
    // peeled so that no load is issued for a phase that does not exist)
    auto phase = [&](int ph, auto more) {
      __builtin_amdgcn_sched_barrier(0);
      split(xr, gr, afr);
      __builtin_amdgcn_sched_barrier(0);
      stage(b);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(more)::value) load_x(xr, gr, ph + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_publish(afr, ph & 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(more)::value) load(b, w_off(ph + 1));
      __syncthreads();
      reduce(ph & 1, 0, ph);
    };
    load_x(xr, gr, 0);
    load(b, w_off(0));
    int ph = 0;
    for (; ph + 1 < phases; ++ph) phase(ph, std::true_type{});
    phase(ph, std::false_type{});
  } else {
    // Several tiles per workgroup: one tile of weights in flight per wave,
    // the next issued as soon as the current one is in LDS (so it overlaps
    // the MFMAs, the reduction and the barrier); the activations and their
    // split once per phase. 16 waves x one tile keep enough bytes in flight
    // per CU to cover the memory latency.
    float4 xr[KBW][XH];
    u32x4 b[NLD], afr[KBW][F], gr[GN];
    load_x(xr, gr, 0);
    load(b, w_off(0));
    __builtin_amdgcn_sched_barrier(0);
    split(xr, gr, afr);
    int j = 0;  // items so far: parity of the reduction buffer
    for (int ph = 0; ph < phases; ++ph) {
      const uint32_t off = w_off(ph);
      for (int t = 0; t < rounds; ++t, ++j) {
        __builtin_amdgcn_sched_barrier(0);
        stage(b);
        __builtin_amdgcn_sched_barrier(0);
        const bool last_t = t + 1 == rounds;
        const bool more = !last_t || ph + 1 < phases;
        if (last_t && more) load_x(xr, gr, ph + 1);
        if (more) load(b, last_t ? w_off(ph + 1) : off + static_cast<uint32_t>(t + 1) * tile_step);
        __builtin_amdgcn_sched_barrier(0);
        mma_publish(afr, j & 1);
        __syncthreads();
        reduce(j & 1, t, ph);
        if (last_t && more) split(xr, gr, afr);
      }
    }
  }
  if constexpr (NORM) {
    // Row sums of squares: the lanes of row m are (m or m + 8 when packed, g = 0..3).
    float t = ss;
    if (PACK) t += __shfl_xor(t, 8);
    t += __shfl_xor(t, 16);
    t += __shfl_xor(t, 32);
    if (lane < (PACK ? 8 : 16)) nrm[w * 16 + lane] = t;
  }
  __syncthreads();
  // The RMSNorm factor of row mm (1 without NORM).
  auto rfac = [&](int mm) -> float {
    if constexpr (!NORM) {
      (void)mm;
      return 1.0f;
    } else {
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) tot += nrm[ww * 16 + mm];
      return 1.0f / sqrtf(tot / static_cast<float>(K) + p.eps);
    }
  };
  if constexpr (GATED) {
    // Activations, once: row pair (n, n + 1) of tile t is (gate, up) of j = n / 2.
    for (int e = tid; e < rounds * M * 8; e += NW * kWave) {
      const int t = e / (M * 8), rem = e - t * M * 8, mm = rem >> 3, pc = rem & 7;
      const int n = r0 + 16 * t + 2 * pc;
      if (n < r1) {
        float g = ysum[(t * ROWS + mm) * 16 + 2 * pc], u = ysum[(t * ROWS + mm) * 16 + 2 * pc + 1];
        if constexpr (NORM) {
          const float rf = rfac(mm);
          g *= rf;
          u *= rf;
        }
        p.Y[static_cast<size_t>(mm) * p.ldy + (n >> 1)] = g / (1.0f + expf(-g)) * u;
      }
    }
    return;
  }
  // Outputs, once: tile t covers columns r0 + 16t + (0..15).
  for (int e = tid; e < rounds * M * 16; e += NW * kWave) {
    const int t = e / (M * 16), rem = e - t * M * 16, mm = rem >> 4, col = rem & 15;
    const int n = r0 + 16 * t + col;
    const size_t idx = static_cast<size_t>(mm) * p.ldy + n;
    float y = ysum[(t * ROWS + mm) * 16 + col];
    if constexpr (NORM) y *= rfac(mm);
    if (n < r1) p.Y[idx] = with_res(p, idx, y);
  }
}

// Streaming variant for M <= 16 (the small-M GEMVs of a draft round).
//
// Every 16-row tile is split along K over the 16 waves of a workgroup: wave w
// owns k-blocks [P*16*KBW + w*KBW, +KBW) of phase P (k-block = 32 values),
// so all waves do equal work on every tile and the A fragments of a wave
// (its K slice of X, split into bf16 hi/lo) fit in registers. K longer than
// 16*KBW k-blocks is covered in phases.
//
// Weight loads are contiguous runs: each instruction covers 16/KBW rows x
// 64*KBW bytes (whole 128-byte lines for KBW >= 2), which the memory system
// serves noticeably faster than the 16-rows x 64-bytes pattern of loading
// the MFMA B operand directly. The wave transposes its segment through a
// private LDS area (rows padded by 16 bytes: conflict-free writes and B
// reads) and runs the MFMAs from there. Loads run two tiles ahead.
//
// The loop issues no global store. On gfx9 loads and stores share one
// counter and may complete out of order with respect to each other, so a
// wave that has a store outstanding must drain every prefetched load before
// it may use one. The outputs of a chunk of tiles are therefore summed into
// LDS (phases add there) and written out, as whole rows, once per chunk.
// All global loads are raw buffer loads over the workgroup's own rows (and
// over X): a lane past the end of its range gets zeros from the hardware
// range check instead of a branch, so the loop body is straight code and
// the compiler counts the loads in flight exactly.
//
// M <= 8 (PACK): rows 0..7 of the A block hold the hi parts, rows 8..15 the
// lo parts, one MFMA per k-block; each wave folds lo onto hi. 8 < M <= 16:
// hi and lo are two A blocks with their own accumulators, added per wave.
// The 16 per-wave partial tiles are summed in wave order (double buffered,
// one barrier per tile).
template <bool PACK, int KBW, bool MULTI>
__global__ __launch_bounds__(16 * kWave) void gemv_tstream_kernel(GemvParams p) {
  constexpr int NW = 16, F = PACK ? 1 : 2, ROWS = PACK ? 8 : 16;
  constexpr int SEG = 64 * KBW;                 // bytes of a row segment
  constexpr int RS = SEG + 16;                  // padded LDS row stride
  constexpr int LPR = SEG / 16;                 // lanes per row in a load instruction
  constexpr int RPI = kWave / LPR;              // rows per load instruction
  constexpr int NLD = 16 / RPI;                 // load instructions per tile
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* tr = smem;                                                          // [NW][16][RS]
  float* red = reinterpret_cast<float*>(smem + static_cast<size_t>(NW) * 16 * RS);  // [2][NW][ROWS][16]
  float* ylds = red + 2 * NW * ROWS * 16;                                            // [chunk][M][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int N = p.N, K = p.K, M = p.M;
  const int KB = (K + 31) / 32;
  const int phases = (KB + 16 * KBW - 1) / (16 * KBW);

  // Row range of this workgroup; tiles are 16 rows from r0, the last one
  // masked at r1.
  const int2 rows = wg_rows(p);
  const int r0 = rows.x, r1 = rows.y;
  const int rounds = (r1 - r0 + 15) / 16;
  // Chunks of this workgroup's tiles, balanced, even sized (but the last).
  const int nchunks = (rounds + p.chunk - 1) / p.chunk;
  const int csize = (((rounds + nchunks - 1) / nchunks) + 1) & ~1;
  const int lrow = lane / LPR, lchunk = lane % LPR;
  unsigned char* wtr = tr + w * 16 * RS;
  unsigned char* wr_base = wtr + lrow * RS + 16 * lchunk;  // + RPI*q*RS
  const unsigned char* rd_base = wtr + i * RS + 16 * g;   // + 64*kb

  const uint32_t rowb = static_cast<uint32_t>(K) * 2;     // bytes per weight row
  const BufRes wres = buf_res(p.W + static_cast<size_t>(r0) * K, static_cast<uint32_t>(r1 - r0) * rowb);
  const BufRes xres = buf_res(p.X, static_cast<uint32_t>(M) * K * 4);

  u32x4 afr[KBW][F];
  u32x4 b0[NLD], b1[NLD];
  int ph = 0, c0 = 0, c1 = 0, lim = 0;
  uint32_t lane_off = 0;

  // Phase ph: this wave's segment starts at k = kseg. A lane whose k lies
  // past K starts out of range, so it reads zeros (the added tile offsets
  // stay below 2^31 and cannot wrap it back in).
  auto set_phase = [&](int phase) {
    ph = phase;
    const int kseg = 32 * KBW * (ph * NW + w);
    lane_off = kseg + 8 * lchunk < K
                   ? static_cast<uint32_t>(lrow) * rowb + static_cast<uint32_t>(kseg + 8 * lchunk) * 2
                   : kBufOutOfRange;
  };
  // A fragments of phase ph: k-block kb covers k = kseg + 32*kb + 8*g + (0..7);
  // lanes past M or K load zeros. The activation loads go out at once, or in
  // two batches where registers are short, and are split into bf16 hi/lo.
  auto build_a = [&]() {
    const int kseg = 32 * KBW * (ph * NW + w);
    constexpr int XH = PACK ? 1 : 2;  // float4 loads per lane and k-block (packed rows: one half each)
    constexpr int KH = KBW * XH * 4 > 32 ? KBW / 2 : KBW;
    const int m = PACK ? (i & 7) : i;
#pragma unroll
    for (int k0 = 0; k0 < KBW; k0 += KH) {
      float4 xr[KH][XH];
#pragma unroll
      for (int kk = 0; kk < KH; ++kk) {
        const int k = kseg + 32 * (k0 + kk) + 8 * g;
        const uint32_t off = (m < M) & (k < K) ? static_cast<uint32_t>(m * K + k) * 4 : kBufOutOfRange;
        if (PACK) {
          xr[kk][0] = buf_load_f32x4(xres, off + 16 * (i >> 3));
        } else {
          xr[kk][0] = buf_load_f32x4(xres, off);
          xr[kk][XH - 1] = buf_load_f32x4(xres, off + 16);
        }
      }
#pragma unroll
      for (int kk = 0; kk < KH; ++kk) {
        float4 x0 = xr[kk][0], x1 = xr[kk][XH - 1];
        if (PACK) pair_halves(xr[kk][0], i, x0, x1);
        const uint2 s0 = split_bf16x2(x0.x, x0.y), s1 = split_bf16x2(x0.z, x0.w);
        const uint2 s2 = split_bf16x2(x1.x, x1.y), s3 = split_bf16x2(x1.z, x1.w);
        const u32x4 h = {s0.x, s1.x, s2.x, s3.x}, l = {s0.y, s1.y, s2.y, s3.y};
        if (PACK) {
          afr[k0 + kk][0] = (i >> 3) ? l : h;
        } else {
          afr[k0 + kk][0] = h;
          afr[k0 + kk][F - 1] = l;
        }
      }
    }
  };
  // Tile rr of this workgroup; rows past r1 and tiles past lim read zeros.
  auto load = [&](u32x4 (&b)[NLD], int rr) {
    const uint32_t off = rr < lim ? lane_off + static_cast<uint32_t>(rr) * 16 * rowb : kBufOutOfRange;
#pragma unroll
    for (int q = 0; q < NLD; ++q) b[q] = buf_load16_nt(wres, off + static_cast<uint32_t>(q * RPI) * rowb);
  };
  // b0 must stay the older group (the loop waits for it with b1 still in
  // flight), so the scheduler may not move the prologue loads. The first
  // tile's loads go out before the A fragments are built: they do not depend
  // on X, so the two memory latencies overlap.
  auto prologue = [&](bool with_a) {
    load(b0, c0);
    __builtin_amdgcn_sched_barrier(0);
    if (with_a) build_a();
    load(b1, c0 + 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute_publish = [&](u32x4 (&b)[NLD], int buf) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) *reinterpret_cast<u32x4*>(wr_base + RPI * q * RS) = b[q];
    f32x4 acc[F];
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(rd_base + 64 * kb);
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = mfma_16x16x32(afr[kb][f], bv, acc[f]);
    }
    float* dst = red + (buf * NW + w) * ROWS * 16;
    if (PACK) {
      // lanes 0..31 hold rows 0..7 (hi), lanes 32..63 rows 8..15 (lo) of the same columns
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float lo = __shfl_down(acc[0][v], 32);
        if (g < 2) dst[(4 * g + v) * 16 + i] = acc[0][v] + lo;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[(4 * g + v) * 16 + i] = acc[0][v] + acc[F - 1][v];
    }
  };
  // Wave-order sum of tile rr into the chunk's LDS outputs (phases add).
  auto reduce = [&](int buf, int rr) {
    if (tid < M * 16) {
      float y = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) y += red[((buf * NW + ww) * ROWS + (tid >> 4)) * 16 + (tid & 15)];
      float* yl = ylds + (rr - c0) * M * 16 + tid;
      *yl = ph == 0 ? y : *yl + y;
    }
  };
  // Tiles [c0, c1), two per iteration: the back edge always carries b0
  // older than b1, so the head waits for b0 alone. Chunks are even sized but
  // the last; its odd last tile is computed alone (after it nothing reads b0
  // or b1 before the next prologue).
  auto run_tiles = [&]() {
    int rr = c0;
    for (; rr + 2 <= c1; rr += 2) {
      compute_publish(b0, 0);
      load(b0, rr + 2);
      __syncthreads();
      reduce(0, rr);
      compute_publish(b1, 1);
      load(b1, rr + 3);
      __syncthreads();
      reduce(1, rr + 1);
    }
    if (rr < c1) {
      compute_publish(b0, 0);
      __syncthreads();
      reduce(0, rr);
    }
  };
  // The chunk's outputs, row by row: columns [r0 + 16*c0, min(r1, r0 + 16*c1)).
  auto write_out = [&]() {
    __syncthreads();
    const int n0 = r0 + 16 * c0, cols = min(r1, r0 + 16 * c1) - n0;
    for (int m = 0; m < M; ++m)
      for (int j = tid; j < cols; j += NW * kWave)
        p.Y[static_cast<size_t>(m) * p.ldy + n0 + j] =
            with_res(p, static_cast<size_t>(m) * p.ldy + n0 + j, ylds[(j >> 4) * M * 16 + m * 16 + (j & 15)]);
    __syncthreads();  // the next chunk reuses the LDS outputs
  };

  if (!MULTI) {
    // One phase: the A fragments are built once and the prefetch runs on
    // across chunk boundaries, so a chunk's outputs go out while the next
    // chunk's first tiles are already on their way.
    set_phase(0);
    lim = rounds;
    c0 = 0;
    prologue(true);
    for (; c0 < rounds; c0 += csize) {
      c1 = min(rounds, c0 + csize);
      run_tiles();
      write_out();
    }
  } else {
    // Each chunk runs every phase; tiles past the chunk read zeros.
    for (c0 = 0; c0 < rounds; c0 += csize) {
      c1 = min(rounds, c0 + csize);
      lim = c1;
      for (int q = 0; q < phases; ++q) {
        set_phase(q);
        prologue(true);
        run_tiles();
      }
      write_out();
    }
  }
}

// Dynamically scheduled streaming variant, M <= 8 and K <= 4096 (the
// lm_head of a single request's draft round).
//
// With every workgroup owning an equal contiguous share, the launch ends
// when the slowest XCD does. Measured on MI355X with a plain streaming read
// of the Qwen3-8B lm_head's 1.25 GB: the workgroups of the odd XCDs finish
// 20-35 us after those of the even ones (shares assigned cyclically instead
// of contiguously change nothing), 203 us in all; handing out 256 KB pieces
// from a counter instead brings every XCD to within ~7 us of the others and
// the read to 177 us.
//
// So the weight rows are cut into units of two tiles (32 rows, 256 KB at
// K = 4096). Each workgroup first runs a contiguous run of units of its own
// (90% of an equal share, fixed on the host), then takes units from a
// counter in caller memory until they run out: the workgroups of the faster
// XCDs take more of them. Handing out every unit was slower per CU (the
// contiguous runs stream faster) and handing out none leaves the XCDs
// unbalanced; the mix beats both. A unit is processed like two tiles of the streaming
// kernel, phase by phase; with U = 2 each (unit, phase) is one pair of tiles
// (b0, b1), and each tile of the next pair (the next phase, or the next
// unit's first) is loaded as soon as its buffer is free, two tiles ahead as
// in the streaming kernel, so the stream does not stop at phase or unit
// boundaries. The A fragments of every phase
// stay in registers (X is read once). The next units' indices are known
// two units ahead: thread 0 issues the atomic for the unit after next when a
// unit starts and publishes its result in LDS when the unit ends, so no wave
// waits for it. Outputs stay in LDS (phases add there) and are written after
// the loop, with the unit list, or when that LDS fills (64 units, far more
// than a workgroup takes at the sizes in use).
//
// The counter must read 0 when a launch starts, and the launch leaves it 0
// (the workgroup whose take is the last of the launch stores 0; see
// UnitSched). Launches that share a counter must be ordered (one stream).
constexpr int kSchedU = 2;     // tiles per unit
constexpr int kSchedCap = 64;  // units whose outputs a workgroup holds in LDS

template <int NPH>
__global__ __launch_bounds__(16 * kWave) void gemv_sched_kernel(GemvParams p, uint32_t* __restrict__ counter) {
  constexpr int NW = 16, KBW = 4, ROWS = 8, U = kSchedU;
  constexpr int SEG = 64 * KBW;     // bytes of a row segment
  constexpr int RS = SEG + 16;      // padded LDS row stride
  constexpr int LPR = SEG / 16;     // lanes per row in a load instruction
  constexpr int RPI = kWave / LPR;  // rows per load instruction
  constexpr int NLD = 16 / RPI;     // load instructions per tile
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* tr = smem;                                                            // [NW][16][RS]
  float* red = reinterpret_cast<float*>(smem + static_cast<size_t>(NW) * 16 * RS);    // [2][NW][ROWS][16]
  float* ylds = red + 2 * NW * ROWS * 16;                                              // [cap][U][ROWS][16]
  uint32_t* ulist = reinterpret_cast<uint32_t*>(ylds + kSchedCap * U * ROWS * 16);    // [cap] unit of each slot
  uint32_t* sgrab = ulist + kSchedCap;                                                 // [2] published takes

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int N = p.N, K = p.K, M = p.M;
  const uint32_t nunits = static_cast<uint32_t>(((N + 15) / 16 + U - 1) / U);
  const uint32_t last_take = nunits + gridDim.x - 1;
  const int lrow = lane / LPR, lchunk = lane % LPR;
  unsigned char* wtr = tr + w * 16 * RS;
  unsigned char* wr_base = wtr + lrow * RS + 16 * lchunk;  // + RPI*q*RS
  const unsigned char* rd_base = wtr + i * RS + 16 * g;   // + 64*kb
  const uint32_t rowb = static_cast<uint32_t>(K) * 2;
  const BufRes xres = buf_res(p.X, static_cast<uint32_t>(M) * K * 4);

  // A fragments of every phase (packed rows: hi in rows 0..7, lo in 8..15).
  u32x4 afr[NPH][KBW];
  {
    const int m = i & 7;
    float4 xr[NPH][KBW];
#pragma unroll
    for (int q = 0; q < NPH; ++q)
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        const int k = 32 * KBW * (q * NW + w) + 32 * kb + 8 * g;
        const uint32_t off = (m < M) & (k < K) ? static_cast<uint32_t>(m * K + k) * 4 : kBufOutOfRange;
        xr[q][kb] = buf_load_f32x4(xres, off + 16 * (i >> 3));
      }
#pragma unroll
    for (int q = 0; q < NPH; ++q)
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        float4 x0, x1;
        pair_halves(xr[q][kb], i, x0, x1);
        const uint2 s0 = split_bf16x2(x0.x, x0.y), s1 = split_bf16x2(x0.z, x0.w);
        const uint2 s2 = split_bf16x2(x1.x, x1.y), s3 = split_bf16x2(x1.z, x1.w);
        afr[q][kb] = (i >> 3) ? u32x4{s0.y, s1.y, s2.y, s3.y} : u32x4{s0.x, s1.x, s2.x, s3.x};
      }
  }

  // Tile t of unit u in phase q (unit u covers rows 32u .. 32u + 31; rows
  // past N, lanes past K and units past the last read zeros).
  const uint16_t* const Wmat = p.W;
  auto load_tile = [&](u32x4 (&b)[NLD], uint32_t u, int q, int t) {
    u = __builtin_amdgcn_readfirstlane(u);
    const bool live = u < nunits;
    const int row0 = live ? static_cast<int>(u) * U * 16 + 16 * t : 0;
    const int nrows = live ? max(0, min(16, N - row0)) : 0;
    // (the descriptor from scalar values only, or every load becomes a
    // loop over the lanes' distinct descriptors; readfirstlane returns an
    // int, so each half goes back through uint32_t before it is widened, or
    // a low half >= 2^31 would sign-extend into the high half)
    const uint64_t addr = reinterpret_cast<uint64_t>(Wmat + static_cast<size_t>(row0) * K);
    const uint32_t alo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr)));
    const uint32_t ahi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr >> 32)));
    const uint32_t bytes = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(nrows) * rowb));
    const BufRes res =
        buf_res(reinterpret_cast<const void*>((static_cast<uint64_t>(ahi) << 32) | static_cast<uint64_t>(alo)), bytes);
    const int kseg = 32 * KBW * (q * NW + w);
    const uint32_t off = kseg + 8 * lchunk < K
                             ? static_cast<uint32_t>(lrow) * rowb + static_cast<uint32_t>(kseg + 8 * lchunk) * 2
                             : kBufOutOfRange;
#pragma unroll
    for (int j = 0; j < NLD; ++j) b[j] = buf_load16_nt(res, off + static_cast<uint32_t>(j * RPI) * rowb);
  };
  auto compute_publish = [&](const u32x4 (&b)[NLD], const u32x4 (&a)[KBW], int buf) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) *reinterpret_cast<u32x4*>(wr_base + RPI * j * RS) = b[j];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) acc = mfma_16x16x32(a[kb], *reinterpret_cast<const u32x4*>(rd_base + 64 * kb), acc);
    float* dst = red + (buf * NW + w) * ROWS * 16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float lo = __shfl_down(acc[v], 32);
      if (g < 2) dst[(4 * g + v) * 16 + i] = acc[v] + lo;
    }
  };
  // Wave-order sum of tile t of the unit in slot s into its LDS outputs.
  auto reduce = [&](int buf, int s, int t, int q) {
    if (tid < M * 16) {
      float y = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) y += red[((buf * NW + ww) * ROWS + (tid >> 4)) * 16 + (tid & 15)];
      float* yl = ylds + ((s * U + t) * ROWS + (tid >> 4)) * 16 + (tid & 15);
      *yl = q == 0 ? y : *yl + y;
    }
  };
  // The outputs of slots [0, ns), row by row.
  auto write_out = [&](int ns) {
    __syncthreads();
    for (int e = tid; e < ns * M * U * 16; e += NW * kWave) {
      const int s = e / (M * U * 16), rem = e - s * (M * U * 16), m = rem / (U * 16), j = rem - m * (U * 16);
      const int n = static_cast<int>(ulist[s]) * U * 16 + j;
      if (n < N) {
        const size_t idx = static_cast<size_t>(m) * p.ldy + n;
        p.Y[idx] = with_res(p, idx, ylds[((s * U + (j >> 4)) * ROWS + m) * 16 + (j & 15)]);
      }
    }
    __syncthreads();
  };

  // This workgroup's units: a static run, then takes (UnitSched).
  const UnitSched us(nunits, p.chunk);
  uint32_t ucur = us.static_unit(0), unext = us.static_unit(1);
  if (ucur >= nunits) {  // uniform (only where T < G): no unit here; this workgroup's one take is final
    if (tid == 0) us.settle(counter, us.take(counter));
    return;
  }

  // Two tiles in flight, as in the streaming kernel: the back edge always
  // carries b0 older than b1, so the head waits for b0 alone.
  u32x4 b0[NLD], b1[NLD];
  load_tile(b0, ucur, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_tile(b1, ucur, 0, 1);
  __builtin_amdgcn_sched_barrier(0);
  int ns = 0;
  uint32_t pending = 0;
  for (uint32_t pos = 0;; ++pos) {
    const bool take = us.take_at(pos, unext);  // the unit after next comes from a take
    if (tid == 0 && take) pending = us.take(counter);
    if (tid == 0) ulist[ns] = ucur;
#pragma unroll
    for (int q = 0; q < NPH; ++q) {
      const bool lastq = q + 1 == NPH;
      const uint32_t nu = lastq ? unext : ucur;  // the next pair: next phase, or the next unit's first
      const int nq = lastq ? 0 : q + 1;
      compute_publish(b0, afr[q], 0);
      load_tile(b0, nu, nq, 0);
      __syncthreads();
      reduce(0, ns, 0, q);
      compute_publish(b1, afr[q], 1);
      load_tile(b1, nu, nq, 1);
      if (lastq && tid == 0 && take) {
        us.settle(counter, pending);
        sgrab[0] = pending;
      }
      __syncthreads();
      reduce(1, ns, 1, q);
    }
    ++ns;
    // (sgrab is rewritten only after the next unit's first barrier, which
    // every wave passes after this read)
    const uint32_t after = take ? us.D0 + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(sgrab[0]))
                                : (pos + 2 < us.S2 ? us.static_unit(pos + 2) : nunits);
    ucur = unext;
    unext = after;
    if (ucur >= nunits) break;  // uniform
    if (ns == kSchedCap) {
      write_out(ns);
      ns = 0;
    }
  }
  write_out(ns);
}

// Medium-M variant, 16 < M <= 80 (the batched lm_head of several requests):
// a small GEMM. With the hi/lo split the A side has 2M rows, too many to
// keep per wave, so the workgroup streams K in chunks through LDS: a chunk
// holds the workgroup's 64*NT weight rows and all 2M A rows (hi parts in
// rows 0..M-1, lo parts in rows M..2M-1), each KC k-blocks long. Eight waves
// split the 4*NT x ceil(M/8) output tiles of the workgroup 4 x 2 (16*NT
// weight rows by half the A blocks), so each B fragment read from LDS feeds
// up to 5 MFMAs and each A fragment NT, which keeps LDS traffic under its
// bandwidth and the registers of a wave under 256.
// Loads run two chunks ahead in registers (weights first, then X, in the
// order they are consumed), and there is no global store before the end, so
// the compiler never drains the prefetch. The output tile is assembled in
// LDS and y = hi + lo is written row by row.
// Two tiles are used: 128 rows x all of K (NT = 2), and, with K split in
// halves (SPLIT), 256 rows x half of K (NT = 4), both in chunks of 2
// k-blocks (KC = 2). For a compute unit's share of the weights the split
// reads half the activation bytes and does 2/3 of the LDS traffic per
// weight byte (larger wave tiles).
// LDS rows are padded by 32 bytes: on gfx950 a ds_read_b128 whose 16 lanes
// of a fragment column read 16 rows is conflict-free when the row stride
// is 32 mod 64 bytes (measured with the LDS bank-conflict counter: 4
// cycles per read at strides 160, 224, 288, 352; 8 cycles at 144, 272 and
// every other multiple of 16 tried). A 16-byte pad doubled the fragment
// reads' LDS time. With the 32-byte pad a K chunk of 4 k-blocks no longer
// fits twice in LDS beside the A rows, hence KC = 2. Measured on MI355X at
// [72 x 5120] x [32000 x 5120]: one pass 87.5 -> 79 us, split 82 -> 77 us.
constexpr int kMrMaxM = 80;                     // activation rows per launch
constexpr int kMrWaves = 8;
constexpr int kMrThreads = kMrWaves * kWave;
// Tile of a workgroup with NT weight tiles per wave (4 wave groups of 16*NT
// rows) and K chunks of KC k-blocks.
template <int NT, int KC>
struct MrShape {
  static constexpr int rows = 64 * NT;                              // weight rows per workgroup
  static constexpr int stride = KC * 64 + 32;                       // bytes per LDS row of a chunk (padded)
  static constexpr int tpr = KC * 4;                                // threads per weight row of a chunk
  static constexpr int rpq = kMrThreads / tpr;                      // weight rows per load instruction
  static constexpr int bq = rows / rpq;                             // weight loads per thread per chunk
  static constexpr int aq = (kMrMaxM * KC * 8 + kMrThreads - 1) / kMrThreads;  // X float4 loads per thread
};

template <int MB2, int NT, int KC, bool SPLIT>
__global__ __launch_bounds__(kMrThreads) void gemv_mrows_kernel(GemvParams p) {
  using S = MrShape<NT, KC>;
  // Row block and K half of this workgroup. With SPLIT, workgroup b takes
  // half h = (b / 8) % 2 of row block 8 * (b / 16) + b % 8, so the two
  // halves of a block are 8 apart (the same XCD when workgroups go to the
  // XCDs in turn); blocks past the last leave at once.
  const int rb = SPLIT ? static_cast<int>(((blockIdx.x >> 4) << 3) | (blockIdx.x & 7)) : static_cast<int>(blockIdx.x);
  const int h = SPLIT ? static_cast<int>((blockIdx.x >> 3) & 1) : 0;
  if (SPLIT && rb * S::rows >= p.N) return;  // uniform: before any barrier
  // 2*MB2 A blocks of 16 rows (rows past 2M are zero), MB2 per wave group,
  // then one scratch row that takes the writes of lanes past M. The two
  // chunk buffers are separate arrays, so the compiler can see that staging
  // one never touches what the MFMAs read from the other.
  constexpr int arows = 32 * MB2;
  constexpr int bufbytes = (S::rows + arows + 1) * S::stride;
  __shared__ __align__(16) unsigned char lds0[bufbytes];
  __shared__ __align__(16) unsigned char lds1[bufbytes];
  const int M = p.M, N = p.N, K = p.K;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int ng = w & 3, mg = w >> 2;  // 32-row weight group, A block group
  const int mb0 = mg * MB2;
  const int n0 = rb * S::rows;
  const int nrows = min(S::rows, N - n0);
  const int nchunks_all = (K + 32 * KC - 1) / (32 * KC);
  // SPLIT: half 0 takes the first ceil(chunks / 2) K chunks, half 1 the rest.
  const int cbase = SPLIT && h ? (nchunks_all + 1) / 2 : 0;
  const int nchunks = SPLIT ? (h ? nchunks_all - cbase : (nchunks_all + 1) / 2) : nchunks_all;
  const uint32_t rowb = static_cast<uint32_t>(K) * 2;
  const BufRes wres = buf_res(p.W + static_cast<size_t>(n0) * K, static_cast<uint32_t>(nrows) * rowb);
  const BufRes xres = buf_res(p.X, static_cast<uint32_t>(M) * K * 4);

  // Rows of the last A block past 2M stay zero in both buffers.
  for (int e = tid; e < (arows - 2 * M) * S::stride / 16; e += kMrThreads) {
    const int off = (S::rows + 2 * M) * S::stride + 16 * e;
    *reinterpret_cast<u32x4*>(lds0 + off) = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(lds1 + off) = u32x4{0u, 0u, 0u, 0u};
  }

  // Chunk c: weight piece q of thread t is row rpq*q + t/tpr, bytes
  // 16*(t%tpr) of the chunk; X float4 q is f = t + 512q: row f/(8 KC),
  // floats 4*(f%(8 KC)).
  // Anything past N, K, M or the last chunk reads zeros.
  const int brow = tid / S::tpr, bpc = tid % S::tpr;
  u32x4 bq[3][S::bq];   // weights of chunk j: set j%3
  float4 aq[2][S::aq];  // X of chunk j: set j%2 (from L2, so one chunk less ahead)
  // Workgroup b walks its K chunks starting at chunk (b / 8) % nchunks
  // (b / 16 with SPLIT): workgroups go to the 8 XCDs in turn, so those of
  // one XCD start at different chunks and read X from different lines of its
  // L2 at any one time. (Step c of the walk is chunk rot(c); past the last step, out of
  // range.)
  const int r0 = nchunks > 0 ? static_cast<int>((blockIdx.x >> (SPLIT ? 4 : 3)) % static_cast<unsigned>(nchunks)) : 0;
  auto rot = [&](int c) { return c >= nchunks ? nchunks : (c + r0 >= nchunks ? c + r0 - nchunks : c + r0); };
  auto issue_b = [&](int set, int cs) {
    const int c = rot(cs);
    const int kb = 32 * KC * (cbase + c) + 8 * bpc;
#pragma unroll
    for (int q = 0; q < S::bq; ++q) {
      const uint32_t off = c < nchunks && kb < K
                               ? static_cast<uint32_t>(S::rpq * q + brow) * rowb + static_cast<uint32_t>(kb) * 2
                               : kBufOutOfRange;
      bq[set][q] = buf_load16_nt(wres, off);
    }
  };
  auto issue_a = [&](int set, int cs) {
    const int c = rot(cs);
    const int kc = 32 * KC * (cbase + c);
#pragma unroll
    for (int q = 0; q < S::aq; ++q) {
      const int f = tid + kMrThreads * q, m = f / (8 * KC), k = kc + 4 * (f % (8 * KC));
      const uint32_t off =
          c < nchunks && m < M && k < K ? static_cast<uint32_t>(m * K + k) * 4 : kBufOutOfRange;
      aq[set][q] = buf_load_f32x4(xres, off);
    }
  };
  // Part `part` (of KC) of moving register set -> LDS buffer b; X is
  // split into its bf16 hi and lo rows.
  auto stage_part = [&](int bset, int aset, int b, int part) {
    unsigned char* Bs = b ? lds1 : lds0;
    unsigned char* As = Bs + S::rows * S::stride;
#pragma unroll
    for (int q = 0; q < S::bq; ++q)
      if (q % KC == part) *reinterpret_cast<u32x4*>(Bs + (S::rpq * q + brow) * S::stride + 16 * bpc) = bq[bset][q];
#pragma unroll
    for (int q = 0; q < S::aq; ++q) {
      if (q % KC != part) continue;
      const int f = tid + kMrThreads * q, m = f / (8 * KC), col = f % (8 * KC);
      const float4 x = aq[aset][q];
      const uint2 s0 = split_bf16x2(x.x, x.y), s1 = split_bf16x2(x.z, x.w);
      const int rh = m < M ? m : arows, rl = m < M ? M + m : arows;  // no branch: scratch row
      *reinterpret_cast<uint2*>(As + rh * S::stride + 8 * col) = uint2{s0.x, s1.x};
      *reinterpret_cast<uint2*>(As + rl * S::stride + 8 * col) = uint2{s0.y, s1.y};
    }
  };
  auto stage = [&](int bset, int aset, int b) {
#pragma unroll
    for (int part = 0; part < KC; ++part) stage_part(bset, aset, b, part);
  };
  f32x4 acc[NT][MB2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mb = 0; mb < MB2; ++mb) acc[nt][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Computes the chunk in buffer b; part kb of staging register sets
  // (bset, aset) into buffer 1-b is placed after each k-block, so the
  // conversions and LDS writes sit between the MFMAs in program order.
  auto compute_stage = [&](int b, int bset, int aset) {
    const unsigned char* base = b ? lds1 : lds0;
    const unsigned char* Bs = base + (16 * NT * ng + i) * S::stride + 16 * g;
    const unsigned char* As = base + (S::rows + 16 * mb0 + i) * S::stride + 16 * g;
#pragma unroll
    for (int kb = 0; kb < KC; ++kb) {
      u32x4 bf[NT], af[MB2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bf[nt] = *reinterpret_cast<const u32x4*>(Bs + 16 * nt * S::stride + 64 * kb);
#pragma unroll
      for (int mb = 0; mb < MB2; ++mb) af[mb] = *reinterpret_cast<const u32x4*>(As + 16 * mb * S::stride + 64 * kb);
#pragma unroll
      for (int mb = 0; mb < MB2; ++mb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][mb] = mfma_16x16x32(af[mb], bf[nt], acc[nt][mb]);
      stage_part(bset, aset, 1 - b, kb);
    }
  };

  // Chunk j: weights in register set j%3, X in set j%2, LDS buffer j%2.
  // While chunk j is computed, the weights of chunks j+1..j+3 and the X of
  // j+1..j+2 are in flight. Step j stages chunk j+1 (interleaved with the
  // MFMAs of chunk j), then issues X of chunk j+3 and weights of chunk j+4,
  // in that order, so that each wait covers exactly the loads it needs.
  // Six steps per iteration keep every index static; the main loop has a
  // single exit (the tail after it may wait more conservatively).
  auto step = [&](auto J) {
    constexpr int j = decltype(J)::value;
    compute_stage(j % 2, (j + 1) % 3, (j + 1) % 2);
    return j;
  };
  issue_a(0, 0);
  issue_b(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_a(1, 1);
  issue_b(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  issue_b(2, 2);
  __builtin_amdgcn_sched_barrier(0);
  stage(0, 0, 0);
  issue_a(0, 2);
  issue_b(0, 3);
  __syncthreads();
  int c = 0;
#define DSPARK_MR_STEP(J)                                        \
  step(std::integral_constant<int, J>{});                        \
  issue_a((J + 1) % 2, c + J + 3);                               \
  issue_b((J + 1) % 3, c + J + 4);                               \
  __syncthreads();
  for (; c + 6 <= nchunks; c += 6) {
    DSPARK_MR_STEP(0)
    DSPARK_MR_STEP(1)
    DSPARK_MR_STEP(2)
    DSPARK_MR_STEP(3)
    DSPARK_MR_STEP(4)
    DSPARK_MR_STEP(5)
  }
  const int rest = nchunks - c;
  if (rest > 0) { DSPARK_MR_STEP(0) }
  if (rest > 1) { DSPARK_MR_STEP(1) }
  if (rest > 2) { DSPARK_MR_STEP(2) }
  if (rest > 3) { DSPARK_MR_STEP(3) }
  if (rest > 4) { DSPARK_MR_STEP(4) }
#undef DSPARK_MR_STEP

  // Output tile [2M x rows] through LDS in pieces of 64 columns (one piece
  // fits in a chunk buffer), then y[m] = hi row m + lo row M+m. Tile nt of
  // wave group ng covers workgroup rows 16*(NT*ng + nt) .. + 15.
  // SPLIT: y is this half's partial. Each half stores it (agent-scope
  // stores, which other XCDs see once they complete), waits until they have
  // completed, and then takes a ticket from its row block's word; the half
  // that draws 1 finishes second, so the other's partial is complete: it
  // reads both partials back (agent-scope loads, all in flight at once),
  // writes Y = P0 + P1 and puts the word back to 0. A sum of two terms does
  // not depend on their order, and Y does not depend on which half finished
  // first.
  float* L = reinterpret_cast<float*>(lds0);  // [arows][64]
#pragma unroll
  for (int piece = 0; piece < NT; ++piece) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = 16 * (NT * ng + nt);
      if ((r >> 6) == piece)
#pragma unroll
        for (int mb = 0; mb < MB2; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) L[(16 * (mb0 + mb) + 4 * g + v) * 64 + (r & 63) + i] = acc[nt][mb][v];
    }
    __syncthreads();
    if constexpr (SPLIT) {
      const BufRes pres = buf_res(p.part + (static_cast<size_t>(h * p.nrb + rb) * M) * S::rows,
                                  static_cast<uint32_t>(M) * S::rows * 4);
      for (int f = tid; f < M * 16; f += kMrThreads) {
        const int m = f >> 4, c = 4 * (f & 15);
        const float4 hi = *reinterpret_cast<const float4*>(L + m * 64 + c);
        const float4 lo = *reinterpret_cast<const float4*>(L + (M + m) * 64 + c);
        buf_store16_coherent(pres, static_cast<uint32_t>(m * S::rows + 64 * piece + c) * 4,
                             __builtin_bit_cast(u32x4, float4{hi.x + lo.x, hi.y + lo.y, hi.z + lo.z, hi.w + lo.w}));
      }
      if (piece + 1 == NT) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every store of the partial has completed
      }
    } else {
      for (int e = tid; e < M * 64; e += kMrThreads) {
        const int m = e >> 6, col = 64 * piece + (e & 63);
        const size_t idx = static_cast<size_t>(m) * p.ldy + n0 + col;
        if (col < nrows) p.Y[idx] = with_res(p, idx, L[m * 64 + (e & 63)] + L[(M + m) * 64 + (e & 63)]);
      }
    }
    __syncthreads();
  }
  if constexpr (SPLIT) {
    __shared__ uint32_t ticket;
    if (tid == 0) {
      ticket = __hip_atomic_fetch_add(p.tick + rb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // A ticket past 1 means the word was not 0 before this launch (a
      // workspace never zero-filled): the outputs of this block may be
      // wrong, and the caller's flag word says so.
      if (ticket > 1u && p.dirty) __hip_atomic_store(p.dirty, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (ticket == 0) return;  // uniform: the other half finishes the block
    if (tid == 0) __hip_atomic_store(p.tick + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t pbytes = static_cast<uint32_t>(M) * S::rows * 4;
    const BufRes r0 = buf_res(p.part + (static_cast<size_t>(rb) * M) * S::rows, pbytes);
    const BufRes r1 = buf_res(p.part + (static_cast<size_t>(p.nrb + rb) * M) * S::rows, pbytes);
    // Float4 q = tid + 512 j of each partial, in rounds of kQ per thread
    // (past the partial: zeros, never used).
    constexpr int kQ = (kMrMaxM * S::rows / 4 + 2 * kMrThreads - 1) / (2 * kMrThreads);
    const int nq = M * (S::rows / 4);
    for (int j0 = 0; j0 * kMrThreads < nq; j0 += kQ) {
      u32x4 a[kQ], b[kQ];
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        a[j] = buf_load16_coherent(r0, static_cast<uint32_t>(tid + kMrThreads * (j0 + j)) * 16);
        b[j] = buf_load16_coherent(r1, static_cast<uint32_t>(tid + kMrThreads * (j0 + j)) * 16);
      }
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        const int q = tid + kMrThreads * (j0 + j);
        if (q >= nq) break;
        const int m = q / (S::rows / 4), c = 4 * (q % (S::rows / 4));
        const float4 x = __builtin_bit_cast(float4, a[j]), z = __builtin_bit_cast(float4, b[j]);
        const float y[4] = {x.x + z.x, x.y + z.y, x.z + z.z, x.w + z.w};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const size_t idx = static_cast<size_t>(m) * p.ldy + n0 + c + v;
          if (c + v < nrows) p.Y[idx] = with_res(p, idx, y[v]);
        }
      }
    }
  }
}

struct Plan {
  int tkbw;     // k-blocks per wave
  bool pack;    // M <= 8: hi and lo rows share one A block
  bool shortk;  // gemv_short_kernel (at most kShortTiles tiles per workgroup)
  bool many;    // some workgroup has more than one tile
  int chunk;    // gemv_tstream_kernel tiles per LDS output chunk
  int grid;
  size_t lds;
};

constexpr size_t kLdsBytes = 160 * 1024;
constexpr int kShortTiles = 16;  // workgroups with at most this many tiles take gemv_short_kernel

// M <= 16: K slices of 32*KBW per wave, phases for longer K. Workgroups with
// at most kShortTiles tiles take the short kernel, longer ones the streaming
// kernel with its LDS output chunks.
// norm: the NORM variant, whose gamma values take registers: with hi and lo
// A blocks (M > 8) at most 2 k-blocks per wave (4 spill).
Plan make_plan(int M, int N, int K, int cus, bool norm = false) {
  Plan pl{};
  pl.pack = M <= 8;
  const int tiles = (N + 15) / 16;
  const int KB = (K + 31) / 32;
  pl.grid = std::max(1, std::min(cus, std::min(tiles, N / 2)));
  const int rounds = (wg_rows_max(N, pl.grid) + 15) / 16;
  pl.shortk = rounds <= kShortTiles;
  pl.many = rounds > 1;
  // Measured on MI355X (M = 7 and 15, K = 4096 and 12288): one tile per
  // workgroup runs fastest with 2 k-blocks per wave and phase, several tiles
  // with 4, and the short kernel beats the streaming one up to 16 tiles.
  const int kbw_max = pl.shortk ? (pl.many && !(norm && !pl.pack) ? 4 : 2) : 4;
  int kbw = 1;
  while (kbw < kbw_max && 16 * kbw < KB) kbw *= 2;
  pl.tkbw = kbw;
  const int rows = pl.pack ? 8 : 16;
  const size_t fixed = static_cast<size_t>(16) * 16 * (64 * kbw + 16) + static_cast<size_t>(2) * 16 * rows * 16 * 4;
  if (pl.shortk) {
    pl.chunk = 0;
    pl.lds = fixed + static_cast<size_t>(rounds) * rows * 16 * 4  // + the LDS outputs of its tiles
             + static_cast<size_t>(16) * 16 * 4;                     // + the NORM variant's row sums
    return pl;
  }
  const size_t per_tile = static_cast<size_t>(M) * 16 * 4;
  int chunk = static_cast<int>((kLdsBytes - fixed) / per_tile) & ~1;
  chunk = std::max(2, std::min(chunk, (rounds + 1) & ~1));
  pl.chunk = chunk;
  pl.lds = fixed + chunk * per_tile;
  return pl;
}

template <bool PACK, int KBW>
hipError_t launch_tstream(const GemvParams& prm, const Plan& pl, hipStream_t st) {
  const void* one = reinterpret_cast<const void*>(&gemv_tstream_kernel<PACK, KBW, false>);
  const void* multi = reinterpret_cast<const void*>(&gemv_tstream_kernel<PACK, KBW, true>);
  static const hipError_t attr = [&] {
    const hipError_t e = hipFuncSetAttribute(one, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
    return e != hipSuccess ? e
                           : hipFuncSetAttribute(multi, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(kLdsBytes));
  }();
  if (attr != hipSuccess) return attr;
  const bool phased = (prm.K + 32 * 16 * KBW - 1) / (32 * 16 * KBW) > 1;  // more than one K phase
  GemvParams a = prm;
  void* args[] = {&a};
  return hipLaunchKernel(phased ? multi : one, dim3(pl.grid), dim3(16 * kWave), args, pl.lds, st);
}

template <bool PACK, int KBW, bool GATED = false, bool NORM = false>
hipError_t launch_short(const GemvParams& prm, const Plan& pl, hipStream_t st) {
  const void* one = reinterpret_cast<const void*>(&gemv_short_kernel<PACK, KBW, false, GATED, NORM>);
  const void* many = reinterpret_cast<const void*>(&gemv_short_kernel<PACK, KBW, true, GATED, NORM>);
  static const hipError_t attr = [&] {
    const hipError_t e = hipFuncSetAttribute(one, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
    return e != hipSuccess ? e
                           : hipFuncSetAttribute(many, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(kLdsBytes));
  }();
  if (attr != hipSuccess) return attr;
  GemvParams a = prm;
  void* args[] = {&a};
  return hipLaunchKernel(pl.many ? many : one, dim3(pl.grid), dim3(16 * kWave), args, pl.lds, st);
}

template <bool GATED, bool NORM>
hipError_t dispatch_short(const GemvParams& prm, const Plan& pl, hipStream_t st) {
  if (pl.pack) {
    switch (pl.tkbw) {
      case 1: return launch_short<true, 1, GATED, NORM>(prm, pl, st);
      case 2: return launch_short<true, 2, GATED, NORM>(prm, pl, st);
      default: return launch_short<true, 4, GATED, NORM>(prm, pl, st);
    }
  }
  switch (pl.tkbw) {
    case 1: return launch_short<false, 1, GATED, NORM>(prm, pl, st);
    case 2: return launch_short<false, 2, GATED, NORM>(prm, pl, st);
    default:
      if constexpr (NORM) {
        return hipErrorInvalidValue;  // the plan caps NORM at 2 here
      } else {
        return launch_short<false, 4, GATED, NORM>(prm, pl, st);
      }
  }
}

hipError_t dispatch(const GemvParams& prm, const Plan& pl, hipStream_t st) {
  if (pl.tkbw > 0 && pl.shortk) return dispatch_short<false, false>(prm, pl, st);
  if (pl.tkbw > 0) {
    if (pl.pack) {
      switch (pl.tkbw) {
        case 1: return launch_tstream<true, 1>(prm, pl, st);
        case 2: return launch_tstream<true, 2>(prm, pl, st);
        default: return launch_tstream<true, 4>(prm, pl, st);
      }
    }
    switch (pl.tkbw) {
      case 1: return launch_tstream<false, 1>(prm, pl, st);
      case 2: return launch_tstream<false, 2>(prm, pl, st);
      default: return launch_tstream<false, 4>(prm, pl, st);
    }
  }
  return hipErrorInvalidValue;
}

template <int MB2, int NT = 2, int KC = 2, bool SPLIT = false>
hipError_t launch_mrows(const GemvParams& prm, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&gemv_mrows_kernel<MB2, NT, KC, SPLIT>);  // static LDS only
  GemvParams a = prm;
  void* args[] = {&a};
  const int grid = SPLIT ? 2 * prm.nrb : (prm.N + MrShape<NT, KC>::rows - 1) / MrShape<NT, KC>::rows;
  return hipLaunchKernel(fn, dim3(grid), dim3(kMrThreads), args, 0, st);
}

// Split-K launches (16 < M): ticket words, then the two halves' partials,
// each [nrb][kMrMaxM][256] fp32.
constexpr int kSplitRows = MrShape<4, 2>::rows;
int split_row_blocks(int N) { return ((N + kSplitRows - 1) / kSplitRows + 7) / 8 * 8; }
size_t split_tick_bytes(int N) { return (static_cast<size_t>(split_row_blocks(N)) * 4 + 255) / 256 * 256; }

template <int MB2>
hipError_t launch_mrows_split(const GemvParams& prm, hipStream_t st) {
  return launch_mrows<MB2, 4, 2, true>(prm, st);
}

}  // namespace

int gemv_split_tick_words(int N) { return split_row_blocks(N); }

size_t gemv_split_workspace_bytes(int N, int K, int M) {
  if (!gemv_split_fits(N, K, M)) return 0;
  return split_tick_bytes(N) + static_cast<size_t>(2) * split_row_blocks(N) * kMrMaxM * kSplitRows * 4;
}

bool gemv_split_fits(int N, int K, int M) {
  // A workgroup's weight range (256 rows of K) must stay below 2^31 bytes.
  return N >= 1 && M > 16 && K >= 1 && K <= (1 << 21);
}

hipError_t launch_gemv_split(const uint16_t* W, int N, int K, const float* X, int M, float* Y, void* workspace,
                             hipStream_t stream, const float* res, uint32_t* dirty) {
  if (!gemv_split_fits(N, K, M) || !workspace) return launch_gemv(W, N, K, X, M, Y, stream, res);
  GemvParams prm{};
  prm.W = W;
  prm.N = N;
  prm.K = K;
  prm.ldy = N;
  prm.nrb = split_row_blocks(N);
  prm.tick = static_cast<uint32_t*>(workspace);
  prm.part = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + split_tick_bytes(N));
  prm.dirty = dirty;
  // Balanced parts of at most kMrMaxM rows, one after the other on the
  // stream: each leaves the ticket words at 0 for the next.
  const int parts = (M + kMrMaxM - 1) / kMrMaxM;
  for (int part = 0; part < parts; ++part) {
    const int m0 = M * part / parts, mc = M * (part + 1) / parts - m0;
    prm.X = X + static_cast<size_t>(m0) * K;
    prm.Y = Y + static_cast<size_t>(m0) * N;
    prm.res = res ? res + static_cast<size_t>(m0) * N : nullptr;
    prm.M = mc;
    hipError_t e;
    switch (((mc + 7) / 8 + 1) / 2) {
      case 2: e = launch_mrows_split<2>(prm, stream); break;
      case 3: e = launch_mrows_split<3>(prm, stream); break;
      case 4: e = launch_mrows_split<4>(prm, stream); break;
      default: e = launch_mrows_split<5>(prm, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

bool gemv_shape_fits(int N, int K, int M) {
  if (K > (1 << 22)) return false;  // X of a launch part: <= 80 rows * K * 4 bytes; W: 128 rows * 2K
  if (M > 16) return true;
  const int cus = device_cu_count();
  if (cus <= 0) return true;  // the launch reports the missing device
  const Plan pl = make_plan(M, N, K, cus);
  return static_cast<long long>(wg_rows_max(N, pl.grid)) * K * 2 < (1LL << 31);
}

hipError_t launch_gemv(const uint16_t* W, int N, int K, const float* X, int M, float* Y,
                       hipStream_t stream, const float* res) {
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorNoDevice;
  GemvParams prm{};
  prm.W = W;
  prm.res = res;
  prm.N = N;
  prm.K = K;
  prm.ldy = N;
  if (M <= 16) {
    const Plan pl = make_plan(M, N, K, cus);
    prm.X = X;
    prm.Y = Y;
    prm.M = M;
    prm.chunk = pl.chunk;
    prm.pq = (N / 2) / pl.grid;
    prm.prem = (N / 2) % pl.grid;
    return dispatch(prm, pl, stream);
  }
  // More rows: balanced parts of at most kMrMaxM rows (each above 16).
  const int parts = (M + kMrMaxM - 1) / kMrMaxM;
  for (int part = 0; part < parts; ++part) {
    const int m0 = M * part / parts, mc = M * (part + 1) / parts - m0;
    prm.X = X + static_cast<size_t>(m0) * K;
    prm.Y = Y + static_cast<size_t>(m0) * N;
    prm.res = res ? res + static_cast<size_t>(m0) * N : nullptr;
    prm.M = mc;
    hipError_t e;
    switch (((mc + 7) / 8 + 1) / 2) {
      case 2: e = launch_mrows<2>(prm, stream); break;
      case 3: e = launch_mrows<3>(prm, stream); break;
      case 4: e = launch_mrows<4>(prm, stream); break;
      default: e = launch_mrows<5>(prm, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemv_gated(const uint16_t* W, int F, int K, const float* X, int M, float* act, float* gu,
                             hipStream_t stream) {
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorNoDevice;
  const int N = 2 * F;
  if (M <= 16 && static_cast<long long>(N) * K * 2 < (1LL << 31)) {
    const Plan pl = make_plan(M, N, K, cus);
    if (pl.shortk && pl.tkbw > 0) {
      GemvParams prm{};
      prm.W = W;
      prm.X = X;
      prm.Y = act;
      prm.N = N;
      prm.K = K;
      prm.M = M;
      prm.ldy = F;
      prm.pq = (N / 2) / pl.grid;
      prm.prem = (N / 2) % pl.grid;
      return dispatch_short<true, false>(prm, pl, stream);
    }
  }
  // Other shapes: the projection into gu [M, 2F], then the gate.
  hipError_t e = launch_gemv(W, N, K, X, M, gu, stream);
  if (e != hipSuccess) return e;
  return launch_silu_gate(gu, M, F, act, stream);
}

bool gemv_norm_fits(int N, int K, int M) {
  if (N < 2 || M < 1 || M > 16 || K < 8 || static_cast<long long>(N) * K * 2 >= (1LL << 31)) return false;
  const int cus = device_cu_count();
  if (cus <= 0) return false;
  const Plan pl = make_plan(M, N, K, cus, true);
  return pl.shortk && pl.tkbw > 0;
}

hipError_t launch_gemv_norm(const uint16_t* W, int N, int K, const float* X, int M, const uint16_t* gamma, float eps,
                            float* Y, hipStream_t stream) {
  if (!gemv_norm_fits(N, K, M)) return hipErrorInvalidValue;
  const Plan pl = make_plan(M, N, K, device_cu_count(), true);
  GemvParams prm{};
  prm.W = W;
  prm.X = X;
  prm.Y = Y;
  prm.N = N;
  prm.K = K;
  prm.M = M;
  prm.ldy = N;
  prm.pq = (N / 2) / pl.grid;
  prm.prem = (N / 2) % pl.grid;
  prm.gamma = gamma;
  prm.eps = eps;
  return dispatch_short<false, true>(prm, pl, stream);
}

hipError_t launch_gemv_gated_norm(const uint16_t* W, int F, int K, const float* X, int M, const uint16_t* gamma,
                                  float eps, float* act, hipStream_t stream) {
  const int N = 2 * F;
  if (F < 1 || !gemv_norm_fits(N, K, M)) return hipErrorInvalidValue;
  const Plan pl = make_plan(M, N, K, device_cu_count(), true);
  GemvParams prm{};
  prm.W = W;
  prm.X = X;
  prm.Y = act;
  prm.N = N;
  prm.K = K;
  prm.M = M;
  prm.ldy = F;
  prm.pq = (N / 2) / pl.grid;
  prm.prem = (N / 2) % pl.grid;
  prm.gamma = gamma;
  prm.eps = eps;
  return dispatch_short<true, true>(prm, pl, stream);
}

// Long streams only (more than kShortTiles tiles per workgroup, where the
// plan would take the streaming kernel): on a few tiles per CU the short
// kernel is faster (the tiny round's [4 x 256] x [4096 x 256] lm_head: 7.2
// against 10.9 us) and there is no tail to balance.
bool gemv_sched_fits(int N, int K, int M) {
  const int KB = (K + 31) / 32;
  if (N < 1 || M < 1 || M > 8 || K < 8 || KB > 2 * 16 * 4) return false;
  const int cus = device_cu_count();
  return cus > 0 && !make_plan(M, N, K, cus).shortk;
}

size_t gemv_sched_lds_bytes() {
  return static_cast<size_t>(16) * 16 * (64 * 4 + 16) + static_cast<size_t>(2) * 16 * 8 * 16 * 4 +
         static_cast<size_t>(kSchedCap) * kSchedU * 8 * 16 * 4 + static_cast<size_t>(kSchedCap) * 4 + 2 * 4;
}

template <int NPH>
hipError_t launch_sched(const GemvParams& prm, uint32_t* counter, int grid, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&gemv_sched_kernel<NPH>);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (attr != hipSuccess) return attr;
  GemvParams a = prm;
  uint32_t* c = counter;
  void* args[] = {&a, &c};
  return hipLaunchKernel(fn, dim3(grid), dim3(16 * kWave), args, gemv_sched_lds_bytes(), st);
}

hipError_t launch_gemv_sched(const uint16_t* W, int N, int K, const float* X, int M, float* Y, uint32_t* counter,
                             hipStream_t stream) {
  if (!gemv_sched_fits(N, K, M) || !counter) return launch_gemv(W, N, K, X, M, Y, stream);
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorNoDevice;
  GemvParams prm{};
  prm.W = W;
  prm.X = X;
  prm.Y = Y;
  prm.N = N;
  prm.K = K;
  prm.M = M;
  prm.ldy = N;
  const int KB = (K + 31) / 32;
  // Static contiguous units per workgroup: 90% of an equal share (the rest
  // is handed out). Measured on MI355X at [7 x 4096] x [151936 x 4096]:
  // 0% (b and b + G, then all from the counter) 188.5 us, 50% 180 us, 80%
  // 179 us, 90% 178.5 us, 100% (only the remainder handed out) 185 us, equal
  // shares 187 us; at K = 2048: 102, 96, 92.5, 91.4, 93 and 93.6 us.
  const int S = sched_static_units(((N + 15) / 16 + kSchedU - 1) / kSchedU, cus);
  prm.chunk = S >= 2 ? S : 0;
  return KB <= 16 * 4 ? launch_sched<1>(prm, counter, cus, stream) : launch_sched<2>(prm, counter, cus, stream);
}

}  // namespace dspark
