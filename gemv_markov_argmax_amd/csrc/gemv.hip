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
//  * The weights stream from HBM exactly once, 16 bytes per lane per load,
//    straight into the B operand of v_mfma_f32_16x16x32_bf16: lane l loads
//    8 consecutive bf16 of weight row (16*tile + l%16), so one instruction
//    covers 16 rows x 64 contiguous bytes and no repacking is needed.
//  * The activations are fp32. Each is split exactly into two bf16 terms,
//    x = hi + lo + O(2^-17 |x|), and both terms enter the A operand, so the
//    product keeps ~16 bits of the activation against the bf16 weight and
//    accumulates in fp32. For M <= 8 the hi and lo rows share one 16-row A
//    block (rows 0..7 hi, 8..15 lo): one MFMA per 1 KB of weights.
//    The A fragments of a K-chunk sit in LDS, built once per chunk by the
//    whole workgroup.
//  * With M <= 16 the MFMA work per weight byte is tiny (an MFMA per KB),
//    so the kernel is bound by HBM: the design goal is bytes in flight.
//    Each wave keeps two stages of 8 outstanding 16-byte loads per lane.
//  * Work split: 16-row tiles are dealt to workgroups in contiguous ranges.
//    When there are few tiles (small N), a tile's K range is split over S
//    waves of one workgroup in 64-element granules (granule q goes to
//    segment q mod S) and the S partial tiles are added in LDS in a fixed
//    order. The summation order of an output depends on (K, S) only, never
//    on M or on the tile's position, so equal weight rows give bit-equal
//    outputs and a row's result does not depend on the other rows.
#include "dspark_internal.h"

#include <algorithm>

namespace dspark {
namespace {

struct GemvParams {
  const uint16_t* W;
  const float* X;
  float* Y;
  int N, K, M;   // M rows in this launch
  int ldy;       // row stride of Y
  int S;         // K segments per tile
  int KG;        // 64-element granules in K
  int KGC;       // granules per LDS chunk
  int tiles;     // ceil(N / 16)
  int chunk;     // gemv_tstream_kernel: tiles whose outputs are staged in LDS at once (even)
};

template <int NA, bool PACK, int NW, int TB>
__global__ __launch_bounds__(NW * kWave) void gemv_kernel(GemvParams p) {
  constexpr int F = PACK ? 1 : 2 * NA;           // A fragments per k-block (= accumulators per tile)
  constexpr int GU = TB >= 4 ? 1 : 4 / TB;       // granules per pipeline stage
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4* Alds = reinterpret_cast<u32x4*>(smem);  // [KGC*2][F][64]
  float* red = reinterpret_cast<float*>(smem + static_cast<size_t>(p.KGC) * 2 * F * kWave * 16);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int S = p.S, P = NW / S, pw = w / S, s = w - pw * S;
  const int N = p.N, K = p.K, M = p.M, KGC = p.KGC, KG = p.KG;
  const int nchunks = (KG + KGC - 1) / KGC;

  const int t0 = static_cast<int>((static_cast<long long>(blockIdx.x) * p.tiles) / gridDim.x);
  const int t1 = static_cast<int>((static_cast<long long>(blockIdx.x + 1) * p.tiles) / gridDim.x);
  const int per_round = P * TB;
  const int rounds = (t1 - t0 + per_round - 1) / per_round;

  for (int rd = 0; rd < rounds; ++rd) {
    int tile[TB];
    bool tvalid[TB];
    const uint16_t* wrow[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      tile[tb] = t0 + (rd * P + pw) * TB + tb;
      tvalid[tb] = tile[tb] < t1;
      const int row = min(tile[tb] * 16 + i, N - 1);  // out-of-range rows read a valid row, never stored
      wrow[tb] = p.W + static_cast<size_t>(row) * K + 8 * g;
    }
    f32x4 acc[TB][F];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int f = 0; f < F; ++f) acc[tb][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < nchunks; ++c) {
      const int q0 = c * KGC, q1 = min(KG, q0 + KGC);
      if (nchunks > 1 || rd == 0) {
        if (!(rd == 0 && c == 0)) __syncthreads();  // previous chunk fully consumed
        // Build the A fragments of granules [q0, q1): entry e = (kbl*F + f)*64 + lane.
        const int nent = (q1 - q0) * 2 * F * kWave;
        for (int e = tid; e < nent; e += NW * kWave) {
          const int ln = e & 63, fk = e >> 6, f = fk % F, kbl = fk / F;
          const int ii = ln & 15, gg = ln >> 4;
          const int k = (q0 * 2 + kbl) * 32 + 8 * gg;
          int m, half;
          if (PACK) {
            m = ii & 7;
            half = ii >> 3;
          } else {
            m = 16 * (f >> 1) + ii;
            half = f & 1;
          }
          u32x4 v = {0u, 0u, 0u, 0u};
          if (m < M && k < K) {
            const float4* xp = reinterpret_cast<const float4*>(p.X + static_cast<size_t>(m) * K + k);
            const float4 x0 = xp[0], x1 = xp[1];
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            uint32_t hb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const uint32_t h = bf16_bits_rne(xs[j]);
              hb[j] = half ? bf16_bits_rne(xs[j] - bf16_bits_to_f32(h)) : h;
            }
            v = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                      hb[6] | (hb[7] << 16)};
          }
          Alds[e] = v;
        }
        __syncthreads();
      }

      // This wave's granules of the chunk: q = qs + j*S, j < nq.
      const int qs = q0 + ((s - q0 % S) % S + S) % S;
      const int nq = qs < q1 ? (q1 - qs + S - 1) / S : 0;

      auto load_stage = [&](u32x4 (&buf)[GU][TB][2], int j0) {
#pragma unroll
        for (int u = 0; u < GU; ++u) {
          const int j = j0 + u;
          const int q = qs + j * S;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int kk = (2 * q + h) * 32;
            const bool ok = (j < nq) && (kk + 8 * g < K);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
              buf[u][tb][h] = ok ? load16_stream(wrow[tb] + kk) : u32x4{0u, 0u, 0u, 0u};
          }
        }
      };
      auto compute_stage = [&](u32x4 (&buf)[GU][TB][2], int j0) {
#pragma unroll
        for (int u = 0; u < GU; ++u) {
          const int j = j0 + u;
          if (j < nq) {
            const int ql = qs + j * S - q0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
              for (int f = 0; f < F; ++f) {
                const u32x4 av = Alds[((ql * 2 + h) * F + f) * kWave + lane];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) acc[tb][f] = mfma_16x16x32(av, buf[u][tb][h], acc[tb][f]);
              }
            }
          }
        }
      };

      u32x4 bufA[GU][TB][2], bufB[GU][TB][2];
      load_stage(bufA, 0);
      for (int j0 = 0; j0 < nq; j0 += 2 * GU) {
        load_stage(bufB, j0 + GU);
        compute_stage(bufA, j0);
        load_stage(bufA, j0 + 2 * GU);
        compute_stage(bufB, j0 + GU);
      }
    }

    // ---- epilogue: y = (sum of hi products) + (sum of lo products)
    if (S == 1) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (!tvalid[tb]) continue;
        const int n = tile[tb] * 16 + i;
        if (PACK) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float lo = __shfl_down(acc[tb][0][v], 32);
            const int m = 4 * g + v;
            if (g < 2 && m < M && n < N) p.Y[static_cast<size_t>(m) * p.ldy + n] = acc[tb][0][v] + lo;
          }
        } else {
#pragma unroll
          for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int m = 16 * a + 4 * g + v;
              if (m < M && n < N)
                p.Y[static_cast<size_t>(m) * p.ldy + n] = acc[tb][2 * a][v] + acc[tb][2 * a + 1][v];
            }
        }
      }
    } else {
      // Partial tiles of the S segments -> LDS, then a fixed-order sum.
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int f = 0; f < F; ++f)
          reinterpret_cast<f32x4*>(red)[((w * TB + tb) * F + f) * kWave + lane] = acc[tb][f];
      __syncthreads();
      constexpr int ROWS = PACK ? 8 : 16 * NA;
      const int items = P * TB * ROWS * 16;
      for (int it = tid; it < items; it += NW * kWave) {
        const int col = it & 15;
        const int rest = it >> 4;
        const int m = rest % ROWS;
        const int tb = (rest / ROWS) % TB;
        const int pp = rest / (ROWS * TB);
        const int t = t0 + (rd * P + pp) * TB + tb;
        const int n = t * 16 + col;
        if (t >= t1 || m >= M || n >= N) continue;
        int fh, fl, rh, rl;
        if (PACK) {
          fh = fl = 0;
          rh = m;
          rl = m + 8;
        } else {
          fh = 2 * (m >> 4);
          fl = fh + 1;
          rh = rl = m & 15;
        }
        float hi = 0.f, lo = 0.f;
        for (int ss = 0; ss < S; ++ss) {
          const int wv = pp * S + ss;
          hi += red[(((wv * TB + tb) * F + fh) * kWave + 16 * (rh >> 2) + col) * 4 + (rh & 3)];
          lo += red[(((wv * TB + tb) * F + fl) * kWave + 16 * (rl >> 2) + col) * 4 + (rl & 3)];
        }
        p.Y[static_cast<size_t>(m) * p.ldy + n] = hi + lo;
      }
      __syncthreads();
    }
  }
}

// Short variant for M <= 16: at most two 16-row tiles per workgroup (the
// small projections of a draft layer). It follows the same plan as
// gemv_tstream_kernel below but with the shortest dependency chain: plain
// guarded loads and a direct store of each output tile. (The store makes the
// wave wait for every load in flight before its next tile, which only
// matters when there are many tiles per workgroup.)
//
// Every 16-row tile is split along K over the 16 waves of a workgroup: wave w
// owns k-blocks [P*16*KBW + w*KBW, +KBW) of phase P (k-block = 32 values),
// so all waves do equal work on every tile and the A fragments of a wave
// (its K slice of X, split into bf16 hi/lo) fit in registers. K longer than
// 16*KBW k-blocks is covered in phases; phase P > 0 adds into Y, in order.
//
// Weight loads are contiguous runs: each instruction covers 16/KBW rows x
// 64*KBW bytes (whole 128-byte lines for KBW >= 2), which the memory system
// serves noticeably faster than the 16-rows x 64-bytes pattern of loading
// the MFMA B operand directly. The wave transposes its segment through a
// private LDS area (rows padded by 16 bytes: conflict-free writes and B
// reads) and runs the MFMAs from there. Loads run two tiles ahead.
//
// M <= 8 (PACK): rows 0..7 of the A block hold the hi parts, rows 8..15 the
// lo parts, one MFMA per k-block; each wave folds lo onto hi. 8 < M <= 16:
// hi and lo are two A blocks with their own accumulators, added per wave.
// The 16 per-wave partial tiles are summed in LDS in wave order (double
// buffered, one barrier per tile).
template <bool PACK, int KBW>
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

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int N = p.N, K = p.K, M = p.M;
  const int KB = (K + 31) / 32;
  const int phases = (KB + 16 * KBW - 1) / (16 * KBW);

  // Contiguous row range [r0, r1) of this workgroup, balanced to 2 rows (the
  // granularity of a load instruction); tiles are 16 rows from r0, the last
  // one masked at r1.
  const int r0 = static_cast<int>((static_cast<long long>(blockIdx.x) * (N / 2)) / gridDim.x) * 2;
  const int r1 = blockIdx.x + 1 == gridDim.x
                     ? N
                     : static_cast<int>((static_cast<long long>(blockIdx.x + 1) * (N / 2)) / gridDim.x) * 2;
  const int rounds = (r1 - r0 + 15) / 16;
  const int lrow = lane / LPR, lchunk = lane % LPR;
  unsigned char* wtr = tr + w * 16 * RS;
  unsigned char* wr_base = wtr + lrow * RS + 16 * lchunk;  // + RPI*q*RS
  const unsigned char* rd_base = wtr + i * RS + 16 * g;   // + 64*kb

  for (int ph = 0; ph < phases; ++ph) {
    const int kseg = 32 * KBW * (ph * NW + w);  // first k of this wave's segment
    const bool lk_ok = kseg + 8 * lchunk < K;
    u32x4 afr[KBW][F];

    auto load = [&](u32x4 (&b)[NLD], int rr) {
      const int row0 = r0 + rr * 16 + lrow;
      const bool ok = rr < rounds && lk_ok;
      const uint16_t* src = p.W + static_cast<size_t>(ok ? row0 : 0) * K + kseg + 8 * lchunk;
      const size_t step = static_cast<size_t>(RPI) * K;
#pragma unroll
      for (int q = 0; q < NLD; ++q)
        b[q] = (ok && row0 + RPI * q < r1) ? load16_stream(src + q * step) : u32x4{0u, 0u, 0u, 0u};
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
    auto reduce_store = [&](int buf, int rr) {
      for (int it = tid; it < ROWS * 16; it += NW * kWave) {
        const int col = it & 15, m = it >> 4;
        const int n = r0 + rr * 16 + col;
        if (m < M && n < r1) {
          float y = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) y += red[((buf * NW + ww) * ROWS + m) * 16 + col];
          float* yp = p.Y + static_cast<size_t>(m) * p.ldy + n;
          *yp = ph == 0 ? y : *yp + y;  // the same thread wrote it in the previous phase
        }
      }
    };

    // The first two tiles' weight loads go out before the A fragments are
    // built: they do not depend on X, so the two memory latencies overlap.
    u32x4 b0[NLD], b1[NLD];
    load(b0, 0);
    load(b1, 1);
    // A fragments: k-block kb of the segment covers k = kseg + 32*kb + 8*g + (0..7).
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      const int k = kseg + 32 * kb + 8 * g;
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int m = PACK ? (i & 7) : i;
        const int half = PACK ? (i >> 3) : f;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < M && k < K) {
          const float4* xp = reinterpret_cast<const float4*>(p.X + static_cast<size_t>(m) * K + k);
          const float4 x0 = xp[0], x1 = xp[1];
          const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          uint32_t hb[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t hv = bf16_bits_rne(xs[e]);
            hb[e] = half ? bf16_bits_rne(xs[e] - bf16_bits_to_f32(hv)) : hv;
          }
          v = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
        }
        afr[kb][f] = v;
      }
    }
    for (int rr = 0; rr < rounds; rr += 2) {
      compute_publish(b0, 0);
      load(b0, rr + 2);
      __syncthreads();
      reduce_store(0, rr);
      if (rr + 1 < rounds) {
        compute_publish(b1, 1);
        load(b1, rr + 3);
        __syncthreads();
        reduce_store(1, rr + 1);
      }
    }
    if (phases > 1) {
      __threadfence_block();  // this phase's Y stores complete before the next phase reads them
      __syncthreads();
    }
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

  // Contiguous row range [r0, r1) of this workgroup, balanced to 2 rows (the
  // granularity of a load instruction); tiles are 16 rows from r0, the last
  // one masked at r1.
  const int r0 = static_cast<int>((static_cast<long long>(blockIdx.x) * (N / 2)) / gridDim.x) * 2;
  const int r1 = blockIdx.x + 1 == gridDim.x
                     ? N
                     : static_cast<int>((static_cast<long long>(blockIdx.x + 1) * (N / 2)) / gridDim.x) * 2;
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
    constexpr int KH = KBW * F * 8 > 32 ? KBW / 2 : KBW;
#pragma unroll
    for (int k0 = 0; k0 < KBW; k0 += KH) {
      float4 xr[KH][F][2];
#pragma unroll
      for (int kk = 0; kk < KH; ++kk)
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const int m = PACK ? (i & 7) : i, k = kseg + 32 * (k0 + kk) + 8 * g;
          const uint32_t off = m < M && k < K ? static_cast<uint32_t>(m * K + k) * 4 : kBufOutOfRange;
          xr[kk][f][0] = buf_load_f32x4(xres, off);
          xr[kk][f][1] = buf_load_f32x4(xres, off + 16);
        }
#pragma unroll
      for (int kk = 0; kk < KH; ++kk)
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const int half = PACK ? (i >> 3) : f;
          const float4 x0 = xr[kk][f][0], x1 = xr[kk][f][1];
          const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          uint32_t hb[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t hv = bf16_bits_rne(xs[e]);
            hb[e] = half ? bf16_bits_rne(xs[e] - bf16_bits_to_f32(hv)) : hv;
          }
          afr[k0 + kk][f] = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                                  hb[6] | (hb[7] << 16)};
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
  // Tiles [c0, c1), two per iteration with a single exit: the back edge
  // always carries b0 older than b1, so the head waits for b0 alone. Chunks
  // are even sized but the last; its odd tail runs the second half on the
  // zeros of tile c1 and keeps nothing.
  auto run_tiles = [&]() {
    for (int rr = c0; rr < c1; rr += 2) {
      compute_publish(b0, 0);
      load(b0, rr + 2);
      __syncthreads();
      reduce(0, rr);
      compute_publish(b1, 1);
      load(b1, rr + 3);
      __syncthreads();
      if (rr + 1 < c1) reduce(1, rr + 1);
    }
  };
  // The chunk's outputs, row by row: columns [r0 + 16*c0, min(r1, r0 + 16*c1)).
  auto write_out = [&]() {
    __syncthreads();
    const int n0 = r0 + 16 * c0, cols = min(r1, r0 + 16 * c1) - n0;
    for (int m = 0; m < M; ++m)
      for (int j = tid; j < cols; j += NW * kWave)
        p.Y[static_cast<size_t>(m) * p.ldy + n0 + j] = ylds[(j >> 4) * M * 16 + m * 16 + (j & 15)];
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

struct Plan {
  int tkbw;     // gemv_tstream_kernel / gemv_short_kernel k-blocks per wave (0: neither)
  bool shortk;  // gemv_short_kernel (at most two tiles per workgroup)
  int chunk;    // gemv_tstream_kernel tiles per LDS output chunk
  int NA;
  bool pack;
  int NW;
  int TB;
  int S;
  int KGC;
  int grid;
  size_t lds;
};

constexpr size_t kLdsBytes = 160 * 1024;

Plan make_plan(int M, int N, int K, int cus) {
  Plan pl{};
  if (M <= 8) {
    pl.NA = 1, pl.pack = true, pl.NW = 16;
  } else if (M <= 16) {
    pl.NA = 1, pl.pack = false, pl.NW = 16;
  } else {
    pl.NA = (M + 15) / 16, pl.pack = false, pl.NW = 8;
  }
  const int F = pl.pack ? 1 : 2 * pl.NA;
  const int tiles = (N + 15) / 16, KG = (K + 63) / 64;
  if (M <= 16) {
    // K slices of 32*KBW per wave, phases for longer K. Workgroups with at
    // most two tiles take the short kernel (up to 8 k-blocks per wave with
    // packed rows); longer ones the LDS-staged streaming kernel, whose
    // registers allow 4.
    const int KB = (K + 31) / 32;
    pl.grid = std::max(1, std::min(cus, std::min(tiles, N / 2)));
    const int rows_max = 2 * ((N / 2 + pl.grid - 1) / pl.grid) + 1;  // rows of the largest workgroup
    const int rounds = (rows_max + 15) / 16;
    pl.shortk = rounds <= 2;
    const int kbw_max = pl.shortk && pl.pack ? 8 : 4;
    int kbw = 1;
    while (kbw < kbw_max && 16 * kbw < KB) kbw *= 2;
    pl.tkbw = kbw;
    pl.S = 16;
    pl.TB = 1;
    pl.KGC = KG;
    const int rows = pl.pack ? 8 : 16;
    const size_t fixed = static_cast<size_t>(16) * 16 * (64 * kbw + 16) + static_cast<size_t>(2) * 16 * rows * 16 * 4;
    if (pl.shortk) {
      pl.chunk = 0;
      pl.lds = fixed;
      return pl;
    }
    const size_t per_tile = static_cast<size_t>(M) * 16 * 4;
    int chunk = static_cast<int>((kLdsBytes - fixed) / per_tile) & ~1;
    chunk = std::max(2, std::min(chunk, (rounds + 1) & ~1));
    pl.chunk = chunk;
    pl.lds = fixed + chunk * per_tile;
    return pl;
  }
  const int cap = cus * pl.NW;
  int S = 1;
  if (2 * tiles < cap)
    while (S < pl.NW && S < KG && tiles * S < cap) S *= 2;
  pl.S = S;
  const int P = pl.NW / S;
  const size_t gran = static_cast<size_t>(2) * F * kWave * 16;
  const size_t red1 = S > 1 ? static_cast<size_t>(pl.NW) * F * kWave * 16 : 0;
  if (static_cast<size_t>(KG) * gran + red1 <= kLdsBytes) {
    pl.TB = 1;
    pl.KGC = KG;
    pl.grid = std::min(cus, (tiles + P - 1) / P);
    pl.lds = KG * gran + red1;
    return pl;
  }
  const int tbmax = F <= 2 ? 4 : 1;
  int tb = (tiles + P * cus - 1) / (P * cus);
  tb = tb <= 1 ? 1 : (tb <= 2 ? 2 : 4);
  pl.TB = std::min(tb, tbmax);
  const size_t red = S > 1 ? static_cast<size_t>(pl.NW) * pl.TB * F * kWave * 16 : 0;
  pl.KGC = std::max<int>(1, static_cast<int>((kLdsBytes - red) / gran));
  pl.grid = (tiles + P * pl.TB - 1) / (P * pl.TB);
  pl.lds = pl.KGC * gran + red;
  return pl;
}

template <int NA, bool PACK, int NW, int TB>
hipError_t launch_inst(const GemvParams& prm, const Plan& pl, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&gemv_kernel<NA, PACK, NW, TB>);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (attr != hipSuccess) return attr;
  GemvParams a = prm;
  void* args[] = {&a};
  return hipLaunchKernel(fn, dim3(pl.grid), dim3(NW * kWave), args, pl.lds, st);
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

template <bool PACK, int KBW>
hipError_t launch_short(const GemvParams& prm, const Plan& pl, hipStream_t st) {
  const void* fn = reinterpret_cast<const void*>(&gemv_short_kernel<PACK, KBW>);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (attr != hipSuccess) return attr;
  GemvParams a = prm;
  void* args[] = {&a};
  return hipLaunchKernel(fn, dim3(pl.grid), dim3(16 * kWave), args, pl.lds, st);
}

hipError_t dispatch(const GemvParams& prm, const Plan& pl, hipStream_t st) {
  if (pl.tkbw > 0 && pl.shortk) {
    if (pl.pack) {
      switch (pl.tkbw) {
        case 1: return launch_short<true, 1>(prm, pl, st);
        case 2: return launch_short<true, 2>(prm, pl, st);
        case 4: return launch_short<true, 4>(prm, pl, st);
        default: return launch_short<true, 8>(prm, pl, st);
      }
    }
    switch (pl.tkbw) {
      case 1: return launch_short<false, 1>(prm, pl, st);
      case 2: return launch_short<false, 2>(prm, pl, st);
      default: return launch_short<false, 4>(prm, pl, st);
    }
  }
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
  switch (pl.NA) {
    case 2: return launch_inst<2, false, 8, 1>(prm, pl, st);
    case 3: return launch_inst<3, false, 8, 1>(prm, pl, st);
    case 4: return launch_inst<4, false, 8, 1>(prm, pl, st);
    case 5: return launch_inst<5, false, 8, 1>(prm, pl, st);
    case 6: return launch_inst<6, false, 8, 1>(prm, pl, st);
    case 7: return launch_inst<7, false, 8, 1>(prm, pl, st);
    default: return launch_inst<8, false, 8, 1>(prm, pl, st);
  }
}

}  // namespace

hipError_t launch_gemv(const uint16_t* W, int N, int K, const float* X, int M, float* Y,
                       hipStream_t stream) {
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorNoDevice;
  constexpr int kMaxRows = 128;  // 8 row groups of 16 per launch
  for (int m0 = 0; m0 < M; m0 += kMaxRows) {
    const int mc = std::min(kMaxRows, M - m0);
    const Plan pl = make_plan(mc, N, K, cus);
    GemvParams prm{};
    prm.W = W;
    prm.X = X + static_cast<size_t>(m0) * K;
    prm.Y = Y + static_cast<size_t>(m0) * N;
    prm.N = N;
    prm.K = K;
    prm.M = mc;
    prm.ldy = N;
    prm.S = pl.S;
    prm.KG = (K + 63) / 64;
    prm.KGC = pl.KGC;
    prm.tiles = (N + 15) / 16;
    prm.chunk = pl.chunk;
    const hipError_t e = dispatch(prm, pl, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
