// Weight-stationary small-M GEMV over Q8_0 weights on gfx950 matrix cores.
//
// Y[m, n] = sum_t X[m, t] * W[n, t], with W in Q8_0 blocks: entries
// 32b .. 32b + 31 of row n are d[n, b] * q[n, t], q int8 [N, K], d IEEE
// binary16 [N, K / 32]; X fp32 [M, K], Y fp32 [M, N].
//
// SharpInference #441, "Proposed work": the weight-stationary matvec it
// would reuse targets quantized weights; ds4 #772, "Summary": the GPU path
// takes Q8_0 weights. A Q8_0 weight costs 1.0625 bytes instead of 2.
//
// Design on gfx950 (the bf16 streaming kernel's structure, one byte per
// weight):
//  * 16 waves per workgroup, one workgroup per CU over a balanced contiguous
//    row range; every 16-row tile is split along K over the waves (8 blocks
//    of 32 entries per wave and phase, 4 for more than 8 rows of X), two
//    tiles of loads in flight.
//  * Each wave loads its 16 x 256-byte (128-byte) segment of a tile in whole
//    128-byte lines (non-temporal raw buffer loads; zeros past the range),
//    together with the tile's scales, and stages both in a private LDS area.
//    The scales come two per 32-bit load where rows allow (K / 32 even):
//    a wave's scales of a tile are 16 rows apart, so each load instruction
//    touches 16 lines for a few bytes of each, and halving the instructions
//    took the Qwen3-8B-shaped Q8_0 lm_head from ~114 to ~109 us.
//  * B fragments: 8 quants per lane, converted exactly to bf16 (a signed
//    byte has at most 8 significant bits: one sign-extending convert per
//    value and a byte permute per pair). A fragments: X split exactly into
//    bf16 hi and lo (residual <= 2^-17 |x|), as in the bf16 kernel.
//  * Each 32-entry block is one v_mfma_f32_16x16x32_bf16 on a fresh
//    accumulator, scaled by its block's scale and added in fp32. The 16
//    per-wave partial tiles are summed in LDS in wave order; phases add
//    there; outputs go out once per chunk of tiles. The summation order
//    depends on the shape only.
#include "dspark_internal.h"

#include <algorithm>

namespace dspark {
namespace {

struct Q8Params {
  const int8_t* Wq;
  const uint16_t* Wd;
  const float* X;
  float* Y;
  int N, K, M;  // M rows in this launch (<= 16)
  int ldy;
  int ldd;      // binary16 scales per row of Wd (>= K / 32; more when rows are padded)
  int chunk;    // tiles whose outputs are staged in LDS at once (even)
  int pq, prem; // row pairs per workgroup: N/2 = pq * gridDim.x + prem
};

constexpr int kQNW = 16;  // waves per workgroup
constexpr size_t kQLds = 160 * 1024;
constexpr int kQShortTiles = 16;  // workgroups with at most this many tiles take gemv_q8_short_kernel

__device__ __forceinline__ int2 q8_rows(const Q8Params& p) {
  const int b = blockIdx.x;
  const int r0 = 2 * (b * p.pq + min(b, p.prem));
  const int r1 = b + 1 == static_cast<int>(gridDim.x) ? p.N : 2 * ((b + 1) * p.pq + min(b + 1, p.prem));
  return int2{r0, r1};
}

inline int q8_rows_max(int N, int grid) {
  const int q = (N / 2) / grid, rem = (N / 2) % grid;
  return std::max(2 * (q + (rem > 0 ? 1 : 0)), 2 * q + (N & 1));
}

// Eight signed bytes (two dwords, entry order) as eight bf16 values, exactly.
__device__ __forceinline__ u32x4 q8x8_to_bf16(uint2 v) {
  auto cv = [](uint32_t w, int byte) { return __builtin_bit_cast(uint32_t, static_cast<float>(static_cast<int8_t>(w >> (8 * byte)))); };
  auto pk = [](uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x07060302u); };
  return u32x4{pk(cv(v.x, 0), cv(v.x, 1)), pk(cv(v.x, 2), cv(v.x, 3)), pk(cv(v.y, 0), cv(v.y, 1)),
               pk(cv(v.y, 2), cv(v.y, 3))};
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// KBW: 32-entry blocks per wave and phase (4 or 8: 128 or 256 quant bytes
// of each row per wave). MULTI: more than one K phase (the chunk loop runs
// every phase per chunk).
template <bool PACK, bool MULTI, int KBW, bool PAIRED>
__global__ __launch_bounds__(kQNW * kWave) void gemv_q8_kernel(Q8Params p) {
  constexpr int NW = kQNW;
  constexpr int SEG = 32 * KBW;     // quant bytes of a row segment
  constexpr int RS = SEG + 16;      // padded LDS row stride
  constexpr int LPR = SEG / 16;     // lanes per row in a load instruction
  constexpr int RPI = kWave / LPR;  // rows per load instruction
  constexpr int NLD = 16 / RPI;     // load instructions per tile
  constexpr int SPL = KBW / 4;      // scale loads per lane and tile
  constexpr int F = PACK ? 1 : 2, ROWS = PACK ? 8 : 16;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* tr = smem;                                                           // [NW][16][RS] quants
  uint16_t* sc = reinterpret_cast<uint16_t*>(smem + static_cast<size_t>(NW) * 16 * RS);  // [NW][16][KBW] scales
  float* red = reinterpret_cast<float*>(sc + NW * 16 * KBW);                         // [2][NW][ROWS][16]
  float* ylds = red + 2 * NW * ROWS * 16;                                            // [chunk][M][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int K = p.K, M = p.M;
  const int KB = K / 32;
  const int phases = (KB + NW * KBW - 1) / (NW * KBW);

  const int2 rows = q8_rows(p);
  const int r0 = rows.x, r1 = rows.y;
  const int rounds = (r1 - r0 + 15) / 16;
  const int nchunks = (rounds + p.chunk - 1) / p.chunk;
  const int csize = (((rounds + nchunks - 1) / nchunks) + 1) & ~1;
  const int lrow = lane / LPR, lchunk = lane % LPR;
  unsigned char* wtr = tr + w * 16 * RS;
  unsigned char* wr_base = wtr + lrow * RS + 16 * lchunk;  // + RPI*q*RS
  const unsigned char* rd_base = wtr + i * RS + 8 * g;    // + 32*kb
  uint16_t* wsc = sc + w * 16 * KBW;

  const uint32_t rowb = static_cast<uint32_t>(K);       // quant bytes per row
  const uint32_t drow = static_cast<uint32_t>(p.ldd) * 2;  // scale bytes per row (with any padding)
  const BufRes qres = buf_res(p.Wq + static_cast<size_t>(r0) * K, static_cast<uint32_t>(r1 - r0) * rowb);
  const BufRes dres = buf_res(p.Wd + static_cast<size_t>(r0) * p.ldd, static_cast<uint32_t>(r1 - r0) * drow);
  const BufRes xres = buf_res(p.X, static_cast<uint32_t>(M) * K * 4);

  u32x4 afr[KBW][F];
  u32x4 b0[NLD], b1[NLD];
  // Scales of this lane: with an even number of blocks per row, one word of
  // two (row i, blocks 2g and 2g + 1 of the segment, lanes 2g < KBW), so a
  // wave's scales of a tile take one load instruction instead of KBW / 4;
  // else halves (row i, blocks g + 4j).
  constexpr bool paired = PAIRED;  // the host launches it for K / 32 and the row stride even only
  uint32_t s0[SPL], s1[SPL];
  int ph = 0, c0 = 0, c1 = 0, lim = 0;
  uint32_t lane_off = 0, sc_off[SPL];

  // Phase ph: this wave's segment starts at entry kseg (block kseg / 32).
  // Lanes past K start out of range and read zeros.
  auto set_phase = [&](int phase) {
    ph = phase;
    const int kseg = 32 * KBW * (ph * NW + w);
    lane_off = kseg + 16 * lchunk < K ? static_cast<uint32_t>(lrow) * rowb + static_cast<uint32_t>(kseg + 16 * lchunk)
                                      : kBufOutOfRange;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int blk = paired ? kseg / 32 + 2 * g : kseg / 32 + g + 4 * j;
      sc_off[j] = blk < KB && (!paired || 2 * g < KBW)
                      ? static_cast<uint32_t>(i) * drow + static_cast<uint32_t>(blk) * 2
                      : kBufOutOfRange;
    }
  };
  // A fragments of phase ph: block kb covers k = kseg + 32*kb + 8*g + (0..7).
  auto build_a = [&]() {
    const int kseg = 32 * KBW * (ph * NW + w);
    constexpr int XH = PACK ? 1 : 2;
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
        const uint2 sa = split_bf16x2(x0.x, x0.y), sb = split_bf16x2(x0.z, x0.w);
        const uint2 sc2 = split_bf16x2(x1.x, x1.y), sd = split_bf16x2(x1.z, x1.w);
        const u32x4 h = {sa.x, sb.x, sc2.x, sd.x}, l = {sa.y, sb.y, sc2.y, sd.y};
        if (PACK) {
          afr[k0 + kk][0] = (i >> 3) ? l : h;
        } else {
          afr[k0 + kk][0] = h;
          afr[k0 + kk][F - 1] = l;
        }
      }
    }
  };
  // Tile rr: quants and scales; rows past r1 and tiles past lim read zeros.
  auto load = [&](u32x4 (&b)[NLD], uint32_t (&s)[SPL], int rr) {
    const bool live = rr < lim;
    const uint32_t off = live ? lane_off + static_cast<uint32_t>(rr) * 16 * rowb : kBufOutOfRange;
#pragma unroll
    for (int q = 0; q < NLD; ++q) b[q] = buf_load16_nt(qres, off + static_cast<uint32_t>(q * RPI) * rowb);
    if (paired) {
      s[0] = __builtin_amdgcn_raw_buffer_load_b32(
          dres, static_cast<int>(live ? sc_off[0] + static_cast<uint32_t>(rr) * 16 * drow : kBufOutOfRange), 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        s[j] = __builtin_amdgcn_raw_buffer_load_b16(
            dres, static_cast<int>(live ? sc_off[j] + static_cast<uint32_t>(rr) * 16 * drow : kBufOutOfRange), 0, 0);
    }
  };
  auto prologue = [&](bool with_a) {
    load(b0, s0, c0);
    __builtin_amdgcn_sched_barrier(0);
    if (with_a) build_a();
    load(b1, s1, c0 + 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute_publish = [&](u32x4 (&b)[NLD], const uint32_t (&s)[SPL], int buf) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) *reinterpret_cast<u32x4*>(wr_base + RPI * q * RS) = b[q];
    if (paired) {
      if (2 * g < KBW) *reinterpret_cast<uint32_t*>(wsc + i * KBW + 2 * g) = s[0];
    } else {
#pragma unroll
      for (int j = 0; j < SPL; ++j) wsc[i * KBW + g + 4 * j] = static_cast<uint16_t>(s[j]);
    }
    float scale[KBW];  // the KBW scales of row i
#pragma unroll
    for (int j = 0; j < KBW / 4; ++j) {
      const uint2 sh = *reinterpret_cast<const uint2*>(wsc + i * KBW + 4 * j);
      scale[4 * j] = half_bits_to_float(sh.x & 0xffffu);
      scale[4 * j + 1] = half_bits_to_float(sh.x >> 16);
      scale[4 * j + 2] = half_bits_to_float(sh.y & 0xffffu);
      scale[4 * j + 3] = half_bits_to_float(sh.y >> 16);
    }
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      const u32x4 bv = q8x8_to_bf16(*reinterpret_cast<const uint2*>(rd_base + 32 * kb));
      f32x4 acc = mfma_16x16x32(afr[kb][0], bv, f32x4{0.f, 0.f, 0.f, 0.f});
      if (!PACK) acc = mfma_16x16x32(afr[kb][F - 1], bv, acc);
#pragma unroll
      for (int v = 0; v < 4; ++v) tot[v] = __builtin_fmaf(acc[v], scale[kb], tot[v]);
    }
    float* dst = red + (buf * NW + w) * ROWS * 16;
    if (PACK) {
      // lanes 0..31 hold rows 0..7 (hi), lanes 32..63 rows 8..15 (lo) of the same columns
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float lo = __shfl_down(tot[v], 32);
        if (g < 2) dst[(4 * g + v) * 16 + i] = tot[v] + lo;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[(4 * g + v) * 16 + i] = tot[v];
    }
  };
  auto reduce = [&](int buf, int rr) {
    if (tid < M * 16) {
      float y = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) y += red[((buf * NW + ww) * ROWS + (tid >> 4)) * 16 + (tid & 15)];
      float* yl = ylds + (rr - c0) * M * 16 + tid;
      *yl = ph == 0 ? y : *yl + y;
    }
  };
  // Tiles [c0, c1), two per iteration; the back edge carries b0 older than b1.
  // An odd last tile is computed alone (a chunk has an even number of tiles
  // except the last one, after which nothing reads b0 or b1 before the next
  // prologue).
  auto run_tiles = [&]() {
    int rr = c0;
    for (; rr + 2 <= c1; rr += 2) {
      compute_publish(b0, s0, 0);
      load(b0, s0, rr + 2);
      __syncthreads();
      reduce(0, rr);
      compute_publish(b1, s1, 1);
      load(b1, s1, rr + 3);
      __syncthreads();
      reduce(1, rr + 1);
    }
    if (rr < c1) {
      compute_publish(b0, s0, 0);
      __syncthreads();
      reduce(0, rr);
    }
  };
  auto write_out = [&]() {
    __syncthreads();
    const int n0 = r0 + 16 * c0, cols = min(r1, r0 + 16 * c1) - n0;
    for (int m = 0; m < M; ++m)
      for (int j = tid; j < cols; j += NW * kWave)
        p.Y[static_cast<size_t>(m) * p.ldy + n0 + j] = ylds[(j >> 4) * M * 16 + m * 16 + (j & 15)];
    __syncthreads();
  };

  if (!MULTI) {
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

// Short variant: at most kQShortTiles tiles per workgroup (the projections
// of a draft layer, where a workgroup often has a single tile). The
// streaming kernel above issues a tile's activations and weights and then
// waits for both before any MFMA: with one tile per workgroup that is one
// long memory round trip. Here K is covered in phases of 16 * KBW blocks,
// and the activations and weights of phase P + 1 are in flight while phase
// P is converted, multiplied and reduced (as in the bf16 short kernel).
// Per phase, each wave stages its 16 x 32*KBW-byte segment of the tile (and
// the segment's block scales) in a private LDS area; its activations are
// split into bf16 hi/lo in registers while the weights are on their way.
// MANY: several tiles per workgroup, one tile of weights in flight per wave,
// the next issued as soon as the current one is in LDS. The per-block
// arithmetic and the wave-order sum are those of the streaming kernel.
template <bool PACK, int KBW, bool MANY>
__global__ __launch_bounds__(kQNW * kWave) void gemv_q8_short_kernel(Q8Params p) {
  static_assert(KBW == 2 || KBW == 4 || KBW == 8, "16-row tiles need 2, 4 or 8 blocks per wave");
  constexpr int NW = kQNW;
  constexpr int SEG = 32 * KBW;     // quant bytes of a row segment
  constexpr int RS = SEG + 16;      // padded LDS row stride
  constexpr int LPR = SEG / 16;     // lanes per row in a load instruction
  constexpr int RPI = kWave / LPR;  // rows per load instruction
  constexpr int NLD = 16 / RPI;     // load instructions per tile
  constexpr int SPL = (KBW + 3) / 4;  // scale loads per lane and tile
  constexpr int F = PACK ? 1 : 2, ROWS = PACK ? 8 : 16, XH = PACK ? 1 : 2;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* tr = smem;                                                           // [NW][16][RS] quants
  uint16_t* sc = reinterpret_cast<uint16_t*>(smem + static_cast<size_t>(NW) * 16 * RS);  // [NW][16][KBW] scales
  float* red = reinterpret_cast<float*>(sc + NW * 16 * KBW);                         // [2][NW][ROWS][16]
  float* ysum = red + 2 * NW * ROWS * 16;                                            // [tiles][ROWS][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, i = lane & 15;
  const int K = p.K, M = p.M;
  const int KB = K / 32;
  const int phases = (KB + NW * KBW - 1) / (NW * KBW);

  const int2 rows = q8_rows(p);
  const int r0 = rows.x, r1 = rows.y;
  const int rounds = (r1 - r0 + 15) / 16;
  const int lrow = lane / LPR, lchunk = lane % LPR;
  unsigned char* wr_base = tr + (w * 16 + lrow) * RS + 16 * lchunk;  // + RPI*q*RS
  const unsigned char* rd_base = tr + (w * 16 + i) * RS + 8 * g;     // + 32*kb
  uint16_t* wsc = sc + w * 16 * KBW;

  const uint32_t rowb = static_cast<uint32_t>(K);       // quant bytes per row
  const uint32_t drow = static_cast<uint32_t>(p.ldd) * 2;  // scale bytes per row (with any padding)
  const BufRes qres = buf_res(p.Wq + static_cast<size_t>(r0) * K, static_cast<uint32_t>(r1 - r0) * rowb);
  const BufRes dres = buf_res(p.Wd + static_cast<size_t>(r0) * p.ldd, static_cast<uint32_t>(r1 - r0) * drow);
  const BufRes xres = buf_res(p.X, static_cast<uint32_t>(M) * K * 4);

  // Phase ph, tile t: lane offsets of the quants (16 bytes of row lrow) and
  // of the scales (row i, blocks g + 4j of the segment). A lane past K or
  // past the segment, or a phase past the last, reads zeros.
  auto q_off = [&](int ph, int t) -> uint32_t {
    const int kseg = SEG * (ph * NW + w);
    return (ph < phases) & (kseg + 16 * lchunk < K)
               ? static_cast<uint32_t>(16 * t + lrow) * rowb + static_cast<uint32_t>(kseg + 16 * lchunk)
               : kBufOutOfRange;
  };
  auto d_off = [&](int ph, int t, int j) -> uint32_t {
    const int blk = KBW * (ph * NW + w) + g + 4 * j;
    return (ph < phases) & (g + 4 * j < KBW) & (blk < KB)
               ? static_cast<uint32_t>(16 * t + i) * drow + static_cast<uint32_t>(blk) * 2
               : kBufOutOfRange;
  };
  auto load = [&](u32x4 (&b)[NLD], uint32_t (&s)[SPL], int ph, int t) {
    const uint32_t off = q_off(ph, t);
#pragma unroll
    for (int q = 0; q < NLD; ++q)
      b[q] = buf_load16_nt(qres, off + static_cast<uint32_t>(q * RPI) * rowb);
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      s[j] = __builtin_amdgcn_raw_buffer_load_b16(dres, static_cast<int>(d_off(ph, t, j)), 0, 0);
  };
  auto stage = [&](const u32x4 (&b)[NLD], const uint32_t (&s)[SPL]) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) *reinterpret_cast<u32x4*>(wr_base + RPI * q * RS) = b[q];
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (g + 4 * j < KBW) wsc[i * KBW + g + 4 * j] = static_cast<uint16_t>(s[j]);
  };
  // Activations of phase ph, block kb: k = kseg + 32*kb + 8*g + (0..7) of
  // row m (packed rows: each lane of a hi/lo pair loads one half).
  const int m = PACK ? (i & 7) : i;
  const bool mrow = m < M;
  const uint32_t xrow = static_cast<uint32_t>(m) * K * 4;
  auto load_x = [&](float4 (&xr)[KBW][XH], int ph) {
    const int kseg = SEG * (ph * NW + w);
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
    }
  };
  auto split = [&](const float4 (&xr)[KBW][XH], u32x4 (&afr)[KBW][F]) {
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      float4 x0 = xr[kb][0], x1 = xr[kb][XH - 1];
      if (PACK) pair_halves(xr[kb][0], i, x0, x1);
      const uint2 sa = split_bf16x2(x0.x, x0.y), sb = split_bf16x2(x0.z, x0.w);
      const uint2 sc2 = split_bf16x2(x1.x, x1.y), sd = split_bf16x2(x1.z, x1.w);
      const u32x4 h = {sa.x, sb.x, sc2.x, sd.x}, l = {sa.y, sb.y, sc2.y, sd.y};
      if (PACK) {
        afr[kb][0] = (i >> 3) ? l : h;
      } else {
        afr[kb][0] = h;
        afr[kb][F - 1] = l;
      }
    }
  };
  // The staged segment: per block, the exact bf16 conversion of 8 quants,
  // a fresh MFMA (hi, then lo), scaled by row i's block scale and added.
  auto mma_publish = [&](const u32x4 (&afr)[KBW][F], int buf) {
    float scale[KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) scale[kb] = half_bits_to_float(wsc[i * KBW + kb]);
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      const u32x4 bv = q8x8_to_bf16(*reinterpret_cast<const uint2*>(rd_base + 32 * kb));
      f32x4 acc = mfma_16x16x32(afr[kb][0], bv, f32x4{0.f, 0.f, 0.f, 0.f});
      if (!PACK) acc = mfma_16x16x32(afr[kb][F - 1], bv, acc);
#pragma unroll
      for (int v = 0; v < 4; ++v) tot[v] = __builtin_fmaf(acc[v], scale[kb], tot[v]);
    }
    float* dst = red + (buf * NW + w) * ROWS * 16;
    if (PACK) {
      // lanes 0..31 hold rows 0..7 (hi), lanes 32..63 rows 8..15 (lo) of the same columns
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float lo = __shfl_down(tot[v], 32);
        if (g < 2) dst[(4 * g + v) * 16 + i] = tot[v] + lo;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[(4 * g + v) * 16 + i] = tot[v];
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

  float4 xr[KBW][XH];
  u32x4 b[NLD], afr[KBW][F];
  uint32_t s[SPL];
  if (!MANY) {
    // One tile: phase ph + 1's activations go out before phase ph's MFMAs,
    // its weights right after them (when their registers are free); the
    // last phase is peeled so that nothing is loaded past it.
    auto phase = [&](int ph, auto more) {
      __builtin_amdgcn_sched_barrier(0);
      split(xr, afr);
      __builtin_amdgcn_sched_barrier(0);
      stage(b, s);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(more)::value) load_x(xr, ph + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_publish(afr, ph & 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(more)::value) load(b, s, ph + 1, 0);
      __syncthreads();
      reduce(ph & 1, 0, ph);
    };
    load_x(xr, 0);
    load(b, s, 0, 0);
    int ph = 0;
    for (; ph + 1 < phases; ++ph) phase(ph, std::true_type{});
    phase(ph, std::false_type{});
  } else {
    load_x(xr, 0);
    load(b, s, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    split(xr, afr);
    int j = 0;  // items so far: parity of the reduction buffer
    for (int ph = 0; ph < phases; ++ph) {
      for (int t = 0; t < rounds; ++t, ++j) {
        __builtin_amdgcn_sched_barrier(0);
        stage(b, s);
        __builtin_amdgcn_sched_barrier(0);
        const bool last_t = t + 1 == rounds;
        const bool more = !last_t || ph + 1 < phases;
        if (last_t && more) load_x(xr, ph + 1);
        if (more) load(b, s, last_t ? ph + 1 : ph, last_t ? 0 : t + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_publish(afr, j & 1);
        __syncthreads();
        reduce(j & 1, t, ph);
        if (last_t && more) split(xr, afr);
      }
    }
  }
  __syncthreads();
  // Outputs, once: tile t covers columns r0 + 16t + (0..15).
  for (int e = tid; e < rounds * M * 16; e += NW * kWave) {
    const int t = e / (M * 16), rem = e - t * M * 16, mm = rem >> 4, col = rem & 15;
    const int n = r0 + 16 * t + col;
    if (n < r1) p.Y[static_cast<size_t>(mm) * p.ldy + n] = ysum[(t * ROWS + mm) * 16 + col];
  }
}

template <bool PACK, int KBW, bool PAIRED>
hipError_t launch_q8_as(const Q8Params& prm, int grid, size_t lds, bool multi, hipStream_t st) {
  const void* one = reinterpret_cast<const void*>(&gemv_q8_kernel<PACK, false, KBW, PAIRED>);
  const void* many = reinterpret_cast<const void*>(&gemv_q8_kernel<PACK, true, KBW, PAIRED>);
  static const hipError_t attr = [&] {
    const hipError_t e = hipFuncSetAttribute(one, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kQLds));
    return e != hipSuccess ? e
                           : hipFuncSetAttribute(many, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kQLds));
  }();
  if (attr != hipSuccess) return attr;
  Q8Params a = prm;
  void* args[] = {&a};
  return hipLaunchKernel(multi ? many : one, dim3(grid), dim3(kQNW * kWave), args, lds, st);
}

// Scale words of two blocks need 4-byte aligned scale rows: K / 32 and the
// row stride even.
template <bool PACK, int KBW>
hipError_t launch_q8(const Q8Params& prm, int grid, size_t lds, bool multi, hipStream_t st) {
  return (prm.K / 32) % 2 == 0 && prm.ldd % 2 == 0 ? launch_q8_as<PACK, KBW, true>(prm, grid, lds, multi, st)
                                                   : launch_q8_as<PACK, KBW, false>(prm, grid, lds, multi, st);
}

template <bool PACK, int KBW>
hipError_t launch_q8_short(const Q8Params& prm, int grid, size_t lds, bool many, hipStream_t st) {
  const void* one = reinterpret_cast<const void*>(&gemv_q8_short_kernel<PACK, KBW, false>);
  const void* several = reinterpret_cast<const void*>(&gemv_q8_short_kernel<PACK, KBW, true>);
  static const hipError_t attr = [&] {
    const hipError_t e = hipFuncSetAttribute(one, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kQLds));
    return e != hipSuccess ? e
                           : hipFuncSetAttribute(several, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(kQLds));
  }();
  if (attr != hipSuccess) return attr;
  Q8Params a = prm;
  void* args[] = {&a};
  return hipLaunchKernel(many ? several : one, dim3(grid), dim3(kQNW * kWave), args, lds, st);
}

}  // namespace

bool gemv_q8_shape_fits(int N, int K, int M) {
  if (N < 1 || K < 32 || (K % 32) != 0 || M < 1 || K > (1 << 22)) return false;  // X of a launch: <= 16 * K * 4 bytes
  const int cus = device_cu_count();
  if (cus <= 0) return true;  // the launch reports the missing device
  const int grid = std::max(1, std::min(cus, std::min((N + 15) / 16, std::max(1, N / 2))));
  return static_cast<long long>(q8_rows_max(N, grid)) * K < (1LL << 31);
}

hipError_t launch_gemv_q8(const int8_t* Wq, const uint16_t* Wd, int N, int K, const float* X, int M, float* Y,
                          hipStream_t stream, int ldd) {
  const int cus = device_cu_count();
  if (cus <= 0) return hipErrorNoDevice;
  const int tiles = (N + 15) / 16;
  const int grid = std::max(1, std::min(cus, std::min(tiles, std::max(1, N / 2))));
  const int rounds = (q8_rows_max(N, grid) + 15) / 16;
  const int KB = K / 32;
  // Launches of at most 16 rows of X each (the weights are read once per launch).
  for (int m0 = 0; m0 < M; m0 += 16) {
    const int mm = std::min(16, M - m0);
    const bool pack = mm <= 8;
    const int rowsl = pack ? 8 : 16;
    Q8Params prm{};
    prm.Wq = Wq;
    prm.Wd = Wd;
    prm.X = X + static_cast<size_t>(m0) * K;
    prm.Y = Y + static_cast<size_t>(m0) * N;
    prm.N = N;
    prm.K = K;
    prm.M = mm;
    prm.ldy = N;
    prm.ldd = ldd > 0 ? ldd : KB;
    prm.pq = (N / 2) / grid;
    prm.prem = (N / 2) % grid;
    if (rounds <= kQShortTiles) {
      // Few tiles per workgroup. 4 blocks (128 quant bytes of a row) per
      // wave and phase, one tile or several: measured on MI355X at the
      // projections of a draft layer (M = 7 and 15), 2 blocks was as fast or
      // slower, 8 no faster where it does not spill.
      constexpr int kbw = 4;
      const size_t lds = static_cast<size_t>(kQNW) * 16 * (32 * kbw + 16) + static_cast<size_t>(kQNW) * 16 * kbw * 2 +
                         static_cast<size_t>(2) * kQNW * rowsl * 16 * 4 + static_cast<size_t>(rounds) * rowsl * 16 * 4;
      const bool many = rounds > 1;
      const hipError_t e = pack ? launch_q8_short<true, kbw>(prm, grid, lds, many, stream)
                                : launch_q8_short<false, kbw>(prm, grid, lds, many, stream);
      if (e != hipSuccess) return e;
      continue;
    }
    // 8 blocks (256 quant bytes of a row) per wave and phase keep twice the
    // bytes in flight of 4; rows of 9..16 activations take 4 (registers).
    const int kbw = pack ? 8 : 4;
    const bool multi = (KB + kQNW * kbw - 1) / (kQNW * kbw) > 1;
    const size_t fixed = static_cast<size_t>(kQNW) * 16 * (32 * kbw + 16) + static_cast<size_t>(kQNW) * 16 * kbw * 2 +
                         static_cast<size_t>(2) * kQNW * rowsl * 16 * 4;
    const size_t per_tile = static_cast<size_t>(mm) * 16 * 4;
    int chunk = static_cast<int>((kQLds - fixed) / per_tile) & ~1;
    chunk = std::max(2, std::min(chunk, (rounds + 1) & ~1));
    prm.chunk = chunk;
    const size_t lds = fixed + chunk * per_tile;
    const hipError_t e = pack ? launch_q8<true, 8>(prm, grid, lds, multi, stream)
                              : launch_q8<false, 4>(prm, grid, lds, multi, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
