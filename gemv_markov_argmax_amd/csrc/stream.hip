// A measurement aid, not a step of the method: a plain streaming read of a
// device buffer, to measure the HBM read ceiling of this device beside the
// kernels of the round, in the same process and run.
//
// The pages quote the draft round's kernels against a bandwidth bound
// (vllm.cpp #436, "W7 LANDED": the Markov GEMV sits at the device's
// streaming bound; SharpInference #441, "Observation": the round against
// its bandwidth floor). What a GEMV can reach depends on what a pure read
// reaches at the same launch shape, which this kernel measures.
//
// Workgroup b reads the contiguous b-th share of the buffer (shares
// balanced to 16 bytes), each thread 16-byte non-temporal loads strided by
// the workgroup's width, eight loads in flight per thread, and folds what
// it read into one word per workgroup (so no load can be dropped). With
// zero bytes it is an empty launch: the launch-latency floor.
#include "dspark_internal.h"

namespace dspark {
namespace {

template <int NT>
__global__ __launch_bounds__(NT) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t G = gridDim.x, b = blockIdx.x;
  const size_t lo = n16 * b / G, hi = n16 * (b + 1) / G;
  uint32_t acc = 0;
  constexpr int kInFlight = 8;
  size_t e = lo + threadIdx.x;
  for (; e + (kInFlight - 1) * NT < hi; e += kInFlight * NT) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(p + e + u * NT);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; e < hi; e += NT) {
    const u32x4 v = __builtin_nontemporal_load(p + e);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup: the xor of its lanes' words (wave, then waves in order)
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t part[NT / kWave];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < NT / kWave; ++w) t ^= part[w];
    sink[b] = t;
  }
}

// The same read with the lm_head's schedule (gemv_sched_kernel): units of
// 256 KB, a contiguous run of S units per workgroup, then units S*G + v for
// each take v from the counter, until a take is past the last unit; the
// last take of the launch (max(0, T - S*G) + G - 1) stores 0 back. So the
// ceiling measured this way is the one that kernel streams against.
constexpr size_t kUnit16 = 16384;  // 16-byte elements per unit

template <int NT>
__global__ __launch_bounds__(NT) void stream_read_sched_kernel(const u32x4* __restrict__ p, size_t n16,
                                                               uint32_t S, uint32_t* __restrict__ counter,
                                                               uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[NT / kWave];
  __shared__ uint32_t take_s;
  const uint32_t G = gridDim.x, b = blockIdx.x;
  const uint32_t T = static_cast<uint32_t>((n16 + kUnit16 - 1) / kUnit16);
  const uint32_t D0 = S * G;
  const uint32_t final_take = (T > D0 ? T - D0 : 0u) + G - 1;
  uint32_t acc = 0;
  auto read_unit = [&](uint32_t u) {
    const size_t lo = static_cast<size_t>(u) * kUnit16, hi = lo + kUnit16 < n16 ? lo + kUnit16 : n16;
    constexpr int kInFlight = 8;
    size_t e = lo + threadIdx.x;
    for (; e + (kInFlight - 1) * NT < hi; e += kInFlight * NT) {
      u32x4 v[kInFlight];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) v[k] = __builtin_nontemporal_load(p + e + k * NT);
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; e < hi; e += NT) {
      const u32x4 v = __builtin_nontemporal_load(p + e);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  };
  for (uint32_t k = 0; k < S; ++k) read_unit(b * S + k);  // host: S * G <= T
  for (;;) {
    if (threadIdx.x == 0) {
      const uint32_t v = atomicInc(counter, 0xffffffffu);
      if (v == final_take) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      take_s = v;
    }
    __syncthreads();
    const uint32_t u = D0 + take_s;
    __syncthreads();  // take_s is read before thread 0 rewrites it
    if (u >= T) break;  // uniform
    read_unit(u);
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < NT / kWave; ++w) t ^= part[w];
    sink[b] = t;
  }
}

}  // namespace

hipError_t launch_stream_read_sched(const void* buf, size_t bytes, int groups, int threads, uint32_t* counter,
                                    uint32_t* sink, hipStream_t stream) {
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  const size_t units = (n16 + kUnit16 - 1) / kUnit16;
  const uint32_t S = static_cast<uint32_t>(90 * (units / static_cast<size_t>(groups)) / 100);  // as the lm_head
  switch (threads) {
    case 256: stream_read_sched_kernel<256><<<dim3(groups), dim3(256), 0, stream>>>(p, n16, S, counter, sink); break;
    case 512: stream_read_sched_kernel<512><<<dim3(groups), dim3(512), 0, stream>>>(p, n16, S, counter, sink); break;
    case 1024: stream_read_sched_kernel<1024><<<dim3(groups), dim3(1024), 0, stream>>>(p, n16, S, counter, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, int groups, int threads, uint32_t* sink,
                              hipStream_t stream) {
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  switch (threads) {
    case 256: stream_read_kernel<256><<<dim3(groups), dim3(256), 0, stream>>>(p, n16, sink); break;
    case 512: stream_read_kernel<512><<<dim3(groups), dim3(512), 0, stream>>>(p, n16, sink); break;
    case 1024: stream_read_kernel<1024><<<dim3(groups), dim3(1024), 0, stream>>>(p, n16, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dspark
