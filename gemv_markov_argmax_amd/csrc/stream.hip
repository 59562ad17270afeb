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

}  // namespace

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
