// Confidence probe: logit[m] = sum_t w[t] * x[m, t] + bias; pass = logit >= threshold.
//
// ds4 #772, section "Summary": the proposer's confidence probe becomes one
// small GPU kernel whose only result is a 4-byte scalar per drafted row,
// replacing a device-to-host copy of the hidden state and a host matvec.
// Section "Performance": GPU and CPU evaluations differ only in summation
// order and make the same gating decisions.
//
// One workgroup of four waves per row: wave h computes chain h of the sum
// (lane l takes entries 8l + 512h + 2048j, eight at a time, in one fp32 FMA
// chain, then a fixed butterfly), and the four chain totals are added in a
// fixed order, so the result is deterministic and depends on D alone. A
// row of up to 8192 entries is one round trip to memory. The Markov loop
// computes the same chains in the same order when a draft round asks it
// for the probe.
#include "dspark_internal.h"

namespace dspark {
namespace {

__global__ __launch_bounds__(4 * kWave) void probe_kernel(ProbeArgs a) {
  __shared__ float part[4];
  const int m = blockIdx.x, lane = threadIdx.x & 63, h = threadIdx.x >> 6;
  const float c = probe_chain<4>(a.x + static_cast<size_t>(m) * a.D, a.D, a.w, lane, h);
  if (lane == 0) part[h] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float l = probe_logit(part, a.bias);
    a.logit[m] = l;
    if (a.pass) a.pass[m] = l >= a.threshold ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_probe(const float* x, int M, int D, const uint16_t* w, float bias, float threshold,
                        float* logit, int32_t* pass, hipStream_t stream) {
  ProbeArgs a{x, M, D, w, bias, threshold, logit, pass};
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&probe_kernel), dim3(M), dim3(4 * kWave), args, 0, stream);
}

}  // namespace dspark
