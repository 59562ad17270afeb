// Confidence probe: logit[m] = sum_t w[t] * x[m, t] + bias; pass = logit >= threshold.
//
// ds4 #772, section "Summary": the proposer's confidence probe becomes one
// small GPU kernel whose only result is a 4-byte scalar per drafted row,
// replacing a device-to-host copy of the hidden state and a host matvec.
// Section "Performance": GPU and CPU evaluations differ only in summation
// order and make the same gating decisions.
//
// One workgroup per row. Each lane reads 8 bf16 weights (16 bytes) and 8
// fp32 activations per iteration and accumulates them in one fp32 FMA
// chain; lanes are then combined by a fixed butterfly and waves in index
// order, so the result is deterministic.
#include "dspark_internal.h"

namespace dspark {
namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void probe_kernel(const float* __restrict__ x, int D,
                                                              const uint16_t* __restrict__ w, float bias,
                                                              float threshold, float* __restrict__ logit,
                                                              int32_t* __restrict__ pass) {
  __shared__ float part[kProbeThreads / kWave];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* xr = x + static_cast<size_t>(m) * D;
  float acc = 0.f;
  for (int t = tid * 8; t < D; t += kProbeThreads * 8) {
    const u32x4 wb = load16(w + t);
    const float4 x0 = *reinterpret_cast<const float4*>(xr + t);
    const float4 x1 = *reinterpret_cast<const float4*>(xr + t + 4);
    acc = __builtin_fmaf(x0.x, __uint_as_float(wb.x << 16), acc);
    acc = __builtin_fmaf(x0.y, __uint_as_float(wb.x & 0xFFFF0000u), acc);
    acc = __builtin_fmaf(x0.z, __uint_as_float(wb.y << 16), acc);
    acc = __builtin_fmaf(x0.w, __uint_as_float(wb.y & 0xFFFF0000u), acc);
    acc = __builtin_fmaf(x1.x, __uint_as_float(wb.z << 16), acc);
    acc = __builtin_fmaf(x1.y, __uint_as_float(wb.z & 0xFFFF0000u), acc);
    acc = __builtin_fmaf(x1.z, __uint_as_float(wb.w << 16), acc);
    acc = __builtin_fmaf(x1.w, __uint_as_float(wb.w & 0xFFFF0000u), acc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) part[wv] = acc;
  __syncthreads();
  if (tid == 0) {
    float s = part[0];
#pragma unroll
    for (int j = 1; j < kProbeThreads / kWave; ++j) s += part[j];
    const float l = s + bias;
    logit[m] = l;
    if (pass) pass[m] = l >= threshold ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_probe(const float* x, int M, int D, const uint16_t* w, float bias, float threshold,
                        float* logit, int32_t* pass, hipStream_t stream) {
  void* args[] = {&x, &D, &w, &bias, &threshold, &logit, &pass};
  return hipLaunchKernel(reinterpret_cast<const void*>(&probe_kernel), dim3(M), dim3(kProbeThreads), args, 0,
                         stream);
}

}  // namespace dspark
