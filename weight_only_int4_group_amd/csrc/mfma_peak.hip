// Dense fp16 MFMA throughput ceiling: the benchmark times it beside the
// prefill GEMM, as the rate the matrix cores sustain on this GPU at the clock
// they run at under full load.  Not part of the W4A16 library: it is built
// into the benchmark's small ceiling library with the streaming-read kernel.
//
// Every wave issues `chains` independent v_mfma_f32_16x16x32_f16 accumulations
// from registers, `iters` times each: no memory traffic, no LDS, no VALU work
// in the loop.  The operands are pseudo-random fp16 values in [-1, 1) (a hash
// of the lane), so the multipliers switch like they do on real data.  A lane
// writes its sum only if it equals a value the caller passes that the data
// never produces, so the MFMAs cannot be dropped and nothing is written in
// practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ _Float16 next_half(uint32_t &h) {
  h = h * 1664525u + 1013904223u;  // LCG step (Numerical Recipes constants)
  return (_Float16)((float)((int)(h >> 16) - 32768) * (1.0f / 32768.0f));
}

template <int kChains>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, uint32_t never, uint32_t *sink) {
  const uint32_t id = blockIdx.x * 256u + threadIdx.x;
  uint32_t h = id * 2654435761u + 12345u;
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = next_half(h);
    b[e] = next_half(h);
  }
  float4v acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = float4v{(float)c, 0.f, 0.f, 0.f};  // distinct chains
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (__builtin_bit_cast(uint32_t, s) == never) sink[id] = 1u;
}

}  // namespace

extern "C" {

// One launch of `blocks` workgroups of 256 threads (four waves), each wave
// running `chains` (4, 8, 16 or 32) independent accumulations `iters` times:
// blocks * 4 * chains * iters MFMAs of 16 x 16 x 32 (16384 flops each).
// `sink` needs blocks * 256 32-bit words of device memory (written only in
// theory).  Returns 0, -1 on a bad argument, or the HIP error of the launch.
int mfma_peak(int chains, int blocks, int iters, void *sink, void *stream) {
  if (!sink || blocks < 1 || blocks > (1 << 20) || iters < 1 ||
      (chains != 4 && chains != 8 && chains != 16 && chains != 32))
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t *s = static_cast<uint32_t *>(sink);
  const uint32_t never = 0x7FBADBADu;  // a NaN payload sums of finite values never take
  if (chains == 4)
    hipLaunchKernelGGL(mfma_peak_kernel<4>, dim3(blocks), dim3(256), 0, st, iters, never, s);
  else if (chains == 8)
    hipLaunchKernelGGL(mfma_peak_kernel<8>, dim3(blocks), dim3(256), 0, st, iters, never, s);
  else if (chains == 16)
    hipLaunchKernelGGL(mfma_peak_kernel<16>, dim3(blocks), dim3(256), 0, st, iters, never, s);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<32>, dim3(blocks), dim3(256), 0, st, iters, never, s);
  return (int)hipGetLastError();
}

}  // extern "C"
