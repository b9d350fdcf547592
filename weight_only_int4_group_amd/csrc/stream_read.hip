// Plain streaming-read kernel: the measured read-bandwidth ceiling that the
// benchmark reports beside the decode kernel (same bytes per launch, same
// rotating buffers).  Not part of the W4A16 library: it is built into its own
// small shared object, libw4a16_ceiling.so, and only the benchmark loads it.
//
// Each workgroup streams one contiguous slice of the buffer: every thread
// keeps kUnroll independent 16-byte loads in flight per iteration, the
// workgroup's threads covering kUnroll * threads * 16 consecutive bytes, and
// XORs what it reads into one register.  A thread writes its register only if
// it equals a value the caller passes that the data never produces, so the
// loads cannot be dropped and nothing is written in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format

template <int kThreads, int kUnroll, int kCpol>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint8_t *buf, uint32_t bytes,
                                                               uint32_t slice, uint32_t never,
                                                               uint32_t *sink) {
  const uint32_t b0 = blockIdx.x * slice;
  const uint32_t b1 = min(bytes, b0 + slice);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)buf, (short)0, (int)bytes, kRsrcWord3);
  u32x4 acc = {0, 0, 0, 0};
  constexpr uint32_t kStep = (uint32_t)kThreads * kUnroll * 16;
  for (uint32_t off = b0 + threadIdx.x * 16; off < b1; off += kStep) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)  // past the buffer: out of range, reads zeros
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, off + (uint32_t)u * kThreads * 16, 0, kCpol));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == never) sink[blockIdx.x * kThreads + threadIdx.x] = x;
}

// Slices are whole iterations (kUnroll * kThreads * 16 bytes), so no load
// strays into a neighbour's slice; the last slice's loads past the buffer are
// out of the resource's range and return zeros without touching memory.  At
// most `blocks` workgroups.
template <int kThreads, int kUnroll, int kCpol>
hipError_t launch(const void *buf, uint32_t bytes, int blocks, uint32_t *sink, hipStream_t st) {
  constexpr uint32_t kStep = (uint32_t)kThreads * kUnroll * 16;
  const uint32_t per = (bytes + (uint32_t)blocks - 1) / (uint32_t)blocks;
  const uint32_t slice = (per + kStep - 1) / kStep * kStep;
  const uint32_t used = (bytes + slice - 1) / slice;
  hipLaunchKernelGGL((stream_read_kernel<kThreads, kUnroll, kCpol>), dim3(used), dim3(kThreads),
                     0, st, static_cast<const uint8_t *>(buf), bytes, slice, 0x9E3779B9u, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Variants: bit 0 = non-temporal loads, bits 1-2 = loads in flight per thread
// (4, 8, 16), bit 3 = 512 threads per workgroup (else 256).  `sink` needs
// blocks * threads 32-bit words of device memory (written only in theory).
// bytes < 2^31, a multiple of 16.  Returns 0, or -1 on a bad argument, or the
// HIP error of the launch.
int stream_read(const void *buf, size_t bytes, int variant, int blocks, void *sink, void *stream) {
  if (!buf || !sink || bytes == 0 || bytes >= ((size_t)1 << 31) || (bytes & 15) || blocks < 1 ||
      variant < 0 || variant > 15 || ((variant >> 1) & 3) == 3)
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t n = (uint32_t)bytes;
  uint32_t *s = static_cast<uint32_t *>(sink);
  const int u = (variant >> 1) & 3;
  const bool nt = variant & 1, wide = (variant & 8) != 0;
#define W4_SR(T, U)                                                      \
  return (int)(nt ? launch<T, U, 2>(buf, n, blocks, s, st) : launch<T, U, 0>(buf, n, blocks, s, st))
  if (wide) {
    if (u == 0) W4_SR(512, 4);
    if (u == 1) W4_SR(512, 8);
    W4_SR(512, 16);
  }
  if (u == 0) W4_SR(256, 4);
  if (u == 1) W4_SR(256, 8);
  W4_SR(256, 16);
#undef W4_SR
}

}  // extern "C"
