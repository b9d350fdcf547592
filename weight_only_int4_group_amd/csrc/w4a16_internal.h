// Host-side launchers shared between the C-ABI front end and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// Bits of the packer's device status word.
constexpr unsigned kPackNonFinite = 1u;
constexpr unsigned kPackRange = 2u;

hipError_t launch_pack(const void *W, const void *s, int N, int K, void *Wq, void *scales,
                       void *zeros, unsigned *status, hipStream_t stream);

// One problem of the streaming kernel (validated by the caller).
struct SkinnyDesc {
  const void *X, *Wq, *scales, *zeros, *s;
  void *Y;
  int M, N, K;
};

// Streaming kernel for small M (decode and speculative verify): M <= 16.
// launch_skinny_set runs up to skinny_max_problems() independent problems in
// one launch.
int skinny_max_problems();
hipError_t launch_skinny_set(const SkinnyDesc *problems, int count, hipStream_t stream);
hipError_t launch_skinny(const void *X, const void *Wq, const void *scales, const void *zeros,
                         const void *s, void *Y, int M, int N, int K, hipStream_t stream);

// LDS-tiled MFMA GEMM for large M (batched decode and prefill): any M >= 1.
hipError_t launch_tiled(const void *X, const void *Wq, const void *scales, const void *zeros,
                        const void *s, void *Y, int M, int N, int K, hipStream_t stream);

}  // namespace w4a16
