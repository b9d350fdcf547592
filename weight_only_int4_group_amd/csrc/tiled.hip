// LDS-tiled dequantize-matmul for large M (batched decode, prefill):
// Y[M][N] = X[M][K] . W_hat^T.
//
// The nano-vllm tutorial (discosf.com), section 1.1, describes prefill as one
// large matmul bounded by arithmetic, so this kernel is organised around the
// MFMA units: a 256-thread workgroup owns a BM x BN = 128 x 128 block of Y
// and walks K one quantization group (128 columns) at a time.  Per group:
//   * X rows are loaded (X * s rounded to fp16 when an AWQ scale is given)
//     and stored to LDS;
//   * the 8 packed tiles of the 128 W rows are loaded (one 128-bit load per
//     lane per tile), dequantized once per workgroup to fp16
//     (q - z) * scale -- the weight-only "dequantize to FP16, then multiply"
//     of "Chapter 22" (aiwing.uk) section 22.3 -- and stored to LDS;
//   * each of the 4 waves computes a 64 x 64 sub-block with 16x16x32 fp16
//     MFMAs and fp32 accumulation.
// The next group's global loads are issued before the current group's MFMAs
// so that HBM/L2 latency overlaps the math.
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = kGroup;
constexpr int LDS_STRIDE = BK + 8;  // halves; 16-byte pad keeps ds_read_b128 conflict-free
constexpr int THREADS = 256;

__global__ __launch_bounds__(THREADS) void tiled_kernel(
    const _Float16 *__restrict__ X, const u32x4 *__restrict__ Wq,
    const _Float16 *__restrict__ scales, const _Float16 *__restrict__ zeros,
    const _Float16 *__restrict__ s, _Float16 *__restrict__ Y, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[BN * LDS_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4, r = lane & 15;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int G = K / kGroup;
  const int Gq = meta_groups(G) / kMetaQuad;
  const int wm = wave >> 1, wn = wave & 1;

  // A loader: 128 rows x 16 chunks of 8 halves; thread takes chunk tid + 256i.
  const int a_col = (tid & 15) * 8;
  const int a_row0 = tid >> 4;  // + 16i
  // B loader: 8 tiles x 64 lanes; thread takes tile (wave + 4i), lane `lane`.

  half8 areg[8];
  u32x4 breg[2];
  _Float16 bsc[2], bz[2];

  auto load_group = [&](int g) {
    half8 sv;
    if (s) sv = load_half8(s + (size_t)g * BK + a_col);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + a_row0 + 16 * i;
      half8 v = zero_half8();
      if (m < M) {
        v = load_half8(X + (size_t)m * K + (size_t)g * BK + a_col);
        if (s) v = v * sv;
      }
      areg[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int bb = wave + 4 * i;
      const int nrow = n0 + 16 * bb;
      if (nrow < N) {
        breg[i] = Wq[((size_t)(nrow / kTileRows) * G + g) * 64 + lane];
        bsc[i] = scales[meta_index(nrow + r, g, Gq)];
        bz[i] = zeros[meta_index(nrow + r, g, Gq)];
      } else {
        const u32x4 z4 = {0, 0, 0, 0};
        breg[i] = z4;
        bsc[i] = 0;
        bz[i] = 0;
      }
    }
  };

  float4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  load_group(0);
  for (int g = 0; g < G; ++g) {
    __syncthreads();  // previous group's MFMAs are done reading LDS
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<half8 *>(&As[(a_row0 + 16 * i) * LDS_STRIDE + a_col]) = areg[i];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int bb = wave + 4 * i;
      const half2v bias = zero_bias(bz[i]);
      const _Float16 sc = bsc[i];
      const half8 sc8 = {sc, sc, sc, sc, sc, sc, sc, sc};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const half8 w = decode_word(breg[i][t], bias) * sc8;
        *reinterpret_cast<half8 *>(&Bs[(16 * bb + r) * LDS_STRIDE + 32 * t + 8 * c]) = w;
      }
    }
    __syncthreads();
    if (g + 1 < G) load_group(g + 1);

#pragma unroll
    for (int t = 0; t < 4; ++t) {
      half8 a_op[4], b_op[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a_op[i] = *reinterpret_cast<const half8 *>(
            &As[(64 * wm + 16 * i + r) * LDS_STRIDE + 32 * t + 8 * c]);
        b_op[i] = *reinterpret_cast<const half8 *>(
            &Bs[(64 * wn + 16 * i + r) * LDS_STRIDE + 32 * t + 8 * c]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a_op[i], b_op[j], acc[i][j]);
    }
  }

  // lane holds D[4c + v][r] of each 16x16 block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wn + 16 * j + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 64 * wm + 16 * i + 4 * c + v;
        if (m < M && n < N) Y[(size_t)m * N + n] = (_Float16)acc[i][j][v];
      }
    }
  }
}

}  // namespace

hipError_t launch_tiled(const void *X, const void *Wq, const void *scales, const void *zeros,
                        const void *s, void *Y, int M, int N, int K, hipStream_t stream) {
  const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  hipLaunchKernelGGL(tiled_kernel, grid, dim3(THREADS), 0, stream, (const _Float16 *)X,
                     (const u32x4 *)Wq, (const _Float16 *)scales, (const _Float16 *)zeros,
                     (const _Float16 *)s, (_Float16 *)Y, M, N, K);
  return hipGetLastError();
}

}  // namespace w4a16
