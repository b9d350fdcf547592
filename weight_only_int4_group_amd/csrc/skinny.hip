// Streaming dequantize-matmul for small M (decode M = 1, speculative verify
// M = draft length + 1): Y[M][N] = X[M][K] . W_hat^T with M <= 16.
//
// Where the time goes: the nano-vllm tutorial (discosf.com), section 1.1 and
// section 2.2, and "Chapter 22" (aiwing.uk) section 22.2's comparison table
// describe decode as bandwidth-bound -- every token streams all weights -- so
// this kernel is built to read each packed byte exactly once at HBM rate and
// to keep the arithmetic off the critical path.
//
// Work split: one workgroup owns one 16-row block of W (a column of packed
// tiles along K).  Its waves split K: wave w takes chunks of GW consecutive
// groups, chunk w, w + WAVES, ...  For each group the wave
//   * loads the 1 KB tile with one 128-bit load per lane (fully coalesced),
//   * turns each 32-bit word into the exact fp16 values (q - z) (two ALU ops
//     per pair of codes) -- that register is the lane's MFMA B operand,
//   * multiplies by X (rows 0..M-1 of the A operand; X * s rounded to fp16
//     once when an AWQ scale is given) with four 16x16x32 MFMAs, and
//   * folds the group's fp32 result into the accumulator times the group
//     scale, so the scale is applied in fp32, once per group and row.
// The per-wave partials (16 rows x M) are summed in a fixed order through
// LDS, so results are bit-reproducible run to run.
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int WAVES, int GW>
__global__ __launch_bounds__(WAVES * 64) void skinny_kernel(
    const _Float16 *__restrict__ X, const u32x4 *__restrict__ Wq,
    const _Float16 *__restrict__ scales, const _Float16 *__restrict__ zeros,
    const _Float16 *__restrict__ s, _Float16 *__restrict__ Y, int M, int N, int K) {
  const int G = K / kGroup;
  const int NB = N / kTileRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane >> 4;   // column octet (A/B operands), row quad (D)
  const int r = lane & 15;   // X row m (A), W row in the tile (B), column n (D)
  __shared__ float red[WAVES][16][17];

  const bool a_live = r < M;
  const _Float16 *xrow = X + (size_t)(a_live ? r : 0) * K + 8 * c;
  const _Float16 *srow = s ? s + 8 * c : nullptr;

  for (int b = blockIdx.x; b < NB; b += gridDim.x) {
    const int n = b * kTileRows + r;
    const u32x4 *tiles = Wq + (size_t)b * G * 64 + lane;
    const _Float16 *sc_row = scales + (size_t)n * G;
    const _Float16 *z_row = zeros + (size_t)n * G;
    float4v acc = {0.f, 0.f, 0.f, 0.f};

    for (int g0 = wave * GW; g0 < G; g0 += WAVES * GW) {
      u32x4 code[GW];
      _Float16 sc[GW], zp[GW];
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const int g = min(g0 + i, G - 1);
        code[i] = __builtin_nontemporal_load(tiles + (size_t)g * 64);
        sc[i] = sc_row[g];
        zp[i] = z_row[g];
      }
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        if (g0 + i < G) {
          const int g = g0 + i;
          half8 a[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const size_t k = (size_t)g * kGroup + 32 * t;
            half8 xv = zero_half8();
            if (a_live) {
              xv = load_half8(xrow + k);
              if (srow) xv = xv * load_half8(srow + k);
            }
            a[t] = xv;
          }
          const half2v bias = zero_bias(zp[i]);
          float4v tmp = {0.f, 0.f, 0.f, 0.f};
          tmp = mfma16(a[0], decode_word(code[i][0], bias), tmp);
          tmp = mfma16(a[1], decode_word(code[i][1], bias), tmp);
          tmp = mfma16(a[2], decode_word(code[i][2], bias), tmp);
          tmp = mfma16(a[3], decode_word(code[i][3], bias), tmp);
          const float scf = (float)sc[i];
          acc += tmp * scf;
        }
      }
    }

    // lane holds D[m = 4c + v][n = r] summed over this wave's groups
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * c + v][r] = acc[v];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * M; idx += WAVES * 64) {
      const int m = idx >> 4, nn = idx & 15;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) sum += red[w][m][nn];
      Y[(size_t)m * N + (size_t)b * kTileRows + nn] = (_Float16)sum;
    }
    __syncthreads();
  }
}

template <int WAVES>
hipError_t launch_waves(const void *X, const void *Wq, const void *scales, const void *zeros,
                        const void *s, void *Y, int M, int N, int K, hipStream_t stream) {
  constexpr int GW = 4;
  const int NB = N / kTileRows;
  hipLaunchKernelGGL((skinny_kernel<WAVES, GW>), dim3(NB), dim3(WAVES * 64), 0, stream,
                     (const _Float16 *)X, (const u32x4 *)Wq, (const _Float16 *)scales,
                     (const _Float16 *)zeros, (const _Float16 *)s, (_Float16 *)Y, M, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const void *X, const void *Wq, const void *scales, const void *zeros,
                         const void *s, void *Y, int M, int N, int K, hipStream_t stream) {
  // enough waves that each takes about one chunk of 4 groups, at most 16
  const int chunks = (K / kGroup + 3) / 4;
  if (chunks <= 2) return launch_waves<2>(X, Wq, scales, zeros, s, Y, M, N, K, stream);
  if (chunks <= 4) return launch_waves<4>(X, Wq, scales, zeros, s, Y, M, N, K, stream);
  if (chunks <= 8) return launch_waves<8>(X, Wq, scales, zeros, s, Y, M, N, K, stream);
  return launch_waves<16>(X, Wq, scales, zeros, s, Y, M, N, K, stream);
}

}  // namespace w4a16
