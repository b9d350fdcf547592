// Quantize-and-pack: fp16 W[N][K] (and optional fp16 AWQ scale s[K]) ->
// packed 4-bit codes, fp16 per-group scales and fp16 zero points.
//
// The arithmetic follows "Chapter 22: Advanced inference optimisation"
// (aiwing.uk), section 22.3, AWQ equation (divide W by s, then quantize), and
// the nano-vllm tutorial (discosf.com), section 2.1 (a scale and a zero point
// per group of 128 elements map the float range onto the integer range).
// Every quotient is one correctly rounded fp64 division and nothing is fused,
// so the result is unique: the group range [min(0, min W'), max(0, max W')],
// scale = range / 15 rounded up to fp16, z = rint(-min / scale),
// q = clamp(rint(W' / scale) + z, 0, 15), ties to even.
//
// The per-channel and per-tensor granularities of the same tutorial (section
// 2.1: one scale per channel, or per tensor) take the range over the row or
// the whole tensor (row_range_kernel, tensor_range_kernel) and repeat its
// scale and zero point in every group of the row.
//
// The symmetric variant (the signed -7..7 grid of the practitioner notes at
// mhpq.cn, section 2.1) keeps every step but the grid: scale = max|W'| / 7
// rounded up to fp16, signed code c = clamp(rint(W' / scale), -7, 7) stored as
// c + 8 with the constant zero point 8 (so (q - z) * scale is unchanged for
// the GEMM kernels); an all-zero group stores scale 0 and codes 8.
//
// One 64-lane wave handles one packed tile (16 rows x 128 columns = one group
// of 16 rows).  Lane L = 16c + r reads the 32 values of row r that it will
// own in the packed tile (columns 32t + 8c + j), so the group's min/max is a
// reduction over the four lanes r, r+16, r+32, r+48 and the lane then writes
// its 16 packed bytes directly.  Lane r of octet 0 writes the row's scale and
// zero point; the wave of a row's last group also zeroes its padding slots.
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool finite_h(_Float16 x) {
  const uint16_t b = __builtin_bit_cast(uint16_t, x);
  return (b & 0x7C00u) != 0x7C00u;
}

// keep (optional): one bit per weight, row-major (bit k % 8 of byte
// (n * K + k) / 8); a set bit marks a weight kept in fp16 elsewhere, which is
// quantized here as 0 (it leaves the group range, and its code is the zero
// point, so it decodes to exactly 0).
// rmin, rmax (optional): the range of each row's W' (per-channel or
// per-tensor granularity) in place of each group's own.
// W8: INT8 codes (0..255, scale = range / 255), a 2048-byte tile per group of
// a row block, 32 bytes per lane (byte 8 t + j holds column 32 t + 8 c + j).
// Row blocks b0 .. b0 + nbw - 1 only (the whole matrix in one launch, or one
// chunk of rows whose ranges rmin/rmax hold: row n reads entry (n - 16 b0) *
// rstride, so rstride 0 gives every row the tensor's range).
template <bool SYM, bool W8>
__global__ __launch_bounds__(256) void pack_kernel(const _Float16 *__restrict__ W,
                                                   const _Float16 *__restrict__ s, int N, int K,
                                                   int b0, int nbw,
                                                   const uint8_t *__restrict__ keep,
                                                   const double *__restrict__ rmin,
                                                   const double *__restrict__ rmax, int rstride,
                                                   u32x4 *__restrict__ Wq,
                                                   _Float16 *__restrict__ scales,
                                                   _Float16 *__restrict__ zeros,
                                                   unsigned *__restrict__ status) {
#pragma clang fp contract(off)
  const int G = K / kGroup, NB = N / kTileRows;
  const long long tiles = (long long)nbw * G;
  // the wave's tile among the window's: group-major like the stored order
  const long long local = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (local >= tiles) return;  // uniform per wave
  const int lane = threadIdx.x & 63;
  const int c = lane >> 4, r = lane & 15;
  const int g = (int)(local / nbw), b = b0 + (int)(local % nbw);
  const long long tile = (long long)g * NB + b;  // stored position
  const int n = b * kTileRows + r;

  double wp[32];
  unsigned bad = 0;
  double mn = 0.0, mx = 0.0;  // the range always contains 0
  const _Float16 *wrow = W + (size_t)n * K + (size_t)g * kGroup + 8 * c;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const half8 wv = load_half8(wrow + 32 * t);
    // the 8 columns g * 128 + 32 t + 8 c .. + 7 are one byte of the mask
    const unsigned kb =
        keep ? keep[((size_t)n * K + (size_t)g * kGroup + 32 * t + 8 * c) >> 3] : 0u;
    half8 sv;
    if (s) {
      sv = load_half8(s + (size_t)g * kGroup + 32 * t + 8 * c);
    } else {
      const half8 one = {1, 1, 1, 1, 1, 1, 1, 1};
      sv = one;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!finite_h(wv[j]) || !finite_h(sv[j]) || !((double)sv[j] > 0.0)) bad |= kPackNonFinite;
      const double q = (kb >> j) & 1u ? 0.0 : (double)wv[j] / (double)sv[j];
      wp[8 * t + j] = q;
      mn = q < mn ? q : mn;
      mx = q > mx ? q : mx;
    }
  }
  // The four lanes that share row r hold the four column octets of the group.
  mn = fmin(mn, __shfl_xor(mn, 16));
  mn = fmin(mn, __shfl_xor(mn, 32));
  mx = fmax(mx, __shfl_xor(mx, 16));
  mx = fmax(mx, __shfl_xor(mx, 32));
  if (rmin) {  // a coarser granularity: the row's (or tensor's) range, still containing 0
    const int ri = (n - b0 * kTileRows) * rstride;
    mn = fmin(rmin[ri], 0.0);
    mx = fmax(rmax[ri], 0.0);
  }

  // asymmetric: the range [mn, mx]; symmetric: the largest magnitude
  const double range = SYM ? (mx > -mn ? mx : -mn) : mx - mn;
  _Float16 sc16 = 0, z16 = SYM ? (_Float16)8 : (_Float16)0;
  double scale = 1.0, z = SYM ? 8.0 : 0.0;
  const bool live = range > 0.0;
  if (live) {
    if (!fp16_ceil(range / (SYM ? 7.0 : (W8 ? 255.0 : 15.0)), &sc16)) {
      bad |= kPackRange;
      sc16 = 0;
    } else {
      scale = (double)sc16;
      if (!SYM) {
        z = rint(-mn / scale);
        z16 = (_Float16)(int)z;  // the integer 0..15; via int so that -0.0 stores as +0
      }
    }
  }

  if (W8) {  // byte 8 t + j of the lane's 32 bytes: column 32 t + 8 c + j
    uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (live) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          double v = rint(wp[8 * t + j] / scale) + z;
          v = v < 0.0 ? 0.0 : (v > 255.0 ? 255.0 : v);
          words[2 * t + j / 4] |= (uint32_t)v << (8 * (j % 4));
        }
    }
    u32x4 lo = {words[0], words[1], words[2], words[3]}, hi = {words[4], words[5], words[6], words[7]};
    Wq[tile * 128 + lane * 2] = lo;
    Wq[tile * 128 + lane * 2 + 1] = hi;
  }
  // an all-zero group: codes 0 (asymmetric) or 8 (symmetric, the zero point)
  const uint32_t fill = SYM ? 0x88888888u : 0u;
  u32x4 out = {fill, fill, fill, fill};
  if (live && !W8) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        double v;
        if (SYM) {
          v = rint(wp[8 * t + j] / scale);
          v = (v < -7.0 ? -7.0 : (v > 7.0 ? 7.0 : v)) + 8.0;
        } else {
          v = rint(wp[8 * t + j] / scale) + z;
          v = v < 0.0 ? 0.0 : (v > 15.0 ? 15.0 : v);
        }
        const uint32_t code = (uint32_t)v;
        const int slot = (j >> 1) + 4 * (j & 1);  // column j -> 4-bit slot
        word |= code << (4 * slot);
      }
      out[t] = word;
    }
  }
  if (!W8) Wq[tile * 64 + lane] = out;
  if (c == 0) {
    scales[meta_index(n, g, NB)] = sc16;
    zeros[meta_index(n, g, NB)] = z16;
  } else if (g == G - 1 && G - 1 + c < meta_groups(G)) {
    // the last tile of a row also clears the row's padding slots (at most 3)
    scales[meta_index(n, G - 1 + c, NB)] = (_Float16)0;
    zeros[meta_index(n, G - 1 + c, NB)] = (_Float16)0;
  }
  if (bad) atomicOr(status, bad);
}

// Per row n = n0 + i: the least and largest W' = W / s over the row (kept
// weights count as 0) into rmin[i], rmax[i], one workgroup per row.  Exact:
// min and max round nothing.
__global__ __launch_bounds__(256) void row_range_kernel(const _Float16 *__restrict__ W,
                                                        const _Float16 *__restrict__ s, int K,
                                                        int n0, const uint8_t *__restrict__ keep,
                                                        double *__restrict__ rmin,
                                                        double *__restrict__ rmax) {
#pragma clang fp contract(off)
  __shared__ double red[2][4];
  const int i = blockIdx.x, n = n0 + i, tid = threadIdx.x;
  double lo = 0.0, hi = 0.0;  // 0 is in every range anyway
  for (int k0 = 8 * tid; k0 < K; k0 += 8 * 256) {
    const half8 wv = load_half8(W + (size_t)n * K + k0);
    const unsigned kb = keep ? keep[((size_t)n * K + k0) >> 3] : 0u;
    half8 sv;
    if (s) {
      sv = load_half8(s + k0);
    } else {
      const half8 one = {1, 1, 1, 1, 1, 1, 1, 1};
      sv = one;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double q = (kb >> j) & 1u ? 0.0 : (double)wv[j] / (double)sv[j];
      lo = q < lo ? q : lo;
      hi = q > hi ? q : hi;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fmin(lo, __shfl_xor(lo, o));
    hi = fmax(hi, __shfl_xor(hi, o));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = lo;
    red[1][tid >> 6] = hi;
  }
  __syncthreads();
  if (tid == 0) {
    rmin[i] = fmin(fmin(red[0][0], red[0][1]), fmin(red[0][2], red[0][3]));
    rmax[i] = fmax(fmax(red[1][0], red[1][1]), fmax(red[1][2], red[1][3]));
  }
}

// The tensor's range, one chunk of rows at a time: acc[0] = the least of the
// chunk's rmin[0 .. rows) and of acc[0] (of 0 for the first chunk), acc[1] the
// largest of rmax and acc[1].  One workgroup.
__global__ __launch_bounds__(256) void tensor_range_kernel(int rows, const double *__restrict__ rmin,
                                                           const double *__restrict__ rmax,
                                                           double *__restrict__ acc, int first) {
  __shared__ double red[2][4];
  const int tid = threadIdx.x;
  double lo = first ? 0.0 : acc[0], hi = first ? 0.0 : acc[1];
  for (int n = tid; n < rows; n += 256) {
    lo = fmin(lo, rmin[n]);
    hi = fmax(hi, rmax[n]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fmin(lo, __shfl_xor(lo, o));
    hi = fmax(hi, __shfl_xor(hi, o));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = lo;
    red[1][tid >> 6] = hi;
  }
  __syncthreads();
  if (tid == 0) {
    acc[0] = fmin(fmin(red[0][0], red[0][1]), fmin(red[0][2], red[0][3]));
    acc[1] = fmax(fmax(red[1][0], red[1][1]), fmax(red[1][2], red[1][3]));
  }
}

}  // namespace

hipError_t launch_row_range(const void *W, const void *s, int n0, int rows, int K,
                            const uint8_t *keep, double *rmin, double *rmax, hipStream_t stream) {
  hipLaunchKernelGGL(row_range_kernel, dim3(rows), dim3(256), 0, stream, (const _Float16 *)W,
                     (const _Float16 *)s, K, n0, keep, rmin, rmax);
  return hipGetLastError();
}

hipError_t launch_tensor_range(int rows, const double *rmin, const double *rmax, double *acc,
                               bool first, hipStream_t stream) {
  hipLaunchKernelGGL(tensor_range_kernel, dim3(1), dim3(256), 0, stream, rows, rmin, rmax, acc,
                     first ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_pack(const void *W, const void *s, int N, int K, int b0, int nbw,
                       const uint8_t *keep, const double *rmin, const double *rmax, int rstride,
                       void *Wq, void *scales, void *zeros, unsigned *status, bool symmetric,
                       hipStream_t stream, bool w8) {
  const long long tiles = (long long)nbw * (K / kGroup);
  const long long blocks = (tiles + 3) / 4;
  if (w8)
    hipLaunchKernelGGL((pack_kernel<false, true>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const _Float16 *)W, (const _Float16 *)s, N, K, b0, nbw, keep, rmin, rmax,
                       rstride, (u32x4 *)Wq, (_Float16 *)scales, (_Float16 *)zeros, status);
  else if (symmetric)
    hipLaunchKernelGGL((pack_kernel<true, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const _Float16 *)W, (const _Float16 *)s, N, K, b0, nbw, keep, rmin, rmax,
                       rstride, (u32x4 *)Wq, (_Float16 *)scales, (_Float16 *)zeros, status);
  else
    hipLaunchKernelGGL((pack_kernel<false, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const _Float16 *)W, (const _Float16 *)s, N, K, b0, nbw, keep, rmin, rmax,
                       rstride, (u32x4 *)Wq, (_Float16 *)scales, (_Float16 *)zeros, status);
  return hipGetLastError();
}

}  // namespace w4a16
