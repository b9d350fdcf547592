// FP16 outlier side path, offline part: pick the weights that stay in fp16.
//
// The practitioner notes at mhpq.cn (section 2.2, outlier handling) keep the
// top 0.1% of the weights by magnitude in an FP16 sub-tensor and quantize the
// rest to INT4; the two are merged with where(mask, fp16, int4).  Here:
//   * the ranking key of W[n][k] is |W[n][k] / s[k]| (|W| without s), one
//     correctly rounded fp64 division -- for fp16 operands it keeps the order
//     of the exact quotients and keeps distinct quotients distinct -- compared
//     as its IEEE bit pattern (non-negative doubles order like their bits);
//   * exactly `count` weights are kept; ties at the threshold go to the lower
//     flat index n * K + k;
//   * the kept weights are written row-compressed (row_ptr, col, val = the
//     original fp16 W) and as a bit mask (bit k % 64 of word n * K / 64 + k / 64)
//     that the packer reads: it quantizes the other weights as usual and
//     treats the kept ones as 0, so their codes decode to exactly 0.
//
// The threshold is found by an exact radix select over the 64-bit keys: eight
// passes of 8 bits, each a histogram (LDS per workgroup, then global) of the
// next digit among the keys that match the digits fixed so far; the host picks
// the digit holding the count-th largest key after each pass.  Then one pass
// counts, per row, the keys above the threshold and equal to it; the host
// turns the counts into the row pointers and into how many of each row's ties
// are kept (the first ones in flat order); one wave per row writes its kept
// weights in column order.
#include <algorithm>
#include <vector>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint64_t rank_key(_Float16 w, _Float16 s) {
  const double q = (double)w / (double)s;
  return __builtin_bit_cast(uint64_t, fabs(q));
}

// Histogram of digit (key >> shift) & 255 over the keys whose bits above the
// digit equal those of `prefix`.  Eight consecutive elements per thread step.
__global__ __launch_bounds__(kThreads) void digit_hist_kernel(const _Float16 *__restrict__ W,
                                                              const _Float16 *__restrict__ s,
                                                              long long octets, int K,
                                                              uint64_t prefix, int shift,
                                                              unsigned *__restrict__ hist) {
  __shared__ unsigned h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int above = shift + 8;  // bits [above, 64) must match
  for (long long o = (long long)blockIdx.x * kThreads + threadIdx.x; o < octets;
       o += (long long)gridDim.x * kThreads) {
    const long long e0 = o * 8;
    const int k0 = (int)(e0 % K);
    const half8 wv = load_half8(W + e0);
    half8 sv;
    if (s) {
      sv = load_half8(s + k0);
    } else {
      const half8 one = {1, 1, 1, 1, 1, 1, 1, 1};
      sv = one;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t key = rank_key(wv[j], sv[j]);
      if (above >= 64 || (key >> above) == (prefix >> above))
        atomicAdd(&h[(key >> shift) & 255u], 1u);
    }
  }
  __syncthreads();
  const unsigned v = h[threadIdx.x];
  if (v) atomicAdd(&hist[threadIdx.x], v);
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Per row n: keys above T and keys equal to T.  One workgroup per row.
__global__ __launch_bounds__(kThreads) void row_count_kernel(const _Float16 *__restrict__ W,
                                                             const _Float16 *__restrict__ s, int K,
                                                             uint64_t T, int *__restrict__ cnt_gt,
                                                             int *__restrict__ cnt_eq) {
  __shared__ int red[2][kThreads / 64];
  const int n = blockIdx.x, tid = threadIdx.x;
  int gt = 0, eq = 0;
  for (int k0 = 8 * tid; k0 < K; k0 += 8 * kThreads) {
    const half8 wv = load_half8(W + (size_t)n * K + k0);
    half8 sv;
    if (s) {
      sv = load_half8(s + k0);
    } else {
      const half8 one = {1, 1, 1, 1, 1, 1, 1, 1};
      sv = one;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t key = rank_key(wv[j], sv[j]);
      gt += key > T;
      eq += key == T;
    }
  }
  gt = wave_sum_int(gt);
  eq = wave_sum_int(eq);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = gt;
    red[1][tid >> 6] = eq;
  }
  __syncthreads();
  if (tid < 2) {
    int v = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) v += red[tid][w];
    (tid == 0 ? cnt_gt : cnt_eq)[n] = v;
  }
}

// One wave per row: walk the row 64 columns at a time, keep the keys above T
// and the first take_eq[n] keys equal to T, write them at row_ptr[n] onwards
// in column order, and write the row's mask words.
__global__ __launch_bounds__(kThreads) void fill_kernel(
    const _Float16 *__restrict__ W, const _Float16 *__restrict__ s, int N, int K, uint64_t T,
    const int *__restrict__ take_eq, const int32_t *__restrict__ row_ptr, int32_t *__restrict__ col,
    _Float16 *__restrict__ val, uint64_t *__restrict__ mask) {
  const int n = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (n >= N) return;  // uniform per wave
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes under this one
  int out = row_ptr[n], seen_eq = 0;
  const int take = take_eq[n];
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int k = k0 + lane;
    const _Float16 w = W[(size_t)n * K + k];
    const uint64_t key = rank_key(w, s ? s[k] : (_Float16)1);
    const bool eq = key == T;
    const uint64_t eqb = __ballot(eq);
    const bool keep = key > T || (eq && seen_eq + __popcll(eqb & below) < take);
    const uint64_t kb = __ballot(keep);
    if (keep) {
      const int pos = out + __popcll(kb & below);
      col[pos] = k;
      val[pos] = w;
    }
    if (lane == 0) mask[((size_t)n * K + k0) / 64] = kb;
    out += __popcll(kb);
    seen_eq += __popcll(eqb);
  }
}

}  // namespace

size_t outlier_workspace_bytes(int N, int K) {
  const size_t head = 1024 + ((size_t)3 * N * sizeof(int) + 255) / 256 * 256;
  return head + ((size_t)N * K / 8 + 255) / 256 * 256;
}

int select_outliers(const void *W, const void *s, int N, int K, long long count, int32_t *row_ptr,
                    int32_t *col, _Float16 *val, void *workspace, const uint8_t **mask_out,
                    hipStream_t st) {
  char *ws = static_cast<char *>(workspace);
  unsigned *hist = reinterpret_cast<unsigned *>(ws);
  int *cnt_gt = reinterpret_cast<int *>(ws + 1024);
  int *cnt_eq = cnt_gt + N;
  int *take_d = cnt_eq + N;
  uint64_t *mask =
      reinterpret_cast<uint64_t *>(ws + 1024 + ((size_t)3 * N * sizeof(int) + 255) / 256 * 256);
  *mask_out = reinterpret_cast<const uint8_t *>(mask);
  const _Float16 *Wh = static_cast<const _Float16 *>(W), *sh = static_cast<const _Float16 *>(s);
  const long long total = (long long)N * K;

  std::vector<int32_t> rp(N + 1, 0);
  if (count == 0) {
    if (hipMemsetAsync(mask, 0, (size_t)total / 8, st) != hipSuccess) return -1;
    if (hipMemcpyAsync(row_ptr, rp.data(), sizeof(int32_t) * (N + 1), hipMemcpyHostToDevice,
                       st) != hipSuccess)
      return -1;
    return hipStreamSynchronize(st) == hipSuccess ? 0 : -1;
  }

  // radix select: the count-th largest key T, and how many keys equal to T
  // are kept (`need`)
  const long long octets = total / 8;
  const int grid = (int)std::min<long long>(2048, (octets + kThreads - 1) / kThreads);
  uint64_t prefix = 0;
  long long need = count;
  unsigned h[256];
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (hipMemsetAsync(hist, 0, sizeof(h), st) != hipSuccess) return -1;
    hipLaunchKernelGGL(digit_hist_kernel, dim3(grid), dim3(kThreads), 0, st, Wh, sh, octets, K,
                       prefix, shift, hist);
    if (hipGetLastError() != hipSuccess) return -1;
    if (hipMemcpyAsync(h, hist, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess) return -1;
    if (hipStreamSynchronize(st) != hipSuccess) return -1;
    int d = 255;
    for (; d > 0 && need > (long long)h[d]; --d) need -= h[d];
    prefix |= (uint64_t)d << shift;
  }
  const uint64_t T = prefix;

  // per-row counts -> row pointers and kept ties per row (the first `need`
  // ties in flat order)
  hipLaunchKernelGGL(row_count_kernel, dim3(N), dim3(kThreads), 0, st, Wh, sh, K, T, cnt_gt,
                     cnt_eq);
  if (hipGetLastError() != hipSuccess) return -1;
  std::vector<int> gt(N), eq(N), take(N);
  if (hipMemcpyAsync(gt.data(), cnt_gt, sizeof(int) * N, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(eq.data(), cnt_eq, sizeof(int) * N, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return -1;
  long long ties_before = 0;
  for (int n = 0; n < N; ++n) {
    const long long t = std::min<long long>(eq[n], std::max<long long>(0, need - ties_before));
    take[n] = (int)t;
    ties_before += eq[n];
    rp[n + 1] = rp[n] + gt[n] + (int)t;
  }
  if (rp[N] != count) return -1;  // cannot happen: the select counted these keys
  if (hipMemcpyAsync(take_d, take.data(), sizeof(int) * N, hipMemcpyHostToDevice, st) !=
          hipSuccess ||
      hipMemcpyAsync(row_ptr, rp.data(), sizeof(int32_t) * (N + 1), hipMemcpyHostToDevice, st) !=
          hipSuccess)
    return -1;
  hipLaunchKernelGGL(fill_kernel, dim3((N + 3) / 4), dim3(kThreads), 0, st, Wh, sh, N, K, T,
                     take_d, row_ptr, col, val, mask);
  if (hipGetLastError() != hipSuccess) return -1;
  // the host vectors above are read by the copies: finish before they go
  return hipStreamSynchronize(st) == hipSuccess ? 0 : -1;
}

}  // namespace w4a16
