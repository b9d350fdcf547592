// Tiled dequantize-matmul for large M (batched decode, prefill):
// Y[M][N] = X[M][K] . W_hat^T.
//
// The nano-vllm tutorial (discosf.com), section 1.1, describes prefill as one
// large matmul bounded by arithmetic, so this kernel is organised around the
// MFMA units.  A workgroup of WM x WN waves owns a BM x BN block of Y; each
// wave owns TM x TN 16x16 sub-blocks (TM*16 rows of X, TN*16 rows of W) and
// accumulates them in fp32 with 16x16x32 fp16 MFMAs.  K is walked in stages
// of KSTAGE columns (one quantization group, or half of one):
//   * X * s for the block's rows (rounded to fp16 once) goes through LDS,
//     double-buffered: the next stage's global loads are issued before the
//     current stage's MFMAs and written to the other buffer after them, with
//     one LDS barrier per stage;
//   * the packed weight tile layout makes each lane's 32-bit code word its
//     MFMA B operand, so W never touches LDS: every wave loads its own tiles
//     one group ahead (a 128-bit load per lane per 16-row tile), decodes them
//     to exact (q - z) and multiplies by the group scale in fp16 -- the
//     weight-only "dequantize to FP16, then multiply" of "Chapter 22"
//     (aiwing.uk) section 22.3 -- just before use.
#include <type_traits>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;      // raw buffer resource, 32-bit data format

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its outstanding global loads (which stay in flight across the barrier).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(bits));
  return r;
}

// Eight codes of one word -> (q_j - z) * scale in fp16, j = 0..7: (q - z) is
// formed exactly (see the streaming kernel), then rounded once by the scale.
__device__ __forceinline__ half8 dequant_word(uint32_t w, half2v bias_lo, half2v bias_hi,
                                              half2v scale) {
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = kMagic2;
  const uint32_t w8 = w >> 8;
  const half2v a = (as_half2(and_or(w, m_lo, magic)) - bias_lo) * scale;
  const half2v b = (as_half2(and_or(w, m_hi, magic)) * sixteenth - bias_hi) * scale;
  const half2v c = (as_half2(and_or(w8, m_lo, magic)) - bias_lo) * scale;
  const half2v d = (as_half2(and_or(w8, m_hi, magic)) * sixteenth - bias_hi) * scale;
  half8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// Two waves per SIMD: with one, the waits on LDS and the barriers are not
// hidden and MFMA throughput roughly halves (measured on the 70B shapes).
template <int WM, int WN, int TM, int TN, int KSTAGE, bool HAS_S>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void tiled_kernel(
    const _Float16 *__restrict__ X, const uint8_t *__restrict__ Wq,
    const _Float16 *__restrict__ scales, const _Float16 *__restrict__ zeros,
    const _Float16 *__restrict__ s, _Float16 *__restrict__ Y, int M, int N, int K) {
  constexpr int THREADS = WM * WN * 64;
  constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
  constexpr int kStageK = KSTAGE;                       // K columns per stage (64 or 128)
  constexpr int kLdsStride = kStageK + 8;               // halves; the pad spreads rows over banks
  constexpr int kStagesPerGroup = kGroup / kStageK;
  constexpr int kChunksPerRow = kStageK / 8;            // 16-byte chunks per A row per stage
  constexpr int ROWS_PER_PASS = THREADS / kChunksPerRow;  // A rows one load pass covers
  constexpr int A_PER_T = BM / ROWS_PER_PASS;           // 16-byte A chunks per thread
  static_assert(BM % ROWS_PER_PASS == 0, "A tile rows must divide evenly");
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * kLdsStride];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform_int(tid >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int wm = wave / WN, wn = wave % WN;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int G = K / kGroup, NB = N / kTileRows;
  const int Gq = meta_groups(G) / kMetaQuad;
  const int stages = kStagesPerGroup * G;  // stage st covers columns [KSTAGE st, +KSTAGE)

  // ---- X * s staging: thread covers one 16-byte column chunk of rows a_row + pass*ROWS_PER_PASS
  const int a_col = (tid % kChunksPerRow) * 8;
  const int a_row = tid / kChunksPerRow;
  // The loads are unconditional (rows past M read row M-1) and nothing uses
  // their results until store_a, after the stage's MFMAs, so their latency is
  // hidden; rows past M are zeroed and X * s is formed only then.
  half8 areg[A_PER_T], sreg;
  auto load_a = [&](int st) {
    const int k0 = st * kStageK + a_col;
    if (HAS_S) sreg = load_half8(s + k0);
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int m = min(m0 + a_row + i * ROWS_PER_PASS, M - 1);
      areg[i] = load_half8(X + (size_t)m * K + k0);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      half8 v = areg[i];
      if (HAS_S) v = v * sreg;
      if (m0 + a_row + i * ROWS_PER_PASS >= M) v = zero_half8();
      *reinterpret_cast<half8 *>(&As[buf][(a_row + i * ROWS_PER_PASS) * kLdsStride + a_col]) = v;
    }
  };

  // ---- weights: this wave's TN row blocks, loaded a group ahead
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)Wq, (short)0, (int)min((size_t)0x7fffffff, (size_t)N * K / 2), kRsrcWord3);
  const size_t meta_bytes = (size_t)N * Gq * kMetaQuad * 2;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)scales, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)zeros, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const int rb0 = n0 / kTileRows + wn * TN;  // first row block of this wave
  u32x4 bcode[TN], bnext[TN];
  // raw fp16 bits of each row block's scale and zero point for the group
  uint32_t bsc[TN], bzp[TN], bsc_next[TN], bzp_next[TN];
  auto load_b = [&](int g, u32x4 *code, uint32_t *sc, uint32_t *zp) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      // row blocks past N read zeros (bounds-checked buffer loads) and are never stored
      const int rb = min(rb0 + j, NB);
      code[j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, (rb * G * 64 + lane) * 16,
                                                        g * kTileBytes, 0));
      const int mo = ((rb * Gq + g / kMetaQuad) * kTileRows + r) * kMetaQuad * 2;
      sc[j] = __builtin_amdgcn_raw_buffer_load_b16(srs, mo, (g % kMetaQuad) * 2, 0);
      zp[j] = __builtin_amdgcn_raw_buffer_load_b16(zrs, mo, (g % kMetaQuad) * 2, 0);
    }
  };

  float4v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  // MFMAs of the k steps of stage h of a group (k steps t = h*KS .. h*KS + KS-1,
  // KS = KSTAGE / 32) with the group's codes / metadata, reading X from LDS buffer `buf`.
  constexpr int KS = kStageK / 32;
  auto compute_stage = [&](auto H, const u32x4 *code, const uint32_t *sc, const uint32_t *zp,
                           int buf) {
    constexpr int h = decltype(H)::value;
    const _Float16 *abuf = As[buf] + (wm * TM * 16 + r) * kLdsStride + 8 * c;
#pragma unroll
    for (int tt = 0; tt < KS; ++tt) {
      half8 bop[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)zp[j]);
        const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)sc[j]);
        const _Float16 blo = (_Float16)1024.0f + z, bhi = (_Float16)64.0f + z;
        const half2v bias_lo = {blo, blo}, bias_hi = {bhi, bhi}, scale = {sv, sv};
        bop[j] = dequant_word(code[j][h * KS + tt], bias_lo, bias_hi, scale);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const half8 aop = *reinterpret_cast<const half8 *>(abuf + i * 16 * kLdsStride + 32 * tt);
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(aop, bop[j], acc[i][j]);
      }
    }
  };

  load_a(0);
  load_b(0, bcode, bsc, bzp);
  store_a(0);
  lds_barrier();
  // One group per iteration, kStagesPerGroup stages; stage st uses LDS buffer
  // st % 2.  The next group's codes are loaded during the first stage and moved
  // into place at the end of the group.
  for (int g = 0; g < G; ++g) {
    const int st = kStagesPerGroup * g;
    if (st + 1 < stages) load_a(st + 1);
    if (g + 1 < G) load_b(g + 1, bnext, bsc_next, bzp_next);
    if constexpr (kStagesPerGroup == 2) {
      compute_stage(std::integral_constant<int, 0>(), bcode, bsc, bzp, 0);
      store_a(1);
      lds_barrier();
      if (st + 2 < stages) load_a(st + 2);
      compute_stage(std::integral_constant<int, 1>(), bcode, bsc, bzp, 1);
      if (st + 2 < stages) store_a(0);
    } else {
      compute_stage(std::integral_constant<int, 0>(), bcode, bsc, bzp, g & 1);
      if (st + 1 < stages) store_a((g + 1) & 1);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      bcode[j] = bnext[j];
      bsc[j] = bsc_next[j];
      bzp[j] = bzp_next[j];
    }
    lds_barrier();
  }

  // lane holds D[4c + v][r] of each 16x16 sub-block
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + (wn * TN + j) * 16 + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + (wm * TM + i) * 16 + 4 * c + v;
        if (m < M && n < N) Y[(size_t)m * N + n] = (_Float16)acc[i][j][v];
      }
    }
  }
}

template <int WM, int WN, int TM, int TN, int KSTAGE>
hipError_t launch_cfg(const void *X, const void *Wq, const void *scales, const void *zeros,
                      const void *s, void *Y, int M, int N, int K, hipStream_t stream) {
  constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
  const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(WM * WN * 64);
  if (s)
    hipLaunchKernelGGL((tiled_kernel<WM, WN, TM, TN, KSTAGE, true>), grid, block, 0, stream,
                       (const _Float16 *)X, (const uint8_t *)Wq, (const _Float16 *)scales,
                       (const _Float16 *)zeros, (const _Float16 *)s, (_Float16 *)Y, M, N, K);
  else
    hipLaunchKernelGGL((tiled_kernel<WM, WN, TM, TN, KSTAGE, false>), grid, block, 0, stream,
                       (const _Float16 *)X, (const uint8_t *)Wq, (const _Float16 *)scales,
                       (const _Float16 *)zeros, (const _Float16 *)s, (_Float16 *)Y, M, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tiled(const void *X, const void *Wq, const void *scales, const void *zeros,
                        const void *s, void *Y, int M, int N, int K, hipStream_t stream) {
  // 64 x 256 blocks of 4 waves (64 x 64 each), one group per stage, two
  // workgroups per CU: the fastest of the measured shapes and stage widths at
  // every M of the workloads.
  return launch_cfg<1, 4, 4, 4, 128>(X, Wq, scales, zeros, s, Y, M, N, K, stream);
}

}  // namespace w4a16
