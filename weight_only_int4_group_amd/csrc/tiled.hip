// Tiled dequantize-matmul for large M (batched decode, prefill):
// Y[M][N] = X[M][K] . W_hat^T.
//
// The nano-vllm tutorial (discosf.com), section 1.1, describes prefill as one
// large matmul bounded by arithmetic, so this kernel is organised around the
// MFMA units.  A workgroup of WM x WN waves owns a BM x BN block of Y; each
// wave owns TM x TN 16x16 sub-blocks (TM*16 rows of X, TN*16 rows of W) and
// accumulates them in fp32 with 16x16x32 fp16 MFMAs.  K is walked one
// quantization group (128 columns) per stage:
//   * X * s for the block's rows (rounded to fp16 once) goes through LDS,
//     double-buffered: the next stage's global loads are issued before the
//     current stage's MFMAs and written to the other buffer after them, with
//     one LDS barrier per stage;
//   * the packed weight tile layout makes each lane's 32-bit code word its
//     MFMA B operand, so W is never rearranged: every wave fetches its own
//     tiles one group ahead (16 bytes per lane per 16-row tile, copied
//     unchanged into the wave's LDS slots by DMA loads, which costs no
//     registers while in flight), takes them into registers, decodes them to
//     exact (q - z) and multiplies by the group scale in fp16 -- the
//     weight-only "dequantize to FP16, then multiply" of "Chapter 22"
//     (aiwing.uk) section 22.3 -- just before use.
//
// Several problems share one launch (a layer's projections), and when the
// blocks of a call would leave CUs idle (few output blocks, long K: batched
// decode, small projections) K is split across workgroups: each split writes
// its fp32 partial block to a caller-provided workspace and a second small
// kernel adds the splits in a fixed order and rounds to fp16 once, so results
// are reproducible run to run.
#include <algorithm>
#include <type_traits>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

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

// bf16 activations: eight codes -> bf16((q_j - z) * scale), each rounded once.
// and_or builds the exact bf16 128 + q (see the streaming kernel); as fp32 it
// is one shift or mask away, and one FMA with the fp32 scale, minus
// (128 + z) * scale, leaves (q - z) * scale before the bf16 rounding.
__device__ __forceinline__ u32x4 dequant_word_bf16(uint32_t w, float scale, float zb) {
  const uint32_t m = 0x000F000Fu;
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t x = and_or(w >> (4 * p), m, kMagicBF);
    const float lo = __builtin_fmaf(__builtin_bit_cast(float, x << 16), scale, -zb);
    const float hi = __builtin_fmaf(__builtin_bit_cast(float, x & 0xFFFF0000u), scale, -zb);
    r[p] = pack_bf16x2(lo, hi);
  }
  return r;
}

// INT8 codes: two words (columns j = 0..3 and 4..7, one byte each) ->
// (q_j - z) * scale in fp16: v_perm_b32 builds the exact 1024 + q (see the
// streaming kernel), minus (1024 + z) is exact, one rounding by the scale.
__device__ __forceinline__ half8 dequant_words8(uint32_t wa, uint32_t wb, half2v bias, half2v scale) {
  const uint32_t magic = 0x64646464u;
  const half2v a = (as_half2(__builtin_amdgcn_perm(magic, wa, 0x05010400u)) - bias) * scale;
  const half2v b = (as_half2(__builtin_amdgcn_perm(magic, wa, 0x05030402u)) - bias) * scale;
  const half2v c = (as_half2(__builtin_amdgcn_perm(magic, wb, 0x05010400u)) - bias) * scale;
  const half2v d = (as_half2(__builtin_amdgcn_perm(magic, wb, 0x05030402u)) - bias) * scale;
  half8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// INT8 codes, bf16 activations: eight codes (columns j = 0..3 in wa, 4..7 in
// wb) -> bf16((q_j - z) * scale), each rounded once: a byte converts to fp32
// exactly, one FMA with the fp32 scale minus z * scale.
__device__ __forceinline__ u32x4 dequant_words8_bf16(uint32_t wa, uint32_t wb, float scale,
                                                     float zs) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t w = p < 2 ? wa : wb;
    const int sh = (p & 1) * 16;
    const float lo = __builtin_fmaf((float)((w >> sh) & 0xFFu), scale, -zs);
    const float hi = __builtin_fmaf((float)((w >> (sh + 8)) & 0xFFu), scale, -zs);
    r[p] = pack_bf16x2(lo, hi);
  }
  return r;
}

constexpr int kMaxTiled = 8;  // problems per launch

struct TiledProblem {
  const _Float16 *X;
  const uint8_t *Wq;
  const _Float16 *scales, *zeros, *s;
  _Float16 *Y;
  float *part;      // split > 1: split fp32 [M][N] partial slabs
  int M, N, K;
  int tiles_n;      // output blocks along N
  int tiles;        // output blocks (tiles_n * blocks along M)
  int split;        // K ranges per output block
  int block0;       // first workgroup of this problem in the GEMM launch
  int rblock0;      // first workgroup of this problem in the reduction launch
  const int32_t *orp, *ocol;  // fp16 outliers, row-compressed (null: none)
  const _Float16 *oval;
  int bf16;                   // X and Y are bf16 (one value per launch)
  const _Float16 *xs;         // tiled_dma_kernel: X * s (prescaled), or X when s is null
};

struct TiledSet {
  TiledProblem p[kMaxTiled];
  int count;
};

template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

// The problem of workgroup `block` (first workgroups given by `first`), every
// field in scalar registers.
template <bool REDUCE>
__device__ __forceinline__ TiledProblem find_tiled(const TiledSet &ts, int block) {
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxTiled; ++i)
    if (i < ts.count && block >= (REDUCE ? ts.p[i].rblock0 : ts.p[i].block0)) pi = i;
  const TiledProblem &q = ts.p[pi];
  TiledProblem P;
  P.X = uniform_ptr(q.X);
  P.Wq = uniform_ptr(q.Wq);
  P.scales = uniform_ptr(q.scales);
  P.zeros = uniform_ptr(q.zeros);
  P.s = uniform_ptr(q.s);
  P.Y = uniform_ptr(q.Y);
  P.part = uniform_ptr(q.part);
  P.M = uniform_int(q.M);
  P.N = uniform_int(q.N);
  P.K = uniform_int(q.K);
  P.tiles_n = uniform_int(q.tiles_n);
  P.tiles = uniform_int(q.tiles);
  P.split = uniform_int(q.split);
  P.block0 = uniform_int(q.block0);
  P.rblock0 = uniform_int(q.rblock0);
  P.orp = uniform_ptr(q.orp);
  P.ocol = uniform_ptr(q.ocol);
  P.oval = uniform_ptr(q.oval);
  P.bf16 = uniform_int(q.bf16);
  P.xs = uniform_ptr(q.xs);
  return P;
}

// Two waves per SIMD: with one, the waits on LDS and the barriers are not
// hidden and MFMA throughput roughly halves (measured on the 70B shapes).
template <int WM, int WN, int TM, int TN, bool OUT, bool BF, bool W8 = false>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void tiled_kernel(
    TiledSet ts) {
  constexpr int THREADS = WM * WN * 64;
  constexpr int kCW = W8 ? 2 : 1;  // 16-byte code pieces per lane per tile
  constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
  constexpr int kLdsStride = kGroup + 8;                  // halves; the pad spreads rows over banks
  constexpr int kChunksPerRow = kGroup / 8;               // 16-byte chunks per A row per stage
  constexpr int ROWS_PER_PASS = THREADS / kChunksPerRow;  // A rows one load pass covers
  constexpr int A_PER_T = BM / ROWS_PER_PASS;             // 16-byte A chunks per thread
  static_assert(BM % ROWS_PER_PASS == 0, "A tile rows must divide evenly");
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * kLdsStride];

  const int block = (int)blockIdx.x;
  const TiledProblem P = find_tiled<false>(ts, block);
  const _Float16 *__restrict__ X = P.X;
  const uint8_t *__restrict__ Wq = P.Wq;
  const _Float16 *__restrict__ scales = P.scales;
  const _Float16 *__restrict__ zeros = P.zeros;
  const _Float16 *__restrict__ s = P.s;
  const bool has_s = s != nullptr;  // else s = 1
  const int M = P.M, N = P.N, K = P.K;

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform_int(tid >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int wm = wave / WN, wn = wave % WN;
  // block -> (split sp, output block t); consecutive blocks share a K range
  // and walk N first, so neighbours share their rows of X
  const int local = block - P.block0;
  const int sp = local / P.tiles, t = local - sp * P.tiles;
  const int mt = t / P.tiles_n;
  const int n0 = (t - mt * P.tiles_n) * BN, m0 = mt * BM;
  const int G = K / kGroup, NB = N / kTileRows;
  const int Gq = meta_groups(G) / kMetaQuad;
  // this block's groups [gb, ge): the split-th of G, in whole groups
  const int gb = (int)((long long)G * sp / P.split), ge = (int)((long long)G * (sp + 1) / P.split);

  // ---- X * s, one group (128 columns) per stage: a thread covers one 16-byte
  // column chunk of rows a_row + i * ROWS_PER_PASS.  The loads are
  // unconditional (rows past M read row M - 1: rows of A only reach the same
  // rows of D, which are not stored) and nothing uses their results until
  // store_a, after the stage's MFMAs, so their latency is hidden.
  const int a_col = (tid % kChunksPerRow) * 8;
  const int a_row = tid / kChunksPerRow;
  half8 areg[A_PER_T], sreg;
  auto load_a = [&](int g) {
    const int k0 = g * kGroup + a_col;
    if (has_s) {
      sreg = load_half8(s + k0);
    } else {
      const _Float16 one = (_Float16)1.0f;
      sreg = (half8){one, one, one, one, one, one, one, one};  // x * 1 is exact
    }
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int m = min(m0 + a_row + i * ROWS_PER_PASS, M - 1);
      areg[i] = load_half8(X + (size_t)m * K + k0);
    }
  };
  // with fp16 outliers, the group's s goes to LDS too (the outlier terms
  // divide the staged X * s by it)
  __shared__ __attribute__((aligned(16))) _Float16 Ss[OUT ? 2 : 1][OUT ? kGroup : 8];
  const bool has_out = OUT && P.orp != nullptr;
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      u32x4 v;
      if (BF) {  // bf16 X times fp16 s: exact in fp32, rounded once to bf16
        const u32x4 xw = __builtin_bit_cast(u32x4, areg[i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_to_f32((uint16_t)xw[q]) * (float)sreg[2 * q];
          const float hi = bf16_to_f32((uint16_t)(xw[q] >> 16)) * (float)sreg[2 * q + 1];
          v[q] = pack_bf16x2(lo, hi);
        }
      } else {
        v = __builtin_bit_cast(u32x4, areg[i] * sreg);
      }
      *reinterpret_cast<u32x4 *>(&As[buf][(a_row + i * ROWS_PER_PASS) * kLdsStride + a_col]) = v;
    }
    if (OUT && has_out && a_row == 0) *reinterpret_cast<half8 *>(&Ss[OUT ? buf : 0][a_col]) = sreg;
  };

  // ---- weights: this wave's TN row blocks.  The next group's code tiles go
  // straight from HBM to this wave's own LDS slots (one 16-byte DMA load per
  // lane per tile), so only the current group's codes occupy registers;
  // scales and zero points come as raw 16-bit words into one of two register
  // sets.
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)Wq, (short)0, (int)min((size_t)0x7fffffff, (size_t)N * K * kCW / 2), kRsrcWord3);
  const size_t meta_bytes = (size_t)N * Gq * kMetaQuad * 2;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)scales, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)zeros, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const int rb0 = n0 / kTileRows + wn * TN;  // first row block of this wave
  // INT8 tiles are twice as large: two 16-byte pieces per lane, the second
  // 1 KB after the first in LDS.  They use one LDS buffer, not two, so that
  // two workgroups still fit in a CU's LDS: each wave DMAs into and reads only
  // its own slots, so it can take the group's codes into registers, wait for
  // those reads, and then let the next group's DMA overwrite the slots.
  constexpr int kBBufs = W8 ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t Bs0[WM * WN * TN * kTileBytes * kCW];
  __shared__ __attribute__((aligned(16))) uint8_t Bs1[kBBufs > 1 ? WM * WN * TN * kTileBytes * kCW : 16];
  struct BRegs {
    u32x4 code[TN][kCW];
    uint32_t sc[TN], zp[TN];  // raw fp16 bits of each row block's scale and zero point
  };
  BRegs b0, b1;
  // group-major tiles and quad-major metadata: the row block's part of each
  // offset is per lane, the group's part uniform
  const int tile_stride = NB * kTileBytes * kCW, meta_stride = NB * kTileRows * kMetaQuad * 2;
  // code buffer `buf` of this wave: two separate LDS arrays (not one array
  // of two), so the compiler can tell a read of one from a DMA into the other
  auto bslot = [&](int buf) -> uint8_t * {
    return (kBBufs == 1 || buf % kBBufs == 0) ? Bs0 : Bs1;
  };
  // row blocks past N re-read the last one (in bounds) and are never stored
  auto load_codes = [&](int g, int buf) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int rb = min(rb0 + j, NB - 1);
#pragma unroll
      for (int h = 0; h < kCW; ++h)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wrs,
            (__attribute__((address_space(3))) void *)(bslot(buf) + ((wave * TN + j) * kCW + h) * kTileBytes),
            16, (rb * 64 + lane) * 16 * kCW + 16 * h, g * tile_stride, 0, 0);
    }
  };
  auto load_meta = [&](int g, BRegs &b) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int rb = min(rb0 + j, NB - 1);
      const int mo = (rb * kTileRows + r) * kMetaQuad * 2;
      const int qo = (g / kMetaQuad) * meta_stride + (g % kMetaQuad) * 2;
      b.sc[j] = __builtin_amdgcn_raw_buffer_load_b16(srs, mo, qo, 0);
      b.zp[j] = __builtin_amdgcn_raw_buffer_load_b16(zrs, mo, qo, 0);
    }
  };

  float4v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  // the four k steps of a group: dequantize this wave's B operands, then
  // TM x TN MFMAs reading A from LDS buffer `buf`
  auto compute = [&](const BRegs &b, int buf) {
    const _Float16 *abuf = As[buf] + (wm * TM * 16 + r) * kLdsStride + 8 * c;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (BF) {
        u32x4 bop[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)b.zp[j]);
          const float sv = (float)__builtin_bit_cast(_Float16, (uint16_t)b.sc[j]);
          bop[j] = W8 ? dequant_words8_bf16(b.code[j][tt >> 1 & (kCW - 1)][2 * (tt & 1)],
                                            b.code[j][tt >> 1 & (kCW - 1)][2 * (tt & 1) + 1], sv,
                                            z * sv)
                      : dequant_word_bf16(b.code[j][0][tt], sv, (128.0f + z) * sv);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const u32x4 aop = *reinterpret_cast<const u32x4 *>(abuf + i * 16 * kLdsStride + 32 * tt);
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma16_bf16(aop, bop[j], acc[i][j]);
        }
      } else {
        half8 bop[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)b.zp[j]);
          const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)b.sc[j]);
          const _Float16 blo = (_Float16)1024.0f + z, bhi = (_Float16)64.0f + z;
          const half2v bias_lo = {blo, blo}, bias_hi = {bhi, bhi}, scale = {sv, sv};
          bop[j] = W8 ? dequant_words8(b.code[j][tt >> 1 & (kCW - 1)][2 * (tt & 1)],
                                       b.code[j][tt >> 1 & (kCW - 1)][2 * (tt & 1) + 1], bias_lo,
                                       scale)
                      : dequant_word(b.code[j][0][tt], bias_lo, bias_hi, scale);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const half8 aop = *reinterpret_cast<const half8 *>(abuf + i * 16 * kLdsStride + 32 * tt);
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(aop, bop[j], acc[i][j]);
        }
      }
    }
    // let the scheduler interleave the MFMAs with the dequantization and LDS
    // reads around them (LLVM's single-wave small-GEMM strategy; measured
    // best of the available strategies and of hand-placed group barriers)
    __builtin_amdgcn_iglp_opt(1);
  };

  // ---- fp16 outliers.  Lane (c, r) holds outputs of rows n_j = n0 + (wn TN +
  // j) 16 + r, j = 0..3, and keeps the walk over the kept weights of row n_c
  // (columns increasing) with the next two of them in registers; each step
  // the four lanes of a row share their entries by shuffles.  An entry whose
  // column lies in group g is applied in step g, from the staged X * s of that
  // group (divided by s, so the term is X[m][col] * val up to the rounding of
  // X * s), to the 16 rows m the lane holds.  Entries of groups outside this
  // block's K range belong to another split.  Slots refilled in a step are
  // first read in the next one (after its wait for all loads), so no step
  // waits on them; a third entry of one row in one group arrives a step late
  // and is then applied from global X.
  static_assert(TN == 4, "one row walk per lane of a row's four lanes");
  constexpr int kNone = 0x7fffffff;
  int oe = 0, oend = 0, ocol0 = kNone, ocol1 = kNone;
  float oval0 = 0.f, oval1 = 0.f;
  auto refill = [&](int &col, float &val) {
    col = kNone;
    if (oe < oend) {
      col = P.ocol[oe];
      val = (float)P.oval[oe];
      ++oe;
    }
  };
  auto outlier_start = [&]() {
    const int n = n0 + (wn * TN + c) * 16 + r;
    int lo = n < N ? P.orp[n] : 0, hi = n < N ? P.orp[n + 1] : 0;
    oend = hi;
    // first entry at or after this K range (binary search; nothing to skip
    // for the first range)
    if (gb > 0) {
      const int kb = gb * kGroup;
      while (__any(lo < hi)) {
        if (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (P.ocol[mid] < kb)
            lo = mid + 1;
          else
            hi = mid;
        }
      }
    }
    oe = lo;
    refill(ocol0, oval0);
    refill(ocol1, oval1);
  };
  // entry (col, val) of row j on the lane's 16 rows: from LDS for group g
  // (buffer buf), or from global X when its group has already passed
  auto apply_entry = [&](int j, int col, float val, int g, int buf) {
    const int kk = col - g * kGroup;
    if (kk >= 0) {
      // the staged X * s times val / s: the hardware reciprocal (about 1 ulp of
      // fp32, far below the fp16 rounding of X * s) instead of a full division
      const float vs = has_s ? val * __builtin_amdgcn_rcpf((float)Ss[OUT ? buf : 0][kk]) : val;
      const _Float16 *xb = As[buf] + (wm * TM * 16 + 4 * c) * kLdsStride + kk;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const _Float16 xv = xb[(i * 16 + v) * kLdsStride];
          acc[i][j][v] += (BF ? bf16_to_f32(__builtin_bit_cast(uint16_t, xv)) : (float)xv) * vs;
        }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = min(m0 + (wm * TM + i) * 16 + 4 * c + v, M - 1);
          const _Float16 xv = X[(size_t)m * K + col];
          acc[i][j][v] += (BF ? bf16_to_f32(__builtin_bit_cast(uint16_t, xv)) : (float)xv) * val;
        }
    }
  };
  auto apply_outliers = [&](int g, int buf) {
    const int khi = (g + 1) * kGroup;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int src = 16 * j + r;  // the lane walking row n_j
      const int c0 = __shfl(ocol0, src), c1 = __shfl(ocol1, src);
      const float v0 = __shfl(oval0, src), v1 = __shfl(oval1, src);
      if (c0 < khi) apply_entry(j, c0, v0, g, buf);
      if (c0 < khi && c1 < khi) apply_entry(j, c1, v1, g, buf);
    }
    // advance this lane's own walk past what was applied
    const bool take0 = ocol0 < khi, take1 = take0 && ocol1 < khi;
    if (take1) {
      refill(ocol0, oval0);
      refill(ocol1, oval1);
    } else if (take0) {
      ocol0 = ocol1;
      oval0 = oval1;
      refill(ocol1, oval1);
    }
  };

  // One group per step.  The group's codes and metadata were issued a step
  // ago: wait for them (the only loads in flight) and take the codes into
  // registers; then issue the next group's X and weight loads, run this
  // group's MFMAs, and write the next X * s to the other LDS buffer.  Steps
  // alternate LDS buffers and metadata register sets, two steps per
  // iteration, so nothing is copied between them.
  auto take_codes = [&](BRegs &b, int buf) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int h = 0; h < kCW; ++h)
        b.code[j][h] = *reinterpret_cast<const u32x4 *>(
            bslot(buf) + ((wave * TN + j) * kCW + h) * kTileBytes + lane * 16);
  };
  auto step = [&](int g, BRegs &cur, BRegs &nxt, int buf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the DMA writes are not seen by the compiler
    take_codes(cur, buf);
    // one INT8 buffer: the reads must land before the next DMA overwrites it
    if (W8) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const bool more = g + 1 < ge;
    if (more) {
      load_a(g + 1);
      load_codes(g + 1, buf ^ 1);
      load_meta(g + 1, nxt);
    }
    compute(cur, buf);
    if (has_out) apply_outliers(g, buf);
    if (more) store_a(buf ^ 1);
    lds_barrier();
  };
  // Two groups of codes in flight (INT4 codes, no outliers), with the same
  // two code buffers.  A step's codes are taken into registers at the end of
  // the step before; once they have landed the buffer is free, and the step
  // refills it with group g + 2's codes, issued last, after group g + 1's X
  // and metadata.  All three, and the store of the next X * s, happen
  // unconditionally (past the range they re-read the last group into
  // registers and buffers nobody reads again), so a step has no branches (at
  // a join the compiler forgets which buffer a DMA in flight writes), every
  // step issues the same loads, and the wait before taking the next group's
  // codes is always "all but the newest kCodeLoads loads" (this step's DMA).
  constexpr bool kDepth2 = !OUT && !W8;
  constexpr int kCodeLoads = TN * kCW;  // vector memory loads of one load_codes
  static_assert(!kDepth2 || kCodeLoads == 4, "the two-deep wait below counts 4 loads");
  auto step2 = [&](int g, BRegs &cur, BRegs &nxt, int buf) {
    const int gn = min(g + 1, ge - 1);
    load_a(gn);
    load_meta(gn, nxt);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this buffer's code reads have landed
    load_codes(min(g + 2, ge - 1), buf);
    // keep the DMA here, ahead of the MFMAs (the scheduler would sink it)
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, buf);
    store_a(buf ^ 1);  // (past the range: the last group again, never read)
    // group g + 1's codes (DMA'd a step earlier): s_waitcnt vmcnt(4), expcnt
    // and lgkmcnt at their maxima (7, 15), through the builtin so that the
    // compiler's own wait counting knows it
    __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8));
    take_codes(nxt, buf ^ 1);
    lds_barrier();
  };
  load_a(gb);
  load_meta(gb, b0);
  load_codes(gb, 0);
  if (kDepth2) load_codes(min(gb + 1, ge - 1), 1);  // issued last: the first wait leaves it in flight
  if (has_out) outlier_start();  // its waits overlap the first group's loads
  store_a(0);
  if (kDepth2) {
    __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8));
    take_codes(b0, 0);
  }
  lds_barrier();
  if (kDepth2) {
    // both steps unconditional, so the register sets keep their roles across
    // the back edge (nothing is copied, so nothing waits for loads in flight)
    int g = gb;
    for (; g + 1 < ge; g += 2) {
      step2(g, b0, b1, 0);
      step2(g + 1, b1, b0, 1);
    }
    if (g < ge) step2(g, b0, b1, 0);
    // the last steps' loads re-read the range's last group into registers
    // and LDS nothing reads; they must land before the workgroup's LDS is
    // released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    for (int g = gb; g < ge; g += 2) {
      step(g, b0, b1, 0);
      if (g + 1 < ge) step(g + 1, b1, b0, 1);
    }
  }
  if (has_out) {
    // late entries of the last group (a third or later in one row), from global X
    const int kend = ge * kGroup;
    while (__any(ocol0 < kend)) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int src = 16 * j + r;
        const int c0 = __shfl(ocol0, src);
        const float v0 = __shfl(oval0, src);
        if (c0 < kend) apply_entry(j, c0, v0, ge, 0);
      }
      if (ocol0 < kend) {
        ocol0 = ocol1;
        oval0 = oval1;
        refill(ocol1, oval1);
      }
    }
  }

  // lane holds D[4c + v][r] of each 16x16 sub-block: the output, or this
  // split's fp32 partial
  float *part = P.split > 1 ? P.part + (size_t)sp * M * N : nullptr;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + (wn * TN + j) * 16 + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + (wm * TM + i) * 16 + 4 * c + v;
        if (m < M && n < N) {
          if (part)
            part[(size_t)m * N + n] = acc[i][j][v];
          else if (BF)
            reinterpret_cast<uint16_t *>(P.Y)[(size_t)m * N + n] = f32_to_bf16(acc[i][j][v]);
          else
            P.Y[(size_t)m * N + n] = (_Float16)acc[i][j][v];
        }
      }
    }
  }
}

// The tiled GEMM for INT4 codes without outliers (fp16 or bf16 activations,
// BF) and for INT8 codes with fp16 activations (W8), with TM = 8 (128 rows of
// X per wave) for large M.  The dequantization of a weight
// costs the same VALU work whatever the rows it feeds, so a wave tile of 128
// rows halves it per MFMA against 64 rows; the registers for that come from
// moving X * s off the register path:
//   * X * s (rounded to fp16, or bf16, once: prescaled into the workspace by
//     prescale_f16_kernel when s is given, else X itself) goes straight from
//     memory into LDS with DMA loads (buffer_load ... lds), one group (128
//     columns) per stage, double-buffered, one barrier per stage.  A row's 16
//     chunks of 16 bytes are stored XOR-swizzled (chunk c of row m at c ^ (m %
//     16)), so the MFMA A-operand reads of 16 rows hit distinct banks without
//     padding; each DMA lane fetches the chunk that belongs in its slot;
//   * the wave's code tiles (16 bytes per lane per tile, 32 for INT8 codes:
//     its MFMA B operands) and their scales and zero points are loaded into
//     registers one group ahead, in two register sets that alternate.
// The bf16 and INT8 instances cost more registers; their 128-row tiles fit
// in 256 VGPRs because each pair of bf16 weights comes from one packed
// conversion (pack_bf16x2) and INT8 codes keep a row block's scale and zero
// point in one register (otherwise both spilled).
// Blocks are BM x BN (BM = 16 TM, BN = 64 TN), four waves of BM x 16 TN per
// K slice; K is split across workgroups the same way as in tiled_kernel.
// Batched decode (M up to 64) takes TN = 2 (and TM = 2, 3 or 4, as few rows
// as cover M): twice the blocks of TN = 4, so fewer K splits (whose fp32
// partials cost HBM traffic) are needed to fill the GPU, and half the
// accumulators.  Its blocks have one K slice of four waves
// or KS = 2: each slice walks every other group of the workgroup's K range
// into its own X * s stages, and the two sums are added through LDS at the end
// (slice 0's plus slice 1's, a fixed order).  Two slices double the waves per
// block without fp32 partials in memory: the Qwen2-7B M = 64 layer then splits
// only down across workgroups and took 52-56 us against 61, while layers with
// more blocks than slots (70B at M = 64) keep one slice.  (KS = 2 at TM = 8
// needs more than 256 VGPRs.)
template <int TM, int TN, int KS, bool BF = false, bool W8 = false>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(TN == 2 ? 4 : 2, TN == 2 ? 4 : 2))) void tiled_dma_kernel(
    TiledSet ts) {
  constexpr int WN = 4;
  constexpr int kCW = W8 ? 2 : 1;  // 16-byte code pieces per lane per tile
  static_assert(!(BF && W8), "INT8 codes: fp16 activations");
  constexpr int BM = TM * 16, BN = WN * TN * 16;
  constexpr int kRowChunks = kGroup / 8;            // 16-byte chunks per row per group
  constexpr int kDma = BM * kRowChunks / (4 * 64);  // DMA loads per wave per group
  static_assert(kDma * 4 * 64 == BM * kRowChunks, "a stage is whole DMA loads");
  static_assert(KS == 1 || BM * BN * 4 <= KS * 2 * BM * kGroup * 2, "the slices' sums fit the X stages");
  __shared__ __attribute__((aligned(16))) _Float16 As[KS][2][BM * kGroup];

  const int block = (int)blockIdx.x;
  const TiledProblem P = find_tiled<false>(ts, block);
  const int M = P.M, N = P.N, K = P.K;
  const int tid = threadIdx.x, lane = tid & 63, wv = uniform_int(tid >> 6);
  const int ks = KS == 1 ? 0 : wv >> 2, wave = KS == 1 ? wv : wv & 3;  // K slice; the wave's column
  const int c = lane >> 4, r = lane & 15;
  // Workgroups go to the eight XCDs (each with its own L2) round robin,
  // workgroup i to XCD i mod 8.  A split launch is renumbered so that each XCD
  // takes one contiguous run of (split, block) pairs: neighbouring blocks of
  // one K range, which share X rows and code panels in that L2 (measured 8%
  // faster on the 70B k and v projections, split 4; unsplit launches gain
  // nothing and keep the plain order).  The first 8 * (L / 8) workgroups are
  // permuted among themselves, the rest keep their numbers.
  const int local0 = block - P.block0;
  const int L = P.split * P.tiles, q8 = L >> 3;
  const int local =
      (P.split > 1 && local0 < 8 * q8) ? (local0 & 7) * q8 + (local0 >> 3) : local0;
  const int sp = local / P.tiles, t = local - sp * P.tiles;
  const int mt = t / P.tiles_n;
  const int n0 = (t - mt * P.tiles_n) * BN, m0 = mt * BM;
  const int G = K / kGroup, NB = N / kTileRows;
  const int gb = (int)((long long)G * sp / P.split), ge = (int)((long long)G * (sp + 1) / P.split);
  // K slice ks of the workgroup takes groups gb + ks, gb + ks + KS, ...: every
  // slice runs the same number of steps (and barriers); past ge a step loads
  // the range's last group again and skips its MFMAs
  const int nsteps = (ge - gb + KS - 1) / KS;
  auto group_at = [&](int i) { return min(gb + ks + i * KS, ge - 1); };

  // X * s: wave load u fills LDS chunks p = (wave * kDma + u) * 64 + lane of a
  // stage; chunk p is row p / 16, physical chunk p % 16, holding logical chunk
  // (p % 16) ^ (row % 16) of that row.  Rows past M read row M - 1 (rows of A
  // only reach the same rows of D, which are not stored).  M * K * 2 < 2^31
  // (checked by the launcher), so offsets fit the buffer resource.
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void *)P.xs, (short)0, M * K * 2, kRsrcWord3);
  int xoff[kDma];
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int p = (wave * kDma + u) * 64 + lane;
    const int row = p / kRowChunks, lc = (p % kRowChunks) ^ (row % 16);
    xoff[u] = (min(m0 + row, M - 1) * K + 8 * lc) * 2;
  }
  auto load_x = [&](int g, int buf) {
#pragma unroll
    for (int u = 0; u < kDma; ++u)
    {
      // (an array element passed straight to the builtin keeps the kernel from
      // being instantiated in the host compilation)
      const int vo = xoff[u];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (__attribute__((address_space(3))) void *)(&As[ks][buf][(wave * kDma + u) * 64 * 8]), 16,
          vo, g * kGroup * 2, 0, 0);
    }
  };

  // the wave's TN row blocks; blocks past N re-read the last one (never stored)
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.Wq, (short)0, (int)min((size_t)0x7fffffff, (size_t)N * K / 2 * kCW), kRsrcWord3);
  const int Gq = meta_groups(G) / kMetaQuad;
  const size_t meta_bytes = (size_t)N * Gq * kMetaQuad * 2;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.scales, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.zeros, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const int rb0 = n0 / kTileRows + wave * TN;
  const int tile_stride = NB * kTileBytes * kCW, meta_stride = NB * kTileRows * kMetaQuad * 2;
  // raw fp16 bits of each row block's scale and zero point: INT8 codes keep
  // both in one register (x: scale, y: zero point), which leaves the 128-row
  // instance within 256 VGPRs
  struct BStagePair {
    u32x4 code[TN][kCW];
    uint32_t sc[TN], zp[TN];
  };
  struct BStagePacked {
    u32x4 code[TN][kCW];
    u16x2 sz[TN];
  };
  using BStage = std::conditional_t<W8, BStagePacked, BStagePair>;
  auto load_b = [&](int g, BStage &b) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int rb = min(rb0 + j, NB - 1);
#pragma unroll
      for (int h = 0; h < kCW; ++h)
        b.code[j][h] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, (rb * 64 + lane) * 16 * kCW + 16 * h,
                                                         g * tile_stride, 0));
      const int mo = (rb * kTileRows + r) * kMetaQuad * 2;
      const int qo = (g / kMetaQuad) * meta_stride + (g % kMetaQuad) * 2;
      if constexpr (W8) {
        b.sz[j][0] = __builtin_amdgcn_raw_buffer_load_b16(srs, mo, qo, 0);
        b.sz[j][1] = __builtin_amdgcn_raw_buffer_load_b16(zrs, mo, qo, 0);
      } else {
        b.sc[j] = __builtin_amdgcn_raw_buffer_load_b16(srs, mo, qo, 0);
        b.zp[j] = __builtin_amdgcn_raw_buffer_load_b16(zrs, mo, qo, 0);
      }
    }
  };

  float4v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  // the four k steps of a group: this wave's B operands dequantized once per
  // k step, then TM x TN MFMAs with A read from LDS buffer `buf`
  auto compute = [&](const BStage &b, int buf) {
    half2v bias_lo[TN], bias_hi[TN], scale[TN];
    float fsc[TN], fzb[TN];  // bf16: the fp32 scale and (128 + z) * scale
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      uint16_t zr, sr;
      if constexpr (W8) {
        sr = b.sz[j][0];
        zr = b.sz[j][1];
      } else {
        sr = (uint16_t)b.sc[j];
        zr = (uint16_t)b.zp[j];
      }
      const _Float16 z = __builtin_bit_cast(_Float16, zr);
      const _Float16 sv = __builtin_bit_cast(_Float16, sr);
      if (BF) {
        fsc[j] = (float)sv;
        fzb[j] = (128.0f + (float)z) * fsc[j];
      } else {
        const _Float16 blo = (_Float16)1024.0f + z, bhi = (_Float16)64.0f + z;
        const half2v bl = {blo, blo}, bh = {bhi, bhi}, sc = {sv, sv};
        bias_lo[j] = bl;
        bias_hi[j] = bh;
        scale[j] = sc;
      }
    }
    // a B operand: eight dequantized weights, fp16 or bf16 bits
    auto dequant = [&](int j, int t) -> u32x4 {
      if constexpr (BF)
        return dequant_word_bf16(b.code[j][0][t], fsc[j], fzb[j]);
      else if constexpr (W8)  // k step t: the lane's code words 2t and 2t + 1
        return __builtin_bit_cast(u32x4, dequant_words8(b.code[j][t >> 1][2 * (t & 1)],
                                                        b.code[j][t >> 1][2 * (t & 1) + 1],
                                                        bias_lo[j], scale[j]));
      else
        return __builtin_bit_cast(u32x4, dequant_word(b.code[j][0][t], bias_lo[j], bias_hi[j], scale[j]));
    };
    const _Float16 *abuf = As[ks][buf];
    // software pipeline: k step tt + 1's B operands are dequantized while k
    // step tt's MFMAs run, interleaved by the scheduler (one LDS read, TN
    // MFMAs and about seven VALU ops at a time; twice that for bf16, whose
    // dequantization costs twice the ops)
    u32x4 bop[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bop[j] = dequant(j, 0);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      u32x4 bnx[TN];
      if (tt < 3) {
#pragma unroll
        for (int j = 0; j < TN; ++j) bnx[j] = dequant(j, tt + 1);
      }
      const int pc = (4 * tt + c) ^ r;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const u32x4 aop = *reinterpret_cast<const u32x4 *>(abuf + (16 * i + r) * kGroup + 8 * pc);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = BF ? mfma16_bf16(aop, bop[j], acc[i][j])
                         : mfma16(__builtin_bit_cast(half8, aop), __builtin_bit_cast(half8, bop[j]),
                                  acc[i][j]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);  // TN MFMAs
        if (tt < 3) __builtin_amdgcn_sched_group_barrier(0x002, BF ? 14 : 7, 0);  // VALU
      }
      if (tt < 3) {
#pragma unroll
        for (int j = 0; j < TN; ++j) bop[j] = bnx[j];
      }
    }
  };

  // One group per step: wait until this group's DMA and code loads (issued a
  // step ago) have landed and every wave is past the previous step (so the
  // other buffer is free), then issue the next group's loads, which land
  // while this group's MFMAs run.  Past the range they re-read the last group
  // (into a buffer and registers nobody reads).  Buffers and register sets
  // alternate with the loop unrolled by two, so nothing is copied.
  BStage b0, b1;
  if constexpr (KS == 1) {
    auto step = [&](int g, BStage &cur, BStage &nxt, int buf) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      const int gn = min(g + 1, ge - 1);
      load_x(gn, buf ^ 1);
      load_b(gn, nxt);
      compute(cur, buf);
    };
    load_x(gb, 0);
    load_b(gb, b0);
    for (int g = gb; g < ge; g += 2) {
      step(g, b0, b1, 0);
      if (g + 1 < ge) step(g + 1, b1, b0, 1);
    }
  } else {
    auto step = [&](int i, BStage &cur, BStage &nxt, int buf) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      const int gn = group_at(min(i + 1, nsteps - 1));
      load_x(gn, buf ^ 1);
      load_b(gn, nxt);
      if (gb + ks + i * KS < ge) compute(cur, buf);
    };
    load_x(group_at(0), 0);
    load_b(group_at(0), b0);
    for (int i = 0; i < nsteps; i += 2) {
      step(i, b0, b1, 0);
      if (i + 1 < nsteps) step(i + 1, b1, b0, 1);
    }
  }
  // the last step's DMA must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (KS == 2) {
    // slice 1 hands its sums to slice 0 through the X stages' LDS, and slice 0
    // adds them to its own (a fixed order)
    float *red = reinterpret_cast<float *>(&As[0][0][0]);
    __syncthreads();  // every wave is done with the X stages
    if (ks == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          *reinterpret_cast<float4v *>(&red[((i * TN + j) * 4 + wave) * 256 + lane * 4]) = acc[i][j];
    }
    __syncthreads();
    if (ks == 1) return;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] += *reinterpret_cast<const float4v *>(&red[((i * TN + j) * 4 + wave) * 256 + lane * 4]);
  }

  // lane holds D[4c + v][r] of each 16x16 sub-block: the output, or this
  // split's fp32 partial
  if constexpr (TM <= 4) {
    // Small tiles (the epilogue is a larger share of the work): buffer
    // stores through a resource that starts at the block's first row and ends
    // at row M, so rows past M are dropped by the hardware's range check and
    // no element needs a branch or a 64-bit address (offsets within a block
    // stay below 2^31); a 16-column block lies inside N or outside it as a
    // whole (N is a multiple of 16), a uniform test.
    const bool split = P.split > 1;
    const int esize = split ? 4 : 2;
    char *out = split ? reinterpret_cast<char *>(P.part + (size_t)sp * M * N + (size_t)m0 * N)
                      : reinterpret_cast<char *>(P.Y) + (size_t)m0 * N * 2;
    const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
        out, (short)0, (int)min((size_t)(M - m0) * N * esize, (size_t)0x7fffffff), kRsrcWord3);
    auto store_all = [&](auto &&store) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int nb = n0 + (wave * TN + j) * 16;
        if (nb >= N) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) store((i * 16 + 4 * c + v) * N + nb + r, acc[i][j][v]);
      }
    };
    if (split)
      store_all([&](int e, float a) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, a), yrs, e * 4, 0, 0);
      });
    else
      store_all([&](int e, float a) {
        __builtin_amdgcn_raw_buffer_store_b16(
            BF ? f32_to_bf16(a) : __builtin_bit_cast(uint16_t, (_Float16)a), yrs, e * 2, 0, 0);
      });
    return;
  }
  float *part = P.split > 1 ? P.part + (size_t)sp * M * N : nullptr;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + (wave * TN + j) * 16 + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + i * 16 + 4 * c + v;
        if (m < M && n < N) {
          if (part)
            part[(size_t)m * N + n] = acc[i][j][v];
          else if (BF)
            reinterpret_cast<uint16_t *>(P.Y)[(size_t)m * N + n] = f32_to_bf16(acc[i][j][v]);
          else
            P.Y[(size_t)m * N + n] = (_Float16)acc[i][j][v];
        }
      }
    }
  }
}

// fp16(X * s) of the problems of a launch that have an s, rounded once like
// the kernels' own staging, in one launch: one thread per 8 columns, the
// problems' workgroups concatenated.
struct PrescaleItem {
  const _Float16 *X, *s;
  _Float16 *out;
  int K;
  int block0;  // first workgroup of this problem
  int bf16;    // X and out are bf16: bf16(X * s), the product exact in fp32
  long long n8;
};
struct PrescaleSet {
  PrescaleItem p[kMaxTiled];
  int count;
};

__global__ __launch_bounds__(256) void prescale_f16_kernel(PrescaleSet ps) {
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxTiled; ++i)
    if (i < ps.count && (int)blockIdx.x >= ps.p[i].block0) pi = i;
  const _Float16 *X = uniform_ptr(ps.p[pi].X), *sv = uniform_ptr(ps.p[pi].s);
  _Float16 *out = uniform_ptr(ps.p[pi].out);
  const int K = uniform_int(ps.p[pi].K), block0 = uniform_int(ps.p[pi].block0);
  const long long i = (long long)((int)blockIdx.x - block0) * 256 + threadIdx.x;
  if (i >= ps.p[pi].n8) return;
  const long long e = i * 8;
  const int k = (int)(e % K);
  if (uniform_int(ps.p[pi].bf16)) {
    const u32x4 xw = *reinterpret_cast<const u32x4 *>(X + e);
    const half8 s8 = load_half8(sv + k);
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bf16_to_f32((uint16_t)xw[q]) * (float)s8[2 * q];
      const float hi = bf16_to_f32((uint16_t)(xw[q] >> 16)) * (float)s8[2 * q + 1];
      v[q] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4 *>(out + e) = v;
  } else {
    *reinterpret_cast<half8 *>(out + e) = load_half8(X + e) * load_half8(sv + k);
  }
}

// Y = fp16(sum of the split partials, in split order) for the problems with
// split > 1; four outputs per thread.
constexpr int kReduceThreads = 256;

__global__ __launch_bounds__(kReduceThreads) void split_reduce_kernel(TiledSet ts) {
  const TiledProblem P = find_tiled<true>(ts, (int)blockIdx.x);
  const long long quads = (long long)P.M * P.N / 4;
  const long long i = (long long)((int)blockIdx.x - P.rblock0) * kReduceThreads + threadIdx.x;
  if (i >= quads) return;
  const float4v *src = reinterpret_cast<const float4v *>(P.part) + i;
  float4v acc = src[0];
  for (int k = 1; k < P.split; ++k) acc += src[(size_t)k * quads];
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
  if (P.bf16) {
    const u16x4 out = {f32_to_bf16(acc[0]), f32_to_bf16(acc[1]), f32_to_bf16(acc[2]),
                       f32_to_bf16(acc[3])};
    reinterpret_cast<u16x4 *>(P.Y)[i] = out;
  } else {
    const half4 out = {(_Float16)acc[0], (_Float16)acc[1], (_Float16)acc[2], (_Float16)acc[3]};
    reinterpret_cast<half4 *>(P.Y)[i] = out;
  }
}

// 64 x 256 blocks of 4 waves (64 x 64 each), two workgroups per CU: the
// fastest of the measured shapes at every M of the workloads.
template <int WM_, int WN_, int TM_, int TN_>
struct Shape {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
};
using TileShape = Shape<1, 4, 4, 4>;
constexpr int kWM = TileShape::WM, kWN = TileShape::WN, kTM = TileShape::TM, kTN = TileShape::TN;
constexpr int kBM = kWM * kTM * 16, kBN = kWN * kTN * 16;
// CUs x resident workgroups per CU (two waves per SIMD, four SIMDs)
constexpr long long kBlockSlots = 256 * 8 / (kWM * kWN);
constexpr int kMinSplitGroups = 8;          // splits about this many groups long at the shortest
constexpr int kMaxSplit = 16;
// Cost model of one launch (measured on the 70B prefill and Qwen2-7B batched
// shapes): with every slot busy, a workgroup takes about kStageUs per group
// plus kBlockStages groups' worth of prologue, epilogue and tail; workgroups
// run in rounds of kBlockSlots; split partials cost their fp32 writes and the
// reduction's reads at about kReduceBytesPerUs.
constexpr double kStageUs = 2.3;
constexpr double kBlockStages = 2.0;
constexpr double kReduceBytesPerUs = 4.0e6;

int tiles_of(const GemmDesc &d, int bm = kBM, int bn = kBN) {
  return ((d.N + bn - 1) / bn) * ((d.M + bm - 1) / bm);
}

// tiled_dma_kernel takes fp16 or bf16 activations with INT4 codes, or fp16
// activations with INT8 codes, without outliers, whose X (M x K, 2 bytes
// each) a buffer resource can cover; it serves launches whose largest M
// exceeds 16.
bool dma_capable(const GemmDesc &d) {
  return !(d.w8 && d.bf16) && !d.o_row_ptr && (size_t)d.M * d.K * 2 < ((size_t)1 << 31);
}
constexpr int kDmaMinM = 17;

// Geometry of the tiled_dma_kernel instances: TM = 8, TN = 4 (128 x 256
// blocks of four waves, two workgroups per CU) when the launch's largest M
// exceeds 96, TM = 6, TN = 4 (96 x 256) from 65 to 96 rows, else TN = 2 and
// the fewest 16-row tiles that cover M (TM = 2, 3 or 4: blocks of 32, 48 or
// 64 x 128) with one K slice (four waves) or two (eight waves), whichever the
// launch model below prefers; bf16 activations and INT8 codes take the same
// tiles (the 70B prefill layer with bf16 activations ran at 898-918 TFLOP/s
// with 96-row tiles and 1090-1102 with 128-row ones; with INT8 codes at
// 941-944 and 1073-1076).  Below 64 rows the padded rows'
// MFMAs and A reads are not free: the Qwen2-7B layer at M = 17 took 43 us
// with 64-row tiles and 34 us with 32-row ones (bf16: 54 and 47 us; INT8
// codes: 52 and 49 us), at M = 33 45 and 42 us with 64- and 48-row ones.
// Covering 64 rows with two 32-row tiles instead (each weight read twice) was
// slower: 62 against 50 us.  At M = 65 96-row tiles took 62 against 69 us
// with 128-row ones.
struct DmaShape {
  int tm, tn;
  int bm() const { return 16 * tm; }
  int bn() const { return 64 * tn; }
};
DmaShape dma_shape(int tm) { return tm >= 6 ? DmaShape{tm, 4} : DmaShape{tm, 2}; }
long long dma_slots(int tm, int ks) { return tm >= 6 || ks == 2 ? 512 : 1024; }

// 0 when the launch cannot take tiled_dma_kernel, else its TM: the fewest
// 16-row tiles that cover the largest M among 2, 3, 4, 6 and 8 (32 to 128
// rows)
int dma_tm(const GemmDesc *d, int count) {
  int mmax = 0;
  for (int i = 0; i < count; ++i) {
    if (!dma_capable(d[i])) return 0;
    mmax = std::max(mmax, d[i].M);
  }
  if (mmax < kDmaMinM) return 0;
  return mmax > 96 ? 8 : mmax > 64 ? 6 : mmax > 48 ? 4 : mmax > 32 ? 3 : 2;
}
bool dma_launch(const GemmDesc *d, int count) { return dma_tm(d, count) != 0; }

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// workspace bytes of the prescaled X * s of the problems that have an s
size_t prescale_need(const GemmDesc *d, int count) {
  size_t n = 0;
  for (int i = 0; i < count; ++i)
    if (d[i].s) n += align256((size_t)d[i].M * d[i].K * 2);
  return n;
}

size_t part_bytes(const GemmDesc &d, int split) {
  return split > 1 ? ((size_t)split * d.M * d.N * sizeof(float) + 255) / 256 * 256 : 0;
}

// Modelled time of one launch with the given splits: ceil(workgroups /
// slots) rounds, each as long as the longest range (in steps: a workgroup of
// ks K slices takes ceil(range / ks) of them) plus a fixed cost, plus the
// reduction of the partials.
double launch_model(const GemmDesc *d, int count, const int *s, int bm, int bn, long long slots,
                    int ks) {
  long long blocks = 0;
  int longest = 0;
  double reduce_bytes = 0.0;
  for (int i = 0; i < count; ++i) {
    const int G = d[i].K / kGroup;
    blocks += (long long)tiles_of(d[i], bm, bn) * s[i];
    longest = std::max(longest, ((G + s[i] - 1) / s[i] + ks - 1) / ks);
    if (s[i] > 1) reduce_bytes += (double)(4 * s[i] + 2) * d[i].M * d[i].N;
  }
  const long long rounds = (blocks + slots - 1) / slots;
  return (double)rounds * (longest + kBlockStages) * kStageUs + reduce_bytes / kReduceBytesPerUs;
}

// K splits of each problem of one launch.  Every problem's groups are cut
// into ranges of at most T groups; T is the one whose modelled launch time is
// least.  Counting whole rounds matters: a launch a few workgroups past a
// multiple of the slots takes a whole extra round.  Ties keep the longer
// ranges (fewer partials).  Returns the modelled time.
double choose_splits(const GemmDesc *d, int count, int *split, int bm = kBM, int bn = kBN,
                     long long slots = kBlockSlots, int ks = 1) {
  // Only range lengths ceil(G / n) for some problem's G and n <= kMaxSplit give
  // distinct split vectors; try those, longest first.
  int cand[kMaxTiled * kMaxSplit];
  int nc = 0;
  for (int i = 0; i < count; ++i) {
    const int G = d[i].K / kGroup;
    for (int n = 1; n <= kMaxSplit && n <= G; ++n) cand[nc++] = (G + n - 1) / n;
  }
  std::sort(cand, cand + nc, [](int a, int b) { return a > b; });
  nc = (int)(std::unique(cand, cand + nc) - cand);
  double best = 0.0;
  for (int ci = 0; ci < nc; ++ci) {
    const int T = cand[ci];
    int s[kMaxTiled];
    for (int i = 0; i < count; ++i) {
      const int G = d[i].K / kGroup;
      const int cap = std::min(std::min(kMaxSplit, G), (G + kMinSplitGroups - 1) / kMinSplitGroups);
      s[i] = std::max(1, std::min(cap, (G + T - 1) / T));
    }
    const double t = launch_model(d, count, s, bm, bn, slots, ks);
    if (ci == 0 || t < best) {
      best = t;
      for (int i = 0; i < count; ++i) split[i] = s[i];
    }
  }
  return best;
}

// The DMA kernel's plan for a launch of TM = tm: splits per problem (all 1
// when `unsplit`: no room for partials) and K slices per block; returns the
// slices.  With TM = 4 both slice counts are modelled and the faster kept
// (ties: two slices, no more partials than one).
int dma_plan(const GemmDesc *d, int count, int tm, bool unsplit, int *split) {
  const DmaShape ds = dma_shape(tm);
  const int kss[2] = {2, 1};
  int best_ks = 1;
  double best = 0.0;
  for (int v = 0; v < (tm >= 6 ? 1 : 2); ++v) {
    const int ks = tm >= 6 ? 1 : kss[v];
    int s[kMaxTiled];
    double t;
    if (unsplit) {
      for (int i = 0; i < count; ++i) s[i] = 1;
      t = launch_model(d, count, s, ds.bm(), ds.bn(), dma_slots(tm, ks), ks);
    } else {
      t = choose_splits(d, count, s, ds.bm(), ds.bn(), dma_slots(tm, ks), ks);
    }
    if (v == 0 || t < best) {
      best = t;
      best_ks = ks;
      for (int i = 0; i < count; ++i) split[i] = s[i];
    }
  }
  return best_ks;
}

// The tiled_dma_kernel instance of a DMA plan (dma_tm's TM, dma_plan's K
// slices) for one activation type and code width; any other shape is an
// error, never a launch with a grid planned for another tile.
template <bool BF, bool W8>
hipError_t launch_dma(int tm, int ks, dim3 grid, hipStream_t stream, const TiledSet &ts) {
  if (tm == 8 && ks == 1)
    hipLaunchKernelGGL((tiled_dma_kernel<8, 4, 1, BF, W8>), grid, dim3(256), 0, stream, ts);
  else if (tm == 6 && ks == 1)
    hipLaunchKernelGGL((tiled_dma_kernel<6, 4, 1, BF, W8>), grid, dim3(256), 0, stream, ts);
  else if (tm == 4 && ks == 2)
    hipLaunchKernelGGL((tiled_dma_kernel<4, 2, 2, BF, W8>), grid, dim3(512), 0, stream, ts);
  else if (tm == 4 && ks == 1)
    hipLaunchKernelGGL((tiled_dma_kernel<4, 2, 1, BF, W8>), grid, dim3(256), 0, stream, ts);
  else if (tm == 3 && ks == 2)
    hipLaunchKernelGGL((tiled_dma_kernel<3, 2, 2, BF, W8>), grid, dim3(512), 0, stream, ts);
  else if (tm == 3 && ks == 1)
    hipLaunchKernelGGL((tiled_dma_kernel<3, 2, 1, BF, W8>), grid, dim3(256), 0, stream, ts);
  else if (tm == 2 && ks == 2)
    hipLaunchKernelGGL((tiled_dma_kernel<2, 2, 2, BF, W8>), grid, dim3(512), 0, stream, ts);
  else if (tm == 2 && ks == 1)
    hipLaunchKernelGGL((tiled_dma_kernel<2, 2, 1, BF, W8>), grid, dim3(256), 0, stream, ts);
  else
    return hipErrorInvalidValue;
  return hipSuccess;
}

}  // namespace

size_t tiled_workspace_bytes(const GemmDesc *d, int count) {
  if (count < 1 || count > kMaxTiled) return 0;
  const int tm = dma_tm(d, count);
  const bool dma = tm != 0;
  int split[kMaxTiled];
  if (dma)
    dma_plan(d, count, tm, false, split);
  else
    choose_splits(d, count, split);
  size_t bytes = dma ? prescale_need(d, count) : 0;
  for (int i = 0; i < count; ++i) bytes += part_bytes(d[i], split[i]);
  return bytes;
}

int tiled_max_problems() { return kMaxTiled; }

hipError_t launch_tiled_set(const GemmDesc *d, int count, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  if (count < 1 || count > kMaxTiled) return hipErrorInvalidValue;
  // The DMA kernel needs the prescaled X * s of problems with an s in the
  // workspace; without room for it the launch takes tiled_kernel.  Without
  // room for the split partials as well, K is not split.
  const size_t have = workspace ? workspace_bytes : 0;
  const size_t pre = prescale_need(d, count);
  const int tm = dma_tm(d, count);
  const bool dma = tm != 0 && pre <= have;
  const DmaShape ds = dma_shape(tm);
  const int bm = dma ? ds.bm() : kBM, bn = dma ? ds.bn() : kBN;
  int split[kMaxTiled];
  int ks = 1;
  if (dma)
    ks = dma_plan(d, count, tm, false, split);
  else
    choose_splits(d, count, split);
  size_t parts = 0;
  for (int i = 0; i < count; ++i) parts += part_bytes(d[i], split[i]);
  if ((dma ? pre : 0) + parts > have) {  // no room for partials: one K range
    for (int i = 0; i < count; ++i) split[i] = 1;
    if (dma) ks = dma_plan(d, count, tm, true, split);
  }
  TiledSet ts = {};
  int blocks = 0, rblocks = 0;
  size_t off = 0;
  // prescaled X * s after the partials
  size_t pre_off = 0;
  for (int i = 0; i < count; ++i) pre_off += part_bytes(d[i], split[i]);
  bool out = false;  // some problem has fp16 outliers
  PrescaleSet pset = {};
  int pblocks = 0;
  for (int i = 0; i < count; ++i) {
    TiledProblem &p = ts.p[i];
    p.X = static_cast<const _Float16 *>(d[i].X);
    p.Wq = static_cast<const uint8_t *>(d[i].Wq);
    p.scales = static_cast<const _Float16 *>(d[i].scales);
    p.zeros = static_cast<const _Float16 *>(d[i].zeros);
    p.s = static_cast<const _Float16 *>(d[i].s);
    p.Y = static_cast<_Float16 *>(d[i].Y);
    p.M = d[i].M;
    p.N = d[i].N;
    p.K = d[i].K;
    p.tiles_n = (d[i].N + bn - 1) / bn;
    p.tiles = tiles_of(d[i], bm, bn);
    p.split = split[i];
    p.part = split[i] > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + off) : nullptr;
    off += part_bytes(d[i], split[i]);
    p.orp = static_cast<const int32_t *>(d[i].o_row_ptr);
    p.ocol = static_cast<const int32_t *>(d[i].o_col);
    p.oval = static_cast<const _Float16 *>(d[i].o_val);
    out |= d[i].o_row_ptr != nullptr;
    p.bf16 = d[i].bf16;
    p.xs = static_cast<const _Float16 *>(d[i].X);
    if (dma && d[i].s) {
      // problems with the same X, s and shape (q, k and v of one layer, say)
      // share one prescaled copy
      int twin = -1;
      for (int j = 0; j < i && twin < 0; ++j)
        if (d[j].s == d[i].s && d[j].X == d[i].X && d[j].M == d[i].M && d[j].K == d[i].K) twin = j;
      if (twin >= 0) {
        p.xs = ts.p[twin].xs;
      } else {
        _Float16 *xs = reinterpret_cast<_Float16 *>(static_cast<char *>(workspace) + pre_off);
        pre_off += align256((size_t)d[i].M * d[i].K * 2);
        PrescaleItem &q = pset.p[pset.count++];
        q.X = static_cast<const _Float16 *>(d[i].X);
        q.s = static_cast<const _Float16 *>(d[i].s);
        q.out = xs;
        q.K = d[i].K;
        q.bf16 = d[i].bf16;
        q.n8 = (long long)d[i].M * d[i].K / 8;
        q.block0 = pblocks;
        pblocks += (int)((q.n8 + 255) / 256);
        p.xs = xs;
      }
    }
    p.block0 = blocks;
    blocks += p.tiles * p.split;
    p.rblock0 = rblocks;
    if (split[i] > 1)
      rblocks += (int)(((long long)d[i].M * d[i].N / 4 + kReduceThreads - 1) / kReduceThreads);
  }
  ts.count = count;
  if (pset.count > 0) {
    hipLaunchKernelGGL(prescale_f16_kernel, dim3(pblocks), dim3(256), 0, stream, pset);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(blocks), threads(kWM * kWN * 64);
  if (dma) {
    const hipError_t e = d[0].w8     ? launch_dma<false, true>(tm, ks, grid, stream, ts)
                         : d[0].bf16 ? launch_dma<true, false>(tm, ks, grid, stream, ts)
                                     : launch_dma<false, false>(tm, ks, grid, stream, ts);
    if (e != hipSuccess) return e;
  } else if (d[0].w8 && d[0].bf16 && out)  // INT8 codes
    hipLaunchKernelGGL((tiled_kernel<kWM, kWN, kTM, kTN, true, true, true>), grid, threads, 0,
                       stream, ts);
  else if (d[0].w8 && d[0].bf16)
    hipLaunchKernelGGL((tiled_kernel<kWM, kWN, kTM, kTN, false, true, true>), grid, threads, 0,
                       stream, ts);
  else if (d[0].w8 && out)
    hipLaunchKernelGGL((tiled_kernel<kWM, kWN, kTM, kTN, true, false, true>), grid, threads, 0,
                       stream, ts);
  else if (d[0].w8)
    hipLaunchKernelGGL((tiled_kernel<kWM, kWN, kTM, kTN, false, false, true>), grid, threads, 0,
                       stream, ts);
  else if (d[0].bf16 && out)  // one activation type (and code width) per launch
    hipLaunchKernelGGL((tiled_kernel<kWM, kWN, kTM, kTN, true, true>), grid, threads, 0, stream, ts);
  else if (d[0].bf16)
    hipLaunchKernelGGL((tiled_kernel<kWM, kWN, kTM, kTN, false, true>), grid, threads, 0, stream,
                       ts);
  else if (out)
    hipLaunchKernelGGL((tiled_kernel<kWM, kWN, kTM, kTN, true, false>), grid, threads, 0, stream,
                       ts);
  else
    hipLaunchKernelGGL((tiled_kernel<kWM, kWN, kTM, kTN, false, false>), grid, threads, 0, stream,
                       ts);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && rblocks > 0) {
    hipLaunchKernelGGL(split_reduce_kernel, dim3(rblocks), dim3(kReduceThreads), 0, stream, ts);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_tiled(const void *X, const void *Wq, const void *scales, const void *zeros,
                        const void *s, void *Y, int M, int N, int K, hipStream_t stream) {
  const GemmDesc d = {X, Wq, scales, zeros, s, Y, M, N, K};
  return launch_tiled_set(&d, 1, nullptr, 0, stream);
}

}  // namespace w4a16
