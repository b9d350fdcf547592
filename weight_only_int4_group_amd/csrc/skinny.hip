// Streaming dequantize-matmul for small M (decode M = 1, speculative verify
// M = draft length + 1): Y[M][N] = X[M][K] . W_hat^T with M <= 16, for one or
// several independent problems in a single launch.
//
// Where the time goes: the nano-vllm tutorial (discosf.com), section 1.1 and
// section 2.2, and "Chapter 22" (aiwing.uk) section 22.2's comparison table
// describe decode as bandwidth-bound -- every token streams all weights -- so
// this kernel is built to keep HBM busy: each packed byte is read exactly once
// and all other work hides behind the weight stream.
//
// Work split.  A wave owns one 16-row block of W and a slice of its K groups
// (S waves share a row block when the launch has too few row blocks to fill
// the GPU, or when a row is long); it walks its slice in chunks of GW groups,
// issuing the next chunk's loads before computing the current one, so every
// wave keeps a steady stream of 128-bit loads in flight.  Several problems
// share a launch by concatenating their workgroups.  Per group a wave
//   * loads the 1 KB tile with one 128-bit buffer load per lane (coalesced;
//     buffer loads are bounds-checked by the hardware); the scales and zero
//     points of a chunk's 4 groups are one 8-byte load each per lane (the
//     metadata is stored in 4-group quads, 128 contiguous bytes per row block),
//   * turns each 32-bit word into the exact fp16 values (q - z) in nine ALU
//     ops -- that register is the lane's 16x16x32 MFMA B operand,
//   * multiplies by X * s (staged in LDS once per workgroup, rounded to fp16
//     once; lanes of rows m >= M read row M - 1, whose products only reach
//     rows of Y that are not stored) with four MFMAs, and
//   * folds the group's fp32 dot products into the accumulator times the group
//     scale, in fp32.
// When S > 1 the S partial sums of a row block are added in a fixed order
// through LDS, so results are bit-reproducible run to run.
//
// X * s of all K columns fits in LDS for decode and short rows; when it does
// not (long rows at M > 1: the verify and batched-decode shapes), the
// workgroup walks K in windows instead.  A window is S chunks: the S waves of
// a row block take one chunk each, all row blocks of the workgroup share the
// window, and the next window's X * s is loaded into registers while the
// current one is multiplied.  When two windows fit, they alternate between two
// LDS buffers (one barrier per window); otherwise the next one is written over
// the current one between two barriers.  A call whose fp16 problems are of
// both kinds (speculative verify: the down projection's long rows do not fit,
// the others do) runs as one launch in which each workgroup stages its
// problem's X * s the way it fits.  Calls whose rows all fit a larger stage
// than two workgroups per CU allow run whole rows in 16-wave workgroups, one
// per CU, instead of windows.  Whole-row launches without outliers keep each
// wave's scales and zero points in an LDS slab when that costs no workgroup
// per CU.
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxProblems = 8;
// Cache policy of the code and metadata loads.  Every code byte is read once
// per call, so INT4 code loads are marked non-temporal (the NT bit, 2, of the
// buffer load's cache-policy operand on gfx950): measured 6% faster on the
// Llama-3-8B decode layer and 2-6% at the verify shapes.  INT8 codes keep the
// default: a lane's 32 bytes of a tile come from two loads 16 bytes apart, so
// each cache line is touched by two instructions, and with NT the INT8 decode
// layer measured 19% slower.  Metadata loads, shared by four lanes each, keep
// the default too (NT measured no better).
constexpr int kCodeCachePolicy = 2;  // NT
constexpr int kMetaCachePolicy = 0;
constexpr int kLdsPad = 8;         // halves of padding per staged X row
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format

struct Problem {
  const _Float16 *X;
  const uint8_t *Wq;
  const _Float16 *scales, *zeros, *s;
  _Float16 *Y;
  int M, N, K;
  int block0;  // first workgroup of this problem
  int split;   // waves per row block (a power of two, at most the workgroup's waves)
  const int32_t *orp, *ocol;  // fp16 outliers, row-compressed (null: none)
  const _Float16 *oval;
  // bf16 only (else null): X * s [M][K] as bf16 bits and its per-group sums
  // [M][G], written by prescale_kernel earlier in the call
  uint16_t *xpre;
  float *gpre;
  int window;  // hybrid launches: this problem walks K in windows
  // windowed: halves from the first window buffer to the second (0: a single
  // buffer, restaged between two barriers)
  int wpair;
};

struct ProblemSet {
  Problem p[kMaxProblems];
  int count;
};

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(bits));
  return r;
}

// Eight codes of one word -> the exact fp16 values (q_j - z), j = 0..7.
// Masks 0x000F000F and 0x00F000F0 pick the two 4-bit slots of each byte of a
// half-word directly; OR-ing them into 1024.0 gives 1024 + q and 1024 + 16q,
// both exact.  The first minus (1024 + z) is exact; the second times 1/16
// minus (64 + z) is exact as well.  Slots (0,4), (1,5), (2,6), (3,7) hold
// columns (0,1), (2,3), (4,5), (6,7).
__device__ __forceinline__ half8 decode_word9(uint32_t w, uint32_t m_lo, uint32_t m_hi,
                                              uint32_t magic, half2v bias_lo, half2v bias_hi) {
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const half2v a = as_half2(and_or(w, m_lo, magic)) - bias_lo;
  const half2v b = as_half2(and_or(w, m_hi, magic)) * sixteenth - bias_hi;
  const half2v c = as_half2(and_or(w8, m_lo, magic)) - bias_lo;
  const half2v d = as_half2(and_or(w8, m_hi, magic)) * sixteenth - bias_hi;
  half8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// INT8 codes: two words (columns j = 0..3 and 4..7, one byte each, in order)
// -> the exact fp16 values (q_j - z): v_perm_b32 pairs each code byte with the
// 0x64 high byte of 1024.0 (1024 + q, exact: fp16 spacing is 1 there), then
// minus (1024 + z).  Eight ops for eight codes.
__device__ __forceinline__ half8 decode_words8(uint32_t wa, uint32_t wb, half2v bias) {
  const uint32_t magic = 0x64646464u;
  const half2v a = as_half2(__builtin_amdgcn_perm(magic, wa, 0x05010400u)) - bias;
  const half2v b = as_half2(__builtin_amdgcn_perm(magic, wa, 0x05030402u)) - bias;
  const half2v c = as_half2(__builtin_amdgcn_perm(magic, wb, 0x05010400u)) - bias;
  const half2v d = as_half2(__builtin_amdgcn_perm(magic, wb, 0x05030402u)) - bias;
  half8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// bf16 operands: eight codes of one word -> the exact bf16 values 128 + q_j,
// j = 0..7, in seven ALU ops (the same slot-to-column order as above).  The
// zero point is taken off after the product: sum_k a_k (q_k - z) =
// sum_k a_k (128 + q_k) - (128 + z) sum_k a_k, with sum_k a_k staged per group.
__device__ __forceinline__ u32x4 decode_word_bf16(uint32_t w) {
  const uint32_t m = 0x000F000Fu;
  u32x4 r = {and_or(w, m, kMagicBF), and_or(w >> 4, m, kMagicBF), and_or(w >> 8, m, kMagicBF),
             and_or(w >> 12, m, kMagicBF)};
  return r;
}

// INT8 codes for bf16 operands: two words (columns j = 0..3 and 4..7, one
// byte each) -> the exact bf16 values q_j (a code 0..255 has at most 8
// significant bits, as many as bf16 holds): each byte converts to fp32
// exactly, and the fp32's upper half is the bf16.  The zero point comes off
// after the product, as for INT4 codes.
__device__ __forceinline__ uint32_t bytes_to_bf16x2(uint32_t w, int sh) {
  const float a = (float)((w >> sh) & 0xFFu), b = (float)((w >> (sh + 8)) & 0xFFu);
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                               0x07060302u);
}
__device__ __forceinline__ u32x4 decode_words8_bf16(uint32_t wa, uint32_t wb) {
  u32x4 r = {bytes_to_bf16x2(wa, 0), bytes_to_bf16x2(wa, 16), bytes_to_bf16x2(wb, 0),
             bytes_to_bf16x2(wb, 16)};
  return r;
}

// X * s of 8 consecutive columns, rounded once to the activation type (the
// exact product of a bf16 and an fp16 fits an fp32, so bf16 rounds once too),
// and the fp32 sum of the 8 rounded values (bf16 only).
template <bool kBF>
__device__ __forceinline__ u32x4 scale_x8(u32x4 xw, const _Float16 *s8, float &sum) {
  if (!kBF) {
    half8 v = __builtin_bit_cast(half8, xw);
    if (s8) v = v * load_half8(s8);
    return __builtin_bit_cast(u32x4, v);
  }
  half8 sv;
  if (s8) {
    sv = load_half8(s8);
  } else {
    const _Float16 one = (_Float16)1.0f;
    sv = (half8){one, one, one, one, one, one, one, one};
  }
  u32x4 out;
  sum = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = bf16_to_f32((uint16_t)xw[q]) * (float)sv[2 * q];
    const float hi = bf16_to_f32((uint16_t)(xw[q] >> 16)) * (float)sv[2 * q + 1];
    out[q] = pack_bf16x2(lo, hi);
    sum += bf16_to_f32((uint16_t)out[q]) + bf16_to_f32((uint16_t)(out[q] >> 16));
  }
  return out;
}

// Sum over the 16 lanes of a lane's 16-lane segment (one group of one row when
// the segment stages its 128 columns), in a fixed order.
__device__ __forceinline__ float segment_sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float x_value(const _Float16 *X, size_t i, bool bf) {
  const uint16_t h = __builtin_bit_cast(uint16_t, X[i]);
  return bf ? bf16_to_f32(h) : (float)X[i];
}

// The problem a workgroup works on is the same for all its lanes; say so, so
// that its pointers and sizes live in scalar registers.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its outstanding global loads (which stay in flight across the barrier).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The problem this workgroup works on, with every field in scalar registers.
__device__ __forceinline__ Problem find_problem(const ProblemSet &ps) {
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxProblems; ++i)
    if (i < ps.count && (int)blockIdx.x >= ps.p[i].block0) pi = i;
  Problem P;
  P.X = uniform_ptr(ps.p[pi].X);
  P.Wq = uniform_ptr(ps.p[pi].Wq);
  P.scales = uniform_ptr(ps.p[pi].scales);
  P.zeros = uniform_ptr(ps.p[pi].zeros);
  P.s = uniform_ptr(ps.p[pi].s);
  P.Y = uniform_ptr(ps.p[pi].Y);
  P.block0 = uniform_int(ps.p[pi].block0);
  P.M = uniform_int(ps.p[pi].M);
  P.N = uniform_int(ps.p[pi].N);
  P.K = uniform_int(ps.p[pi].K);
  P.split = uniform_int(ps.p[pi].split);
  P.orp = uniform_ptr(ps.p[pi].orp);
  P.ocol = uniform_ptr(ps.p[pi].ocol);
  P.oval = uniform_ptr(ps.p[pi].oval);
  P.xpre = uniform_ptr(ps.p[pi].xpre);
  P.gpre = uniform_ptr(ps.p[pi].gpre);
  P.window = uniform_int(ps.p[pi].window);
  P.wpair = uniform_int(ps.p[pi].wpair);
  return P;
}

// fp16 outliers of a row block, added by the wave that stores it, all 64
// lanes at once.  The kept weights of the block's 16 rows are one range
// e0 .. e1 - 1 of the row-compressed arrays; round u hands entry e0 + 64 u +
// lane to each lane.  The columns and values of the first kOutRounds rounds
// are loaded early (once X is staged, when the row pointers have arrived), so
// that only the X values they select are loaded in the epilogue.
constexpr int kOutRounds = 4;
struct OutPrefetch {
  int e0, e1;
  int col[kOutRounds];
  uint32_t val[kOutRounds];  // fp16 bits
};

// The loads go through buffer resources that cover only e0 .. e1 - 1:
// entries past e1 read 0 and are masked by index (e < e1) where used, so the
// loads are unconditional and nothing waits for them before the epilogue.
__device__ __forceinline__ OutPrefetch outlier_prefetch(const Problem &P, int2 orange, int lane) {
  OutPrefetch f;
  // lanes 0..15 (c = 0) hold the pairs of rows 0..15
  f.e0 = __builtin_amdgcn_readfirstlane(__shfl(orange.x, 0));
  f.e1 = __builtin_amdgcn_readfirstlane(__shfl(orange.y, 15));
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(P.ocol + f.e0), (short)0, (f.e1 - f.e0) * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(P.oval + f.e0), (short)0, (f.e1 - f.e0) * 2, kRsrcWord3);
#pragma unroll
  for (int u = 0; u < kOutRounds; ++u) {
    const int i = 64 * u + lane;
    f.col[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(crs, 4 * i, 0, 0);
    f.val[u] = __builtin_amdgcn_raw_buffer_load_b16(vrs, 2 * i, 0, 0);
  }
  return f;
}

__device__ __forceinline__ float wave_prefix_sum(float x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(x, o);
    x += lane >= o ? t : 0.f;
  }
  return x;
}

// o[v] for lane (c, r) of the storing wave: the sum over row r's kept weights
// of X[4c + v][col] * val (rows past M give 0 and are not stored).  In each
// round the lanes holding row r's entries are one run lo .. hi - 1 (entries
// are in row order); a wave-wide prefix sum of the terms gives the run's sum
// as a difference of two prefix values.  The order of the additions depends
// only on the row pointers, so results are reproducible.
template <bool kBF>
__device__ float4v outlier_terms(const Problem &P, const OutPrefetch &f, int2 orange, int lane,
                                 int c) {
  float4v o = {0.f, 0.f, 0.f, 0.f};
  const int M = P.M, K = P.K;
  auto round = [&](int base, int col, float val) {
    const int lo = min(max(orange.x - base, 0), 64), hi = min(max(orange.y - base, 0), 64);
    for (int m0 = 0; m0 < M; m0 += 4) {  // uniform
      float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (col >= 0 && m0 + v < M) t[v] = x_value(P.X, (size_t)(m0 + v) * K + col, kBF) * val;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (m0 + v >= M) break;  // uniform
        const float pre = wave_prefix_sum(t[v], lane);
        const float ph = __shfl(pre, max(hi - 1, 0)), pl = __shfl(pre, max(lo - 1, 0));
        if (c == (m0 >> 2) && hi > lo) o[v] += ph - (lo > 0 ? pl : 0.f);
      }
    }
  };
  const int rounds = (f.e1 - f.e0 + 63) / 64;
#pragma unroll
  for (int u = 0; u < kOutRounds; ++u) {
    if (u >= rounds) break;  // uniform
    const bool in = f.e0 + 64 * u + lane < f.e1;
    round(f.e0 + 64 * u, in ? f.col[u] : -1,
          (float)__builtin_bit_cast(_Float16, (uint16_t)f.val[u]));
  }
  for (int u = kOutRounds; u < rounds; ++u) {  // rows with many kept weights
    const int e = f.e0 + 64 * u + lane;
    int col = -1;
    float val = 0.f;
    if (e < f.e1) {
      col = P.ocol[e];
      val = (float)P.oval[e];
    }
    round(f.e0 + 64 * u, col, val);
  }
  return o;
}

// The lane's row-pointer pair when its wave stores outputs with outliers (the
// first K slice of a row block), else an empty range; issued first thing so
// that it has arrived by the epilogue.
__device__ __forceinline__ int2 outlier_range(const Problem &P, int b, bool has_rows, int ks,
                                              int r) {
  int2 e = {0, 0};
  if (P.orp && has_rows && ks == 0) {
    const int n = b * kTileRows + r;
    e.x = P.orp[n];
    e.y = P.orp[n + 1];
  }
  return e;
}

// Lane (c, r) holds D[m = 4c + v][n = r] of row block b summed over this
// wave's groups.  With S waves per row block the partial sums are added in
// the fixed order ks = 0, 1, ..., S - 1.  Every wave of the workgroup calls
// this (it may synchronise the workgroup).
// One output, rounded once to the activation type.
template <bool kBF>
__device__ __forceinline__ void store_y(_Float16 *Y, size_t i, float v) {
  if (kBF)
    reinterpret_cast<uint16_t *>(Y)[i] = f32_to_bf16(v);
  else
    Y[i] = (_Float16)v;
}

template <int kWaves, bool kOut, bool kBF>
__device__ __forceinline__ void store_rows(const Problem &P, float4v acc, int b, bool has_rows,
                                           int wave, int ks, int c, int r,
                                           float (*red)[16][17], int2 orange,
                                           const OutPrefetch &of) {
  const int lane = 16 * c + r;
  const int M = P.M, N = P.N, S = P.split;
  if (S == 1) {
    if (has_rows) {
      if (kOut) acc += outlier_terms<kBF>(P, of, orange, lane, c);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * c + v;
        if (m < M) store_y<kBF>(P.Y, (size_t)m * N + (size_t)b * kTileRows + r, acc[v]);
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * c + v][r] = acc[v];
    __syncthreads();
    if (ks == 0 && has_rows) {
      float4v o = {0.f, 0.f, 0.f, 0.f};
      if (kOut) o = outlier_terms<kBF>(P, of, orange, lane, c);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * c + v;
        if (m < M) {
          float sum = 0.f;
          for (int w = 0; w < S; ++w) sum += red[wave + w][m][r];
          if (kOut) sum += o[v];
          store_y<kBF>(P.Y, (size_t)m * N + (size_t)b * kTileRows + r, sum);
        }
      }
    }
  }
}

// Whole-row body: xs (dynamic LDS) holds X * s, then (after the last use of
// X) the split-K reduction.
template <int kGW, int kWaves, int kDepth, bool kOut, bool kBF, bool kW8 = false, bool kML = false>
__device__ __forceinline__ void skinny_body(const ProblemSet &ps, _Float16 *xs) {
  constexpr int kCW = kW8 ? 2 : 1;  // 16-byte code loads per lane per tile

  const Problem P = find_problem(ps);
  const int M = P.M, N = P.N, K = P.K, S = P.split;
  const int G = K / kGroup, NB = N / kTileRows;
  const int lane = threadIdx.x & 63, wave = uniform_int(threadIdx.x >> 6);
  const int c = lane >> 4;   // column octet (A/B operands), row quad (D)
  const int r = lane & 15;   // X row m (A), W row in the tile (B), column n (D)
  const int b = ((int)blockIdx.x - P.block0) * (kWaves / S) + wave / S;  // row block
  const int ks = wave % S;                                               // K slice
  const bool has_rows = b < NB;
  const int bb = has_rows ? b : NB - 1;
  // this wave's groups: [gb, ge), split on chunk boundaries
  const int chunks = (G + kGW - 1) / kGW;
  const int gb = min(G, (chunks * ks / S) * kGW);
  const int ge = has_rows ? min(G, (chunks * (ks + 1) / S) * kGW) : gb;
  const int nch = (ge - gb + kGW - 1) / kGW;  // chunks of this wave
  const int glast = max(gb, ge - 1);          // loads past the slice re-read this group

  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.Wq, (short)0, (int)min((size_t)0x7fffffff, (size_t)N * K * kCW / 2), kRsrcWord3);
  const int Gq = meta_groups(G) / kMetaQuad;
  const size_t meta_bytes = (size_t)N * Gq * kMetaQuad * 2;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.scales, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.zeros, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  // group-major tiles and quad-major metadata: the row block's part of the
  // offset is per lane, the group's part is uniform
  const int tile_off = bb * kTileBytes * kCW + lane * 16 * kCW;    // + g * tile_stride
  const int meta_off = (bb * kTileRows + r) * kMetaQuad * 2;      // + quad * meta_stride
  const int tile_stride = NB * kTileBytes * kCW, meta_stride = NB * kTileRows * kMetaQuad * 2;

  // A chunk is one or two metadata quads: 4 groups' scales (and zero points)
  // of this lane's row are one 8-byte load.
  static_assert(kGW % kMetaQuad == 0, "a chunk is whole metadata quads");
  static_assert(kDepth == 1, "one chunk of codes in flight (measured best)");
  constexpr int kQ = kGW / kMetaQuad;
  // Codes are loaded one chunk ahead, metadata two chunks ahead into one of
  // two register sets (so its loads never hold up a chunk's codes), steps
  // alternating between the sets so that nothing is copied.  Every step issues
  // the same loads: past the wave's last group they re-read it (in bounds and
  // in cache, never used), so the compiler's wait counts are the same on
  // every path.
  struct Meta {
    uint32_t sq[2 * kQ], zq[2 * kQ];  // scales, zero points (fp16 pairs)
  };
  u32x4 code[kGW][kCW];
  Meta m0, m1;
  auto load_codes = [&](int g0) {
#pragma unroll
    for (int i = 0; i < kGW; ++i)
#pragma unroll
      for (int h = 0; h < kCW; ++h)
        code[i][h] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, tile_off + 16 * h,
                                                         min(g0 + i, glast) * tile_stride,
                                                         kW8 ? 0 : kCodeCachePolicy));
  };
  // kML: the wave's scales and zero points (its range is at most 8 quads, 32
  // groups, as the launcher checks) come into a 2 KB LDS slab of the wave
  // with two DMA loads at the start, and each chunk reads its quad there
  // instead of issuing two loads (the launcher takes this instance when the
  // slabs cost no workgroup per CU).
  static_assert(!kML || (kQ == 1 && !kOut && !kW8), "LDS metadata: INT4 codes, one quad per chunk");
  unsigned char *mlds = nullptr;
  if constexpr (kML) {
    // after X * s (and, bf16, its group sums) or the reduction's partial sums
    const size_t xbytes = (size_t)M * (K + kLdsPad) * sizeof(_Float16) + (kBF ? (size_t)M * G * 4 : 0);
    const size_t rbytes = (size_t)kWaves * 16 * 17 * sizeof(float);
    mlds = reinterpret_cast<unsigned char *>(xs) + ((xbytes > rbytes ? xbytes : rbytes) + 15) / 16 * 16 +
           wave * 2048;
    // lane l: quad l / 8 of the range (clamped to the last), 16-byte piece l % 8
    const int u = min(gb / kMetaQuad + (lane >> 3), Gq - 1);
    const int off = (u * NB + bb) * 128 + (lane & 7) * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (__attribute__((address_space(3))) void *)mlds, 16,
                                             off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        zrs, (__attribute__((address_space(3))) void *)(mlds + 1024), 16, off, 0, 0, 0);
  }
  auto load_meta = [&](Meta &mt, int g0) {
    if constexpr (kML) {
      const int ql = (min(g0, glast) - gb) / kMetaQuad;
      const uint2 sv = *reinterpret_cast<const uint2 *>(mlds + ql * 128 + r * 8);
      const uint2 zv = *reinterpret_cast<const uint2 *>(mlds + 1024 + ql * 128 + r * 8);
      mt.sq[0] = sv.x;
      mt.sq[1] = sv.y;
      mt.zq[0] = zv.x;
      mt.zq[1] = zv.y;
    } else {
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int qoff = (min(g0, glast) / kMetaQuad + q) * meta_stride;
        const auto sv = __builtin_amdgcn_raw_buffer_load_b64(srs, meta_off, qoff, kMetaCachePolicy);
        const auto zv = __builtin_amdgcn_raw_buffer_load_b64(zrs, meta_off, qoff, kMetaCachePolicy);
        mt.sq[2 * q] = (uint32_t)sv[0];
        mt.sq[2 * q + 1] = (uint32_t)sv[1];
        mt.zq[2 * q] = (uint32_t)zv[0];
        mt.zq[2 * q + 1] = (uint32_t)zv[1];
      }
    }
  };
  // issue order: outlier row range, meta 0, codes 0, meta 1 (kML: the
  // metadata DMA, codes 0)
  const int2 orange = kOut ? outlier_range(P, b, has_rows, ks, r) : int2{0, 0};
  if (!kML) load_meta(m0, gb);
  load_codes(gb);
  if (!kML) load_meta(m1, gb + kGW);

  // stage X * s for rows 0..M-1; lanes of rows m >= M read row M - 1 (rows of
  // the A operand only reach the same rows of D, and those are not stored)
  // (bf16: also each group's sum of X * s per row, gsum[m][g], after the rows;
  // a 16-lane segment stages exactly one group of one row)
  float *gsum = reinterpret_cast<float *>(xs + M * (K + kLdsPad));
  {
    const int ldx = K + kLdsPad, k8 = K / 8;
    for (int idx = threadIdx.x; idx < M * k8; idx += kWaves * 64) {
      const int m = idx / k8, kk = (idx - m * k8) * 8;
      float part = 0.f;
      const u32x4 v = scale_x8<kBF>(*reinterpret_cast<const u32x4 *>(P.X + (size_t)m * K + kk),
                                    P.s ? P.s + kk : nullptr, part);
      *reinterpret_cast<u32x4 *>(&xs[m * ldx + kk]) = v;
      if (kBF) {
        part = segment_sum16(part);
        if ((idx & 15) == 0) gsum[m * G + kk / kGroup] = part;
      }
    }
    __syncthreads();
  }
  if constexpr (kML) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the metadata DMA has landed
    load_meta(m0, gb);
    load_meta(m1, gb + kGW);
  }
  OutPrefetch of = {};
  if (kOut) of = outlier_prefetch(P, orange, lane);
  const _Float16 *xrow = xs + min(r, M - 1) * (K + kLdsPad) + 8 * c;
  int gs_row[4];  // bf16: rows 4c + v of gsum (rows past M read row M - 1)
#pragma unroll
  for (int v = 0; v < 4; ++v) gs_row[v] = min(4 * c + v, M - 1) * G;

  const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = kMagic2;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  // chunk j: its codes and metadata (in `mt`) were issued earlier; take them,
  // issue chunk j+1's codes and chunk j+2's metadata (into `mt`), compute
  auto step = [&](int j, Meta &mt) {
    const int g0 = gb + j * kGW;
    u32x4 cur[kGW][kCW];
    half2v cs[2 * kQ], cz[2 * kQ];
#pragma unroll
    for (int i = 0; i < kGW; ++i)
#pragma unroll
      for (int h = 0; h < kCW; ++h) cur[i][h] = code[i][h];
#pragma unroll
    for (int q = 0; q < 2 * kQ; ++q) {
      cs[q] = as_half2(mt.sq[q]);
      cz[q] = as_half2(mt.zq[q]);
    }
    load_codes(g0 + kGW);
    load_meta(mt, g0 + 2 * kGW);
#pragma unroll
    for (int i = 0; i < kGW; ++i) {
      const int g = g0 + i;
      if (g < ge) {
        const _Float16 zp = cz[i >> 1][i & 1], sc = cs[i >> 1][i & 1];
        float4v tmp = {0.f, 0.f, 0.f, 0.f};
        if (kBF) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            tmp = mfma16_bf16(*reinterpret_cast<const u32x4 *>(xrow + g * kGroup + 32 * t),
                              kW8 ? decode_words8_bf16(cur[i][t >> 1 & (kCW - 1)][2 * (t & 1)],
                                                       cur[i][t >> 1 & (kCW - 1)][2 * (t & 1) + 1])
                                  : decode_word_bf16(cur[i][0][t]),
                              tmp);
          const float zb = (kW8 ? 0.0f : 128.0f) + (float)zp;
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] += (tmp[v] - zb * gsum[gs_row[v] + g]) * (float)sc;
        } else {
          half8 a[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const half8 *>(xrow + g * kGroup + 32 * t);
          const _Float16 blo = (_Float16)1024.0f + zp, bhi = (_Float16)64.0f + zp;
          const half2v bias_lo = {blo, blo}, bias_hi = {bhi, bhi};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const half8 bop = kW8 ? decode_words8(cur[i][t >> 1 & (kCW - 1)][2 * (t & 1)],
                                                  cur[i][t >> 1 & (kCW - 1)][2 * (t & 1) + 1], bias_lo)
                                  : decode_word9(cur[i][0][t], m_lo, m_hi, magic, bias_lo, bias_hi);
            tmp = mfma16(a[t], bop, tmp);
          }
          acc += tmp * (float)sc;
        }
      }
    }
  };
  for (int j = 0; j < nch; j += 2) {
    step(j, m0);
    if (j + 1 < nch) step(j + 1, m1);
  }

  if (S > 1) __syncthreads();  // every wave is done with X * s: its LDS takes the partial sums
  store_rows<kWaves, kOut, kBF>(P, acc, b, has_rows, wave, ks, c, r,
                                reinterpret_cast<float (*)[16][17]>(xs), orange, of);
}

template <int kGW, int kWaves, int kDepth, bool kOut, bool kBF, bool kW8 = false, bool kML = false>
__global__ __launch_bounds__(kWaves * 64) void skinny_kernel(ProblemSet ps) {
  extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
  skinny_body<kGW, kWaves, kDepth, kOut, kBF, kW8, kML>(ps, xs);
}

// bf16 X * s and its per-group sums, once per call, for the windowed kernel
// (which otherwise recomputes them in every workgroup, for every window).
// One 16-lane segment per (row m, group g), the same arithmetic and
// summation order as the staging in the kernels, so the values are identical.
__global__ __launch_bounds__(256) void prescale_kernel(ProblemSet ps) {
  const Problem P = find_problem(ps);
  const int K = P.K, G = K / kGroup;
  const int seg = ((int)blockIdx.x - P.block0) * 16 + (int)(threadIdx.x >> 4);
  if (seg >= P.M * G) return;  // whole segments
  const int m = seg / G, g = seg - m * G;
  const size_t k = (size_t)m * K + (size_t)g * kGroup + (threadIdx.x & 15) * 8;
  float part = 0.f;
  const u32x4 v = scale_x8<true>(*reinterpret_cast<const u32x4 *>(P.X + k),
                                 P.s ? P.s + g * kGroup + (threadIdx.x & 15) * 8 : nullptr, part);
  part = segment_sum16(part);
  *reinterpret_cast<u32x4 *>(P.xpre + k) = v;
  if ((threadIdx.x & 15) == 0) P.gpre[m * G + g] = part;
}

// Windowed variant: X * s staged one window of S chunks at a time (see the
// header).  kSlots bounds the 8-column pieces of a window each thread stages.
// xs (dynamic LDS) holds the window (two windows, alternating, when the
// launch has room for both), then (after the last window) the split-K
// reduction.
template <int kGW, int kWaves, int kDepth, int kSlots, bool kOut, bool kBF, bool kW8 = false,
          bool kPre = false>
__device__ __forceinline__ void skinny_window_body(const ProblemSet &ps, _Float16 *xs) {
  constexpr int kCW = kW8 ? 2 : 1;  // 16-byte code loads per lane per tile
  constexpr int kThreads = kWaves * 64;

  const Problem P = find_problem(ps);
  const int M = P.M, N = P.N, K = P.K, S = P.split;
  const int G = K / kGroup, NB = N / kTileRows;
  const int lane = threadIdx.x & 63, wave = uniform_int(threadIdx.x >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int b = ((int)blockIdx.x - P.block0) * (kWaves / S) + wave / S;
  const int ks = wave % S;
  const bool has_rows = b < NB;
  const int bb = has_rows ? b : NB - 1;
  const int chunks = (G + kGW - 1) / kGW;
  const int steps = (chunks + S - 1) / S;  // windows
  const int wcols = S * kGW * kGroup;      // columns per window
  const int ldx = wcols + kLdsPad;

  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.Wq, (short)0, (int)min((size_t)0x7fffffff, (size_t)N * K * kCW / 2), kRsrcWord3);
  const int Gq = meta_groups(G) / kMetaQuad;
  const size_t meta_bytes = (size_t)N * Gq * kMetaQuad * 2;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.scales, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P.zeros, (short)0, (int)min((size_t)0x7fffffff, meta_bytes), kRsrcWord3);
  const int2 orange = kOut ? outlier_range(P, b, has_rows, ks, r) : int2{0, 0};
  const int tile_off = bb * kTileBytes * kCW + lane * 16 * kCW;    // + g * tile_stride
  static_assert(!kPre || kBF, "prescaled X * s is a bf16 path");
  const int meta_off = (bb * kTileRows + r) * kMetaQuad * 2;      // + quad * meta_stride
  const int tile_stride = NB * kTileBytes * kCW, meta_stride = NB * kTileRows * kMetaQuad * 2;

  static_assert(kGW % kMetaQuad == 0, "a chunk is whole metadata quads");
  constexpr int kQ = kGW / kMetaQuad;
  u32x4 code[kDepth][kGW][kCW];
  uint32_t sq[kDepth][2 * kQ], zq[kDepth][2 * kQ];
  auto load_chunk = [&](int slot, int g0) {
#pragma unroll
    for (int i = 0; i < kGW; ++i)  // past the row: re-read its last tile (never used)
#pragma unroll
      for (int h = 0; h < kCW; ++h)
        code[slot][i][h] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, tile_off + 16 * h,
                                                         min(g0 + i, G - 1) * tile_stride,
                                                         kW8 ? 0 : kCodeCachePolicy));
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int qoff = min(g0 / kMetaQuad + q, Gq - 1) * meta_stride;
      const auto sv = __builtin_amdgcn_raw_buffer_load_b64(srs, meta_off, qoff, kMetaCachePolicy);
      const auto zv = __builtin_amdgcn_raw_buffer_load_b64(zrs, meta_off, qoff, kMetaCachePolicy);
      sq[slot][2 * q] = (uint32_t)sv[0];
      sq[slot][2 * q + 1] = (uint32_t)sv[1];
      zq[slot][2 * q] = (uint32_t)zv[0];
      zq[slot][2 * q + 1] = (uint32_t)zv[1];
    }
  };
  // first group of this wave's chunk in window j (may be >= G: nothing to do)
  auto chunk_g0 = [&](int j) { return (j * S + ks) * kGW; };

  // Staging map: thread -> one 8-column piece of the window (cs) and rows
  // r0, r0 + rstep, ...  The window's eighths (S * kGW * 16, a power of two
  // no larger than kThreads) divide kThreads.  Columns past K read zeros
  // (buffer loads out of range), and are never multiplied.
  const int c8 = wcols / 8;
  const int cs = (int)threadIdx.x & (c8 - 1), r0 = (int)threadIdx.x / c8, rstep = kThreads / c8;
  // bf16 with a prescaled X * s (prescale_kernel): the window is a plain copy
  // of it and of its group sums
  constexpr bool pre = kBF && kPre;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      pre ? (void *)P.xpre : (void *)P.X, (short)0, M * K * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ssr =
      __builtin_amdgcn_make_buffer_rsrc((void *)P.s, (short)0, P.s ? K * 2 : 0, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t grs =
      __builtin_amdgcn_make_buffer_rsrc((void *)P.gpre, (short)0, pre ? M * G * 4 : 0, kRsrcWord3);
  half8 xr[kSlots], sv;
  float gp[kBF ? kSlots : 1];
  auto load_window = [&](int w) {
    const int k = w * wcols + cs * 8;
    const int koff = k < K ? 2 * k : 2 * M * K;  // past K: out of range, reads zeros
    if (pre) {
      // the group sum of this lane's segment (groups past G read zeros)
      const int gw = k / kGroup;
#pragma unroll
      for (int i = 0; i < kSlots; ++i) {
        const int m = r0 + i * rstep;
        gp[kBF ? i : 0] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       grs, m < M && gw < G ? 4 * (m * G + gw) : 4 * M * G, 0, 0));
      }
    } else if (P.s) {
      sv = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ssr, k < K ? 2 * k : 2 * K, 0, 0));
    } else {
      const _Float16 one = (_Float16)1.0f;
      sv = (half8){one, one, one, one, one, one, one, one};
    }
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      // rows past M read zeros too (out of range); they are not written to LDS
      const int m = r0 + i * rstep;
      xr[i] = __builtin_bit_cast(
          half8, __builtin_amdgcn_raw_buffer_load_b128(xrs, m < M ? koff + 2 * m * K : 2 * M * K, 0, 0));
    }
  };
  // bf16: each window group's sum of X * s per row, wsum[m][window group],
  // after the window's rows (a 16-lane segment stages one group of one row)
  const int wgroups = S * kGW;
  // Window j is in buffer j % 2 when the launch has room for two (wpair > 0):
  // a window is staged while the one before is read, one barrier per window.
  // With one buffer, restaging waits for every wave to be done with it.
  const int wpair = uniform_int(P.wpair);
  auto store_window = [&](_Float16 *wx) {
    float *wsum = reinterpret_cast<float *>(wx + M * ldx);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const int m = r0 + i * rstep;
      if (!kBF) {
        if (m < M) *reinterpret_cast<half8 *>(&wx[m * ldx + cs * 8]) = xr[i] * sv;
      } else if (pre) {
        if (m < M) {
          *reinterpret_cast<half8 *>(&wx[m * ldx + cs * 8]) = xr[i];
          if ((cs & 15) == 0) wsum[m * wgroups + cs / 16] = gp[kBF ? i : 0];
        }
      } else {
        float part = 0.f;
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t xw = __builtin_bit_cast(u32x4, xr[i])[q];
          const float lo = bf16_to_f32((uint16_t)xw) * (float)sv[2 * q];
          const float hi = bf16_to_f32((uint16_t)(xw >> 16)) * (float)sv[2 * q + 1];
          out[q] = pack_bf16x2(lo, hi);
          part += bf16_to_f32((uint16_t)out[q]) + bf16_to_f32((uint16_t)(out[q] >> 16));
        }
        part = segment_sum16(part);  // all 16 lanes of the segment share m
        if (m < M) {
          *reinterpret_cast<u32x4 *>(&wx[m * ldx + cs * 8]) = out;
          if ((cs & 15) == 0) wsum[m * wgroups + cs / 16] = part;
        }
      }
    }
  };

  // Every step issues the same loads, also past the last window or chunk
  // (clamped to the row's last group, or out-of-range buffer offsets that read
  // zeros; the data is never used), so that the compiler's wait counts are the
  // same on every path through the loop.
  load_window(0);
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_chunk(d, chunk_g0(d));
  store_window(xs);
  lds_barrier();
  OutPrefetch of = {};
  if (kOut) of = outlier_prefetch(P, orange, lane);
  load_window(1);

  // rows m >= M of the A operand only feed rows of D that are not stored
  const _Float16 *xrow0 = xs + min(r, M - 1) * ldx + ks * kGW * kGroup + 8 * c;
  int ws_row[4];  // bf16: rows 4c + v of wsum (after the window's rows) at this wave's chunk
#pragma unroll
  for (int v = 0; v < 4; ++v) ws_row[v] = M * ldx / 2 + min(4 * c + v, M - 1) * wgroups + ks * kGW;
  const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = kMagic2;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  // Issue order per step: this wave's next chunk, then (after the window
  // swap) the window after next.  Each wait then leaves only younger loads in
  // flight: the weights for the window's X, that X for the next weights.
  for (int j = 0; j < steps; ++j) {
    u32x4 cur[kGW][kCW];
    half2v cs2[2 * kQ], cz2[2 * kQ];
#pragma unroll
    for (int i = 0; i < kGW; ++i)
#pragma unroll
      for (int h = 0; h < kCW; ++h) cur[i][h] = code[0][i][h];
#pragma unroll
    for (int q = 0; q < 2 * kQ; ++q) {
      cs2[q] = as_half2(sq[0][q]);
      cz2[q] = as_half2(zq[0][q]);
    }
#pragma unroll
    for (int d = 0; d + 1 < kDepth; ++d) {
#pragma unroll
      for (int i = 0; i < kGW; ++i)
#pragma unroll
        for (int h = 0; h < kCW; ++h) code[d][i][h] = code[d + 1][i][h];
#pragma unroll
      for (int q = 0; q < 2 * kQ; ++q) {
        sq[d][q] = sq[d + 1][q];
        zq[d][q] = zq[d + 1][q];
      }
    }
    load_chunk(kDepth - 1, chunk_g0(j + kDepth));

    const int g0 = chunk_g0(j);
    const _Float16 *xrow = xrow0 + (j & 1) * wpair;
    const float *wsum = reinterpret_cast<const float *>(xs + (j & 1) * wpair);
    if (has_rows && g0 < G) {
#pragma unroll
      for (int i = 0; i < kGW; ++i) {
        if (g0 + i < G) {
          const _Float16 zp = cz2[i >> 1][i & 1], sc = cs2[i >> 1][i & 1];
          float4v tmp = {0.f, 0.f, 0.f, 0.f};
          if (kBF) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
              tmp = mfma16_bf16(
                  *reinterpret_cast<const u32x4 *>(xrow + i * kGroup + 32 * t),
                  kW8 ? decode_words8_bf16(cur[i][t >> 1 & (kCW - 1)][2 * (t & 1)],
                                           cur[i][t >> 1 & (kCW - 1)][2 * (t & 1) + 1])
                      : decode_word_bf16(cur[i][0][t]),
                  tmp);
            const float zb = (kW8 ? 0.0f : 128.0f) + (float)zp;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] += (tmp[v] - zb * wsum[ws_row[v] + i]) * (float)sc;
          } else {
            const _Float16 blo = (_Float16)1024.0f + zp, bhi = (_Float16)64.0f + zp;
            const half2v bias_lo = {blo, blo}, bias_hi = {bhi, bhi};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const half8 bop =
                  kW8 ? decode_words8(cur[i][t >> 1 & (kCW - 1)][2 * (t & 1)],
                                      cur[i][t >> 1 & (kCW - 1)][2 * (t & 1) + 1], bias_lo)
                      : decode_word9(cur[i][0][t], m_lo, m_hi, magic, bias_lo, bias_hi);
              tmp = mfma16(*reinterpret_cast<const half8 *>(xrow + i * kGroup + 32 * t), bop, tmp);
            }
            acc += tmp * (float)sc;
          }
        }
      }
    }
    // window j + 1: into the other buffer (every wave was done with window j
    // - 1 there at the last barrier), or into the one buffer once every wave
    // is done with window j
    if (!wpair) lds_barrier();
    store_window(xs + ((j + 1) & 1) * wpair);
    load_window(j + 2);
    lds_barrier();
  }
  // every wave is past the last barrier: the window's LDS takes the partial sums
  store_rows<kWaves, kOut, kBF>(P, acc, b, has_rows, wave, ks, c, r,
                                reinterpret_cast<float (*)[16][17]>(xs), orange, of);
}

template <int kGW, int kWaves, int kDepth, int kSlots, bool kOut, bool kBF, bool kW8 = false,
          bool kPre = false>
__global__ __launch_bounds__(kWaves * 64) void skinny_window_kernel(ProblemSet ps) {
  extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
  skinny_window_body<kGW, kWaves, kDepth, kSlots, kOut, kBF, kW8, kPre>(ps, xs);
}

// Both kinds in one launch (fp16 INT4 codes without outliers): a workgroup
// stages the whole rows of its problem's X * s when they fit in LDS, and
// walks K in windows otherwise (the problem's `window` flag).
template <int kGW, int kWaves, int kDepth, int kSlots>
__global__ __launch_bounds__(kWaves * 64) void skinny_hybrid_kernel(ProblemSet ps) {
  extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxProblems; ++i)
    if (i < ps.count && (int)blockIdx.x >= ps.p[i].block0) pi = i;
  if (uniform_int(ps.p[pi].window))
    skinny_window_body<kGW, kWaves, kDepth, kSlots, false, false>(ps, xs);
  else
    skinny_body<kGW, kWaves, kDepth, false, false>(ps, xs);
}

constexpr size_t kMaxStageBytes = 96 * 1024;
constexpr int kChunk = 4;  // groups per chunk (weight loads in flight per wave)
constexpr int kWaves = 8;  // waves per workgroup
// fp16 INT4 calls whose X * s all fit in kWideStageBytes but not all in
// kMaxStageBytes (the Llama-3-8B layer at M = 4 and 5: down's rows take 115
// and 143 KB) stage
// whole rows in 16-wave workgroups, one per CU: the same waves per CU as two
// 8-wave workgroups, and no windows (measured 26.1 -> 24.9 us at M = 5).
// Launches with windows keep 8 waves: 16-wave hybrid launches were slower
// (M = 9: 26.9 -> 31.5 us; Qwen2-7B M = 16: 32.1 -> 37.3 us).
constexpr int kWideWaves = 16;
// LDS metadata slabs of the whole-row kernel: 2 KB per wave (8 quads of
// scales and zero points, 32 groups), taken when they cost no workgroup per
// CU: the kernel's registers allow three 8-wave workgroups, LDS 160 KB
constexpr int kMetaSlabChunks = 8;
constexpr size_t kMetaSlabBytes = (size_t)kWaves * 2048;
constexpr size_t kCuLdsBytes = 160 * 1024;
constexpr size_t kWholeWgsPerCu = 3;
size_t wgs_per_cu(size_t lds) {
  const size_t by_lds = lds ? kCuLdsBytes / lds : kWholeWgsPerCu;
  return by_lds < kWholeWgsPerCu ? by_lds : kWholeWgsPerCu;
}
constexpr size_t kWideStageBytes = 150 * 1024;
constexpr int kDepth = 1;  // chunks in flight per wave
// 1: window the problems whose X * s does not fit, 2: always window, 3:
// window the whole call when one problem does not fit (measured best; 1 and 2
// are kept as the documented alternatives)
constexpr int kWindowMode = 3;
// fp16 INT4 calls with problems of both kinds: one launch in which each
// problem stages its X * s the way it fits (skinny_hybrid_kernel)
constexpr bool kHybridLaunch = true;
static_assert(kWindowMode >= 1 && kWindowMode <= 3, "X * s must fit in LDS or go in windows");
constexpr size_t kMaxWindowBytes = 72 * 1024;  // two workgroups per CU
// Two window buffers when both fit in this (still two workgroups per CU)
constexpr size_t kMaxWindowPairBytes = 80 * 1024;
constexpr int kWindowSlots = 8;  // staged 8-column pieces per thread
// bf16 and INT8 codes: fewer pieces cut the registers (the prescaled bf16
// instance needs 110 instead of 146: two 8-wave workgroups per CU instead of
// one); the bf16 instance that scales X itself uses the same count, so both
// choose the same splits and give the same bits
constexpr int kWindowSlotsBF = 4;
// LDS bytes of the whole-row kernel: X * s of one problem, at least the
// reduction's partial sums (which reuse it).
size_t stage_bytes(int M, int K, bool bf16) {
  const size_t x = (size_t)M * (K + kLdsPad) * sizeof(_Float16) +
                   (bf16 ? (size_t)M * (K / kGroup) * sizeof(float) : 0);
  const size_t red = (size_t)kWaves * 16 * 17 * sizeof(float);
  return x > red ? x : red;
}

constexpr int kTargetWaves = 2048;     // enough waves in flight to cover HBM latency
constexpr int kMaxGroupsPerWave = 32;  // longer rows are split across waves

// LDS bytes of one window of S chunks, M rows.
size_t window_bytes(int M, int S, bool bf16) {
  return (size_t)M * (S * kChunk * kGroup + kLdsPad) * sizeof(_Float16) +
         (bf16 ? (size_t)M * S * kChunk * sizeof(float) : 0);
}

// 8-column pieces of a window each thread stages (0: the window is wider than
// the workgroup has threads).
int window_slots(int M, int S) {
  const int c8 = S * kChunk * kGroup / 8, threads = kWaves * 64;
  if (c8 > threads) return 0;
  const int rstep = threads / c8;
  return (M + rstep - 1) / rstep;
}

int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p *= 2;
  return p;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of one bf16 problem's prescaled X * s: bf16 [M][K], then fp32
// group sums [M][G].
size_t prescale_bytes(int M, int K) {
  return align256((size_t)M * K * 2) + align256((size_t)M * (K / kGroup) * 4);
}

}  // namespace

int skinny_max_problems() { return kMaxProblems; }

namespace {

// The windowed instances over INT8 codes.
void launch_window8(bool bf, bool out, bool pre, dim3 grid, dim3 threads, size_t lds,
                    hipStream_t stream, const ProblemSet &ps) {
  constexpr int S = kWindowSlotsBF;
  if (bf && out && pre)
    hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, S, true, true, true, true>),
                       grid, threads, lds, stream, ps);
  else if (bf && pre)
    hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, S, false, true, true, true>),
                       grid, threads, lds, stream, ps);
  else if (bf && out)
    hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, S, true, true, true>), grid,
                       threads, lds, stream, ps);
  else if (bf)
    hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, S, false, true, true>), grid,
                       threads, lds, stream, ps);
  else if (out)
    hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, S, true, false, true>), grid,
                       threads, lds, stream, ps);
  else
    hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, S, false, false, true>), grid,
                       threads, lds, stream, ps);
}


enum LaunchKind { kWhole = 0, kWindowed = 1, kHybrid = 2 };

// One launch over the problems d[0..count): whole-row X * s staging, K
// windows, or (kHybrid: fp16 INT4 codes without outliers) each problem the
// way its X * s fits.
hipError_t launch_group(const GemmDesc *const *d, int count, LaunchKind kind, hipStream_t stream,
                        int waves = kWaves) {
  if (count == 0) return hipSuccess;
  // How many waves share a row block: enough waves in the whole launch to keep
  // HBM busy, and no wave walking more than kMaxGroupsPerWave groups.
  long long rows = 0;
  for (int i = 0; i < count; ++i) rows += d[i]->N / kTileRows;
  const int s_fill =
      (int)min((long long)waves, (long long)pow2_at_least((int)((kTargetWaves + rows - 1) / rows)));
  // Problems are laid out longest-rows first so that the waves with the most
  // work start first.
  int order[kMaxProblems];
  for (int i = 0; i < count; ++i) order[i] = i;
  for (int i = 1; i < count; ++i)
    for (int j = i; j > 0 && d[order[j]]->K > d[order[j - 1]]->K; --j) {
      const int t = order[j];
      order[j] = order[j - 1];
      order[j - 1] = t;
    }
  ProblemSet ps = {};
  int blocks = 0;
  size_t lds = 0;
  bool out = false;  // some problem has fp16 outliers
  bool meta_fits = true;  // every wave's groups fit an LDS metadata slab
  const bool window = kind == kWindowed;
  // bf16 with prescaled X * s: all or none of a launch (launch_skinny_set)
  const bool pre = window && d[0]->bf16 && d[0]->xpre != nullptr;
  const int slot_cap = d[0]->bf16 || d[0]->w8 ? kWindowSlotsBF : kWindowSlots;
  for (int i = 0; i < count; ++i) {
    const GemmDesc &q = *d[order[i]];
    Problem &p = ps.p[i];
    const int G = q.K / kGroup, NB = q.N / kTileRows;
    const bool win = kind == kWindowed ||
                     (kind == kHybrid && stage_bytes(q.M, q.K, q.bf16) > kMaxStageBytes);
    int split = s_fill;
    while (split < waves && (G + split - 1) / split > kMaxGroupsPerWave) split *= 2;
    while (split > 1 && (G + kChunk - 1) / kChunk < split) split /= 2;  // a chunk per wave
    if (win)  // a window of split chunks must fit in LDS and in the staging registers
      while (split > 1 && (window_bytes(q.M, split, q.bf16) > kMaxWindowBytes ||
                           window_slots(q.M, split) < 1 || window_slots(q.M, split) > slot_cap))
        split /= 2;
    p.X = static_cast<const _Float16 *>(q.X);
    p.Wq = static_cast<const uint8_t *>(q.Wq);
    p.scales = static_cast<const _Float16 *>(q.scales);
    p.zeros = static_cast<const _Float16 *>(q.zeros);
    p.s = static_cast<const _Float16 *>(q.s);
    p.Y = static_cast<_Float16 *>(q.Y);
    p.M = q.M;
    p.N = q.N;
    p.K = q.K;
    p.split = split;
    p.orp = static_cast<const int32_t *>(q.o_row_ptr);
    p.ocol = static_cast<const int32_t *>(q.o_col);
    p.oval = static_cast<const _Float16 *>(q.o_val);
    p.xpre = static_cast<uint16_t *>(q.xpre);
    p.gpre = q.xpre ? reinterpret_cast<float *>(static_cast<char *>(q.xpre) +
                                                align256((size_t)q.M * q.K * 2))
                    : nullptr;
    out |= q.o_row_ptr != nullptr;
    p.window = win;
    p.block0 = blocks;
    const int rb_per_wg = waves / split;
    blocks += (NB + rb_per_wg - 1) / rb_per_wg;
    const size_t wb = window_bytes(q.M, split, q.bf16), wb16 = (wb + 15) / 16 * 16;
    const bool pair = win && 2 * wb16 <= kMaxWindowPairBytes;
    p.wpair = pair ? (int)(wb16 / 2) : 0;
    const size_t wlds = pair ? 2 * wb16 : wb;
    // the split-K partial sums reuse the X * s space
    const size_t red = (size_t)waves * 16 * 17 * sizeof(float), sb = stage_bytes(q.M, q.K, q.bf16);
    const size_t need = win ? (wlds > red ? wlds : red) : (sb > red ? sb : red);
    lds = need > lds ? need : lds;
    meta_fits &= ((G + kChunk - 1) / kChunk + split - 1) / split <= kMetaSlabChunks;
  }
  ps.count = count;
  // whole rows, INT4 codes without outliers: each wave's scales and zero
  // points in an LDS slab when every wave's range fits one and the slabs cost
  // no workgroup per CU (measured 22.72 -> 22.52 us on the 8B layer at M = 1
  // and 23.0 -> 22.7 us at M = 2; slabs that cost a workgroup per CU made the
  // M = 9 verify launch slower, 28.1 -> 31.8 us)
  const size_t lds_ml = (lds + 15) / 16 * 16 + kMetaSlabBytes;
  const bool ml = kind == kWhole && waves == kWaves && !d[0]->w8 && !out &&
                  meta_fits && wgs_per_cu(lds_ml) == wgs_per_cu(lds);
  if (ml) lds = lds_ml;
  const dim3 grid(blocks), threads(waves * 64);
  const bool bf = d[0]->bf16;  // one activation type (and code width) per launch
  if (waves == kWideWaves) {
    if (kind != kWhole || bf || out || d[0]->w8) return hipErrorInvalidValue;  // not instantiated
    hipLaunchKernelGGL((skinny_kernel<kChunk, kWideWaves, kDepth, false, false>), grid, threads,
                       lds, stream, ps);
  } else if (kind == kHybrid) {
    if (bf || out || d[0]->w8) return hipErrorInvalidValue;  // not instantiated
    hipLaunchKernelGGL((skinny_hybrid_kernel<kChunk, kWaves, kDepth, kWindowSlots>), grid, threads,
                       lds, stream, ps);
  } else if (d[0]->w8) {  // INT8 codes
    if (window)
      launch_window8(bf, out, pre, grid, threads, lds, stream, ps);
    else if (bf && out)
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, true, true, true>), grid, threads,
                         lds, stream, ps);
    else if (bf)
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, false, true, true>), grid, threads,
                         lds, stream, ps);
    else if (out)
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, true, false, true>), grid, threads,
                         lds, stream, ps);
    else
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, false, false, true>), grid, threads,
                         lds, stream, ps);
  } else if (window) {
    if (bf && out && pre)
      hipLaunchKernelGGL(
          (skinny_window_kernel<kChunk, kWaves, kDepth, kWindowSlotsBF, true, true, false, true>),
          grid, threads, lds, stream, ps);
    else if (bf && pre)
      hipLaunchKernelGGL(
          (skinny_window_kernel<kChunk, kWaves, kDepth, kWindowSlotsBF, false, true, false, true>),
          grid, threads, lds, stream, ps);
    else if (bf && out)
      hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, kWindowSlotsBF, true, true>),
                         grid, threads, lds, stream, ps);
    else if (bf)
      hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, kWindowSlotsBF, false, true>),
                         grid, threads, lds, stream, ps);
    else if (out)
      hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, kWindowSlots, true, false>),
                         grid, threads, lds, stream, ps);
    else
      hipLaunchKernelGGL((skinny_window_kernel<kChunk, kWaves, kDepth, kWindowSlots, false, false>),
                         grid, threads, lds, stream, ps);
  } else {
    if (bf && out)
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, true, true>), grid, threads, lds,
                         stream, ps);
    else if (bf && ml)
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, false, true, false, true>), grid,
                         threads, lds, stream, ps);
    else if (bf)
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, false, true>), grid, threads, lds,
                         stream, ps);
    else if (out)
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, true, false>), grid, threads, lds,
                         stream, ps);
    else if (ml)
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, false, false, false, true>), grid,
                         threads, lds, stream, ps);
    else
      hipLaunchKernelGGL((skinny_kernel<kChunk, kWaves, kDepth, false, false>), grid, threads, lds,
                         stream, ps);
  }
  return hipGetLastError();
}

// bf16 X * s and group sums of the problems d[0..count) into their xpre.
hipError_t launch_prescale(const GemmDesc *const *d, int count, hipStream_t stream) {
  ProblemSet ps = {};
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    const GemmDesc &q = *d[i];
    Problem &p = ps.p[i];
    p.X = static_cast<const _Float16 *>(q.X);
    p.s = static_cast<const _Float16 *>(q.s);
    p.M = q.M;
    p.N = q.N;
    p.K = q.K;
    p.xpre = static_cast<uint16_t *>(q.xpre);
    p.gpre = reinterpret_cast<float *>(static_cast<char *>(q.xpre) + align256((size_t)q.M * q.K * 2));
    p.block0 = blocks;
    blocks += (q.M * (q.K / kGroup) + 15) / 16;  // 16 segments of 16 lanes per workgroup
  }
  ps.count = count;
  hipLaunchKernelGGL(prescale_kernel, dim3(blocks), dim3(256), 0, stream, ps);
  return hipGetLastError();
}

}  // namespace

size_t skinny_workspace_bytes(const GemmDesc *d, int count) {
  size_t n = 0;
  for (int i = 0; i < count; ++i)
    if (d[i].bf16) n += prescale_bytes(d[i].M, d[i].K);
  return n;
}

hipError_t launch_skinny_set(const GemmDesc *d, int count, hipStream_t stream, bool force_window,
                             void *workspace, size_t workspace_bytes) {
  if (count < 1 || count > kMaxProblems) return hipErrorInvalidValue;
  // By default the whole launch uses windows as soon as one problem's X * s does
  // not fit: one launch over all problems beats a second, smaller one.  Like
  // the split factor, the choice depends on all problems of the call, so a
  // problem's bits can differ between a grouped and a single call (both stay
  // within rounding of the exact result; each call is reproducible).  fp16 and
  // bf16 problems go in separate launches (one kernel instance each).
  hipError_t err = hipSuccess;
  for (int cls = 0; cls < 4 && err == hipSuccess; ++cls) {
    // classes: fp16 INT4, bf16 INT4, fp16 INT8, bf16 INT8
    const bool want_bf = (cls & 1) != 0, want_w8 = cls >= 2;
    auto in_class = [&](const GemmDesc &q) { return q.bf16 == want_bf && q.w8 == want_w8; };
    const GemmDesc *whole[kMaxProblems], *windowed[kMaxProblems];
    int nwhole = 0, nwin = 0;
    bool any = false, all = true, outl = false, wide = true;
    const GemmDesc *members[kMaxProblems];
    int nm = 0;
    for (int i = 0; i < count; ++i)
      if (in_class(d[i])) {
        const bool big = stage_bytes(d[i].M, d[i].K, d[i].bf16) > kMaxStageBytes;
        any |= big;
        all &= big;
        wide &= stage_bytes(d[i].M, d[i].K, d[i].bf16) <= kWideStageBytes;
        outl |= d[i].o_row_ptr != nullptr;
        members[nm++] = d + i;
      }
    // fp16 INT4 without outliers, all X * s within kWideStageBytes: whole rows
    // in 16-wave workgroups
    if (cls == 0 && any && wide && !outl && !force_window) {
      err = launch_group(members, nm, kWhole, stream, kWideWaves);
      continue;
    }
    // fp16 INT4 without outliers: problems that fit stage whole rows and the
    // others walk windows, in the same launch
    if (kHybridLaunch && cls == 0 && any && !all && !outl && !force_window && kWindowMode == 3) {
      err = launch_group(members, nm, kHybrid, stream);
      continue;
    }
    for (int i = 0; i < count; ++i) {
      if (!in_class(d[i])) continue;
      const bool fits = stage_bytes(d[i].M, d[i].K, d[i].bf16) <= kMaxStageBytes;
      const bool win = force_window || kWindowMode == 2 || (kWindowMode == 1 && !fits) ||
                       (kWindowMode == 3 && any);
      if (win)
        windowed[nwin++] = d + i;
      else
        whole[nwhole++] = d + i;
    }
    // bf16 windows: X * s once per call when the workspace has room for it
    GemmDesc pre[kMaxProblems];
    size_t need = 0;
    if (want_bf && nwin > 0 && workspace) {
      for (int i = 0; i < nwin; ++i) need += prescale_bytes(windowed[i]->M, windowed[i]->K);
      if (need <= workspace_bytes) {
        char *ws = static_cast<char *>(workspace);
        for (int i = 0; i < nwin; ++i) {
          pre[i] = *windowed[i];
          pre[i].xpre = ws;
          ws += prescale_bytes(pre[i].M, pre[i].K);
          windowed[i] = pre + i;
        }
        err = launch_prescale(windowed, nwin, stream);
      }
    }
    if (err == hipSuccess) err = launch_group(windowed, nwin, kWindowed, stream);
    if (err == hipSuccess) err = launch_group(whole, nwhole, kWhole, stream);
  }
  return err;
}

hipError_t launch_skinny(const void *X, const void *Wq, const void *scales, const void *zeros,
                         const void *s, void *Y, int M, int N, int K, hipStream_t stream) {
  const GemmDesc d = {X, Wq, scales, zeros, s, Y, M, N, K};
  return launch_skinny_set(&d, 1, stream);
}

}  // namespace w4a16
