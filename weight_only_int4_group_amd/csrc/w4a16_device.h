// Device-side helpers shared by the packer and the two GEMM kernels.
//
// Packed code tile (16 rows x 128 columns, 1024 bytes): lane L = 16c + r owns
// 16 bytes, i.e. four 32-bit words; word t holds the eight codes of columns
// 32t + 8c + j (j = 0..7) of row r, column j sitting in the 4-bit slot i with
// j = 2*(i % 4) + i / 4.  So the masks 0x000F000F, after shifting the word
// right by 4p, select exactly the pair of columns (2p, 2p+1) as the low and
// high halves of a 32-bit register.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;
constexpr int kTileRows = 16;
constexpr int kTileBytes = 1024;
constexpr int kWave = 64;
constexpr int kMetaQuad = 4;   // groups per metadata quad

// Code tiles are group-major: tile (row block b, group g) is the 1 KB at
// (g * NB + b) * 1024, NB = N / 16, so the tiles that concurrently running
// waves stream (neighbouring row blocks, same group) are neighbours in memory.
//
// Metadata (scale / zero point) layout: quads of 4 groups, quad-major in the
// same way.  Element index of row n, group g, for NB row blocks.
__host__ __device__ constexpr int meta_groups(int G) { return (G + kMetaQuad - 1) / kMetaQuad * kMetaQuad; }
__host__ __device__ inline size_t meta_index(int n, int g, int NB) {
  return (((size_t)(g / kMetaQuad) * NB + n / kTileRows) * kTileRows + n % kTileRows) * kMetaQuad +
         g % kMetaQuad;
}

// fp16 bit pattern 0x6400 is 1024.0; OR-ing a 4-bit code q into its low
// mantissa bits gives the fp16 value 1024 + q exactly (the ulp at 1024 is 1).
constexpr uint32_t kMagic2 = 0x64006400u;

__device__ __forceinline__ half2v as_half2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

// Packed pair (1024 + z, 1024 + z) for an integer-valued fp16 zero point z.
__device__ __forceinline__ half2v zero_bias(_Float16 z) {
  _Float16 b = (_Float16)1024.0f + z;   // exact: z is an integer in 0..15
  half2v r = {b, b};
  return r;
}

// Eight codes of one word -> the eight exact fp16 values (q_j - z), j = 0..7.
// (1024 + q) - (1024 + z) is an exact fp16 subtraction of two integers.
__device__ __forceinline__ half8 decode_word(uint32_t w, half2v bias) {
  half2v p0 = as_half2((w & 0x000F000Fu) | kMagic2) - bias;
  half2v p1 = as_half2(((w >> 4) & 0x000F000Fu) | kMagic2) - bias;
  half2v p2 = as_half2(((w >> 8) & 0x000F000Fu) | kMagic2) - bias;
  half2v p3 = as_half2(((w >> 12) & 0x000F000Fu) | kMagic2) - bias;
  half8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

// 16 bytes from device memory as a global (not flat) load: flat loads count
// against both the vector-memory and the LDS wait counters and may complete
// out of order, so a pending one makes every later wait a full drain.
__device__ __forceinline__ half8 load_half8(const _Float16 *p) {
  typedef const __attribute__((address_space(1))) half8 *global_half8;
  return *(global_half8)(p);
}

__device__ __forceinline__ half8 zero_half8() {
  half8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  return z;
}

// D += A . B for one 16x16x32 fp16 MFMA with fp32 accumulation.  Lane l
// supplies A[l % 16][8(l/16) .. 8(l/16)+7] and B[8(l/16) .. +7][l % 16] and
// receives D[4(l/16) + v][l % 16], v = 0..3.
__device__ __forceinline__ float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The same MFMA on bf16 operands (the operands' bits as four 32-bit words).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4v mfma16_bf16(u32x4v a, u32x4v b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// bf16 <-> fp32 on raw 16-bit patterns (bf16 is the top half of an fp32)
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two floats to a bf16 pair (lo in the low half), each rounded to nearest
// even: one v_cvt_pk_bf16_f32, where two scalar conversions and a merge would
// take three instructions.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2x __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2x){lo, hi}, bf16x2));
}

// bf16 128.0 in both halves: OR-ing a 4-bit code q into the low mantissa bits
// gives the exact bf16 value 128 + q
constexpr uint32_t kMagicBF = 0x43004300u;

// Smallest fp16 value >= v for finite v > 0, built from the binary16 grid:
// below 2^-14 the grid step is 2^-24; in [2^e, 2^(e+1)) it is 2^(e-10).
// Returns false when that value would exceed the largest finite fp16.
__device__ inline bool fp16_ceil(double v, _Float16 *out) {
  if (!(v <= 65504.0)) return false;
  double step;
  if (v < 0x1p-14) {
    step = 0x1p-24;
  } else {
    int e;
    (void)frexp(v, &e);          // v = m * 2^e, m in [0.5, 1): v in [2^(e-1), 2^e)
    step = ldexp(1.0, e - 11);   // 2^((e-1) - 10)
  }
  const double h = ceil(v / step) * step;   // exact: step is a power of two
  if (h > 65504.0) return false;
  *out = (_Float16)h;                       // exact: h lies on the fp16 grid
  return true;
}

}  // namespace w4a16
