// GPTQ-style quantize-and-pack: the same packed INT4 format, with each weight's
// quantization error spread over the not yet quantized weights of its row.
//
// "Chapter 22: Advanced inference optimisation" (aiwing.uk), section 22.3,
// GPTQ: minimise ||W X - W_hat X||_F^2 for the layer's input activations X on
// calibration data, using the Hessian H = 2 X X^T to compensate each
// quantized weight's error on the rest of its row.  Steps, in fp64:
//   1. X' = X diag(s) (calibration rows of K features; s the AWQ scale);
//   2. H = 2 X'^T X' (a library GEMM), plus damp * mean(diag H) on the diagonal;
//   3. H^-1 from its Cholesky factorisation, then the upper Cholesky factor U of
//      H^-1 (H^-1 = U^T U) -- library factorisations (rocSOLVER);
//   4. W' = W / s;
//   5. for each group of 128 columns, in order: sweep_kernel forms the group's
//      scale and zero point from the current W' (rules of the plain packer),
//      then, column by column, codes each weight, takes err = (w - dequant) /
//      U[k][k] and subtracts err * U[k][j] from the group's later columns j;
//      it writes the packed tile, the metadata and the errors of the group;
//      the rest of every row then takes all 128 errors at once, W'[:, after]
//      -= E . U[group, after] (a library GEMM).
// Columns go in their natural order, so every group keeps its 128 consecutive
// columns.  rocBLAS and rocSOLVER are loaded on the first call (dlopen), so
// the rest of the library does not depend on them.
#include <dlfcn.h>

#include <cmath>
#include <mutex>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSweepWaves = kTileRows;  // one wave per row of a row block

// X' = X * s in fp64, row-major [n][K]
__global__ __launch_bounds__(256) void scale_x_kernel(const _Float16 *__restrict__ X,
                                                      const _Float16 *__restrict__ s, long long n,
                                                      int K, double *__restrict__ Xs) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n * K;
       i += (long long)gridDim.x * 256) {
    const int k = (int)(i % K);
    Xs[i] = (double)X[i] * (s ? (double)s[k] : 1.0);
  }
}

// W' = W / s in fp64 (one correctly rounded division), row-major [N][K];
// non-finite W or s, or s <= 0, set kPackNonFinite in *status
__global__ __launch_bounds__(256) void scale_w_kernel(const _Float16 *__restrict__ W,
                                                      const _Float16 *__restrict__ s, long long total,
                                                      int K, double *__restrict__ Wp,
                                                      unsigned *__restrict__ status) {
#pragma clang fp contract(off)
  unsigned bad = 0;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (long long)gridDim.x * 256) {
    const double w = (double)W[i], sv = s ? (double)s[i % K] : 1.0;
    if (!std::isfinite(w) || !std::isfinite(sv) || !(sv > 0.0)) bad = kPackNonFinite;
    Wp[i] = w / sv;
  }
  if (bad) atomicOr(status, bad);
}

// diag(H) += damp * mean(diag(H)); one workgroup
__global__ __launch_bounds__(256) void damp_kernel(double *__restrict__ H, int K, double damp) {
  __shared__ double red[4];
  double v = 0.0;
  for (int k = threadIdx.x; k < K; k += 256) v += H[(size_t)k * K + k];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const double add = damp * ((red[0] + red[1]) + (red[2] + red[3])) / K;
  __syncthreads();
  for (int k = threadIdx.x; k < K; k += 256) H[(size_t)k * K + k] += add;
}

// copy the lower triangle (column-major) over the upper one
__global__ __launch_bounds__(256) void symmetrize_kernel(double *__restrict__ A, int K) {
  const long long total = (long long)K * K;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (long long)gridDim.x * 256) {
    const int col = (int)(i / K), row = (int)(i % K);
    if (row < col) A[i] = A[(size_t)row * K + col];  // (row, col) <- (col, row)
  }
}

// One group (128 columns from k0) of one row block (16 rows): wave w owns row
// n = 16 b + w, lane l its columns k0 + l and k0 + 64 + l.  U (row-major view,
// upper) supplies U[k][j]; its 128 x 128 block sits in LDS.
__global__ __launch_bounds__(kSweepWaves * 64) void sweep_kernel(
    double *__restrict__ Wp, const double *__restrict__ U, int N, int K, int g,
    u32x4 *__restrict__ Wq, _Float16 *__restrict__ scales, _Float16 *__restrict__ zeros,
    double *__restrict__ E, unsigned *__restrict__ status) {
#pragma clang fp contract(off)
  __shared__ double Ub[kGroup][kGroup];
  __shared__ uint8_t codes[kSweepWaves][kGroup];
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k0 = g * kGroup, G = K / kGroup, NB = N / kTileRows;
  for (int i = threadIdx.x; i < kGroup * kGroup; i += kSweepWaves * 64)
    Ub[i / kGroup][i % kGroup] = U[(size_t)(k0 + i / kGroup) * K + k0 + i % kGroup];
  const int n = b * kTileRows + wave;
  double *row = Wp + (size_t)n * K + k0;
  double w0 = row[lane], w1 = row[64 + lane];
  __syncthreads();

  // the group's range (containing 0) from the current weights -> scale, zero point
  double mn = fmin(fmin(w0, w1), 0.0), mx = fmax(fmax(w0, w1), 0.0);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, o));
    mx = fmax(mx, __shfl_xor(mx, o));
  }
  const double range = mx - mn;
  _Float16 sc16 = 0, z16 = 0;
  double scale = 1.0, z = 0.0;
  const bool live = range > 0.0;
  if (live) {
    if (!fp16_ceil(range / 15.0, &sc16)) {
      if (lane == 0) atomicOr(status, kPackRange);
      sc16 = 0;
    } else {
      scale = (double)sc16;
      z = rint(-mn / scale);
      z16 = (_Float16)(int)z;
    }
  }

  // column by column: code, error, compensation of the group's later columns
  for (int k = 0; k < kGroup; ++k) {
    const double wk = __shfl(k < 64 ? w0 : w1, k & 63);
    double code = 0.0, deq = 0.0;
    if (live) {
      code = rint(wk / scale) + z;
      code = code < 0.0 ? 0.0 : (code > 15.0 ? 15.0 : code);
      deq = (code - z) * scale;
    }
    const double err = (wk - deq) / Ub[k][k];
    if (lane == (k & 63)) {
      codes[wave][k] = (uint8_t)code;
      E[(size_t)n * kGroup + k] = err;
    }
    if (lane > k) w0 -= err * Ub[k][lane];
    if (64 + lane > k) w1 -= err * Ub[k][64 + lane];
  }
  __syncthreads();

  // the packed tile: lane L = 16c + r takes row r, columns 32t + 8c + j
  if (wave == 0) {
    const int c = lane >> 4, r = lane & 15;
    u32x4 out;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        word |= (uint32_t)codes[r][32 * t + 8 * c + j] << (4 * ((j >> 1) + 4 * (j & 1)));
      out[t] = word;
    }
    Wq[((size_t)g * NB + b) * 64 + lane] = out;
  }
  if (lane == 0) {
    scales[meta_index(n, g, NB)] = sc16;
    zeros[meta_index(n, g, NB)] = z16;
    if (g == G - 1)
      for (int p = G; p < meta_groups(G); ++p) {  // the row's padding slots
        scales[meta_index(n, p, NB)] = (_Float16)0;
        zeros[meta_index(n, p, NB)] = (_Float16)0;
      }
  }
}

// ---- the libraries, loaded once
struct Solver {
  void *blas = nullptr, *solver = nullptr;
  int (*create)(void **) = nullptr;
  int (*destroy)(void *) = nullptr;
  int (*set_stream)(void *, hipStream_t) = nullptr;
  int (*dgemm)(void *, int, int, int, int, int, const double *, const double *, int,
               const double *, int, const double *, double *, int) = nullptr;
  int (*potrf)(void *, int, int, double *, int, int *) = nullptr;
  int (*potri)(void *, int, int, double *, int, int *) = nullptr;
  bool ok = false;
};
constexpr int kOpN = 111, kOpT = 112, kFillUpper = 121, kFillLower = 122;  // rocBLAS enums

Solver &solver() {
  static Solver S;
  static std::once_flag once;
  std::call_once(once, [] {
    const char *blas_names[] = {"librocblas.so.5", "librocblas.so"};
    const char *solver_names[] = {"librocsolver.so.0", "librocsolver.so"};
    for (const char *nm : blas_names)
      if (!S.blas) S.blas = dlopen(nm, RTLD_NOW | RTLD_LOCAL);
    for (const char *nm : solver_names)
      if (!S.solver) S.solver = dlopen(nm, RTLD_NOW | RTLD_LOCAL);
    if (!S.blas || !S.solver) return;
    S.create = reinterpret_cast<decltype(S.create)>(dlsym(S.blas, "rocblas_create_handle"));
    S.destroy = reinterpret_cast<decltype(S.destroy)>(dlsym(S.blas, "rocblas_destroy_handle"));
    S.set_stream = reinterpret_cast<decltype(S.set_stream)>(dlsym(S.blas, "rocblas_set_stream"));
    S.dgemm = reinterpret_cast<decltype(S.dgemm)>(dlsym(S.blas, "rocblas_dgemm"));
    S.potrf = reinterpret_cast<decltype(S.potrf)>(dlsym(S.solver, "rocsolver_dpotrf"));
    S.potri = reinterpret_cast<decltype(S.potri)>(dlsym(S.solver, "rocsolver_dpotri"));
    S.ok = S.create && S.destroy && S.set_stream && S.dgemm && S.potrf && S.potri;
  });
  return S;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t gptq_workspace_bytes(int N, int K, long long n) {
  return align256((size_t)n * K * 8) + align256((size_t)K * K * 8) + align256((size_t)N * K * 8) +
         align256((size_t)N * kGroup * 8) + 256;
}

int gptq_pack(const void *W, const void *s, int N, int K, const void *X, long long n, double damp,
              void *Wq, void *scales, void *zeros, void *workspace, unsigned *status,
              hipStream_t st) {
  Solver &S = solver();
  if (!S.ok) return 1;  // libraries missing
  char *ws = static_cast<char *>(workspace);
  double *Xs = reinterpret_cast<double *>(ws);
  double *H = reinterpret_cast<double *>(ws + align256((size_t)n * K * 8));
  double *Wp = reinterpret_cast<double *>(reinterpret_cast<char *>(H) + align256((size_t)K * K * 8));
  double *E = reinterpret_cast<double *>(reinterpret_cast<char *>(Wp) + align256((size_t)N * K * 8));
  int *info = reinterpret_cast<int *>(reinterpret_cast<char *>(E) + align256((size_t)N * kGroup * 8));
  const _Float16 *Wh = static_cast<const _Float16 *>(W), *sh = static_cast<const _Float16 *>(s);

  void *h = nullptr;
  if (S.create(&h) != 0) return -1;
  int rc = 0;
  auto fail = [&](bool bad) {
    if (bad && !rc) rc = -1;
    return rc != 0;
  };
  if (!fail(S.set_stream(h, st) != 0)) {
    const int grid = 2048;
    hipLaunchKernelGGL(scale_x_kernel, dim3(grid), dim3(256), 0, st, static_cast<const _Float16 *>(X),
                       sh, n, K, Xs);
    hipLaunchKernelGGL(scale_w_kernel, dim3(grid), dim3(256), 0, st, Wh, sh, (long long)N * K, K, Wp,
                       status);
    fail(hipGetLastError() != hipSuccess);
    // H = 2 X'^T X': X' row-major [n][K] is column-major K x n (ld K)
    const double two = 2.0, zero = 0.0, one = 1.0, minus = -1.0;
    if (!rc) fail(S.dgemm(h, kOpN, kOpT, K, K, (int)n, &two, Xs, K, Xs, K, &zero, H, K) != 0);
    if (!rc) {
      hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, st, H, K, damp);
      fail(hipGetLastError() != hipSuccess);
    }
    // H^-1 (lower triangle, column-major), made symmetric, then its lower
    // Cholesky factor L: read row-major, L^T = U is upper with H^-1 = U^T U
    if (!rc) fail(S.potrf(h, kFillLower, K, H, K, info) != 0);
    if (!rc) fail(S.potri(h, kFillLower, K, H, K, info + 1) != 0);
    if (!rc) {
      hipLaunchKernelGGL(symmetrize_kernel, dim3(grid), dim3(256), 0, st, H, K);
      fail(hipGetLastError() != hipSuccess);
    }
    if (!rc) fail(S.potrf(h, kFillLower, K, H, K, info + 2) != 0);
    const double *U = H;
    const int G = K / kGroup, NB = N / kTileRows;
    for (int g = 0; g < G && !rc; ++g) {
      hipLaunchKernelGGL(sweep_kernel, dim3(NB), dim3(kSweepWaves * 64), 0, st, Wp, U, N, K, g,
                         static_cast<u32x4 *>(Wq), static_cast<_Float16 *>(scales),
                         static_cast<_Float16 *>(zeros), E, status);
      if (fail(hipGetLastError() != hipSuccess)) break;
      const int k1 = (g + 1) * kGroup;
      if (k1 < K)  // W'^T[k1.., :] -= U[group, k1..]^T-view . E^T-view
        fail(S.dgemm(h, kOpN, kOpN, K - k1, N, kGroup, &minus, U + (size_t)g * kGroup * K + k1, K,
                     E, kGroup, &one, Wp + k1, K) != 0);
    }
  }
  int host_info[3] = {0, 0, 0};
  if (!rc && hipMemcpyAsync(host_info, info, sizeof(host_info), hipMemcpyDeviceToHost, st) != hipSuccess)
    rc = -1;
  if (hipStreamSynchronize(st) != hipSuccess) rc = -1;
  S.destroy(h);
  if (rc) return rc;
  if (host_info[0] || host_info[1] || host_info[2]) return 2;  // not positive definite
  return 0;
}

}  // namespace w4a16
