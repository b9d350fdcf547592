// Host-side launchers shared between the C-ABI front end and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// Bits of the packer's device status word.
constexpr unsigned kPackNonFinite = 1u;
constexpr unsigned kPackRange = 2u;

// Packs row blocks b0 .. b0 + nbw - 1 of the N x K matrix.  rmin/rmax (or
// null for per-group ranges): row n takes entry (n - 16 b0) * rstride.
hipError_t launch_pack(const void *W, const void *s, int N, int K, int b0, int nbw,
                       const uint8_t *keep, const double *rmin, const double *rmax, int rstride,
                       void *Wq, void *scales, void *zeros, unsigned *status, bool symmetric,
                       hipStream_t stream, bool w8 = false);
// Range of W / s (kept weights as 0) of rows n0 .. n0 + rows - 1 into
// rmin/rmax [rows].
hipError_t launch_row_range(const void *W, const void *s, int n0, int rows, int K,
                            const uint8_t *keep, double *rmin, double *rmax, hipStream_t stream);
// acc[0..1] = the least of rmin[0 .. rows) and the largest of rmax, combined
// with acc's earlier value unless `first` (and with 0 always).
hipError_t launch_tensor_range(int rows, const double *rmin, const double *rmax, double *acc,
                               bool first, hipStream_t stream);

// The weights kept in fp16 (validated by the caller): writes row_ptr [N + 1],
// col and val [count], and a keep bit mask in the workspace (returned in
// *mask) for launch_pack.  Blocks until done.  0 on success, -1 on a HIP error.
size_t outlier_workspace_bytes(int N, int K);
int select_outliers(const void *W, const void *s, int N, int K, long long count, int32_t *row_ptr,
                    int32_t *col, _Float16 *val, void *workspace, const uint8_t **mask,
                    hipStream_t stream);

// GPTQ quantize-and-pack (validated by the caller; blocks until done).  0 on
// success, 1 when rocBLAS / rocSOLVER cannot be loaded, 2 when the damped
// Hessian is not positive definite, -1 on a HIP or library error; non-finite
// inputs and scale overflow are flagged in *status as for launch_pack.
size_t gptq_workspace_bytes(int N, int K, long long n);
int gptq_pack(const void *W, const void *s, int N, int K, const void *X, long long n, double damp,
              void *Wq, void *scales, void *zeros, void *workspace, unsigned *status,
              hipStream_t stream);

// One dequantize-matmul problem (validated by the caller).
struct GemmDesc {
  const void *X, *Wq, *scales, *zeros, *s;
  void *Y;
  int M, N, K;
  // optional fp16 outliers, row-compressed (all set or all null)
  const void *o_row_ptr = nullptr, *o_col = nullptr, *o_val = nullptr;
  bool bf16 = false;  // X and Y are bf16 (else fp16)
  bool w8 = false;    // INT8 codes (2048-byte tiles), else INT4
  // streaming path, bf16: workspace for X * s prescaled once per call
  // (skinny_prescale_bytes(M, K) bytes), set by launch_skinny_set
  void *xpre = nullptr;
};

// Streaming kernel for small M (decode and speculative verify): M <= 16.
// launch_skinny_set runs up to skinny_max_problems() independent problems in
// one launch; X * s is staged in K windows when it does not fit in LDS whole,
// or always with force_window.  When the workspace holds
// skinny_workspace_bytes() for the same problems, bf16 problems that run in
// windows get X * s computed once by a small kernel first (else every
// workgroup computes its windows' share itself).
int skinny_max_problems();
size_t skinny_workspace_bytes(const GemmDesc *problems, int count);
hipError_t launch_skinny_set(const GemmDesc *problems, int count, hipStream_t stream,
                             bool force_window = false, void *workspace = nullptr,
                             size_t workspace_bytes = 0);
hipError_t launch_skinny(const void *X, const void *Wq, const void *scales, const void *zeros,
                         const void *s, void *Y, int M, int N, int K, hipStream_t stream);

// LDS-tiled MFMA GEMM for large M (batched decode and prefill): any M >= 1.
// launch_tiled_set runs up to tiled_max_problems() problems in one launch.
// When the workspace holds tiled_workspace_bytes() for the same problems, K
// is split across workgroups where that fills the GPU better (fp32 partials
// in the workspace, then a second launch adds them); otherwise (NULL, or too
// small) every output block walks all of K.
int tiled_max_problems();
size_t tiled_workspace_bytes(const GemmDesc *problems, int count);
hipError_t launch_tiled_set(const GemmDesc *problems, int count, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);
hipError_t launch_tiled(const void *X, const void *Wq, const void *scales, const void *zeros,
                        const void *s, void *Y, int M, int N, int K, hipStream_t stream);

// Speculative-sampling verification of B sequences (validated by the caller):
// the vocabulary is cut into spec_verify_chunks(V) chunks, and the workspace
// (spec_verify_workspace_bytes(B, V) bytes, 256-byte aligned) holds the
// per-chunk sums and the first rejection of every sequence.
int spec_verify_chunks(int V);
size_t spec_verify_workspace_bytes(int B, int V);
hipError_t launch_spec_verify(const float *p_target, const float *p_draft, const int32_t *draft,
                              const float *u_accept, const float *u_sample, int B, int K, int V,
                              void *workspace, int32_t *n_accepted, int32_t *token,
                              hipStream_t stream);

}  // namespace w4a16
