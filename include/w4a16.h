/*
 * w4a16.h -- weight-only INT4 per-group quantization and the fused
 * dequantize-matmul, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are web pages, cited by title and section):
 *
 *  - "Chapter 22: Advanced inference optimisation" (aiwing.uk), section 22.3,
 *    AWQ paragraph and its equation: the weight is divided by a per-input-
 *    channel activation magnitude s before it is quantized, and the quantized
 *    value is multiplied by s again:  W_hat = quant(W / s) * s.
 *  - The nano-vllm tutorial (discosf.com), section 2.1: quant() maps the
 *    float range of a group onto the integer range with a scale and a zero
 *    point; per-group granularity with 128 elements per group is the usual
 *    choice for 4-bit GPTQ/AWQ.  Section 2.3: the scale and zero point travel
 *    with the weights, and the loader either dequantizes or feeds operators
 *    that take the low-precision weights directly.
 *  - Same chapter 22, section 22.3, weight-only paragraph: activations stay in
 *    FP16 and the product is the plain matmul against the dequantized
 *    weights; a mixed-precision kernel only computes it faster.
 *
 * Readings where the pages leave a step open (all taken identically by the
 * library and by the CPU reference it is tested against):
 *  - codes are unsigned 4-bit 0..15 with an integer zero point z (0..15)
 *    stored as fp16, and dequantization is (q - z) * scale;
 *  - a group is 128 consecutive input features (K) of one output row (N);
 *  - the group range is [min(0, min W'), max(0, max W')] with W' = W / s;
 *    scale = range / 15 rounded UP to the next fp16 value; z = rint(-min /
 *    scale); q = clamp(rint(W' / scale) + z, 0, 15); rint ties to even; all
 *    of it in fp64 with one correctly rounded division per quotient;
 *  - an all-zero group has scale 0, zero point 0 and codes 0.
 *
 * Shapes: W is [N][K] (output x input features, like a linear layer's
 * weight), X is [M][K], Y = X . W_hat^T is [M][N].  K must be a multiple of
 * 128, N a multiple of 16, N and K at most 2^24, and the packed codes of one
 * matrix (N*K/2 bytes) under 2 GiB - 1 MiB.  fp16 means IEEE binary16.
 *
 * Packed layout (this library's own; the pages only fix the content):
 *  - Wq: N*K/2 bytes.  Tile (b, g) covers rows 16b..16b+15 and the 128
 *    columns of group g; it is 1024 bytes at byte offset (g*NB + b)*1024,
 *    NB = N/16 (group-major: the tiles of one group are contiguous, which
 *    spreads the concurrent streams of neighbouring row blocks over memory
 *    channels).  Inside a tile, lane L = 16c + r (row r, column octet c =
 *    0..3) owns the 16 bytes at 16L: four little-endian 32-bit words, word t
 *    holding the codes of columns 128g + 32t + 8c + j, j = 0..7, with column
 *    j in the 4-bit slot i (bits 4i..4i+3) where j = 2*(i % 4) + i / 4.
 *    One 64-lane wave therefore reads a whole tile with one 128-bit load per
 *    lane, and word t of a lane is exactly that lane's B operand of a
 *    16x16x32 fp16 MFMA.
 *  - scales, zeros: fp16, in quads of 4 groups.  With G = K/128 and
 *    Gq = ceil(G / 4), the value of row n = 16b + r and group g = 4u + i is
 *    element ((u*NB + b)*16 + r)*4 + i; each buffer holds N*4*Gq elements,
 *    and the slots of groups G..4*Gq-1 are zero.  The metadata of one 16-row
 *    block and 4 consecutive groups is thus one contiguous 128-byte run, and
 *    the runs of one quad follow each other row block after row block.
 *
 * Ownership and streams: the caller allocates and owns every buffer (device
 * memory unless noted) and passes a hipStream_t as `stream` (NULL = the null
 * stream).  All pointers must be 16-byte aligned.  The packers' status word
 * and row-range scratch (about 512 KB) are a device array of the library's own
 * code object, one copy per GPU, held until the process ends; the packers
 * (w4a16_quantize_pack*) share it and run one at a time within a process
 * (each call blocks anyway).  The library allocates nothing, except that the
 * GPTQ packer's rocBLAS and rocSOLVER calls manage memory of their own.
 *
 * Errors: every argument is validated on the host before any HIP call, so an
 * invalid call returns its status without touching the GPU.  Status codes are
 * the W4A16_* values below; w4a16_strerror() names them.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_GROUP 128      /* elements per quantization group along K     */
#define W4A16_TILE_ROWS 16   /* rows of W per packed tile (N % 16 == 0)      */

enum {
  W4A16_OK = 0,
  W4A16_EINVAL = -1,       /* NULL pointer, M/N/K out of range, K % 128, N % 16 */
  W4A16_EALIGN = -2,       /* a pointer is not 16-byte aligned                  */
  W4A16_EUNSUPPORTED = -3, /* unknown kernel path or quantization mode requested */
  W4A16_ENONFINITE = -4,   /* NaN/Inf in W or s, or some s <= 0 (packer)        */
  W4A16_ERANGE = -5,       /* a group scale rounds up past the fp16 range       */
  W4A16_EHIP = -6,         /* a HIP runtime call or kernel launch failed        */
  W4A16_ESCRATCH = -7      /* w4a16_gemm_grouped_static: the call needs more
                              workspace than W4A16_STATIC_SCRATCH_BYTES         */
};

/* Kernel choice for w4a16_gemm_path(); w4a16_gemm() always uses AUTO. */
enum {
  W4A16_PATH_AUTO = 0,     /* pick by M (decode / verify / prefill)               */
  W4A16_PATH_SKINNY = 1,   /* streaming split-K MFMA kernel, M <= 16 per pass     */
  W4A16_PATH_TILED = 2,    /* LDS-tiled MFMA GEMM for large M                     */
  W4A16_PATH_SKINNY_WINDOW = 3 /* streaming kernel with X*s staged in K windows;
                              SKINNY takes it by itself when X*s of the whole
                              row does not fit in LDS (long K at M > 1)        */
};

/* Byte sizes of the three packed buffers of an [N][K] weight (host outputs).
 * wq = N*K/2, scales = zeros = 2*N*4*ceil(K/512).  EINVAL on bad shapes or
 * NULL. */
int w4a16_packed_sizes(int64_t N, int64_t K, size_t *wq_bytes, size_t *scales_bytes,
                       size_t *zeros_bytes);

/* Quantize and pack (offline step; chapter 22 section 22.3 notes weights are
 * quantized offline).  W: fp16 [N][K] row-major.  s: fp16 [K] AWQ scale, or
 * NULL for s = 1.  Writes Wq, scales, zeros in the layout above.  Blocks on
 * `stream` before returning so that it can report ENONFINITE (non-finite W or
 * s, or s <= 0) or ERANGE (a group's fp16 scale would overflow); on such an
 * error the outputs hold unspecified values. */
int w4a16_quantize_pack(const void *W, const void *s, int64_t N, int64_t K, void *Wq,
                        void *scales, void *zeros, void *stream);

/* Quantization grids and granularities for w4a16_quantize_pack_mode(). */
enum {
  W4A16_QUANT_ASYM = 0,         /* the readings above (w4a16_quantize_pack)        */
  W4A16_QUANT_SYM = 1,          /* signed -7..7 around a constant zero point 8     */
  W4A16_QUANT_ASYM_CHANNEL = 2, /* asymmetric, one scale/zero per row (channel)    */
  W4A16_QUANT_ASYM_TENSOR = 3,  /* asymmetric, one scale/zero for the whole tensor */
  W4A16_QUANT_ASYM8 = 4         /* INT8 codes 0..255 (W8A16), group 128            */
};

/* Quantize and pack on a chosen grid; same arguments, layout, blocking and
 * errors as w4a16_quantize_pack, plus `mode` (EUNSUPPORTED if unknown).
 * W4A16_QUANT_SYM is the signed 4-bit grid of the practitioner notes at
 * mhpq.cn, section 2.1 (INT4 spans -7..7): per group, scale = max|W'| / 7
 * rounded UP to fp16 (so no code clamps), signed code rint(W' / scale) (ties
 * to even) stored as code + 8, zero point 8; an all-zero group stores scale 0
 * and codes 8.  The packed buffers are in the same layout and feed the same
 * GEMM entry points: (q - z) * scale reproduces the signed value.
 * W4A16_QUANT_ASYM_CHANNEL and W4A16_QUANT_ASYM_TENSOR are the per-channel and
 * per-tensor granularities of the nano-vllm tutorial (discosf.com, section
 * 2.1): the range [min(0, min W'), max(0, max W')] is taken over the row or
 * over the whole tensor instead of the group, and every group slot of the row
 * repeats the resulting scale and zero point (same layout, same kernels).
 * W4A16_QUANT_ASYM8 is the INT8 (W8A16) variant ("Chapter 22", aiwing.uk,
 * section 22.3's table: INT8 at one byte per parameter): the same rules with
 * codes 0..255 (scale = range / 255 rounded up), one byte per weight in
 * 2048-byte tiles -- tile (b, g) at (g * NB + b) * 2048, lane L = 16 c + r at
 * 32 L, its byte 8 t + j holding column 128 g + 32 t + 8 c + j -- and the same
 * metadata layout.  Wq holds N * K bytes (w4a16_packed_sizes_mode); the GEMM
 * reads it with w4a16_problem.wbits = 8. */
int w4a16_packed_sizes_mode(int64_t N, int64_t K, int mode, size_t *wq_bytes, size_t *scales_bytes,
                            size_t *zeros_bytes);
int w4a16_quantize_pack_mode(const void *W, const void *s, int64_t N, int64_t K, int mode,
                             void *Wq, void *scales, void *zeros, void *stream);

/* FP16 outlier side path (the practitioner notes at mhpq.cn, section 2.2,
 * outlier handling: the top 0.1% of the weights by magnitude stay in FP16,
 * the rest go to INT4, merged as where(mask, fp16, int4)).
 * Keeps exactly `count` weights of W in fp16 -- the largest |W[n][k] / s[k]|
 * (|W| when s is NULL; one correctly rounded fp64 division, so the ranking is
 * exact), ties to the lower flat index n * K + k -- and quantizes and packs
 * the rest exactly as w4a16_quantize_pack_mode would (any mode, INT8 codes
 * included) with the kept weights replaced by 0: they leave their groups'
 * ranges and their codes decode to exactly 0.  The kept weights are written
 * row-compressed:
 *   o_row_ptr int32 [N + 1] (o_row_ptr[0] = 0, o_row_ptr[N] = count),
 *   o_col int32 [count] and o_val fp16 [count]: the columns (increasing
 *   within a row) and the original fp16 values of row n at
 *   o_row_ptr[n] .. o_row_ptr[n + 1] - 1.
 * The page's share is count = round(0.001 * N * K).  0 <= count <= N * K and
 * count < 2^31 (EINVAL); o_col and o_val may be NULL when count = 0.
 * workspace: caller-owned device memory of w4a16_outlier_workspace_size()
 * bytes (EINVAL if smaller), 256-byte aligned; contents on entry do not
 * matter.  Alignment (EALIGN): W, Wq, scales, zeros, s 16 bytes, o_row_ptr
 * and o_col 4, o_val 2.  Blocks until done; errors as w4a16_quantize_pack
 * (ENONFINITE also for a non-finite kept weight).  The packed buffers feed
 * the GEMM entry points together with the three outlier arrays
 * (w4a16_problem's o_row_ptr, o_col, o_val). */
int w4a16_outlier_workspace_size(int64_t N, int64_t K, size_t *bytes);
int w4a16_quantize_pack_outliers(const void *W, const void *s, int64_t N, int64_t K, int mode,
                                 int64_t count, void *Wq, void *scales, void *zeros,
                                 void *o_row_ptr, void *o_col, void *o_val, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* GPTQ-style quantize-and-pack ("Chapter 22: Advanced inference
 * optimisation", aiwing.uk, section 22.3: minimise ||W X - W_hat X||_F^2 for
 * calibration activations X, with H = 2 X X^T spreading each quantized
 * weight's error over the rest of its row).  Same packed output as
 * w4a16_quantize_pack (asymmetric grid, group 128, AWQ s optional).
 *   X: fp16 [n_samples][K] calibration activations (device, 16-byte aligned);
 *   the Hessian is H = 2 (X s)^T (X s) in fp64, plus damp * mean(diag H) on its
 *   diagonal (damp >= 0, typically 0.01); columns are quantized in their
 *   natural order; error compensation uses the upper Cholesky factor U of H^-1
 *   (H^-1 = U^T U); each group's scale and zero point come from its current
 *   (compensated) weights when the group starts, by the packer's rules.
 * All arithmetic is fp64.  The Cholesky factorisations use rocSOLVER and the
 * two large products rocBLAS, loaded on the first call: EUNSUPPORTED if they
 * cannot be loaded.  EINVAL also when the damped Hessian is not positive
 * definite.  Limits: K <= 65536, 1 <= n_samples <= 2^24, n_samples * K <= 2^32.
 * workspace: caller-owned device memory of w4a16_gptq_workspace_size() bytes,
 * 256-byte aligned (about 8 * (n_samples * K + K * K + N * K) bytes).
 * Blocks until done; other errors as w4a16_quantize_pack. */
int w4a16_gptq_workspace_size(int64_t N, int64_t K, int64_t n_samples, size_t *bytes);
int w4a16_quantize_pack_gptq(const void *W, const void *s, int64_t N, int64_t K, const void *X,
                             int64_t n_samples, double damp, void *Wq, void *scales, void *zeros,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Y[M][N] = X[M][K] . W_hat^T with W_hat[n][k] = (q - z) * scale * s[k].
 * X: fp16 [M][K]; Wq/scales/zeros: packed as above; s: fp16 [K] or NULL;
 * Y: fp16 [M][N] row-major, fully overwritten.  fp32 accumulation; X * s is
 * rounded to fp16 once.  Asynchronous on `stream`.  M >= 0 (0: nothing).
 * The same operation and bits as w4a16_gemm_grouped_ws on this one problem
 * with its queried workspace, which this call takes from the library's
 * shared scratch (below) when it fits; otherwise (or under stream capture)
 * K is not split across workgroups and the bits are those of
 * w4a16_gemm_path(..., W4A16_PATH_AUTO, ...). */
int w4a16_gemm(const void *X, const void *Wq, const void *scales, const void *zeros,
               const void *s, void *Y, int64_t M, int64_t N, int64_t K, void *stream);

/* The shared scratch of the entry points without a workspace argument
 * (w4a16_gemm, w4a16_gemm_grouped): W4A16_SHARED_SCRATCH_BYTES of device
 * memory inside the library on each GPU it runs on (held from the first such
 * call there until the process ends), for split-K partial sums and prescaled
 * activations of calls that need at most that much workspace (batched
 * decode; a 70B prefill matrix with an AWQ s needs more and runs without).
 * Such calls on one GPU are ordered through an event the library keeps per
 * GPU: each waits on its stream for the previous one's work, whatever stream
 * that ran on, so they never race; their work does not overlap in time.  A
 * call on a stream that is being captured does not use the scratch. */
#define W4A16_SHARED_SCRATCH_BYTES ((size_t)32 << 20)

/* Same as w4a16_gemm with an explicit kernel path (tests and benchmarks); it
 * never uses a workspace, so large-M problems are not split across
 * workgroups. */
int w4a16_gemm_path(const void *X, const void *Wq, const void *scales, const void *zeros,
                    const void *s, void *Y, int64_t M, int64_t N, int64_t K, int path,
                    void *stream);

/* One independent dequantize-matmul of a grouped call; fields as in
 * w4a16_gemm (device pointers; s may be NULL; M may be 0). */
typedef struct w4a16_problem {
  const void *X;
  const void *Wq;
  const void *scales;
  const void *zeros;
  const void *s;
  void *Y;
  int64_t M, N, K;
  /* Optional fp16 outliers (w4a16_quantize_pack_outliers), all NULL or all
   * set: W_hat[n][k] = o_val[e] where o_col[e] = k for some e in
   * o_row_ptr[n] .. o_row_ptr[n + 1] - 1 (the codes there decode to 0), so
   * Y = X . W_hat^T gains X[m][k] * o_val[e] per kept weight, summed in fp32
   * in stored order into the output before its rounding.  o_row_ptr int32
   * [N + 1] and o_col int32 4-byte aligned, o_val fp16 2-byte aligned. */
  const void *o_row_ptr;
  const void *o_col;
  const void *o_val;
  /* Activation type of X and Y: W4A16_DTYPE_F16 (0, the default of a zeroed
   * struct) or W4A16_DTYPE_BF16 (1); s and the packed weights stay fp16.  With
   * bf16, X * s is rounded to bf16 once, the streaming kernels multiply the
   * exact codes and apply scale and zero point in fp32 per group, and the tiled
   * kernel rounds each dequantized weight to bf16 once (fp32 accumulation
   * throughout; Y rounded to bf16 once).  Another value is EUNSUPPORTED. */
  int32_t dtype;
  /* Code width: 0 or 4 (INT4, the default) or 8 (INT8 codes packed by
   * W4A16_QUANT_ASYM8, N * K bytes, the same size limit as the INT4 code
   * bytes else EINVAL), with fp16 or bf16 activations and with or without
   * fp16 outliers; any other width is EUNSUPPORTED. */
  int32_t wbits;
} w4a16_problem;

enum { W4A16_DTYPE_F16 = 0, W4A16_DTYPE_BF16 = 1 };

/* Several independent dequantize-matmuls, each the operation w4a16_gemm
 * computes, in as few launches as possible (with the shared scratch, above,
 * as the workspace of w4a16_gemm_grouped_ws when it fits, else none): problems that the M-dispatch
 * sends to the streaming kernel (small M) share one launch, up to 8 problems
 * per launch, so a layer's small projections ride along with its large ones;
 * the others get a launch each.  How a shared launch splits K across waves,
 * and whether it stages X * s in K windows, depends on all of its problems,
 * so the fp32 summation order (and the last bit of a result) can differ from
 * a single w4a16_gemm call; the same call always gives the same bits.  `problems` is a host array of
 * `count` entries (count 0 is a no-op).  Every problem is validated first; on
 * an error nothing is launched.  Outputs must not overlap each other or any
 * input.  Asynchronous on `stream`. */
int w4a16_gemm_grouped(const w4a16_problem *problems, int count, void *stream);

/* Bytes of device workspace that lets w4a16_gemm_grouped_ws split K across
 * workgroups and prescale bf16 activations for these problems (host only; no
 * GPU call).  0 when no problem benefits (fp16 streaming-path problems, and
 * tiled-path calls whose output blocks already fill the GPU).  Validates like
 * w4a16_gemm_grouped; *bytes is a host pointer. */
int w4a16_gemm_workspace_size(const w4a16_problem *problems, int count, size_t *bytes);

/* w4a16_gemm_grouped with a caller-owned device workspace.  Step 7 of the
 * method (the K reduction) may then run across workgroups: for large-M
 * problems whose output blocks are too few to fill the GPU (batched decode;
 * small projections), each of S K-ranges writes fp32 partial sums to the
 * workspace, and a second kernel adds the S partials in a fixed order and
 * rounds to fp16 once, so results are reproducible run to run (they may
 * differ in the last bit from an unsplit call).  For bf16 streaming-path
 * problems whose X * s is staged in K windows, a small first kernel computes
 * bf16(X * s) and its group sums once into the workspace, and the GEMM kernel
 * copies them instead of recomputing them in every workgroup (the same
 * values, so the results are identical).  The workspace needs no
 * initialisation, must hold w4a16_gemm_workspace_size() bytes for the same
 * problems (else, or when NULL, K is not split), must be 16-byte aligned
 * (EALIGN), must not overlap any input or output, and may be reused as soon
 * as the call's work on `stream` has completed.  Asynchronous on `stream`. */
int w4a16_gemm_grouped_ws(const w4a16_problem *problems, int count, void *workspace,
                          size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * w4a16_gemm_grouped_ws with its workspace taken from a device array inside
 * the library instead of a caller argument.  The array holds
 * W4A16_STATIC_SCRATCH_BYTES (64 MiB) on each GPU the library runs on, from
 * the first call there until the process ends; a call calls no hipMalloc,
 * hipFree or allocating library routine.  A call whose
 * w4a16_gemm_workspace_size() exceeds the array returns W4A16_ESCRATCH
 * without launching anything (checked on the host); other arguments and
 * errors as w4a16_gemm_grouped_ws, and the results are the bits that call
 * gives with a workspace of the queried size.  Every call on a GPU shares
 * that GPU's array (nothing in it needs to start at zero): calls on one GPU
 * whose work overlaps in time -- on different streams, or from different host
 * threads without ordering -- race, and their results are undefined.
 * Asynchronous on `stream`. */
#define W4A16_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int w4a16_gemm_grouped_static(const w4a16_problem *problems, int count, void *stream);

/* Speculative-sampling verification: the accept / reject step that consumes a
 * verify pass ("Chapter 22: Advanced inference optimisation", aiwing.uk,
 * section 22.1).  For each of B sequences: draft token x_i (i < K) is
 * accepted if u_i <= p_target(x_i) / p_draft(x_i); at the first rejection
 * one token is drawn from normalize(max(0, p_target_i - p_draft_i)) and the
 * later drafts are dropped; after K acceptances one more token is drawn from
 * the target distribution of position K.
 *   p_target fp32 [B][K+1][V], p_draft fp32 [B][K][V] (probabilities, not
 *   necessarily normalised; NaN and negatives count as 0), draft int32 [B][K]
 *   token ids (an id outside 0..V-1 is rejected), u_accept fp32 [B][K] and
 *   u_sample fp32 [B] uniforms in [0, 1) supplied by the caller, all
 *   row-major and contiguous.
 *   Outputs: n_accepted int32 [B] (0..K) and token int32 [B] (the drawn
 *   token, or -1 if the row it is drawn from has no mass).
 * Every decision is exact: the test is u * p_draft <= p_target in fp64; a draw
 * is an inverse-CDF draw in fixed point, with fx(p) = floor(p * 2^40), weights
 * fx(p_target) for the target row and fx(max(0, p_target - p_draft)) for the
 * corrected residual (the difference formed in fp64 from the two fp32 values),
 * exact integer sums, and threshold
 * (floor(u' * 2^32) * S) >> 32 (u' clamped to [0, 1), NaN as 0), taking the
 * smallest id whose inclusive prefix sum exceeds it; with no mass in the
 * residual the target row of that position is used.
 * Limits (EINVAL beyond them): K <= 1024, V and B <= 2^24, B * (K+1) * V <=
 * 2^40, B * ceil(V / 4096) < 2^24.  Rows whose entries sum to 2^12 or more
 * (infinities included) are outside the contract: the call still ends and
 * writes only its outputs, whose values are then unspecified.
 * workspace: caller-owned device memory of at least the size
 * w4a16_spec_verify_workspace_size reports, 256-byte aligned (EALIGN), not
 * cleared by the caller; calls that share a workspace must not overlap.
 * Device pointers, 4-byte aligned (EALIGN); p_draft, draft and u_accept may be
 * NULL when K = 0; B = 0 is a no-op.  Asynchronous on `stream` (two launches). */
int w4a16_spec_verify_workspace_size(int64_t B, int64_t K, int64_t V, size_t *bytes);
int w4a16_spec_verify(const void *p_target, const void *p_draft, const void *draft,
                      const void *u_accept, const void *u_sample, int64_t B, int64_t K, int64_t V,
                      void *workspace, size_t workspace_bytes, void *n_accepted, void *token,
                      void *stream);

/* Which path AUTO takes for this shape (host only; no GPU call). */
int w4a16_select_path(int64_t M, int64_t N, int64_t K);

/* Static description of a status code. */
const char *w4a16_strerror(int status);

/* Library ABI version (major * 100 + minor). */
int w4a16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
