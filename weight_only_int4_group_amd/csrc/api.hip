// C-ABI front end: argument validation (host only, before any HIP call),
// kernel choice by M, and launches on the caller's stream.
#include <mutex>
#include <vector>

#include "../../include/w4a16.h"
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 24;  // rows / columns per operand
constexpr int64_t kMaxM = int64_t(1) << 22;    // batch rows per call
// Packed codes of one matrix are addressed with 32-bit byte offsets.
constexpr int64_t kMaxPackedBytes = (int64_t(1) << 31) - (int64_t(1) << 20);

// Largest M the streaming kernel takes in one pass (its A operand is 16 rows).
constexpr int64_t kSkinnyMaxM = 16;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim) return W4A16_EINVAL;
  if (N % W4A16_TILE_ROWS || K % W4A16_GROUP) return W4A16_EINVAL;
  if (N * K / 2 > kMaxPackedBytes) return W4A16_EINVAL;
  return W4A16_OK;
}

// The packers' scratch: a status word (offset 0), the running tensor range
// (two doubles at 256) and the ranges of one chunk of kRangeRows rows (rmin
// then rmax from 512).  It is device memory of this library's own code object,
// one copy per GPU, held until the process ends: the packers allocate nothing.
// Host code never passes the array's name (a host-side stand-in) to the GPU,
// only the address hipGetSymbolAddress gives on each device.  Pack calls hold
// g_pack_mu from start to end (they block on their stream anyway), so calls
// from several host threads take turns instead of sharing the scratch.
constexpr int kRangeRows = 32768;  // rows per range pass of the coarser granularities
constexpr size_t kPackScratchBytes = 512 + (size_t)kRangeRows * 2 * sizeof(double);
static __device__ __align__(256) unsigned char pack_scratch[kPackScratchBytes];

std::mutex g_pack_mu;
std::vector<unsigned char *> g_pack_ptr;  // per device, set on the first pack call there

// The scratch address on the current device (g_pack_mu held).
int pack_scratch_ptr(unsigned char **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W4A16_EHIP;
  if ((int)g_pack_ptr.size() <= dev) g_pack_ptr.resize(dev + 1, nullptr);
  if (!g_pack_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(pack_scratch)) != hipSuccess || !p) return W4A16_EHIP;
    g_pack_ptr[dev] = static_cast<unsigned char *>(p);
  }
  *out = g_pack_ptr[dev];
  return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_version(void) { return 100; }

const char *w4a16_strerror(int status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_EINVAL: return "invalid argument (NULL pointer, or M/N/K out of range, K % 128 != 0, N % 16 != 0)";
    case W4A16_EALIGN: return "pointer not 16-byte aligned";
    case W4A16_EUNSUPPORTED: return "unsupported kernel path or quantization mode";
    case W4A16_ENONFINITE: return "non-finite W or s, or s <= 0";
    case W4A16_ERANGE: return "group scale exceeds the fp16 range";
    case W4A16_EHIP: return "HIP runtime error";
    case W4A16_ESCRATCH: return "the call needs more workspace than the library's static scratch holds";
    default: return "unknown status";
  }
}

int w4a16_packed_sizes(int64_t N, int64_t K, size_t *wq_bytes, size_t *scales_bytes,
                       size_t *zeros_bytes) {
  if (!wq_bytes || !scales_bytes || !zeros_bytes) return W4A16_EINVAL;
  const int rc = check_shape(N, K);
  if (rc) return rc;
  *wq_bytes = (size_t)N * (size_t)K / 2;
  *scales_bytes = (size_t)N * (size_t)w4a16::meta_groups((int)(K / W4A16_GROUP)) * 2;
  *zeros_bytes = *scales_bytes;
  return W4A16_OK;
}

static bool known_mode(int mode) {
  return mode == W4A16_QUANT_ASYM || mode == W4A16_QUANT_SYM || mode == W4A16_QUANT_ASYM_CHANNEL ||
         mode == W4A16_QUANT_ASYM_TENSOR || mode == W4A16_QUANT_ASYM8;
}

// INT8 codes take N * K bytes
static int check_shape_mode(int64_t N, int64_t K, int mode) {
  const int rc = check_shape(N, K);
  if (rc) return rc;
  if (mode == W4A16_QUANT_ASYM8 && N * K > kMaxPackedBytes) return W4A16_EINVAL;
  return W4A16_OK;
}

int w4a16_packed_sizes_mode(int64_t N, int64_t K, int mode, size_t *wq_bytes, size_t *scales_bytes,
                            size_t *zeros_bytes) {
  if (!known_mode(mode)) return W4A16_EUNSUPPORTED;
  if (!wq_bytes || !scales_bytes || !zeros_bytes) return W4A16_EINVAL;
  const int rc = check_shape_mode(N, K, mode);
  if (rc) return rc;
  *wq_bytes = (size_t)N * (size_t)K / (mode == W4A16_QUANT_ASYM8 ? 1 : 2);
  *scales_bytes = (size_t)N * (size_t)w4a16::meta_groups((int)(K / W4A16_GROUP)) * 2;
  *zeros_bytes = *scales_bytes;
  return W4A16_OK;
}

// Quantize and pack with the scratch `scr` (g_pack_mu held); blocks.  The
// coarser granularities take the row (or tensor) ranges first, kRangeRows rows
// per pass: per channel, each pass's rows are packed right after their ranges;
// per tensor, every pass folds its rows into one running range, then one pack
// launch reads it for every row.
static int pack_and_check(const void *W, const void *s, int64_t N, int64_t K,
                          const uint8_t *keep, int mode, void *Wq, void *scales, void *zeros,
                          unsigned char *scr, hipStream_t st) {
  unsigned *status = reinterpret_cast<unsigned *>(scr);
  double *acc = reinterpret_cast<double *>(scr + 256);
  double *rmin = reinterpret_cast<double *>(scr + 512), *rmax = rmin + kRangeRows;
  const bool sym = mode == W4A16_QUANT_SYM, w8 = mode == W4A16_QUANT_ASYM8;
  const int n = (int)N, k = (int)K, NB = n / W4A16_TILE_ROWS;
  hipError_t e = hipMemsetAsync(status, 0, sizeof(unsigned), st);
  if (e == hipSuccess && mode == W4A16_QUANT_ASYM_TENSOR) {
    for (int n0 = 0; e == hipSuccess && n0 < n; n0 += kRangeRows) {
      const int rows = n - n0 < kRangeRows ? n - n0 : kRangeRows;
      e = w4a16::launch_row_range(W, s, n0, rows, k, keep, rmin, rmax, st);
      if (e == hipSuccess) e = w4a16::launch_tensor_range(rows, rmin, rmax, acc, n0 == 0, st);
    }
    if (e == hipSuccess)
      e = w4a16::launch_pack(W, s, n, k, 0, NB, keep, acc, acc + 1, 0, Wq, scales, zeros, status,
                             sym, st, w8);
  } else if (e == hipSuccess && mode == W4A16_QUANT_ASYM_CHANNEL) {
    for (int n0 = 0; e == hipSuccess && n0 < n; n0 += kRangeRows) {
      const int rows = n - n0 < kRangeRows ? n - n0 : kRangeRows;  // a multiple of 16
      e = w4a16::launch_row_range(W, s, n0, rows, k, keep, rmin, rmax, st);
      if (e == hipSuccess)
        e = w4a16::launch_pack(W, s, n, k, n0 / W4A16_TILE_ROWS, rows / W4A16_TILE_ROWS, keep,
                               rmin, rmax, 1, Wq, scales, zeros, status, sym, st, w8);
    }
  } else if (e == hipSuccess) {
    e = w4a16::launch_pack(W, s, n, k, 0, NB, keep, nullptr, nullptr, 0, Wq, scales, zeros,
                           status, sym, st, w8);
  }
  unsigned host = 0;
  if (e == hipSuccess)
    e = hipMemcpyAsync(&host, status, sizeof(unsigned), hipMemcpyDeviceToHost, st);
  if (hipStreamSynchronize(st) != hipSuccess || e != hipSuccess) return W4A16_EHIP;
  if (host & w4a16::kPackNonFinite) return W4A16_ENONFINITE;
  if (host & w4a16::kPackRange) return W4A16_ERANGE;
  return W4A16_OK;
}

int w4a16_quantize_pack_mode(const void *W, const void *s, int64_t N, int64_t K, int mode,
                             void *Wq, void *scales, void *zeros, void *stream) {
  if (!known_mode(mode)) return W4A16_EUNSUPPORTED;
  if (!W || !Wq || !scales || !zeros) return W4A16_EINVAL;
  int rc = check_shape_mode(N, K, mode);
  if (rc) return rc;
  if (!aligned16(W) || !aligned16(Wq) || !aligned16(scales) || !aligned16(zeros) ||
      (s && !aligned16(s)))
    return W4A16_EALIGN;
  std::lock_guard<std::mutex> lock(g_pack_mu);
  unsigned char *scr = nullptr;
  if ((rc = pack_scratch_ptr(&scr))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return pack_and_check(W, s, N, K, nullptr, mode, Wq, scales, zeros, scr, st);
}

static bool gptq_shape_ok(int64_t N, int64_t K, int64_t n) {
  return check_shape(N, K) == W4A16_OK && n >= 1 && n <= (int64_t(1) << 24) &&
         K <= 65536 && n * K <= (int64_t(1) << 32);
}

int w4a16_gptq_workspace_size(int64_t N, int64_t K, int64_t n_samples, size_t *bytes) {
  if (!bytes || !gptq_shape_ok(N, K, n_samples)) return W4A16_EINVAL;
  *bytes = w4a16::gptq_workspace_bytes((int)N, (int)K, n_samples);
  return W4A16_OK;
}

int w4a16_quantize_pack_gptq(const void *W, const void *s, int64_t N, int64_t K, const void *X,
                             int64_t n_samples, double damp, void *Wq, void *scales, void *zeros,
                             void *workspace, size_t workspace_bytes, void *stream) {
  if (!gptq_shape_ok(N, K, n_samples) || !(damp >= 0.0 && damp < 1e30)) return W4A16_EINVAL;
  if (!W || !X || !Wq || !scales || !zeros || !workspace) return W4A16_EINVAL;
  if (workspace_bytes < w4a16::gptq_workspace_bytes((int)N, (int)K, n_samples)) return W4A16_EINVAL;
  if (!aligned16(W) || !aligned16(Wq) || !aligned16(scales) || !aligned16(zeros) ||
      (s && !aligned16(s)) || !aligned16(X) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return W4A16_EALIGN;
  std::lock_guard<std::mutex> lock(g_pack_mu);
  unsigned char *scr = nullptr;
  int rc = pack_scratch_ptr(&scr);
  if (rc) return rc;
  unsigned *status = reinterpret_cast<unsigned *>(scr);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemsetAsync(status, 0, sizeof(unsigned), st) != hipSuccess) return W4A16_EHIP;
  const int g = w4a16::gptq_pack(W, s, (int)N, (int)K, X, n_samples, damp, Wq, scales, zeros,
                                 workspace, status, st);
  if (g == 1) return W4A16_EUNSUPPORTED;
  if (g == 2) return W4A16_EINVAL;
  if (g != 0) return W4A16_EHIP;
  unsigned host = 0;
  if (hipMemcpy(&host, status, sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess)
    return W4A16_EHIP;
  if (host & w4a16::kPackNonFinite) return W4A16_ENONFINITE;
  if (host & w4a16::kPackRange) return W4A16_ERANGE;
  return W4A16_OK;
}

int w4a16_outlier_workspace_size(int64_t N, int64_t K, size_t *bytes) {
  if (!bytes) return W4A16_EINVAL;
  const int rc = check_shape(N, K);
  if (rc) return rc;
  *bytes = w4a16::outlier_workspace_bytes((int)N, (int)K);
  return W4A16_OK;
}

int w4a16_quantize_pack_outliers(const void *W, const void *s, int64_t N, int64_t K, int mode,
                                 int64_t count, void *Wq, void *scales, void *zeros,
                                 void *o_row_ptr, void *o_col, void *o_val, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  if (!known_mode(mode)) return W4A16_EUNSUPPORTED;
  int rc = check_shape_mode(N, K, mode);
  if (rc) return rc;
  if (count < 0 || count > N * K || count > INT32_MAX) return W4A16_EINVAL;
  if (!W || !Wq || !scales || !zeros || !o_row_ptr || !workspace) return W4A16_EINVAL;
  if (count > 0 && (!o_col || !o_val)) return W4A16_EINVAL;
  if (workspace_bytes < w4a16::outlier_workspace_bytes((int)N, (int)K)) return W4A16_EINVAL;
  auto aligned = [](const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  if (!aligned16(W) || !aligned16(Wq) || !aligned16(scales) || !aligned16(zeros) ||
      (s && !aligned16(s)) || !aligned(o_row_ptr, 4) || !aligned(o_col, 4) || !aligned(o_val, 2) ||
      !aligned(workspace, 256))
    return W4A16_EALIGN;
  std::lock_guard<std::mutex> lock(g_pack_mu);
  unsigned char *scr = nullptr;
  if ((rc = pack_scratch_ptr(&scr))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t *keep = nullptr;
  if (w4a16::select_outliers(W, s, (int)N, (int)K, count, static_cast<int32_t *>(o_row_ptr),
                             static_cast<int32_t *>(o_col), static_cast<_Float16 *>(o_val),
                             workspace, &keep, st) != 0)
    return W4A16_EHIP;
  return pack_and_check(W, s, N, K, keep, mode, Wq, scales, zeros, scr, st);
}

int w4a16_quantize_pack(const void *W, const void *s, int64_t N, int64_t K, void *Wq,
                        void *scales, void *zeros, void *stream) {
  return w4a16_quantize_pack_mode(W, s, N, K, W4A16_QUANT_ASYM, Wq, scales, zeros, stream);
}

int w4a16_select_path(int64_t M, int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return M <= kSkinnyMaxM ? W4A16_PATH_SKINNY : W4A16_PATH_TILED;
}

}  // extern "C"

namespace {

int check_gemm(const void *X, const void *Wq, const void *scales, const void *zeros, const void *s,
               const void *Y, int64_t M, int64_t N, int64_t K) {
  int rc = check_shape(N, K);
  if (rc) return rc;
  if (M < 0 || M > kMaxM) return W4A16_EINVAL;
  if (M == 0) return W4A16_OK;  // empty batch: nothing to read or write
  if (!X || !Wq || !scales || !zeros || !Y) return W4A16_EINVAL;
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(scales) || !aligned16(zeros) ||
      !aligned16(Y) || (s && !aligned16(s)))
    return W4A16_EALIGN;
  return W4A16_OK;
}

// Streaming-kernel pieces of one problem: 16 rows of X per piece.
void skinny_pieces(const w4a16_problem &p, std::vector<w4a16::GemmDesc> &out) {
  for (int64_t m0 = 0; m0 < p.M; m0 += kSkinnyMaxM) {
    const int64_t mb = (p.M - m0) < kSkinnyMaxM ? (p.M - m0) : kSkinnyMaxM;
    out.push_back({static_cast<const _Float16 *>(p.X) + m0 * p.K, p.Wq, p.scales, p.zeros, p.s,
                   static_cast<_Float16 *>(p.Y) + m0 * p.N, (int)mb, (int)p.N, (int)p.K,
                   p.o_row_ptr, p.o_col, p.o_val, p.dtype == W4A16_DTYPE_BF16, p.wbits == 8});
  }
}

// The streaming-path launches of a call, up to skinny_max_problems() pieces
// each, in order on one stream: each may reuse the whole workspace.
hipError_t launch_pieces(const std::vector<w4a16::GemmDesc> &pieces, hipStream_t st,
                         bool force_window = false, void *workspace = nullptr,
                         size_t workspace_bytes = 0) {
  const int cap = w4a16::skinny_max_problems();
  for (size_t i = 0; i < pieces.size(); i += cap) {
    const int n = (int)((pieces.size() - i) < (size_t)cap ? (pieces.size() - i) : (size_t)cap);
    const hipError_t err = w4a16::launch_skinny_set(pieces.data() + i, n, st, force_window,
                                                    workspace, workspace_bytes);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

size_t pieces_workspace_bytes(const std::vector<w4a16::GemmDesc> &pieces) {
  const int cap = w4a16::skinny_max_problems();
  size_t need = 0;
  for (size_t i = 0; i < pieces.size(); i += cap) {
    const int n = (int)((pieces.size() - i) < (size_t)cap ? (pieces.size() - i) : (size_t)cap);
    const size_t b = w4a16::skinny_workspace_bytes(pieces.data() + i, n);
    need = b > need ? b : need;
  }
  return need;
}

}  // namespace

extern "C" {

int w4a16_gemm_path(const void *X, const void *Wq, const void *scales, const void *zeros,
                    const void *s, void *Y, int64_t M, int64_t N, int64_t K, int path,
                    void *stream) {
  if (path != W4A16_PATH_AUTO && path != W4A16_PATH_SKINNY && path != W4A16_PATH_TILED &&
      path != W4A16_PATH_SKINNY_WINDOW)
    return W4A16_EUNSUPPORTED;
  const int rc = check_gemm(X, Wq, scales, zeros, s, Y, M, N, K);
  if (rc || M == 0) return rc;
  if (path == W4A16_PATH_AUTO) path = w4a16_select_path(M, N, K);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (path == W4A16_PATH_SKINNY || path == W4A16_PATH_SKINNY_WINDOW) {
    std::vector<w4a16::GemmDesc> pieces;
    skinny_pieces({X, Wq, scales, zeros, s, Y, M, N, K}, pieces);
    err = launch_pieces(pieces, st, path == W4A16_PATH_SKINNY_WINDOW);
  } else {
    err = w4a16::launch_tiled(X, Wq, scales, zeros, s, Y, (int)M, (int)N, (int)K, st);
  }
  return err == hipSuccess ? W4A16_OK : W4A16_EHIP;
}

}  // extern "C"

namespace {

int check_problems(const w4a16_problem *problems, int count) {
  if (count < 0 || (count > 0 && !problems)) return W4A16_EINVAL;
  for (int i = 0; i < count; ++i) {
    const w4a16_problem &p = problems[i];
    const int rc = check_gemm(p.X, p.Wq, p.scales, p.zeros, p.s, p.Y, p.M, p.N, p.K);
    if (rc) return rc;
    if (p.dtype != W4A16_DTYPE_F16 && p.dtype != W4A16_DTYPE_BF16) return W4A16_EUNSUPPORTED;
    if (p.wbits != 0 && p.wbits != 4 && p.wbits != 8) return W4A16_EUNSUPPORTED;
    if (p.wbits == 8 && p.N * p.K > kMaxPackedBytes) return W4A16_EINVAL;
    const bool any = p.o_row_ptr || p.o_col || p.o_val;
    if (any && !(p.o_row_ptr && p.o_col && p.o_val)) return W4A16_EINVAL;  // all or none
    if (any && ((reinterpret_cast<uintptr_t>(p.o_row_ptr) & 3u) ||
                (reinterpret_cast<uintptr_t>(p.o_col) & 3u) ||
                (reinterpret_cast<uintptr_t>(p.o_val) & 1u)))
      return W4A16_EALIGN;
  }
  return W4A16_OK;
}

w4a16::GemmDesc desc_of(const w4a16_problem &p) {
  return {p.X,      p.Wq,        p.scales, p.zeros, p.s,  p.Y, (int)p.M, (int)p.N,
          (int)p.K, p.o_row_ptr, p.o_col,  p.o_val, p.dtype == W4A16_DTYPE_BF16, p.wbits == 8};
}

// The tiled-path problems of a grouped call, in call order, in launches of up
// to tiled_max_problems(): the same batches for the size query and the call.
std::vector<std::vector<w4a16::GemmDesc>> tiled_batches(const w4a16_problem *problems, int count) {
  std::vector<std::vector<w4a16::GemmDesc>> out;
  const size_t cap = (size_t)w4a16::tiled_max_problems();
  for (int i = 0; i < count; ++i) {
    const w4a16_problem &p = problems[i];
    if (p.M == 0 || w4a16_select_path(p.M, p.N, p.K) != W4A16_PATH_TILED) continue;
    const w4a16::GemmDesc d = desc_of(p);
    // a launch is one kernel instance: one activation type
    if (out.empty() || out.back().size() == cap || out.back().back().bf16 != d.bf16 ||
        out.back().back().w8 != d.w8)
      out.emplace_back();
    out.back().push_back(d);
  }
  return out;
}

}  // namespace

extern "C" {

int w4a16_gemm_workspace_size(const w4a16_problem *problems, int count, size_t *bytes) {
  if (!bytes) return W4A16_EINVAL;
  const int rc = check_problems(problems, count);
  if (rc) return rc;
  // launches run in order on one stream, so they share the workspace
  size_t need = 0;
  for (const auto &b : tiled_batches(problems, count)) {
    const size_t n = w4a16::tiled_workspace_bytes(b.data(), (int)b.size());
    need = n > need ? n : need;
  }
  std::vector<w4a16::GemmDesc> pieces;
  for (int i = 0; i < count; ++i) {
    const w4a16_problem &p = problems[i];
    if (p.M > 0 && w4a16_select_path(p.M, p.N, p.K) == W4A16_PATH_SKINNY) skinny_pieces(p, pieces);
  }
  const size_t sk = pieces_workspace_bytes(pieces);
  *bytes = sk > need ? sk : need;
  return W4A16_OK;
}

int w4a16_gemm_grouped_ws(const w4a16_problem *problems, int count, void *workspace,
                          size_t workspace_bytes, void *stream) {
  const int rc = check_problems(problems, count);
  if (rc) return rc;
  if (workspace && !aligned16(workspace)) return W4A16_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<w4a16::GemmDesc> pieces;
  for (int i = 0; i < count; ++i) {
    const w4a16_problem &p = problems[i];
    if (p.M > 0 && w4a16_select_path(p.M, p.N, p.K) == W4A16_PATH_SKINNY) skinny_pieces(p, pieces);
  }
  for (const auto &b : tiled_batches(problems, count))
    if (w4a16::launch_tiled_set(b.data(), (int)b.size(), workspace, workspace_bytes, st) !=
        hipSuccess)
      return W4A16_EHIP;
  return launch_pieces(pieces, st, false, workspace, workspace_bytes) == hipSuccess ? W4A16_OK
                                                                                   : W4A16_EHIP;
}

}  // extern "C"

namespace {

// The scratch of the entry points that take no workspace (w4a16_gemm,
// w4a16_gemm_grouped): W4A16_SHARED_SCRATCH_BYTES of device memory in this
// library's code object, one copy per GPU, held until the process ends, with
// one event per GPU that marks the end of the last call's work in it.  A call
// whose workspace fits makes its stream wait for that event, launches with
// the scratch as its workspace and records the event again, under one mutex:
// the work of such calls runs one after the other on the GPU, whatever their
// streams, so they never race.  The device address comes from
// hipGetSymbolAddress (the name is a host-side stand-in in host code).
static __device__ __align__(256) unsigned char shared_scratch[W4A16_SHARED_SCRATCH_BYTES];

struct SharedScratch {
  void *ptr = nullptr;
  hipEvent_t done = nullptr;
};
std::mutex g_shared_mu;
std::vector<SharedScratch> g_shared;  // per device

int grouped_shared(const w4a16_problem *problems, int count, void *stream) {
  size_t need = 0;
  const int rc = w4a16_gemm_workspace_size(problems, count, &need);  // validates too
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  // under capture the event could not order work outside the graph: no split
  if (need == 0 || need > W4A16_SHARED_SCRATCH_BYTES ||
      hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return w4a16_gemm_grouped_ws(problems, count, nullptr, 0, stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W4A16_EHIP;
  std::lock_guard<std::mutex> lock(g_shared_mu);
  if ((int)g_shared.size() <= dev) g_shared.resize(dev + 1);
  SharedScratch &sh = g_shared[dev];
  if (!sh.ptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(shared_scratch)) != hipSuccess || !ptr)
      return W4A16_EHIP;
    hipEvent_t ev = nullptr;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return W4A16_EHIP;
    sh.ptr = ptr;
    sh.done = ev;
  }
  if (hipStreamWaitEvent(st, sh.done, 0) != hipSuccess) return W4A16_EHIP;
  const int r = w4a16_gemm_grouped_ws(problems, count, sh.ptr, need, stream);
  // recorded whatever the outcome: later calls must wait for any launched work
  const bool recorded = hipEventRecord(sh.done, st) == hipSuccess;
  return r ? r : (recorded ? W4A16_OK : W4A16_EHIP);
}

}  // namespace

extern "C" {

int w4a16_gemm_grouped(const w4a16_problem *problems, int count, void *stream) {
  return grouped_shared(problems, count, stream);
}

}  // extern "C"

namespace {

// The workspace of w4a16_gemm_grouped_static: W4A16_STATIC_SCRATCH_BYTES of
// device memory in this library's code object, one copy per GPU, held until
// the process ends.  Its name is a host-side stand-in in host code: kernels
// get the address hipGetSymbolAddress returns on each device (taken once per
// device, with that device current, on the entry point's first call there).
static __device__ __align__(256) unsigned char scratch[W4A16_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;  // per device

int scratch_ptr(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W4A16_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4A16_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_gemm_grouped_static(const w4a16_problem *problems, int count, void *stream) {
  size_t need = 0;
  const int rc = w4a16_gemm_workspace_size(problems, count, &need);  // validates too
  if (rc) return rc;
  if (need > W4A16_STATIC_SCRATCH_BYTES) return W4A16_ESCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    const int r = scratch_ptr(&ws);
    if (r) return r;
  }
  // the partial sums and prescaled activations are written before they are
  // read within the call, so nothing in the scratch needs clearing
  return w4a16_gemm_grouped_ws(problems, count, ws, need, stream);
}

static bool spec_shape_ok(int64_t B, int64_t K, int64_t V) {
  if (B < 0 || K < 0 || V < 1 || B > (int64_t(1) << 24) || K > 1024 || V > (int64_t(1) << 24))
    return false;
  if (B * (K + 1) * V > (int64_t(1) << 40)) return false;
  // the first launch has B * chunks workgroups of 256 threads
  return B * (int64_t)w4a16::spec_verify_chunks((int)V) < (int64_t(1) << 24);
}

int w4a16_spec_verify_workspace_size(int64_t B, int64_t K, int64_t V, size_t *bytes) {
  if (!bytes || !spec_shape_ok(B, K, V)) return W4A16_EINVAL;
  *bytes = B == 0 ? 0 : w4a16::spec_verify_workspace_bytes((int)B, (int)V);
  return W4A16_OK;
}

int w4a16_spec_verify(const void *p_target, const void *p_draft, const void *draft,
                      const void *u_accept, const void *u_sample, int64_t B, int64_t K, int64_t V,
                      void *workspace, size_t workspace_bytes, void *n_accepted, void *token,
                      void *stream) {
  if (!spec_shape_ok(B, K, V)) return W4A16_EINVAL;
  if (B == 0) return W4A16_OK;
  if (!p_target || !u_sample || !n_accepted || !token || !workspace) return W4A16_EINVAL;
  if (K > 0 && (!p_draft || !draft || !u_accept)) return W4A16_EINVAL;
  if (workspace_bytes < w4a16::spec_verify_workspace_bytes((int)B, (int)V)) return W4A16_EINVAL;
  auto al4 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (!al4(p_target) || !al4(u_sample) || !al4(n_accepted) || !al4(token) ||
      (K > 0 && (!al4(p_draft) || !al4(draft) || !al4(u_accept))) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return W4A16_EALIGN;
  return w4a16::launch_spec_verify(
             static_cast<const float *>(p_target), static_cast<const float *>(p_draft),
             static_cast<const int32_t *>(draft), static_cast<const float *>(u_accept),
             static_cast<const float *>(u_sample), (int)B, (int)K, (int)V, workspace,
             static_cast<int32_t *>(n_accepted), static_cast<int32_t *>(token),
             static_cast<hipStream_t>(stream)) == hipSuccess
             ? W4A16_OK
             : W4A16_EHIP;
}

int w4a16_gemm(const void *X, const void *Wq, const void *scales, const void *zeros,
               const void *s, void *Y, int64_t M, int64_t N, int64_t K, void *stream) {
  const int rc = check_gemm(X, Wq, scales, zeros, s, Y, M, N, K);
  if (rc || M == 0) return rc;
  w4a16_problem p = {};
  p.X = X;
  p.Wq = Wq;
  p.scales = scales;
  p.zeros = zeros;
  p.s = s;
  p.Y = Y;
  p.M = M;
  p.N = N;
  p.K = K;
  return grouped_shared(&p, 1, stream);
}

}  // extern "C"
