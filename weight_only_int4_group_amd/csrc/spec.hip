// Speculative-sampling verification: the accept / reject step that consumes the
// target model's distributions for the K + 1 positions of a verify pass.
//
// "Chapter 22: Advanced inference optimisation" (aiwing.uk), section 22.1:
// draft token x_i is accepted if u_i <= p_target(x_i) / p_draft(x_i); at the
// first rejection one token is drawn from normalize(max(0, p_target - p_draft))
// and the later drafts are dropped; when all K are accepted a (K+1)-th token is
// drawn from the target distribution of position K (the section's expected
// token count (1 - a^(K+1)) / (1 - a) includes it).
//
// Every decision is exact, so the result is unique:
//   * the test is u * p_draft <= p_target in fp64 (a product of two fp32
//     values is exact there); p_draft = 0 accepts, an id outside 0..V-1
//     rejects; NaN and negative probabilities count as 0;
//   * a draw is an inverse-CDF draw in fixed point: with fx(p) = floor(p *
//     2^40), the target row's weights are fx(p_target) and the corrected
//     residual's fx(max(0, p_target - p_draft)), the difference formed in fp64
//     from the two fp32 values; sums are exact (order-
//     free), T = (floor(u' * 2^32) * S) >> 32, and the token is the smallest x
//     whose inclusive prefix sum exceeds T; with no mass in the residual the
//     target row is used, and with none there either the token is -1.
//
// Two launches.  partial_kernel: one 256-thread workgroup per (sequence, chunk
// of kChunk ids); each finds the first rejection (K tests, an LDS minimum),
// then sums the fixed-point weights of its chunk of the drawn row -- both the
// residual and the target row when a draft was rejected, so the fallback needs
// no second pass -- with coalesced loads, and stores the two sums.
// draw_kernel: one workgroup per sequence; it adds the chunk sums, forms T,
// finds the chunk holding T with a block scan over the sums (staged in LDS),
// then scans that chunk alone (kPerThread consecutive ids per thread) to the
// token.  The rows are read once in full and once more for one chunk; rows
// whose length is a multiple of 4 and whose start is 16-byte aligned are read
// with 16-byte loads.
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int kThreads = 256, kWaves = kThreads / 64;
constexpr int kChunk = 4096;                   // ids per partial-sum workgroup
constexpr int kPerThread = kChunk / kThreads;  // ids per thread in the final scan
constexpr int kMaxChunks = (1 << 24) / kChunk;   // V <= 2^24
constexpr double kFix = 0x1p40;     // fixed-point scale of the weights
constexpr double kUScale = 0x1p32;  // fixed-point scale of the sampling uniform

__device__ __forceinline__ double clean(float p) { return p > 0.f ? (double)p : 0.0; }

// fx(p) = floor(p * 2^40) for p > 0 (0 for p <= 0 and NaN: fmax returns the
// non-NaN operand), as an integer-valued double.  Rows sum to less than 2^12,
// so every weight and every partial sum of a row is an integer below 2^52 and
// fp64 adds of them are exact.
__device__ __forceinline__ double fx(float p) { return floor(fmax((double)p, 0.0) * kFix); }

// the corrected residual weight fx(max(0, p_target - p_draft)): the difference
// of the two cleaned values in fp64 (exact unless their exponents are more
// than 29 apart, then rounded once to nearest), in fixed point
__device__ __forceinline__ double residual(float pt, float pd) {
  return floor(fmax(fmax((double)pt, 0.0) - fmax((double)pd, 0.0), 0.0) * kFix);
}

// an exact integer-valued double below 2^52 to an integer (clamped far above
// anything inside the contract)
__device__ __forceinline__ uint64_t to_int(double v) {
  return v < 0x1p62 ? (uint64_t)v : (uint64_t)1 << 62;
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint64_t wave_inclusive_scan(uint64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum of v over the workgroup in thread order; `total` gets
// the sum over all threads.  Uses s_tot[kWaves]; starts and ends with a barrier
// so it can be called back to back.
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t v, uint64_t *s_tot,
                                                         uint64_t &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t inc = wave_inclusive_scan(v, lane);
  __syncthreads();
  if (lane == 63) s_tot[wave] = inc;
  __syncthreads();
  uint64_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    before += w < wave ? s_tot[w] : 0;
    total += s_tot[w];
  }
  return before + inc - v;
}

// Rows that can be read with 16-byte loads: V a multiple of 4 and both row
// starts 16-byte aligned (then every row of the tensors is).
__device__ __forceinline__ bool vec4_rows(const float *rt, const float *rd, int V) {
  return (V & 3) == 0 && ((reinterpret_cast<uintptr_t>(rt) |
                           reinterpret_cast<uintptr_t>(rd)) & 15) == 0;
}

// Index of the first rejected draft of sequence b (K if none), in every thread.
__device__ __forceinline__ int first_rejection(const float *p_target, const float *p_draft,
                                               const int32_t *draft, const float *u_accept, int b,
                                               int K, int V, int *s_rej) {
  if (threadIdx.x == 0) *s_rej = K;
  __syncthreads();
  for (int i = threadIdx.x; i < K; i += kThreads) {
    const int x = draft[(size_t)b * K + i];
    bool accept = false;
    if (x >= 0 && x < V) {
      const double pt = clean(p_target[((size_t)b * (K + 1) + i) * V + x]);
      const double pd = clean(p_draft[((size_t)b * K + i) * V + x]);
      accept = (double)u_accept[(size_t)b * K + i] * pd <= pt;
    }
    if (!accept) atomicMin(s_rej, i);
  }
  __syncthreads();
  return *s_rej;
}

// grid: B * C workgroups, workgroup b * C + c.  part[(b * C + c) * 2 + {0, 1}] =
// the chunk's residual and target sums (residual 0 when every draft was
// accepted); rej_out[b] = the first rejection.
__global__ __launch_bounds__(kThreads) void partial_kernel(
    const float *__restrict__ p_target, const float *__restrict__ p_draft,
    const int32_t *__restrict__ draft, const float *__restrict__ u_accept, int K, int V, int C,
    uint64_t *__restrict__ part, int32_t *__restrict__ rej_out) {
  __shared__ int s_rej;
  __shared__ uint64_t s_red[2][kWaves];
  const int b = blockIdx.x / C, c = blockIdx.x - b * C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rej = first_rejection(p_target, p_draft, draft, u_accept, b, K, V, &s_rej);
  if (c == 0 && tid == 0) rej_out[b] = rej;

  const float *rt = p_target + ((size_t)b * (K + 1) + rej) * V;
  const float *rd = rej < K ? p_draft + ((size_t)b * K + rej) * V : nullptr;
  const int x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  double sr = 0, st = 0;
  if (vec4_rows(rt, rd, V)) {
    // 16-byte loads: thread tid takes ids x0 + 4 (tid + kThreads j) .. + 3
    // (V % 4 == 0, so a quad never crosses x1)
    if (rd) {
#pragma unroll
      for (int j = 0; j < kChunk / (4 * kThreads); ++j) {
        const int x = x0 + 4 * (tid + kThreads * j);
        if (x < x1) {
          const float4 t = *reinterpret_cast<const float4 *>(rt + x);
          const float4 d = *reinterpret_cast<const float4 *>(rd + x);
          const double f0 = fx(t.x), f1 = fx(t.y), f2 = fx(t.z), f3 = fx(t.w);
          st += (f0 + f1) + (f2 + f3);
          sr += (residual(t.x, d.x) + residual(t.y, d.y)) + (residual(t.z, d.z) + residual(t.w, d.w));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kChunk / (4 * kThreads); ++j) {
        const int x = x0 + 4 * (tid + kThreads * j);
        if (x < x1) {
          const float4 t = *reinterpret_cast<const float4 *>(rt + x);
          st += (fx(t.x) + fx(t.y)) + (fx(t.z) + fx(t.w));
        }
      }
    }
  } else if (rd) {
#pragma unroll 8
    for (int x = x0 + tid; x < x1; x += kThreads) {
      const float t = rt[x];
      st += fx(t);
      sr += residual(t, rd[x]);
    }
  } else {
#pragma unroll 8
    for (int x = x0 + tid; x < x1; x += kThreads) st += fx(rt[x]);
  }
  const uint64_t wr = wave_sum(to_int(sr)), wt = wave_sum(to_int(st));
  if (lane == 0) {
    s_red[0][wave] = wr;
    s_red[1][wave] = wt;
  }
  __syncthreads();
  if (tid < 2) {
    uint64_t v = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += s_red[tid][w];
    part[(size_t)blockIdx.x * 2 + tid] = v;
  }
}

// grid: B workgroups.
__global__ __launch_bounds__(kThreads) void draw_kernel(
    const float *__restrict__ p_target, const float *__restrict__ p_draft,
    const float *__restrict__ u_sample, int K, int V, int C, const uint64_t *__restrict__ part,
    const int32_t *__restrict__ rej_in, int32_t *__restrict__ n_accepted,
    int32_t *__restrict__ token) {
  __shared__ uint64_t s_part[2][kMaxChunks];
  __shared__ uint64_t s_tot[kWaves];
  __shared__ uint64_t s_base;
  __shared__ int s_chunk;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int rej = rej_in[b];
  const uint64_t *pb = part + (size_t)b * C * 2;
  // defaults: only rows outside the contract (sums of 2^12 or more) leave them
  if (tid == 0) {
    n_accepted[b] = rej;
    token[b] = -1;
  }
  for (int i = tid; i < 2 * C; i += kThreads) s_part[i & 1][i >> 1] = pb[i];
  __syncthreads();

  // this thread's run of chunk sums: chunks [c0, c1)
  const int per = (C + kThreads - 1) / kThreads;
  const int c0 = min(C, tid * per), c1 = min(C, c0 + per);
  uint64_t lr = 0, lt = 0;
  for (int c = c0; c < c1; ++c) {
    lr += s_part[0][c];
    lt += s_part[1][c];
  }
  uint64_t Sr, St;
  const uint64_t er = block_exclusive_scan(lr, s_tot, Sr);
  const uint64_t et = block_exclusive_scan(lt, s_tot, St);
  const bool use_residual = rej < K && Sr > 0;
  const uint64_t S = use_residual ? Sr : St;
  if (S == 0) return;  // no mass in either row: the defaults stand
  // T = (floor(u' * 2^32) * S) >> 32 exactly (u' < 2^32, S < 2^64 split in halves)
  const float uf = u_sample[b];
  uint64_t ui = uf > 0.f ? (uint64_t)floor((double)uf * kUScale) : 0;
  ui = ui < ((uint64_t)1 << 32) ? ui : ((uint64_t)1 << 32) - 1;
  const uint64_t T = ui * (S >> 32) + ((ui * (S & 0xffffffffu)) >> 32);

  // the chunk holding T (T < S, so exactly one thread's run [e, e + l) contains
  // it); that thread walks its run
  const uint64_t e = use_residual ? er : et, l = use_residual ? lr : lt;
  if (e <= T && T < e + l) {
    uint64_t acc = e;
    for (int c = c0; c < c1; ++c) {
      const uint64_t v = s_part[use_residual ? 0 : 1][c];
      if (acc + v > T) {
        s_chunk = c;
        s_base = acc;
        break;
      }
      acc += v;
    }
  }
  __syncthreads();
  const int cs = s_chunk;
  const uint64_t base = s_base;

  // scan that chunk: thread tid owns ids [xa, xa + kPerThread)
  const float *rt = p_target + ((size_t)b * (K + 1) + rej) * V;
  const float *rd = use_residual ? p_draft + ((size_t)b * K + rej) * V : nullptr;
  const int xa = cs * kChunk + tid * kPerThread;
  float pt[kPerThread], pd[kPerThread];
  if (vec4_rows(rt, rd, V)) {
#pragma unroll
    for (int q = 0; q < kPerThread / 4; ++q) {
      const int x = xa + 4 * q;
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f), d = t;
      if (x < V) {
        t = *reinterpret_cast<const float4 *>(rt + x);
        if (rd) d = *reinterpret_cast<const float4 *>(rd + x);
      }
      pt[4 * q] = t.x, pt[4 * q + 1] = t.y, pt[4 * q + 2] = t.z, pt[4 * q + 3] = t.w;
      pd[4 * q] = d.x, pd[4 * q + 1] = d.y, pd[4 * q + 2] = d.z, pd[4 * q + 3] = d.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int x = xa + j;
      pt[j] = x < V ? rt[x] : 0.f;
      pd[j] = x < V && rd ? rd[x] : 0.f;
    }
  }
  double w[kPerThread], wsum = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    w[j] = use_residual ? residual(pt[j], pd[j]) : fx(pt[j]);
    wsum += w[j];
  }
  const uint64_t sum = to_int(wsum);
  uint64_t chunk_total;
  uint64_t acc = base + block_exclusive_scan(sum, s_tot, chunk_total);
  if (acc <= T && T < acc + sum) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      acc += to_int(w[j]);
      if (acc > T) {
        n_accepted[b] = rej;
        token[b] = xa + j;
        break;
      }
    }
  }
}

}  // namespace

int spec_verify_chunks(int V) { return (V + kChunk - 1) / kChunk; }

size_t spec_verify_workspace_bytes(int B, int V) {
  const size_t C = (size_t)spec_verify_chunks(V);
  return ((size_t)B * C * 16 + (size_t)B * 4 + 255) / 256 * 256;
}

hipError_t launch_spec_verify(const float *p_target, const float *p_draft, const int32_t *draft,
                              const float *u_accept, const float *u_sample, int B, int K, int V,
                              void *workspace, int32_t *n_accepted, int32_t *token,
                              hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int C = spec_verify_chunks(V);
  uint64_t *part = static_cast<uint64_t *>(workspace);
  int32_t *rej = reinterpret_cast<int32_t *>(part + (size_t)B * C * 2);
  hipLaunchKernelGGL(partial_kernel, dim3((unsigned)B * C), dim3(kThreads), 0, stream, p_target,
                     p_draft, draft, u_accept, K, V, C, part, rej);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(draw_kernel, dim3(B), dim3(kThreads), 0, stream, p_target, p_draft, u_sample,
                     K, V, C, part, rej, n_accepted, token);
  return hipGetLastError();
}

}  // namespace w4a16
