// gfx950 kernels of the element-wise companions of the Muon step: gradient
// clipping (norm partials, per-bucket finalize, scale) and the AdamW update.
// All are bound by HBM bandwidth: one flat pass over the tensors, 16
// elements per thread in 16-byte (fp32) or 8-byte (bf16) vector accesses,
// consecutive threads on consecutive vectors.
#include <math.h>

#include "dmuon_device.h"
#include "dmuon_internal.h"

namespace dmuon {
namespace {

// Task of flat block b (tasks sorted by blk_begin).
__device__ __forceinline__ int find_flat(const FlatTask* tasks, int ntasks, int b) {
  int lo = 0, hi = ntasks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tasks[mid].blk_begin <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Maximum that keeps a NaN (fmaxf would drop it).
__device__ __forceinline__ float nanmax(float a, float b) {
  return a != a ? a : (b != b ? b : fmaxf(a, b));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ float wave_nanmax(float v) {
  v = nanmax(v, dpp_f<0xB1>(v));
  v = nanmax(v, dpp_f<0x4E>(v));
  v = nanmax(v, dpp_f<0x141>(v));
  v = nanmax(v, dpp_f<0x140>(v));
  v = nanmax(v, __shfl_xor(v, 16));
  v = nanmax(v, __shfl_xor(v, 32));
  return v;
}

// Four elements starting at i of a tensor of n elements (zeros past n).
__device__ __forceinline__ f32x4 load4_tail(const void* base, int dtype, int64_t i, int64_t n,
                                            bool vec) {
  if (vec && i + 3 < n) return load4(base, dtype, (size_t)i);
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (i + e < n) x[e] = load1(base, dtype, (size_t)(i + e));
  return x;
}

__device__ __forceinline__ void store1_dt(void* base, int dtype, size_t i, float v) {
  if (dtype == 0)
    st_f32(static_cast<float*>(base) + i, v);
  else
    st_u16(static_cast<uint16_t*>(base) + i, to_bf16(v));
}

__device__ __forceinline__ void store4_tail(void* base, int dtype, int64_t i, int64_t n, bool vec,
                                            f32x4 x) {
  if (vec && i + 3 < n) {
    if (dtype == 0)
      st_f32x4_nt(static_cast<float*>(base) + i, x);
    else
      st_u32x2_nt(static_cast<uint16_t*>(base) + i, pack_bf16x4(x[0], x[1], x[2], x[3]));
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (i + e < n) store1_dt(base, dtype, (size_t)(i + e), x[e]);
}

// The ITERS x 16 elements of this thread in a chunk starting at `chunk`:
// element chunk + it*FLAT_STEP + (k*FLAT_THREADS + tid)*4 + e.  A chunk that
// lies wholly inside an aligned tensor (every chunk but a tensor's last)
// loads without per-lane conditions, so nothing separates the loads from
// each other; the tail chunk checks each element.
template <int ITERS>
__device__ __forceinline__ void load_chunk(const void* base, int dtype, int64_t chunk, int64_t n,
                                           bool vec, int tid, f32x4 (&x)[ITERS][4]) {
  if (vec && chunk + (int64_t)ITERS * FLAT_STEP <= n) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[it][k] = load4(base, dtype,
                         (size_t)(chunk + (int64_t)it * FLAT_STEP + (k * FLAT_THREADS + tid) * 4));
  } else {
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[it][k] = load4_tail(base, dtype,
                              chunk + (int64_t)it * FLAT_STEP + (k * FLAT_THREADS + tid) * 4, n,
                              vec);
  }
}

template <int ITERS>
__device__ __forceinline__ void store_chunk(void* base, int dtype, int64_t chunk, int64_t n,
                                            bool vec, int tid, const f32x4 (&x)[ITERS][4]) {
  const bool full = vec && chunk + (int64_t)ITERS * FLAT_STEP <= n;
#pragma unroll
  for (int it = 0; it < ITERS; ++it)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      store4_tail(base, dtype, chunk + (int64_t)it * FLAT_STEP + (k * FLAT_THREADS + tid) * 4,
                  full ? INT64_MAX : n, vec, x[it][k]);
}

// ---------------------------------------------------------------------------
// Clipping, pass 1: every block reduces its chunk (FLAT_ITERS_CLIP steps of
// 16 elements per thread) to one partial (sum of squares, sum of
// magnitudes, sum of |g|^p, or NaN-keeping max of |g|), in a fixed order:
// per thread, then the wave, then the 4 waves.
__global__ __launch_bounds__(FLAT_THREADS) void clip_norm_kernel(
    const FlatTask* __restrict__ tasks, int ntasks, int total_blocks, int mode, float p,
    float* __restrict__ partial) {
  __shared__ float wpart[FLAT_THREADS / 64];
  const int b = blockIdx.x;
  if (b >= total_blocks) return;
  const FlatTask T = tasks[find_flat(tasks, ntasks, b)];
  const int64_t chunk = (int64_t)(b - T.blk_begin) * FLAT_STEP * FLAT_ITERS_CLIP;
  const int tid = threadIdx.x;
  // One step of 16 elements per thread at a time (past the end they read
  // as zeros, which no norm changes), accumulated in a fixed order.
  float acc = 0.f;
  for (int it = 0; it < FLAT_ITERS_CLIP; ++it) {
    const int64_t base = chunk + (int64_t)it * FLAT_STEP;
    if (base >= T.n) break;
    f32x4 x[1][4];
    load_chunk<1>(T.p, T.dtype, base, T.n, T.vec, tid, x);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = fabsf(x[0][k][e]);
        if (mode == NORM_L2) acc = fmaf(a, a, acc);
        else if (mode == NORM_L1) acc += a;
        else if (mode == NORM_INF) acc = nanmax(acc, a);
        else acc += powf(a, p);
      }
  }
  acc = mode == NORM_INF ? wave_nanmax(acc) : wave_sum(acc);
  if ((tid & 63) == 0) wpart[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    float s = wpart[0];
#pragma unroll
    for (int w = 1; w < FLAT_THREADS / 64; ++w) s = mode == NORM_INF ? nanmax(s, wpart[w]) : s + wpart[w];
    st_f32(partial + b, s);
  }
}

// Clipping, pass 2: one block per bucket combines the partials of its
// tensors in fp64, in a fixed order, and writes the bucket's stats and the
// factor its gradients are multiplied by: min(max_norm / (total + 1e-6), 1)
// (kept NaN when the coefficient is NaN), or 1 for a stats-only call.
__global__ __launch_bounds__(256) void clip_finalize_kernel(
    const FlatTask* __restrict__ tasks, int ntasks, int mode, double p, double max_norm,
    int stats_only, const float* __restrict__ partial, ClipStats* __restrict__ stats,
    float* __restrict__ scale) {
  __shared__ double part[256];
  const int bucket = blockIdx.x;
  const int tid = threadIdx.x;
  double acc = 0.0;
  int64_t count = 0;
  for (int t = 0; t < ntasks; ++t) {
    const FlatTask T = tasks[t];
    if (T.bucket != bucket) continue;
    count += T.n;
    for (int j = tid; j < T.nblk; j += 256) {
      const double v = (double)ld_f32(partial + T.blk_begin + j);
      if (mode == NORM_INF)
        acc = (acc != acc) ? acc : ((v != v) ? v : fmax(acc, v));
      else
        acc += v;
    }
  }
  part[tid] = acc;
  __syncthreads();
  if (tid == 0) {
    double s = part[0];
    for (int j = 1; j < 256; ++j)
      s = mode == NORM_INF ? ((s != s) ? s : ((part[j] != part[j]) ? part[j] : fmax(s, part[j])))
                           : s + part[j];
    double total;
    if (mode == NORM_L2) total = sqrt(s);
    else if (mode == NORM_L1 || mode == NORM_INF) total = s;
    else total = pow(s, 1.0 / p);
    const double coef = stats_only ? 1.0 : max_norm / (total + 1e-6);
    ClipStats st;
    st.total_norm = total;
    st.clip_coef = coef;
    st.clipped = coef < 1.0;
    st.found_inf = !isfinite(total);
    st.param_count = count;
    stats[bucket] = st;
    float f = 1.f;
    if (!stats_only) f = (coef != coef) ? (float)coef : (float)fmin(coef, 1.0);
    st_f32(scale + bucket, f);
  }
}

// Clipping, pass 3: g <- g * factor of its bucket (blocks of a bucket whose
// factor is exactly 1 write nothing).
__global__ __launch_bounds__(FLAT_THREADS) void clip_scale_kernel(
    const FlatTask* __restrict__ tasks, int ntasks, int total_blocks,
    const float* __restrict__ scale) {
  const int b = blockIdx.x;
  if (b >= total_blocks) return;
  const FlatTask T = tasks[find_flat(tasks, ntasks, b)];
  const float f = ld_f32(scale + T.bucket);
  if (f == 1.f) return;
  const int64_t chunk = (int64_t)(b - T.blk_begin) * FLAT_STEP * FLAT_ITERS_CLIP;
  const int tid = threadIdx.x;
  for (int it = 0; it < FLAT_ITERS_CLIP; ++it) {
    const int64_t base = chunk + (int64_t)it * FLAT_STEP;
    if (base >= T.n) break;
    f32x4 x[1][4];
    load_chunk<1>(T.p, T.dtype, base, T.n, T.vec, tid, x);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[0][k][e] *= f;
    store_chunk<1>(T.p, T.dtype, base, T.n, T.vec, tid, x);
  }
}

// ---------------------------------------------------------------------------
// AdamW (decoupled weight decay), fp32 arithmetic, moments in fp32:
//   p <- p (1 - lr wd); m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
//   p <- p - (lr / (1-b1^t)) m / (sqrt(v) / sqrt(1-b2^t) + eps)
__global__ __launch_bounds__(FLAT_THREADS) void adamw_kernel(
    const FlatTask* __restrict__ tasks, int ntasks, int total_blocks, AdamArgs A) {
  const int b = blockIdx.x;
  if (b >= total_blocks) return;
  const FlatTask T = tasks[find_flat(tasks, ntasks, b)];
  static_assert(FLAT_ITERS_ADAMW == 1, "one step of 16 elements per thread");
  const int64_t base = (int64_t)(b - T.blk_begin) * FLAT_STEP;
  const int tid = threadIdx.x;
  f32x4 p[1][4], g[1][4], m[1][4], v[1][4];
  load_chunk<1>(T.p, T.dtype, base, T.n, T.vec, tid, p);
  load_chunk<1>(T.g, T.gdtype, base, T.n, T.vec, tid, g);
  load_chunk<1>(T.m, 0, base, T.n, T.vec, tid, m);
  load_chunk<1>(T.v, 0, base, T.n, T.vec, tid, v);
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gg = g[0][k][e];
      const float mm = fmaf(A.beta1, m[0][k][e], A.one_minus_beta1 * gg);
      const float vv = fmaf(A.beta2, v[0][k][e], A.one_minus_beta2 * gg * gg);
      const float den = fmaf(sqrtf(vv), A.inv_bc2_sqrt, A.eps);
      p[0][k][e] = fmaf(-A.step_size, mm / den, p[0][k][e] * A.decay);
      m[0][k][e] = mm;
      v[0][k][e] = vv;
    }
  store_chunk<1>(T.p, T.dtype, base, T.n, T.vec, tid, p);
  store_chunk<1>(T.m, 0, base, T.n, T.vec, tid, m);
  store_chunk<1>(T.v, 0, base, T.n, T.vec, tid, v);
}

}  // namespace

hipError_t launch_clip_norm(const FlatTask* tasks, int ntasks, int total_blocks, int mode,
                            float p, float* partial, hipStream_t s) {
  hipLaunchKernelGGL(clip_norm_kernel, dim3(total_blocks), dim3(FLAT_THREADS), 0, s, tasks,
                     ntasks, total_blocks, mode, p, partial);
  return hipGetLastError();
}

hipError_t launch_clip_finalize(const FlatTask* tasks, int ntasks, int nbuckets, int mode,
                                double p, double max_norm, int stats_only,
                                const float* partial, ClipStats* stats, float* scale,
                                hipStream_t s) {
  hipLaunchKernelGGL(clip_finalize_kernel, dim3(nbuckets), dim3(256), 0, s, tasks, ntasks, mode,
                     p, max_norm, stats_only, partial, stats, scale);
  return hipGetLastError();
}

hipError_t launch_clip_scale(const FlatTask* tasks, int ntasks, int total_blocks,
                             const float* scale, hipStream_t s) {
  hipLaunchKernelGGL(clip_scale_kernel, dim3(total_blocks), dim3(FLAT_THREADS), 0, s, tasks,
                     ntasks, total_blocks, scale);
  return hipGetLastError();
}

hipError_t launch_adamw(const FlatTask* tasks, int ntasks, int total_blocks,
                        const AdamArgs& args, hipStream_t s) {
  hipLaunchKernelGGL(adamw_kernel, dim3(total_blocks), dim3(FLAT_THREADS), 0, s, tasks, ntasks,
                     total_blocks, args);
  return hipGetLastError();
}

}  // namespace dmuon
