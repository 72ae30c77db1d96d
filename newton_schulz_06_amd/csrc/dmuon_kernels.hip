// gfx950 (CDNA4) kernels of the per-owner Muon step.
//
// Data layout in the workspace, per matrix (p = min(m, n), q = max(m, n),
// P and Q padded up to the GEMM tile; every pad element is kept at zero):
//   xm    fp32 X (the oriented G), P x Q row-major         [fp32 mode]
//   xb    bf16 X (the SYRK operand), P x Q                  [bf16 modes]
//   xlo   bf16 (X - xb): xb + xlo is the master X          [bf16 modes]
//   xt    X^T, Q x P, two buffers used in turn (the B X operand)
//   a32   fp32 A = X X^T, P x P                     [unless A is split]
//   aop   A as MFMA operand: bf16 P x P, or [hi|lo|hi|hi] rows (4P)
//   bop   B = bA + cA^2 as MFMA operand (fp32 / bf16 / [hi|lo] rows)
// With every operand stored K-contiguous, all three products of one NS
// iteration are "NT" products C = L R^T and share one MFMA main loop.
#include <cstring>
#include <mutex>
#include <type_traits>

#include "dmuon_device.h"
#include "dmuon_internal.h"

namespace dmuon {
namespace {

static_assert(Op16<1>::kAScale == kF16AScale && Op16<1>::kBScale == kF16BScale,
              "the host's fp16 operand scales are the kernels'");

// --------------------------------------------------------------------------
// Launch tables hold Refs (see Bases): resolved once per block.
template <class T>
__device__ __forceinline__ T* at(Ref r, const Bases& b) {
  if (r >= 0) return reinterpret_cast<T*>(b.ws + r);
  if (r == kRefNone) return nullptr;
  typedef void* const GMEM* SlotPtr;
  return static_cast<T*>(((SlotPtr)b.slots)[-2 - r]);
}

__device__ __forceinline__ EwTask resolve(const EwTab& t, const Bases& b) {
  EwTask r = __builtin_bit_cast(EwTask, t);
  r.src = at<const void>(t.src, b);
  r.buf = at<float>(t.buf, b);
  r.xm = at<float>(t.xm, b);
  r.xb = at<uint16_t>(t.xb, b);
  r.xlo = at<uint16_t>(t.xlo, b);
  r.xt = at<void>(t.xt, b);
  r.partial = at<float>(t.partial, b);
  r.scale = at<float>(t.scale, b);
  return r;
}

__device__ __forceinline__ GemmTask resolve(const GemmTab& t, const Bases& b) {
  GemmTask r = __builtin_bit_cast(GemmTask, t);
  r.L = at<const void>(t.L, b);
  r.R0 = at<const void>(t.R0, b);
  r.R1 = at<const void>(t.R1, b);
  r.fbuf = at<float>(t.fbuf, b);
  r.out0 = at<void>(t.out0, b);
  r.out1 = at<void>(t.out1, b);
  r.out2 = at<void>(t.out2, b);
  r.scale = at<const float>(t.scale, b);
  r.xlo = at<uint16_t>(t.xlo, b);
  r.ahl = at<const uint16_t>(t.ahl, b);
  r.sink = at<void>(t.sink, b);
  r.dst = at<void>(t.dst, b);
  return r;
}

__device__ __forceinline__ NormTask resolve(const NormTab& t, const Bases& b) {
  NormTask r = __builtin_bit_cast(NormTask, t);
  r.partial = at<const float>(t.partial, b);
  r.scale = at<float>(t.scale, b);
  r.sumsq = at<float>(t.sumsq, b);
  return r;
}

__device__ __forceinline__ FinTask resolve(const FinTab& t, const Bases& b) {
  FinTask r = __builtin_bit_cast(FinTask, t);
  r.a = at<float>(t.a, b);
  r.sumsq = at<const float>(t.sumsq, b);
  r.scale = at<float>(t.scale, b);
  return r;
}

// Host-to-device upload through kernel arguments: n <= kUploadWords
// 8-byte words of one chunk go to dst.  Stream-ordered like any launch,
// with no host staging buffer and no device allocation.
struct UploadChunk {
  uint64_t* dst;
  int32_t n;
  int32_t pad_;
  uint64_t w[kUploadWords];
};

__global__ __launch_bounds__(kUploadWords) void upload_kernel(UploadChunk c) {
  const int i = threadIdx.x;
  if (i < c.n) *(uint64_t GMEM*)(c.dst + i) = c.w[i];
}

// The master copy of X, four consecutive elements at offset o (of the
// fp32 row stride ldx or the bf16 row stride ldxb): fp32 only (fp32
// operands); fp32 plus its bf16 rounding (bf16 operands, no xlo); or the
// bf16 rounding `hi` plus the bf16 rounding of the remainder (xlo given),
// which keeps about 16 significant bits.  The bf16 X is the SYRK operand.
__device__ __forceinline__ void store_master4(const EwTask& T, size_t row, int col, f32x4 u) {
  if (T.f32_ops) {
    st_f32x4(T.xm + row * T.ldx + col, u);
    return;
  }
  const u32x2 hi = pack_bf16x4(u[0], u[1], u[2], u[3]);
  st_u32x2(T.xb + row * T.ldxb + col, hi);
  if (T.xlo) {
    const f32x4 h = unpack_bf16x4(hi);
    st_u32x2(T.xlo + row * T.ldxb + col,
             pack_bf16x4(u[0] - h[0], u[1] - h[1], u[2] - h[2], u[3] - h[3]));
  } else {
    st_f32x4(T.xm + row * T.ldx + col, u);
  }
}

// --------------------------------------------------------------------------
// Momentum / input pass.  One 64 x 64 tile of the caller's layout per block:
//   buf <- mu*buf + g ; u <- nesterov ? g + mu*buf : buf   (or u <- G)
// u is written to the oriented workspace in both layouts (X and X^T, the
// transposed one through LDS), pads are written as zeros, and the tile's
// sum of u^2 goes to partial[tile].
__global__ __launch_bounds__(EW_THREADS) void momentum_kernel(
    const EwTab* __restrict__ tasks, int ntasks, int total_tiles, float mu,
    int nesterov, int ns_only, Bases bases) {
  __shared__ float tile[EW_TILE][EW_TILE + 1];
  __shared__ float wsum[EW_THREADS / 64];
  const int gt = blockIdx.x;
  if (gt >= total_tiles) return;
  // A copy, not a reference: stores through the task's pointers could
  // otherwise alias it and force a reload of every field after each store.
  const EwTask T = resolve(tasks[find_task(tasks, ntasks, gt)], bases);
  // 16-byte (fp32) / 8-byte (bf16) accesses of 4 elements when the caller's
  // buffers allow them
  const bool vec = T.n % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(T.src) % (T.in_dtype == 0 ? 16 : 8) == 0 &&
                   reinterpret_cast<uintptr_t>(T.buf) % 16 == 0;
  const int lt = gt - T.tile_begin;
  const int r0 = (lt / T.tiles_c) * EW_TILE;
  const int c0 = (lt % T.tiles_c) * EW_TILE;
  const int tid = threadIdx.x;
  const int cx = (tid & 15) * 4;
  const int ry = tid >> 4;
  const bool f32ops = T.f32_ops != 0;
  float ss = 0.f;

  // A whole tile inside the matrix (the common case) issues all its loads
  // before the first store: the stores to buf could alias later loads for
  // all the compiler knows, which would serialize the rows' round trips.
  constexpr int RK = EW_TILE / 16;  // rows per thread
  const bool interior = vec && r0 + EW_TILE <= T.m && c0 + EW_TILE <= T.n;
  f32x4 gpre[RK], bpre[RK];
  if (interior) {
#pragma unroll
    for (int k = 0; k < RK; ++k) {
      const size_t idx = (size_t)(r0 + ry + 16 * k) * T.n + c0 + cx;
      gpre[k] = load4(T.src, T.in_dtype, idx);
      if (!ns_only) bpre[k] = ld_f32x4_nt(T.buf + idx);
    }
  }

#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int r = ry + 16 * k;
    const int gr = r0 + r;
    const int gc = c0 + cx;
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
    if (gr < T.m && gc < T.n) {
      const size_t idx = (size_t)gr * T.n + gc;
      if (vec && gc + 3 < T.n) {
        const f32x4 g = interior ? gpre[k] : load4(T.src, T.in_dtype, idx);
        if (ns_only) {
          u = g;
        } else {
          const f32x4 b = interior ? bpre[k] : ld_f32x4(T.buf + idx);
          f32x4 bn;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bn[e] = fmaf(mu, b[e], g[e]);
            u[e] = nesterov ? fmaf(mu, bn[e], g[e]) : bn[e];
          }
          st_f32x4_nt(T.buf + idx, bn);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (gc + e < T.n) {
            const float g = load1(T.src, T.in_dtype, idx + e);
            if (ns_only) {
              u[e] = g;
            } else {
              const float bn = fmaf(mu, ld_f32(T.buf + idx + e), g);
              st_f32(T.buf + idx + e, bn);
              u[e] = nesterov ? fmaf(mu, bn, g) : bn;
            }
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss = fmaf(u[e], u[e], ss);
      tile[r][cx + e] = u[e];
    }
    // Same-layout copy: X itself for a wide matrix, X^T for a tall one.
    if (!T.transposed) {
      store_master4(T, (size_t)gr, gc, u);
    } else {
      const size_t o = (size_t)gr * T.ldt + gc;
      if (f32ops)
        st_f32x4(static_cast<float*>(T.xt) + o, u);
      else
        st_u32x2(static_cast<uint16_t*>(T.xt) + o, pack_bf16x4(u[0], u[1], u[2], u[3]));
    }
  }
  __syncthreads();
  // Transposed copy: X^T for a wide matrix, X (and its bf16 copy) for a tall one.
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int oc = ry + 16 * k;  // column of the tile = row of the output
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = tile[cx + e][oc];
    const int orow = c0 + oc;
    const int ocol = r0 + cx;
    if (!T.transposed) {
      const size_t o = (size_t)orow * T.ldt + ocol;
      if (f32ops)
        st_f32x4(static_cast<float*>(T.xt) + o, v);
      else
        st_u32x2(static_cast<uint16_t*>(T.xt) + o, pack_bf16x4(v[0], v[1], v[2], v[3]));
    } else {
      store_master4(T, (size_t)orow, ocol, v);
    }
  }
  // Block sum of squares, fixed order.
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < EW_THREADS / 64; ++w) s += wsum[w];
    st_f32(T.partial + gt, s);
  }
}

// --------------------------------------------------------------------------
// Norm finalize: one block per matrix sums its tiles' partials in fp64 in a
// fixed order and stores 1/(||u||_F + eps) and its square.
__global__ __launch_bounds__(256) void norm_kernel(const NormTab* __restrict__ tasks,
                                                   float eps, Bases bases) {
  __shared__ double wpart[4];
  const NormTask T = resolve(tasks[blockIdx.x], bases);
  double acc = 0.0;
  for (int i = threadIdx.x; i < T.tile_count; i += 256)
    acc += (double)ld_f32(T.partial + T.tile_begin + i);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) wpart[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = (wpart[0] + wpart[1]) + (wpart[2] + wpart[3]);
    if (T.sumsq) {  // a shard: the group's norm is not known yet
      st_f32(T.sumsq, (float)tot);
      st_f32(T.scale + 0, 1.f);
      st_f32(T.scale + 1, 1.f);
      st_f32(T.scale + 2, 0.f);
    } else {
      const double s = sqrt(tot);
      const double inv = 1.0 / (s + (double)eps);
      st_f32(T.scale + 0, (float)inv);
      st_f32(T.scale + 1, (float)(inv * inv));
      st_f32(T.scale + 2, (float)s);
    }
  }
}

// Gram-space NS with fp16 operands, once the norm is known: one 64 x 64
// tile of the oriented, padded X per block.  Reads the master X as the input
// pass left it (bf16 X + bf16 remainder, or fp32), scales it by
// 1/(||u|| + eps), and writes it back as the fp16 operands read it: the
// master as fp16 X + fp16 remainder times 2^11 (or fp32 beside an fp16
// copy), and fp16 X^T through LDS.  The window products then see X in
// fp16's normal range from the first SYRK on.
__global__ __launch_bounds__(EW_THREADS) void gram16_x_kernel(const EwTab* __restrict__ tasks,
                                                              int ntasks, int total_tiles,
                                                              Bases bases) {
  __shared__ float tile[EW_TILE][EW_TILE + 1];
  const int gt = blockIdx.x;
  if (gt >= total_tiles) return;
  const EwTask T = resolve(tasks[find_task(tasks, ntasks, gt)], bases);
  const int lt = gt - T.tile_begin;
  const int r0 = (lt / T.tiles_c) * EW_TILE;
  const int c0 = (lt % T.tiles_c) * EW_TILE;
  const int tid = threadIdx.x;
  const int cx = (tid & 15) * 4;
  const int ry = tid >> 4;
  const float s = ld_f32(T.scale);
  const bool hilo = T.xlo != nullptr;
  constexpr int RK = EW_TILE / 16;
  constexpr float ls = Op16<1>::kLoScale;
  f32x4 x[RK];
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const size_t row = (size_t)(r0 + ry + 16 * k);
    if (hilo) {
      const f32x4 h = unpack_bf16x4(ld_u32x2(T.xb + row * T.ldxb + c0 + cx));
      const f32x4 l = unpack_bf16x4(ld_u32x2(T.xlo + row * T.ldxb + c0 + cx));
#pragma unroll
      for (int e = 0; e < 4; ++e) x[k][e] = h[e] + l[e];
    } else {
      x[k] = ld_f32x4(T.xm + row * T.ldx + c0 + cx);
    }
  }
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int r = ry + 16 * k;
    const size_t row = (size_t)(r0 + r);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = x[k][e] * s;
      tile[r][cx + e] = v[e];
    }
    const u32x2 h4 = pack4<1>(v[0], v[1], v[2], v[3]);
    st_u32x2(T.xb + row * T.ldxb + c0 + cx, h4);
    if (hilo) {
      const f32x4 hf = unpack4<1>(h4);
      st_u32x2(T.xlo + row * T.ldxb + c0 + cx,
               pack4<1>((v[0] - hf[0]) * ls, (v[1] - hf[1]) * ls, (v[2] - hf[2]) * ls,
                        (v[3] - hf[3]) * ls));
    } else {
      st_f32x4(T.xm + row * T.ldx + c0 + cx, v);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int oc = ry + 16 * k;  // column of the tile = row of X^T
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = tile[cx + e][oc];
    st_u32x2(static_cast<uint16_t*>(T.xt) + (size_t)(c0 + oc) * T.ldt + r0 + cx,
             pack4<1>(v[0], v[1], v[2], v[3]));
  }
}

// Gram NS on a shard, after the group sum: inv = 1/(sqrt(sumsq) + eps) as in
// norm_kernel, A *= inv^2 (the same fp32 factor the SYRK epilogue applies
// when the norm is known up front), and the scales for the X update.
__global__ __launch_bounds__(256) void gram_finalize_kernel(const FinTab* __restrict__ tasks,
                                                            int ntasks, float eps, Bases bases) {
  const int b = blockIdx.x;
  const FinTask T = resolve(tasks[find_task(tasks, ntasks, b)], bases);
  const double tot = (double)ld_f32(T.sumsq);
  const double s = sqrt(tot);
  const double inv = 1.0 / (s + (double)eps);
  const float s2 = (float)(inv * inv);
  const int r0 = (b - T.tile_begin) * FIN_ROWS;
  const int r1 = min(r0 + FIN_ROWS, T.P);
  for (int r = r0; r < r1; ++r) {
    float* row = T.a + (size_t)r * T.ld;
    for (int c = 4 * threadIdx.x; c < T.P; c += 4 * 256) {
      f32x4 v = ld_f32x4(row + c);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] *= s2;
      st_f32x4(row + c, v);
    }
  }
  if (b == T.tile_begin && threadIdx.x == 0) {
    st_f32(T.scale + 0, (float)inv);
    st_f32(T.scale + 1, s2);
    st_f32(T.scale + 2, (float)s);
  }
}

// --------------------------------------------------------------------------
// Grouped NT GEMM on MFMA: C (T x T tile) = L[tm] * R[tn]^T over K, then a
// kind-specific epilogue.  256 threads = 4 waves in a 2 x 2 grid, each wave
// owns (T/2) x (T/2) = NT x NT blocks of 32 x 32 MFMA output.  K advances
// 128 bytes per stage (64 bf16 or 32 fp32) through double-buffered LDS rows
// padded by 16 bytes so that the 16-byte operand reads are conflict free.

// Workgroups are handed to the 8 XCDs round robin (workgroup b runs on XCD
// b % 8).  Tile order: windows of 8 * kXcdChunk consecutive tiles, XCD x
// taking the x-th contiguous chunk of each window, so that each XCD's L2
// sees neighbouring tiles while all XCDs work in the same region of the
// launch, whose operands the Infinity Cache (shared by the XCDs) then holds
// once.  The last, partial window is split evenly; a launch of less than
// one window gets one contiguous range per XCD.  Measured against giving
// each XCD one contiguous eighth of the launch: Llama-8B step 83.2 -> 74.0
// ms, 70B MLP step 218 -> 209 ms.  `grid` is total rounded up to 8.
constexpr int kXcdChunk = 32;
__device__ __forceinline__ int xcd_remap(int b, int grid, int total) {
  constexpr int W = 8 * kXcdChunk;
  const int full = total / W * W;
  if (b < full) return b / W * W + (b & 7) * kXcdChunk + ((b >> 3) & (kXcdChunk - 1));
  const int c = (grid - full) >> 3;  // chunk per XCD in the last window
  return full + (b & 7) * c + ((b - full) >> 3);
}

constexpr int GROUP = 8;  // tile rows per group of the full-product order

// Upper-triangle tile order in 8 x 8 super-tiles (row-major over the
// super-tiles, row-major inside), so concurrently running tiles share
// operand panels.
__device__ __forceinline__ void tri_decode(int t, int nt, int& tm, int& tn) {
  const int ns = (nt + GROUP - 1) / GROUP;
  for (int si = 0; si < ns; ++si) {
    const int rows = min(GROUP, nt - si * GROUP);
    for (int sj = si; sj < ns; ++sj) {
      const int cols = min(GROUP, nt - sj * GROUP);
      const int cnt = (si == sj) ? rows * (rows + 1) / 2 : rows * cols;
      if (t < cnt) {
        if (si == sj) {
          int r = 0;
          while (t >= rows - r) { t -= rows - r; ++r; }
          tm = si * GROUP + r;
          tn = si * GROUP + r + t;
        } else {
          tm = si * GROUP + t / cols;
          tn = sj * GROUP + t % cols;
        }
        return;
      }
      t -= cnt;
    }
  }
  tm = tn = 0;  // not reached for t < nt(nt+1)/2
}

// Full-product order in column windows, for a matrix whose tiles start at
// a multiple of 8 * kXcdChunk in the launch and fill whole windows (the host
// checks; tiles_m 8, 16, 32 or 64): window W holds all tile rows
// of 8 * kXcdChunk / tiles_m tile columns, and XCD x (chunk x of the window
// in xcd_remap's order) takes an 8-row by 4-column block of it.  Each XCD's
// L2 sees the same 12 operand panels per wave of tiles as in full_decode's
// order, but a panel of the short operand (rows) is fetched again in every
// window while it is still in the Infinity Cache, and a panel of the long
// one (columns) is fetched once per launch instead of once per group of 8
// tile rows.  Measured on the operand stream of a 8192 x 28672 X update:
// 5% more bytes per clock.
__device__ __forceinline__ void win_decode(int t, int tiles_m, int& tm, int& tn) {
  constexpr int W = 8 * kXcdChunk;
  const int r = t % W, x = r / kXcdChunk, i = r % kXcdChunk;
  const int rb = tiles_m / 8;  // 8-row blocks of a window
  tm = (x % rb) * 8 + (i & 7);
  tn = (t / W) * (W / tiles_m) + (x / rb) * 4 + (i >> 3);
}

__device__ __forceinline__ void full_decode(int t, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  const int group = t / (GROUP * tiles_n);
  const int first = group * GROUP;
  const int gsz = min(GROUP, tiles_m - first);
  const int w = t - group * GROUP * tiles_n;
  tm = first + w % gsz;
  tn = w / gsz;
}

// Epilogues of one T x T output tile.  32x32 MFMA output layout: lane l,
// register r holds row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of its
// block; a wave's row of NT blocks is handled at a time, with every global
// load of that row issued before the first use (no branch in between), so
// the loads overlap instead of costing one round trip each.

// SYRK (A = s X X^T), POLY (B = b A + c A A^T, plus a I for Gram-space P)
// and GRAMMUL (C = L R^T) tiles of the upper triangle; off-diagonal tiles
// are also written mirrored.  AHL: POLY reads
// A as hi + lo from the split operand rows instead of the fp32 A.
template <int KIND, int T, bool F32, int NT, bool AHL, int H>
__device__ __forceinline__ void sym_epilogue(const GemmTask& G, f32x16 (&acc)[NT][NT], int tm,
                                             int tn, int wr, int wc, int lane,
                                             const IterArgs& A) {
  const int row_base = tm * T + wr + 4 * (lane >> 5);
  const int col_base = tn * T + wc + (lane & 31);
  const bool mirror = G.tri && (tm != tn);
  const float s = (KIND == KIND_SYRK && A.iter == 0) ? G.scale[1] : 1.f;
  // 16-bit operands: A is stored times kA, so the POLY product A A^T comes
  // times kA^2 (undone by folding 1/kA^2 into c, exactly); B is stored
  // times kB
  constexpr float kA = Op16<H>::kAScale, kB = Op16<H>::kBScale;
  const float cb = A.b, cc = (F32 || KIND != KIND_POLY) ? A.c : A.c * (1.f / (kA * kA));
  const int P = G.P;
  float* F = G.fbuf;
  const int ldf = G.ld_f;

#pragma unroll
  for (int i = 0; i < NT; ++i) {
    f32x4 av[NT][4];  // POLY: the A values of this block row
    if constexpr (KIND == KIND_POLY) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int r = row_base + i * 32 + 8 * g + rr, c = col_base + j * 32;
            if constexpr (AHL) {
              const uint16_t* h = G.ahl + (size_t)r * G.ld_ahl + c;
              av[j][g][rr] = from_bf16(ld_u16(h)) + from_bf16(ld_u16(h + P));
            } else {
              av[j][g][rr] = ld_f32(F + (size_t)r * ldf + c);
            }
          }
      // keep the loads together: the scheduler would otherwise sink each
      // one to its use to save registers, serializing the round trips
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gi = row_base + i * 32 + 8 * g;  // rows gi .. gi+3
        const int gj = col_base + j * 32;
        f32x4 v;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) v[rr] = acc[i][j][4 * g + rr];

        if constexpr (KIND == KIND_SYRK) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) v[rr] *= s;
          if (!G.split) {
            // fp32 A: with bf16 operands only the polynomial epilogue reads
            // it, on upper tiles, so the mirrored tile is written only when
            // A is itself the fp32 operand
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) st_f32(F + (size_t)(gi + rr) * ldf + gj, v[rr]);
            if (F32 && mirror) st_f32x4(F + (size_t)gj * ldf + gi, v);
          }
          if constexpr (!F32) {
            uint16_t* o0 = static_cast<uint16_t*>(G.out0);
            const int ld0 = G.ld0;
            if (H == 1 || !G.split) {
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) st_u16(o0 + (size_t)(gi + rr) * ld0 + gj, Op16<H>::to(v[rr] * kA));
              if (mirror)
                st_u32x2(o0 + (size_t)gj * ld0 + gi, pack4<H>(v[0] * kA, v[1] * kA, v[2] * kA, v[3] * kA));
            } else if constexpr (H == 0) {  // the split modes are bf16 only
              // Rows [hi | lo | hi | hi] along K (4P).  The polynomial
              // product pairs columns 0..3P (hi, lo, hi) with columns
              // P..4P (lo, hi, hi): hi lo^T + lo hi^T + hi hi^T.
              const u32x2 h4 = pack_bf16x4(v[0], v[1], v[2], v[3]);
              const f32x4 hf = unpack_bf16x4(h4);
              const u32x2 l4 =
                  pack_bf16x4(v[0] - hf[0], v[1] - hf[1], v[2] - hf[2], v[3] - hf[3]);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const size_t o = (size_t)(gi + rr) * ld0 + gj;
                const uint16_t h = (uint16_t)((rr & 1 ? h4[rr >> 1] >> 16 : h4[rr >> 1]) & 0xffffu);
                const uint16_t l = (uint16_t)((rr & 1 ? l4[rr >> 1] >> 16 : l4[rr >> 1]) & 0xffffu);
                st_u16(o0 + o, h); st_u16(o0 + o + P, l);
                st_u16(o0 + o + 2 * P, h); st_u16(o0 + o + 3 * P, h);
              }
              if (mirror) {
                const size_t o = (size_t)gj * ld0 + gi;
                st_u32x2(o0 + o, h4);
                st_u32x2(o0 + o + P, l4);
                st_u32x2(o0 + o + 2 * P, h4);
                st_u32x2(o0 + o + 3 * P, h4);
              }
            }
          }
        } else if constexpr (KIND == KIND_GRAMMUL) {
          // C = L R^T (L, R symmetric and commuting, so C is symmetric)
          if constexpr (F32) {
            float* o0 = static_cast<float*>(G.out0);
            const int ld0 = G.ld0;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) st_f32(o0 + (size_t)(gi + rr) * ld0 + gj, v[rr]);
            if (mirror) st_f32x4(o0 + (size_t)gj * ld0 + gi, v);
          } else {
            // fp16 operands: unscale; the fp32 C (upper tiles, for the
            // polynomial's linear term) when asked for, and the fp16
            // operand form times g_out, mirrored
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v[rr] *= G.g_in;
            if (F) {
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) st_f32(F + (size_t)(gi + rr) * ldf + gj, v[rr]);
            }
            uint16_t* o0 = static_cast<uint16_t*>(G.out0);
            const int ld0 = G.ld0;
            const float go = G.g_out;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) st_u16(o0 + (size_t)(gi + rr) * ld0 + gj, Op16<H>::to(v[rr] * go));
            if (mirror)
              st_u32x2(o0 + (size_t)gj * ld0 + gi, pack4<H>(v[0] * go, v[1] * go, v[2] * go, v[3] * go));
          }
        } else {  // KIND_POLY
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) v[rr] = fmaf(cb, av[j][g][rr], cc * v[rr]);
          if (G.add_diag) {  // Gram-space P = a I + b A + c A^2
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (gi + rr == gj) v[rr] += A.a;
          }
          if constexpr (F32) {
            float* o0 = static_cast<float*>(G.out0);
            const int ld0 = G.ld0;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) st_f32(o0 + (size_t)(gi + rr) * ld0 + gj, v[rr]);
            if (mirror) st_f32x4(o0 + (size_t)gj * ld0 + gi, v);
          } else {
            uint16_t* o0 = static_cast<uint16_t*>(G.out0);
            const int ld0 = G.ld0;
            if (H == 1 || !G.split) {
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) st_u16(o0 + (size_t)(gi + rr) * ld0 + gj, Op16<H>::to(v[rr] * kB));
              if (mirror)
                st_u32x2(o0 + (size_t)gj * ld0 + gi, pack4<H>(v[0] * kB, v[1] * kB, v[2] * kB, v[3] * kB));
            } else if constexpr (H == 0) {  // the split modes are bf16 only
              // [hi | lo] along K (2P); the B X product pairs both halves
              // with the same X^T.
              f32x4 hi, lo;
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                hi[rr] = from_bf16(to_bf16(v[rr]));
                lo[rr] = v[rr] - hi[rr];
              }
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const size_t o = (size_t)(gi + rr) * ld0 + gj;
                st_u16(o0 + o, to_bf16(hi[rr]));
                st_u16(o0 + o + P, to_bf16(lo[rr]));
              }
              if (mirror) {
                const size_t o = (size_t)gj * ld0 + gi;
                st_u32x2(o0 + o, pack_bf16x4(hi[0], hi[1], hi[2], hi[3]));
                st_u32x2(o0 + o + P, pack_bf16x4(lo[0], lo[1], lo[2], lo[3]));
              }
            }
          }
        }
      }
  }
}

// How bf16-operand tiles of size T keep the master X: as bf16 X plus its
// bf16 remainder (T < 256: fewer bytes, and at several blocks per CU the
// extra access instructions are hidden), or in fp32 next to the bf16 copy
// (T = 256: one block per CU, where the epilogue is bound by the number of
// memory instructions).  The host picks the same layout per tile size.
template <int T>
constexpr bool kHiLoMaster = T < 256;

// The master X at (r, c): fp32, or xb + xlo / kLoScale in format H.
template <bool F32, bool HL, int H>
__device__ __forceinline__ float load_master(const GemmTask& G, int r, int c) {
  if constexpr (!F32 && !HL) {  // 256-wide tiles: streamed (see ld_f32_nt)
    return ld_f32_nt(G.fbuf + (size_t)r * G.ld_f + c);
  } else if constexpr (F32) {
    return ld_f32(G.fbuf + (size_t)r * G.ld_f + c);
  } else {
    const size_t o = (size_t)r * G.ld0 + c;
    return Op16<H>::from(ld_u16(static_cast<const uint16_t*>(G.out0) + o)) +
           Op16<H>::from(ld_u16(G.xlo + o)) * (1.f / Op16<H>::kLoScale);
  }
}

// UPDX, not the last iteration: X <- s (a X + B X_raw) with s = 1/(||u||+eps)
// on iteration 0.  Writes the master X (fp32, or bf16 X and its bf16
// remainder), and X^T: in fp32 with fp32 operands, else in bf16 transposed
// through LDS (8-byte groups XOR-swizzled) so that it leaves the tile as
// full rows.
template <int T, bool F32, int NT, int H, int HN>
__device__ __forceinline__ void updx_epilogue(const GemmTask& G, f32x16 (&acc)[NT][NT], int tm,
                                              int tn, int wr, int wc, int lane,
                                              const IterArgs& A, uint16_t* stage) {
  constexpr bool HL = kHiLoMaster<T>;
  if constexpr (!F32) __syncthreads();  // main-loop LDS reads are done
  const int row_base = tm * T + wr + 4 * (lane >> 5);
  const int col_base = tn * T + wc + (lane & 31);
  const float s = A.iter == 0 ? G.scale[0] : 1.f;
  const float ca = A.a;
  float* X = G.fbuf;
  const int ldf = G.ld_f;
  void* xt_next = (A.iter & 1) ? G.out1 : G.out2;
  const int ld1 = G.ld1;

#pragma unroll
  for (int i = 0; i < NT; ++i) {
    f32x4 xv[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          xv[j][g][rr] = load_master<F32, HL, H>(G, row_base + i * 32 + 8 * g + rr,
                                                 col_base + j * 32);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads together (see sym_epilogue)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gi = row_base + i * 32 + 8 * g;  // rows gi .. gi+3
        const int gj = col_base + j * 32;
        f32x4 v;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          v[rr] = s * fmaf(ca, xv[j][g][rr], acc[i][j][4 * g + rr] * (1.f / Op16<H>::kBScale));
        if constexpr (F32) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) st_f32(X + (size_t)(gi + rr) * ldf + gj, v[rr]);
          st_f32x4(static_cast<float*>(xt_next) + (size_t)gj * ld1 + gi, v);
        } else if constexpr (!HL) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) st_f32_nt(X + (size_t)(gi + rr) * ldf + gj, v[rr]);
          uint16_t* xb = static_cast<uint16_t*>(G.out0);
          const int ld0 = G.ld0;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) st_u16_nt(xb + (size_t)(gi + rr) * ld0 + gj, Op16<HN>::to(v[rr]));
          const int il = gi - tm * T, jl = gj - tn * T;
          const int x = 4 * (jl & (T / 4 - 1));
          *reinterpret_cast<u32x2*>(stage + jl * T + (il ^ x)) = pack4<HN>(v[0], v[1], v[2], v[3]);
        } else {
          uint16_t* xb = static_cast<uint16_t*>(G.out0);
          const int ld0 = G.ld0;
          const u32x2 h4 = pack4<HN>(v[0], v[1], v[2], v[3]);
          const f32x4 hf = unpack4<HN>(h4);
          constexpr float ls = Op16<HN>::kLoScale;
          const u32x2 l4 = pack4<HN>((v[0] - hf[0]) * ls, (v[1] - hf[1]) * ls,
                                     (v[2] - hf[2]) * ls, (v[3] - hf[3]) * ls);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const size_t o = (size_t)(gi + rr) * ld0 + gj;
            st_u16(xb + o, (uint16_t)((rr & 1 ? h4[rr >> 1] >> 16 : h4[rr >> 1]) & 0xffffu));
            st_u16(G.xlo + o, (uint16_t)((rr & 1 ? l4[rr >> 1] >> 16 : l4[rr >> 1]) & 0xffffu));
          }
          const int il = gi - tm * T, jl = gj - tn * T;
          const int x = 4 * (jl & (T / 4 - 1));
          *reinterpret_cast<u32x2*>(stage + jl * T + (il ^ x)) = h4;
        }
      }
  }
  if constexpr (!F32) {
    __syncthreads();
    uint16_t* xt = static_cast<uint16_t*>(xt_next);
    constexpr int CPR = T / 8;            // 16-byte chunks per row
    constexpr int RPP = 256 / CPR;        // rows per pass of the block
    const int tid = threadIdx.x;
    const int c = tid % CPR;
#pragma unroll 4
    for (int jl = tid / CPR; jl < T; jl += RPP) {
      const int x = 4 * (jl & (T / 4 - 1));
      const int pos = (8 * c) ^ x;
      u32x4 w = *reinterpret_cast<const u32x4*>(stage + jl * T + (pos & ~7));
      if (pos & 4) { const uint32_t a = w.x, b = w.y; w.x = w.z; w.y = w.w; w.z = a; w.w = b; }
      st_u32x4(xt + (size_t)(tn * T + jl) * ld1 + tm * T + 8 * c, w);
    }
  }
}

// UPDX, last iteration: the new X goes straight to the caller's buffer
// (dtype DT: 0 fp32, 1 bf16), as p <- p*decay - lr*O (FIN_UPDATE) or as
// O (FIN_OUTPUT).  Oriented element (r, c) lives at dst[r*qv + c], or at
// dst[c*pv + r] for a transposed caller matrix.  Lanes on padding (outside
// pv x qv) load dst element 0 and store into the task's sink (workspace
// bytes nothing reads): every access is unconditional, so no branch
// separates the loads from their uses.
template <int DT>
__device__ __forceinline__ float dst_load(const void* dst, size_t i) {
  if constexpr (DT == 0) return ld_f32(static_cast<const float*>(dst) + i);
  else return from_bf16(ld_u16(static_cast<const uint16_t*>(dst) + i));
}

template <int DT>
__device__ __forceinline__ void dst_store(void* p, float v) {
  if constexpr (DT == 0) st_f32(static_cast<float*>(p), v);
  else st_u16(static_cast<uint16_t*>(p), to_bf16(v));
}

template <int T, bool F32, int NT, int DT, int H>
__device__ __forceinline__ void updx_final(const GemmTask& G, f32x16 (&acc)[NT][NT], int tm,
                                           int tn, int wr, int wc, int lane,
                                           const IterArgs& A) {
  const int row_base = tm * T + wr + 4 * (lane >> 5);
  const int col_base = tn * T + wc + (lane & 31);
  const float s = A.iter == 0 ? G.scale[0] : 1.f;
  const float ca = A.a;
  void* dst = G.dst;
  constexpr int ESZ = DT == 0 ? 4 : 2;
  const int pv = G.pv, qv = G.qv;
  // strides of the oriented row and column index in the caller's buffer
  const size_t rs = G.dst_trans ? 1 : (size_t)qv;
  const size_t cs = G.dst_trans ? (size_t)pv : 1;
  const bool upd = A.fin == FIN_UPDATE;

#pragma unroll
  for (int i = 0; i < NT; ++i) {
    f32x4 xv[NT][4], pv4[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          xv[j][g][rr] = load_master<F32, kHiLoMaster<T>, H>(G, row_base + i * 32 + 8 * g + rr,
                                                             col_base + j * 32);
    if (upd) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int r = row_base + i * 32 + 8 * g + rr, c = col_base + j * 32;
            const size_t idx = (r < pv && c < qv) ? r * rs + c * cs : 0;
            pv4[j][g][rr] = dst_load<DT>(dst, idx);
          }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads together (see sym_epilogue)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = row_base + i * 32 + 8 * g + rr, c = col_base + j * 32;
          float o = s * fmaf(ca, xv[j][g][rr], acc[i][j][4 * g + rr] * (1.f / Op16<H>::kBScale));
          if (upd) o = fmaf(-A.lr, o, pv4[j][g][rr] * A.decay);
          char* to = (r < pv && c < qv) ? static_cast<char*>(dst) + (r * rs + c * cs) * ESZ
                                        : static_cast<char*>(G.sink);
          dst_store<DT>(to, o);
        }
  }
}

// Dispatch of a finished tile to its epilogue.
// UPDX, not the last iteration, bf16 hi/lo master (tiles below 256): the
// accumulators pass through LDS in slabs of R rows, so that every thread
// then owns 8-column row chunks and the master's two bf16 halves move in
// 16-byte loads and stores (in the 32x32 output layout each lane holds 4
// rows of one column, which costs one 2-byte access per element and
// half).  The chunks' master loads go out before the barrier that
// publishes the slab.  The new hi X also goes, transposed, into the bf16
// stage the X^T rows are written from (same swizzle as updx_epilogue).
// LDS: T*T bf16 stage, then R x (T+8) fp32 rows (row stride T+8 puts the
// two half-waves' rows on disjoint banks): 26 KB (T=64), 49 KB (T=128).
template <int T, int NT, int H, int HN>
__device__ __forceinline__ void updx_epilogue_hl(const GemmTask& G, f32x16 (&acc)[NT][NT],
                                                 int tm, int tn, int wr, int wc, int lane,
                                                 const IterArgs& A, uint16_t* lds) {
  constexpr int RB = T == 64 ? 2 : 1;  // 32-row blocks per slab
  constexpr int R = 32 * RB;
  constexpr int LDR = T + 8;
  constexpr int CPR = T / 8;            // 8-column chunks per row
  constexpr int CPT = R * CPR / 256;    // chunks per thread per slab
  static_assert(CPT >= 1 && (R * CPR) % 256 == 0, "slab shape");
  uint16_t* stage = lds;
  float* rows = reinterpret_cast<float*>(lds + T * T);
  const int tid = threadIdx.x;
  const float s = A.iter == 0 ? G.scale[0] : 1.f;
  const float ca = A.a;
  const int ld0 = G.ld0;
  uint16_t* xb = static_cast<uint16_t*>(G.out0);
  uint16_t* xlo = G.xlo;
  __syncthreads();  // main-loop LDS reads are done

#pragma unroll
  for (int r0 = 0; r0 < T; r0 += R) {
    u32x4 hv[CPT], lv[CPT];
    size_t go[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int id = tid + 256 * k;
      go[k] = (size_t)(tm * T + r0 + id / CPR) * ld0 + tn * T + 8 * (id % CPR);
      hv[k] = *(const GMEM u32x4*)(xb + go[k]);
      lv[k] = *(const GMEM u32x4*)(xlo + go[k]);
    }
    // the waves holding the slab's rows write them
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int br = r0 + 32 * b;  // tile row of this 32-row block
#pragma unroll
      for (int i = 0; i < NT; ++i)
        if (wr + 32 * i == br) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr)
                rows[(32 * b + 8 * g + 4 * (lane >> 5) + rr) * LDR + wc + 32 * j + (lane & 31)] =
                    acc[i][j][4 * g + rr];
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int id = tid + 256 * k;
      const int rl = id / CPR, c = 8 * (id % CPR);
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(rows + rl * LDR + c);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(rows + rl * LDR + c + 4);
      const uint32_t hw[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
      const uint32_t lw[4] = {lv[k].x, lv[k].y, lv[k].z, lv[k].w};
      uint32_t ho[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        constexpr float rin = 1.f / Op16<H>::kLoScale, lout = Op16<HN>::kLoScale;
        const float x0 = Op16<H>::e0(hw[e]) + Op16<H>::e0(lw[e]) * rin;
        const float x1 = Op16<H>::e1(hw[e]) + Op16<H>::e1(lw[e]) * rin;
        const float acc0 = e < 2 ? a0[2 * e] : a1[2 * e - 4];
        const float acc1 = e < 2 ? a0[2 * e + 1] : a1[2 * e - 3];
        constexpr float rb = 1.f / Op16<H>::kBScale;  // B was stored times kB
        const float v0 = s * fmaf(ca, x0, acc0 * rb), v1 = s * fmaf(ca, x1, acc1 * rb);
        ho[e] = Op16<HN>::to2(v0, v1);
        lo[e] = Op16<HN>::to2((v0 - Op16<HN>::e0(ho[e])) * lout, (v1 - Op16<HN>::e1(ho[e])) * lout);
      }
      *(GMEM u32x4*)(xb + go[k]) = u32x4{ho[0], ho[1], ho[2], ho[3]};
      *(GMEM u32x4*)(xlo + go[k]) = u32x4{lo[0], lo[1], lo[2], lo[3]};
      const int il = r0 + rl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jl = c + e;
        const int x = 4 * (jl & (T / 4 - 1));
        stage[jl * T + (il ^ x)] = (uint16_t)(e & 1 ? ho[e >> 1] >> 16 : ho[e >> 1] & 0xffffu);
      }
    }
    __syncthreads();  // the slab is read before the next one is written
  }

  // X^T from the stage, as full rows
  uint16_t* xt = static_cast<uint16_t*>((A.iter & 1) ? G.out1 : G.out2);
  const int ld1 = G.ld1;
  constexpr int RPP = 256 / CPR;  // rows per pass of the block
  const int c = tid % CPR;
#pragma unroll 4
  for (int jl = tid / CPR; jl < T; jl += RPP) {
    const int x = 4 * (jl & (T / 4 - 1));
    const int pos = (8 * c) ^ x;
    u32x4 w = *reinterpret_cast<const u32x4*>(stage + jl * T + (pos & ~7));
    if (pos & 4) { const uint32_t a = w.x, b = w.y; w.x = w.z; w.y = w.w; w.z = a; w.w = b; }
    st_u32x4(xt + (size_t)(tn * T + jl) * ld1 + tm * T + 8 * c, w);
  }
}

// SYRK epilogue with A split into [hi | lo | hi | hi] bf16 rows (tiles
// below 256): the scaled tile passes through LDS in slabs of 64 rows; each
// thread then writes 8-column row chunks of the four segments, and for an
// off-diagonal tile 8-row column chunks of the mirrored tile, as 16-byte
// stores (in the 32x32 output layout each element costs four 2-byte stores
// and the mirror 8-byte ones).  Same values as sym_epilogue.  LDS: 64 x
// (T+8) fp32 (T+8: the two half-waves' rows on disjoint banks).
template <int T, int NT>
__device__ __forceinline__ void syrk_split_epilogue(const GemmTask& G, f32x16 (&acc)[NT][NT],
                                                    int tm, int tn, int wr, int wc, int lane,
                                                    const IterArgs& A, uint16_t* lds) {
  constexpr int R = 64;
  constexpr int LDR = T + 8;
  constexpr int CPT = R * T / 8 / 256;  // chunks per thread per slab, each direction
  static_assert((R * T / 8) % 256 == 0 && R % 32 == 0, "slab shape");
  float* rows = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x;
  const float s = A.iter == 0 ? G.scale[1] : 1.f;
  const bool mirror = tm != tn;
  const int P = G.P;
  const int ld0 = G.ld0;
  uint16_t* o0 = static_cast<uint16_t*>(G.out0);
  auto put = [&](size_t o, const float (&v)[8]) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = to_bf16x2(v[2 * e], v[2 * e + 1]);
      l[e] = to_bf16x2(v[2 * e] - __uint_as_float(h[e] << 16),
                       v[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u));
    }
    const u32x4 hv = {h[0], h[1], h[2], h[3]}, lv = {l[0], l[1], l[2], l[3]};
    st_u32x4(o0 + o, hv);
    st_u32x4(o0 + o + P, lv);
    st_u32x4(o0 + o + 2 * P, hv);
    st_u32x4(o0 + o + 3 * P, hv);
  };
  __syncthreads();  // main-loop LDS reads are done
#pragma unroll
  for (int r0 = 0; r0 < T; r0 += R) {
#pragma unroll
    for (int b = 0; b < R / 32; ++b)
#pragma unroll
      for (int i = 0; i < NT; ++i)
        if (wr + 32 * i == r0 + 32 * b) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr)
                rows[(32 * b + 8 * g + 4 * (lane >> 5) + rr) * LDR + wc + 32 * j + (lane & 31)] =
                    s * acc[i][j][4 * g + rr];
        }
    __syncthreads();
    // row chunks: tile row r0 + rl, columns c .. c+7
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int id = tid + 256 * k;
      const int rl = id / (T / 8), c = 8 * (id % (T / 8));
      float v[8];
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(rows + rl * LDR + c);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(rows + rl * LDR + c + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = a0[e]; v[4 + e] = a1[e]; }
      put((size_t)(tm * T + r0 + rl) * ld0 + tn * T + c, v);
    }
    // mirrored tile: row tn*T + c, columns tm*T + r0 + r8 .. +7
    if (mirror) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int id = tid + 256 * k;
        const int c = id % T, r8 = 8 * (id / T);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = rows[(r8 + e) * LDR + c];
        put((size_t)(tn * T + c) * ld0 + tm * T + r0 + r8, v);
      }
    }
    __syncthreads();  // the slab is read before the next one is written
  }
}

// H: the operand format of this launch's products (and of the A or B it
// writes); HN: the format of the X copies an X update writes for the next
// iteration.  The split modes are bf16 only.
template <int KIND, int T, bool F32, int NT, int H = 0, int HN = H>
__device__ __forceinline__ void epilogue(const GemmTask& G, f32x16 (&acc)[NT][NT], int tm, int tn,
                                         int wr, int wc, int lane, const IterArgs& A,
                                         uint16_t* stage) {
  if constexpr (KIND == KIND_UPDX) {
    if (A.fin == FIN_NONE) {
      if constexpr (!F32 && kHiLoMaster<T>)
        updx_epilogue_hl<T, NT, H, HN>(G, acc, tm, tn, wr, wc, lane, A, stage);
      else
        updx_epilogue<T, F32, NT, H, HN>(G, acc, tm, tn, wr, wc, lane, A, stage);
    }
    else if (G.dst_dtype == 0)
      updx_final<T, F32, NT, 0, H>(G, acc, tm, tn, wr, wc, lane, A);
    else
      updx_final<T, F32, NT, 1, H>(G, acc, tm, tn, wr, wc, lane, A);
  } else if constexpr (KIND == KIND_SYRK && !F32 && T < 256 && H == 0) {
    if (G.split)
      syrk_split_epilogue<T, NT>(G, acc, tm, tn, wr, wc, lane, A, stage);
    else
      sym_epilogue<KIND, T, F32, NT, false, H>(G, acc, tm, tn, wr, wc, lane, A);
  } else if constexpr (KIND == KIND_POLY && !F32 && H == 0) {
    if (G.ahl)
      sym_epilogue<KIND, T, F32, NT, true, H>(G, acc, tm, tn, wr, wc, lane, A);
    else
      sym_epilogue<KIND, T, F32, NT, false, H>(G, acc, tm, tn, wr, wc, lane, A);
  } else {
    sym_epilogue<KIND, T, F32, NT, false, H>(G, acc, tm, tn, wr, wc, lane, A);
  }
}

template <int KIND, int T, bool F32>
__global__ __launch_bounds__(256) void gemm_reg_kernel(const GemmTab* __restrict__ tasks,
                                                   int ntasks, int total_tiles, IterArgs A,
                                                   Bases bases) {
  using E = typename std::conditional<F32, float, uint16_t>::type;
  constexpr int ESZ = sizeof(E);
  constexpr int BK = 128 / ESZ;           // K elements per stage
  constexpr int VEC = 16 / ESZ;           // elements per 16-byte chunk
  constexpr int STRIDE = BK + VEC;        // LDS row stride in elements
  constexpr int WT = T / 2;               // wave tile
  constexpr int NT = WT / 32;             // 32x32 MFMA blocks per wave side
  constexpr int LOADS = T * 8 / 256;      // 16-byte chunks per thread per operand
  __shared__ __attribute__((aligned(16))) E lds[2][2][T * STRIDE];

  const int vb = xcd_remap(blockIdx.x, gridDim.x, total_tiles);
  if (vb >= total_tiles) return;
  // By value (see momentum_kernel): the epilogue's stores must not force
  // reloads of the descriptor.
  const GemmTask G = resolve(tasks[find_task(tasks, ntasks, vb)], bases);
  const int lt = vb - G.tile_begin;
  int tm, tn;
  if (G.tri)
    tri_decode(lt, G.tiles_m, tm, tn);
  else
    full_decode(lt, G.tiles_m, G.tiles_n, tm, tn);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = (wave >> 1) * WT;
  const int wc = (wave & 1) * WT;

  const E* __restrict__ Lp = static_cast<const E*>(G.L) + (size_t)tm * T * G.ldl;
  const E* __restrict__ Rp =
      static_cast<const E*>((A.iter & 1) ? G.R1 : G.R0) + (size_t)tn * T * G.ldr;
  const int ldl = G.ldl, ldr = G.ldr, kper = G.kper;
  const int nk = G.K / BK;

  uint4 regL[LOADS], regR[LOADS];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    const int kr = k0 % kper;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3;
      const int col = (c & 7) * VEC;
      regL[i] = ld_u128(Lp + (size_t)row * ldl + k0 + col);
      regR[i] = ld_u128(Rp + (size_t)row * ldr + kr + col);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3;
      const int col = (c & 7) * VEC;
      *reinterpret_cast<uint4*>(&lds[st][0][row * STRIDE + col]) = regL[i];
      *reinterpret_cast<uint4*>(&lds[st][1][row * STRIDE + col]) = regR[i];
    }
  };

  f32x16 acc[NT][NT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int st) {
    const E* sL = lds[st][0];
    const E* sR = lds[st][1];
    const int lrow = lane & 31;
    const int khalf = lane >> 5;
    if constexpr (!F32) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 a[NT], b[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          a[t] = *reinterpret_cast<const bf16x8*>(
              &sL[(wr + t * 32 + lrow) * STRIDE + ks * 16 + khalf * 8]);
          b[t] = *reinterpret_cast<const bf16x8*>(
              &sR[(wc + t * 32 + lrow) * STRIDE + ks * 16 + khalf * 8]);
        }
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // fp32: each lane reads 4 consecutive k; instruction t of a group
      // takes element t, so lane half h covers k = 8*ks + 4*h + t.
#pragma unroll
      for (int ks = 0; ks < BK / 8; ++ks) {
        f32x4 a[NT], b[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          a[t] = *reinterpret_cast<const f32x4*>(
              &sL[(wr + t * 32 + lrow) * STRIDE + ks * 8 + khalf * 4]);
          b[t] = *reinterpret_cast<const f32x4*>(
              &sR[(wc + t * 32 + lrow) * STRIDE + ks * 8 + khalf * 4]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    compute(st);
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  epilogue<KIND, T, F32, NT>(G, acc, tm, tn, wr, wc, lane, A, nullptr);
}

// fp32 SYRK and polynomial of small matrices (direct NS, min side <= 256)
// on 16 x 16 output tiles, so a launch of a few small matrices spreads over
// all CUs (the fp32 TinyMLP d=256: 408 blocks, against 30 of 64 x 64 and 108
// of 32 x 32; each block is bound by one CU's fp32 MFMA rate).  The block's
// 4 waves each take a quarter of K, straight from global memory (the
// operands are L2-resident at these sizes), and add their partials through
// LDS in wave order -- a fixed order, inside the block, so no device-scope
// synchronization -- before wave 0 writes the tile.  fp32 MFMA 16x16x4:
// lane quarter q supplies k = k0 + 4q + t to instruction t of a group of 4
// (both operands); the output holds rows 4q + i (i < 4) of column lane %
// 16.  K (the task's padded extent, a multiple of 64) splits into 4 x
// 16-aligned quarters.  The SYRK writes the fp32 A (scaled on iteration 0)
// and the polynomial B = b A + c A A^T, both mirrored on off-diagonal tiles.
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_small_kernel(const GemmTab* __restrict__ tasks,
                                                        int ntasks, int total_tiles, IterArgs A,
                                                        Bases bases) {
  static_assert(KIND == KIND_SYRK || KIND == KIND_POLY, "SYRK and polynomial only");
  constexpr int T = 16;
  __shared__ f32x4 part[3][64];
  const int vb = xcd_remap(blockIdx.x, gridDim.x, total_tiles);
  if (vb >= total_tiles) return;
  const GemmTask G = resolve(tasks[find_task(tasks, ntasks, vb)], bases);
  const int lt = vb - G.tile_begin;
  int tm, tn;
  if (G.tri)
    tri_decode(lt, G.tiles_m, tm, tn);
  else
    full_decode(lt, G.tiles_m, G.tiles_n, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const float* lrow =
      static_cast<const float*>(G.L) + ((size_t)tm * T + r) * G.ldl + 4 * q;
  const float* rrow = static_cast<const float*>((A.iter & 1) ? G.R1 : G.R0) +
                      ((size_t)tn * T + r) * G.ldr + 4 * q;
  const int kq = G.K / 4;
  const int kper = G.kper;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k0 = wave * kq; k0 < (wave + 1) * kq; k0 += 16) {
    const f32x4 a = ld_f32x4(lrow + k0);
    const f32x4 b = ld_f32x4(rrow + k0 % kper);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], acc, 0, 0, 0);
  }
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 v = ((acc + part[0][lane]) + part[1][lane]) + part[2][lane];
  const int row0 = tm * T + 4 * q;  // rows row0 .. row0 + 3
  const int col = tn * T + r;
  const bool mirror = G.tri && tm != tn;
  float* F = G.fbuf;
  const int ldf = G.ld_f;
  float* dst = F;
  int ld = ldf;
  if constexpr (KIND == KIND_SYRK) {
    const float s = A.iter == 0 ? G.scale[1] : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= s;
  } else {
    f32x4 av;
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = ld_f32(F + (size_t)(row0 + i) * ldf + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = fmaf(A.b, av[i], A.c * v[i]);
      if (G.add_diag && row0 + i == col) v[i] += A.a;
    }
    dst = static_cast<float*>(G.out0);
    ld = G.ld0;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) st_f32(dst + (size_t)(row0 + i) * ld + col, v[i]);
  if (mirror) st_f32x4(dst + (size_t)col * ld + row0, v);
}

// bf16 main loop fed by direct global->LDS loads (global_load_lds_dwordx4):
// STAGES buffers of BK k-values per row are kept in flight, so each K-step's
// loads were issued STAGES-1 steps before they are consumed.  Rows are
// stored without padding as CPR = BK/8 chunks of 16 bytes; k-chunk `kc` of
// row r lives at slot kc ^ swz(r).  The LDS has 64 banks of 4 bytes (a
// 256-byte bank line) and serves a 16-byte read 16 lanes at a time, so the
// reads of 16 consecutive rows must cover the 16 groups of 4 banks once:
// 128-byte rows pair up in a bank line (row parity picks the half), so the
// slot is swizzled by r/2; a 256-byte row spans the whole line, swizzled by
// r; 64-byte rows (four to a line) by r/4.  (Swizzling 128-byte rows by
// r mod 8 left a 2-way conflict: rocprofv3 counted 4 conflict cycles per
// 16-byte read.)
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 4) return (r >> 2) & 3;
  else if constexpr (CPR == 8) return (r >> 1) & 7;
  else return r & (CPR - 1);
}

// 16 bytes per lane from global memory straight into LDS at the wave-uniform
// base `lds` (lane l lands at lds + 16*l).  Kept out of the kernel templates:
// the host compilation pass cannot type-check this builtin, and inside a
// kernel body that silently drops the kernel's host-side launch stub.
__device__ void lds_dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at no-wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) only: every LDS read of this wave has returned.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Waits until at most `younger` stages of LOADS loads each are outstanding
// (younger <= MAXY; a wave-uniform value, so the branches are scalar).
template <int LOADS, int MAXY>
__device__ __forceinline__ void wait_stages(int younger) {
  if constexpr (MAXY == 0) {
    wait_vmcnt<0>();
  } else {
    if (younger >= MAXY) wait_vmcnt<MAXY * LOADS>();
    else wait_stages<LOADS, MAXY - 1>(younger);
  }
}

// Stages in flight per K depth BK of a stage (bf16 per row) and tile size.
// LDS holds STAGES x 2 operands x T rows x 2*BK bytes: 48 KB (T = 64,
// BK = 64), 64 KB (T = 64, BK = 128; T = 128), 128 KB (T = 256).  128-byte
// rows halve the number of L2 requests against 64-byte rows; measured on
// the NS shapes, that beats keeping more (shallower) stages in flight.
// BK = 128 (256-byte rows, half the stages and waits) serves the 64-wide
// SYRK and polynomial products, whose long K loops run at under two blocks
// per CU: 10% faster there, slower for the X update's short K.  The host
// gives it only tasks whose K is a multiple of 128.
template <int T, int BK>
constexpr int kStages = (T == 64 && BK == 64) ? 3 : 2;

template <int KIND, int T, int BK, int H, int HN>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const GemmTab* __restrict__ tasks,
                                                        int ntasks, int total_tiles, IterArgs A,
                                                        Bases bases) {
  constexpr int STAGES = kStages<T, BK>;
  constexpr int CPR = BK / 8;             // 16-byte chunks per row
  constexpr int WT = T / 2;               // wave tile (2 x 2 waves)
  constexpr int NT = WT / 32;             // 32x32 MFMA blocks per wave side
  constexpr int LPW = T * CPR / 256;      // 1 KB load instructions per wave per operand
  static_assert(LPW >= 1 && (STAGES - 2) * 2 * LPW < 64, "stage shape");
  constexpr int LOADS = 2 * LPW;          // loads per thread per stage
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES][2][T * BK];

  const int vb = xcd_remap(blockIdx.x, gridDim.x, total_tiles);
  if (vb >= total_tiles) return;
  // By value (see momentum_kernel): the epilogue's stores must not force
  // reloads of the descriptor.
  const GemmTask G = resolve(tasks[find_task(tasks, ntasks, vb)], bases);
  const int lt = vb - G.tile_begin;
  int tm, tn;
  if (G.tri)
    tri_decode(lt, G.tiles_m, tm, tn);
  else if (G.win)
    win_decode(lt, G.tiles_m, tm, tn);
  else
    full_decode(lt, G.tiles_m, G.tiles_n, tm, tn);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: wr, wc in SGPRs
  const int wr = (wave >> 1) * WT;
  const int wc = (wave & 1) * WT;
  const int nk = G.K / BK;
  const int kper = G.kper;

  // Per-lane global source of each load instruction: chunk c of the stage
  // (row c/CPR, slot c%CPR) holds global k-chunk slot ^ swz(row).
  const uint16_t* srcL[LPW];
  const uint16_t* srcR[LPW];
  {
    const uint16_t* Lp = static_cast<const uint16_t*>(G.L) + (size_t)tm * T * G.ldl;
    const uint16_t* Rp =
        static_cast<const uint16_t*>((A.iter & 1) ? G.R1 : G.R0) + (size_t)tn * T * G.ldr;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int c = (wave * LPW + i) * 64 + lane;
      const int row = c / CPR;
      const int kc = (c % CPR) ^ swz<CPR>(row);
      srcL[i] = Lp + (size_t)row * G.ldl + kc * 8;
      srcR[i] = Rp + (size_t)row * G.ldr + kc * 8;
    }
  }
  auto issue = [&](int kt) {
    const int st = kt % STAGES;
    const int k0 = kt * BK;
    const int kr = k0 % kper;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      lds_dma16(srcL[i] + k0, &lds[st][0][(wave * LPW + i) * 512]);
      lds_dma16(srcR[i] + kr, &lds[st][1][(wave * LPW + i) * 512]);
    }
  };

  f32x16 acc[NT][NT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Operand read offsets (elements) inside a stage buffer, per k-substep.
  constexpr int KS = BK / 16;  // MFMA k-substeps per stage
  static_assert(KS % 2 == 0, "operand register sets alternate per substep");
  int offA[KS][NT], offB[KS][NT];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int kc = ks * 2 + (lane >> 5);
      const int ra = wr + t * 32 + (lane & 31);
      const int rb = wc + t * 32 + (lane & 31);
      offA[ks][t] = ra * BK + 8 * (kc ^ swz<CPR>(ra));
      offB[ks][t] = rb * BK + 8 * (kc ^ swz<CPR>(rb));
    }

  // Two operand register sets: the LDS reads of substep ks+1 (or of the
  // next stage's first substep) are in flight while substep ks's MFMAs run,
  // so the LDS latency is not paid once per MFMA row.
  using V8 = typename Op16<H>::vec8;
  V8 ra[2][NT], rb[2][NT];
  auto read_ops = [&](int set, const uint16_t* sa, const uint16_t* sb, int ks) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      ra[set][t] = *reinterpret_cast<const V8*>(sa + offA[ks][t]);
      rb[set][t] = *reinterpret_cast<const V8*>(sb + offB[ks][t]);
    }
  };
  // MFMAs [first, last) of one substep, row-major over the NT x NT blocks.
  auto mfmas = [&](int set, int first, int last) {
#pragma unroll
    for (int x = first; x < last; ++x)
      acc[x / NT][x % NT] =
          Op16<H>::mfma(ra[set][x / NT], rb[set][x % NT], acc[x / NT][x % NT]);
  };
  // Interleave a substep's MFMAs with the next substep's 2*NT LDS reads.
  auto interleave = [&]() {
    constexpr int R = 2 * NT, M = NT * NT;
    constexpr int PER = (R + M - 1) / M;  // reads after each MFMA
#pragma unroll
    for (int x = 0; x < M; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (x * PER < R) __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);  // DS reads
    }
  };

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st);
  if constexpr (NT == 1) {
    // 64-wide tiles run three blocks per CU, whose waves hide each other's
    // LDS latency: one operand set, read right before its MFMA (measured
    // faster here than the prefetching loop below).
    for (int kt = 0; kt < nk; ++kt) {
      wait_stages<LOADS, STAGES - 2>(min(nk - 1 - kt, STAGES - 2));
      __builtin_amdgcn_s_barrier();
      if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
      const uint16_t* sa = lds[kt % STAGES][0];
      const uint16_t* sb = lds[kt % STAGES][1];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        read_ops(0, sa, sb, ks);
        mfmas(0, 0, 1);
      }
    }
    epilogue<KIND, T, false, NT, H, HN>(G, acc, tm, tn, wr, wc, lane, A, &lds[0][0][0]);
    return;
  }
  wait_stages<LOADS, STAGES - 2>(min(nk - 1, STAGES - 2));
  __builtin_amdgcn_s_barrier();
  if (STAGES - 1 < nk) issue(STAGES - 1);
  read_ops(0, lds[0][0], lds[0][1], 0);

  // Split of the last substep's MFMAs around the hand-over to the next
  // stage: the first half keeps the matrix cores busy through the wait and
  // the barrier, the second covers the first LDS reads of the next stage.
  constexpr int HALF = NT * NT / 2;
  for (int kt = 0; kt < nk; ++kt) {
    const uint16_t* sa = lds[kt % STAGES][0];
    const uint16_t* sb = lds[kt % STAGES][1];
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      read_ops((ks + 1) & 1, sa, sb, ks + 1);
      mfmas(ks & 1, 0, NT * NT);
      interleave();
    }
    mfmas(1, 0, HALF);
    if (kt + 1 < nk) {
      // Stage kt+1 must have landed (the younger stages stay in flight) and
      // every wave's reads of stage kt must be complete before its buffer is
      // refilled with stage kt+STAGES.
      wait_stages<LOADS, STAGES - 2>(min(nk - 2 - kt, STAGES - 2));
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      if (kt + STAGES < nk) issue(kt + STAGES);
      read_ops(0, lds[(kt + 1) % STAGES][0], lds[(kt + 1) % STAGES][1], 0);
    }
    mfmas(1, HALF, NT * NT);
  }

  epilogue<KIND, T, false, NT, H, HN>(G, acc, tm, tn, wr, wc, lane, A, &lds[0][0][0]);
}

template <int KIND, int T>
hipError_t launch_gemm_f32(const GemmTab* tasks, int ntasks, int total_tiles, const IterArgs& A,
                           Bases b, hipStream_t s) {
  const int grid = (total_tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_reg_kernel<KIND, T, true>), dim3(grid), dim3(256), 0, s, tasks, ntasks,
                     total_tiles, A, b);
  return hipGetLastError();
}

template <int KIND, int T, int BK, int H, int HN>
hipError_t launch_gemm_bf16(const GemmTab* tasks, int ntasks, int total_tiles, const IterArgs& A,
                            Bases b, hipStream_t s) {
  const int grid = (total_tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_bf16_kernel<KIND, T, BK, H, HN>), dim3(grid), dim3(256), 0, s, tasks,
                     ntasks, total_tiles, A, b);
  return hipGetLastError();
}

// 16-bit operand kernels by tile class and stage depth; H/HN as in epilogue
// (SYRK and polynomial launches write their output in their own format).
template <int KIND, int H, int HN>
hipError_t launch_gemm_h(int tile, int bk, const GemmTab* tasks, int ntasks, int total_tiles,
                         const IterArgs& A, Bases b, hipStream_t s) {
  if constexpr (KIND != KIND_UPDX) {
    if (tile == 64 && bk == 128)
      return launch_gemm_bf16<KIND, 64, 128, H, HN>(tasks, ntasks, total_tiles, A, b, s);
  }
  if (bk != 64) return hipErrorInvalidValue;
  if (tile == 64) return launch_gemm_bf16<KIND, 64, 64, H, HN>(tasks, ntasks, total_tiles, A, b, s);
  if (tile == 128)
    return launch_gemm_bf16<KIND, 128, 64, H, HN>(tasks, ntasks, total_tiles, A, b, s);
  if (tile == 256)
    return launch_gemm_bf16<KIND, 256, 64, H, HN>(tasks, ntasks, total_tiles, A, b, s);
  return hipErrorInvalidValue;
}

template <int KIND>
hipError_t launch_gemm_k(int tile, int f32_ops, int bk, int h, int hn, const GemmTab* tasks,
                         int ntasks, int total_tiles, const IterArgs& A, Bases b, hipStream_t s) {
  if (f32_ops) {
    if (tile == 16) {
      if constexpr (KIND == KIND_SYRK || KIND == KIND_POLY) {
        const int grid = (total_tiles + 7) / 8 * 8;
        hipLaunchKernelGGL((gemm_f32_small_kernel<KIND>), dim3(grid), dim3(256), 0, s, tasks,
                           ntasks, total_tiles, A, b);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    }
    if (tile == 64) return launch_gemm_f32<KIND, 64>(tasks, ntasks, total_tiles, A, b, s);
    if (tile == 128) return launch_gemm_f32<KIND, 128>(tasks, ntasks, total_tiles, A, b, s);
    return hipErrorInvalidValue;
  }
  if (h == 0 && hn == 0)
    return launch_gemm_h<KIND, 0, 0>(tile, bk, tasks, ntasks, total_tiles, A, b, s);
  if (h == 1 && hn == 1)
    return launch_gemm_h<KIND, 1, 1>(tile, bk, tasks, ntasks, total_tiles, A, b, s);
  if constexpr (KIND == KIND_UPDX) {  // the first X update of the fp16 mode
    if (h == 0 && hn == 1)
      return launch_gemm_h<KIND, 0, 1>(tile, bk, tasks, ntasks, total_tiles, A, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Scratch of dmuon_muon_step_noalloc (see kScratchBytes): every GPU the
// library runs on holds one copy until the process ends.  In host code the
// name is only a handle; the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes % 8 || reinterpret_cast<uintptr_t>(dst) % 8) return hipErrorInvalidValue;
  const size_t words = bytes / 8;
  for (size_t off = 0; off < words; off += kUploadWords) {
    UploadChunk c{};
    c.dst = static_cast<uint64_t*>(dst) + off;
    c.n = (int32_t)(words - off < (size_t)kUploadWords ? words - off : (size_t)kUploadWords);
    std::memcpy(c.w, static_cast<const char*>(src) + 8 * off, 8 * (size_t)c.n);
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(kUploadWords), 0, s, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_momentum(const EwTab* tasks, int ntasks, int total_tiles, float momentum,
                           int nesterov, int ns_only, Bases b, hipStream_t s) {
  hipLaunchKernelGGL(momentum_kernel, dim3(total_tiles), dim3(EW_THREADS), 0, s, tasks, ntasks,
                     total_tiles, momentum, nesterov, ns_only, b);
  return hipGetLastError();
}

hipError_t launch_gram_finalize(const FinTab* tasks, int ntasks, int nblocks, float eps,
                                Bases b, hipStream_t s) {
  hipLaunchKernelGGL(gram_finalize_kernel, dim3(nblocks), dim3(256), 0, s, tasks, ntasks, eps, b);
  return hipGetLastError();
}

hipError_t launch_norm(const NormTab* tasks, int ntasks, float eps, Bases b, hipStream_t s) {
  hipLaunchKernelGGL(norm_kernel, dim3(ntasks), dim3(256), 0, s, tasks, eps, b);
  return hipGetLastError();
}

hipError_t launch_gram16_x(const EwTab* tasks, int ntasks, int total_tiles, Bases b,
                           hipStream_t s) {
  hipLaunchKernelGGL(gram16_x_kernel, dim3(total_tiles), dim3(EW_THREADS), 0, s, tasks, ntasks,
                     total_tiles, b);
  return hipGetLastError();
}

hipError_t launch_gemm(int kind, int tile, int f32_ops, int bk, int h, int hn,
                       const GemmTab* tasks, int ntasks, int total_tiles, const IterArgs& A,
                       Bases b, hipStream_t s) {
  switch (kind) {
    case KIND_SYRK:
      return launch_gemm_k<KIND_SYRK>(tile, f32_ops, bk, h, h, tasks, ntasks, total_tiles, A, b,
                                      s);
    case KIND_POLY:
      return launch_gemm_k<KIND_POLY>(tile, f32_ops, bk, h, h, tasks, ntasks, total_tiles, A, b,
                                      s);
    case KIND_UPDX:
      return launch_gemm_k<KIND_UPDX>(tile, f32_ops, bk, h, hn, tasks, ntasks, total_tiles, A, b,
                                      s);
    case KIND_GRAMMUL:
      if (!f32_ops) {  // fp16 operands only
        if (h != 1 || hn != 1) return hipErrorInvalidValue;
        return launch_gemm_h<KIND_GRAMMUL, 1, 1>(tile, bk, tasks, ntasks, total_tiles, A, b, s);
      }
      if (tile == 64)
        return launch_gemm_f32<KIND_GRAMMUL, 64>(tasks, ntasks, total_tiles, A, b, s);
      if (tile == 128)
        return launch_gemm_f32<KIND_GRAMMUL, 128>(tasks, ntasks, total_tiles, A, b, s);
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dmuon
