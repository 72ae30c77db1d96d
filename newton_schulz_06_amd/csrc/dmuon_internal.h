// Internal launch descriptors shared by the host runtime and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dmuon {

// Kernel kinds, used for profiling rows and launch bookkeeping.
enum Kind : int {
  KIND_MOMENTUM = 0,  // momentum (+ Nesterov), orientation, sum of squares
  KIND_INPUT,         // NS-only input pass: orientation, sum of squares
  KIND_NORM,          // per-matrix norm finalize -> 1/(||u|| + eps)
  KIND_SYRK,          // A = X X^T (upper tiles, mirrored write)
  KIND_POLY,          // B = b A + c A A^T (upper tiles, mirrored write)
  KIND_UPDX,          // X <- a X + B X; on the last iteration the result
                      // goes straight to the caller: p <- p (1 - lr wd) - lr O
                      // (step) or out <- O (NS only)
  KIND_CLIP_NORM,     // gradient clipping: norm partials + per-bucket finalize
  KIND_CLIP_SCALE,    // gradient clipping: g <- g * factor
  KIND_ADAMW,         // AdamW update of non-Muon parameters
  KIND_GRAMMUL,       // Gram-space NS: a product of two commuting symmetric
                      // p x p matrices (P A, P (P A), P Q), fp32 or fp16
                      // operands
  KIND_GRAM_X,        // Gram-space NS with fp16 operands: X normalized into
                      // the fp16 operand layout
  KIND_COUNT
};

// Device addresses in launch tables.  A table depends only on the shapes
// and options of a call, so it is built once per device and shape set and
// reused by every later call: each address in it is a Ref, either a byte
// offset into the call's workspace (>= 0), one of the call's pointer slots
// (the caller's buffers, ref_slot(s)), or none.  Kernels turn Refs into
// pointers once per block from the call's Bases.
typedef int64_t Ref;
constexpr Ref kRefNone = -1;
__host__ __device__ constexpr Ref ref_slot(int s) { return -2 - (Ref)s; }

// Per-call bases of the Refs: the workspace and its pointer-slot array,
// which launch_upload fills from the call's buffer pointers before the
// first kernel of the call.  Slots per matrix: [source, destination,
// momentum buffer].
struct Bases {
  char* ws;
  void* const* slots;
};
constexpr int kSlotsPerMat = 3;

// Maps an address field of a launch table (Ref) or of its resolved form
// (a pointer of type T).
template <class T> using Ptr = T*;
template <class T> using RefOf = Ref;

// Power-of-two scales of the fp16 operand forms (the kernels' Op16<1>): A
// (and, in Gram-space NS, P A) is stored times kF16AScale, B (Gram-space: P
// and Q) times kF16BScale; the consumers' epilogues divide them out, exactly.
constexpr float kF16AScale = 4096.f, kF16BScale = 1024.f;

// Element-wise tile size (original-layout tiles of EW_TILE x EW_TILE).
constexpr int EW_TILE = 64;
constexpr int EW_THREADS = 256;

// One matrix of an element-wise launch.  Tiles cover `rows` x `cols` in
// the caller's layout; for the input passes these are the padded extents of
// the oriented workspace mapped back to the caller's layout.
template <template <class> class A>
struct EwTaskT {
  int32_t m, n;            // caller's shape
  int32_t rows, cols;      // extent covered by this launch's tiles
  int32_t tiles_c;         // tiles along cols
  int32_t tile_begin;      // first global tile of this task
  int32_t tile_count;      // tiles of this task
  int32_t transposed;      // m > n: the oriented X is the transpose
  int32_t in_dtype;        // dtype of `src` (grad / input G)
  int32_t ldx;             // row stride of xm (elements)
  int32_t ldxb;            // row stride of xb (elements)
  int32_t ldt;             // row stride of xt (elements)
  int32_t f32_ops;         // 1: xt holds fp32 (NS in fp32), 0: bf16
  int32_t pad0_;
  A<const void> src;       // grad (step) or G (NS only)
  A<float> buf;            // momentum buffer (step) or none
  A<float> xm;             // fp32 X, P x Q (f32_ops only)
  A<uint16_t> xb;          // bf16 X = high part of X, P x Q (bf16 modes)
  A<uint16_t> xlo;         // bf16 X - xb, P x Q, stride ldxb (bf16 modes)
  A<void> xt;              // X^T, Q x P (bf16 or fp32)
  A<float> partial;        // per-tile sums of squares (indexed by global tile)
  A<float> scale;          // per-matrix scalars: [0]=1/(s+eps) [1]=its square
};
using EwTask = EwTaskT<Ptr>;
using EwTab = EwTaskT<RefOf>;

// One matrix of a grouped NT-GEMM launch: C = L * R^T over K, tile T x T.
// L is (tiles_m*T) x K row-major with stride ldl; R is (tiles_n*T) x K with
// stride ldr and column index taken modulo kper (for hi/lo split operands
// that reuse one R for two K segments).
template <template <class> class A>
struct GemmTaskT {
  A<const void> L;
  A<const void> R0;        // R on even NS iterations
  A<const void> R1;        // R on odd NS iterations
  int32_t ldl, ldr, K, kper;
  int32_t tiles_m, tiles_n, tile_begin, tile_count;
  int32_t tri;             // 1: upper-triangle tiles only (+ mirrored write)
  int32_t split;           // SYRK: write A as [hi|lo|hi|hi]; POLY: write B as [hi|lo]
  int32_t P;               // padded p (segment offset of split layouts)
  int32_t ld_f;            // stride of fbuf
  A<float> fbuf;           // fp32 A (SYRK out, POLY in; none when A is split)
                           // or fp32 X (UPDX, fp32 operands)
  A<void> out0;            // SYRK: A operand  POLY: B operand  UPDX: bf16 X
  A<void> out1;            // UPDX: X^T (even iter)
  A<void> out2;            // UPDX: X^T (odd iter)
  int32_t ld0, ld1;
  A<const float> scale;    // per-matrix scalars (see EwTask::scale)
  A<uint16_t> xlo;         // UPDX, bf16 operands: X - bf16 X (stride ld0)
  A<const uint16_t> ahl;   // POLY with split A: A as [hi | lo | ...] rows
  int32_t ld_ahl;          // its row stride
  // GRAMMUL with fp16 operands: the product is multiplied by g_in (undoing
  // the operands' power-of-two scales) and stored times g_out
  float g_in;
  A<void> sink;            // 16 writable, never-read bytes (see updx_final)
  // UPDX, last iteration: the caller's param (step) or output (NS only).
  // Oriented element (r, c), r < pv, c < qv, sits at dst[r*qv + c], or at
  // dst[c*pv + r] when dst_trans (caller's matrix is the transpose).
  A<void> dst;
  int32_t pv, qv;          // valid oriented extents p x q
  int32_t dst_trans;
  int32_t dst_dtype;
  int32_t add_diag;        // POLY (Gram-space P): add the iteration's a on the diagonal
  int32_t win;             // full product: tiles in column windows (see win_decode)
  float g_out;
  int32_t pad1_;
};
using GemmTask = GemmTaskT<Ptr>;
using GemmTab = GemmTaskT<RefOf>;

// What the UPDX epilogue does with the new X.
enum Fin : int32_t {
  FIN_NONE = 0,    // keep iterating: write X (fp32, bf16) and X^T
  FIN_UPDATE = 1,  // p <- p * decay - lr * O
  FIN_OUTPUT = 2,  // out <- O
};

// Per-launch scalars of one NS iteration.
struct IterArgs {
  int32_t iter;
  int32_t fin;             // Fin; only read by UPDX
  float a, b, c;           // this iteration's coefficients
  float lr, decay;         // FIN_UPDATE only
};

template <template <class> class A>
struct NormTaskT {
  int32_t tile_begin, tile_count;
  A<const float> partial;
  A<float> scale;
  // Gram NS on a shard: the shard's sum of squares goes here (to be summed
  // over the shard group) and the scales stay 1 until the group's norm is
  // known.
  A<float> sumsq;
};
using NormTask = NormTaskT<Ptr>;
using NormTab = NormTaskT<RefOf>;

// Gram NS on a shard, once the group's sums are in: the normalization from
// the summed squared norm, and the summed raw Gram matrix A (P x P rows of
// stride ld) scaled by its square.  FIN_ROWS rows of A per block.
constexpr int FIN_ROWS = 16;
template <template <class> class A>
struct FinTaskT {
  int32_t tile_begin, tile_count;  // blocks
  int32_t P, ld;
  A<float> a;
  A<const float> sumsq;
  A<float> scale;
};
using FinTask = FinTaskT<Ptr>;
using FinTab = FinTaskT<RefOf>;

// ---------------------------------------------------------------------------
// Flat element-wise launches (gradient clipping, AdamW): every tensor is
// cut into chunks, one block per chunk.  A block handles 16 elements per
// thread at a time (FLAT_STEP), FLAT_ITERS_* times: AdamW keeps four arrays
// per element live, clipping only one and needs bigger blocks to stream.
constexpr int FLAT_THREADS = 256;
constexpr int FLAT_STEP = FLAT_THREADS * 16;
constexpr int FLAT_ITERS_ADAMW = 1;
constexpr int FLAT_ITERS_CLIP = 4;

struct FlatTask {
  int64_t n;               // elements of the tensor
  int32_t blk_begin;       // first block (chunk) of this tensor
  int32_t nblk;            // blocks of this tensor
  int32_t bucket;          // clipping: bucket index
  int32_t dtype;           // dtype of `p` (0 fp32, 1 bf16)
  int32_t gdtype;          // AdamW: dtype of `g`
  int32_t vec;             // every pointer allows 4-element vector access
  void* p;                 // clipping: the gradient; AdamW: the parameter
  const void* g;           // AdamW: the gradient
  float* m;                // AdamW: first moment
  float* v;                // AdamW: second moment
};

// How the clipping norm is formed: sum of squares, sum of magnitudes, max
// magnitude, or sum of |g|^p.
enum NormMode : int32_t { NORM_L2 = 0, NORM_L1 = 1, NORM_INF = 2, NORM_P = 3 };

// Per-bucket result of the clipping finalize, in the caller's layout (the
// public dmuon_clip_stats_t).
struct ClipStats {
  double total_norm;
  double clip_coef;
  int32_t clipped;
  int32_t found_inf;
  int64_t param_count;
};

// Scalars of one AdamW launch, derived on the host from (lr, betas, eps,
// weight decay, step).
struct AdamArgs {
  float decay;             // 1 - lr * weight_decay
  float beta1, one_minus_beta1;
  float beta2, one_minus_beta2;
  float step_size;         // lr / (1 - beta1^t)
  float inv_bc2_sqrt;      // 1 / sqrt(1 - beta2^t)
  float eps;
};

// Launch helpers implemented in dmuon_optim.hip.
hipError_t launch_clip_norm(const FlatTask* tasks, int ntasks, int total_blocks, int mode,
                            float p, float* partial, hipStream_t s);
hipError_t launch_clip_finalize(const FlatTask* tasks, int ntasks, int nbuckets, int mode,
                                double p, double max_norm, int stats_only,
                                const float* partial, ClipStats* stats, float* scale,
                                hipStream_t s);
hipError_t launch_clip_scale(const FlatTask* tasks, int ntasks, int total_blocks,
                             const float* scale, hipStream_t s);
hipError_t launch_adamw(const FlatTask* tasks, int ntasks, int total_blocks,
                        const AdamArgs& args, hipStream_t s);

// Launch helpers implemented in dmuon_kernels.hip.
// Copies `bytes` (a multiple of 8; dst 8-byte aligned) from host memory to
// the device through kernel arguments, kUploadWords words per launch: a
// stream-ordered upload that needs no host staging memory and allocates
// nothing (the call's pointer slots; the launch tables of the
// allocation-free entry point).
constexpr int kUploadWords = 256;
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s);

// Device memory of the allocation-free step (dmuon_muon_step_noalloc): a
// static array of kScratchBytes per device, holding that call's workspace,
// pointer slots and launch tables.  scratch_address gives this device's
// address of it (looked up once per device).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_address(void** out);
hipError_t launch_momentum(const EwTab* tasks, int ntasks, int total_tiles,
                           float momentum, int nesterov, int ns_only, Bases b,
                           hipStream_t s);
hipError_t launch_gram_finalize(const FinTab* tasks, int ntasks, int nblocks, float eps,
                                Bases b, hipStream_t s);
hipError_t launch_norm(const NormTab* tasks, int ntasks, float eps, Bases b,
                       hipStream_t s);
// Gram-space NS with fp16 operands, after the norm: the master X (bf16 hi +
// remainder, or fp32) becomes X / (||u|| + eps) in the fp16 layout, with
// its fp16 copy (xb) and fp16 X^T (xt).  Tiles of 64 x 64 over the oriented
// padded P x Q.
hipError_t launch_gram16_x(const EwTab* tasks, int ntasks, int total_tiles, Bases b,
                           hipStream_t s);
// kind in {KIND_SYRK, KIND_POLY, KIND_UPDX, KIND_GRAMMUL}; tile in {64, 128, 256}
// (16-bit operands) or {16 (SYRK and polynomial only), 64, 128} (fp32
// operands); bk, the K depth of a
// 16-bit main-loop stage: 64, or 128 for the 64-wide SYRK and polynomial
// (every task's K then a multiple of 128).  h: operand format of the
// products (0 bf16, 1 fp16); hn: format of the X copies an X update writes
// for the next iteration (h, or 1 after a bf16 first iteration).  GRAMMUL
// with 16-bit operands: fp16 only (h = hn = 1).
hipError_t launch_gemm(int kind, int tile, int f32_ops, int bk, int h, int hn,
                       const GemmTab* tasks, int ntasks, int total_tiles,
                       const IterArgs& args, Bases b, hipStream_t s);

}  // namespace dmuon
