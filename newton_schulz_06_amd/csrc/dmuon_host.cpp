// Host runtime of the C ABI declared in include/dmuon.h: argument
// validation, workspace layout, per-device launch-table cache, the launch
// sequence of one Muon step / one NS call, and optional event timing.
#include "dmuon.h"

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "dmuon_internal.h"

using namespace dmuon;

namespace {

thread_local std::string g_last_error;

dmuon_status_t fail(dmuon_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

constexpr int kMaxSteps = 16;
constexpr int64_t kMaxSide = int64_t(1) << 20;
constexpr size_t kWsAlign = 256;
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
size_t esize(int dtype) { return dtype == DMUON_F32 ? 4 : 2; }

// GEMM tile classes (square T x T output tiles).  16-bit operands: the
// largest of 256 (min side >= 1024) / 128 (>= 768) whose padding of the
// min side stays within 1/8, else 64 -- small matrices are latency-bound and
// want many small tiles.  fp32 operands: 16 up to 256 (direct NS only: the
// 16-wide kernel splits K over its waves), 64 up to 512, 128 above.
// Matrices are padded to multiples of max(T, 64) (the element-wise passes
// work on 64 x 64 tiles).
constexpr int kTiles[4] = {16, 64, 128, 256};
int tile_index(int tile) { return tile == 16 ? 0 : tile == 64 ? 1 : tile == 128 ? 2 : 3; }

int tile_class(int64_t p, bool f32_ops, bool gram = false) {
  if (f32_ops) return p <= 256 && !gram ? 16 : p <= 512 ? 64 : 128;
  auto fits = [p](int64_t t) { return round_up(p, t) * 8 <= p * 9; };
  if (p >= 1024 && fits(256)) return 256;
  if (p >= 768 && fits(128)) return 128;
  return 64;
}
constexpr float kQuintic[3] = {3.4445f, -4.7750f, 2.0315f};
// Shortest K for 128-deep main-loop stages (see build_plan).  Measured: the
// TinyMLP SYRK (K 2048) and polynomial (1536) run 10% faster with them, the
// packed batch's short-K products slower.
constexpr int64_t kDeepMinK = 1536;


// Row stride (elements) for a workspace matrix with `n` columns of `esz`
// bytes: rounded up to an odd multiple of 256 bytes, so that consecutive
// rows start in different L2 channels (the NS shapes are multiples of large
// powers of two; unpadded, all rows of a tile would share one channel).
int64_t ld_for(int64_t n, int64_t esz) {
  int64_t units = (n * esz + 255) / 256;
  if (units % 2 == 0) ++units;
  return units * 256 / esz;
}

// Shape-derived geometry of one matrix in the workspace.
struct Geom {
  int64_t m, n, p, q, P, Q;
  int tile, transposed, split_a, split_b;
  int hilo;  // master X as bf16 X + bf16 remainder (else fp32, next to bf16 X)
  int64_t ld_xm, ld_xb, ld_xt, ld_a32, ld_aop, ld_bop;  // row strides (elements)
  size_t xm, xb, xlo, xt0, xt1, a32, aop, bop;         // byte offsets in ws
  size_t pm, pa, qa, qb;  // Gram-space NS: P, P A, and the Q pair (fp32 P x P)
};

struct Layout {
  std::vector<Geom> g;
  // slot_off: the call's buffer pointers, kSlotsPerMat per matrix (written
  // by launch_upload at the start of every call)
  size_t partial_off = 0, scale_off = 0, sink_off = 0, slot_off = 0, total = 0;
  int64_t in_tiles = 0;
  int f32_ops = 0;
  // Tile classes whose products take fp16 operands after the first
  // iteration (bit tile_index(T)): all with DMUON_NS_F16; with
  // DMUON_NS_AUTO those below 256.  Measured: fp16 makes the 64- and 128-wide launches
  // faster than the hi/lo bf16 splits it replaces (TinyMLP x4 0.475 -> 0.427
  // ms, 512 small matrices 1.93 -> 1.52 ms), but the 256-wide ones 2-4%
  // slower than plain bf16 (same MFMA peak; Llama-8B 71.4 -> 73.0 ms, 70B
  // MLP 195.8 -> 202.7 ms), where plain bf16 already has a wide margin.
  int f16 = 0;
  int gram = 0;  // Gram-space NS layout (fp32 operands)
  // Gram NS on column shards: every matrix's sum of squares (one float
  // each, padded to kWsAlign), then every fp32 Gram matrix back to back, so
  // one in-place sum over the shard group covers the whole batch.
  int local = 0;
  size_t bucket_off = 0, bucket_bytes = 0;
};

// `orient` < 0: transpose iff m > n; 0 / 1 force it (a shard takes the full
// matrix's orientation, so its p may exceed its q).  `local`: the shard
// layout (Gram backend only).
dmuon_status_t make_layout(const dmuon_batch_t* b, int prec, int backend, Layout* out,
                           int orient = -1, bool local = false) {
  Layout L;
  L.gram = backend == DMUON_NS_GRAM;
  L.local = local;
  // Gram-space NS: fp32 operands, or fp16 with DMUON_NS_F16 (not on shards)
  L.f32_ops = (prec == DMUON_NS_F32) || (L.gram && (prec != DMUON_NS_F16 || local));
  // bits: tile_index (the 16-wide class has fp32 operands only)
  L.f16 = L.f32_ops ? 0 : prec == DMUON_NS_F16 ? 0xe : prec == DMUON_NS_AUTO ? 0x6 : 0;
  const int n = b->count;
  L.g.resize(n);
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    Geom& G = L.g[i];
    G.m = b->mats[i].m;
    G.n = b->mats[i].n;
    G.transposed = orient < 0 ? G.m > G.n : orient;
    G.p = G.transposed ? G.n : G.m;
    G.q = G.transposed ? G.m : G.n;
    G.tile = tile_class(G.p, L.f32_ops != 0, L.gram || L.local);
    G.P = round_up(G.p, std::max(G.tile, EW_TILE));
    G.Q = round_up(G.q, std::max(G.tile, EW_TILE));
    if (G.P * ld_for(G.Q, 4) > INT32_MAX || G.Q * ld_for(G.P, 4) > INT32_MAX ||
        G.P * ld_for(3 * G.P, 2) > INT32_MAX)
      return fail(DMUON_E_UNSUPPORTED, "matrix " + std::to_string(i) +
                                           ": padded size exceeds 2^31 elements");
    G.split_b = !L.f32_ops && prec == DMUON_NS_BF16_SPLIT;
    G.split_a = !L.f32_ops && (prec == DMUON_NS_BF16_SPLIT || prec == DMUON_NS_BF16_SPLIT_A);
    tiles += (G.P / EW_TILE) * (G.Q / EW_TILE);
  }
  if (tiles > INT32_MAX) return fail(DMUON_E_UNSUPPORTED, "batch too large (tile count)");
  L.in_tiles = tiles;
  size_t off = 0;
  L.partial_off = off;
  off = align_up(off + sizeof(float) * (size_t)tiles, kWsAlign);
  L.scale_off = off;
  off = align_up(off + sizeof(float) * 4 * (size_t)n, kWsAlign);
  L.sink_off = off;  // writable bytes nothing reads (padding lanes' stores)
  off = align_up(off + 16, kWsAlign);
  L.slot_off = off;
  off = align_up(off + sizeof(void*) * kSlotsPerMat * (size_t)n, kWsAlign);
  if (L.local) {
    L.bucket_off = off;
    off = align_up(off + sizeof(float) * (size_t)n, kWsAlign);
    for (int i = 0; i < n; ++i) {  // whole multiples of kWsAlign: no gaps
      Geom& G = L.g[i];
      G.ld_a32 = ld_for(G.P, 4);
      G.a32 = off;
      off = align_up(off + 4 * (size_t)G.P * G.ld_a32, kWsAlign);
    }
    L.bucket_bytes = off - L.bucket_off;
  }
  const int64_t e = L.f32_ops ? 4 : 2;
  for (int i = 0; i < n; ++i) {
    Geom& G = L.g[i];
    auto take = [&](size_t bytes) {
      const size_t o = off;
      off = align_up(off + bytes, kWsAlign);
      return o;
    };
    const size_t P = (size_t)G.P, Q = (size_t)G.Q;
    G.ld_xm = ld_for(G.Q, 4);
    G.ld_xb = ld_for(G.Q, 2);
    G.ld_xt = ld_for(G.P, e);
    G.ld_a32 = ld_for(G.P, 4);
    G.xm = G.xb = G.xlo = 0;
    if (!L.local) G.a32 = 0;
    // Same rule as the kernels' kHiLoMaster: tiles below 256.
    G.hilo = !L.f32_ops && G.tile < 256;
    if (!G.hilo) G.xm = take(4 * P * G.ld_xm);       // fp32 X
    if (!L.f32_ops) G.xb = take(2 * P * G.ld_xb);    // bf16 X
    if (G.hilo) G.xlo = take(2 * P * G.ld_xb);       // bf16 (X - bf16 X)
    G.xt0 = take(e * Q * G.ld_xt);
    G.xt1 = take(e * Q * G.ld_xt);
    if (!L.local && (L.f32_ops || !G.split_a)) G.a32 = take(4 * P * G.ld_a32);
    G.pm = G.pa = G.qa = G.qb = 0;
    if (L.gram && !L.f32_ops) {
      // fp16 operands: A, P, P A and the Q pair as fp16 (power-of-two
      // scaled); the fp32 A above feeds the polynomial's linear term
      G.ld_aop = G.ld_bop = ld_for(G.P, 2);
      G.aop = take(2 * P * G.ld_aop);
      G.bop = 0;
      G.pm = take(2 * P * G.ld_aop);
      G.pa = take(2 * P * G.ld_aop);
      G.qa = take(2 * P * G.ld_aop);
      G.qb = take(2 * P * G.ld_aop);
    } else if (L.gram) {
      G.aop = G.a32;
      G.ld_aop = G.ld_a32;
      G.ld_bop = G.ld_a32;
      G.bop = 0;
      G.pm = take(4 * P * G.ld_a32);
      G.pa = take(4 * P * G.ld_a32);
      G.qa = take(4 * P * G.ld_a32);
      G.qb = take(4 * P * G.ld_a32);
    } else if (L.f32_ops) {
      G.aop = G.a32;
      G.ld_aop = G.ld_a32;
      G.ld_bop = ld_for(G.P, 4);
      G.bop = take(4 * P * G.ld_bop);
    } else {
      G.ld_aop = ld_for(G.split_a ? 4 * G.P : G.P, 2);  // [hi|lo|hi|hi] rows when split
      G.aop = take(2 * P * G.ld_aop);
      G.ld_bop = ld_for(G.split_b ? 2 * G.P : G.P, 2);
      G.bop = take(2 * P * G.ld_bop);
    }
  }
  L.total = off;
  *out = std::move(L);
  return DMUON_OK;
}

// ------------------------------------------------------------ validation --

dmuon_status_t check_batch(const dmuon_batch_t* b, const char* name, bool need_ptrs) {
  if (!b) return fail(DMUON_E_INVALID, std::string(name) + ": null batch");
  if (b->count < 0) return fail(DMUON_E_INVALID, std::string(name) + ": negative count");
  if (b->count > 0 && !b->mats) return fail(DMUON_E_INVALID, std::string(name) + ": null mats");
  if (b->dtype != DMUON_F32 && b->dtype != DMUON_BF16)
    return fail(DMUON_E_INVALID, std::string(name) + ": unknown dtype");
  for (int i = 0; i < b->count; ++i) {
    const dmuon_mat_t& M = b->mats[i];
    const std::string where = std::string(name) + "[" + std::to_string(i) + "]";
    if (M.m < 1 || M.n < 1) return fail(DMUON_E_INVALID, where + ": empty or negative shape");
    if (M.m > kMaxSide || M.n > kMaxSide)
      return fail(DMUON_E_UNSUPPORTED, where + ": side longer than 2^20");
    if (need_ptrs) {
      if (!M.ptr) return fail(DMUON_E_INVALID, where + ": null pointer");
      if (reinterpret_cast<uintptr_t>(M.ptr) % esize(b->dtype))
        return fail(DMUON_E_INVALID, where + ": pointer not aligned to its element size");
    }
  }
  return DMUON_OK;
}

std::vector<int> gram_cuts(const dmuon_ns_cfg_t* cfg);

// Gram-space NS with fp16 operands stores P times 2^10 and Q (a product of
// a window's P's) times 2^10, so both must stay below 64 in magnitude.  A
// starts with eigenvalues in [0, 1] (X is normalized by its Frobenius norm),
// and a step maps an eigenvalue l to l p(l)^2, which NS schedules keep
// within about [0, 1.2].  Over l in [0, 1.25], max |p_k(l)| then bounds
// ||P_k||, and the product over a window's steps bounds ||Q||.  Tables whose
// bound exceeds 48 are rejected (the quintic: 3.44 per step, 41 over three
// steps).
dmuon_status_t check_gram16_coeffs(const dmuon_ns_cfg_t* cfg) {
  const std::vector<int> cuts = gram_cuts(cfg);
  for (size_t w = 0; w + 1 < cuts.size(); ++w) {
    double bound = 1.0;
    for (int k = cuts[w]; k < cuts[w + 1]; ++k) {
      const float* c = cfg->coeffs ? cfg->coeffs + 3 * k : kQuintic;
      double mx = 0.0;
      for (int j = 0; j <= 1000; ++j) {
        const double l = 1.25 * j / 1000.0;
        mx = std::max(mx, std::fabs((double)c[0] + (double)c[1] * l + (double)c[2] * l * l));
      }
      bound *= mx;
    }
    if (!(bound <= 48.0))
      return fail(DMUON_E_UNSUPPORTED,
                  "cfg: Gram-space NS with fp16 operands: the coefficients of window " +
                      std::to_string(w) + " can grow Q to " + std::to_string(bound) +
                      ", beyond the fp16 range of its scaled form (48)");
  }
  return DMUON_OK;
}

// Backend and restart list (also needed by the workspace-size query).
dmuon_status_t check_backend(const dmuon_ns_cfg_t* cfg) {
  if (cfg->backend != DMUON_NS_DIRECT && cfg->backend != DMUON_NS_GRAM)
    return fail(DMUON_E_INVALID, "cfg: unknown backend");
  if (cfg->nrestarts < 0 || (!cfg->restarts && cfg->nrestarts != 0))
    return fail(DMUON_E_INVALID, "cfg: restarts must hold nrestarts entries");
  for (int i = 0; i < cfg->nrestarts; ++i)
    if (cfg->restarts[i] < 0) return fail(DMUON_E_INVALID, "cfg: negative restart index");
  if (cfg->backend == DMUON_NS_GRAM && cfg->prec != DMUON_NS_F32 &&
      cfg->prec != DMUON_NS_AUTO && cfg->prec != DMUON_NS_F16)
    return fail(DMUON_E_UNSUPPORTED,
                "cfg: Gram-space NS runs with fp32 (prec F32 or AUTO) or fp16 (F16) operands");
  return DMUON_OK;
}

dmuon_status_t check_cfg(const dmuon_ns_cfg_t* cfg) {
  if (!cfg) return fail(DMUON_E_INVALID, "cfg: null");
  if (cfg->ns_steps < 1 || cfg->ns_steps > kMaxSteps)
    return fail(DMUON_E_INVALID, "cfg: ns_steps must be in [1, 16]");
  if (!std::isfinite(cfg->eps) || cfg->eps < 0.f)
    return fail(DMUON_E_INVALID, "cfg: eps must be finite and >= 0");
  if (cfg->prec < DMUON_NS_F32 || cfg->prec > DMUON_NS_F16)
    return fail(DMUON_E_INVALID, "cfg: unknown precision mode");
  if (cfg->coeffs)
    for (int i = 0; i < 3 * cfg->ns_steps; ++i)
      if (!std::isfinite(cfg->coeffs[i]))
        return fail(DMUON_E_INVALID, "cfg: non-finite coefficient");
  dmuon_status_t st = check_backend(cfg);
  if (!st && cfg->backend == DMUON_NS_GRAM && cfg->prec == DMUON_NS_F16)
    st = check_gram16_coeffs(cfg);
  return st;
}

dmuon_status_t same_shapes(const dmuon_batch_t* a, const dmuon_batch_t* b, const char* an,
                           const char* bn) {
  if (a->count != b->count)
    return fail(DMUON_E_INVALID, std::string(an) + " and " + bn + ": counts differ");
  for (int i = 0; i < a->count; ++i)
    if (a->mats[i].m != b->mats[i].m || a->mats[i].n != b->mats[i].n)
      return fail(DMUON_E_INVALID, std::string(an) + " and " + bn + ": shapes differ at index " +
                                       std::to_string(i));
  return DMUON_OK;
}

struct Span {
  uintptr_t lo, hi;
  int group, index;
};

// No two spans may overlap.
dmuon_status_t check_disjoint(std::vector<Span> v, const char* const* names) {
  std::sort(v.begin(), v.end(), [](const Span& x, const Span& y) { return x.lo < y.lo; });
  size_t far = 0;  // span with the largest end so far
  for (size_t i = 1; i < v.size(); ++i) {
    if (v[i].lo < v[far].hi) {
      char buf[160];
      std::snprintf(buf, sizeof buf, "%s[%d] overlaps %s[%d]", names[v[i].group], v[i].index,
                    names[v[far].group], v[far].index);
      return fail(DMUON_E_INVALID, buf);
    }
    if (v[i].hi > v[far].hi) far = i;
  }
  return DMUON_OK;
}

void add_spans(std::vector<Span>& v, const dmuon_batch_t* b, int group) {
  for (int i = 0; i < b->count; ++i) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(b->mats[i].ptr);
    v.push_back({lo, lo + (uintptr_t)(b->mats[i].m * b->mats[i].n * esize(b->dtype)), group, i});
  }
}

// ----------------------------------------------------------------- plans --

struct GemmLaunch {
  int kind, tile;
  size_t off;  // byte offset of the task array in the device table
  int ntasks, total;
  double flops;
  // Algorithmic HBM bytes of one launch: every operand read once, every
  // output written once, in the designed layout; UPDX differs on the last
  // iteration (caller's param or output instead of the next X copies).
  double bytes, bytes_fin;
  int group;  // direct NS: the kind; Gram-space NS: a GramGroup
  int bk = 64;  // K depth of a main-loop stage (bf16 kernels)
};

// Launch groups of Gram-space NS: one product with its buffers.  P of a
// window's first step lands in Q_a (Q starts as that P); later steps write
// P to pm and multiply into the other Q buffer.
enum GramGroup : int {
  GG_SYRK = 100,   // A = X X^T
  GG_P_QA,         // P = a I + b A + c A^2 -> Q_a
  GG_P_PM,         //                        -> pm
  GG_PA_QA,        // pa = P A, P in Q_a
  GG_PA_PM,        //           P in pm
  GG_A_QA,         // A = P pa, P in Q_a
  GG_A_PM,         //           P in pm
  GG_Q_AB,         // Q_b = pm Q_a
  GG_Q_BA,         // Q_a = pm Q_b
  GG_QX_QA,        // X = Q X, Q in Q_a
  GG_QX_QB,        //          Q in Q_b
};

struct Plan {
  std::vector<int64_t> key;
  uint64_t hash = 0;
  int device = -1;
  void* dtab = nullptr;            // device copy of `image`
  bool owns_dtab = true;           // dtab is this plan's own allocation
  std::vector<char> image;         // the launch tables (host copy)
  int f32_ops = 0;
  int f16 = 0;
  int gram = 0;
  int local = 0;
  size_t in_off = 0, norm_off = 0, fin_off = 0;
  int nmat = 0, in_tiles = 0, fin_blocks = 0;
  // Gram-space NS with fp16 operands: the X conversion after the norm
  size_t x16_off = 0;
  int x16_tiles = 0;
  double x16_bytes = 0;
  double in_bytes = 0, norm_bytes = 0, fin_bytes = 0;
  std::vector<GemmLaunch> gemms;  // SYRK launches, then POLY, then UPDX
  ~Plan() {
    if (dtab && owns_dtab) {
      int cur = -1;
      (void)hipGetDevice(&cur);
      (void)hipSetDevice(device);
      (void)hipDeviceSynchronize();
      (void)hipFree(dtab);
      (void)hipSetDevice(cur);
    }
  }
};

std::mutex g_plan_mu;
// Most recently used last.  Never destroyed: freeing device memory from a
// static destructor could run after the HIP runtime has shut down.  Plans
// are keyed by shapes and options only, so a training loop uses one per
// batch layout; the eviction (a device synchronization and a free) happens
// only past kMaxPlans distinct layouts.  A recorded graph shares its plan,
// so an evicted plan lives on until the last graph that launches its
// tables is destroyed.
std::vector<std::shared_ptr<Plan>>& g_plans = *new std::vector<std::shared_ptr<Plan>>();
constexpr size_t kMaxPlans = 256;
// Plans built so far (dmuon_plan_builds).
int64_t g_plan_builds = 0;

// Slot Refs of matrix i's caller buffers.
Ref src_slot(int i) { return ref_slot(kSlotsPerMat * i + 0); }
Ref dst_slot(int i) { return ref_slot(kSlotsPerMat * i + 1); }
Ref buf_slot(int i) { return ref_slot(kSlotsPerMat * i + 2); }
Ref wsr(size_t off) { return (Ref)off; }

bool vec_ok(const void* p, int dtype, int64_t n) {
  const size_t need = dtype == DMUON_F32 ? 16 : 8;
  return p && reinterpret_cast<uintptr_t>(p) % need == 0 && n % 4 == 0;
}

// Gram-space NS launch groups, appended to `gtasks`: one group per
// (product, buffers), split by tile class like the direct kinds.  fp32
// operands, or (h16) fp16 ones: X as normalized by gram16_x_kernel, A and
// P A stored times kF16AScale, P and Q times kF16BScale (the direct fp16
// mode's A and B scales, which its SYRK, polynomial and X-update epilogues
// apply), fp32 accumulation, and the fp32 A beside its fp16 form for the
// polynomial's linear term.
void build_gram_groups(const Layout& L, const dmuon_batch_t* dst, bool ns_only, Plan* plan,
                       std::vector<GemmTab>& gtasks,
                       std::vector<std::pair<size_t, size_t>>& ranges) {
  const int n = (int)L.g.size();
  const bool h16 = !L.f32_ops;
  const double e = h16 ? 2.0 : 4.0;  // operand bytes
  auto none = [](GemmTab& t) {
    t.L = t.R0 = t.R1 = t.fbuf = t.out0 = t.out1 = t.out2 = t.scale = t.xlo = t.ahl = t.sink =
        t.dst = kRefNone;
  };
  // `fill` sets the product-specific fields of one matrix's task and adds
  // its algorithmic flops and bytes.
  auto add_group = [&](int group, int kind, auto&& fill) {
    for (int tile : kTiles) {
      const size_t begin = gtasks.size();
      int acc = 0;
      double flops = 0, bytes = 0, bytes_fin = 0;
      for (int i = 0; i < n; ++i) {
        const Geom& G = L.g[i];
        if (G.tile != tile) continue;
        GemmTab t{};
        none(t);
        t.P = (int)G.P;
        t.scale = wsr(L.scale_off + 16 * (size_t)i);
        const int nt = (int)G.P / tile;
        t.tiles_m = t.tiles_n = nt;
        t.tri = 1;
        t.tile_count = nt * (nt + 1) / 2;
        t.K = t.kper = (int)G.P;
        t.ldl = t.ldr = t.ld0 = (int32_t)(h16 ? G.ld_aop : G.ld_a32);
        t.ld_f = (int32_t)G.ld_a32;
        fill(t, G, i, tile, flops, bytes, bytes_fin);
        t.tile_begin = acc;
        acc += t.tile_count;
        gtasks.push_back(t);
      }
      if (gtasks.size() > begin) {
        plan->gemms.push_back(GemmLaunch{kind, tile, 0, (int)(gtasks.size() - begin), acc, flops,
                                         bytes, kind == KIND_UPDX ? bytes_fin : bytes, group});
        ranges.push_back({begin, gtasks.size()});
      }
    }
  };
  using D = double;
  // A = X X^T (fp32 operands: scaled by 1/(||u||+eps)^2 on the first
  // window; fp16: X is normalized already)
  add_group(GG_SYRK, KIND_SYRK, [&](GemmTab& t, const Geom& G, int, int, D& f, D& b, D&) {
    t.L = t.R0 = t.R1 = wsr(h16 ? G.xb : G.xm);
    t.ldl = t.ldr = (int32_t)(h16 ? G.ld_xb : G.ld_xm);
    t.K = t.kper = (int)G.Q;
    t.fbuf = wsr(G.a32);
    if (h16) t.out0 = wsr(G.aop);
    const D p = (D)G.p, q = (D)G.q;
    f += p * (p + 1) * q;
    // fp16: X in; A's fp16 form and its fp32 upper triangle out
    b += h16 ? 2 * p * q + 2 * p * p + 2 * p * (p + 1) : 4 * p * q + 4 * p * p;
  });
  // P = a I + b A + c A^2 (reads A as both operands and for the b A term)
  for (int g : {GG_P_QA, GG_P_PM})
    add_group(g, KIND_POLY, [&](GemmTab& t, const Geom& G, int, int, D& f, D& b, D&) {
      t.L = t.R0 = t.R1 = wsr(h16 ? G.aop : G.a32);
      t.fbuf = wsr(G.a32);
      t.out0 = wsr(g == GG_P_QA ? G.qa : G.pm);
      t.add_diag = 1;
      const D p = (D)G.p;
      f += p * p * (p + 1);
      b += h16 ? 2 * p * p + 2 * p * (p + 1) + 2 * p * p : 8 * p * p;
    });
  // symmetric products C = L R (all operands commuting polynomials in A);
  // `a_out`: the product is the next A (fp16: its fp32 copy too)
  struct Mul { int group; size_t Geom::*l; size_t Geom::*r; bool a_out; size_t Geom::*out; };
  const Mul muls[] = {{GG_PA_QA, &Geom::qa, nullptr, false, &Geom::pa},
                      {GG_PA_PM, &Geom::pm, nullptr, false, &Geom::pa},
                      {GG_A_QA, &Geom::qa, &Geom::pa, true, nullptr},
                      {GG_A_PM, &Geom::pm, &Geom::pa, true, nullptr},
                      {GG_Q_AB, &Geom::pm, &Geom::qa, false, &Geom::qb},
                      {GG_Q_BA, &Geom::pm, &Geom::qb, false, &Geom::qa}};
  for (const Mul& mu : muls)
    add_group(mu.group, KIND_GRAMMUL, [&](GemmTab& t, const Geom& G, int, int, D& f, D& b, D&) {
      const size_t a_op = h16 ? G.aop : G.a32;  // A as an operand
      t.L = wsr(G.*mu.l);
      t.R0 = t.R1 = wsr(mu.r ? G.*mu.r : a_op);
      t.out0 = wsr(mu.a_out ? a_op : G.*mu.out);
      const D p = (D)G.p;
      f += p * p * (p + 1);
      if (h16) {
        // L is P (times kF16BScale); R is A or P A (kF16AScale) or Q
        // (kF16BScale)
        const bool r_is_q = mu.group == GG_Q_AB || mu.group == GG_Q_BA;
        const float r_scale = r_is_q ? kF16BScale : kF16AScale;
        t.g_in = 1.f / (kF16BScale * r_scale);
        t.g_out = r_scale;
        if (mu.a_out) t.fbuf = wsr(G.a32);
        b += 6 * p * p + (mu.a_out ? 2 * p * (p + 1) : 0.0);
      } else {
        b += 12 * p * p;
      }
    });
  // X = Q X at a window's end (the X update with a = 0); the last window
  // writes the caller's matrix
  for (int g : {GG_QX_QA, GG_QX_QB})
    add_group(g, KIND_UPDX, [&](GemmTab& t, const Geom& G, int i, int tile, D& f, D& b,
                                D& bfin) {
      t.L = wsr(g == GG_QX_QA ? G.qa : G.qb);
      t.R0 = wsr(G.xt0);
      t.R1 = wsr(G.xt1);
      t.ldl = (int32_t)(h16 ? G.ld_aop : G.ld_a32);
      t.ldr = (int32_t)G.ld_xt;
      t.K = t.kper = (int)G.P;
      t.tiles_m = (int)G.P / tile;
      t.tiles_n = (int)G.Q / tile;
      t.tri = 0;
      t.tile_count = t.tiles_m * t.tiles_n;
      t.fbuf = G.hilo ? kRefNone : wsr(G.xm);
      t.ld_f = (int32_t)G.ld_xm;
      if (h16) {  // fp16 X copy and, below 256-wide tiles, its remainder
        t.out0 = wsr(G.xb);
        t.ld0 = (int32_t)G.ld_xb;
        t.xlo = G.hilo ? wsr(G.xlo) : kRefNone;
      }
      t.out1 = wsr(G.xt0);
      t.out2 = wsr(G.xt1);
      t.ld1 = (int32_t)G.ld_xt;
      t.dst = dst_slot(i);
      t.pv = (int32_t)G.p;
      t.qv = (int32_t)G.q;
      t.dst_trans = G.transposed;
      t.dst_dtype = dst->dtype;
      t.sink = wsr(L.sink_off);
      const D p = (D)G.p, q = (D)G.q;
      f += 2 * p * p * q;
      // Q, X^T, and the master X (read for the a X term: fp32, or fp16 hi +
      // remainder, 4 bytes either way); then the master X (fp16 operands:
      // hi + remainder, or fp32 + fp16 copy) and X^T out
      const D master_out = h16 ? (G.hilo ? 4.0 : 6.0) : 4.0;
      const D in = e * p * p + p * q * (e + 4.0);
      b += in + p * q * (e + master_out);
      bfin += in + p * q * esize(dst->dtype) * (ns_only ? 1.0 : 2.0);
    });
}

// Builds the launch tables for one call shape and uploads them.
// `upload`: allocate the plan's device copy of its tables and copy them
// there (blocking); otherwise the caller places plan->image itself.
dmuon_status_t build_plan(const Layout& L, const dmuon_batch_t* src, const dmuon_batch_t* dst,
                          const dmuon_batch_t* bufs, bool ns_only, int device,
                          std::vector<int64_t> key, uint64_t hash, bool upload, Plan** out) {
  auto plan = std::make_unique<Plan>();
  plan->key = std::move(key);
  plan->hash = hash;
  plan->device = device;
  plan->f32_ops = L.f32_ops;
  plan->f16 = L.f16;
  plan->gram = L.gram;
  plan->local = L.local;
  const int n = src->count;
  plan->nmat = n;
  auto scale = [&](int i) { return wsr(L.scale_off + 16 * (size_t)i); };

  std::vector<EwTab> tin(n);
  std::vector<NormTab> tnorm(n);
  int in_begin = 0;
  for (int i = 0; i < n; ++i) {
    const Geom& G = L.g[i];
    EwTab t{};
    t.m = (int32_t)G.m;
    t.n = (int32_t)G.n;
    t.transposed = G.transposed;
    t.in_dtype = src->dtype;
    t.ldx = (int32_t)G.ld_xm;
    t.ldxb = (int32_t)G.ld_xb;
    t.ldt = (int32_t)G.ld_xt;
    t.f32_ops = L.f32_ops;
    t.src = src_slot(i);
    t.buf = bufs ? buf_slot(i) : kRefNone;
    t.xm = G.hilo ? kRefNone : wsr(G.xm);
    t.xb = L.f32_ops ? kRefNone : wsr(G.xb);
    t.xlo = G.hilo ? wsr(G.xlo) : kRefNone;
    t.xt = wsr(G.xt0);
    t.partial = wsr(L.partial_off);
    t.scale = scale(i);
    // input pass: padded oriented extents, mapped to the caller's layout
    EwTab a = t;
    a.rows = (int32_t)(G.transposed ? G.Q : G.P);
    a.cols = (int32_t)(G.transposed ? G.P : G.Q);
    a.tiles_c = a.cols / EW_TILE;
    a.tile_begin = in_begin;
    a.tile_count = (a.rows / EW_TILE) * a.tiles_c;
    in_begin += a.tile_count;
    tin[i] = a;
    tnorm[i] = NormTab{a.tile_begin, a.tile_count, wsr(L.partial_off), scale(i),
                       L.local ? wsr(L.bucket_off + sizeof(float) * i) : kRefNone};
    const double mn = (double)G.m * (double)G.n;
    plan->in_bytes += ns_only ? mn * esize(src->dtype) : mn * (esize(src->dtype) + 8.0);
    plan->norm_bytes += 4.0 * a.tile_count;
  }
  plan->in_tiles = in_begin;
  std::vector<FinTab> tfin;
  if (L.local) {
    int blk = 0;
    for (int i = 0; i < n; ++i) {
      const Geom& G = L.g[i];
      const int nb = (int)((G.P + FIN_ROWS - 1) / FIN_ROWS);
      tfin.push_back(FinTab{blk, nb, (int32_t)G.P, (int32_t)G.ld_a32, wsr(G.a32),
                            wsr(L.bucket_off + sizeof(float) * i), scale(i)});
      blk += nb;
      plan->fin_bytes += 8.0 * (double)G.p * (double)G.p;
    }
    plan->fin_blocks = blk;
  }

  // Gram-space NS with fp16 operands: the conversion of the normalized X
  // (oriented, padded P x Q) into the fp16 operand layout; its X^T goes to
  // xt1, the buffer the first window's X update reads (iteration 1).
  std::vector<EwTab> tx16;
  if (L.gram && !L.f32_ops) {
    int blk = 0;
    for (int i = 0; i < n; ++i) {
      const Geom& G = L.g[i];
      EwTab t{};
      t.m = (int32_t)G.P;
      t.n = (int32_t)G.Q;
      t.rows = (int32_t)G.P;
      t.cols = (int32_t)G.Q;
      t.tiles_c = t.cols / EW_TILE;
      t.tile_begin = blk;
      t.tile_count = (t.rows / EW_TILE) * t.tiles_c;
      t.ldx = (int32_t)G.ld_xm;
      t.ldxb = (int32_t)G.ld_xb;
      t.ldt = (int32_t)G.ld_xt;
      t.src = t.buf = t.partial = kRefNone;
      t.xm = G.hilo ? kRefNone : wsr(G.xm);
      t.xb = wsr(G.xb);
      t.xlo = G.hilo ? wsr(G.xlo) : kRefNone;
      t.xt = wsr(G.xt1);
      t.scale = scale(i);
      blk += t.tile_count;
      tx16.push_back(t);
      // master in (4 bytes); master (4, or fp32 + fp16 copy: 6) and fp16 X^T out
      plan->x16_bytes += (double)G.p * (double)G.q * (4.0 + (G.hilo ? 4.0 : 6.0) + 2.0);
    }
    plan->x16_tiles = blk;
  }

  // GEMM tasks, grouped by (kind, tile class).
  std::vector<GemmTab> gtasks;
  const int kinds_direct[3] = {KIND_SYRK, KIND_POLY, KIND_UPDX};
  std::vector<std::pair<size_t, size_t>> ranges;  // [begin, end) in gtasks per launch
  if (L.gram) build_gram_groups(L, dst, ns_only, plan.get(), gtasks, ranges);
  for (int kind : (L.gram ? std::vector<int>() : std::vector<int>(kinds_direct, kinds_direct + 3))) {
    for (int tile : kTiles) {
      // 128-deep stages for a 64-wide SYRK or polynomial launch (bf16) whose
      // every K is a multiple of 128 and at least kDeepMinK (long loops at
      // few blocks per CU); otherwise 64.  Never two launches per group.
      int bk = 64;
      if (!L.f32_ops && tile == 64 && kind != KIND_UPDX) {
        bool deep = false;
        for (const Geom& G : L.g) {
          if (G.tile != tile) continue;
          const int64_t Kt = kind == KIND_SYRK ? G.Q : (G.split_a ? 3 * G.P : G.P);
          deep = Kt % 128 == 0 && Kt >= kDeepMinK;
          if (!deep) break;
        }
        if (deep) bk = 128;
      }
      // The 16-wide class speeds the SYRK and polynomial (K split over the
      // block's waves); its X updates run on 64-wide tiles (P and Q are
      // multiples of 64 for every class).
      const int ltile = (kind == KIND_UPDX && tile < 64) ? 64 : tile;
      const size_t begin = gtasks.size();
      int acc = 0;
      double flops = 0, bytes = 0, bytes_fin = 0;
      for (int i = 0; i < n; ++i) {
        const Geom& G = L.g[i];
        if (G.tile != tile) continue;
        GemmTab t{};
        t.L = t.R0 = t.R1 = t.fbuf = t.out0 = t.out1 = t.out2 = t.scale = t.xlo = t.ahl =
            t.sink = t.dst = kRefNone;
        const int P = (int)G.P, Q = (int)G.Q;
        const int nt = P / ltile;
        const double p = (double)G.p, q = (double)G.q;
        t.P = P;
        t.scale = scale(i);
        if (kind == KIND_SYRK) {
          t.L = wsr(L.f32_ops ? G.xm : G.xb);
          t.R0 = t.R1 = t.L;
          t.ldl = t.ldr = (int32_t)(L.f32_ops ? G.ld_xm : G.ld_xb);
          t.K = t.kper = Q;
          t.tiles_m = t.tiles_n = nt;
          t.tri = 1;
          t.tile_count = nt * (nt + 1) / 2;
          t.split = G.split_a;  // writes A as [hi|lo|hi|hi] rows, no fp32 A
          t.fbuf = t.split ? kRefNone : wsr(G.a32);
          t.ld_f = (int32_t)G.ld_a32;
          t.out0 = L.f32_ops ? kRefNone : wsr(G.aop);
          t.ld0 = (int32_t)G.ld_aop;
          flops += p * (p + 1) * q;
          // X operand in; fp32 A (bf16 operands: upper triangle only) and/or
          // its operand form out
          bytes += (L.f32_ops ? 4.0 : 2.0) * p * q +
                   (L.f32_ops ? 4.0 * p * p
                              : G.split_a ? 8.0 * p * p : 2.0 * p * p + 2.0 * p * (p + 1));
        } else if (kind == KIND_POLY) {
          t.split = G.split_b;  // writes B as [hi|lo]
          // Split A: L = columns 0..3P of the [hi|lo|hi|hi] rows, R =
          // columns P..4P, so L R^T = hi lo^T + lo hi^T + hi hi^T.
          t.L = wsr(G.aop);
          t.R0 = t.R1 = wsr(G.aop + (G.split_a ? 2 * (size_t)P : 0));
          t.ldl = t.ldr = (int32_t)G.ld_aop;
          t.K = t.kper = G.split_a ? 3 * P : P;
          t.tiles_m = t.tiles_n = nt;
          t.tri = 1;
          t.tile_count = nt * (nt + 1) / 2;
          t.fbuf = G.split_a ? kRefNone : wsr(G.a32);
          t.ld_f = (int32_t)G.ld_a32;
          t.ahl = G.split_a ? wsr(G.aop) : kRefNone;
          t.ld_ahl = (int32_t)G.ld_aop;
          t.out0 = wsr(G.bop);
          t.ld0 = (int32_t)G.ld_bop;
          flops += p * p * (p + 1);
          // A in (fp32; bf16 + fp32; or the split rows); B operand out
          bytes += p * p * ((L.f32_ops ? 4.0 : G.split_a ? 8.0 : 6.0) +
                            (L.f32_ops ? 4.0 : G.split_b ? 4.0 : 2.0));
        } else {
          t.L = wsr(G.bop);
          t.R0 = wsr(G.xt0);
          t.R1 = wsr(G.xt1);
          t.ldl = (int32_t)G.ld_bop;
          t.ldr = (int32_t)G.ld_xt;
          t.K = G.split_b ? 2 * P : P;
          t.kper = P;
          t.tiles_m = nt;
          t.tiles_n = Q / ltile;
          t.tri = 0;
          t.tile_count = t.tiles_m * t.tiles_n;
          t.fbuf = G.hilo ? kRefNone : wsr(G.xm);
          t.ld_f = (int32_t)G.ld_xm;
          t.out0 = L.f32_ops ? kRefNone : wsr(G.xb);
          t.xlo = G.hilo ? wsr(G.xlo) : kRefNone;
          t.ld0 = (int32_t)G.ld_xb;
          t.sink = wsr(L.sink_off);
          t.out1 = wsr(G.xt0);
          t.out2 = wsr(G.xt1);
          t.ld1 = (int32_t)G.ld_xt;
          t.dst = dst_slot(i);
          t.pv = (int32_t)G.p;
          t.qv = (int32_t)G.q;
          t.dst_trans = G.transposed;
          t.dst_dtype = dst->dtype;
          flops += 2.0 * p * p * q;
          // B operand, X^T and the master X (fp32, or bf16 X + remainder)
          // in; then the master X and X^T out, or (last iteration) the
          // caller's matrix read (update only) and written
          {
            const double bop = L.f32_ops ? 4.0 : G.split_b ? 4.0 : 2.0;
            const double xt = L.f32_ops ? 4.0 : 2.0;
            const double in = p * p * bop + p * q * (xt + 4.0);
            // master out: fp32 (+ bf16 copy), or bf16 X + remainder
            bytes += in + p * q * (xt + (L.f32_ops ? 4.0 : G.hilo ? 4.0 : 6.0));
            bytes_fin += in + p * q * esize(dst->dtype) * (ns_only ? 1.0 : 2.0);
          }
        }
        t.tile_begin = acc;
        // column windows (win_decode): whole windows of 256 tiles starting on
        // a window boundary, 8, 16, 32 or 64 tile rows
        t.win = !t.tri && !L.f32_ops && t.tiles_m % 8 == 0 && 256 % t.tiles_m == 0 &&
                t.tile_count % 256 == 0 && t.tile_begin % 256 == 0;
        acc += t.tile_count;
        gtasks.push_back(t);
      }
      if (gtasks.size() > begin) {
        GemmLaunch gl{kind, ltile, 0, (int)(gtasks.size() - begin), acc, flops, bytes,
                      kind == KIND_UPDX ? bytes_fin : bytes, kind, bk};
        plan->gemms.push_back(gl);
        ranges.push_back({begin, gtasks.size()});
      }
    }
  }

  // One device allocation holds every table.
  size_t off = 0;
  auto place = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 64);
    return o;
  };
  plan->in_off = place(sizeof(EwTab) * n);
  plan->norm_off = place(sizeof(NormTab) * n);
  plan->fin_off = place(sizeof(FinTab) * tfin.size());
  plan->x16_off = place(sizeof(EwTab) * tx16.size());
  const size_t g_off = place(sizeof(GemmTab) * gtasks.size());
  for (size_t k = 0; k < plan->gemms.size(); ++k)
    plan->gemms[k].off = g_off + sizeof(GemmTab) * ranges[k].first;
  std::vector<char>& host = plan->image;
  host.assign(off, 0);
  std::memcpy(host.data() + plan->in_off, tin.data(), sizeof(EwTab) * n);
  std::memcpy(host.data() + plan->norm_off, tnorm.data(), sizeof(NormTab) * n);
  if (!tfin.empty())
    std::memcpy(host.data() + plan->fin_off, tfin.data(), sizeof(FinTab) * tfin.size());
  if (!tx16.empty())
    std::memcpy(host.data() + plan->x16_off, tx16.data(), sizeof(EwTab) * tx16.size());
  if (!gtasks.empty())
    std::memcpy(host.data() + g_off, gtasks.data(), sizeof(GemmTab) * gtasks.size());
  if (!upload) {
    plan->owns_dtab = false;
    *out = plan.release();
    return DMUON_OK;
  }
  hipError_t e = hipMalloc(&plan->dtab, off);
  if (e != hipSuccess) {
    plan->dtab = nullptr;
    return fail(DMUON_E_HIP, std::string("hipMalloc(launch tables): ") + hipGetErrorString(e));
  }
  e = hipMemcpy(plan->dtab, host.data(), off, hipMemcpyHostToDevice);
  if (e != hipSuccess)
    return fail(DMUON_E_HIP, std::string("hipMemcpy(launch tables): ") + hipGetErrorString(e));
  *out = plan.release();
  return DMUON_OK;
}

// Looks up (or builds) the plan of a call's shapes and options; caller
// holds g_plan_mu.  Nothing in the key depends on the call's pointers: a
// later call with other buffers (or another workspace) of the same shapes
// reuses the plan without touching device memory.
dmuon_status_t get_plan(const Layout& L, const dmuon_batch_t* src, const dmuon_batch_t* dst,
                        const dmuon_batch_t* bufs, bool ns_only, std::shared_ptr<Plan>* out) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(DMUON_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::vector<int64_t> key;
  key.reserve(10 + 3 * (size_t)src->count);
  key.push_back(device);
  key.push_back(ns_only);
  key.push_back(L.f32_ops + 2 * L.f16);  // f16: a tile-class mask
  key.push_back(L.gram);
  key.push_back(L.local);
  key.push_back(src->dtype);
  key.push_back(dst->dtype);
  key.push_back(bufs != nullptr);
  key.push_back(src->count);
  for (int i = 0; i < src->count; ++i) {
    key.push_back(src->mats[i].m);
    key.push_back(src->mats[i].n);
    key.push_back(L.g[i].split_a + 2 * L.g[i].split_b + 4 * L.g[i].transposed);
  }
  uint64_t hash = 1469598103934665603ull;  // FNV-1a over the key words
  for (int64_t w : key) {
    hash ^= (uint64_t)w;
    hash *= 1099511628211ull;
  }
  for (size_t k = g_plans.size(); k-- > 0;) {
    if (g_plans[k]->hash == hash && g_plans[k]->key == key) {
      if (k + 1 != g_plans.size()) {
        std::shared_ptr<Plan> hit = std::move(g_plans[k]);
        g_plans.erase(g_plans.begin() + (long)k);
        g_plans.push_back(std::move(hit));
      }
      *out = g_plans.back();
      return DMUON_OK;
    }
  }
  Plan* p = nullptr;
  dmuon_status_t st =
      build_plan(L, src, dst, bufs, ns_only, device, std::move(key), hash, true, &p);
  if (st != DMUON_OK) return st;
  ++g_plan_builds;
  if (g_plans.size() >= kMaxPlans) g_plans.erase(g_plans.begin());
  g_plans.emplace_back(p);
  *out = g_plans.back();
  return DMUON_OK;
}

// Uploads the call's buffer pointers into the workspace's slot array (see
// Bases), stream-ordered before the call's kernels.
dmuon_status_t upload_slots(const Layout& L, const dmuon_batch_t* src, const dmuon_batch_t* dst,
                            const dmuon_batch_t* bufs, char* ws, hipStream_t s, Bases* b) {
  const int n = src->count;
  std::vector<void*> v((size_t)kSlotsPerMat * n, nullptr);
  for (int i = 0; i < n; ++i) {
    v[kSlotsPerMat * i + 0] = src->mats[i].ptr;
    v[kSlotsPerMat * i + 1] = dst->mats[i].ptr;
    v[kSlotsPerMat * i + 2] = bufs ? bufs->mats[i].ptr : nullptr;
  }
  void** slots = reinterpret_cast<void**>(ws + L.slot_off);
  const hipError_t e = launch_upload(slots, v.data(), sizeof(void*) * v.size(), s);
  if (e != hipSuccess) return fail(DMUON_E_HIP, std::string("pointer upload: ") + hipGetErrorString(e));
  b->ws = ws;
  b->slots = slots;
  return DMUON_OK;
}

// ------------------------------------------------------------- profiling --

struct ProfRec {
  int kind;
  hipEvent_t e0, e1;
  double flops, bytes;
};

struct Prof {
  bool on = false;
  uint32_t mask = 0;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local Prof g_prof;

const char* kKindNames[KIND_COUNT] = {"momentum", "input", "norm", "syrk", "poly",
                                      "update_x", "clip_norm", "clip_scale", "adamw",
                                      "gram_mul", "gram_x"};

template <class F>
hipError_t timed(int kind, double flops, double bytes, hipStream_t s, F&& launch) {
  if (!g_prof.on || !(g_prof.mask & (1u << kind))) return launch();
  hipEvent_t e0 = g_prof.get(), e1 = g_prof.get();
  if (e0) (void)hipEventRecord(e0, s);
  const hipError_t err = launch();
  if (e1) (void)hipEventRecord(e1, s);
  if (e0 && e1) g_prof.recs.push_back({kind, e0, e1, flops, bytes});
  return err;
}

// Step indices where Gram-space NS windows start, plus ns_steps at the end.
std::vector<int> gram_cuts(const dmuon_ns_cfg_t* cfg) {
  const int n = cfg->ns_steps;
  std::vector<int> cuts = {0, n};
  if (cfg->restarts) {
    for (int i = 0; i < cfg->nrestarts; ++i)
      if (cfg->restarts[i] > 0 && cfg->restarts[i] < n) cuts.push_back(cfg->restarts[i]);
  } else if (2 < n) {
    cuts.push_back(2);  // default restart
  }
  std::sort(cuts.begin(), cuts.end());
  cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
  return cuts;
}

// Launches every group `gid` of a Gram-space plan.
dmuon_status_t gram_group(const Plan& plan, int gid, const IterArgs& args, Bases b,
                          hipStream_t s) {
  const char* tab = static_cast<const char*>(plan.dtab);
  for (const GemmLaunch& gl : plan.gemms) {
    if (gl.group != gid) continue;
    const GemmTab* tasks = reinterpret_cast<const GemmTab*>(tab + gl.off);
    const double bytes = args.fin != FIN_NONE ? gl.bytes_fin : gl.bytes;
    const int h = plan.f32_ops ? 0 : 1;  // fp16 operands
    const hipError_t e = timed(gl.kind, gl.flops, bytes, s, [&] {
      return launch_gemm(gl.kind, gl.tile, plan.f32_ops, gl.bk, h, h, tasks, gl.ntasks, gl.total,
                         args, b, s);
    });
    if (e != hipSuccess)
      return fail(DMUON_E_HIP, std::string("Gram NS product launch: ") + hipGetErrorString(e));
  }
  return DMUON_OK;
}

// The iteration index the kernels see for window w.  Iteration 0 applies
// the norm's scale (the SYRK by 1/(||u||+eps)^2, the X update by
// 1/(||u||+eps)) and its X update reads X^T from xt0; with fp16 operands X
// is normalized before the first window (gram16_x_kernel, which leaves X^T
// in xt1), so the windows count from 1.
int gram_iter(const Plan& plan, int w) { return plan.f32_ops ? w : w + 1; }

// A = X X^T at the start of window w (window 0 scales by 1/(||u||+eps)^2
// through the norm's scale, which is 1 for a shard until the group sum).
dmuon_status_t gram_syrk(const Plan& plan, int w, Bases b, hipStream_t s) {
  IterArgs base{};
  base.iter = gram_iter(plan, w);
  return gram_group(plan, GG_SYRK, base, b, s);
}

// The steps of window w on its A: per step P, then Q <- P Q and A <- P (P A)
// (not after the window's last step); then X <- Q X, which on the last
// window writes the caller's matrix (`fin`).
dmuon_status_t gram_window(const Plan& plan, const dmuon_ns_cfg_t* cfg,
                           const std::vector<int>& cuts, int w, int fin, float lr, float decay,
                           Bases b, hipStream_t s) {
  IterArgs base{};
  base.iter = gram_iter(plan, w);  // window 0's X update applies 1/(||u||+eps); X^T ping-pong
  dmuon_status_t st;
  bool q_in_a = true;  // the window's Q lives in Q_a
  for (int k = cuts[w]; k < cuts[w + 1]; ++k) {
    const float* c = cfg->coeffs ? cfg->coeffs + 3 * k : kQuintic;
    IterArgs pa = base;
    pa.a = c[0];
    pa.b = c[1];
    pa.c = c[2];
    const bool first = k == cuts[w];
    if ((st = gram_group(plan, first ? GG_P_QA : GG_P_PM, pa, b, s))) return st;
    if (!first) {
      if ((st = gram_group(plan, q_in_a ? GG_Q_AB : GG_Q_BA, base, b, s))) return st;
      q_in_a = !q_in_a;
    }
    if (k + 1 < cuts[w + 1]) {
      if ((st = gram_group(plan, first ? GG_PA_QA : GG_PA_PM, base, b, s))) return st;
      if ((st = gram_group(plan, first ? GG_A_QA : GG_A_PM, base, b, s))) return st;
    }
  }
  IterArgs qx = base;  // a = 0: X <- s Q X
  qx.fin = fin;
  qx.lr = lr;
  qx.decay = decay;
  return gram_group(plan, q_in_a ? GG_QX_QA : GG_QX_QB, qx, b, s);
}

// Gram-space NS on whole matrices: every window in turn.
dmuon_status_t run_gram(const Plan& plan, const dmuon_ns_cfg_t* cfg, bool ns_only, float lr,
                        float decay, Bases b, hipStream_t s) {
  const std::vector<int> cuts = gram_cuts(cfg);
  const int windows = (int)cuts.size() - 1;
  dmuon_status_t st;
  if (!plan.f32_ops) {
    const EwTab* tx = reinterpret_cast<const EwTab*>(static_cast<const char*>(plan.dtab) +
                                                     plan.x16_off);
    const hipError_t e = timed(KIND_GRAM_X, 0, plan.x16_bytes, s, [&] {
      return launch_gram16_x(tx, plan.nmat, plan.x16_tiles, b, s);
    });
    if (e != hipSuccess)
      return fail(DMUON_E_HIP, std::string("Gram fp16 X launch: ") + hipGetErrorString(e));
  }
  for (int w = 0; w < windows; ++w) {
    if ((st = gram_syrk(plan, w, b, s))) return st;
    const int fin = w == windows - 1 ? (ns_only ? FIN_OUTPUT : FIN_UPDATE) : FIN_NONE;
    if ((st = gram_window(plan, cfg, cuts, w, fin, lr, decay, b, s))) return st;
  }
  return DMUON_OK;
}

dmuon_status_t run(const Plan& plan, const dmuon_ns_cfg_t* cfg, bool ns_only, float momentum,
                   int nesterov, float lr, float decay, Bases b, hipStream_t s) {
  const char* tab = static_cast<const char*>(plan.dtab);
  auto check = [](hipError_t e, const char* what) -> dmuon_status_t {
    if (e == hipSuccess) return DMUON_OK;
    return fail(DMUON_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  };
  const EwTab* tin = reinterpret_cast<const EwTab*>(tab + plan.in_off);
  const NormTab* tnorm = reinterpret_cast<const NormTab*>(tab + plan.norm_off);
  dmuon_status_t st = check(
      timed(ns_only ? KIND_INPUT : KIND_MOMENTUM, 0, plan.in_bytes, s,
            [&] { return launch_momentum(tin, plan.nmat, plan.in_tiles, momentum, nesterov,
                                         ns_only, b, s); }),
      "momentum/input launch");
  if (st) return st;
  st = check(timed(KIND_NORM, 0, plan.norm_bytes, s,
                   [&] { return launch_norm(tnorm, plan.nmat, cfg->eps, b, s); }),
             "norm launch");
  if (st) return st;
  // a shard stops at its first partial Gram matrix: the group sums come next
  if (plan.local) return gram_syrk(plan, 0, b, s);
  if (plan.gram) return run_gram(plan, cfg, ns_only, lr, decay, b, s);
  for (int it = 0; it < cfg->ns_steps; ++it) {
    const float* c = cfg->coeffs ? cfg->coeffs + 3 * it : kQuintic;
    IterArgs args{};
    args.iter = it;
    args.a = c[0];
    args.b = c[1];
    args.c = c[2];
    // The last X update writes the caller's param (or output) directly.
    if (it == cfg->ns_steps - 1) {
      args.fin = ns_only ? FIN_OUTPUT : FIN_UPDATE;
      args.lr = lr;
      args.decay = decay;
    }
    for (const GemmLaunch& gl : plan.gemms) {
      const GemmTab* tasks = reinterpret_cast<const GemmTab*>(tab + gl.off);
      const double bytes = args.fin != FIN_NONE ? gl.bytes_fin : gl.bytes;
      // fp16 mode: bf16 products on iteration 0 (its input is not yet
      // normalized), fp16 after; iteration 0's X update writes fp16 copies
      const bool f16 = (plan.f16 >> tile_index(gl.tile)) & 1;
      const int h = f16 && it > 0;
      const int hn = f16 && it + 1 < cfg->ns_steps ? 1 : h;
      st = check(timed(gl.kind, gl.flops, bytes, s,
                       [&] {
                         return launch_gemm(gl.kind, gl.tile, plan.f32_ops, gl.bk, h, hn, tasks,
                                            gl.ntasks, gl.total, args, b, s);
                       }),
                 "NS product launch");
      if (st) return st;
    }
  }
  return DMUON_OK;
}

// Gram NS on a shard, window w, once the bucket holds the group's sums:
// (window 0) the normalization, the window's steps and X <- Q X, then the
// next window's partial Gram matrix, or (last window) the output.
dmuon_status_t run_local_advance(const Plan& plan, const dmuon_ns_cfg_t* cfg, int w, Bases b,
                                 hipStream_t s) {
  const std::vector<int> cuts = gram_cuts(cfg);
  const int windows = (int)cuts.size() - 1;
  dmuon_status_t st;
  if (w == 0) {
    const FinTab* tfin =
        reinterpret_cast<const FinTab*>(static_cast<const char*>(plan.dtab) + plan.fin_off);
    const hipError_t e = timed(KIND_NORM, 0, plan.fin_bytes, s, [&] {
      return launch_gram_finalize(tfin, plan.nmat, plan.fin_blocks, cfg->eps, b, s);
    });
    if (e != hipSuccess)
      return fail(DMUON_E_HIP, std::string("Gram finalize launch: ") + hipGetErrorString(e));
  }
  const bool last = w == windows - 1;
  if ((st = gram_window(plan, cfg, cuts, w, last ? FIN_OUTPUT : FIN_NONE, 0.f, 1.f, b, s)))
    return st;
  return last ? DMUON_OK : gram_syrk(plan, w + 1, b, s);
}

dmuon_status_t check_ws(const Layout& L, void* ws, size_t ws_bytes) {
  if (L.total == 0) return DMUON_OK;
  if (!ws) return fail(DMUON_E_WORKSPACE, "workspace: null pointer");
  if (reinterpret_cast<uintptr_t>(ws) % kWsAlign)
    return fail(DMUON_E_WORKSPACE, "workspace: pointer not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(DMUON_E_WORKSPACE, "workspace: " + std::to_string(ws_bytes) + " bytes given, " +
                                       std::to_string(L.total) + " needed");
  return DMUON_OK;
}

// ------------------------------------------------------- flat launches --
// Task tables of the element-wise companions (clipping, AdamW), cached per
// call signature like the NS plans.
struct FlatPlan {
  std::vector<int64_t> key;
  int device = -1;
  void* dtab = nullptr;
  int ntasks = 0, nblocks = 0;
  ~FlatPlan() {
    if (dtab) {
      int cur = -1;
      (void)hipGetDevice(&cur);
      (void)hipSetDevice(device);
      (void)hipDeviceSynchronize();
      (void)hipFree(dtab);
      (void)hipSetDevice(cur);
    }
  }
};
std::vector<std::unique_ptr<FlatPlan>>& g_flat = *new std::vector<std::unique_ptr<FlatPlan>>();

int64_t numel(const dmuon_mat_t& M) { return M.m * M.n; }

// Chunk counts per tensor (chunks of `chunk` elements); fails when the
// launch would not fit int32.
dmuon_status_t flat_blocks(const dmuon_batch_t* b, int64_t chunk, std::vector<FlatTask>* tasks,
                           int* nblocks) {
  int64_t blk = 0;
  tasks->assign(b->count, FlatTask{});
  for (int i = 0; i < b->count; ++i) {
    FlatTask& t = (*tasks)[i];
    t.n = numel(b->mats[i]);
    const int64_t nb = (t.n + chunk - 1) / chunk;
    t.blk_begin = (int32_t)blk;
    t.nblk = (int32_t)nb;
    blk += nb;
    if (blk > INT32_MAX) return fail(DMUON_E_UNSUPPORTED, "batch too large (block count)");
  }
  *nblocks = (int)blk;
  return DMUON_OK;
}

// Looks up (or uploads) the task table for `tasks`; caller holds g_plan_mu.
dmuon_status_t get_flat_plan(const std::vector<FlatTask>& tasks, int nblocks, int64_t op,
                             FlatPlan** out) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(DMUON_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::vector<int64_t> key;
  key.reserve(2 + 8 * tasks.size());
  key.push_back(op);
  key.push_back(device);
  for (const FlatTask& t : tasks) {
    key.push_back(t.n);
    key.push_back(t.bucket);
    key.push_back(t.dtype + 4 * t.gdtype + 16 * t.vec);
    key.push_back((int64_t)reinterpret_cast<uintptr_t>(t.p));
    key.push_back((int64_t)reinterpret_cast<uintptr_t>(t.g));
    key.push_back((int64_t)reinterpret_cast<uintptr_t>(t.m));
    key.push_back((int64_t)reinterpret_cast<uintptr_t>(t.v));
  }
  for (size_t k = 0; k < g_flat.size(); ++k) {
    if (g_flat[k]->key == key) {
      std::unique_ptr<FlatPlan> hit = std::move(g_flat[k]);
      g_flat.erase(g_flat.begin() + (long)k);
      g_flat.push_back(std::move(hit));
      *out = g_flat.back().get();
      return DMUON_OK;
    }
  }
  auto plan = std::make_unique<FlatPlan>();
  plan->key = std::move(key);
  plan->device = device;
  plan->ntasks = (int)tasks.size();
  plan->nblocks = nblocks;
  const size_t bytes = sizeof(FlatTask) * tasks.size();
  e = hipMalloc(&plan->dtab, bytes);
  if (e != hipSuccess) {
    plan->dtab = nullptr;
    return fail(DMUON_E_HIP, std::string("hipMalloc(task table): ") + hipGetErrorString(e));
  }
  e = hipMemcpy(plan->dtab, tasks.data(), bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess)
    return fail(DMUON_E_HIP, std::string("hipMemcpy(task table): ") + hipGetErrorString(e));
  if (g_flat.size() >= kMaxPlans) g_flat.erase(g_flat.begin());
  g_flat.push_back(std::move(plan));
  *out = g_flat.back().get();
  return DMUON_OK;
}

// Clipping workspace: per-block partials, then one factor per bucket.
size_t clip_ws_bytes(int nblocks, int nbuckets) {
  return align_up(sizeof(float) * (size_t)nblocks, kWsAlign) +
         align_up(sizeof(float) * (size_t)nbuckets, kWsAlign);
}

// Gram NS on shards: the flag and backend checks shared by every entry point.
dmuon_status_t check_local(const dmuon_ns_cfg_t* cfg, int32_t transposed) {
  if (transposed != 0 && transposed != 1) return fail(DMUON_E_INVALID, "transposed must be 0 or 1");
  if (!cfg) return fail(DMUON_E_INVALID, "cfg: null");
  if (cfg->backend != DMUON_NS_GRAM)
    return fail(DMUON_E_INVALID, "cfg: the shard entry points run Gram-space NS "
                                 "(backend DMUON_NS_GRAM)");
  if (cfg->prec == DMUON_NS_F16)
    return fail(DMUON_E_UNSUPPORTED, "cfg: Gram-space NS on shards runs with fp32 operands "
                                     "(prec F32 or AUTO)");
  return DMUON_OK;
}

// Validation and layout of a begin / advance call (the shapes, pointers and
// workspace are those of dmuon_ns_orthogonalize).
dmuon_status_t local_setup(const dmuon_batch_t* g, const dmuon_batch_t* out, int32_t transposed,
                           const dmuon_ns_cfg_t* cfg, void* ws, size_t ws_bytes, Layout* L) {
  dmuon_status_t st = check_local(cfg, transposed);
  if (st) return st;
  if ((st = check_batch(g, "g", true))) return st;
  if ((st = check_batch(out, "out", true))) return st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = same_shapes(g, out, "g", "out"))) return st;
  if (g->dtype != out->dtype) return fail(DMUON_E_INVALID, "out dtype must equal g dtype");
  if (g->count == 0) return DMUON_OK;
  if ((st = make_layout(g, cfg->prec, cfg->backend, L, transposed, true))) return st;
  if ((st = check_ws(*L, ws, ws_bytes))) return st;
  std::vector<Span> spans;
  add_spans(spans, g, 0);
  for (int i = 0; i < out->count; ++i)
    if (out->mats[i].ptr != g->mats[i].ptr) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(out->mats[i].ptr);
      spans.push_back({lo, lo + (uintptr_t)(out->mats[i].m * out->mats[i].n * esize(out->dtype)),
                       1, i});
    }
  const uintptr_t wlo = reinterpret_cast<uintptr_t>(ws);
  spans.push_back({wlo, wlo + L->total, 2, 0});
  static const char* const names[] = {"g", "out", "ws"};
  return check_disjoint(spans, names);
}

// Validation of a Muon step's arguments (everything but the workspace and
// the overlap check) and its workspace layout (unset when count == 0).
dmuon_status_t check_step(const dmuon_batch_t* params, const dmuon_batch_t* grads,
                          const dmuon_batch_t* bufs, const dmuon_ns_cfg_t* cfg, float momentum,
                          float lr, float weight_decay, Layout* L) {
  dmuon_status_t st = check_batch(params, "params", true);
  if (st) return st;
  if ((st = check_batch(grads, "grads", true))) return st;
  if ((st = check_batch(bufs, "bufs", true))) return st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = same_shapes(params, grads, "params", "grads"))) return st;
  if ((st = same_shapes(params, bufs, "params", "bufs"))) return st;
  if (bufs->dtype != DMUON_F32) return fail(DMUON_E_INVALID, "bufs must be F32");
  if (!std::isfinite(momentum) || !std::isfinite(lr) || !std::isfinite(weight_decay))
    return fail(DMUON_E_INVALID, "momentum, lr and weight_decay must be finite");
  if (params->count == 0) return DMUON_OK;
  return make_layout(grads, cfg->prec, cfg->backend, L);
}

// Validation of one dmuon_ns_orthogonalize call (also its graph form).
dmuon_status_t check_ns_call(const dmuon_batch_t* g, const dmuon_batch_t* out,
                             const dmuon_ns_cfg_t* cfg, void* ws, size_t ws_bytes, Layout* L) {
  dmuon_status_t st = check_batch(g, "g", true);
  if (st) return st;
  if ((st = check_batch(out, "out", true))) return st;
  if ((st = check_cfg(cfg))) return st;
  if ((st = same_shapes(g, out, "g", "out"))) return st;
  if (g->dtype != out->dtype) return fail(DMUON_E_INVALID, "out dtype must equal g dtype");
  if (g->count == 0) return DMUON_OK;
  if ((st = make_layout(g, cfg->prec, cfg->backend, L))) return st;
  if ((st = check_ws(*L, ws, ws_bytes))) return st;
  // out[i] may be exactly g[i]; nothing else may overlap.
  std::vector<Span> spans;
  add_spans(spans, g, 0);
  for (int i = 0; i < out->count; ++i)
    if (out->mats[i].ptr != g->mats[i].ptr) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(out->mats[i].ptr);
      spans.push_back({lo, lo + (uintptr_t)(out->mats[i].m * out->mats[i].n * esize(out->dtype)),
                       1, i});
    }
  const uintptr_t wlo = reinterpret_cast<uintptr_t>(ws);
  spans.push_back({wlo, wlo + L->total, 2, 0});
  static const char* const names[] = {"g", "out", "ws"};
  return check_disjoint(spans, names);
}

// Validation of one dmuon_muon_step call (also its graph form).
dmuon_status_t check_step_call(const dmuon_batch_t* params, const dmuon_batch_t* grads,
                               const dmuon_batch_t* bufs, const dmuon_ns_cfg_t* cfg,
                               float momentum, float lr, float weight_decay, void* ws,
                               size_t ws_bytes, Layout* L) {
  dmuon_status_t st = check_step(params, grads, bufs, cfg, momentum, lr, weight_decay, L);
  if (st || params->count == 0) return st;
  if ((st = check_ws(*L, ws, ws_bytes))) return st;
  std::vector<Span> spans;
  add_spans(spans, params, 0);
  add_spans(spans, grads, 1);
  add_spans(spans, bufs, 2);
  const uintptr_t wlo = reinterpret_cast<uintptr_t>(ws);
  spans.push_back({wlo, wlo + L->total, 3, 0});
  static const char* const names[] = {"params", "grads", "bufs", "ws"};
  return check_disjoint(spans, names);
}

// The kernels of one NS call on stream s: the pointer upload, then run().
dmuon_status_t enqueue_ns(const Plan& plan, const Layout& L, const dmuon_batch_t* g,
                          const dmuon_batch_t* out, const dmuon_ns_cfg_t* cfg, void* ws,
                          hipStream_t s) {
  Bases b;
  dmuon_status_t st = upload_slots(L, g, out, nullptr, static_cast<char*>(ws), s, &b);
  if (st) return st;
  return run(plan, cfg, true, 0.f, 0, 0.f, 1.f, b, s);
}

// The kernels of one Muon step on stream s.
dmuon_status_t enqueue_step(const Plan& plan, const Layout& L, const dmuon_batch_t* params,
                            const dmuon_batch_t* grads, const dmuon_batch_t* bufs,
                            const dmuon_ns_cfg_t* cfg, float momentum, float lr,
                            float weight_decay, int32_t nesterov, void* ws, hipStream_t s) {
  // decoupled weight decay on the pre-update parameter
  const float decay = (float)(1.0 - (double)lr * (double)weight_decay);
  Bases b;
  dmuon_status_t st = upload_slots(L, grads, params, bufs, static_cast<char*>(ws), s, &b);
  if (st) return st;
  return run(plan, cfg, false, momentum, nesterov ? 1 : 0, lr, decay, b, s);
}

}  // namespace

// A recorded call: its executable graph and the plan whose launch tables the
// graph's kernels read.
struct dmuon_graph_s {
  std::shared_ptr<Plan> plan;
  hipGraphExec_t exec = nullptr;
  int device = -1;
};

namespace {

// Records what `enqueue` launches on a private stream into an executable
// graph.  Capture is thread-local: other threads' HIP calls are unaffected.
// Event timing is off while recording (an event would become a graph node).
template <class F>
dmuon_status_t record_graph(std::shared_ptr<Plan> plan, dmuon_graph_t* out, F&& enqueue) {
  int device = -1;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(DMUON_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  hipStream_t cs = nullptr;
  e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess)
    return fail(DMUON_E_HIP, std::string("capture stream: ") + hipGetErrorString(e));
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return fail(DMUON_E_HIP, std::string("hipStreamBeginCapture: ") + hipGetErrorString(e));
  }
  const bool prof = g_prof.on;
  g_prof.on = false;
  const dmuon_status_t st = enqueue(cs);
  g_prof.on = prof;
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(cs, &graph);
  (void)hipStreamDestroy(cs);
  if (st != DMUON_OK || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    if (st != DMUON_OK) return st;
    return fail(DMUON_E_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess)
    return fail(DMUON_E_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
  dmuon_graph_s* g = new dmuon_graph_s;
  g->plan = std::move(plan);
  g->exec = exec;
  g->device = device;
  *out = g;
  return DMUON_OK;
}

}  // namespace

static_assert(sizeof(dmuon_clip_stats_t) == sizeof(dmuon::ClipStats), "clip stats layout");
static_assert(offsetof(dmuon_clip_stats_t, param_count) == offsetof(dmuon::ClipStats, param_count),
              "clip stats layout");

// ================================================================== C ABI ==

extern "C" {

dmuon_status_t dmuon_ns_workspace_size(const dmuon_batch_t* g, const dmuon_ns_cfg_t* cfg,
                                       size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(DMUON_E_INVALID, "bytes: null");
  dmuon_status_t st = check_batch(g, "g", false);
  if (st) return st;
  if (!cfg) return fail(DMUON_E_INVALID, "cfg: null");
  if (cfg->prec < DMUON_NS_F32 || cfg->prec > DMUON_NS_F16)
    return fail(DMUON_E_INVALID, "cfg: unknown precision mode");
  if ((st = check_backend(cfg))) return st;
  Layout L;
  st = make_layout(g, cfg->prec, cfg->backend, &L);
  if (st) return st;
  *bytes = g->count ? L.total : 0;
  return DMUON_OK;
}

dmuon_status_t dmuon_ns_orthogonalize(const dmuon_batch_t* g, const dmuon_batch_t* out,
                                      const dmuon_ns_cfg_t* cfg, void* ws, size_t ws_bytes,
                                      void* stream) {
  g_last_error.clear();
  Layout L;
  dmuon_status_t st = check_ns_call(g, out, cfg, ws, ws_bytes, &L);
  if (st || g->count == 0) return st;
  std::lock_guard<std::mutex> lock(g_plan_mu);
  std::shared_ptr<Plan> plan;
  if ((st = get_plan(L, g, out, nullptr, true, &plan))) return st;
  return enqueue_ns(*plan, L, g, out, cfg, ws, static_cast<hipStream_t>(stream));
}

dmuon_status_t dmuon_muon_step(const dmuon_batch_t* params, const dmuon_batch_t* grads,
                               const dmuon_batch_t* bufs, const dmuon_ns_cfg_t* cfg,
                               float momentum, float lr, float weight_decay, int32_t nesterov,
                               void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Layout L;
  dmuon_status_t st =
      check_step_call(params, grads, bufs, cfg, momentum, lr, weight_decay, ws, ws_bytes, &L);
  if (st || params->count == 0) return st;
  std::lock_guard<std::mutex> lock(g_plan_mu);
  std::shared_ptr<Plan> plan;
  if ((st = get_plan(L, grads, params, bufs, false, &plan))) return st;
  return enqueue_step(*plan, L, params, grads, bufs, cfg, momentum, lr, weight_decay, nesterov,
                      ws, static_cast<hipStream_t>(stream));
}

dmuon_status_t dmuon_muon_step_graph(const dmuon_batch_t* params, const dmuon_batch_t* grads,
                                     const dmuon_batch_t* bufs, const dmuon_ns_cfg_t* cfg,
                                     float momentum, float lr, float weight_decay,
                                     int32_t nesterov, void* ws, size_t ws_bytes,
                                     dmuon_graph_t* graph) {
  g_last_error.clear();
  if (!graph) return fail(DMUON_E_INVALID, "graph: null");
  *graph = nullptr;
  Layout L;
  dmuon_status_t st =
      check_step_call(params, grads, bufs, cfg, momentum, lr, weight_decay, ws, ws_bytes, &L);
  if (st) return st;
  if (params->count == 0) return fail(DMUON_E_INVALID, "params: an empty batch has no graph");
  std::lock_guard<std::mutex> lock(g_plan_mu);
  std::shared_ptr<Plan> plan;
  if ((st = get_plan(L, grads, params, bufs, false, &plan))) return st;
  const Plan& pl = *plan;
  return record_graph(std::move(plan), graph, [&](hipStream_t s) {
    return enqueue_step(pl, L, params, grads, bufs, cfg, momentum, lr, weight_decay, nesterov, ws,
                        s);
  });
}

dmuon_status_t dmuon_ns_orthogonalize_graph(const dmuon_batch_t* g, const dmuon_batch_t* out,
                                            const dmuon_ns_cfg_t* cfg, void* ws,
                                            size_t ws_bytes, dmuon_graph_t* graph) {
  g_last_error.clear();
  if (!graph) return fail(DMUON_E_INVALID, "graph: null");
  *graph = nullptr;
  Layout L;
  dmuon_status_t st = check_ns_call(g, out, cfg, ws, ws_bytes, &L);
  if (st) return st;
  if (g->count == 0) return fail(DMUON_E_INVALID, "g: an empty batch has no graph");
  std::lock_guard<std::mutex> lock(g_plan_mu);
  std::shared_ptr<Plan> plan;
  if ((st = get_plan(L, g, out, nullptr, true, &plan))) return st;
  const Plan& pl = *plan;
  return record_graph(std::move(plan), graph,
                      [&](hipStream_t s) { return enqueue_ns(pl, L, g, out, cfg, ws, s); });
}

dmuon_status_t dmuon_graph_launch(dmuon_graph_t graph, void* stream) {
  g_last_error.clear();
  if (!graph) return fail(DMUON_E_INVALID, "graph: null");
  int device = -1;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(DMUON_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (device != graph->device)
    return fail(DMUON_E_INVALID, "graph: recorded on device " + std::to_string(graph->device) +
                                     ", launched with device " + std::to_string(device) +
                                     " current");
  e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DMUON_E_HIP, std::string("hipGraphLaunch: ") + hipGetErrorString(e));
  return DMUON_OK;
}

void dmuon_graph_destroy(dmuon_graph_t graph) {
  if (!graph) return;
  int cur = -1;
  (void)hipGetDevice(&cur);
  (void)hipSetDevice(graph->device);
  // launches still in flight finish before the executable graph goes
  (void)hipDeviceSynchronize();
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipSetDevice(cur);
  std::lock_guard<std::mutex> lock(g_plan_mu);  // the plan's last owner may be this graph
  delete graph;
}

dmuon_status_t dmuon_muon_step_noalloc(const dmuon_batch_t* params, const dmuon_batch_t* grads,
                                       const dmuon_batch_t* bufs, const dmuon_ns_cfg_t* cfg,
                                       float momentum, float lr, float weight_decay,
                                       int32_t nesterov, void* stream) {
  g_last_error.clear();
  Layout L;
  dmuon_status_t st = check_step(params, grads, bufs, cfg, momentum, lr, weight_decay, &L);
  if (st || params->count == 0) return st;
  std::vector<Span> spans;
  add_spans(spans, params, 0);
  add_spans(spans, grads, 1);
  add_spans(spans, bufs, 2);
  static const char* const names[] = {"params", "grads", "bufs"};
  if ((st = check_disjoint(spans, names))) return st;
  // The launch tables, built on the host and not cached: every byte this
  // call needs on the device lives in the static scratch.
  Plan* raw = nullptr;
  if ((st = build_plan(L, grads, params, bufs, false, -1, {}, 0, false, &raw))) return st;
  std::unique_ptr<Plan> plan(raw);
  const size_t tab_off = align_up(L.total, kWsAlign);
  const size_t need = tab_off + plan->image.size();
  if (need > kScratchBytes)
    return fail(DMUON_E_UNSUPPORTED, "this batch needs " + std::to_string(need) +
                                         " bytes of device scratch; the allocation-free step "
                                         "holds " + std::to_string(kScratchBytes) +
                                         " (use dmuon_muon_step with a workspace)");
  void* base = nullptr;
  hipError_t e = scratch_address(&base);
  if (e != hipSuccess)
    return fail(DMUON_E_HIP, std::string("scratch address: ") + hipGetErrorString(e));
  char* ws = static_cast<char*>(base);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  plan->dtab = ws + tab_off;  // not owned: the plan never frees it
  e = launch_upload(plan->dtab, plan->image.data(), plan->image.size(), s);
  if (e != hipSuccess)
    return fail(DMUON_E_HIP, std::string("launch table upload: ") + hipGetErrorString(e));
  const float decay = (float)(1.0 - (double)lr * (double)weight_decay);
  Bases b;
  if ((st = upload_slots(L, grads, params, bufs, ws, s, &b))) return st;
  return run(*plan, cfg, false, momentum, nesterov ? 1 : 0, lr, decay, b, s);
}

dmuon_status_t dmuon_gram_local_workspace_size(const dmuon_batch_t* g, int32_t transposed,
                                               const dmuon_ns_cfg_t* cfg, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(DMUON_E_INVALID, "bytes: null");
  dmuon_status_t st = check_local(cfg, transposed);
  if (st) return st;
  if ((st = check_batch(g, "g", false))) return st;
  if (cfg->prec < DMUON_NS_F32 || cfg->prec > DMUON_NS_F16)
    return fail(DMUON_E_INVALID, "cfg: unknown precision mode");
  if ((st = check_backend(cfg))) return st;
  Layout L;
  if ((st = make_layout(g, cfg->prec, cfg->backend, &L, transposed, true))) return st;
  *bytes = g->count ? L.total : 0;
  return DMUON_OK;
}

dmuon_status_t dmuon_gram_local_bucket(const dmuon_batch_t* g, int32_t transposed,
                                       const dmuon_ns_cfg_t* cfg, size_t* offset,
                                       int64_t* count, int32_t* windows) {
  g_last_error.clear();
  if (!offset || !count || !windows) return fail(DMUON_E_INVALID, "offset, count, windows: null");
  dmuon_status_t st = check_local(cfg, transposed);
  if (st) return st;
  if ((st = check_batch(g, "g", false))) return st;
  if ((st = check_cfg(cfg))) return st;
  Layout L;
  if ((st = make_layout(g, cfg->prec, cfg->backend, &L, transposed, true))) return st;
  *offset = g->count ? L.bucket_off : 0;
  *count = g->count ? (int64_t)(L.bucket_bytes / sizeof(float)) : 0;
  *windows = (int32_t)gram_cuts(cfg).size() - 1;
  return DMUON_OK;
}

dmuon_status_t dmuon_gram_local_begin(const dmuon_batch_t* g, const dmuon_batch_t* out,
                                      int32_t transposed, const dmuon_ns_cfg_t* cfg, void* ws,
                                      size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Layout L;
  dmuon_status_t st = local_setup(g, out, transposed, cfg, ws, ws_bytes, &L);
  if (st || g->count == 0) return st;
  std::lock_guard<std::mutex> lock(g_plan_mu);
  std::shared_ptr<Plan> plan;
  if ((st = get_plan(L, g, out, nullptr, true, &plan))) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Bases b;
  if ((st = upload_slots(L, g, out, nullptr, static_cast<char*>(ws), s, &b))) return st;
  return run(*plan, cfg, true, 0.f, 0, 0.f, 1.f, b, s);
}

dmuon_status_t dmuon_gram_local_advance(const dmuon_batch_t* g, const dmuon_batch_t* out,
                                        int32_t transposed, const dmuon_ns_cfg_t* cfg,
                                        int32_t window, void* ws, size_t ws_bytes,
                                        void* stream) {
  g_last_error.clear();
  Layout L;
  dmuon_status_t st = local_setup(g, out, transposed, cfg, ws, ws_bytes, &L);
  if (st) return st;
  const int windows = (int)gram_cuts(cfg).size() - 1;
  if (window < 0 || window >= windows)
    return fail(DMUON_E_INVALID, "window must be in [0, " + std::to_string(windows) + ")");
  if (g->count == 0) return DMUON_OK;
  std::lock_guard<std::mutex> lock(g_plan_mu);
  std::shared_ptr<Plan> plan;
  if ((st = get_plan(L, g, out, nullptr, true, &plan))) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Bases b;
  if ((st = upload_slots(L, g, out, nullptr, static_cast<char*>(ws), s, &b))) return st;
  return run_local_advance(*plan, cfg, window, b, s);
}

dmuon_status_t dmuon_clip_workspace_size(const dmuon_batch_t* grads, int32_t nbuckets,
                                         size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(DMUON_E_INVALID, "bytes: null");
  dmuon_status_t st = check_batch(grads, "grads", false);
  if (st) return st;
  if (nbuckets < 1) return fail(DMUON_E_INVALID, "nbuckets must be >= 1");
  std::vector<FlatTask> tasks;
  int nblocks = 0;
  if ((st = flat_blocks(grads, (int64_t)FLAT_STEP * FLAT_ITERS_CLIP, &tasks, &nblocks))) return st;
  *bytes = grads->count ? clip_ws_bytes(nblocks, nbuckets) : 0;
  return DMUON_OK;
}

dmuon_status_t dmuon_clip_grad_norm(const dmuon_batch_t* grads, const int32_t* bucket_of,
                                    int32_t nbuckets, double max_norm, int32_t stats_only,
                                    double norm_type, dmuon_clip_stats_t* stats, void* ws,
                                    size_t ws_bytes, void* stream) {
  g_last_error.clear();
  dmuon_status_t st = check_batch(grads, "grads", true);
  if (st) return st;
  if (nbuckets < 1) return fail(DMUON_E_INVALID, "nbuckets must be >= 1");
  if (!bucket_of && nbuckets != 1)
    return fail(DMUON_E_INVALID, "bucket_of may be null only with one bucket");
  if (!(norm_type > 0.0)) return fail(DMUON_E_INVALID, "norm_type must be > 0 (or +inf)");
  if (!stats_only && !(std::isfinite(max_norm) && max_norm >= 0.0))
    return fail(DMUON_E_INVALID, "max_norm must be finite and >= 0");
  if (!stats) return fail(DMUON_E_INVALID, "stats: null");
  if (reinterpret_cast<uintptr_t>(stats) % 8) return fail(DMUON_E_INVALID, "stats: not 8-byte aligned");
  std::vector<int> used(nbuckets, 0);
  for (int i = 0; i < grads->count; ++i) {
    const int b = bucket_of ? bucket_of[i] : 0;
    if (b < 0 || b >= nbuckets)
      return fail(DMUON_E_INVALID, "bucket_of[" + std::to_string(i) + "] out of range");
    used[b] = 1;
  }
  std::vector<FlatTask> tasks;
  int nblocks = 0;
  if ((st = flat_blocks(grads, (int64_t)FLAT_STEP * FLAT_ITERS_CLIP, &tasks, &nblocks))) return st;
  const size_t need = grads->count ? clip_ws_bytes(nblocks, nbuckets) : 0;
  if (need) {
    if (!ws) return fail(DMUON_E_WORKSPACE, "workspace: null pointer");
    if (reinterpret_cast<uintptr_t>(ws) % kWsAlign)
      return fail(DMUON_E_WORKSPACE, "workspace: pointer not 256-byte aligned");
    if (ws_bytes < need)
      return fail(DMUON_E_WORKSPACE, "workspace: " + std::to_string(ws_bytes) + " bytes given, " +
                                         std::to_string(need) + " needed");
  }
  std::vector<Span> spans;
  add_spans(spans, grads, 0);
  if (need) {
    const uintptr_t wlo = reinterpret_cast<uintptr_t>(ws);
    spans.push_back({wlo, wlo + need, 1, 0});
  }
  const uintptr_t slo = reinterpret_cast<uintptr_t>(stats);
  spans.push_back({slo, slo + sizeof(dmuon_clip_stats_t) * (size_t)nbuckets, 2, 0});
  static const char* const names[] = {"grads", "ws", "stats"};
  if ((st = check_disjoint(spans, names))) return st;

  for (int i = 0; i < grads->count; ++i) {
    FlatTask& t = tasks[i];
    t.bucket = bucket_of ? bucket_of[i] : 0;
    t.dtype = grads->dtype;
    t.p = grads->mats[i].ptr;
    t.vec = vec_ok(t.p, grads->dtype, 4);
  }
  const int mode = std::isinf(norm_type) ? NORM_INF
                   : norm_type == 2.0    ? NORM_L2
                   : norm_type == 1.0    ? NORM_L1
                                         : NORM_P;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_plan_mu);
  FlatPlan* plan = nullptr;
  if (grads->count && (st = get_flat_plan(tasks, nblocks, 1, &plan))) return st;
  const FlatTask* dt = plan ? static_cast<const FlatTask*>(plan->dtab) : nullptr;
  float* partial = static_cast<float*>(ws);
  float* scale = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                          align_up(sizeof(float) * (size_t)nblocks, kWsAlign));
  double bytes = 0;
  for (int i = 0; i < grads->count; ++i) bytes += (double)tasks[i].n * esize(grads->dtype);
  auto check = [](hipError_t e, const char* what) -> dmuon_status_t {
    if (e == hipSuccess) return DMUON_OK;
    return fail(DMUON_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  };
  st = check(timed(KIND_CLIP_NORM, 0, bytes, s,
                   [&] {
                     hipError_t e = hipSuccess;
                     if (nblocks)
                       e = launch_clip_norm(dt, plan->ntasks, nblocks, mode, (float)norm_type,
                                            partial, s);
                     if (e != hipSuccess) return e;
                     return launch_clip_finalize(dt, grads->count, nbuckets, mode, norm_type,
                                                 max_norm, stats_only ? 1 : 0, partial,
                                                 reinterpret_cast<ClipStats*>(stats), scale, s);
                   }),
             "clip norm launch");
  if (st || stats_only || nblocks == 0) return st;
  return check(timed(KIND_CLIP_SCALE, 0, 2.0 * bytes, s,
                     [&] { return launch_clip_scale(dt, plan->ntasks, nblocks, scale, s); }),
               "clip scale launch");
}

dmuon_status_t dmuon_adamw_step(const dmuon_batch_t* params, const dmuon_batch_t* grads,
                                const dmuon_batch_t* exp_avg, const dmuon_batch_t* exp_avg_sq,
                                int64_t step, double lr, double beta1, double beta2,
                                double eps, double weight_decay, void* stream) {
  g_last_error.clear();
  dmuon_status_t st = check_batch(params, "params", true);
  if (st) return st;
  if ((st = check_batch(grads, "grads", true))) return st;
  if ((st = check_batch(exp_avg, "exp_avg", true))) return st;
  if ((st = check_batch(exp_avg_sq, "exp_avg_sq", true))) return st;
  if ((st = same_shapes(params, grads, "params", "grads"))) return st;
  if ((st = same_shapes(params, exp_avg, "params", "exp_avg"))) return st;
  if ((st = same_shapes(params, exp_avg_sq, "params", "exp_avg_sq"))) return st;
  if (exp_avg->dtype != DMUON_F32 || exp_avg_sq->dtype != DMUON_F32)
    return fail(DMUON_E_INVALID, "exp_avg and exp_avg_sq must be F32");
  if (step < 1) return fail(DMUON_E_INVALID, "step counts from 1");
  if (!std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(weight_decay) ||
      !(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps > 0.0))
    return fail(DMUON_E_INVALID, "need finite lr and weight_decay, betas in [0, 1), eps > 0");
  if (params->count == 0) return DMUON_OK;
  std::vector<Span> spans;
  add_spans(spans, params, 0);
  add_spans(spans, grads, 1);
  add_spans(spans, exp_avg, 2);
  add_spans(spans, exp_avg_sq, 3);
  static const char* const names[] = {"params", "grads", "exp_avg", "exp_avg_sq"};
  if ((st = check_disjoint(spans, names))) return st;
  std::vector<FlatTask> tasks;
  int nblocks = 0;
  if ((st = flat_blocks(params, (int64_t)FLAT_STEP * FLAT_ITERS_ADAMW, &tasks, &nblocks))) return st;
  double bytes = 0;
  for (int i = 0; i < params->count; ++i) {
    FlatTask& t = tasks[i];
    t.dtype = params->dtype;
    t.gdtype = grads->dtype;
    t.p = params->mats[i].ptr;
    t.g = grads->mats[i].ptr;
    t.m = static_cast<float*>(exp_avg->mats[i].ptr);
    t.v = static_cast<float*>(exp_avg_sq->mats[i].ptr);
    t.vec = vec_ok(t.p, params->dtype, 4) && vec_ok(t.g, grads->dtype, 4) &&
            vec_ok(t.m, DMUON_F32, 4) && vec_ok(t.v, DMUON_F32, 4);
    bytes += (double)t.n * (2.0 * esize(params->dtype) + esize(grads->dtype) + 16.0);
  }
  // Bias corrections in double, handed to the kernel as fp32 factors.
  AdamArgs a;
  a.decay = (float)(1.0 - lr * weight_decay);
  a.beta1 = (float)beta1;
  a.one_minus_beta1 = (float)(1.0 - beta1);
  a.beta2 = (float)beta2;
  a.one_minus_beta2 = (float)(1.0 - beta2);
  const double bc1 = 1.0 - std::pow(beta1, (double)step);
  const double bc2 = 1.0 - std::pow(beta2, (double)step);
  a.step_size = (float)(lr / bc1);
  a.inv_bc2_sqrt = (float)(1.0 / std::sqrt(bc2));
  a.eps = (float)eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_plan_mu);
  FlatPlan* plan = nullptr;
  if ((st = get_flat_plan(tasks, nblocks, 2, &plan))) return st;
  const hipError_t e = timed(KIND_ADAMW, 0, bytes, s, [&] {
    return launch_adamw(static_cast<const FlatTask*>(plan->dtab), plan->ntasks, nblocks, a, s);
  });
  if (e != hipSuccess) return fail(DMUON_E_HIP, std::string("adamw launch: ") + hipGetErrorString(e));
  return DMUON_OK;
}

const char* dmuon_status_str(dmuon_status_t s) {
  switch (s) {
    case DMUON_OK: return "ok";
    case DMUON_E_INVALID: return "invalid argument";
    case DMUON_E_UNSUPPORTED: return "unsupported";
    case DMUON_E_WORKSPACE: return "workspace";
    case DMUON_E_HIP: return "hip error";
  }
  return "unknown status";
}

const char* dmuon_last_error(void) { return g_last_error.c_str(); }

int64_t dmuon_plan_builds(void) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  return g_plan_builds;
}

const char* dmuon_backend_info(void) {
  return "direct NS (SYRK + symmetric poly + update-X) or Gram-space NS (fp32 or fp16 "
         "operands) . gfx950 MFMA "
         "bf16/fp16 32x32x16 (tiles 64/128/256) / fp32 32x32x2 (tiles 64/128) and 16x16x4 "
         "(tiles 16) . "
         "fp32-grade master X . update fused into the last X product";
}

int32_t dmuon_profile_begin(uint32_t kind_mask) {
  for (ProfRec& r : g_prof.recs) {
    g_prof.pool.push_back(r.e0);
    g_prof.pool.push_back(r.e1);
  }
  g_prof.recs.clear();
  g_prof.mask = kind_mask ? kind_mask : 0xffffffffu;
  g_prof.on = true;
  return 0;
}

int32_t dmuon_profile_end(dmuon_profile_row_t* out, int32_t max) {
  g_prof.on = false;
  dmuon_profile_row_t rows[KIND_COUNT];
  std::memset(rows, 0, sizeof rows);
  int32_t status = 0;
  for (ProfRec& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.e1) != hipSuccess || hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess)
      status = -1;
    dmuon_profile_row_t& row = rows[r.kind];
    row.launches += 1;
    row.ms += ms;
    row.flops += r.flops;
    row.bytes += r.bytes;
    g_prof.pool.push_back(r.e0);
    g_prof.pool.push_back(r.e1);
  }
  g_prof.recs.clear();
  if (status) return fail(DMUON_E_HIP, "profile: event query failed"), -1;
  int32_t k = 0;
  for (int kind = 0; kind < KIND_COUNT; ++kind) {
    if (!rows[kind].launches) continue;
    if (out && k < max) {
      out[k] = rows[kind];
      out[k].kind = kind;
      std::snprintf(out[k].name, sizeof out[k].name, "%s", kKindNames[kind]);
    }
    ++k;
  }
  return out ? std::min(k, max) : k;
}

}  // extern "C"
