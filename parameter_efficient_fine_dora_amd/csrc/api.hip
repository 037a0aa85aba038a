// C ABI of libdora.so: argument validation, workspace layout and the launch
// sequence of the norm, forward and backward.  Every step runs in the
// kernels of gemm.hip and rowwise.hip; nothing here touches tensor data.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dora.h"
#include "entry.h"
#include "kernels.h"

namespace dora {
namespace {

// ---- per-kernel timing (opt-in) ----------------------------------------------

std::atomic<int> g_timing{0};
std::mutex g_mu;
struct Rec {
  const char* label;
  hipEvent_t a, b;
};
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_pool.empty()) {
      hipEvent_t e = g_pool.back();
      g_pool.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// ---- shapes and workspace -------------------------------------------------------

constexpr int64_t kTokPerDmBlock = 64;   // tokens per compose-backward partial sum
constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t esize(int dtype) { return dtype == kBF16 ? 2 : 4; }

// Every row stride the kernels see is d_out, d_in or r; keeping them below
// 2^22 keeps a 256-row tile's byte offsets inside the 31 bits the buffer
// loads use.  Tokens only count rows and may reach 2^31 - 1.
constexpr int64_t kMaxFeature = int64_t(1) << 22;

bool shape_ok(const dora_shape& s) {
  const int64_t lim = int64_t(1) << 31;
  if (s.d_out < 1 || s.d_in < 1 || s.r < 0 || s.tokens < 0) return false;
  if (s.d_out >= kMaxFeature || s.d_in >= kMaxFeature || s.r >= kMaxFeature || s.tokens >= lim)
    return false;
  if (s.d_out % 8 || s.d_in % 8 || s.r % 8) return false;
  const double cap = 4.0e18;
  if ((double)s.d_out * s.d_in > cap || (double)s.tokens * s.d_out > cap ||
      (double)s.tokens * s.d_in > cap || (double)s.r * s.d_in > cap)
    return false;
  return true;
}

// K extent of the cross/Gram projection P = [W0 | B | B] [A | G_hi | G_lo]^T.
int64_t p_depth(const dora_shape& s) { return s.d_in + (s.dtype == kBF16 ? 2 : 1) * s.r; }

int gram_splits(const dora_shape& s) {
  return s.r > 0 ? plan_gemm(s.r, s.r, s.d_in, s.dtype).split : 1;
}
// bf16 layers with a rank reduce the projection to per-row partials inside it
// (||W0_i||^2 from its pass over W0, B_i . P_i from its accumulators); P
// itself is never stored.
bool fused_norm(const dora_shape& s) { return s.dtype == kBF16 && s.r > 0; }
// Small float32 layers run the whole forward (factored norm, xs and the
// compose) in two kernels of their own, where the general path would be
// launch latency throughout.
bool small_path(const dora_shape& s) {
  return s.dtype == kF32 && !(s.flags & DORA_FLAG_SEPARATE_COMPOSE) &&
         small_forward_fits(s.tokens, s.d_out, s.d_in, s.r);
}
// bf16 projections use their own planner (one column tile where the rank fits);
// float32 ones (and the undetached gradient's Q, which stores P) the generic one.
GemmPlan p_plan(const dora_shape& s) {
  if (fused_norm(s)) return plan_norm_projection(s.d_out, s.r, p_depth(s), std::max(s.d_in, s.r));
  return plan_gemm(s.d_out, s.r, p_depth(s), s.dtype);
}
int p_cfg(const dora_shape& s) { return p_plan(s).cfg; }
int p_splits(const dora_shape& s) { return s.r > 0 ? p_plan(s).split : 1; }
// the stored-P projection of the undetached gradient (generic planner)
int q_splits(const dora_shape& s) {
  return s.r > 0 ? plan_gemm(s.d_out, s.r, p_depth(s), s.dtype).split : 1;
}

struct Layout {
  size_t gpart = 0, ghi = 0, glo = 0, P = 0;     // norm
  size_t rowsq = 0, rowdot = 0;                  // norm: the projection's per-row partials
  size_t done = 0;                               // norm: the projection's tile-row counters
  int64_t dot_parts = 0;
  size_t xs = 0, slora = 0;                      // forward
  size_t spart = 0;                              // forward of a small float32 layer: partials
  size_t gz = 0, ts = 0, dmpart = 0, bg = 0;     // backward
  size_t mnorm = 0;                              // merge: the row norms when not given
  size_t vpart = 0;                              // DVoRA: row-block partials of grad_d
  // backward with the undetached norm gradient
  size_t dm = 0, kappa = 0, bk = 0, egpart = 0, eghi = 0, eglo = 0, q = 0, hpart = 0, hmat = 0,
         hlo = 0, d1 = 0;
  int qsplits = 1, hsplits = 1, d1splits = 1;
  size_t scratch = 0, scratch_bytes = 0;         // split-K partial sums
  size_t scratch2 = 0, scratch2_bytes = 0;       // backward: ts's split-K on the side stream
  size_t total = 0;
  int splits = 1, psplits = 1;
  int64_t dm_blocks = 0;
};

Layout layout(const dora_shape& s, int op) {
  Layout L;
  const size_t e = esize(s.dtype);
  const size_t r = (size_t)s.r, T = (size_t)s.tokens;
  const int dt = s.dtype;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  };
  if (op == DORA_OP_FORWARD && small_path(s)) {
    L.xs = take(T * r * e);
    L.spart = take(small_forward_plan(s.d_out, s.d_in).part_bytes);
    L.total = off;
    return L;
  }
  size_t scratch = 0;
  auto need = [&](int64_t M, int64_t N, int64_t K, bool akc = true, bool bkc = true) {
    scratch = std::max(scratch, gemm_scratch_bytes(M, N, K, dt, akc, bkc));
  };
  if (op == DORA_OP_NORM || op == DORA_OP_FORWARD || op == DORA_OP_MERGE) {
    L.psplits = p_splits(s);
    if (fused_norm(s)) {   // bf16: the triangular Gram kernel's partial sums
      L.gpart = take(gram_bf16_plan(s.r, s.d_in).part_bytes);
    } else {
      L.splits = gram_splits(s);
      L.gpart = take((size_t)L.splits * r * r * 4);
    }
    L.ghi = take(r * r * (s.dtype == kBF16 ? 2 : 4));
    L.glo = take(s.dtype == kBF16 ? r * r * 2 : 0);
    if (fused_norm(s)) {
      L.dot_parts = L.psplits * gemm_col_slots(p_cfg(s), s.r);
      L.rowsq = take((size_t)L.psplits * s.d_out * 4);
      L.rowdot = take((size_t)L.dot_parts * s.d_out * 4);
      L.done = take((size_t)gemm_tile_rows(p_cfg(s), s.d_out) * 4);
    } else {
      L.P = take((size_t)L.psplits * s.d_out * r * 4);
    }
  }
  if (op == DORA_OP_VERA_GRADS) L.vpart = take((size_t)vera_dd_blocks(s.d_out) * r * 4);
  if (op == DORA_OP_MERGE) {
    L.mnorm = take((size_t)s.d_out * 4);
    need(s.d_out, s.d_in, s.r, true, false);
  }
  if (op == DORA_OP_FORWARD) {
    L.xs = take(T * r * e);
    // the fused GEMM splits K when its tiles cannot fill the chip (the compose
    // then runs in the fixed-order reduction)
    if (!(s.flags & DORA_FLAG_SEPARATE_COMPOSE)) need(s.tokens, s.d_out, s.d_in + s.r);
    if (s.flags & DORA_FLAG_SEPARATE_COMPOSE) {
      L.slora = take(T * (size_t)s.d_out * e);
      need(s.tokens, s.d_out, s.d_in);
      need(s.tokens, s.d_out, s.r);
    }
    need(s.tokens, s.r, s.d_in);
  }
  if (op == DORA_OP_BACKWARD) {
    L.xs = take(T * r * e);
    L.gz = take(T * (size_t)s.d_out * e);
    L.ts = take(T * r * e);
    L.bg = take((size_t)s.d_out * r * e);
    L.dm_blocks = cdiv(s.tokens, kTokPerDmBlock);
    L.dmpart = take((size_t)L.dm_blocks * s.d_out * 4);
    need(s.tokens, s.r, s.d_in);                         // xs recomputed
    need(s.tokens, s.r, s.d_out);                        // ts = gy Bg
    need(s.tokens, s.d_in, s.d_out + s.r, true, false);  // dx
    need(s.d_out, s.r, s.tokens, false, false);          // dB
    need(s.r, s.d_in, s.tokens, false, false);           // dA
    // ts on the side stream, beside the compose backward
    L.scratch2_bytes = gemm_scratch_bytes(s.tokens, s.r, s.d_out, dt, true, true);
    L.scratch2 = take(L.scratch2_bytes);
    if ((s.flags & DORA_FLAG_EXACT_NORM_GRAD) && s.r > 0) {
      L.dm = take((size_t)s.d_out * 4);
      L.kappa = take((size_t)s.d_out * 4);
      L.bk = take((size_t)s.d_out * r * e);
      L.splits = gram_splits(s);
      L.egpart = take((size_t)L.splits * r * r * 4);
      L.eghi = take(r * r * (s.dtype == kBF16 ? 2 : 4));
      L.eglo = take(s.dtype == kBF16 ? r * r * 2 : 0);
      L.qsplits = q_splits(s);
      L.q = take((size_t)L.qsplits * s.d_out * r * 4);
      L.hsplits = plan_gemm(s.r, s.r, s.d_out, dt, false, false).split;
      L.hpart = take((size_t)L.hsplits * r * r * 4);
      L.hmat = take(r * r * e);
      L.hlo = take(r * r * 2);
      L.d1splits = plan_gemm(s.d_out, s.r, s.tokens, dt, false, false).split;
      L.d1 = take((size_t)L.d1splits * s.d_out * r * 4);
      need(s.r, s.d_in, s.tokens + s.d_out + s.r, false, false);   // dA with the A.1 terms
    }
  }
  L.scratch = take(scratch);
  L.scratch_bytes = scratch;
  L.total = off;
  return L;
}

// A second stream for work that does not depend on the caller's stream's
// current chain (e.g. the down-projection beside the norm).  One per host
// thread and device, default priority, created on first use and kept for the
// life of the process; fork and join go through events, so the pair works
// under stream capture too.  Returns null (run everything on the caller's
// stream) if it cannot be created, and while the timing hook is on, so that
// each kernel's events bracket that kernel alone.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

SideStream* side_stream() {
  if (g_timing.load(std::memory_order_relaxed)) return nullptr;
  constexpr int kMaxDevices = 64;
  static thread_local SideStream per_dev[kMaxDevices];
  static thread_local bool failed[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices || failed[dev])
    return nullptr;
  SideStream& ss = per_dev[dev];
  if (!ss.s) {
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      failed[dev] = true;
      ss.s = nullptr;
      return nullptr;
    }
  }
  return &ss;
}

// Side stream `side` starts after everything enqueued on `st` so far.
hipError_t fork_to(hipStream_t st, SideStream* side) {
  hipError_t e = hipEventRecord(side->fork, st);
  if (e != hipSuccess) return e;
  return hipStreamWaitEvent(side->s, side->fork, 0);
}

// Work enqueued on `st` from now on waits for everything enqueued on `side`.
hipError_t join_from(SideStream* side, hipStream_t st) {
  hipError_t e = hipEventRecord(side->join, side->s);
  if (e != hipSuccess) return e;
  return hipStreamWaitEvent(st, side->join, 0);
}

// A fork of `st` to the side stream that is joined back on every way out of
// the scope: join() on the normal path (its error is reported), the destructor
// on an early return after a failed launch (the caller's stream is then still
// ordered after whatever reached the side stream, and a stream capture is not
// left with an open fork).
class SideFork {
 public:
  SideFork(SideStream* side, hipStream_t st) : side_(side), st_(st) {}
  SideFork(const SideFork&) = delete;
  SideFork& operator=(const SideFork&) = delete;
  ~SideFork() {
    if (forked_) (void)join_from(side_, st_);
  }
  hipStream_t side() const { return side_->s; }
  hipError_t fork() {
    forked_ = true;   // a half-made fork (record done, wait failed) is still joined
    return fork_to(st_, side_);
  }
  hipError_t join() {
    if (!forked_) return hipSuccess;
    forked_ = false;
    return join_from(side_, st_);
  }

 private:
  SideStream* side_;
  hipStream_t st_;
  bool forked_ = false;
};

// Validation-only op id of calls that take no workspace.
constexpr int kOpNoWorkspace = -1;

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(const dora_shape* sh, int op, const void* ws, size_t ws_bytes) {
  if (!sh) return DORA_ERR_NULL;
  if (sh->reserved != 0) return DORA_ERR_FLAGS;
  const uint32_t known = DORA_FLAG_EXACT_NORM_GRAD | DORA_FLAG_SEPARATE_COMPOSE;
  if (sh->flags & ~known) return DORA_ERR_FLAGS;
  if (!std::isfinite(sh->s)) return DORA_ERR_FLAGS;
  if (sh->dtype != DORA_F32 && sh->dtype != DORA_BF16) return DORA_ERR_DTYPE;
  if (!shape_ok(*sh)) return DORA_ERR_SHAPE;
  const size_t need = layout(*sh, op).total;
  if (need > 0 && !ws) return DORA_ERR_NULL;
  if (ws && !aligned(ws)) return DORA_ERR_ALIGN;
  if (ws_bytes < need) return DORA_ERR_WORKSPACE;
  return DORA_OK;
}

// Checks a tensor pointer: required unless the tensor is empty.
int check_ptr(const void* p, bool empty) {
  if (!p) return empty ? DORA_OK : DORA_ERR_NULL;
  return aligned(p) ? DORA_OK : DORA_ERR_ALIGN;
}

#define DORA_CHECK(expr)          \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != DORA_OK) return rc_; \
  } while (0)

#define HIP_TRY(expr)                                 \
  do {                                                \
    if ((expr) != hipSuccess) return DORA_ERR_HIP;    \
  } while (0)

uint8_t* at(void* ws, size_t off) { return reinterpret_cast<uint8_t*>(ws) + off; }

void give_scratch(GemmProblem& g, void* ws, const Layout& L) {
  g.scratch = L.scratch_bytes ? at(ws, L.scratch) : nullptr;
  g.scratch_bytes = L.scratch_bytes;
}

// The backward's second split-K region, for ts on the side stream.
void give_scratch2(GemmProblem& g, void* ws, const Layout& L) {
  g.scratch = L.scratch2_bytes ? at(ws, L.scratch2) : nullptr;
  g.scratch_bytes = L.scratch2_bytes;
}

// Factored norm: G = A A^T (split-K), (s/2) G -> hi/lo, P = 2s W0 A^T + s^2 B G,
// n_i = sqrt(||W0_i||^2 + B_i . P_i).  For bf16 the projection itself reduces
// each row: it sums the squares of the W0 rows it streams and dots its
// accumulators with B, so W0 crosses HBM once and P never reaches it; the last
// workgroup to finish each tile row then adds that row's partials into n.
int run_norm(const dora_shape& s, const void* W0, const void* A, const void* B, float* norm,
             void* ws, const Layout& L, hipStream_t st) {
  const int dt = s.dtype;
  if (s.r == 0) {
    HIP_TRY(row_norm(W0, B, nullptr, L.psplits, norm, s.d_out, s.d_in, s.r, dt, st));
    return DORA_OK;
  }
  float* gpart = reinterpret_cast<float*>(at(ws, L.gpart));
  void* ghi = at(ws, L.ghi);
  void* glo = at(ws, L.glo);
  if (fused_norm(s)) {
    const GramPlan gp = gram_bf16_plan(s.r, s.d_in);
    HIP_TRY(gram_bf16(A, s.r, s.d_in, gp, gpart, st));
    // the finisher also zeroes the projection's tile-row counters
    HIP_TRY(gram_bf16_finish(gpart, gp, s.r, 0.5f * s.s, ghi, glo,
                             reinterpret_cast<uint32_t*>(at(ws, L.done)),
                             gemm_tile_rows(p_cfg(s), s.d_out), st));
  } else {
    GemmProblem g;
    g.M = g.N = s.r;
    g.nseg = 1;
    g.seg[0] = {A, A, s.d_in, s.d_in, s.d_in};
    g.c = gpart;
    g.ldc = s.r;
    g.out_f32 = true;
    g.split = L.splits;
    g.split_stride = s.r * s.r;
    g.cfg = plan_gemm(s.r, s.r, s.d_in, dt).cfg;
    HIP_TRY(gemm(g, dt, st, "gram_AAt"));
    HIP_TRY(gram_finalize(gpart, L.splits, s.r, 0.5f * s.s, dt, ghi, glo, st, "gram_finalize"));
  }

  GemmProblem p;
  p.M = s.d_out;
  p.N = s.r;
  p.seg[0] = {W0, A, s.d_in, s.d_in, s.d_in};
  p.seg[1] = {B, ghi, s.r, s.r, s.r};
  p.nseg = 2;
  if (dt == kBF16) {
    p.seg[2] = {B, glo, s.r, s.r, s.r};
    p.nseg = 3;
  }
  p.alpha = 2.f * s.s;
  p.out_f32 = true;
  p.split = L.psplits;
  p.cfg = p_cfg(s);
  if (fused_norm(s)) {
    float* rowsq = reinterpret_cast<float*>(at(ws, L.rowsq));
    float* rowdot = reinterpret_cast<float*>(at(ws, L.rowdot));
    p.epi = kEpiNorm;
    p.rowsq = rowsq;
    p.rowdot = rowdot;
    p.add = B;
    p.ld_add = s.r;
    // the last workgroup of each tile row adds its rows' partials into n
    p.norm_out = norm;
    p.done = reinterpret_cast<uint32_t*>(at(ws, L.done));
    HIP_TRY(gemm(p, dt, st, "cross_gram_proj"));
    return DORA_OK;
  }
  float* P = reinterpret_cast<float*>(at(ws, L.P));
  p.c = P;
  p.ldc = s.r;
  p.split_stride = s.d_out * s.r;
  HIP_TRY(gemm(p, dt, st, "cross_gram_proj"));
  HIP_TRY(row_norm(W0, B, P, L.psplits, norm, s.d_out, s.d_in, s.r, dt, st));
  return DORA_OK;
}

}  // namespace

LaunchTimer::LaunchTimer(const char* label, hipStream_t st) : label_(label), st_(st) {
  ev_[0] = ev_[1] = nullptr;
  if (!g_timing.load(std::memory_order_relaxed)) return;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return;
  if (hipEventRecord(a, st) != hipSuccess) return;
  ev_[0] = a;
  ev_[1] = b;
}

LaunchTimer::~LaunchTimer() {
  if (!ev_[0]) return;
  hipEvent_t a = (hipEvent_t)ev_[0], b = (hipEvent_t)ev_[1];
  if (hipEventRecord(b, st_) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back({label_, a, b});
}

}  // namespace dora

using namespace dora;

extern "C" {

DORA_API size_t dora_workspace_bytes(const dora_shape* shape, int op) {
  if (!shape || (shape->dtype != DORA_F32 && shape->dtype != DORA_BF16) || !shape_ok(*shape))
    return 0;
  if (op < DORA_OP_NORM || op > DORA_OP_VERA_GRADS) return 0;
  return layout(*shape, op).total;
}

DORA_API int dora_norm(const dora_shape* shape, const void* W0, const void* A, const void* B,
                       float* norm_out, void* ws, size_t ws_bytes, void* hip_stream) {
  DORA_CHECK(check_common(shape, DORA_OP_NORM, ws, ws_bytes));
  const dora_shape& s = *shape;
  DORA_CHECK(check_ptr(W0, false));
  DORA_CHECK(check_ptr(A, s.r == 0));
  DORA_CHECK(check_ptr(B, s.r == 0));
  DORA_CHECK(check_ptr(norm_out, false));
  const Layout L = layout(s, DORA_OP_NORM);
  return run_norm(s, W0, A, B, norm_out, ws, L, reinterpret_cast<hipStream_t>(hip_stream));
}

DORA_API int dora_forward(const dora_shape* shape, const void* x, const void* W0, const void* A,
                          const void* B, const void* m, void* y, float* norm_out, void* xs_out,
                          void* ws, size_t ws_bytes, void* hip_stream) {
  return forward_impl(shape, x, W0, A, B, m, y, norm_out, xs_out, ws, ws_bytes, hip_stream, true);
}

}  // extern "C"

namespace dora {

int forward_impl(const dora_shape* shape, const void* x, const void* W0, const void* A,
                 const void* B, const void* m, void* y, float* norm_out, void* xs_out, void* ws,
                 size_t ws_bytes, void* hip_stream, bool allow_side_stream) {
  DORA_CHECK(check_common(shape, DORA_OP_FORWARD, ws, ws_bytes));
  const dora_shape& s = *shape;
  const bool noT = s.tokens == 0;
  DORA_CHECK(check_ptr(x, noT));
  DORA_CHECK(check_ptr(W0, false));
  DORA_CHECK(check_ptr(A, s.r == 0));
  DORA_CHECK(check_ptr(B, s.r == 0));
  DORA_CHECK(check_ptr(m, false));
  DORA_CHECK(check_ptr(y, noT));
  DORA_CHECK(check_ptr(norm_out, false));
  DORA_CHECK(check_ptr(xs_out, true));
  const Layout L = layout(s, DORA_OP_FORWARD);
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const int dt = s.dtype;
  void* xs = xs_out ? xs_out : at(ws, L.xs);

  if (small_path(s)) {
    HIP_TRY(small_forward(reinterpret_cast<const float*>(x), reinterpret_cast<const float*>(W0),
                          reinterpret_cast<const float*>(A), reinterpret_cast<const float*>(B),
                          reinterpret_cast<const float*>(m), s.s, reinterpret_cast<float*>(y),
                          norm_out, reinterpret_cast<float*>(xs),
                          reinterpret_cast<float*>(at(ws, L.spart)), s.tokens, s.d_out, s.d_in,
                          s.r, st));
    return DORA_OK;
  }

  // xs = s (x A^T): the down-projection, pre-scaled by s.  It does not depend
  // on the norm (and uses other workspace regions), so on large layers it runs
  // on a side stream beside the norm's chain and joins before the forward GEMM.
  // Layers whose forward GEMM is under 128 GFLOP keep it on the caller's stream
  // after the norm: there the fork and join cost more than the overlap gains.
  const double fwd_flop = 2.0 * (double)s.tokens * (double)s.d_out * (double)(s.d_in + s.r);
  SideStream* side =
      (allow_side_stream && !noT && s.r > 0 && fwd_flop >= 128e9) ? side_stream() : nullptr;
  auto down_proj = [&](hipStream_t on) -> int {
    GemmProblem d;
    d.M = s.tokens;
    d.N = s.r;
    d.nseg = 1;
    d.seg[0] = {x, A, s.d_in, s.d_in, s.d_in};
    d.alpha = s.s;
    d.c = xs;
    d.ldc = s.r;
    give_scratch(d, ws, L);
    HIP_TRY(gemm(d, dt, on, "down_proj_xs"));
    return DORA_OK;
  };
  SideFork fk(side, st);
  if (side) {
    HIP_TRY(fk.fork());
    DORA_CHECK(down_proj(fk.side()));
  }
  DORA_CHECK(run_norm(s, W0, A, B, norm_out, ws, L, st));
  HIP_TRY(fk.join());
  if (noT) return DORA_OK;
  if (!side && s.r > 0) DORA_CHECK(down_proj(st));

  if (s.flags & DORA_FLAG_SEPARATE_COMPOSE) {
    // base = x W0^T into y; slora = xs B^T; then the one-pass compose.
    GemmProblem b;
    b.M = s.tokens;
    b.N = s.d_out;
    b.nseg = 1;
    b.seg[0] = {x, W0, s.d_in, s.d_in, s.d_in};
    b.c = y;
    b.ldc = s.d_out;
    give_scratch(b, ws, L);
    HIP_TRY(gemm(b, dt, st, "base_gemm"));
    void* slora = at(ws, L.slora);
    GemmProblem u;
    u.M = s.tokens;
    u.N = s.d_out;
    u.nseg = 1;
    u.seg[0] = {xs, B, s.r, s.r, s.r};
    u.c = slora;
    u.ldc = s.d_out;
    give_scratch(u, ws, L);
    HIP_TRY(gemm(u, dt, st, "up_proj_lora"));
    HIP_TRY(compose_fwd(y, slora, m, norm_out, s.tokens, s.d_out, dt, st));
    return DORA_OK;
  }

  // Fused: z = [x | xs] [W0 | B]^T accumulated in one pass, y = z + (g-1) z.
  GemmProblem f;
  f.M = s.tokens;
  f.N = s.d_out;
  f.seg[0] = {x, W0, s.d_in, s.d_in, s.d_in};
  f.seg[1] = {xs, B, s.r, s.r, s.r};
  f.nseg = 2;
  f.c = y;
  f.ldc = s.d_out;
  f.epi = kEpiCompose;
  f.mag = m;
  f.norm = norm_out;
  give_scratch(f, ws, L);
  HIP_TRY(gemm(f, dt, st, "fused_fwd_gemm"));
  return DORA_OK;
}

}  // namespace dora

extern "C" {

DORA_API int dora_backward(const dora_shape* shape, const void* grad_y, const void* x,
                           const void* W0, const void* A, const void* B, const void* m,
                           const float* norm, const void* xs, const void* y, void* grad_x,
                           void* grad_A, void* grad_B, float* grad_m, void* ws, size_t ws_bytes,
                           void* hip_stream) {
  DORA_CHECK(check_common(shape, DORA_OP_BACKWARD, ws, ws_bytes));
  const dora_shape& s = *shape;
  const bool noT = s.tokens == 0;
  DORA_CHECK(check_ptr(grad_y, noT));
  DORA_CHECK(check_ptr(x, noT));
  DORA_CHECK(check_ptr(W0, false));
  DORA_CHECK(check_ptr(A, s.r == 0));
  DORA_CHECK(check_ptr(B, s.r == 0));
  DORA_CHECK(check_ptr(m, false));
  DORA_CHECK(check_ptr(norm, false));
  DORA_CHECK(check_ptr(xs, true));
  DORA_CHECK(check_ptr(y, noT));
  DORA_CHECK(check_ptr(grad_x, true));
  DORA_CHECK(check_ptr(grad_A, true));
  DORA_CHECK(check_ptr(grad_B, true));
  DORA_CHECK(check_ptr(grad_m, true));
  const Layout L = layout(s, DORA_OP_BACKWARD);
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const int dt = s.dtype;
  const bool has_r = s.r > 0;
  // Undetached norm (DoRA reading notes, Appendix A.1): only A and B see it.
  const bool exact = (s.flags & DORA_FLAG_EXACT_NORM_GRAD) && has_r && (grad_A || grad_B);

  // gz = g * gy (for dx and dB) and the dm partial sums; ts = s (gz B) is
  // formed as gy Bg with Bg = s diag(g) B (stored transposed, so both operands
  // are K-contiguous), from the incoming gradient alone.
  void* gz = at(ws, L.gz);
  float* dmpart = reinterpret_cast<float*>(at(ws, L.dmpart));
  const bool need_gz = (grad_x && !noT) || (has_r && grad_B);
  const bool need_ts = has_r && !noT && (grad_x || grad_A);
  float* kappa = nullptr;   // A.1: k' and Q (set below when the norm is undetached)
  float* q = nullptr;
  float* dm = grad_m ? grad_m : (exact ? reinterpret_cast<float*>(at(ws, L.dm)) : nullptr);
  void* ts = at(ws, L.ts);
  auto t_proj = [&](hipStream_t on, bool second_scratch) -> int {
    void* bgt = at(ws, L.bg);   // (s diag(g) B)^T, [r, d_out]
    HIP_TRY(scale_b_rows_t(B, m, norm, s.s, bgt, s.d_out, s.r, dt, on));
    GemmProblem t;
    t.M = s.tokens;
    t.N = s.r;
    t.nseg = 1;
    t.seg[0] = {grad_y, bgt, s.d_out, s.d_out, s.d_out};
    t.c = ts;
    t.ldc = s.r;
    if (second_scratch)
      give_scratch2(t, ws, L);
    else
      give_scratch(t, ws, L);
    HIP_TRY(gemm(t, dt, on, "t_proj"));
    return DORA_OK;
  };
  auto grad_b = [&](const void* xsu) -> int {
    GemmProblem b;
    b.M = s.d_out;
    b.N = s.r;
    b.nseg = 1;
    b.seg[0] = {gz, xsu, s.d_out, s.r, s.tokens};
    b.a_kcontig = false;
    b.b_kcontig = false;
    b.c = grad_B;
    b.ldc = s.r;
    give_scratch(b, ws, L);
    if (exact) {   // float32 partial sums, combined with diag(k') Q in one rounding
      float* d1 = reinterpret_cast<float*>(at(ws, L.d1));
      b.c = d1;
      b.out_f32 = true;
      b.split = L.d1splits;
      b.split_stride = s.d_out * s.r;
      HIP_TRY(gemm(b, dt, st, "dB_gemm"));
      HIP_TRY(db_combine(d1, L.d1splits, q, L.qsplits, kappa, grad_B, s.d_out, s.r, dt, st));
    } else {
      HIP_TRY(gemm(b, dt, st, "dB_gemm"));
    }
    return DORA_OK;
  };
  void* bk = nullptr;     // A.1: Bk' and H' (set below when the norm is undetached)
  void* hmat = nullptr;
  auto grad_a = [&]() -> int {
    GemmProblem a;
    a.M = s.r;
    a.N = s.d_in;
    a.nseg = 1;
    a.seg[0] = {ts, x, s.r, s.d_in, s.tokens};
    if (exact) {   // [ts^T | Bk'^T | H'] [x ; W0 ; A]  (H' is symmetric)
      a.seg[1] = {bk, W0, s.r, s.d_in, s.d_out};
      a.seg[2] = {hmat, A, s.r, s.d_in, s.r};
      a.nseg = 3;
    }
    a.a_kcontig = false;
    a.b_kcontig = false;
    a.c = grad_A;
    a.ldc = s.d_in;
    give_scratch(a, ws, L);
    HIP_TRY(gemm(a, dt, st, "dA_gemm"));
    return DORA_OK;
  };
  // columns with m_i == 0 take dm from its definition (y / m = z / n fails there)
  const DmRecompute zr{norm, grad_y, x, W0, A, B, s.s, s.tokens, s.d_in, s.r};

  // With the norm detached, ts and then dm's finisher run on the side stream
  // beside the compose backward and dB (which need only gz and xs); dx waits
  // for all of them.  dA follows dx on the caller's stream: dx fills the chip in
  // whole rounds of workgroups, and anything beside it only delays its second
  // round.  Layers whose dx is under 128 GFLOP stay on the caller's stream: there
  // the fork and join cost more than the overlap gains.
  const double dx_flop = 2.0 * (double)s.tokens * (double)s.d_in * (double)(s.d_out + s.r);
  SideStream* side = (!exact && need_ts && dx_flop >= 128e9) ? side_stream() : nullptr;
  SideFork fk(side, st);
  if (side) {
    HIP_TRY(fk.fork());
    DORA_CHECK(t_proj(fk.side(), true));
  }
  if (need_gz || dm)
    HIP_TRY(compose_bwd(grad_y, y, m, norm, gz, dmpart, s.tokens, s.d_out, kTokPerDmBlock, dt, st));
  // dm and dB need only the compose backward's outputs (and the caller's xs),
  // so they run before the join: dm's finisher on the side stream after ts
  // (a second fork makes it wait for the compose backward), dB on the caller's.
  if (dm && side) {
    HIP_TRY(fk.fork());
    HIP_TRY(dm_finalize(dmpart, L.dm_blocks, m, dm, s.d_out, zr, dt, fk.side()));
  } else if (dm) {
    HIP_TRY(dm_finalize(dmpart, L.dm_blocks, m, dm, s.d_out, zr, dt, st));
  }
  bool db_done = false;
  if (side && grad_B && has_r && xs && !noT) {
    DORA_CHECK(grad_b(xs));
    db_done = true;
  }
  HIP_TRY(fk.join());   // dx below needs ts

  // A.1 terms: k' = -s m dm / n^2, Bk' = diag(k') B, Q = W0 A^T + s B G,
  // H' = s Bk'^T B.  Then dB += diag(k') Q and dA += Bk'^T W0 + H' A.
  if (exact) {
    kappa = reinterpret_cast<float*>(at(ws, L.kappa));
    bk = at(ws, L.bk);
    HIP_TRY(exact_prep(m, norm, dm, B, s.s, kappa, bk, s.d_out, s.r, dt, st));
    float* gpart = reinterpret_cast<float*>(at(ws, L.egpart));
    void* ghi = at(ws, L.eghi);
    void* glo = at(ws, L.eglo);
    GemmProblem g;
    g.M = g.N = s.r;
    g.nseg = 1;
    g.seg[0] = {A, A, s.d_in, s.d_in, s.d_in};
    g.c = gpart;
    g.ldc = s.r;
    g.out_f32 = true;
    g.split = L.splits;
    g.split_stride = s.r * s.r;
    HIP_TRY(gemm(g, dt, st, "gram_AAt"));
    HIP_TRY(gram_finalize(gpart, L.splits, s.r, s.s, dt, ghi, glo, st, "gram_finalize"));
    q = reinterpret_cast<float*>(at(ws, L.q));
    GemmProblem pq;
    pq.M = s.d_out;
    pq.N = s.r;
    pq.seg[0] = {W0, A, s.d_in, s.d_in, s.d_in};
    pq.seg[1] = {B, ghi, s.r, s.r, s.r};
    pq.nseg = 2;
    if (dt == kBF16) {
      pq.seg[2] = {B, glo, s.r, s.r, s.r};
      pq.nseg = 3;
    }
    pq.c = q;
    pq.ldc = s.r;
    pq.out_f32 = true;
    pq.split = L.qsplits;
    pq.split_stride = s.d_out * s.r;
    HIP_TRY(gemm(pq, dt, st, "exact_q_proj"));
    if (grad_A) {
      float* hpart = reinterpret_cast<float*>(at(ws, L.hpart));
      hmat = at(ws, L.hmat);
      GemmProblem h;
      h.M = h.N = s.r;
      h.nseg = 1;
      h.seg[0] = {bk, B, s.r, s.r, s.d_out};
      h.a_kcontig = false;
      h.b_kcontig = false;
      h.alpha = s.s;
      h.c = hpart;
      h.ldc = s.r;
      h.out_f32 = true;
      h.split = L.hsplits;
      h.split_stride = s.r * s.r;
      HIP_TRY(gemm(h, dt, st, "exact_h_gram"));
      HIP_TRY(gram_finalize(hpart, L.hsplits, s.r, 1.f, dt, hmat, at(ws, L.hlo), st,
                            "exact_h_finalize"));
    }
  }

  if (!side && need_ts) DORA_CHECK(t_proj(st, false));

  if (grad_x && !noT) {
    GemmProblem d;
    d.M = s.tokens;
    d.N = s.d_in;
    d.seg[0] = {gz, W0, s.d_out, s.d_in, s.d_out};
    d.seg[1] = {ts, A, s.r, s.d_in, s.r};
    d.nseg = has_r ? 2 : 1;
    d.b_kcontig = false;
    d.c = grad_x;
    d.ldc = s.d_in;
    give_scratch(d, ws, L);
    HIP_TRY(gemm(d, dt, st, "dx_gemm"));
  }

  if (grad_B && has_r && !db_done) {
    const void* xsu = xs;
    if (!xsu && !noT) {
      void* xw = at(ws, L.xs);
      GemmProblem d;
      d.M = s.tokens;
      d.N = s.r;
      d.nseg = 1;
      d.seg[0] = {x, A, s.d_in, s.d_in, s.d_in};
      d.alpha = s.s;
      d.c = xw;
      d.ldc = s.r;
      give_scratch(d, ws, L);
      HIP_TRY(gemm(d, dt, st, "down_proj_xs"));
      xsu = xw;
    }
    DORA_CHECK(grad_b(xsu));
  }

  if (grad_A && has_r) DORA_CHECK(grad_a());
  HIP_TRY(fk.join());
  return DORA_OK;
}

DORA_API int dora_merge(const dora_shape* shape, const void* W0, const void* A, const void* B,
                        const void* m, const float* norm, void* W_out, void* ws, size_t ws_bytes,
                        void* hip_stream) {
  DORA_CHECK(check_common(shape, DORA_OP_MERGE, ws, ws_bytes));
  const dora_shape& s = *shape;
  DORA_CHECK(check_ptr(W0, false));
  DORA_CHECK(check_ptr(A, s.r == 0));
  DORA_CHECK(check_ptr(B, s.r == 0));
  DORA_CHECK(check_ptr(m, false));
  DORA_CHECK(check_ptr(norm, true));
  DORA_CHECK(check_ptr(W_out, false));
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const Layout L = layout(s, DORA_OP_MERGE);
  const int dt = s.dtype;
  const float* n = norm;
  if (!n) {
    float* nn = reinterpret_cast<float*>(at(ws, L.mnorm));
    DORA_CHECK(run_norm(s, W0, A, B, nn, ws, L, st));
    n = nn;
  }
  // W_out = g (W0 + s B A): C[d_out, d_in] over K = r, A operand B (K-contiguous),
  // B operand A read transposed (element (n, k) at A[k, n])
  GemmProblem g;
  g.M = s.d_out;
  g.N = s.d_in;
  g.nseg = 1;
  g.seg[0] = {B, A, s.r, s.d_in, s.r};
  g.a_kcontig = true;
  g.b_kcontig = false;
  g.c = W_out;
  g.ldc = s.d_in;
  g.alpha = s.s;
  g.epi = kEpiMerge;
  g.mag = m;
  g.norm = n;
  g.add = W0;
  g.ld_add = s.d_in;
  HIP_TRY(gemm(g, dt, st, "merge_gemm"));
  return DORA_OK;
}

DORA_API int dora_vera_scale(const dora_shape* shape, const void* B_shared, const void* b,
                             const void* d, void* B_eff, void* hip_stream) {
  DORA_CHECK(check_common(shape, kOpNoWorkspace, nullptr, 0));
  const dora_shape& s = *shape;
  const bool empty = s.r == 0;
  DORA_CHECK(check_ptr(B_shared, empty));
  DORA_CHECK(check_ptr(b, false));
  DORA_CHECK(check_ptr(d, empty));
  DORA_CHECK(check_ptr(B_eff, empty));
  HIP_TRY(vera_scale(B_shared, b, d, B_eff, s.d_out, s.r, s.dtype,
                     reinterpret_cast<hipStream_t>(hip_stream)));
  return DORA_OK;
}

DORA_API int dora_vera_grads(const dora_shape* shape, const void* grad_B_eff,
                             const void* B_shared, const void* b, const void* d, void* grad_b,
                             void* grad_d, void* ws, size_t ws_bytes, void* hip_stream) {
  DORA_CHECK(check_common(shape, DORA_OP_VERA_GRADS, ws, ws_bytes));
  const dora_shape& s = *shape;
  const bool empty = s.r == 0;
  DORA_CHECK(check_ptr(grad_B_eff, empty));
  DORA_CHECK(check_ptr(B_shared, empty));
  DORA_CHECK(check_ptr(b, false));
  DORA_CHECK(check_ptr(d, empty));
  DORA_CHECK(check_ptr(grad_b, true));
  DORA_CHECK(check_ptr(grad_d, true));
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  // with r == 0 every grad_b_i is an empty sum (written as 0) and grad_d is empty
  const Layout L = layout(s, DORA_OP_VERA_GRADS);
  HIP_TRY(vera_grads(grad_B_eff, B_shared, b, d, grad_b, grad_d,
                     reinterpret_cast<float*>(at(ws, L.vpart)), s.d_out, s.r, s.dtype, st));
  return DORA_OK;
}

DORA_API const char* dora_strerror(int code) {
  switch (code) {
    case DORA_OK: return "ok";
    case DORA_ERR_NULL: return "a required pointer is NULL";
    case DORA_ERR_SHAPE: return "invalid shape (dims out of range or not multiples of 8)";
    case DORA_ERR_DTYPE: return "unsupported dtype";
    case DORA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case DORA_ERR_WORKSPACE: return "workspace too small";
    case DORA_ERR_HIP: return "HIP runtime error";
    case DORA_ERR_FLAGS: return "unsupported flags, nonzero reserved field or non-finite s";
    default: return "unknown error code";
  }
}

DORA_API int dora_timing_enable(int enable) {
  g_timing.store(enable ? 1 : 0);
  return DORA_OK;
}

DORA_API int dora_timing_collect(char* buf, size_t buflen) {
  std::vector<Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    recs.swap(g_recs);
  }
  std::map<std::string, std::pair<long, double>> agg;
  int rc = 0;
  for (const Rec& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      rc = DORA_ERR_HIP;
    auto& e = agg[r.label];
    e.first += 1;
    e.second += ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Rec& r : recs) {
      g_pool.push_back(r.a);
      g_pool.push_back(r.b);
    }
  }
  std::string out = "{";
  bool first = true;
  for (const auto& kv : agg) {
    char tmp[256];
    std::snprintf(tmp, sizeof tmp, "%s\"%s\": [%ld, %.6f]", first ? "" : ", ", kv.first.c_str(),
                  kv.second.first, kv.second.second);
    out += tmp;
    first = false;
  }
  out += "}";
  if (buf && buflen) {
    std::strncpy(buf, out.c_str(), buflen - 1);
    buf[buflen - 1] = '\0';
  }
  return rc ? rc : (int)recs.size();
}

}  // extern "C"
