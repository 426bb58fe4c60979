// C-ABI entry points: host validation, workspace sizing, path selection and
// launches.  No host synchronization and no allocation on any compute path.

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "lora_internal.hpp"

using namespace lora;

namespace {

// Tuning knobs (overridable through the environment for sweeps).
struct Tune {
  int valu_items = 1024;  // aim for about this many VALU work items per launch
  int valu_max_chunks = 8;
  int mfma_items = 256;   // aim for about this many MFMA work items per launch
  int grid_cap = 4096;    // workgroups per launch; the kernels grid-stride over items (2048: the stack 1.7% slower)
  int mfma_half = -1;     // MFMA half-size stages: -1 when they let two workgroups share a CU, 0 never, 1 always
  int mfma_stacked = 1;   // fused launches with 2 .. 4 slots per request: x walked once per stacked tile (0: per slot)
  int mfma_contig = 1;    // MFMA tiles of equal cost dealt to the XCDs in contiguous ranges (0: blocks round-robin)
  int mfma_xonce = 1;     // sliced launches (2 .. 4 slices, one slot per request): x walked once per tile (0: per slice)
};

int env_int(const char *name, int dflt) {
  const char *s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

const Tune &tune() {
  static const Tune t = [] {
    Tune x;
    x.valu_items = env_int("LORA_VALU_ITEMS", x.valu_items);
    x.valu_max_chunks = env_int("LORA_VALU_MAX_CHUNKS", x.valu_max_chunks);
    x.mfma_items = env_int("LORA_MFMA_ITEMS", x.mfma_items);
    x.grid_cap = env_int("LORA_GRID_CAP", x.grid_cap);
    x.mfma_half = env_int("LORA_MFMA_HALF", x.mfma_half);
    x.mfma_stacked = env_int("LORA_MFMA_STACKED", x.mfma_stacked);
    x.mfma_contig = env_int("LORA_MFMA_CONTIG", x.mfma_contig);
    x.mfma_xonce = env_int("LORA_MFMA_XONCE", x.mfma_xonce);
    return x;
  }();
  return t;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(lora_dtype d) { return d == LORA_BF16 ? 2 : 4; }

struct BatchDims {
  int T, S, K, per_token;
};

lora_status check_batch(const lora_batch *b, BatchDims &d) {
  if (!b) return LORA_EINVAL;
  if (b->n_tokens < 0) return LORA_ESHAPE;
  if (b->max_slots < 1) return LORA_ESHAPE;
  if (b->max_slots > LORA_MAX_SLOTS) return LORA_EUNSUPPORTED;
  d.T = b->n_tokens;
  d.K = b->max_slots;
  d.per_token = b->seg_off == nullptr;
  d.S = d.per_token ? d.T : b->n_segments;
  if (d.S < 0) return LORA_ESHAPE;
  if (d.S > 0 && !b->idx) return LORA_EINVAL;
  if ((int64_t)d.S * d.K > INT32_MAX / 2) return LORA_EUNSUPPORTED;
  return LORA_OK;
}

lora_status check_shape(const lora_pool *p) {
  if (!p) return LORA_EINVAL;
  if (p->dtype != LORA_F32 && p->dtype != LORA_BF16) return LORA_EINVAL;
  if (p->n_adapters < 1 || p->rank < 1 || p->d_in < 1 || p->d_out < 1) return LORA_ESHAPE;
  if (p->rank > LORA_MAX_RANK) return LORA_EUNSUPPORTED;
  return LORA_OK;
}

lora_status check_pool(const lora_pool *p) {
  lora_status st = check_shape(p);
  if (st) return st;
  if (!p->A || !p->B) return LORA_EINVAL;
  return LORA_OK;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
  return na && nb && x < y + nb && y < x + na;
}

size_t span_bytes(int rows, int64_t ld, int cols, int eb) {
  if (rows <= 0) return 0;
  return (size_t(rows - 1) * size_t(ld) + size_t(cols)) * size_t(eb);
}

struct Plan {
  PlanLayout L;
  PlanView V;
};

lora_status plan_for(const BatchDims &d, int n, const void *ws, size_t ws_bytes, Plan &P) {
  P.L = plan_layout(d.S, d.T, n);
  if (!ws) return LORA_EWORKSPACE;
  if (ws_bytes < P.L.total) return LORA_EWORKSPACE;
  if (!aligned16(ws)) return LORA_EINVAL;
  P.V = plan_view(const_cast<void *>(ws), P.L, d.K, d.per_token);
  return LORA_OK;
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Compute units of the current device (looked up once per device).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    cached[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cached[dev];
}
int pow2_floor(int x) {
  int p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

// Choose the launches: vector path, MFMA eligibility, chunking, grids and LDS.
struct Launch {
  bool vec;
  int jt;           // rank / 16 when the MFMA kernel runs, else 0
  bool half;        // MFMA kernel with half-size stages
  int smax;         // MFMA kernel's stacked-tile build (2, 3 or 4 slots), or 1
  int nsl;          // MFMA kernel walking x once for the nsl slices of a group (sliced launches), or 0
  int grid_v, grid_m;
  size_t smem_v, smem_m;
};

// n_groups groups of ns slices; slice p writes d_outs[p] columns (plain calls:
// one slice of the shape's d_out).
Launch configure(int mode, const lora_pool *shape, const BatchDims &d, const Plan &P, int n_groups, int ns,
                 const int32_t *d_outs, bool vec, ApplyArgs &a) {
  const Tune &tn = tune();
  const int r = shape->rank;
  int d_sum = 0;
  for (int p = 0; p < ns; ++p) d_sum += d_outs[p];
  Launch L;
  L.vec = vec;
  const bool mfma = vec && shape->dtype == LORA_BF16 && (r == 16 || r == 32 || r == 64 || r == 128) &&
                    d.K * r <= kMfmaMaxSlotRank && d.T >= kMfmaMinBatch;
  L.jt = mfma ? r / 16 : 0;
  a.valu_takes_m = mfma ? 0 : 1;

  // output-column chunks: more chunks per tile when there are few tiles; the
  // chunk width is chosen over all slices' columns and each slice is cut
  // into chunks of that width
  const int est_v = std::max(1, std::min(d.S, shape->n_adapters)) * n_groups;
  const int est_m = std::max(1, (d.T + kMfmaRows - 1) / kMfmaRows) * n_groups;
  int cv = 1, cm = 1;
  if (mode != MODE_SHRINK) {
    cv = std::min(pow2_floor(std::max(1, tn.valu_items / est_v)), tn.valu_max_chunks);
    cv = std::max(1, std::min(cv, std::max(1, d_sum / 256)));
    cm = pow2_floor(std::max(1, tn.mfma_items / est_m));
    cm = std::max(1, std::min(cm, std::max(1, d_sum / 512)));
  }
  const int wv = mode == MODE_SHRINK ? round_up(d_sum, 128) : round_up((d_sum + cv - 1) / cv, 64);
  const int wm = mode == MODE_SHRINK ? round_up(d_sum, 128) : round_up((d_sum + cm - 1) / cm, 128);
  a.ns = ns;
  a.cvo[0] = a.cmo[0] = 0;
  for (int p = 0; p < ns; ++p) {
    a.sd_out[p] = d_outs[p];
    a.wv[p] = wv;
    a.wm[p] = wm;
    a.cv[p] = (d_outs[p] + wv - 1) / wv;
    a.cm[p] = (d_outs[p] + wm - 1) / wm;
    a.cvo[p + 1] = a.cvo[p] + a.cv[p];
    a.cmo[p + 1] = a.cmo[p] + a.cm[p];
  }
  a.items_v_tile = a.cvo[ns];
  a.items_m_tile = a.cmo[ns];

  const int64_t items_m = (int64_t)n_groups * std::max(P.L.bound_m, P.L.bound_ms) * a.cmo[ns];
  // the VALU kernel takes an MFMA-sized tile as one item per row block
  const int64_t items_mv = (int64_t)n_groups * P.L.bound_m * a.cmo[ns] * (kMfmaRows / kRowBlock);
  // VALU tiles come only from adapter groups of fewer than kMfmaMinRows rows
  // (at most four tiles each), and a batch has at most one group per request
  // (per adapter too with one slot per request): a batch of long requests
  // gets a small VALU grid instead of one sized by its rows
  const int64_t groups_max = d.K == 1 ? std::min(d.S, shape->n_adapters) : d.S;
  const int64_t tiles_v =
      std::min<int64_t>(P.L.bound_v, (kMfmaMinRows - 2 + kValuRows) / kValuRows * std::max<int64_t>(groups_max, 1));
  const int64_t items_v = (int64_t)n_groups * (tiles_v * a.cvo[ns]) + (a.valu_takes_m ? items_mv : 0);
  L.grid_v = round_up((int)std::max<int64_t>(std::min<int64_t>(items_v, tn.grid_cap), 1), 8);
  L.grid_m = mfma ? round_up((int)std::max<int64_t>(std::min<int64_t>(items_m, tn.grid_cap), 1), 8) : 0;
  L.smem_v = valu_smem_bytes(a.kr_max);
  // Two MFMA workgroups per CU when they fit in LDS: with many stacked slots
  // (each parks a 64-row intermediate) the half-size stages make them fit.
  L.half = false;
  L.smem_m = mfma ? mfma_smem_bytes(L.jt, d.K, false) : 0;
  const bool want_half = tn.mfma_half < 0 ? (L.smem_m > kMaxLdsBytes / 2 &&
                                              mfma_smem_bytes(L.jt, d.K, true) <= kMaxLdsBytes / 2)
                                           : tn.mfma_half > 0;
  if (mfma && want_half && mfma_half_available(L.jt)) {
    L.half = true;
    L.smem_m = mfma_smem_bytes(L.jt, d.K, true);
  }
  // requests that stack 2 .. 4 adapters: their tiles walk x once for all slots
  // (single-slice launches; a sliced launch keeps one pass per slot)
  L.smax = 1;
  if (mfma && tn.mfma_stacked && mode == MODE_FUSED && ns == 1 && d.K >= 2 && d.K <= 4) {
    L.smax = d.K;  // builds for 2, 3 and 4 slots
    L.half = false;
    L.smem_m = mfma_stacked_smem_bytes(L.jt, L.smax);
  }
  // Sliced launches with one slot per request: one item per row tile for all
  // 2 .. 4 slices of a group, which walks x once for every slice (the tile
  // then covers each slice's whole width: no output chunks).  Taken when the
  // slices' outputs are narrow next to x (q / k / v: the same time as one item
  // per slice, without the slices' re-reads of x); with wide outputs (gate /
  // up) the longer items balance worse over the CUs, 7% slower on the
  // Llama-3-8B-shaped stack.
  L.nsl = 0;
  if (mfma && tn.mfma_xonce && mode == MODE_FUSED && ns >= 2 && ns <= 4 && d.K == 1 &&
      (int64_t)d_sum <= 2 * (int64_t)shape->d_in) {
    L.nsl = ns;
    L.half = false;
    L.smem_m = mfma_stacked_smem_bytes(L.jt, ns);
    const int64_t tiles_m = (int64_t)n_groups * std::max(P.L.bound_m, P.L.bound_ms);
    L.grid_m = round_up((int)std::max<int64_t>(std::min<int64_t>(tiles_m, tn.grid_cap), 1), 8);
  }
  // One slot per request and one rank: every MFMA tile costs about the same,
  // and a launch over many problems deals each XCD whole problems, whose
  // adapters then sit in that XCD's L2 only.  (A single problem keeps the
  // round-robin blocks: a 17k-row, 32-request prefill batch on a 4096-wide
  // rank-64 layer fetched 16% less with contiguous ranges but ran
  // 1.4% slower, its tiles being bound by one round trip per stage.)
  a.mfma_uniform = tn.mfma_contig && n_groups > 1 && d.K == 1 && shape->ranks == nullptr ? 1 : 0;
  // what the MFMA kernel needs to choose between the plan's two tilings
  a.n_cu = cu_count();
  const int per_cu = L.smem_m ? (int)std::min<size_t>(2, std::max<size_t>(1, kMaxLdsBytes / L.smem_m)) : 2;
  a.mfma_slots = a.n_cu * per_cu;
  return L;
}

// A second stream and two events per device, created at the first
// multi-problem launch that runs both kernels on that device.  The fork and
// join are serialised per device (the events are shared).
struct Fork {
  std::mutex m;
  std::once_flag once;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool ok = false;
};
Fork *fork_for(hipStream_t stream) {
  static Fork forks[64];
  hipDevice_t dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  Fork &f = forks[dev];
  std::call_once(f.once, [&] {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess || hipSetDevice(dev) != hipSuccess) return;
    f.ok = hipStreamCreateWithFlags(&f.s, hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&f.e0, hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&f.e1, hipEventDisableTiming) == hipSuccess;
    (void)hipSetDevice(cur);
  });
  return f.ok ? &f : nullptr;
}

hipError_t launch_mfma_any(int mode, const Launch &L, const ApplyArgs &a, hipStream_t stream) {
  return L.nsl > 0    ? launch_mfma_sliced(L.jt, L.nsl, a, L.grid_m, L.smem_m, stream)
         : L.smax > 1 ? launch_mfma_stacked(L.jt, L.smax, a, L.grid_m, L.smem_m, stream)
                      : launch_mfma(mode, L.jt, L.half, a, L.grid_m, L.smem_m, stream);
}

// MFMA tiles (the long groups) first, then the VALU tiles.  A launch over
// several problems whose batch can have both kinds of tiles (the Llama-3-8B
// stack's mixed prefill and decode batch) runs the VALU kernel on the
// device's second stream, concurrently with the MFMA kernel: the two write
// disjoint rows of y and only read the plan, and each fills the other's ramp
// and drain (the stack's step measured 6-8% faster).  The caller's stream
// waits for both.  Single-problem launches keep one stream: there the fork
// and join cost more than they save (a 17k-row prefill batch of 32 requests
// on one 4096-wide rank-64 layer: 142 against 152 us).
hipError_t launch_all(int mode, int dtype, const Launch &L, const ApplyArgs &a, hipStream_t stream) {
  if (L.jt > 0 && a.n_problems > 1 && mode == MODE_FUSED) {
    if (Fork *f = fork_for(stream)) {
      std::lock_guard<std::mutex> g(f->m);
      if (hipEventRecord(f->e0, stream) != hipSuccess || hipStreamWaitEvent(f->s, f->e0, 0) != hipSuccess)
        return hipErrorUnknown;
      hipError_t e = launch_valu(mode, dtype, L.vec, a, L.grid_v, L.smem_v, f->s);
      if (e != hipSuccess) return e;
      if (hipEventRecord(f->e1, f->s) != hipSuccess) return hipErrorUnknown;
      e = launch_mfma_any(mode, L, a, stream);
      if (hipStreamWaitEvent(stream, f->e1, 0) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
      return e;
    }
  }
  if (L.jt > 0) {
    const hipError_t e = launch_mfma_any(mode, L, a, stream);
    if (e != hipSuccess) return e;
  }
  return launch_valu(mode, dtype, L.vec, a, L.grid_v, L.smem_v, stream);
}

void fill_common(ApplyArgs &a, const lora_batch *b, const BatchDims &d, const Plan &P, const lora_pool *shape) {
  std::memset(&a, 0, sizeof(a));
  a.seg_off = b->seg_off;
  a.idx = b->idx;
  a.scale = b->scale;
  a.K = d.K;
  a.T = d.T;
  a.S = d.S;
  a.hdr = P.V.hdr;
  a.sseg = P.V.sseg;
  a.sst = P.V.sst;
  a.cumlen = P.V.cumlen;
  a.tiles_m = P.V.tiles_m;
  a.tiles_ms = P.V.tiles_ms;
  a.tiles_v = P.V.tiles_v;
  a.vrec = P.V.vrec;
  a.n = shape->n_adapters;
  a.r = shape->rank;
  a.ranks = shape->ranks;
  a.d_in = shape->d_in;
  a.d_out = shape->d_out;
  a.kr_max = d.K * shape->rank;
}

lora_status run(int mode, const lora_pool *pool, const lora_batch *batch, const void *ws, size_t ws_bytes,
                bool build, const void *x, int64_t ldx, void *y, int64_t ldy, float *v, int64_t ldv,
                hipStream_t stream) {
  lora_status st = check_pool(pool);
  if (st) return st;
  BatchDims d;
  if ((st = check_batch(batch, d))) return st;
  if ((int64_t)d.K * pool->rank > LORA_MAX_SLOT_RANK) return LORA_EUNSUPPORTED;
  const int eb = elem_bytes(pool->dtype);
  const bool need_x = mode != MODE_EXPAND, need_y = mode != MODE_SHRINK, need_v = mode != MODE_FUSED;
  if (d.T > 0) {
    if (need_x && !x) return LORA_EINVAL;
    if (need_y && !y) return LORA_EINVAL;
    if (need_v && !v) return LORA_EINVAL;
  }
  if (need_x && ldx < pool->d_in) return LORA_ESHAPE;
  if (need_y && ldy < pool->d_out) return LORA_ESHAPE;
  if (need_v && ldv < (int64_t)d.K * pool->rank) return LORA_ESHAPE;
  const size_t xs = need_x ? span_bytes(d.T, ldx, pool->d_in, eb) : 0;
  const size_t ys = need_y ? span_bytes(d.T, ldy, pool->d_out, eb) : 0;
  const size_t vs = need_v ? span_bytes(d.T, ldv, d.K * pool->rank, 4) : 0;
  if (overlap(x, xs, y, ys) || overlap(v, vs, x, xs) || overlap(v, vs, y, ys)) return LORA_EINVAL;
  Plan P;
  if ((st = plan_for(d, pool->n_adapters, ws, ws_bytes, P))) return st;
  if (overlap(ws, P.L.total, x, xs) || overlap(ws, P.L.total, y, ys) || overlap(ws, P.L.total, v, vs))
    return LORA_EINVAL;

  if (build) {
    if (launch_plan(P.V, P.L.lds_bytes, batch->seg_off, batch->idx, stream) != hipSuccess) return LORA_EHIP;
  }
  if (d.T == 0 || d.S == 0) return LORA_OK;

  const int E = pool->dtype == LORA_BF16 ? 8 : 4;
  bool vec = aligned16(pool->A) && aligned16(pool->B) && pool->d_in % E == 0 && pool->d_out % E == 0 &&
             pool->rank % E == 0;
  if (need_x) vec = vec && aligned16(x) && ldx % E == 0;
  if (need_y) vec = vec && aligned16(y) && ldy % E == 0;
  if (need_v) vec = vec && aligned16(v) && ldv % 4 == 0;

  ApplyArgs a;
  fill_common(a, batch, d, P, pool);
  a.single.A = pool->A;
  a.single.B = pool->B;
  a.single.x = x;
  a.single.y = y;
  a.single.ldx = ldx;
  a.single.ldy = ldy;
  a.probs = nullptr;
  a.n_problems = 1;
  a.v = v;
  a.ldv = ldv;
  const Launch L = configure(mode, pool, d, P, 1, 1, &pool->d_out, vec, a);
  if (launch_all(mode, pool->dtype, L, a, stream) != hipSuccess) return LORA_EHIP;
  return LORA_OK;
}

// Plan storage of lora_apply_noalloc: a fixed device array, one copy on every
// GPU the library runs on, held until the process ends.  In host code the
// array's name is only a host-side stand-in: kernels are given the device
// address hipGetSymbolAddress returns for the current device, looked up once
// per device and kept.
constexpr size_t kNoAllocPlanBytes = size_t(8) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocPlanBytes];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device; nullptr if it cannot
// be found.
void *scratch_address() {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int32_t lora_abi_version(void) { return 104; }

const char *lora_status_string(lora_status s) {
  switch (s) {
    case LORA_OK: return "ok";
    case LORA_EINVAL: return "invalid argument (NULL pointer, overlapping buffers or bad enum)";
    case LORA_ESHAPE: return "invalid shape (non-positive size, ld < d or bad counts)";
    case LORA_EWORKSPACE: return "workspace missing or too small";
    case LORA_EUNSUPPORTED: return "unsupported rank, slot count or size";
    case LORA_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t lora_workspace_size(const lora_batch *batch, int32_t n_adapters) {
  BatchDims d;
  if (check_batch(batch, d) != LORA_OK || n_adapters < 1) return 0;
  return plan_layout(d.S, d.T, n_adapters).total;
}

lora_status lora_plan_build(const lora_batch *batch, int32_t n_adapters, void *ws, size_t ws_bytes,
                            hipStream_t stream) {
  BatchDims d;
  lora_status st = check_batch(batch, d);
  if (st) return st;
  if (n_adapters < 1) return LORA_ESHAPE;
  Plan P;
  if ((st = plan_for(d, n_adapters, ws, ws_bytes, P))) return st;
  if (launch_plan(P.V, P.L.lds_bytes, batch->seg_off, batch->idx, stream) != hipSuccess) return LORA_EHIP;
  return LORA_OK;
}

lora_status lora_apply(const lora_pool *pool, const lora_batch *batch, const void *x, int64_t ldx, void *y,
                       int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream) {
  return run(MODE_FUSED, pool, batch, ws, ws_bytes, true, x, ldx, y, ldy, nullptr, 0, stream);
}

lora_status lora_apply_noalloc(const lora_pool *pool, const lora_batch *batch, const void *x, int64_t ldx, void *y,
                               int64_t ldy, hipStream_t stream) {
  lora_status st = check_pool(pool);
  if (st) return st;
  BatchDims d;
  if ((st = check_batch(batch, d))) return st;
  if (pool->n_adapters < 1) return LORA_ESHAPE;
  if (plan_layout(d.S, d.T, pool->n_adapters).total > kNoAllocPlanBytes) return LORA_EUNSUPPORTED;
  void *plan = scratch_address();
  if (!plan) return LORA_EHIP;
  return run(MODE_FUSED, pool, batch, plan, kNoAllocPlanBytes, true, x, ldx, y, ldy, nullptr, 0, stream);
}

lora_status lora_shrink(const lora_pool *pool, const lora_batch *batch, const void *x, int64_t ldx, float *v,
                        int64_t ldv, void *ws, size_t ws_bytes, hipStream_t stream) {
  return run(MODE_SHRINK, pool, batch, ws, ws_bytes, true, x, ldx, nullptr, 0, v, ldv, stream);
}

lora_status lora_expand(const lora_pool *pool, const lora_batch *batch, const float *v, int64_t ldv, void *y,
                        int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream) {
  return run(MODE_EXPAND, pool, batch, ws, ws_bytes, true, nullptr, 0, y, ldy, const_cast<float *>(v), ldv, stream);
}

lora_status lora_apply_planned(const lora_pool *pool, const lora_batch *batch, const void *plan, size_t plan_bytes,
                               const void *x, int64_t ldx, void *y, int64_t ldy, hipStream_t stream) {
  return run(MODE_FUSED, pool, batch, plan, plan_bytes, false, x, ldx, y, ldy, nullptr, 0, stream);
}

lora_status lora_shrink_planned(const lora_pool *pool, const lora_batch *batch, const void *plan, size_t plan_bytes,
                                const void *x, int64_t ldx, float *v, int64_t ldv, hipStream_t stream) {
  return run(MODE_SHRINK, pool, batch, plan, plan_bytes, false, x, ldx, nullptr, 0, v, ldv, stream);
}

lora_status lora_expand_planned(const lora_pool *pool, const lora_batch *batch, const void *plan, size_t plan_bytes,
                                const float *v, int64_t ldv, void *y, int64_t ldy, hipStream_t stream) {
  return run(MODE_EXPAND, pool, batch, plan, plan_bytes, false, nullptr, 0, y, ldy, const_cast<float *>(v), ldv,
             stream);
}

lora_status lora_apply_multi(const lora_pool *shape, const lora_batch *batch, const void *plan, size_t plan_bytes,
                             int32_t n_problems, const lora_problem *problems, int32_t problems_aligned,
                             hipStream_t stream) {
  lora_status st = check_shape(shape);
  if (st) return st;
  BatchDims d;
  if ((st = check_batch(batch, d))) return st;
  if ((int64_t)d.K * shape->rank > LORA_MAX_SLOT_RANK) return LORA_EUNSUPPORTED;
  if (n_problems < 0) return LORA_ESHAPE;
  if (n_problems > 0 && !problems) return LORA_EINVAL;
  if (!aligned16(problems)) return LORA_EINVAL;
  Plan P;
  if ((st = plan_for(d, shape->n_adapters, plan, plan_bytes, P))) return st;
  if (n_problems == 0 || d.T == 0 || d.S == 0) return LORA_OK;
  const int E = shape->dtype == LORA_BF16 ? 8 : 4;
  const bool vec = problems_aligned && shape->d_in % E == 0 && shape->d_out % E == 0 && shape->rank % E == 0;
  ApplyArgs a;
  fill_common(a, batch, d, P, shape);
  a.probs = problems;
  a.n_problems = n_problems;
  const Launch L = configure(MODE_FUSED, shape, d, P, n_problems, 1, &shape->d_out, vec, a);
  if (launch_all(MODE_FUSED, shape->dtype, L, a, stream) != hipSuccess) return LORA_EHIP;
  return LORA_OK;
}

lora_status lora_apply_sliced(const lora_pool *shape, const lora_batch *batch, const void *plan, size_t plan_bytes,
                              int32_t n_groups, int32_t n_slices, const int32_t *d_outs,
                              const lora_problem *problems, int32_t problems_aligned, hipStream_t stream) {
  if (!shape || !d_outs) return LORA_EINVAL;
  if (n_slices < 1 || n_slices > LORA_MAX_SLICES) return LORA_ESHAPE;
  for (int p = 0; p < n_slices; ++p)
    if (d_outs[p] < 1) return LORA_ESHAPE;
  lora_pool sh = *shape;  // the shape's d_out is not used: each slice has its own
  sh.d_out = d_outs[0];
  shape = &sh;
  lora_status st = check_shape(shape);
  if (st) return st;
  BatchDims d;
  if ((st = check_batch(batch, d))) return st;
  if ((int64_t)d.K * shape->rank > LORA_MAX_SLOT_RANK) return LORA_EUNSUPPORTED;
  if (n_groups < 0) return LORA_ESHAPE;
  if (n_groups > 0 && !problems) return LORA_EINVAL;
  if (!aligned16(problems)) return LORA_EINVAL;
  if ((int64_t)n_groups * n_slices > INT32_MAX) return LORA_ESHAPE;
  Plan P;
  if ((st = plan_for(d, shape->n_adapters, plan, plan_bytes, P))) return st;
  if (n_groups == 0 || d.T == 0 || d.S == 0) return LORA_OK;
  const int E = shape->dtype == LORA_BF16 ? 8 : 4;
  bool vec = problems_aligned && shape->d_in % E == 0 && shape->rank % E == 0;
  for (int p = 0; p < n_slices; ++p) vec = vec && d_outs[p] % E == 0;
  ApplyArgs a;
  fill_common(a, batch, d, P, shape);
  a.probs = problems;
  a.n_problems = n_groups;
  const Launch L = configure(MODE_FUSED, shape, d, P, n_groups, n_slices, d_outs, vec, a);
  if (launch_all(MODE_FUSED, shape->dtype, L, a, stream) != hipSuccess) return LORA_EHIP;
  return LORA_OK;
}

// Active slots of a merge (host arrays): indices and alpha-folded scales.
lora_status merge_slots(const lora_pool *shape, const int32_t *idx, const float *scale, int32_t n_slots, float alpha,
                        MergeArgs &a) {
  if (!idx) return LORA_EINVAL;
  if (n_slots < 1) return LORA_ESHAPE;
  if (n_slots > LORA_MAX_SLOTS) return LORA_EUNSUPPORTED;
  for (int k = 0; k < n_slots; ++k) {
    const int i = idx[k];
    if (i == -1) continue;
    if (i < -1 || i >= shape->n_adapters) return LORA_EINVAL;
    a.idx[a.nslots] = i;
    a.s[a.nslots] = alpha * (scale ? scale[k] : 1.0f);
    ++a.nslots;
  }
  a.r = shape->rank;
  a.ranks = shape->ranks;
  a.d_in = shape->d_in;
  a.d_out = shape->d_out;
  return LORA_OK;
}

lora_status lora_merge(const lora_pool *pool, const int32_t *idx, const float *scale, int32_t n_slots, float alpha,
                       void *W, int64_t ldw, hipStream_t stream) {
  lora_status st = check_pool(pool);
  if (st) return st;
  if (!W) return LORA_EINVAL;
  if (ldw < pool->d_in) return LORA_ESHAPE;
  const int eb = elem_bytes(pool->dtype);
  const size_t ws = span_bytes(pool->d_out, ldw, pool->d_in, eb);
  const size_t as = size_t(pool->n_adapters) * pool->rank * pool->d_in * eb;
  const size_t bs = size_t(pool->n_adapters) * pool->d_out * pool->rank * eb;
  if (overlap(W, ws, pool->A, as) || overlap(W, ws, pool->B, bs)) return LORA_EINVAL;
  MergeArgs a;
  std::memset(&a, 0, sizeof(a));
  if ((st = merge_slots(pool, idx, scale, n_slots, alpha, a))) return st;
  if (a.nslots == 0) return LORA_OK;
  a.single = lora_merge_problem{pool->A, pool->B, W, ldw};
  a.n_problems = 1;
  a.aligned = aligned16(pool->A) && aligned16(pool->B) && aligned16(W) && ldw % 8 == 0;
  if (launch_merge(a, pool->dtype, stream) != hipSuccess) return LORA_EHIP;
  return LORA_OK;
}

lora_status lora_merge_multi(const lora_pool *shape, const int32_t *idx, const float *scale, int32_t n_slots,
                             float alpha, int32_t n_problems, const lora_merge_problem *problems,
                             int32_t problems_aligned, hipStream_t stream) {
  if (!shape) return LORA_EINVAL;
  lora_status st = check_shape(shape);
  if (st) return st;
  if (n_problems < 0) return LORA_ESHAPE;
  if (n_problems > 0 && !problems) return LORA_EINVAL;
  MergeArgs a;
  std::memset(&a, 0, sizeof(a));
  if ((st = merge_slots(shape, idx, scale, n_slots, alpha, a))) return st;
  if (a.nslots == 0 || n_problems == 0) return LORA_OK;
  a.probs = problems;
  a.n_problems = n_problems;
  a.aligned = problems_aligned ? 1 : 0;
  if (launch_merge(a, shape->dtype, stream) != hipSuccess) return LORA_EHIP;
  return LORA_OK;
}

lora_status lora_pool_load(const lora_pool *pool, int32_t slot, const void *A_host, const void *B_host,
                           hipStream_t stream) {
  lora_status st = check_pool(pool);
  if (st) return st;
  if (!A_host || !B_host) return LORA_EINVAL;
  if (slot < 0 || slot >= pool->n_adapters) return LORA_ESHAPE;
  const size_t eb = size_t(elem_bytes(pool->dtype));
  const size_t a_bytes = size_t(pool->rank) * pool->d_in * eb, b_bytes = size_t(pool->d_out) * pool->rank * eb;
  void *A = const_cast<char *>(static_cast<const char *>(pool->A)) + size_t(slot) * a_bytes;
  void *B = const_cast<char *>(static_cast<const char *>(pool->B)) + size_t(slot) * b_bytes;
  if (hipMemcpyAsync(A, A_host, a_bytes, hipMemcpyHostToDevice, stream) != hipSuccess) return LORA_EHIP;
  if (hipMemcpyAsync(B, B_host, b_bytes, hipMemcpyHostToDevice, stream) != hipSuccess) return LORA_EHIP;
  return LORA_OK;
}

lora_status lora_read_device_errors(const void *plan, size_t plan_bytes, int32_t *count, hipStream_t stream) {
  if (!plan || !count) return LORA_EINVAL;
  if (plan_bytes < sizeof(int) * H_WORDS) return LORA_EWORKSPACE;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, static_cast<const int *>(plan) + H_ERR, sizeof(v), hipMemcpyDeviceToHost, stream) !=
      hipSuccess)
    return LORA_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return LORA_EHIP;
  *count = v;
  return LORA_OK;
}

}  // extern "C"
