// Internal declarations shared by the plan (scheduler) kernel, the apply
// kernels and the C-ABI host entry points.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lora.h"

namespace lora {

constexpr int kPlanThreads = 1024;  // one workgroup builds the plan
constexpr int kPlanSmallThreads = 256;  // the plan of a batch of at most 64 requests
constexpr int kThreads = 256;       // apply kernels: 4 wave64s per workgroup
constexpr int kValuThreads = 256;   // VALU kernel workgroup
constexpr int kMfmaRows = 64;       // rows per MFMA tile (16 per wave)
constexpr int kMfmaRowsSmall = 48;  // rows per MFMA tile of the plan's second tiling (the fourth wave idles)
constexpr int kValuRows = 4;        // rows per VALU tile (one row block: heavy adapters become several tiles)
constexpr int kMfmaMinRows = 17;    // adapter groups with at least this many rows get MFMA tiles
constexpr int kRowBlock = 4;        // rows per VALU pass (register budget of the VALU tile body)
constexpr int kMfmaMaxRank = 128;   // MFMA tiles serve ranks 16, 32, 64, 128
constexpr int kMfmaMinBatch = 128;  // batches of fewer rows leave every tile to the VALU kernel (one launch)
constexpr int kMfmaMaxSlotRank = 512;
constexpr int kMaxLdsBytes = 160 * 1024;  // LDS a gfx950 workgroup may allocate

// Record of one VALU tile, written by the plan (int32 words): everything the
// apply kernels need to start on the tile except the scales, in one 128-byte
// read.  pos holds, per row and compacted slot, the original slot index (one
// byte each).
enum {
  R_NROWS = 0,   // rows of the tile (1 .. kValuRows)
  R_NACT = 1,    // valid slots (adapters) of the tile's rows
  R_T = 2,       // token row of each row          [kValuRows]
  R_S = 6,       // request of each row            [kValuRows]
  R_A = 10,      // adapter of each compacted slot [LORA_MAX_SLOTS]
  R_POS = 18,    // bytes pos[row][slot]           [kValuRows * LORA_MAX_SLOTS / 4 words]
  kRecWords = 32
};
static_assert(kValuRows == 4 && LORA_MAX_SLOTS == 8, "tile record layout assumes 4 rows and 8 slots");

// Plan header words (int32).
enum {
  H_TILES_M = 0,   // number of MFMA tiles
  H_TILES_V = 1,   // number of VALU tiles
  H_ERR = 2,       // invalid indices + offset violations met by the last build
  H_ACTIVE = 3,    // requests with at least one row and one valid slot
  H_GROUPS = 4,    // adapter groups
  H_ROWS = 5,      // rows covered by active requests
  H_N = 6, H_S = 7, H_T = 8, H_K = 9,
  H_MAGIC = 10,
  H_TILES_MS = 11,  // number of MFMA tiles of the second (kMfmaRowsSmall-row) tiling
  H_WORDS = 64
};
constexpr int kPlanMagic = 0x4c6f5241;  // "LoRA"

// Byte offsets of the plan arrays inside the workspace.
struct PlanLayout {
  size_t hdr, start, key, cnt, cur, sseg, sst, cumlen, gtmp, gstart, toff_m, toff_v, toff_ms, tiles_m, tiles_v,
      tiles_ms, vrec, total;
  int S, T, n, bound_m, bound_v, bound_ms;
  size_t lds_bytes;  // LDS the plan kernel uses for its working arrays (0: they stay in global memory)
};

// The plan kernel keeps its working arrays in LDS when they fit in this budget.
constexpr size_t kPlanLdsBudget = 144 * 1024;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline PlanLayout plan_layout(int S, int T, int n) {
  PlanLayout L{};
  L.S = S; L.T = T; L.n = n;
  L.bound_m = (T + kMfmaRows - 1) / kMfmaRows + S + 1;
  L.bound_v = (T + kValuRows - 1) / kValuRows + S + 1;
  L.bound_ms = (T + kMfmaRowsSmall - 1) / kMfmaRowsSmall + S + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  L.hdr = take(sizeof(int) * H_WORDS);
  L.start = take(sizeof(int) * (size_t(S) + 1));
  L.key = take(sizeof(int) * (size_t(S) + 1));
  L.cnt = take(sizeof(int) * (size_t(n) + 2));
  L.cur = take(sizeof(int) * (size_t(n) + 2));
  L.sseg = take(sizeof(int) * (size_t(S) + 1));
  L.sst = take(sizeof(int) * (size_t(S) + 1));
  L.cumlen = take(sizeof(int) * (size_t(S) + 2));
  L.gtmp = take(sizeof(int) * (size_t(S) + 2));
  L.gstart = take(sizeof(int) * (size_t(S) + 2));
  L.toff_m = take(sizeof(int) * (size_t(S) + 2));
  L.toff_v = take(sizeof(int) * (size_t(S) + 2));
  L.toff_ms = take(sizeof(int) * (size_t(S) + 2));
  L.tiles_m = take(sizeof(int4) * size_t(L.bound_m));
  L.tiles_v = take(sizeof(int4) * size_t(L.bound_v));
  L.tiles_ms = take(sizeof(int4) * size_t(L.bound_ms));
  L.vrec = take(sizeof(int) * kRecWords * size_t(L.bound_v));
  L.total = off;
  // working arrays: start, key, sseg, sst (S+1 each), cumlen, gtmp, gstart, toff_m, toff_v, toff_ms (S+2
  // each), cnt, cur (n+2 each)
  const size_t lds_ints = 4 * (size_t(S) + 1) + 6 * (size_t(S) + 2) + 2 * (size_t(n) + 2);
  L.lds_bytes = lds_ints * sizeof(int) <= kPlanLdsBudget ? lds_ints * sizeof(int) : 0;
  return L;
}

// Device view of a plan.
struct PlanView {
  int *hdr, *start, *key, *cnt, *cur, *sseg, *sst, *cumlen, *gtmp, *gstart, *toff_m, *toff_v, *toff_ms;
  int4 *tiles_m, *tiles_v, *tiles_ms;
  int *vrec;  // per VALU tile: a record of kRecWords words
  int S, T, n, K, per_token;
  int lds_mode;
};

inline PlanView plan_view(void *ws, const PlanLayout &L, int K, int per_token) {
  char *b = static_cast<char *>(ws);
  PlanView P;
  P.hdr = reinterpret_cast<int *>(b + L.hdr);
  P.start = reinterpret_cast<int *>(b + L.start);
  P.key = reinterpret_cast<int *>(b + L.key);
  P.cnt = reinterpret_cast<int *>(b + L.cnt);
  P.cur = reinterpret_cast<int *>(b + L.cur);
  P.sseg = reinterpret_cast<int *>(b + L.sseg);
  P.sst = reinterpret_cast<int *>(b + L.sst);
  P.cumlen = reinterpret_cast<int *>(b + L.cumlen);
  P.gtmp = reinterpret_cast<int *>(b + L.gtmp);
  P.gstart = reinterpret_cast<int *>(b + L.gstart);
  P.toff_m = reinterpret_cast<int *>(b + L.toff_m);
  P.toff_v = reinterpret_cast<int *>(b + L.toff_v);
  P.toff_ms = reinterpret_cast<int *>(b + L.toff_ms);
  P.tiles_m = reinterpret_cast<int4 *>(b + L.tiles_m);
  P.tiles_v = reinterpret_cast<int4 *>(b + L.tiles_v);
  P.tiles_ms = reinterpret_cast<int4 *>(b + L.tiles_ms);
  P.vrec = reinterpret_cast<int *>(b + L.vrec);
  P.S = L.S; P.T = L.T; P.n = L.n; P.K = K; P.per_token = per_token;
  P.lds_mode = L.lds_bytes > 0;
  return P;
}

enum Mode { MODE_FUSED = 0, MODE_SHRINK = 1, MODE_EXPAND = 2 };

struct ApplyArgs {
  // batch
  const int *seg_off;
  const int *idx;
  const float *scale;
  int K;
  int T, S;  // the call's rows and requests (checked against the plan's header)
  // plan (read only but for the error word)
  const int *hdr, *sseg, *sst, *cumlen;
  const int4 *tiles_m, *tiles_v;
  const int4 *tiles_ms;  // the plan's second MFMA tiling (kMfmaRowsSmall rows per tile)
  const int *vrec;
  // shape shared by every problem
  int n, r, d_in, d_out;
  const int *ranks;  // per-adapter ranks (device), or nullptr: every adapter has rank r
  // problems
  lora_problem single;
  const lora_problem *probs;  // device array, or nullptr => `single`
  int n_problems;             // groups of `ns` problems (plain calls: problems)
  // Output slices: a group of `ns` problems (entries g*ns .. g*ns+ns-1 of probs)
  // shares the tiles; slice p writes d_out[p] columns.  A tile's work is split
  // into output-column chunks: slice p has cv[p] chunks of wv[p] columns
  // (VALU tiles) and cm[p] of wm[p] (MFMA tiles); cvo / cmo are their prefix
  // sums (a tile's items across all slices: cvo[ns], cmo[ns]).  Plain calls
  // have one slice of the shape's d_out.
  int ns;
  int sd_out[LORA_MAX_SLICES];
  int cv[LORA_MAX_SLICES], wv[LORA_MAX_SLICES], cm[LORA_MAX_SLICES], wm[LORA_MAX_SLICES];
  int cvo[LORA_MAX_SLICES + 1], cmo[LORA_MAX_SLICES + 1];
  // cvo[ns] and cmo[ns] (a tile's VALU and MFMA items over every slice), as
  // plain fields: an index known only at run time into the tables above would
  // make the kernels copy them to scratch memory
  int items_v_tile, items_m_tile;
  // every MFMA tile costs about the same (one slot per request, one rank):
  // the MFMA kernel deals contiguous ranges of tiles to the XCDs
  int mfma_uniform;
  // split API: float32 intermediate [T][ldv]
  float *v;
  int64_t ldv;
  // layout of dynamic LDS
  int kr_max;      // max_slots * rank (row stride of the VALU intermediate)
  int valu_takes_m;  // the VALU kernel also runs the MFMA-sized tiles (no MFMA kernel launched)
  // MFMA tiling choice: the CUs of the device and the MFMA workgroups that fit on it at once
  int n_cu, mfma_slots;
};

// Merge / unmerge of stacked adapters into weights: for every problem p,
// W_p += sum_k s[k] B_{p,idx[k]} A_{p,idx[k]} (alpha folded into s).
struct MergeArgs {
  lora_merge_problem single;
  const lora_merge_problem *probs;  // device array, or nullptr => `single`
  int n_problems;
  int idx[LORA_MAX_SLOTS];  // active slots' adapter indices
  float s[LORA_MAX_SLOTS];
  int nslots;  // active slots, 1 .. LORA_MAX_SLOTS
  int r, d_in, d_out;
  const int *ranks;  // per-adapter ranks (device), or nullptr
  int aligned;   // every problem's pointers and ldw allow 16-byte accesses
};
bool merge_mfma_eligible(const MergeArgs &a, int dtype);
hipError_t launch_merge(const MergeArgs &a, int dtype, hipStream_t stream);

// Lift a kernel's dynamic-LDS limit to `bytes` (at most what gfx950 allows
// beside the kernel's static LDS); called once per kernel, before its first
// launch.  A refused attribute leaves the limit as it was and is cleared, so
// that it is not reported as the error of the launch that follows.
inline bool raise_lds_limit(const void *kernel, size_t bytes) {
  hipFuncAttributes at;
  size_t stat = 0;
  if (hipFuncGetAttributes(&at, kernel) == hipSuccess) stat = at.sharedSizeBytes;
  const size_t lim = bytes + stat > size_t(kMaxLdsBytes) ? size_t(kMaxLdsBytes) - stat : bytes;
  const bool ok = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(lim)) == hipSuccess;
  (void)hipGetLastError();
  return ok;
}

size_t valu_smem_bytes(int kr_max);
// MFMA kernel LDS per workgroup; `half`: the half-size stages (ranks 64 / 128 only).
size_t mfma_smem_bytes(int jt, int slots, bool half);
bool mfma_half_available(int jt);

hipError_t launch_plan(const PlanView &P, size_t lds_bytes, const int *seg_off, const int *idx, hipStream_t stream);

// VALU kernel: dtype LORA_F32 / LORA_BF16, vec = 16-byte vector path.
hipError_t launch_valu(int mode, int dtype, bool vec, const ApplyArgs &args, int grid, size_t smem,
                       hipStream_t stream);
// MFMA kernel (bf16, vector path): jt = rank / 16 in {1, 2, 4, 8}.
hipError_t launch_mfma(int mode, int jt, bool half, const ApplyArgs &args, int grid, size_t smem,
                       hipStream_t stream);
// MFMA kernel for fused launches whose requests stack 2 .. smax (2 or 4) slots:
// a tile with several slots walks x once for all of them.
size_t mfma_stacked_smem_bytes(int jt, int smax);
hipError_t launch_mfma_stacked(int jt, int smax, const ApplyArgs &args, int grid, size_t smem, hipStream_t stream);
// Sliced launches with one slot per request and nsl (2 .. 4) slices a group:
// one walk over x per row tile for every slice.  LDS: mfma_stacked_smem_bytes(jt, nsl).
hipError_t launch_mfma_sliced(int jt, int nsl, const ApplyArgs &args, int grid, size_t smem, hipStream_t stream);

}  // namespace lora
