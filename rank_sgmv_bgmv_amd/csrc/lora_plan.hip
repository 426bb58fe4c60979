// Segment / index scheduler: groups the requests of a batch by adapter and
// cuts every group into row tiles for the apply kernels.
//
// "Serving several LoRAs, ControlNet and IP-Adapter", "Exercises" (the
// four-request, four-LoRA answer): the batch is partitioned by adapter, each
// partition gets its own low-rank product from a single segmented kernel, and
// the results land back in the rows they came from; requests on one adapter
// share a partition, so its products are bigger and use the hardware better.
// "Punica: Multi-Tenant LoRA Serving" (contribution 1) describes the same
// segmented-gather scheme.
//
// The plan is built on the device by one workgroup, so indices and offsets
// never travel to the host.  Steps:
//   1. sanitise offsets: start[s] = clamp(max(seg_off[0..s]), 0, T), which
//      makes requests disjoint whatever the input; violations are counted;
//   2. key every request: its only valid adapter, or a shared "multi" key n
//      when it stacks several adapters (each such request is its own group),
//      or none when it has no rows or no valid slot; invalid indices counted;
//   3. counting sort of requests by key (histogram, scan, scatter);
//   4. prefix sums of the sorted requests' lengths (rows in sorted order);
//   5. group boundaries; a group of >= kMfmaMinRows rows is cut into MFMA
//      tiles of kMfmaRows rows, and a second time into tiles of
//      kMfmaRowsSmall rows (the MFMA kernel picks one tiling per launch), a
//      smaller group into VALU tiles of kValuRows;
//   6. one tile descriptor per tile.  An MFMA tile inside one request:
//      {first row, request, rows, first token row}; one that spans requests:
//      {first row, first sorted request, rows, -1}.  A VALU tile: {first row,
//      first sorted request, rows, group end}, and a record with each row's
//      token row and request and the tile's compacted adapters, so the apply
//      kernels start streaming after one read (two with per-slot scales).
// The one-wave kernel (batches of up to 64 requests) takes the same steps
// with wave scans and a rank sort instead of the counting sort.
// Rows never move: a tile names rows by (sorted request, offset) and the apply
// kernels read and write x / y rows in place.

#include <climits>

#include "lora_internal.hpp"

namespace lora {
namespace {

// Inclusive prefix sum / maximum over the 64 lanes of a wave, in registers
// (no LDS round trips): DPP row shifts by 1, 2, 4 and 8 lanes scan each row of
// 16 lanes, then the last lane of rows 0 and 2 is folded into rows 1 and 3
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).  A lane with no
// source lane takes the identity.  Every lane of the wave must be active.
__device__ __forceinline__ int wave_incl_scan_add(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ int wave_incl_scan_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x118, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x143, 0xc, 0xf, false));
  return v;
}

// The value lane 63 of the wave holds (a scalar read, no LDS round trip).
__device__ __forceinline__ int wave_last(int v) { return __builtin_amdgcn_readlane(v, 63); }

// Exclusive prefix sum of one value per thread over the 1024-thread block.
__device__ int block_excl_scan_add(int v, int *sh, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan_add(v);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int t = lane < 16 ? sh[lane] : 0;
    const int ti = wave_incl_scan_add(t);
    if (lane < 16) sh[lane] = ti - t;
    if (lane == 15) sh[16] = ti;
  }
  __syncthreads();
  const int res = inc - v + sh[w];
  total = sh[16];
  __syncthreads();
  return res;
}

// Inclusive prefix max of one value per thread over the block.
__device__ int block_incl_scan_max(int v, int *sh, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan_max(v);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int t = lane < 16 ? sh[lane] : INT_MIN;
    const int ti = wave_incl_scan_max(t);
    if (lane < 16) sh[lane] = ti;  // inclusive max of waves 0..lane
  }
  __syncthreads();
  const int res = w > 0 ? max(inc, sh[w - 1]) : inc;
  total = sh[15];
  __syncthreads();
  return res;
}

// out[i] = sum_{j<i} in[j]; in and out may alias.  Returns the total.  Thread
// i % 1024 writes out[i] after the scan's last barrier: other threads may read
// it only after a further __syncthreads().
__device__ int chunked_excl_scan(const int *in, int *out, int N, int *sh) {
  int carry = 0;
  for (int base = 0; base < N; base += kPlanThreads) {
    const int i = base + threadIdx.x;
    const int v = i < N ? in[i] : 0;
    int tot;
    const int ex = block_excl_scan_add(v, sh, tot);
    if (i < N) out[i] = carry + ex;
    carry += tot;
  }
  return carry;
}

// Largest g in [lo, hi] with a[g] <= key (a non-decreasing, a[lo] <= key).
__device__ __forceinline__ int last_le(const int *a, int lo, int hi, int key) {
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= key) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Descriptor of tile uu of an MFMA tiling of `rows_per` rows per tile (toff:
// the tiling's first tile of each group).  A tile inside one request carries
// that request and its first token row ({p0, request, rows, first token row});
// one that spans requests carries {p0, first sorted request, rows, -1} and its
// rows are found through the prefix sums.
__device__ int4 mfma_tile_desc(const int *toff, int rows_per, int uu, int n_groups, const int *gstart,
                               const int *cumlen, const int *sseg, const int *sst) {
  const int g = last_le(toff, 0, n_groups - 1, uu);
  const int gs = gstart[g], ge = gstart[g + 1];
  const int p0 = cumlen[gs] + (uu - toff[g]) * rows_per;
  const int nrows = min(rows_per, cumlen[ge] - p0);
  const int q0 = last_le(cumlen, gs, ge - 1, p0);
  const bool single = cumlen[q0 + 1] >= p0 + nrows;
  return single ? make_int4(p0, sseg[q0], nrows, sst[q0] + (p0 - cumlen[q0])) : make_int4(p0, q0, nrows, -1);
}

// Row i of VALU tile uu (the tile's descriptor {first sorted row, first
// request, rows, group end} and record: rows, requests, compacted slots -- all
// rows of a tile share their adapters).  One thread per row: the row-0 thread
// also writes the descriptor, the row count and the slots; every thread writes
// its row's token, request and slot positions (zeros past the tile's rows).
__device__ void emit_vrow(const PlanView &P, const int *__restrict__ idx, int uu, int i, int n_groups,
                          const int *toff_v, const int *gstart, const int *cumlen, const int *sseg, const int *sst) {
  const int g = last_le(toff_v, 0, n_groups - 1, uu);
  const int gs = gstart[g], ge = gstart[g + 1];
  const int p0 = cumlen[gs] + (uu - toff_v[g]) * kValuRows;
  const int nrows = min(kValuRows, cumlen[ge] - p0);
  int *R = P.vrec + (int64_t)uu * kRecWords;
  uint32_t pw[2] = {0u, 0u};  // pos[i][0 .. 7], one byte per compacted slot
  if (i < nrows) {
    const int p = p0 + i;
    const int q = last_le(cumlen, gs, ge - 1, p);
    const int s = sseg[q];
    R[R_T + i] = sst[q] + (p - cumlen[q]);
    R[R_S + i] = s;
    int kk = 0;
    for (int k = 0; k < P.K; ++k) {
      const int ad = idx[(int64_t)s * P.K + k];
      if (ad < 0 || ad >= P.n) continue;
      if (i == 0) R[R_A + kk] = ad;
      pw[kk >> 2] |= uint32_t(k) << (8 * (kk & 3));
      ++kk;
    }
    if (i == 0) {
      R[R_NROWS] = nrows;
      R[R_NACT] = kk;
      P.tiles_v[uu] = make_int4(p0, q, nrows, ge);
    }
  }
  R[R_POS + 2 * i] = int(pw[0]);
  R[R_POS + 2 * i + 1] = int(pw[1]);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanView P, const int *__restrict__ seg_off,
                                                            const int *__restrict__ idx) {
  extern __shared__ int lds[];
  __shared__ int sh[20];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  const int S = P.S, T = P.T, n = P.n, K = P.K;

  // Working arrays: in LDS when they fit (small batches: no global round trips
  // between the phases), else in the workspace.  Flat pointers serve both.
  int *start = P.start, *key = P.key, *cnt = P.cnt, *cur = P.cur, *sseg = P.sseg, *sst = P.sst,
      *cumlen = P.cumlen, *gtmp = P.gtmp, *gstart = P.gstart, *toff_m = P.toff_m, *toff_v = P.toff_v,
      *toff_ms = P.toff_ms;
  if (P.lds_mode) {
    int *q = lds;
    start = q; q += S + 1;
    key = q; q += S + 1;
    sseg = q; q += S + 1;
    sst = q; q += S + 1;
    cumlen = q; q += S + 2;
    gtmp = q; q += S + 2;
    gstart = q; q += S + 2;
    toff_m = q; q += S + 2;
    toff_v = q; q += S + 2;
    toff_ms = q; q += S + 2;
    cnt = q; q += n + 2;
    cur = q;
  }

  if (tid == 0) s_err = 0;
  for (int b = tid; b <= n; b += kPlanThreads) cnt[b] = 0;
  __syncthreads();  // the error word and the histogram are zero before any thread counts into them

  // 1. sanitised request starts, start[S] = end of the last request.
  if (P.per_token) {
    for (int s = tid; s <= S; s += kPlanThreads) start[s] = s;
  } else {
    int carry = 0;
    for (int base = 0; base <= S; base += kPlanThreads) {
      const int s = base + tid;
      int v = INT_MIN;
      if (s <= S) {
        v = seg_off[s];
        int bad = 0;
        if (s == 0 && v < 0) bad = 1;
        if (s == S && v > T) bad = 1;
        if (s > 0 && v < seg_off[s - 1]) bad = 1;
        if (bad) atomicAdd(&s_err, 1);
      }
      int tot;
      const int m = block_incl_scan_max(v, sh, tot);
      if (s <= S) start[s] = min(max(max(m, carry), 0), T);
      carry = max(carry, tot);
    }
  }
  __syncthreads();

  // 2. keys and histogram.
  for (int s = tid; s < S; s += kPlanThreads) {
    const int len = start[s + 1] - start[s];
    int nact = 0, a0 = -1;
    for (int k = 0; k < K; ++k) {
      const int a = idx[(int64_t)s * K + k];
      if (a == -1) continue;
      if (a < -1 || a >= n) { atomicAdd(&s_err, 1); continue; }
      if (nact == 0) a0 = a;
      ++nact;
    }
    const int kk = (len <= 0 || nact == 0) ? -1 : (nact == 1 ? a0 : n);
    key[s] = kk;
    if (kk >= 0) atomicAdd(&cnt[kk], 1);
  }
  __syncthreads();

  // 3. bucket starts, then scatter (order inside a bucket is not significant).
  const int n_active = chunked_excl_scan(cnt, cur, n + 1, sh);
  __syncthreads();  // the scan writes its output after its last barrier
  for (int s = tid; s < S; s += kPlanThreads) {
    const int kk = key[s];
    if (kk >= 0) sseg[atomicAdd(&cur[kk], 1)] = s;
  }
  __syncthreads();

  // 4. rows in sorted order; group-start flags (a group starts where the key
  //    changes; every multi-adapter request is its own group).
  for (int q = tid; q < n_active; q += kPlanThreads) {
    const int s = sseg[q];
    sst[q] = start[s];
    cumlen[q] = start[s + 1] - start[s];
    const int kq = key[s];
    gtmp[q] = (q == 0 || kq == n || kq != key[sseg[q - 1]]) ? 1 : 0;
  }
  __syncthreads();
  const int total_rows = chunked_excl_scan(cumlen, cumlen, n_active, sh);
  if (tid == 0) cumlen[n_active] = total_rows;
  // 5. group starts: compact the flags (the flag of q is gtmp[q+1] - gtmp[q] after the scan)
  for (int q = tid; q < n_active; q += kPlanThreads) gstart[q] = gtmp[q];
  __syncthreads();
  const int n_groups = chunked_excl_scan(gtmp, gtmp, n_active, sh);
  for (int q = tid; q < n_active; q += kPlanThreads)
    if (gstart[q]) toff_m[gtmp[q]] = q;
  __syncthreads();
  for (int g = tid; g < n_groups; g += kPlanThreads) gstart[g] = toff_m[g];
  if (tid == 0) gstart[n_groups] = n_active;
  __syncthreads();

  // tiles per group
  for (int g = tid; g < n_groups; g += kPlanThreads) {
    const int rows = cumlen[gstart[g + 1]] - cumlen[gstart[g]];
    const bool big = rows >= kMfmaMinRows;
    toff_m[g] = big ? (rows + kMfmaRows - 1) / kMfmaRows : 0;
    toff_v[g] = big ? 0 : (rows + kValuRows - 1) / kValuRows;
    toff_ms[g] = big ? (rows + kMfmaRowsSmall - 1) / kMfmaRowsSmall : 0;
  }
  __syncthreads();
  const int nt_m = chunked_excl_scan(toff_m, toff_m, n_groups, sh);
  const int nt_v = chunked_excl_scan(toff_v, toff_v, n_groups, sh);
  const int nt_ms = chunked_excl_scan(toff_ms, toff_ms, n_groups, sh);
  if (tid == 0) { toff_m[n_groups] = nt_m; toff_v[n_groups] = nt_v; toff_ms[n_groups] = nt_ms; }
  __syncthreads();

  // 6. tile descriptors; VALU tiles also get a record; then the second MFMA tiling
  for (int u = tid; u < nt_m; u += kPlanThreads)
    P.tiles_m[u] = mfma_tile_desc(toff_m, kMfmaRows, u, n_groups, gstart, cumlen, sseg, sst);
  for (int w = tid; w < nt_v * kValuRows; w += kPlanThreads)
    emit_vrow(P, idx, w / kValuRows, w % kValuRows, n_groups, toff_v, gstart, cumlen, sseg, sst);
  for (int u = tid; u < nt_ms; u += kPlanThreads)
    P.tiles_ms[u] = mfma_tile_desc(toff_ms, kMfmaRowsSmall, u, n_groups, gstart, cumlen, sseg, sst);

  // the apply kernels read these three arrays for MFMA tiles
  if (P.lds_mode) {
    for (int q = tid; q < n_active; q += kPlanThreads) {
      P.sseg[q] = sseg[q];
      P.sst[q] = sst[q];
      P.cumlen[q] = cumlen[q];
    }
    if (tid == 0) P.cumlen[n_active] = total_rows;
  }

  __syncthreads();
  if (tid == 0) {
    P.hdr[H_TILES_MS] = nt_ms;
    P.hdr[H_TILES_M] = nt_m;
    P.hdr[H_TILES_V] = nt_v;
    P.hdr[H_ERR] = s_err;
    P.hdr[H_ACTIVE] = n_active;
    P.hdr[H_GROUPS] = n_groups;
    P.hdr[H_ROWS] = total_rows;
    P.hdr[H_N] = n;
    P.hdr[H_S] = S;
    P.hdr[H_T] = T;
    P.hdr[H_K] = K;
    P.hdr[H_MAGIC] = kPlanMagic;
  }
}

// Batches of at most 64 requests: one request per lane of a wave.  The
// counting sort becomes a rank by comparison -- stable, by key and then by
// request, so the order inside a group is fixed -- and every scan a wave scan.
// Same plan as plan_kernel.  Every wave of the workgroup computes the same
// sort and scans from the same inputs (so each holds the tile counts in its
// registers) and wave 0 alone writes the shared arrays; the tile descriptors,
// one binary search over the groups and one over the requests each, are then
// shared out over all kPlanSmallThreads threads (a long prefill batch has
// thousands of tiles).
__global__ __launch_bounds__(kPlanSmallThreads) void plan_kernel_small(PlanView P, const int *__restrict__ seg_off,
                                                                       const int *__restrict__ idx) {
  __shared__ int s_sseg[64], s_sst[64], s_key[64], s_cum[65], s_gstart[65], s_toff_m[65], s_toff_v[65], s_toff_ms[65];
  __shared__ int s_idx[64 * LORA_MAX_SLOTS];  // the batch's idx [S][K], read once from memory
  __shared__ __align__(16) long long s_ck[64];  // every request's (key, request) pair, for the rank
  const int tid = threadIdx.x, lane = tid & 63;
  const bool w0 = tid < 64;  // the wave that writes the shared arrays
  const int S = P.S, T = P.T, n = P.n, K = P.K;
  const bool req = lane < S;
  int err = 0;
  // every load of the batch at once -- both offsets and every slot's index --
  // through clamped addresses (lanes past the batch read its last request and
  // drop the values), so the plan waits for one round trip to memory
  int v0 = INT_MIN, v1 = INT_MIN;
  int ads[LORA_MAX_SLOTS];
#pragma unroll
  for (int k = 0; k < LORA_MAX_SLOTS; ++k) ads[k] = -1;
  if (S > 0) {
    const int ls = min(lane, S - 1);
    if (!P.per_token) {
      v0 = seg_off[ls];
      v1 = seg_off[ls + 1];
    }
#pragma unroll
    for (int k = 0; k < LORA_MAX_SLOTS; ++k) ads[k] = idx[(int64_t)ls * K + min(k, K - 1)];
  }
  if (!req) {
    v0 = v1 = INT_MIN;
#pragma unroll
    for (int k = 0; k < LORA_MAX_SLOTS; ++k) ads[k] = -1;
  }
  // 1. sanitised request bounds [st, en): the prefix maximum of the offsets, clamped to [0, T]
  int st = lane, en = lane + 1;
  if (!P.per_token) {
    if (req) err += (lane == 0 && v0 < 0) + (v1 < v0) + (lane == S - 1 && v1 > T);
    const int m = wave_incl_scan_max(v0);
    st = min(max(m, 0), T);
    en = min(max(max(m, v1), 0), T);
  }
  // 2. key: the only valid adapter, n for several (each such request is its own group), -1 for none
  // (the indices are kept in LDS for the tile records)
  int key = -1;
  if (req) {
    int nact = 0, a0 = -1;
#pragma unroll
    for (int k = 0; k < LORA_MAX_SLOTS; ++k) {
      if (k < K) {
        const int a = ads[k];
        if (w0) s_idx[lane * K + k] = a;
        if (a != -1) {
          if (a < -1 || a >= n) {
            ++err;
          } else {
            if (nact == 0) a0 = a;
            ++nact;
          }
        }
      }
    }
    key = (en - st <= 0 || nact == 0) ? -1 : (nact == 1 ? a0 : n);
  }
  // 3. stable rank among the active requests: (key, request) as one 64-bit
  // value, the inactive requests after every active one, so the rank is a
  // count of smaller values -- one compare and one add per request, on values
  // read back from LDS in 16-byte pieces, all in flight at once
  const long long ck = key >= 0 ? (static_cast<long long>(key) << 6) | lane : LLONG_MAX;
  if (w0) s_ck[lane] = ck;
  __syncthreads();
  int rank = 0;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    longlong2 q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = reinterpret_cast<const longlong2 *>(s_ck)[8 * h + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) rank += int(q[j].x < ck) + int(q[j].y < ck);
  }
  const unsigned long long act = __ballot(key >= 0);
  const int n_active = __popcll(act);
  if (w0 && key >= 0) {
    s_sseg[rank] = lane;
    s_sst[rank] = st;
    s_key[rank] = key;
    s_cum[rank] = en - st;
  }
  __syncthreads();
  // 4. rows in sorted order and group starts
  const bool live = lane < n_active;
  const int len = live ? s_cum[lane] : 0, kq = live ? s_key[lane] : -1;
  const int inc = wave_incl_scan_add(len);
  const int total_rows = wave_last(inc);
  const int kprev = __shfl_up(kq, 1);
  const int flag = live && (lane == 0 || kq == n || kq != kprev) ? 1 : 0;
  const int ginc = wave_incl_scan_add(flag);
  const int n_groups = wave_last(ginc);
  __syncthreads();
  if (w0 && live) s_cum[lane] = inc - len;
  if (tid == 0) s_cum[n_active] = total_rows;
  if (w0 && flag) s_gstart[ginc - 1] = lane;
  if (tid == 0) s_gstart[n_groups] = n_active;
  __syncthreads();
  // 5. tiles per group (lane g)
  int nm = 0, nv = 0, nms = 0;
  if (lane < n_groups) {
    const int rows = s_cum[s_gstart[lane + 1]] - s_cum[s_gstart[lane]];
    const bool big = rows >= kMfmaMinRows;
    nm = big ? (rows + kMfmaRows - 1) / kMfmaRows : 0;
    nv = big ? 0 : (rows + kValuRows - 1) / kValuRows;
    nms = big ? (rows + kMfmaRowsSmall - 1) / kMfmaRowsSmall : 0;
  }
  const int im = wave_incl_scan_add(nm), iv = wave_incl_scan_add(nv), ims = wave_incl_scan_add(nms);
  const int nt_m = wave_last(im), nt_v = wave_last(iv), nt_ms = wave_last(ims);
  if (w0 && lane < n_groups) {
    s_toff_m[lane] = im - nm;
    s_toff_v[lane] = iv - nv;
    s_toff_ms[lane] = ims - nms;
  }
  if (tid == 0) {
    s_toff_m[n_groups] = nt_m;
    s_toff_v[n_groups] = nt_v;
    s_toff_ms[n_groups] = nt_ms;
  }
  __syncthreads();
  // 6. tile descriptors and records
  for (int u = tid; u < nt_m; u += kPlanSmallThreads)
    P.tiles_m[u] = mfma_tile_desc(s_toff_m, kMfmaRows, u, n_groups, s_gstart, s_cum, s_sseg, s_sst);
  for (int w = tid; w < nt_v * kValuRows; w += kPlanSmallThreads)
    emit_vrow(P, s_idx, w / kValuRows, w % kValuRows, n_groups, s_toff_v, s_gstart, s_cum, s_sseg, s_sst);
  for (int u = tid; u < nt_ms; u += kPlanSmallThreads)
    P.tiles_ms[u] = mfma_tile_desc(s_toff_ms, kMfmaRowsSmall, u, n_groups, s_gstart, s_cum, s_sseg, s_sst);
  // the apply kernels read these three arrays for MFMA tiles
  if (w0 && live) {
    P.sseg[lane] = s_sseg[lane];
    P.sst[lane] = s_sst[lane];
    P.cumlen[lane] = s_cum[lane];
  }
  if (tid == 0) P.cumlen[n_active] = total_rows;
  err = wave_last(wave_incl_scan_add(err));
  if (tid == 0) {
    P.hdr[H_TILES_MS] = nt_ms;
    P.hdr[H_TILES_M] = nt_m;
    P.hdr[H_TILES_V] = nt_v;
    P.hdr[H_ERR] = err;
    P.hdr[H_ACTIVE] = n_active;
    P.hdr[H_GROUPS] = n_groups;
    P.hdr[H_ROWS] = total_rows;
    P.hdr[H_N] = n;
    P.hdr[H_S] = S;
    P.hdr[H_T] = T;
    P.hdr[H_K] = K;
    P.hdr[H_MAGIC] = kPlanMagic;
  }
}

}  // namespace

hipError_t launch_plan(const PlanView &P, size_t lds_bytes, const int *seg_off, const int *idx, hipStream_t stream) {
  static const bool lds_limit_raised =
      raise_lds_limit(reinterpret_cast<const void *>(plan_kernel), kPlanLdsBudget);
  (void)lds_limit_raised;
  if (P.S <= 64)
    hipLaunchKernelGGL(plan_kernel_small, dim3(1), dim3(kPlanSmallThreads), 0, stream, P, seg_off, idx);
  else
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), P.lds_mode ? lds_bytes : 0, stream, P, seg_off, idx);
  return hipGetLastError();
}

}  // namespace lora
