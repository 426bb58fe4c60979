// Device helpers shared by the VALU and MFMA apply kernels: bf16 numerics,
// 16-byte vector element ops, the per-tile metadata kept in LDS, tile setup,
// wave reductions and the work-item walk.
#pragma once

#include "lora_internal.hpp"

namespace lora {

// Global-memory accesses.  The tensors reach the kernels as plain pointers
// (inside lora_problem), which the compiler cannot place in an address space;
// it would emit FLAT instructions, which also count against the LDS counter so
// every LDS access would wait for all loads in flight.  Every access to
// caller memory goes through these, as a global (address space 1) access.
#define LORA_GLOBAL __attribute__((address_space(1)))
// raw register types of 2 .. 16 bytes (and 32 / 48 for a lora_merge_problem / lora_problem)
template <int N> struct Raw;
template <> struct Raw<2> { typedef unsigned short type; };
template <> struct Raw<4> { typedef unsigned int type; };
template <> struct Raw<8> { typedef unsigned int type __attribute__((ext_vector_type(2))); };
template <> struct Raw<16> { typedef unsigned int type __attribute__((ext_vector_type(4))); };
template <> struct Raw<32> {
  struct type { Raw<16>::type q[2]; };
};
template <> struct Raw<48> {
  struct type { Raw<16>::type q[3]; };
};
template <typename V, typename T>
__device__ __forceinline__ V gload(const T *p) {
  typedef typename Raw<sizeof(V)>::type R;
  if constexpr (sizeof(V) == 32 || sizeof(V) == 48) {
    const LORA_GLOBAL Raw<16>::type *q = (const LORA_GLOBAL Raw<16>::type *)(p);
    R r;
#pragma unroll
    for (int i = 0; i < int(sizeof(V) / 16); ++i) r.q[i] = q[i];
    return __builtin_bit_cast(V, r);
  } else {
    const R r = *(const LORA_GLOBAL R *)(p);
    return __builtin_bit_cast(V, r);
  }
}
template <typename V, typename T>
__device__ __forceinline__ void gstore(T *p, const V &v) {
  typedef typename Raw<sizeof(V)>::type R;
  *(LORA_GLOBAL R *)(p) = __builtin_bit_cast(R, v);
}

// Access at a 32-bit byte offset from a wave-uniform base: one scalar base
// register pair for many rows instead of one 64-bit address per row (the
// global_load "saddr" form).  The offset must stay below 4 GiB.
template <typename V, typename T>
__device__ __forceinline__ V gload_at(const T *base, uint32_t byte_off) {
  typedef typename Raw<sizeof(V)>::type R;
  const R r = *(const LORA_GLOBAL R *)((const LORA_GLOBAL char *)base + byte_off);
  return __builtin_bit_cast(V, r);
}
template <typename V, typename T>
__device__ __forceinline__ void gstore_at(T *base, uint32_t byte_off, const V &v) {
  typedef typename Raw<sizeof(V)>::type R;
  *(LORA_GLOBAL R *)((LORA_GLOBAL char *)base + byte_off) = __builtin_bit_cast(R, v);
}

// A workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits until every global store the wave issued has completed; the kernels
// here never read, within a launch, global memory another thread wrote, so
// their barriers need not wait: a tile's y stores stay in flight while the
// next tile or stage starts.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A value every lane of the wave holds (read from LDS tile metadata): moved to
// a scalar register, so address arithmetic on it stays scalar and loads use a
// scalar base plus a 32-bit lane offset.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- numerics --
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round two floats to bf16 (round to nearest even, hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ uint16_t f_to_bf(float a) { return uint16_t(pack_bf2(a, 0.f) & 0xffffu); }

// v, or zeros, selected by value where the data is used (a select between
// two vector objects would pick between their addresses and keep them in
// memory; a select right after a load would wait for it).
__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

__device__ __forceinline__ float dot2_bf(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// ----------------------------------------------------- element vector ops --
// A "vector" is 16 bytes (8 bf16 / 4 fp32) on the vector path, one element otherwise.
template <typename T, bool VEC> struct VOps;

template <> struct VOps<uint16_t, true> {
  static constexpr int E = 8;
  typedef uint4 V;
  static __device__ __forceinline__ V load(const uint16_t *p) { return gload<uint4>(p); }
  static __device__ __forceinline__ V zero() { return make_uint4(0, 0, 0, 0); }
  static __device__ __forceinline__ float dot(V a, V b, float acc) {
    acc = dot2_bf(a.x, b.x, acc);
    acc = dot2_bf(a.y, b.y, acc);
    acc = dot2_bf(a.z, b.z, acc);
    return dot2_bf(a.w, b.w, acc);
  }
  // sum_e v[e] * b[e], v in fp32
  static __device__ __forceinline__ float dotf(const float *v, V b, float acc) {
    const float4 v0 = *reinterpret_cast<const float4 *>(v);
    const float4 v1 = *reinterpret_cast<const float4 *>(v + 4);
    acc = fmaf(v0.x, bf_lo(b.x), acc); acc = fmaf(v0.y, bf_hi(b.x), acc);
    acc = fmaf(v0.z, bf_lo(b.y), acc); acc = fmaf(v0.w, bf_hi(b.y), acc);
    acc = fmaf(v1.x, bf_lo(b.z), acc); acc = fmaf(v1.y, bf_hi(b.z), acc);
    acc = fmaf(v1.z, bf_lo(b.w), acc); acc = fmaf(v1.w, bf_hi(b.w), acc);
    return acc;
  }
  // y + d, rounded once (d: 8 floats)
  static __device__ __forceinline__ V add(V y, const float *d) {
    uint4 o;
    o.x = pack_bf2(bf_lo(y.x) + d[0], bf_hi(y.x) + d[1]);
    o.y = pack_bf2(bf_lo(y.y) + d[2], bf_hi(y.y) + d[3]);
    o.z = pack_bf2(bf_lo(y.z) + d[4], bf_hi(y.z) + d[5]);
    o.w = pack_bf2(bf_lo(y.w) + d[6], bf_hi(y.w) + d[7]);
    return o;
  }
  static __device__ __forceinline__ void add_store(uint16_t *p, const float *d) {
    uint4 y = load(p);
    const float4 d0 = *reinterpret_cast<const float4 *>(d);
    const float4 d1 = *reinterpret_cast<const float4 *>(d + 4);
    uint4 o;
    o.x = pack_bf2(bf_lo(y.x) + d0.x, bf_hi(y.x) + d0.y);
    o.y = pack_bf2(bf_lo(y.y) + d0.z, bf_hi(y.y) + d0.w);
    o.z = pack_bf2(bf_lo(y.z) + d1.x, bf_hi(y.z) + d1.y);
    o.w = pack_bf2(bf_lo(y.w) + d1.z, bf_hi(y.w) + d1.w);
    gstore(p, o);
  }
};

template <> struct VOps<uint16_t, false> {
  static constexpr int E = 1;
  typedef uint16_t V;
  static __device__ __forceinline__ V load(const uint16_t *p) { return gload<uint16_t>(p); }
  static __device__ __forceinline__ V zero() { return 0; }
  static __device__ __forceinline__ float dot(V a, V b, float acc) { return fmaf(bf_to_f(a), bf_to_f(b), acc); }
  static __device__ __forceinline__ float dotf(const float *v, V b, float acc) { return fmaf(v[0], bf_to_f(b), acc); }
  static __device__ __forceinline__ void add_store(uint16_t *p, const float *d) {
    gstore(p, f_to_bf(bf_to_f(gload<uint16_t>(p)) + d[0]));
  }
};

template <> struct VOps<float, true> {
  static constexpr int E = 4;
  typedef float4 V;
  static __device__ __forceinline__ V load(const float *p) { return gload<float4>(p); }
  static __device__ __forceinline__ V zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ float dot(V a, V b, float acc) {
    acc = fmaf(a.x, b.x, acc); acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc); return fmaf(a.w, b.w, acc);
  }
  static __device__ __forceinline__ float dotf(const float *v, V b, float acc) {
    const float4 a = *reinterpret_cast<const float4 *>(v);
    return dot(a, b, acc);
  }
  static __device__ __forceinline__ V add(V y, const float *d) {
    return make_float4(y.x + d[0], y.y + d[1], y.z + d[2], y.w + d[3]);
  }
  static __device__ __forceinline__ void add_store(float *p, const float *d) {
    float4 y = load(p);
    const float4 a = *reinterpret_cast<const float4 *>(d);
    y.x += a.x; y.y += a.y; y.z += a.z; y.w += a.w;
    gstore(p, y);
  }
};

template <> struct VOps<float, false> {
  static constexpr int E = 1;
  typedef float V;
  static __device__ __forceinline__ V load(const float *p) { return gload<float>(p); }
  static __device__ __forceinline__ V zero() { return 0.f; }
  static __device__ __forceinline__ float dot(V a, V b, float acc) { return fmaf(a, b, acc); }
  static __device__ __forceinline__ float dotf(const float *v, V b, float acc) { return fmaf(v[0], b, acc); }
  static __device__ __forceinline__ void add_store(float *p, const float *d) { gstore(p, gload<float>(p) + d[0]); }
};

// ------------------------------------------------------------- plan header --
// The header of the plan a launch uses, checked against the call.  A plan
// built for another batch shape or pool size (or a workspace no plan was built
// into) lays its arrays out at other offsets, so its tile descriptors would be
// read from the wrong places: on a mismatch the kernel does no work at all and
// workgroup 0 adds one to the plan's error word.
struct PlanHdr {
  int n_m, n_v, n_active, n_ms;
  bool ok;
};
__device__ inline PlanHdr read_plan_header(const ApplyArgs &a) {
  const int4 w0 = gload<int4>(a.hdr), w1 = gload<int4>(a.hdr + 4), w2 = gload<int4>(a.hdr + 8);
  static_assert(H_TILES_M == 0 && H_TILES_V == 1 && H_ACTIVE == 3 && H_N == 6 && H_S == 7 && H_T == 8 &&
                    H_K == 9 && H_MAGIC == 10 && H_TILES_MS == 11,
                "header words read as three 16-byte pieces");
  PlanHdr h;
  h.n_m = w0.x;
  h.n_v = w0.y;
  h.n_active = w0.w;
  h.n_ms = w2.w;
  h.ok = w2.z == kPlanMagic && w1.z == a.n && w1.w == a.S && w2.x == a.T && w2.y == a.K;
  if (!h.ok && blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(const_cast<int *>(a.hdr) + H_ERR, 1);
  return h;
}

// ------------------------------------------------------------ tile metadata --
constexpr int kMetaRows = kMfmaRows;  // rows of tile metadata
struct Meta {
  int t[kMetaRows];                     // token row of each tile row
  int a[LORA_MAX_SLOTS];                // the tile's adapters (compacted slot order)
  int rk[LORA_MAX_SLOTS];               // their ranks
  int nact;                             // valid slots
  int pad[3];
  int pos[kMetaRows][LORA_MAX_SLOTS];   // original slot index of compacted slot
  float sc[kMetaRows][LORA_MAX_SLOTS];  // scale of compacted slot
  int cum[kMetaRows + 1];               // staging of the sorted row prefix sums (MFMA tiles)
  int rec[kRecWords];                   // staging of a VALU tile's record
};
constexpr size_t kMetaBytes = (sizeof(Meta) + 255) & ~size_t(255);

// Original slot index of compacted slot kk of a row, from the record's two pos words.
__device__ __forceinline__ int rec_pos(uint2 w, int kk) {
  const uint32_t word = kk < 4 ? w.x : w.y;
  return int((word >> (8 * (kk & 3))) & 0xffu);
}

// Fill the metadata of a VALU tile from its record, already in registers
// (word `tid` of it in thread tid < kRecWords); returns the tile's rows.  Only
// per-slot scales are read from memory.  Two barriers.
// Rank of adapter ad: its entry of the pool's rank array, clamped to [1, r].
__device__ __forceinline__ int adapter_rank(const ApplyArgs &a, int ad) {
  return a.ranks ? min(max(gload<int>(a.ranks + ad), 1), a.r) : a.r;
}

__device__ inline int setup_from_record(const ApplyArgs &a, int word, Meta &M) {
  const int tid = threadIdx.x;
  if (tid < kRecWords) M.rec[tid] = word;
  lds_barrier();
  const int nrows = M.rec[R_NROWS], nact = M.rec[R_NACT];
  if (tid < nrows) {
    const int s = M.rec[R_S + tid];
    const uint2 pw = make_uint2(uint32_t(M.rec[R_POS + 2 * tid]), uint32_t(M.rec[R_POS + 2 * tid + 1]));
    M.t[tid] = M.rec[R_T + tid];
    for (int kk = 0; kk < nact; ++kk) {
      const int k = rec_pos(pw, kk);
      M.pos[tid][kk] = k;
      M.sc[tid][kk] = a.scale ? gload<float>(a.scale + (int64_t)s * a.K + k) : 1.0f;
    }
  }
  if (tid < nact) {
    const int ad = M.rec[R_A + tid];
    M.a[tid] = ad;
    M.rk[tid] = adapter_rank(a, ad);
  }
  if (tid == 0) M.nact = nact;
  lds_barrier();
  return nrows;
}

// Compacted slots of request s for tile rows 0 .. nrows-1 that all belong to
// it: `ad` / `sc` hold the request's K adapter indices and scales (thread
// order, already in LDS).
__device__ inline void compact_slots(const ApplyArgs &a, const int *ad, const float *sc, int row, Meta &M) {
  int kk = 0;
  for (int k = 0; k < a.K; ++k) {
    const int i = ad[k];
    if (i < 0 || i >= a.n) continue;
    M.pos[row][kk] = k;
    M.sc[row][kk] = sc[k];
    if (row == 0) {
      M.a[kk] = i;
      M.rk[kk] = adapter_rank(a, i);
    }
    ++kk;
  }
  if (row == 0) M.nact = kk;
}

// Fill an MFMA-sized tile's rows (token index, compacted slots, scales) into
// LDS.  A tile inside one request (td.w >= 0: td.y is the request, td.w its
// first token row) needs one round of loads, its slots and scales.  A tile
// that spans requests finds each row's request by a binary search over the
// sorted rows' prefix sums, staged in LDS with one parallel load, then loads
// every slot of the row at once.  Ends with a barrier.
__device__ inline void setup_rows(const ApplyArgs &a, int4 td, int n_active, Meta &M) {
  const int tid = threadIdx.x;
  const int p0 = td.x, q0 = td.y, nrows = td.z;
  if (td.w >= 0) {
    int *ad = M.rec;
    float *sc = reinterpret_cast<float *>(M.rec + LORA_MAX_SLOTS);
    if (tid < LORA_MAX_SLOTS) {
      const int64_t e = (int64_t)q0 * a.K + min(tid, a.K - 1);
      ad[tid] = gload<int>(a.idx + e);
      sc[tid] = a.scale ? gload<float>(a.scale + e) : 1.0f;
    }
    lds_barrier();
    if (tid < nrows) {
      M.t[tid] = td.w + tid;
      compact_slots(a, ad, sc, tid, M);
    }
    lds_barrier();
    return;
  }
  // a tile's rows lie in requests q0 .. q0 + nrows - 1 (each holds >= 1 row)
  const int nq = min(nrows, n_active - q0);
  if (tid <= nq) M.cum[tid] = gload<int>(a.cumlen + q0 + tid);
  lds_barrier();
  if (tid < nrows) {
    const int p = p0 + tid;
    int lo = 0, hi = min(tid, n_active - 1 - q0);
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (M.cum[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int s = gload<int>(a.sseg + q0 + lo);
    M.t[tid] = gload<int>(a.sst + q0 + lo) + (p - M.cum[lo]);
    int kk = 0;
    for (int k = 0; k < a.K; ++k) {
      const int ad = gload<int>(a.idx + (int64_t)s * a.K + k);
      if (ad < 0 || ad >= a.n) continue;
      M.pos[tid][kk] = k;
      M.sc[tid][kk] = a.scale ? gload<float>(a.scale + (int64_t)s * a.K + k) : 1.0f;
      if (tid == 0) {
        M.a[kk] = ad;
        M.rk[kk] = adapter_rank(a, ad);
      }
      ++kk;
    }
    if (tid == 0) M.nact = kk;
  }
  lds_barrier();
}

// Zero the intermediate columns of the empty slots of every row of a tile
// (lora_shrink writes every column of a touched row).
__device__ inline void zero_empty_slots(const ApplyArgs &a, int row_lo, int row_hi, const Meta &M) {
  for (int e = threadIdx.x; e < (row_hi - row_lo) * a.K; e += blockDim.x) {
    const int m = row_lo + e / a.K, k = e % a.K;
    bool used = false;
    for (int kk = 0; kk < M.nact; ++kk) used |= (M.pos[m][kk] == k);
    if (!used) {
      float *vp = a.v + (int64_t)M.t[m] * a.ldv + (int64_t)k * a.r;
      for (int j = 0; j < a.r; ++j) gstore(vp + j, 0.f);
    }
  }
}

// Item q of a tile's items (in 0 .. cmo[ns] or cvo[ns]): its slice (the
// problem of the group), that slice's output width and the chunk's columns.
struct Chunk {
  int slice, d_out, o_lo, o_hi;
};
// The slice tables are read at constant indices only (an unrolled scan): an
// index known only at run time into the kernel's argument block makes the
// compiler copy the array to scratch memory.  NSL: the slices the build
// handles (1 for every launch but lora_apply_sliced's, which then keeps no
// scan in registers).  IS_M: 1 for the MFMA tiling's chunks, 0 for the VALU
// tiling's, -1 when only `is_m` knows.
template <int NSL = LORA_MAX_SLICES, int IS_M = -1>
__device__ inline Chunk chunk_of(const ApplyArgs &a, bool is_m, int q) {
  const bool m = IS_M < 0 ? is_m : IS_M == 1;
  Chunk c;
  c.slice = 0;
  c.d_out = a.sd_out[0];
  int base = 0, width = m ? a.wm[0] : a.wv[0];
#pragma unroll
  for (int p = 1; p < NSL; ++p) {
    const int off = m ? a.cmo[p] : a.cvo[p];
    if (p < a.ns && q >= off) {  // chunk offsets increase with p: the last match is q's slice
      c.slice = p;
      c.d_out = a.sd_out[p];
      base = off;
      width = m ? a.wm[p] : a.wv[p];
    }
  }
  c.o_lo = (q - base) * width;
  c.o_hi = min(c.d_out, c.o_lo + width);
  return c;
}

// Work items are (group, tile, slice, output chunk), in that order: the
// slices of a group that read one x take a tile's x in consecutive items.
// The items of one tile (every slice and chunk: `per_unit` of them) form a
// unit; blocks of up to kUnitBlock consecutive units (fewer when the launch
// has too few units for about eight blocks per XCD) are dealt round-robin over the
// XCDs (blockIdx % 8 is the XCD a workgroup is dispatched to), and an XCD's
// workgroups take its blocks' items in order.  Round-robin, because tiles of
// very different cost (a request with three stacked adapters runs three
// shrink and expand passes) sit next to each other in the plan's order and
// contiguous ranges per XCD left a few XCDs with all the long tiles; blocks of
// consecutive tiles, because those mostly share an adapter, which an XCD then
// stages into its L2 once per block rather than once per tile; whole units, so
// that the slices and chunks of a tile share one L2 (and its x).
// With `contiguous` (every unit costs about the same) each XCD takes one
// contiguous eighth of the units instead, so the tiles that share an adapter
// stay on one or two XCDs and the adapter is staged into that many L2s.
constexpr int kUnitBlock = 8;
template <class F>
__device__ inline void walk_items(int64_t n_items, int per_unit, F &&body, bool contiguous = false) {
  const int xcd = blockIdx.x & 7, lb = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  const int64_t n_units = (n_items + per_unit - 1) / per_unit;
  const int64_t blk = contiguous ? max<int64_t>(1, (n_units + 7) / 8)
                                 : min<int64_t>(kUnitBlock, max<int64_t>(1, n_units / 64));
  for (int64_t k = lb;; k += per_xcd) {
    const int64_t u = k / per_unit;  // the XCD's u-th unit
    const int64_t unit = (xcd + 8 * (u / blk)) * blk + u % blk;
    const int64_t item = unit * per_unit + k % per_unit;
    if (item >= n_items) break;
    body(item);
    lds_barrier();
  }
}

// Wave-wide sums of NV values per lane at once, as a butterfly
// reduce-scatter: step S halves the values a lane holds, keeping the half
// selected by lane bit S and adding the partner lane's copy of it.  After the
// log2(NV) halving steps an all-reduce over the remaining lane bits finishes
// the sum.  Lane l ends with the wave total of value (l % NV).
template <int S, int NV>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[NV], int lane) {
  const bool upper = (lane & S) != 0;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const float send = upper ? v[i] : v[i + S];
    const float keep = upper ? v[i + S] : v[i];
    v[i] = keep + __shfl_xor(send, S);
  }
}

template <int NV>
__device__ __forceinline__ float wave_sum_scatter(float (&v)[NV]) {
  const int lane = threadIdx.x & 63;
  if constexpr (NV >= 64) reduce_scatter_step<32>(v, lane);
  if constexpr (NV >= 32) reduce_scatter_step<16>(v, lane);
  if constexpr (NV >= 16) reduce_scatter_step<8>(v, lane);
  if constexpr (NV >= 8) reduce_scatter_step<4>(v, lane);
  if constexpr (NV >= 4) reduce_scatter_step<2>(v, lane);
  if constexpr (NV >= 2) reduce_scatter_step<1>(v, lane);
  float s = v[0];
#pragma unroll
  for (int off = NV; off < 64; off <<= 1) s += __shfl_xor(s, off);
  return s;
}

// RT consecutive outputs of one y row, held between a load and the
// read-modify-write that adds the result (rounded once to T): one vector
// access when the vector path allows it, else element by element.  p is a
// (wave-uniform) row base, off the byte offset of the first output.
template <typename T, bool VEC, int RT> struct YRun {
  static constexpr bool kVec = VEC && RT * sizeof(T) >= 4 && RT * sizeof(T) <= 16;
  typedef typename Raw<kVec ? RT * sizeof(T) : 4>::type R;
  R v[kVec ? 1 : RT];
  __device__ __forceinline__ void load(const T *p, uint32_t off) {
    if constexpr (kVec) {
      v[0] = gload_at<R>(p, off);
    } else {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        if constexpr (sizeof(T) == 2) v[i] = gload_at<uint16_t>(p, off + 2 * i);
        else v[i] = gload_at<uint32_t>(p, off + 4 * i);
      }
    }
  }
  __device__ __forceinline__ void add_store(T *p, uint32_t off, const float (&acc)[RT]) const {
    if constexpr (kVec) {
      constexpr int W = RT * sizeof(T) / 4;  // 32-bit words
      uint32_t w[W];
      if constexpr (W == 1) w[0] = v[0];
      else {
#pragma unroll
        for (int i = 0; i < W; ++i) w[i] = v[0][i];
      }
#pragma unroll
      for (int i = 0; i < W; ++i) {
        if constexpr (sizeof(T) == 2) w[i] = pack_bf2(bf_lo(w[i]) + acc[2 * i], bf_hi(w[i]) + acc[2 * i + 1]);
        else w[i] = __float_as_uint(__uint_as_float(w[i]) + acc[i]);
      }
      R o;
      if constexpr (W == 1) o = w[0];
      else {
#pragma unroll
        for (int i = 0; i < W; ++i) o[i] = w[i];
      }
      gstore_at(p, off, o);
    } else {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        if constexpr (sizeof(T) == 2) gstore_at(p, off + 2 * i, f_to_bf(bf_to_f(uint16_t(v[i])) + acc[i]));
        else gstore_at(p, off + 4 * i, __uint_as_float(v[i]) + acc[i]);
      }
    }
  }
};

// y[0 .. RT) += acc at byte offset off from p.
template <typename T, bool VEC, int RT>
__device__ __forceinline__ void add_store_rt(T *p, const float (&acc)[RT], uint32_t off = 0) {
  YRun<T, VEC, RT> y;
  y.load(p, off);
  y.add_store(p, off, acc);
}

}  // namespace lora
