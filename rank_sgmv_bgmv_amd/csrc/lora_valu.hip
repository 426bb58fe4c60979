// VALU apply kernel: decode (BGMV) tiles of up to 4 rows of one adapter group,
// plus every tile when the MFMA path does not apply (fp32, ranks other than
// 16/32/64/128, unaligned or odd sizes).  Computes y += scale * (x A_i^T) B_i^T
// for the tile's rows.
//
// "Serving several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
// alongside": the unmerged form adds x A^T B^T to x W^T; "Exercises" (four
// requests): the requests that share a LoRA form one group and get their own
// x A^T B^T, written back to their original rows.
//
// One workgroup per (problem, tile, output chunk).  A decode tile is a gather
// of one adapter's A and B with very little arithmetic per byte, so both
// phases are written to keep many independent 16-byte loads in flight:
// Shrink: each wave owns four rank rows of A per pass and its lanes split d_in
// into 16-byte pieces; the wave's partial sums are combined by a butterfly
// reduce-scatter over lanes (no LDS, no barrier) and land in LDS as the
// rank-r intermediate.  Expand: each thread owns short runs of consecutive
// outputs and the whole rank, streams those contiguous B rows, reads the
// intermediate from LDS as a broadcast, and updates y in place (loaded at
// the start of the round) with one vector access per run: no cross-lane
// reduction, no staging.

#include <type_traits>

#include "lora_device.hpp"

namespace lora {
namespace {

// ------------------------------------------------------------ VALU tile --
constexpr int kJPW = 4;  // rank rows a wave owns per pass of the VALU shrink

// Type of the intermediate kept in LDS: the fused bf16 vector path keeps it in
// bf16 (as the MFMA path does) so the expand multiplies packed pairs; every
// other path keeps fp32.
template <typename T, bool VEC, int MODE>
using InterT = typename std::conditional<MODE == MODE_FUSED && VEC && sizeof(T) == 2, uint16_t, float>::type;

// Shrink for MB rows (nb of them real): wave w owns rank rows j0 .. j0+3 of a
// pass, its lanes split d_in into 16-byte pieces (lane l takes pieces l,
// l+64, ...), UB pieces per lane per round for x and A each, so a round keeps
// UB*(MB+4) independent 16-byte loads in flight per lane.  Loads use clamped
// (always valid) addresses; pieces past the end are masked to zero.  The MB*4
// partial sums per lane are reduced over the wave by wave_sum_scatter (row by
// row); no LDS traffic and no barrier inside.
template <typename T, bool VEC, int MB, int MODE>
__device__ void valu_shrink(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const Meta &M,
                            InterT<T, VEC, MODE> *s_v) {
  typedef VOps<T, VEC> O;
  typedef typename O::V V;
  constexpr int E = O::E;
  constexpr int NV = MB * kJPW;
  constexpr int UB = MB <= 2 ? 4 : 2;
  const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
  const int r = a.r, d_in = a.d_in, KR = a.kr_max, nact = uniform(M.nact);
  const int nvx = d_in / E;
  const uint32_t row_bytes = uint32_t(d_in) * sizeof(T);
  const T *xrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    xrow[m] = static_cast<const T *>(pr.x) + (int64_t)uniform(M.t[m0 + (m < nb ? m : 0)]) * pr.ldx;

  for (int kk = 0; kk < nact; ++kk) {
    const T *Aa = static_cast<const T *>(pr.A) + (int64_t)uniform(M.a[kk]) * r * d_in;
    const int rk = uniform(M.rk[kk]);  // the adapter's rank: rows past it are not read, their sums are 0
    constexpr int kPass = (kValuThreads / 64) * kJPW;  // rank rows of a pass over the four waves
    for (int p0 = 0; p0 < r; p0 += kPass) {
      // this wave's rows of the pass: jb + js * i.  When the adapter's rank
      // covers the whole pass they are interleaved over the waves (rows w,
      // w + 4, w + 8, w + 12), which reads A faster than four consecutive rows
      // per wave; otherwise consecutive, so that waves past the rank skip it.
      const bool il = p0 + kPass <= rk;
      const int jb = il ? p0 + w : p0 + w * kJPW, js = il ? kValuThreads / 64 : 1;
      float acc[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = 0.f;
      for (int c0 = lane; c0 < (jb < rk ? nvx : 0); c0 += 64 * UB) {
        V xv[UB][MB], av[UB][kJPW];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int cv = c0 + 64 * u;
          const uint32_t off = uint32_t(min(cv, nvx - 1)) * (E * sizeof(T));
#pragma unroll
          for (int m = 0; m < MB; ++m) xv[u][m] = gload_at<V>(xrow[m], off);
#pragma unroll
          for (int i = 0; i < kJPW; ++i) av[u][i] = gload_at<V>(Aa, uint32_t(min(jb + js * i, rk - 1)) * row_bytes + off);
          if (cv >= nvx) {
#pragma unroll
            for (int m = 0; m < MB; ++m) xv[u][m] = O::zero();
          }
        }
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < kJPW; ++i) acc[m * kJPW + i] = O::dot(xv[u][m], av[u][i], acc[m * kJPW + i]);
      }
      // one reduction per row, so a row's sums do not depend on which other
      // rows share its tile (the plan's order inside an adapter group is not fixed)
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        float part[kJPW];
#pragma unroll
        for (int i = 0; i < kJPW; ++i) part[i] = acc[m * kJPW + i];
        const float val = wave_sum_scatter<kJPW>(part);
        const int j = jb + js * lane;
        if (lane < kJPW && m < nb && j < r) {
          const float vs = j < rk ? val * M.sc[m0 + m][kk] : 0.f;
          if constexpr (MODE == MODE_SHRINK)
            gstore(a.v + (int64_t)M.t[m0 + m] * a.ldv + (int64_t)M.pos[m0 + m][kk] * r + j, vs);
          else if constexpr (sizeof(InterT<T, VEC, MODE>) == 2)
            s_v[m * KR + kk * r + j] = f_to_bf(vs);
          else
            s_v[m * KR + kk * r + j] = vs;
        }
      }
    }
  }
}

// B vectors a lane keeps in flight per expand round: 16, halved for four rows
// and for an fp32 intermediate (which unpacks B to fp32 in registers).
template <int MB, int IT_BYTES>
constexpr int expand_nvb() { return (IT_BYTES == 2 ? 16 : 8) / (MB >= 4 ? 2 : 1); }

// Expand for MB rows.  A round gives each thread NBLK blocks of RT
// consecutive outputs (block b starts at o0 + b * 256 * RT), so one load
// instruction of the workgroup covers 256 * RT contiguous B rows and each lane
// reads a short contiguous run of RT rows (about 64 bytes: wider per-lane runs
// make every load instruction touch many more cache lines).  Each output is
// finished inside one lane: per slot the thread loads its B rows (up to NVB
// 16-byte vectors at once), multiplies them with the intermediate read from
// LDS (a broadcast: every lane reads the same address) and finally adds the
// result to the y values it loaded at the start of the round.
template <typename T, bool VEC, int MB, int RT, int NBLK, int MODE>
__device__ void valu_expand(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const Meta &M,
                            const InterT<T, VEC, MODE> *s_v, int o_lo, int o_hi, int d_out) {
  typedef VOps<T, VEC> O;
  typedef typename O::V V;
  typedef InterT<T, VEC, MODE> IT;
  constexpr int E = O::E;
  constexpr int NVB = expand_nvb<MB, sizeof(IT)>();  // B vectors in flight per lane per round
  constexpr int JB = NVB / (RT * NBLK) >= 1 ? NVB / (RT * NBLK) : 1;  // vectors per output row per round
  constexpr int BS = kValuThreads * RT;  // block stride (outputs)
  const int tid = threadIdx.x;
  const int r = a.r, KR = a.kr_max, nact = uniform(M.nact);
  const uint32_t brow_bytes = uint32_t(r) * sizeof(T);
  T *yrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    yrow[m] = static_cast<T *>(pr.y) + (int64_t)uniform(M.t[m0 + (m < nb ? m : 0)]) * pr.ldy;
  for (int o0 = o_lo + tid * RT; o0 < o_hi; o0 += BS * NBLK) {
    // blocks past o_hi load a valid row (the chunk's last RT rows) and store nothing
    int ob[NBLK];
#pragma unroll
    for (int b = 0; b < NBLK; ++b) ob[b] = min(o0 + b * BS, o_hi - RT);
    YRun<T, VEC, RT> yv[MB][NBLK];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
        if (m < nb) yv[m][b].load(yrow[m], uint32_t(ob[b]) * sizeof(T));
    float acc[MB][NBLK][RT];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
#pragma unroll
        for (int i = 0; i < RT; ++i) acc[m][b][i] = 0.f;
    for (int kk = 0; kk < nact; ++kk) {
      const T *Bk = static_cast<const T *>(pr.B) + (int64_t)uniform(M.a[kk]) * d_out * r;
      const IT *vk = s_v + kk * r;
      // vectors of B's row past the adapter's rank are not read (the
      // intermediate is zero there)
      const int nvk = (uniform(M.rk[kk]) + E - 1) / E;
      for (int jv0 = 0; jv0 < nvk; jv0 += JB) {
        V bv[NBLK][RT][JB];
#pragma unroll
        for (int b = 0; b < NBLK; ++b)
#pragma unroll
          for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int jj = 0; jj < JB; ++jj)
              bv[b][i][jj] = gload_at<V>(Bk, uint32_t(ob[b] + i) * brow_bytes +
                                                 uint32_t(min(jv0 + jj, nvk - 1)) * (E * sizeof(T)));
        // vectors past the rank contribute zero (the loads above stay unconditional,
        // so they are all in flight before the first multiply)
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          if (jv0 + jj >= nvk) {
#pragma unroll
            for (int b = 0; b < NBLK; ++b)
#pragma unroll
              for (int i = 0; i < RT; ++i) bv[b][i][jj] = O::zero();
          }
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m < nb) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
              const IT *vp = vk + m * KR + min(jv0 + jj, nvk - 1) * E;
              if constexpr (sizeof(IT) == 2) {
                const V vv = *reinterpret_cast<const V *>(vp);
#pragma unroll
                for (int b = 0; b < NBLK; ++b)
#pragma unroll
                  for (int i = 0; i < RT; ++i) acc[m][b][i] = O::dot(vv, bv[b][i][jj], acc[m][b][i]);
              } else {
#pragma unroll
                for (int b = 0; b < NBLK; ++b)
#pragma unroll
                  for (int i = 0; i < RT; ++i) acc[m][b][i] = O::dotf(vp, bv[b][i][jj], acc[m][b][i]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
        if (m < nb && o0 + b * BS < o_hi) yv[m][b].add_store(yrow[m], uint32_t(ob[b]) * sizeof(T), acc[m][b]);
  }
}

// Coalesced expand (vector path): B is [d_out][r]; the tile's slots use VPR
// 16-byte vectors of each row (VPR = 2, 4, 8 or 16: ranks 16 .. 128 in bf16,
// 8 .. 64 in fp32).  A wave's load instruction reads RPI = 64 / VPR whole
// rows -- lane l takes vector l % VPR of row l / VPR -- so, when the pool is
// stored at the tile's rank, every instruction reads 1 KB of consecutive
// memory (a lane reading a run of whole rows touches up to 64 cache lines
// per instruction).  Each lane multiplies its vector with the matching rank
// slice of the intermediate (from LDS); the VPR lanes of a row add their
// partial sums by lane exchanges; the row sums go through a per-wave LDS
// stage so that each lane updates 16 consecutive bytes of y with one load and
// one store.  A wave's round covers NI instructions (NI * RPI outputs).
constexpr int kExpandStage = 1024;  // fp32 staging slots per wave
constexpr size_t expand_stage_offset(int kr_max) { return (size_t(kRowBlock) * kr_max * 4 + 15) & ~size_t(15); }

template <typename T, int MB, int NI, int MODE>
__device__ void valu_expand_co(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const Meta &M,
                               const InterT<T, true, MODE> *s_v, int o_lo, int o_hi, int d_out, int vpr) {
  extern __shared__ __align__(16) unsigned char smem[];
  typedef VOps<T, true> O;
  typedef typename O::V V;
  typedef InterT<T, true, MODE> IT;
  constexpr int E = O::E;
  static_assert(MB * NI * 32 <= kExpandStage, "a round's sums fit the stage (VPR >= 2)");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane & (vpr - 1), rl = lane / vpr;
  const int rpi = 64 / vpr, wrows = NI * rpi, yv_lanes = wrows / E;
  const int r = a.r, KR = a.kr_max, nact = uniform(M.nact);
  const uint32_t brow_bytes = uint32_t(r) * sizeof(T);
  float *so = reinterpret_cast<float *>(smem + kMetaBytes + expand_stage_offset(KR)) + w * kExpandStage;
  T *yrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    yrow[m] = static_cast<T *>(pr.y) + (int64_t)uniform(M.t[m0 + (m < nb ? m : 0)]) * pr.ldy;
  for (int o0 = o_lo + w * wrows; o0 < o_hi; o0 += (kValuThreads / 64) * wrows) {
    // this lane's y vector (outputs oy .. oy+E-1), loaded first; lanes past
    // the round's outputs load a valid vector and store nothing
    const int oy = o0 + lane * E;
    const bool yok = lane < yv_lanes && oy < o_hi;
    const uint32_t yoff = uint32_t(min(oy, o_hi - E)) * sizeof(T);
    V yv[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) yv[m] = gload_at<V>(yrow[m], yoff);
    float acc[MB][NI];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[m][i] = 0.f;
    for (int kk = 0; kk < nact; ++kk) {
      const T *Bk = static_cast<const T *>(pr.B) + (int64_t)uniform(M.a[kk]) * d_out * r;
      V bv[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        bv[i] = gload_at<V>(Bk, uint32_t(min(o0 + i * rpi + rl, o_hi - 1)) * brow_bytes + uint32_t(q) * 16u);
      // vectors past the adapter's rank hold padding: never used (the
      // intermediate is zero there, and the padding need not be finite)
      if (q * E >= uniform(M.rk[kk])) {
#pragma unroll
        for (int i = 0; i < NI; ++i) bv[i] = O::zero();
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < nb) {
          const IT *vp = s_v + m * KR + kk * r + q * E;
          if constexpr (sizeof(IT) == 2) {
            const V vv = *reinterpret_cast<const V *>(vp);
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[m][i] = O::dot(vv, bv[i], acc[m][i]);
          } else {
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[m][i] = O::dotf(vp, bv[i], acc[m][i]);
          }
        }
      }
    }
    // row sums over the row's vpr lanes; lane q stages the sums of the
    // instructions i with i % vpr == q
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m < nb) {
        for (int bit = 1; bit < vpr; bit <<= 1) {
#pragma unroll
          for (int i = 0; i < NI; ++i) acc[m][i] += __shfl_xor(acc[m][i], bit);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
          if ((i & (vpr - 1)) == q) so[m * wrows + i * rpi + rl] = acc[m][i];
      }
    }
    // the stage is the wave's own: order its writes before its reads (and,
    // below, those reads before the next round's writes)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m < nb && yok) {
        float d[E];
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const float4 f = *reinterpret_cast<const float4 *>(so + m * wrows + lane * E + e);
          d[e] = f.x;
          d[e + 1] = f.y;
          d[e + 2] = f.z;
          d[e + 3] = f.w;
        }
        gstore_at(yrow[m], yoff, O::add(yv[m], d));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
}

// Outputs per block: rows of about 64 bytes per lane (counting the rank the
// tile uses), never more than the vector width, which divides d_out on the vector path (so a block never
// straddles the end of a row).  Blocks per round: about 16 B vectors per lane
// (8 with four rows).  The scalar path takes one output per thread.
template <typename T, bool VEC, int MB, int MODE, bool CO>
__device__ void valu_expand_rt(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const Meta &M,
                               const InterT<T, VEC, MODE> *s_v, int o_lo, int o_hi, int d_out) {
  constexpr int E = VOps<T, VEC>::E;
  if constexpr (!VEC) {
    valu_expand<T, VEC, MB, 1, 1, MODE>(a, pr, m0, nb, M, s_v, o_lo, o_hi, d_out);
    return;
  } else {
    // sized by the largest rank among the tile's slots, not the pool's stored
    // rank: with small adapters in a pool stored at a larger rank, a lane then
    // takes more output rows instead of repeating loads past the rank
    int kr = 1;
    for (int kk = 0; kk < M.nact; ++kk) kr = max(kr, M.rk[kk]);
    const int vpr = (uniform(kr) + E - 1) / E;
    // Tiles whose rows stack several adapters take the coalesced expand when
    // their slots use 2 .. 16 vectors of each row of B (measured: 5% faster on
    // the stacked decode; one-adapter tiles run faster on the runs below)
    if constexpr (CO) {
      constexpr int NI = MB >= 4 ? 8 : 16;
      if (M.nact >= 2 && vpr >= 2 && vpr <= NI && (vpr & (vpr - 1)) == 0 && vpr * E <= a.r) {
        valu_expand_co<T, MB, NI, MODE>(a, pr, m0, nb, M, s_v, o_lo, o_hi, d_out, vpr);
        return;
      }
    }
    const int row_bytes = vpr * E * int(sizeof(T));
    const int rt = min(max(64 / row_bytes, 1), E);
    int nblk = expand_nvb<MB, sizeof(InterT<T, VEC, MODE>)>() / (rt * vpr);
    nblk = nblk >= 4 ? 4 : nblk >= 2 ? 2 : 1;
    while (nblk > 1 && MB * rt * nblk > 16) nblk >>= 1;  // at most 16 accumulators per lane
    // only the (RT, NBLK) pairs within the accumulator budget are compiled
#define LORA_EXPAND(RT_, NB_)                                                           \
  if constexpr (MB * RT_ * NB_ <= 16) {                                                 \
    if (rt == RT_ && nblk == NB_) {                                                     \
      valu_expand<T, VEC, MB, RT_, NB_, MODE>(a, pr, m0, nb, M, s_v, o_lo, o_hi, d_out);\
      return;                                                                           \
    }                                                                                   \
  }
    LORA_EXPAND(4, 4) LORA_EXPAND(4, 2) LORA_EXPAND(4, 1) LORA_EXPAND(2, 4) LORA_EXPAND(2, 2)
    LORA_EXPAND(2, 1) LORA_EXPAND(1, 4) LORA_EXPAND(1, 2)
#undef LORA_EXPAND
    valu_expand<T, VEC, MB, 1, 1, MODE>(a, pr, m0, nb, M, s_v, o_lo, o_hi, d_out);
  }
}

// Rows row_lo .. row_hi-1 of a tile, in blocks of kRowBlock rows.
template <typename T, bool VEC, int MODE, bool CO>
__device__ void valu_tile(const ApplyArgs &a, const lora_problem &pr, int row_lo, int row_hi, int o_lo, int o_hi,
                          int d_out, Meta &M, InterT<T, VEC, MODE> *s_v) {
  const int tid = threadIdx.x;
  const int r = a.r, KR = a.kr_max, nact = M.nact;
  if (MODE == MODE_SHRINK) zero_empty_slots(a, row_lo, row_hi, M);
  for (int m0 = row_lo; m0 < row_hi; m0 += kRowBlock) {
    const int nb = min(kRowBlock, row_hi - m0);
    if (MODE != MODE_EXPAND) {
      if (nb <= 1) valu_shrink<T, VEC, 1, MODE>(a, pr, m0, nb, M, s_v);
      else if (nb <= 2) valu_shrink<T, VEC, 2, MODE>(a, pr, m0, nb, M, s_v);
      else valu_shrink<T, VEC, 4, MODE>(a, pr, m0, nb, M, s_v);
    } else {
      // expand only: the caller's intermediate (compacted slots) into LDS
      for (int w = tid; w < nb * nact * r; w += kValuThreads) {
        const int m = w / (nact * r), rem = w % (nact * r), kk = rem / r, j = rem % r;
        s_v[m * KR + kk * r + j] =
            j < M.rk[kk] ? gload<float>(a.v + (int64_t)M.t[m0 + m] * a.ldv + (int64_t)M.pos[m0 + m][kk] * r + j) : 0.f;
      }
    }
    if (MODE == MODE_SHRINK) continue;
    lds_barrier();  // the intermediate of this row block is complete
    if (nb <= 1) valu_expand_rt<T, VEC, 1, MODE, CO>(a, pr, m0, nb, M, s_v, o_lo, o_hi, d_out);
    else if (nb <= 2) valu_expand_rt<T, VEC, 2, MODE, CO>(a, pr, m0, nb, M, s_v, o_lo, o_hi, d_out);
    else valu_expand_rt<T, VEC, 4, MODE, CO>(a, pr, m0, nb, M, s_v, o_lo, o_hi, d_out);
    lds_barrier();  // before the next row block overwrites the intermediate
  }
}

// ---------------------------------------------------------------- kernel --
// Occupancy: the fused bf16 single-slice build takes about 200 VGPRs, so a
// SIMD holds two waves and a CU two workgroups.  That is kept on purpose:
// holding the kernel to 168 VGPRs (three waves) makes the compiler spill its
// loads in flight and hoisted addresses to scratch, and the 32-layer decode
// launch then runs about 10% slower (1.5x at 128 VGPRs, four waves).
// NSL: the output slices the build handles (LORA_MAX_SLICES for
// lora_apply_sliced's launches, 1 for all others).
template <typename T, bool VEC, int MODE, int NSL>
__global__ __launch_bounds__(kValuThreads) void valu_kernel(ApplyArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Meta &M = *reinterpret_cast<Meta *>(smem);
  InterT<T, VEC, MODE> *s_v = reinterpret_cast<InterT<T, VEC, MODE> *>(smem + kMetaBytes);
  const PlanHdr ph = read_plan_header(a);
  if (!ph.ok) return;
  const int n_m = ph.n_m, n_v = ph.n_v, n_active = ph.n_active;
  // VALU tiles first; MFMA-sized tiles too when the MFMA kernel does not run,
  // each as kSubBlocks items of kRowBlock rows (one workgroup would otherwise
  // take a 64-row tile's row blocks one after another).  A tile's items run
  // over every slice of the group (per_v / per_m of them per row block).
  constexpr int kSubBlocks = kMfmaRows / kRowBlock;
  const int per_v = a.items_v_tile, per_m = a.items_m_tile * kSubBlocks;
  const int64_t items_v = (int64_t)n_v * per_v;
  const int64_t items_m = a.valu_takes_m ? (int64_t)n_m * per_m : 0;
  const int64_t per_grp = items_v + items_m;
  const int64_t n_items = per_grp * a.n_problems;
  if (n_items <= 0) return;
  // Work items are dealt in XCD-contiguous ranges (blockIdx % 8 is the XCD):
  // the chunks of a tile and the neighbouring tiles of one problem share that
  // XCD's L2; the workgroups of an XCD stride through its range.
  const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
  const int64_t ipx = (n_items + 7) >> 3;
  auto item_at = [&](int64_t i) -> int64_t {
    if (i >= ipx) return -1;
    const int64_t it = xcd * ipx + i;
    return it < n_items ? it : -1;
  };
  // What an item needs before it starts -- where it lies, its problem and, for
  // a VALU tile, its record -- is loaded one item ahead, so a workgroup's next
  // item begins without a round trip to memory.
  struct Ahead {
    lora_problem pr;
    int tile, q, word, sb;  // tile, item within the tile (slice and chunk), record word, row block
    bool is_m;
  };
  auto load_ahead = [&](int64_t it, Ahead &h) {
    const int g = int(it / per_grp);
    int64_t rem = it - (int64_t)g * per_grp;
    h.is_m = rem >= items_v;
    if (h.is_m) rem -= items_v;
    const int per = h.is_m ? per_m : per_v;
    h.tile = int(rem / per);
    h.q = int(rem - (int64_t)h.tile * per);
    // tiles in reverse plan order: requests with several adapters (the
    // longest tiles) come last in the plan and should start first
    h.tile = (h.is_m ? n_m : n_v) - 1 - h.tile;
    h.sb = 0;
    if (h.is_m) {  // an MFMA-sized tile: row block, then slice and chunk
      h.sb = h.q / a.items_m_tile;
      h.q -= h.sb * a.items_m_tile;
    }
    const int slice = chunk_of<NSL>(a, h.is_m, h.q).slice;
    h.pr = a.probs ? gload<lora_problem>(a.probs + (int64_t)g * a.ns + slice) : a.single;
    h.word = 0;
    if (!h.is_m && threadIdx.x < kRecWords) h.word = gload<int>(a.vrec + (int64_t)h.tile * kRecWords + threadIdx.x);
  };
  int64_t i = blockIdx.x >> 3;
  int64_t it = item_at(i);
  if (it < 0) return;
  Ahead cur;
  load_ahead(it, cur);
  while (it >= 0) {
    const int64_t nx = item_at(i + per_xcd);
    Ahead nxt;
    nxt.word = 0;
    if (nx >= 0) load_ahead(nx, nxt);
    const Chunk c = chunk_of<NSL>(a, cur.is_m, cur.q);
    const int o_lo = c.o_lo, o_hi = c.o_hi;
    int row_lo = 0, row_hi;
    if (cur.is_m) {
      const int4 td = gload<int4>(a.tiles_m + cur.tile);
      setup_rows(a, td, n_active, M);
      row_lo = cur.sb * kRowBlock;
      row_hi = min(td.z, row_lo + kRowBlock);
    } else {
      row_hi = setup_from_record(a, cur.word, M);
    }
    if (M.nact > 0 && row_lo < row_hi && (MODE == MODE_SHRINK || o_lo < o_hi))
      valu_tile<T, VEC, MODE, MODE == MODE_FUSED && NSL == 1>(a, cur.pr, row_lo, row_hi, o_lo, o_hi, c.d_out, M, s_v);
    lds_barrier();
    it = nx;
    i += per_xcd;
    cur = nxt;
  }
}

// Launch one instantiation; the first launch lifts its dynamic-LDS limit to
// the 160 KB a gfx950 workgroup may use.
template <typename T, bool VEC, int M, int NSL>
hipError_t launch_one(const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  static const bool lds_limit_raised =
      raise_lds_limit(reinterpret_cast<const void *>(&valu_kernel<T, VEC, M, NSL>), kMaxLdsBytes);
  (void)lds_limit_raised;
  hipLaunchKernelGGL((valu_kernel<T, VEC, M, NSL>), dim3(grid), dim3(kValuThreads), smem, stream, a);
  return hipGetLastError();
}

// Launches with several output slices are fused ones (lora_apply_sliced).
template <typename T, bool VEC>
hipError_t launch_mode(int mode, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  if (a.ns > 1)
    return mode == MODE_FUSED ? launch_one<T, VEC, MODE_FUSED, LORA_MAX_SLICES>(a, grid, smem, stream)
                              : hipErrorInvalidValue;
  switch (mode) {
    case MODE_FUSED: return launch_one<T, VEC, MODE_FUSED, 1>(a, grid, smem, stream);
    case MODE_SHRINK: return launch_one<T, VEC, MODE_SHRINK, 1>(a, grid, smem, stream);
    case MODE_EXPAND: return launch_one<T, VEC, MODE_EXPAND, 1>(a, grid, smem, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t valu_smem_bytes(int kr_max) {
  return kMetaBytes + expand_stage_offset(kr_max) + size_t(kValuThreads / 64) * kExpandStage * 4;
}

hipError_t launch_valu(int mode, int dtype, bool vec, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  if (dtype == LORA_F32)
    return vec ? launch_mode<float, true>(mode, a, grid, smem, stream) : launch_mode<float, false>(mode, a, grid, smem, stream);
  return vec ? launch_mode<uint16_t, true>(mode, a, grid, smem, stream)
             : launch_mode<uint16_t, false>(mode, a, grid, smem, stream);
}

}  // namespace lora
