// VALU apply kernel: decode (BGMV) tiles of up to 16 rows, plus every tile when
// the MFMA path does not apply (fp32, ranks other than 16/32/64/128, unaligned
// or odd sizes).  Computes y += scale * (x A_i^T) B_i^T for the tile's rows.
//
// "Serving several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
// alongside": the unmerged form adds x A^T B^T to x W^T; "Exercises" (four
// requests): the requests that share a LoRA form one group and get their own
// x A^T B^T, written back to their original rows.
//
// Shrink: each wave owns four rank rows of A per pass and its lanes split d_in
// into 16-byte pieces, several pieces of A and x in flight per lane; the wave's
// partial sums are combined by a butterfly reduce-scatter over lanes (no LDS,
// no barrier) and land in LDS as the fp32 rank-r intermediate.  Expand: each
// thread owns a few consecutive outputs and the whole rank, streams those
// contiguous B rows with 16-byte loads, reads the intermediate from LDS as a
// broadcast, and updates y in place with one vector access per row: no
// cross-lane reduction, no staging.

#include "lora_device.hpp"

namespace lora {
namespace {

// ------------------------------------------------------------ VALU tile --
constexpr int kJPW = 4;  // rank rows a wave owns per pass of the VALU shrink

// Shrink for MB rows (nb of them real): wave w owns rank rows j0 .. j0+3 of a
// pass, its lanes split d_in into 16-byte pieces (lane l takes pieces l,
// l+64, ...), UB pieces per lane per round for x and A each, so a round keeps
// UB*(MB+4) independent 16-byte loads in flight per lane.  The MB*4 partial
// sums per lane are reduced over the wave by wave_sum_scatter; no LDS traffic
// and no barrier inside.
template <typename T, bool VEC, int MB, int MODE>
__device__ void valu_shrink(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const Meta &M,
                            float *s_v) {
  typedef VOps<T, VEC> O;
  typedef typename O::V V;
  constexpr int E = O::E;
  constexpr int NV = MB * kJPW;
  constexpr int UB = MB <= 2 ? 4 : 2;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = a.r, d_in = a.d_in, KR = a.kr_max, nact = uniform(M.nact);
  const int nvx = d_in / E;
  const T *__restrict__ Ab = static_cast<const T *>(pr.A);
  const T *xrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    xrow[m] = static_cast<const T *>(pr.x) + (int64_t)uniform(M.t[m0 + (m < nb ? m : 0)]) * pr.ldx;

  for (int kk = 0; kk < nact; ++kk) {
    const T *__restrict__ Aa = Ab + (int64_t)uniform(M.a[kk]) * r * d_in;
    for (int j0 = w * kJPW; j0 < r; j0 += 4 * kJPW) {
      float acc[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = 0.f;
      for (int c0 = lane; c0 < nvx; c0 += 64 * UB) {
        V xv[UB][MB], av[UB][kJPW];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int cv = c0 + 64 * u;
          const bool ok = cv < nvx;
#pragma unroll
          for (int m = 0; m < MB; ++m) xv[u][m] = (ok && m < nb) ? O::load(xrow[m] + (int64_t)cv * E) : O::zero();
#pragma unroll
          for (int i = 0; i < kJPW; ++i)
            av[u][i] = (ok && j0 + i < r) ? O::load(Aa + (int64_t)(j0 + i) * d_in + (int64_t)cv * E) : O::zero();
        }
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
          for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < kJPW; ++i) acc[m * kJPW + i] = O::dot(xv[u][m], av[u][i], acc[m * kJPW + i]);
      }
      const float val = wave_sum_scatter<NV>(acc);
      if (lane < NV) {
        const int m = lane / kJPW, j = j0 + lane % kJPW;
        if (m < nb && j < r) {
          const float vs = val * M.sc[m0 + m][kk];
          if (MODE == MODE_SHRINK)
            gstore(a.v + (int64_t)M.t[m0 + m] * a.ldv + (int64_t)M.pos[m0 + m][kk] * r + j, vs);
          else
            s_v[m * KR + kk * r + j] = vs;
        }
      }
    }
  }
}

// Expand for MB rows: thread owns RT consecutive outputs o .. o+RT-1 and all
// of the rank, so each output is finished inside one lane (no cross-lane
// reduction, no staging): per slot it loads the RT contiguous B rows
// (RT * rank elements) in rounds of 16 vectors, multiplies them with the
// intermediate read from LDS (a broadcast: every lane reads the same address)
// and finally adds the result to y with one vector access per row.
template <typename T, bool VEC, int MB, int RT>
__device__ void valu_expand(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const Meta &M,
                            const float *s_v, int o_lo, int o_hi) {
  typedef VOps<T, VEC> O;
  typedef typename O::V V;
  constexpr int E = O::E;
  constexpr int NVB = MB >= 4 ? 8 : 16;  // B vectors in flight per lane per round
  constexpr int JB = NVB / RT >= 1 ? NVB / RT : 1;  // vectors per output row per round
  const int tid = threadIdx.x;
  const int r = a.r, d_out = a.d_out, KR = a.kr_max, nact = uniform(M.nact);
  const int nvr = r / E;
  const T *__restrict__ Bb = static_cast<const T *>(pr.B);
  T *yrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    yrow[m] = static_cast<T *>(pr.y) + (int64_t)uniform(M.t[m0 + (m < nb ? m : 0)]) * pr.ldy;
  for (int o = o_lo + tid * RT; o < o_hi; o += kThreads * RT) {
    float acc[MB][RT];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int i = 0; i < RT; ++i) acc[m][i] = 0.f;
    for (int kk = 0; kk < nact; ++kk) {
      const T *__restrict__ Bk = Bb + (int64_t)uniform(M.a[kk]) * d_out * r;
      const float *vk = s_v + kk * r;
      for (int jv0 = 0; jv0 < nvr; jv0 += JB) {
        V bv[RT][JB];
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int jj = 0; jj < JB; ++jj)
            bv[i][jj] = (jv0 + jj < nvr) ? O::load(Bk + (o + i) * r + (jv0 + jj) * E) : O::zero();
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m < nb) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
              if (jv0 + jj < nvr) {
                const float *vp = vk + m * KR + (jv0 + jj) * E;
#pragma unroll
                for (int i = 0; i < RT; ++i) acc[m][i] = O::dotf(vp, bv[i][jj], acc[m][i]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
      if (m < nb) add_store_rt<T, VEC, RT>(yrow[m] + o, acc[m]);
  }
}

template <typename T, bool VEC, int MB>
__device__ void valu_expand_rt(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const Meta &M,
                               const float *s_v, int o_lo, int o_hi) {
  // outputs per thread: enough that a thread's B rows fill 8 vectors, at most
  // 16 accumulators (MB rows x RT outputs) per lane, and never more than the
  // vector width, which divides d_out on the vector path (so an RT-group never
  // straddles the end of a row).  The scalar path takes one output per thread.
  constexpr int E = VOps<T, VEC>::E;
  if constexpr (!VEC) {
    valu_expand<T, VEC, MB, 1>(a, pr, m0, nb, M, s_v, o_lo, o_hi);
    return;
  }
  const int q = min(min((16 * E) / a.r, 32 / MB), E);
  if (q >= 8) valu_expand<T, VEC, MB, 8>(a, pr, m0, nb, M, s_v, o_lo, o_hi);
  else if (q >= 4) valu_expand<T, VEC, MB, 4>(a, pr, m0, nb, M, s_v, o_lo, o_hi);
  else if (q >= 2) valu_expand<T, VEC, MB, 2>(a, pr, m0, nb, M, s_v, o_lo, o_hi);
  else valu_expand<T, VEC, MB, 1>(a, pr, m0, nb, M, s_v, o_lo, o_hi);
}

template <typename T, bool VEC, int MODE>
__device__ void valu_tile(const ApplyArgs &a, const lora_problem &pr, int nrows, int o_lo, int o_hi, Meta &M,
                          float *s_v) {
  const int tid = threadIdx.x;
  const int r = a.r, KR = a.kr_max, nact = M.nact;
  if (MODE == MODE_SHRINK) zero_empty_slots(a, nrows, M);
  for (int m0 = 0; m0 < nrows; m0 += kRowBlock) {
    const int nb = min(kRowBlock, nrows - m0);
    if (MODE != MODE_EXPAND) {
      if (nb <= 1) valu_shrink<T, VEC, 1, MODE>(a, pr, m0, nb, M, s_v);
      else if (nb <= 2) valu_shrink<T, VEC, 2, MODE>(a, pr, m0, nb, M, s_v);
      else valu_shrink<T, VEC, 4, MODE>(a, pr, m0, nb, M, s_v);
    } else {
      // expand only: the caller's intermediate (compacted slots) into LDS
      for (int w = tid; w < nb * nact * r; w += kThreads) {
        const int m = w / (nact * r), rem = w % (nact * r), kk = rem / r, j = rem % r;
        s_v[m * KR + kk * r + j] = gload<float>(a.v + (int64_t)M.t[m0 + m] * a.ldv + (int64_t)M.pos[m0 + m][kk] * r + j);
      }
    }
    if (MODE == MODE_SHRINK) continue;
    __syncthreads();  // the intermediate of this row block is complete
    if (nb <= 1) valu_expand_rt<T, VEC, 1>(a, pr, m0, nb, M, s_v, o_lo, o_hi);
    else if (nb <= 2) valu_expand_rt<T, VEC, 2>(a, pr, m0, nb, M, s_v, o_lo, o_hi);
    else valu_expand_rt<T, VEC, 4>(a, pr, m0, nb, M, s_v, o_lo, o_hi);
    __syncthreads();  // before the next row block overwrites the intermediate
  }
}

// ---------------------------------------------------------------- kernel --
// At least four waves per SIMD (<= 128 VGPRs): the per-tile phases are short
// dependent chains, and occupancy is what overlaps them.
template <typename T, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void valu_kernel(ApplyArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Meta &M = *reinterpret_cast<Meta *>(smem);
  float *s_v = reinterpret_cast<float *>(smem + kMetaBytes);
  const int n_m = gload<int>(a.hdr + H_TILES_M), n_v = gload<int>(a.hdr + H_TILES_V);
  const int n_active = gload<int>(a.hdr + H_ACTIVE);
  // VALU tiles first; MFMA-sized tiles too when the MFMA kernel does not run
  const int64_t items_v = a.valu_skip_v ? 0 : (int64_t)n_v * a.cv;
  const int64_t items_m = a.valu_takes_m ? (int64_t)n_m * a.cm : 0;
  const int64_t per_prob = items_v + items_m;
  walk_items(per_prob * a.n_problems, [&](int64_t item) {
    const int p = int(item / per_prob);
    int64_t rem = item - (int64_t)p * per_prob;
    const bool is_m = rem >= items_v;
    if (is_m) rem -= items_v;
    const int chunks = is_m ? a.cm : a.cv, width = is_m ? a.wm : a.wv;
    const int tile = int(rem / chunks), chunk = int(rem % chunks);
    const lora_problem pr = a.probs ? gload<lora_problem>(a.probs + p) : a.single;
    const int4 td = gload<int4>(is_m ? a.tiles_m + tile : a.tiles_v + tile);
    const int o_lo = chunk * width, o_hi = min(a.d_out, o_lo + width);
    setup_rows(a, td, is_m ? nullptr : a.rowrec + (int64_t)tile * kValuRows, n_active, M);
    if (M.nact > 0 && (MODE == MODE_SHRINK || o_lo < o_hi)) valu_tile<T, VEC, MODE>(a, pr, td.z, o_lo, o_hi, M, s_v);
  });
}

// Launch one instantiation; the first launch lifts its dynamic-LDS limit to
// the 160 KB a gfx950 workgroup may use.
template <typename T, bool VEC, int M>
hipError_t launch_one(const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  static const bool lds_limit_raised =
      hipFuncSetAttribute(reinterpret_cast<const void *>(&valu_kernel<T, VEC, M>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes) == hipSuccess;
  (void)lds_limit_raised;
  hipLaunchKernelGGL((valu_kernel<T, VEC, M>), dim3(grid), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

template <typename T, bool VEC>
hipError_t launch_mode(int mode, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  switch (mode) {
    case MODE_FUSED: return launch_one<T, VEC, MODE_FUSED>(a, grid, smem, stream);
    case MODE_SHRINK: return launch_one<T, VEC, MODE_SHRINK>(a, grid, smem, stream);
    case MODE_EXPAND: return launch_one<T, VEC, MODE_EXPAND>(a, grid, smem, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t valu_smem_bytes(int kr_max) { return kMetaBytes + size_t(kRowBlock) * kr_max * 4; }

hipError_t launch_valu(int mode, int dtype, bool vec, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  if (dtype == LORA_F32)
    return vec ? launch_mode<float, true>(mode, a, grid, smem, stream) : launch_mode<float, false>(mode, a, grid, smem, stream);
  return vec ? launch_mode<uint16_t, true>(mode, a, grid, smem, stream)
             : launch_mode<uint16_t, false>(mode, a, grid, smem, stream);
}

}  // namespace lora
