// Decode (BGMV) fused apply: one wave per (problem, small tile, output chunk).
//
// "Serving several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
// alongside": the unmerged form adds x A^T B^T to x W^T; "Exercises" (four
// requests): requests that share a LoRA form one group, each group gets its own
// x A^T B^T, written back to the original rows.  "Punica: Multi-Tenant LoRA
// Serving", contribution 1: the decode case is the gather matrix-vector
// product -- every token gathers its adapter's A and B.
//
// A decode tile has 1..16 rows of one adapter group, so its work is a gather of
// that adapter's A (r x d_in) and B (d_out x r): a memory-bound stream with
// very little arithmetic per byte.  What keeps HBM busy is the number of
// independent loads in flight, so the unit of work is a single wave with no
// barrier and no sharing: thousands of them are resident at once and their
// short dependent chains (setup -> shrink -> expand) overlap.
//
//   setup   lanes 0..rows-1 read their (token row, request) record and the
//           request's slots; the compacted slots, the scales and the token
//           rows go to a small per-wave LDS area.
//   shrink  per slot and pass of JW rank rows: lanes split d_in into 16-byte
//           pieces of x and A (coalesced along the row), the wave's MB*JW
//           partial sums are combined by a butterfly reduce-scatter across
//           lanes, scaled and parked in the wave's LDS as the fp32 rank-r
//           intermediate.
//   expand  each lane owns RT consecutive outputs and the whole rank: it
//           streams those RT contiguous B rows with 16-byte loads, reads the
//           intermediate as an LDS broadcast, and updates y with one vector
//           access per row; every output is finished inside one lane.

#include "lora_device.hpp"

namespace lora {
namespace {

constexpr int kWaves = kDecodeWaves;

// Per-wave metadata of one tile (kValuRows rows at most).
struct WaveMeta {
  int t[kValuRows];                     // token row
  int a[LORA_MAX_SLOTS];                // adapters of the compacted slots
  int nact;
  int pad[3];
  float sc[kValuRows][LORA_MAX_SLOTS];  // scale of compacted slot
};
constexpr size_t kWaveMetaBytes = (sizeof(WaveMeta) + 15) & ~size_t(15);

// Make LDS writes of some lanes visible to the other lanes of the same wave:
// the wave's LDS operations complete in order, so only the compiler has to be
// kept from moving accesses across this point.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lanes 0..nrows-1 fill the wave's metadata.
__device__ inline void wave_setup(const ApplyArgs &a, const int2 *rec, int nrows, WaveMeta &W) {
  const int lane = threadIdx.x & 63;
  if (lane < nrows) {
    const int2 rr = gload<int2>(rec + lane);
    W.t[lane] = rr.x;
    const int s = rr.y;
    int kk = 0;
    for (int k = 0; k < a.K; ++k) {
      const int ad = gload<int>(a.idx + (int64_t)s * a.K + k);
      if (ad < 0 || ad >= a.n) continue;
      W.sc[lane][kk] = a.scale ? gload<float>(a.scale + (int64_t)s * a.K + k) : 1.0f;
      if (lane == 0) W.a[kk] = ad;
      ++kk;
    }
    if (lane == 0) W.nact = kk;
  }
  wave_sync();
}

// Shrink of MB rows (nb real) for every slot: wv[m][kk*r + j] = sc * sum_c x[t_m][c] A_kk[j][c],
// accumulated in fp32 and kept in the activation type.
template <typename T, int MB, int JW>
__device__ void wave_shrink(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const WaveMeta &W, T *wv) {
  typedef VOps<T, true> O;
  typedef typename O::V V;
  constexpr int E = O::E;
  constexpr int NV = MB * JW;
  const int lane = threadIdx.x & 63;
  const int r = a.r, d_in = a.d_in, KR = a.kr_max, nact = uniform(W.nact);
  const int nvx = d_in / E;
  const T *xrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    xrow[m] = static_cast<const T *>(pr.x) + (int64_t)uniform(W.t[m0 + (m < nb ? m : 0)]) * pr.ldx;
  const uint32_t row_bytes = uint32_t(d_in) * sizeof(T);
  for (int kk = 0; kk < nact; ++kk) {
    const T *Aa = static_cast<const T *>(pr.A) + (int64_t)uniform(W.a[kk]) * r * d_in;
    for (int j0 = 0; j0 < r; j0 += JW) {
      float acc[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = 0.f;
      for (int cv = lane; cv < nvx; cv += 64) {
        const uint32_t off = uint32_t(cv) * 16u;
        V xv[MB], av[JW];
#pragma unroll
        for (int m = 0; m < MB; ++m) xv[m] = gload_at<V>(xrow[m], off);
#pragma unroll
        for (int j = 0; j < JW; ++j) av[j] = gload_at<V>(Aa, uint32_t(min(j0 + j, r - 1)) * row_bytes + off);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int j = 0; j < JW; ++j) acc[m * JW + j] = O::dot(xv[m], av[j], acc[m * JW + j]);
      }
      const float val = wave_sum_scatter<NV>(acc);
      if (lane < NV) {
        const int m = lane / JW, j = j0 + lane % JW;
        if (m < nb && j < r) {
          const float sv = val * W.sc[m0 + m][kk];
          if constexpr (sizeof(T) == 2) wv[m * KR + kk * r + j] = f_to_bf(sv);
          else wv[m * KR + kk * r + j] = sv;
        }
      }
    }
  }
  wave_sync();
}

// Expand of MB rows: lane owns outputs o .. o+RT-1 (RT consecutive B rows).
template <typename T, int MB, int RT>
__device__ void wave_expand(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const WaveMeta &W,
                            const T *wv, int o_lo, int o_hi) {
  typedef VOps<T, true> O;
  typedef typename O::V V;
  constexpr int E = O::E;
  constexpr int NVB = 8;                          // B vectors per lane per round
  constexpr int JB = NVB / RT >= 1 ? NVB / RT : 1;
  const int lane = threadIdx.x & 63;
  const int r = a.r, d_out = a.d_out, KR = a.kr_max, nact = uniform(W.nact);
  const int nvr = r / E;
  T *yrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    yrow[m] = static_cast<T *>(pr.y) + (int64_t)uniform(W.t[m0 + (m < nb ? m : 0)]) * pr.ldy;
  const uint32_t brow_bytes = uint32_t(r) * sizeof(T);
  for (int o = o_lo + lane * RT; o < o_hi; o += 64 * RT) {
    float acc[MB][RT];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int i = 0; i < RT; ++i) acc[m][i] = 0.f;
    for (int kk = 0; kk < nact; ++kk) {
      const T *Bk = static_cast<const T *>(pr.B) + (int64_t)uniform(W.a[kk]) * d_out * r;
      for (int jv0 = 0; jv0 < nvr; jv0 += JB) {
        V bv[RT][JB];
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int jj = 0; jj < JB; ++jj)
            bv[i][jj] = gload_at<V>(Bk, uint32_t(o + i) * brow_bytes + uint32_t(min(jv0 + jj, nvr - 1)) * 16u);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m < nb) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
              if (jv0 + jj < nvr) {
                const V vv = *reinterpret_cast<const V *>(wv + m * KR + kk * r + (jv0 + jj) * E);
#pragma unroll
                for (int i = 0; i < RT; ++i) acc[m][i] = O::dot(vv, bv[i][jj], acc[m][i]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
      if (m < nb) add_store_rt<T, true, RT>(yrow[m], acc[m], uint32_t(o) * sizeof(T));
  }
}

template <typename T, int MB>
__device__ void wave_rows(const ApplyArgs &a, const lora_problem &pr, int m0, int nb, const WaveMeta &W, T *wv,
                          int o_lo, int o_hi) {
  constexpr int E = VOps<T, true>::E;
  // rank rows per shrink pass: MB*JW <= 16 partial sums per lane
  constexpr int JW = MB <= 1 ? 16 : 16 / MB;
  wave_shrink<T, MB, JW>(a, pr, m0, nb, W, wv);
  // outputs per lane: B rows of 8 vectors, <= 16 accumulators, <= the vector width
  const int q = min(min((8 * E) / a.r, 16 / MB), E);
  if (q >= 8) wave_expand<T, MB, 8>(a, pr, m0, nb, W, wv, o_lo, o_hi);
  else if (q >= 4) wave_expand<T, MB, 4>(a, pr, m0, nb, W, wv, o_lo, o_hi);
  else if (q >= 2) wave_expand<T, MB, 2>(a, pr, m0, nb, W, wv, o_lo, o_hi);
  else wave_expand<T, MB, 1>(a, pr, m0, nb, W, wv, o_lo, o_hi);
  wave_sync();
}

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(ApplyArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int w = uniform(threadIdx.x >> 6);
  const size_t per_wave = kWaveMetaBytes + size_t(kRowBlock) * a.kr_max * sizeof(T);
  WaveMeta &W = *reinterpret_cast<WaveMeta *>(smem + w * per_wave);
  T *wv = reinterpret_cast<T *>(smem + w * per_wave + kWaveMetaBytes);

  // item counts fit in 32 bits (checked by the host)
  const int n_v = gload<int>(a.hdr + H_TILES_V);
  const int per_prob = n_v * a.cv;
  const int n_items = per_prob * a.n_problems;
  if (n_items <= 0) return;
  // XCD-contiguous item ranges (blockIdx % 8 is the XCD), waves of an XCD stride through them
  const int xcd = blockIdx.x & 7;
  const int lw = (blockIdx.x >> 3) * kWaves + w, per_xcd = (gridDim.x >> 3) * kWaves;
  const int ipx = (n_items + 7) >> 3;
  for (int i = lw; i < ipx; i += per_xcd) {
    const int item = xcd * ipx + i;
    if (item >= n_items) break;
    const int p = item / per_prob;
    const int rem = item - p * per_prob;
    const int tile = rem / a.cv, chunk = rem - tile * a.cv;
    const lora_problem pr = a.probs ? gload<lora_problem>(a.probs + p) : a.single;
    const int nrows = gload<int4>(a.tiles_v + tile).z;
    const int o_lo = chunk * a.wv, o_hi = min(a.d_out, o_lo + a.wv);
    wave_setup(a, a.rowrec + (int64_t)tile * kValuRows, nrows, W);
    if (uniform(W.nact) == 0 || o_lo >= o_hi) continue;
    for (int m0 = 0; m0 < nrows; m0 += kRowBlock) {
      const int nb = min(kRowBlock, nrows - m0);
      if (nb <= 1) wave_rows<T, 1>(a, pr, m0, nb, W, wv, o_lo, o_hi);
      else if (nb <= 2) wave_rows<T, 2>(a, pr, m0, nb, W, wv, o_lo, o_hi);
      else wave_rows<T, 4>(a, pr, m0, nb, W, wv, o_lo, o_hi);
    }
  }
}

template <typename T>
hipError_t launch_t(const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  static const bool lds_limit_raised =
      hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_kernel<T>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes) == hipSuccess;
  (void)lds_limit_raised;
  hipLaunchKernelGGL((decode_kernel<T>), dim3(grid), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

}  // namespace

// (sized for fp32, the wider intermediate)
size_t decode_smem_bytes(int kr_max) { return kWaves * (kWaveMetaBytes + size_t(kRowBlock) * kr_max * 4); }

hipError_t launch_decode(int dtype, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  return dtype == LORA_F32 ? launch_t<float>(a, grid, smem, stream) : launch_t<uint16_t>(a, grid, smem, stream);
}

}  // namespace lora
