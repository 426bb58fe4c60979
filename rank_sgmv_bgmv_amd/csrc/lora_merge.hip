// Merge / unmerge kernels: W += alpha * sum_k s_k B_k A_k in place.
//
// "Serving several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
// alongside": the merged form adds BA into W ahead of time (A is r x d_in, B
// is d_out x r), stacked LoRAs merge as a weighted sum (comparison table,
// stacking row), and switching unmerges the old one and merges the new one --
// one read and one write of the affected weights, which is the roofline the
// page itself gives (its cost model: twice the weight bytes over the HBM
// bandwidth).
//
// bf16: the update is a dense contraction of rank K*r, so it runs on the
// matrix cores.  A workgroup owns a strip of 128 or 256 columns of W and walks
// down it in steps of 64 rows (16 per wave).  A^T of the strip (every slot,
// rank padded to a multiple of 32 with zeros) is staged once in LDS, with the
// columns of each 32-column group interleaved so that the accumulators of two
// neighbouring 16-column tiles give a lane 8 consecutive columns of its row:
// W moves in 16-byte pieces.  B rows go straight into the MFMA operand
// registers.  Per step and slot: D^T (columns x rows) = A^T B^T on
// v_mfma_f32_16x16x32_bf16, then total += s_k D in fp32; W + total is rounded
// once.  W and B are loaded two steps ahead.
//
// fp32, and bf16 shapes the matrix-core path does not take: a VALU kernel in
// which each thread keeps 4 consecutive columns of 16 rows in fp32.

#include <algorithm>
#include <utility>

#include "lora_device.hpp"

namespace lora {
namespace {

// Columns of W per strip (MFMA path): 256 where the build keeps its ring in
// registers without spilling (one slot up to rank 64, or rank 128 alone), 128
// otherwise.  Each row of a step then moves 512 bytes in and out rather than
// 256: the FLUX-sized rank-64 merge ran 2085 -> 1929 us.
template <int KSR, int NE>
constexpr int strip_cols() {
  return (NE <= 2 || (KSR == 4 && NE == 4)) ? 256 : 128;
}
constexpr int kStepRows = 64;    // rows per step: 16 per wave
constexpr int kStepsPerItem = 8;  // 512 rows per item, one item per workgroup: 4, 6, 16, 24 and 48 measured 3-8% slower

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1: ring slot indices
// that are constant expressions, so the ring stays in registers.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ f32x4 mfma32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

// LDS row of strip column c: in each group of 32, column 8a + 4h + b goes to
// row 16h + 4a + b, so that 16-column tile 2p + h reads its rows in order and
// its row 4a + b holds column 32p + 8a + 4h + b.
__device__ __forceinline__ int strip_row(int c) {
  return (c & ~31) | (((c >> 2) & 1) << 4) | (((c >> 3) & 3) << 2) | (c & 3);
}

// KSR: k-steps of 32 per slot (rank padded to 32 * KSR); NE >= slots * KSR:
// B operand registers per lane and step.
template <int KSR, int NE>
__global__ __launch_bounds__(kThreads, 2) void merge_mfma_kernel(MergeArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kStripCols = strip_cols<KSR, NE>();
  uint16_t *at = reinterpret_cast<uint16_t *>(smem);  // [slot][kStripCols][RP + 8]
  constexpr int RP = 32 * KSR, AST = RP + 8;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  const int r = a.r, d_in = a.d_in, d_out = a.d_out, ns = a.nslots;
  const int n_chunks = (d_out + kStepRows * kStepsPerItem - 1) / (kStepRows * kStepsPerItem);
  const int64_t per_prob = (int64_t)((d_in + kStripCols - 1) / kStripCols) * n_chunks;

  walk_items(per_prob * a.n_problems, 1, [&](int64_t item) {
    const int p = int(item / per_prob);
    const int64_t rem = item - (int64_t)p * per_prob;
    const int strip = int(rem / n_chunks), chunk = int(rem % n_chunks);
    const int c0 = strip * kStripCols, row0 = chunk * kStepRows * kStepsPerItem;
    const lora_merge_problem pr = a.probs ? gload<lora_merge_problem>(a.probs + p) : a.single;
    uint16_t *__restrict__ W = static_cast<uint16_t *>(pr.W);
    const int64_t ldw = pr.ldw;
    auto Ak = [&](int k) { return static_cast<const uint16_t *>(pr.A) + (int64_t)a.idx[k] * r * d_in; };
    // each slot's rank: A rows and B columns past it are not read
    int rks[LORA_MAX_SLOTS];
#pragma unroll
    for (int k = 0; k < LORA_MAX_SLOTS; ++k)
      rks[k] = (k < ns && a.ranks) ? min(max(gload<int>(a.ranks + a.idx[k]), 1), r) : r;
    auto Bk = [&](int k) { return static_cast<const uint16_t *>(pr.B) + (int64_t)a.idx[k] * d_out * r; };
    // --- stage A^T of the strip: at[k][strip_row(c)][j] = A_k[j][c0 + c], zeros past r and d_in
    for (int e = tid; e < ns * RP * (kStripCols / 8); e += kThreads) {
      const int k = e / (RP * (kStripCols / 8)), rem = e % (RP * (kStripCols / 8));
      const int j = rem / (kStripCols / 8), c = 8 * (rem % (kStripCols / 8));
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < rks[k] && c0 + c < d_in) v = gload<uint4>(Ak(k) + (int64_t)j * d_in + c0 + c);
      uint16_t *dst = at + ((int64_t)k * kStripCols) * AST + j;
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[strip_row(c + 2 * i) * AST] = uint16_t(wv[i] & 0xffffu);
        dst[strip_row(c + 2 * i + 1) * AST] = uint16_t(wv[i] >> 16);
      }
    }
    lds_barrier();

    // --- walk the rows: lane (l16, kg) of wave w owns row o = row0 + 64 step + 16 w + l16
    //     and, in each 32-column group q, the columns 32 q + 8 kg .. +7.  The B
    //     operands are (slot, k-step) entries, slot-major.  A step's W pieces and
    //     B operands are loaded D - 1 steps ahead into a ring of registers whose
    //     slots are fixed at compile time (no copies: copying a register whose
    //     load is in flight would wait for it).  Steps past the end re-read the
    //     last one (never used), so that every path issues the same loads.
    constexpr int NP = kStripCols / 32, D = (NE >= 8 || NP > 4) ? 2 : 3;
    uint4 wr[D][NP], br[D][NE];
    const int n_steps = min(kStepsPerItem, (d_out - row0 + kStepRows - 1) / kStepRows);
    auto load = [&](int step, uint4(&wv)[NP], uint4(&bv)[NE]) {
      const int o = row0 + step * kStepRows + 16 * w + l16;
      const int oc = o < d_out ? o : d_out - 1;  // rows past d_out read the last row; never stored
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int c = c0 + 32 * q + 8 * kg;
        wv[q] = gload<uint4>(W + (int64_t)oc * ldw + (c < d_in ? c : 0));
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int k = min(e / KSR, ns - 1), j = 32 * (e % KSR) + 8 * kg;
        bv[e] = gload<uint4>(Bk(k) + (int64_t)oc * r + (j < rks[k] ? j : 0));
      }
    };
    auto compute = [&](int step, const uint4(&wv)[NP], const uint4(&bv)[NE]) {
      f32x4 tot[2 * NP], acc[2 * NP];
#pragma unroll
      for (int t = 0; t < 2 * NP; ++t) tot[t] = acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int k = e / KSR, ks = e % KSR;
        if (k < ns) {
          // B columns past the slot's rank are zero (A^T is zero there too, but B may hold anything)
          const uint4 b = keep_if(32 * ks + 8 * kg < rks[k], bv[e]);
#pragma unroll
          for (int t = 0; t < 2 * NP; ++t) {
            const uint4 av =
                *reinterpret_cast<const uint4 *>(at + ((int64_t)k * kStripCols + 16 * t + l16) * AST + 32 * ks + 8 * kg);
            acc[t] = mfma32(av, b, acc[t]);
          }
          if (ks == KSR - 1) {  // the slot is complete: scale it in fp32
            const float s = a.s[k];
#pragma unroll
            for (int t = 0; t < 2 * NP; ++t) {
              tot[t] += s * acc[t];
              acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
      }
      // lane: row o, columns 32 q + 8 kg + (0..3) in tot[2q], (4..7) in tot[2q+1]
      const int o = row0 + step * kStepRows + 16 * w + l16;
      if (o < d_out) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const int c = c0 + 32 * q + 8 * kg;
          if (c < d_in) {
            const uint4 y0 = wv[q];
            const f32x4 lo = tot[2 * q], hi = tot[2 * q + 1];
            gstore(W + (int64_t)o * ldw + c,
                   make_uint4(pack_bf2(bf_lo(y0.x) + lo[0], bf_hi(y0.x) + lo[1]),
                              pack_bf2(bf_lo(y0.y) + lo[2], bf_hi(y0.y) + lo[3]),
                              pack_bf2(bf_lo(y0.z) + hi[0], bf_hi(y0.z) + hi[1]),
                              pack_bf2(bf_lo(y0.w) + hi[2], bf_hi(y0.w) + hi[3])));
          }
        }
      }
    };
    static_for<D - 1>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      load(min(d, n_steps - 1), wr[d], br[d]);
    });
    for (int s0 = 0; s0 < n_steps; s0 += D) {
      static_for<D>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        const int step = s0 + d;
        load(min(step + D - 1, n_steps - 1), wr[(d + D - 1) % D], br[(d + D - 1) % D]);
        if (step < n_steps) compute(step, wr[d], br[d]);
      });
    }
  });
}

// VALU path: thread t of a workgroup keeps columns c0 + 4 (t % 64) .. +3 of
// rows row0 + t / 64 + 4 i (i < 16) in fp32; A is read per rank index (4
// columns, L2-resident), B one element per row (the same for the whole wave).
constexpr int kValuCols = 256, kValuRowsPerItem = 64;

template <typename T>
__global__ __launch_bounds__(kThreads) void merge_valu_kernel(MergeArgs a) {
  const int tid = threadIdx.x, cq = tid & 63, rq = tid >> 6;
  const int r = a.r, d_in = a.d_in, d_out = a.d_out, ns = a.nslots;
  const int n_strips = (d_in + kValuCols - 1) / kValuCols;
  const int n_chunks = (d_out + kValuRowsPerItem - 1) / kValuRowsPerItem;
  const int64_t per_prob = (int64_t)n_strips * n_chunks;
  walk_items(per_prob * a.n_problems, 1, [&](int64_t item) {
    const int p = int(item / per_prob);
    const int64_t rem = item - (int64_t)p * per_prob;
    const int strip = int(rem / n_chunks), chunk = int(rem % n_chunks);
    const lora_merge_problem pr = a.probs ? gload<lora_merge_problem>(a.probs + p) : a.single;
    T *__restrict__ W = static_cast<T *>(pr.W);
    const int c = strip * kValuCols + 4 * cq;
    const int row0 = chunk * kValuRowsPerItem + rq;
    float acc[16][4];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i][0] = acc[i][1] = acc[i][2] = acc[i][3] = 0.f;
    for (int k = 0; k < ns; ++k) {
      const T *__restrict__ Ak = static_cast<const T *>(pr.A) + (int64_t)a.idx[k] * r * d_in;
      const T *__restrict__ Bk = static_cast<const T *>(pr.B) + (int64_t)a.idx[k] * d_out * r;
      const float s = a.s[k];
      const int rk = a.ranks ? min(max(gload<int>(a.ranks + a.idx[k]), 1), r) : r;
      for (int j = 0; j < rk; ++j) {
        float av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cc = c + q;
          const T v = cc < d_in ? gload<T>(Ak + (int64_t)j * d_in + cc) : T(0);
          if constexpr (sizeof(T) == 2) av[q] = s * bf_to_f(v);
          else av[q] = s * v;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o = row0 + 4 * i;
          const int oc = o < d_out ? o : d_out - 1;
          const T bv = gload<T>(Bk + (int64_t)oc * r + j);
          float b;
          if constexpr (sizeof(T) == 2) b = bf_to_f(bv);
          else b = bv;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(b, av[q], acc[i][q]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int o = row0 + 4 * i;
      if (o >= d_out) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (c + q >= d_in) continue;
        T *pw = W + (int64_t)o * pr.ldw + c + q;
        if constexpr (sizeof(T) == 2) *pw = f_to_bf(bf_to_f(*pw) + acc[i][q]);
        else *pw = *pw + acc[i][q];
      }
    }
  });
}

template <int KSR, int NE>
hipError_t launch_mfma_ksr(const MergeArgs &a, hipStream_t stream) {
  constexpr int kStripCols = strip_cols<KSR, NE>();
  const int n_chunks = (a.d_out + kStepRows * kStepsPerItem - 1) / (kStepRows * kStepsPerItem);
  const int64_t items = (int64_t)((a.d_in + kStripCols - 1) / kStripCols) * n_chunks * a.n_problems;
  // one item per workgroup up to 65536 items: the FLUX-sized merge's 8208
  // items ran 1.5% faster this way than walked by 2048 workgroups
  const int grid = int(std::min<int64_t>((items + 7) / 8 * 8, 65536));
  const size_t smem = size_t(a.nslots) * kStripCols * (32 * KSR + 8) * 2;
  static const bool lds_limit_raised =
      raise_lds_limit(reinterpret_cast<const void *>(&merge_mfma_kernel<KSR, NE>), kMaxLdsBytes);
  (void)lds_limit_raised;
  hipLaunchKernelGGL((merge_mfma_kernel<KSR, NE>), dim3(grid), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

// NE: the (slot, k-step) entries, rounded up to 1, 2, 4 or 8.
template <int KSR>
hipError_t launch_mfma_ne(const MergeArgs &a, hipStream_t stream) {
  const int ne = a.nslots * KSR;
  if (ne <= 1 && KSR <= 1) return launch_mfma_ksr<KSR, (KSR <= 1 ? 1 : KSR)>(a, stream);
  if (ne <= 2 && KSR <= 2) return launch_mfma_ksr<KSR, (KSR <= 2 ? 2 : KSR)>(a, stream);
  if (ne <= 4 && KSR <= 4) return launch_mfma_ksr<KSR, (KSR <= 4 ? 4 : KSR)>(a, stream);
  return launch_mfma_ksr<KSR, 8>(a, stream);
}

}  // namespace

bool merge_mfma_eligible(const MergeArgs &a, int dtype) {
  return dtype == LORA_BF16 && a.aligned && a.r % 8 == 0 && a.nslots * ((a.r + 31) / 32 * 32) <= 256 &&
         a.d_in % 8 == 0;
}

hipError_t launch_merge(const MergeArgs &a, int dtype, hipStream_t stream) {
  if (merge_mfma_eligible(a, dtype)) {
    const int ksr = (a.r + 31) / 32;
    const int k2 = ksr <= 1 ? 1 : ksr <= 2 ? 2 : ksr <= 4 ? 4 : 8;
    switch (k2) {
      case 1: return launch_mfma_ne<1>(a, stream);
      case 2: return launch_mfma_ne<2>(a, stream);
      case 4: return launch_mfma_ne<4>(a, stream);
      default: return launch_mfma_ne<8>(a, stream);
    }
  }
  const int64_t items = (int64_t)((a.d_in + kValuCols - 1) / kValuCols) *
                        ((a.d_out + kValuRowsPerItem - 1) / kValuRowsPerItem) * a.n_problems;
  const int grid = int(std::min<int64_t>((items + 7) / 8 * 8, 2048));
  if (dtype == LORA_F32)
    hipLaunchKernelGGL((merge_valu_kernel<float>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((merge_valu_kernel<uint16_t>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lora
