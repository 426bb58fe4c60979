// MFMA apply kernel: prefill tiles of 64 rows of one adapter group, bf16,
// rank 16 / 32 / 64 / 128.  Computes y += scale * (x A_i^T) B_i^T for the
// tile's rows with both contractions on the matrix cores.
//
// "Serving several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
// alongside": the unmerged form adds x A^T B^T to x W^T; "Exercises" (four
// requests): requests on one adapter form one partition, whose products grow
// with its size -- the long partitions are the ones dense enough for MFMA.
// Comparison table, row on stacking several LoRAs: stacked adapters are
// summed; here the slots of a tile share one accumulator.
//
// Layout of the work.  Wave w owns tile rows 16w .. 16w+15.
//   Shrink (per slot): V^T[j][t] = sum_c A[j][c] x[t][c] on
//     v_mfma_f32_16x16x32_bf16.  d_in is walked in stages of KC columns.  A
//     (L2-resident: every tile of the group reads it) is staged through LDS,
//     shared by the four waves, with the next stage prefetched into
//     registers; x (the HBM stream) goes straight into MFMA operand registers,
//     one stage ahead, double buffered.  Two barriers per stage.
//     The accumulator layout gives lane (t, q) the values v[t][16 jt + 4q ..
//     +3]; scaled and rounded once to bf16 they are exactly the B operand of
//     the expand's v_mfma_f32_16x16x16_bf16.  Each lane parks them in LDS
//     (its own row, read back only by itself) until the expand.
//   Expand: Y^T[o][t] += sum_j B[o][j] v[t][j] per stage of 128 outputs (and
//     per slot).  B is staged through LDS with the next stage prefetched into
//     registers; y is read one stage ahead straight into the accumulator
//     layout, added and rounded once to bf16, and written back.  The B rows
//     of each pair of 16-wide output tiles are interleaved as they are staged
//     so that a lane's two accumulators hold 8 consecutive outputs of its
//     row: y moves in 16-byte pieces.
// Every bf16 product is exact in fp32 and accumulation is fp32; the rank-r
// intermediate is rounded once to bf16 before the expand.
//
// A second build halves both stages (d_in columns per shrink stage, outputs
// per expand stage) for tiles with many stacked slots, whose parked
// intermediates would otherwise leave LDS for one workgroup per CU.
//
// Stacked slots (comparison table, stacking row: every stacked LoRA adds its
// own alongside product to the same x).  In a launch whose requests stack
// two to four adapters, a tile with several slots walks x once for all of
// them: each x stage is multiplied by every slot's staged A into that slot's
// accumulators, and the slots' bf16 intermediates stay in registers through
// the expand (instead of parking in LDS), so all slots' A stages fit beside
// each other.  Single-slot tiles of the same launch take the path above.

#include "lora_device.hpp"

namespace lora {
namespace {

__device__ __forceinline__ f32x4 mfma32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ f32x4 mfma16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                    0, 0);
}

// HS = 2 halves both stages (d_in columns per shrink stage, outputs per expand
// stage): less LDS per workgroup, for tiles with many stacked slots, whose
// parked intermediates would otherwise leave room for one workgroup per CU.
template <int JT, int HS = 1>
struct MfmaCfg {
  static constexpr int R = 16 * JT;
  static constexpr int KC = (R <= 64 ? 256 : 128) / HS;    // d_in columns per shrink stage
  static constexpr int KS = KC / 32;                       // k-steps per stage
  static constexpr int AST = KC + 8;                       // staged A row stride (elements)
  static constexpr int NAV = R * (KC / 8) / kThreads;      // 16-byte A pieces per thread per stage
  static constexpr int NO = 128 / HS;                      // outputs per expand stage
  static constexpr int OT = NO / 16;                       // 16-wide output tiles per stage
  static constexpr int BST = R + 8;                        // staged B row stride (elements)
  static constexpr int NBV = NO * (R / 8) / kThreads;      // 16-byte B pieces per thread per stage
  static constexpr size_t LDS = (size_t(R) * AST > size_t(NO) * BST ? size_t(R) * AST : size_t(NO) * BST) * 2;
  static constexpr int VST = R + 8;                        // row stride (elements) of the parked intermediate
  static_assert(NAV >= 1 && NBV >= 1 && KC % 32 == 0 && NO % 32 == 0, "stage sizes");
};

template <int JT, int HS, int MODE>
__device__ void mfma_tile(const ApplyArgs &a, const lora_problem &pr, int nrows, int o_lo, int o_hi, int d_out,
                          const Meta &M, uint16_t *stage, uint16_t *vpark) {
  typedef MfmaCfg<JT, HS> C;
  constexpr int R = C::R, KC = C::KC, KS = C::KS, AST = C::AST, NAV = C::NAV;
  constexpr int NO = C::NO, OT = C::OT, BST = C::BST, NBV = C::NBV, VST = C::VST;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  const int m = 16 * w + l16;  // this lane's tile row
  const bool row_ok = m < nrows;
  const bool wave_live = 16 * w < nrows;
  const int d_in = a.d_in, nact = M.nact;
  const int64_t trow = M.t[row_ok ? m : 0];
  const uint16_t *__restrict__ xrow = static_cast<const uint16_t *>(pr.x) + trow * pr.ldx;
  uint16_t *__restrict__ yrow = static_cast<uint16_t *>(pr.y) + trow * pr.ldy;

  // parked bf16 intermediate of this lane: v[t][16 jt + 4 kg .. +3] of compacted slot kk
  auto vslot = [&](int kk, int jt) -> uint2 * {
    return reinterpret_cast<uint2 *>(vpark + ((int64_t)kk * kMfmaRows + m) * VST + 16 * jt + 4 * kg);
  };

  // ------------------------------------------------------------ shrink --
  for (int kk = 0; kk < nact; ++kk) {
    if (MODE == MODE_EXPAND) {
      const int rk = M.rk[kk];
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        const int j = 16 * jt + 4 * kg;
        if (row_ok)
          f = gload<float4>(a.v + trow * a.ldv + (int64_t)M.pos[m][kk] * R + j);
        // columns past the adapter's rank are zero
        *vslot(kk, jt) = make_uint2(pack_bf2(j < rk ? f.x : 0.f, j + 1 < rk ? f.y : 0.f),
                                    pack_bf2(j + 2 < rk ? f.z : 0.f, j + 3 < rk ? f.w : 0.f));
      }
      continue;
    }
    const uint16_t *__restrict__ Aa = static_cast<const uint16_t *>(pr.A) + (int64_t)M.a[kk] * R * d_in;
    const int rk = M.rk[kk];  // A rows past the adapter's rank are not read (zeros in LDS)
    f32x4 acc[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 ar[NAV];      // next A stage (cooperative, all threads)
    uint4 x0[KS], x1[KS];  // x operands of the current / next stage (this lane's row)

    auto load_a = [&](int kc) {
#pragma unroll
      for (int i = 0; i < NAV; ++i) {
        const int e = tid + i * kThreads;
        const int row = e / (KC / 8), c = kc + 8 * (e % (KC / 8));
        ar[i] = (c < d_in && row < rk) ? gload<uint4>(Aa + (int64_t)row * d_in + c) : make_uint4(0, 0, 0, 0);
      }
    };
    auto load_x = [&](int kc, uint4(&xr)[KS]) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = kc + 32 * ks + 8 * kg;
        xr[ks] = (row_ok && c < d_in) ? gload<uint4>(xrow + c) : make_uint4(0, 0, 0, 0);
      }
    };
    // one stage: publish the A stage held in `ar`, prefetch the next, multiply
    auto step = [&](int kc, const uint4(&xc)[KS], uint4(&xn)[KS]) {
      lds_barrier();  // every wave is done reading the previous stage
#pragma unroll
      for (int i = 0; i < NAV; ++i) {
        const int e = tid + i * kThreads;
        *reinterpret_cast<uint4 *>(stage + (e / (KC / 8)) * AST + 8 * (e % (KC / 8))) = ar[i];
      }
      lds_barrier();
      if (kc + KC < d_in) {
        load_a(kc + KC);
        load_x(kc + KC, xn);
      }
      if (wave_live) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int jt = 0; jt < JT; ++jt) {
            // rows past the adapter's rank are zeros in the stage (no branch
            // here: a condition per rank tile would split the MFMA chain)
            const uint4 av = *reinterpret_cast<const uint4 *>(stage + (16 * jt + l16) * AST + 32 * ks + 8 * kg);
            acc[jt] = mfma32(av, xc[ks], acc[jt]);
          }
        }
      }
    };
    load_a(0);
    load_x(0, x0);
    for (int kc = 0; kc < d_in; kc += 2 * KC) {
      step(kc, x0, x1);
      if (kc + KC < d_in) step(kc + KC, x1, x0);
    }
    // acc[jt][q] = v[t_m][16 jt + 4 kg + q], unscaled
    const float sc = row_ok ? M.sc[m][kk] : 0.f;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const f32x4 s = acc[jt] * sc;
      if (MODE == MODE_SHRINK) {
        if (row_ok)
          gstore(a.v + trow * a.ldv + (int64_t)M.pos[m][kk] * R + 16 * jt + 4 * kg, make_float4(s[0], s[1], s[2], s[3]));
      } else {
        *vslot(kk, jt) = make_uint2(pack_bf2(s[0], s[1]), pack_bf2(s[2], s[3]));
      }
    }
  }
  if (MODE == MODE_SHRINK) {
    zero_empty_slots(a, 0, nrows, M);
    return;
  }

  // ------------------------------------------------------------ expand --
  // stages are (output block ob, slot kk), slot-minor
  const int n_ob = (o_hi - o_lo + NO - 1) / NO;
  const int n_st = n_ob * nact;
  uint4 br[NBV];                     // next B stage (cooperative)
  uint4 yc[OT / 2], yn[OT / 2];      // y pieces of the current / next output block
  f32x4 yacc[OT];
  auto load_b = [&](int st) {
    const int ob = o_lo + (st / nact) * NO, kk = st % nact;
    const uint16_t *__restrict__ Bk = static_cast<const uint16_t *>(pr.B) + (int64_t)M.a[kk] * d_out * R;
    const int rk = M.rk[kk];  // B columns past the adapter's rank are not read
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int e = tid + i * kThreads;
      const int row = e / (R / 8), c = 8 * (e % (R / 8));
      br[i] = (ob + row < o_hi && c < rk) ? gload<uint4>(Bk + (int64_t)(ob + row) * R + c) : make_uint4(0, 0, 0, 0);
    }
  };
  auto load_y = [&](int ob, uint4(&yr)[OT / 2]) {
#pragma unroll
    for (int p = 0; p < OT / 2; ++p) {
      const int o = ob + 32 * p + 8 * kg;
      yr[p] = (row_ok && o < o_hi) ? gload<uint4>(yrow + o) : make_uint4(0, 0, 0, 0);
    }
  };
  if (n_st > 0) {
    load_b(0);
    load_y(o_lo, yc);
  }
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) yacc[ot] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < n_st; ++st) {
    const int ob = o_lo + (st / nact) * NO, kk = st % nact;
    lds_barrier();  // every wave is done reading the previous stage
    // block row o' = 32p + 8a + 4h + b goes to LDS row 32p + 16h + 4a + b:
    // output tile 2p + h then reads its rows 16(2p+h) .. +15 in order (no bank
    // conflicts), and its row 4a + b holds output 32p + 8a + 4h + b, so that
    // the accumulators of tiles 2p and 2p+1 give each lane 8 consecutive
    // outputs of its row (one 16-byte y piece)
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int e = tid + i * kThreads;
      const int row = e / (R / 8);
      const int lrow = (row & ~31) | (((row >> 2) & 1) << 4) | (((row >> 3) & 3) << 2) | (row & 3);
      *reinterpret_cast<uint4 *>(stage + lrow * BST + 8 * (e % (R / 8))) = br[i];
    }
    lds_barrier();
    if (st + 1 < n_st) {
      load_b(st + 1);
      if ((st + 1) % nact == 0) load_y(ob + NO, yn);
    }
    if (wave_live) {
      uint2 v[JT];
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) v[jt] = *vslot(kk, jt);
      // B columns past the adapter's rank are zeros in the stage and so is the
      // intermediate there: those products add exact zeros
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const uint2 bv = *reinterpret_cast<const uint2 *>(stage + (16 * ot + l16) * BST + 16 * jt + 4 * kg);
          yacc[ot] = mfma16(bv, v[jt], yacc[ot]);
        }
      }
    }
    if (kk == nact - 1) {
      // output block done: y += delta, rounded once, written back
#pragma unroll
      for (int p = 0; p < OT / 2; ++p) {
        const int o = ob + 32 * p + 8 * kg;
        if (row_ok && o < o_hi) {
          const uint4 y0 = yc[p];
          const f32x4 lo = yacc[2 * p], hi = yacc[2 * p + 1];
          gstore(yrow + o, make_uint4(pack_bf2(bf_lo(y0.x) + lo[0], bf_hi(y0.x) + lo[1]),
                                      pack_bf2(bf_lo(y0.y) + lo[2], bf_hi(y0.y) + lo[3]),
                                      pack_bf2(bf_lo(y0.z) + hi[0], bf_hi(y0.z) + hi[1]),
                                      pack_bf2(bf_lo(y0.w) + hi[2], bf_hi(y0.w) + hi[3])));
        }
        yc[p] = yn[p];
      }
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) yacc[ot] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// ---------------------------------------------------------- stacked tiles --
// A stages of SMAX slots side by side in LDS: d_in columns per stage chosen so
// that they hold about 16 K elements together (32 KB), which keeps the next
// stage's A (prefetched into registers) at 32 registers a lane.
template <int JT, int SMAX>
struct StackCfg {
  static constexpr int R = 16 * JT;
  static constexpr int KC0 = 16384 / (SMAX * R);
  static constexpr int KC = KC0 >= 256 ? 256 : KC0 >= 128 ? 128 : KC0 >= 64 ? 64 : 32;  // d_in columns per stage
  static constexpr int KS = KC / 32;                       // k-steps per stage
  static constexpr int AST = KC + 8;                       // staged A row stride (elements)
  static constexpr int NAV = R * (KC / 8) / kThreads;      // 16-byte A pieces per thread per stage and slot
  static constexpr int SST = R * AST;                      // elements between two slots' A stages
  static constexpr int NO = 128;                           // outputs per expand stage
  static constexpr int OT = NO / 16;
  static constexpr int BST = R + 8;
  static constexpr int NBV = NO * (R / 8) / kThreads;
  static constexpr size_t LDS = (size_t(SMAX) * SST > size_t(NO) * BST ? size_t(SMAX) * SST : size_t(NO) * BST) * 2;
  static_assert(NAV >= 1 && NBV >= 1, "stage sizes");
};

// A tile whose rows carry 2 .. SMAX slots (fused mode): one walk over d_in,
// the slots' intermediates in registers, then the expand of every output
// block over every slot.
//
// SL (sliced launches, one slot per request): the "slots" are instead nsl
// slices of a group that read the same x -- entries p0 .. p0 + nsl - 1 of the
// group's problems `gp` -- each with its own A and B (the same adapter index
// and scale), so one walk over x feeds every slice's intermediate; the expand
// then writes each slice's whole output width to its own y.  `pr`, o_lo, o_hi
// and d_out are unused then.
template <int JT, int SMAX, bool SL = false>
__device__ void mfma_tile_stacked(const ApplyArgs &a, const lora_problem &pr, int nrows, int o_lo, int o_hi,
                                  int d_out, const Meta &M, uint16_t *stage, const lora_problem *gp = nullptr,
                                  int p0 = 0, int nsl = 0) {
  typedef StackCfg<JT, SMAX> C;
  constexpr int R = C::R, KC = C::KC, KS = C::KS, AST = C::AST, NAV = C::NAV, SST = C::SST;
  constexpr int NO = C::NO, OT = C::OT, BST = C::BST, NBV = C::NBV;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  const int m = 16 * w + l16;  // this lane's tile row
  const bool row_ok = m < nrows;
  const bool wave_live = 16 * w < nrows;
  const int d_in = a.d_in, nact = SL ? nsl : uniform(M.nact);
  const int64_t trow = M.t[row_ok ? m : 0];
  const lora_problem &px = SL ? gp[p0] : pr;  // the x every slot reads
  const uint16_t *__restrict__ xrow = static_cast<const uint16_t *>(px.x) + trow * px.ldx;
  uint16_t *__restrict__ yrow = static_cast<uint16_t *>(pr.y) + trow * pr.ldy;
  // A of every slot (a slice's own pool at the tile's one adapter when SL)
  const uint16_t *Abase[SMAX];
#pragma unroll
  for (int g = 0; g < SMAX; ++g) {
    const int gg = min(g, nact - 1);
    Abase[g] = SL ? static_cast<const uint16_t *>(gp[p0 + gg].A) + (int64_t)M.a[0] * R * d_in
                  : static_cast<const uint16_t *>(pr.A) + (int64_t)M.a[gg] * R * d_in;
  }

  // ------------------------------------------------------------ shrink --
  f32x4 acc[SMAX][JT];
#pragma unroll
  for (int g = 0; g < SMAX; ++g)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[g][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 ar[SMAX][NAV];    // next A stage of every slot (cooperative)
  uint4 x0[KS], x1[KS];   // x operands of the current / next stage (this lane's row)
  auto load_a = [&](int kc) {
#pragma unroll
    for (int g = 0; g < SMAX; ++g) {
      const int gg = min(g, nact - 1);
      const uint16_t *__restrict__ Ag = Abase[g];
      // rows past the adapter's rank (or an unused slot) are zeros
      const int rk = g < nact ? (SL ? M.rk[0] : M.rk[gg]) : 0;
#pragma unroll
      for (int i = 0; i < NAV; ++i) {
        const int e = tid + i * kThreads;
        const int row = e / (KC / 8), c = kc + 8 * (e % (KC / 8));
        ar[g][i] = (c < d_in && row < rk) ? gload<uint4>(Ag + (int64_t)row * d_in + c) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto load_x = [&](int kc, uint4(&xr)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = kc + 32 * ks + 8 * kg;
      xr[ks] = (row_ok && c < d_in) ? gload<uint4>(xrow + c) : make_uint4(0, 0, 0, 0);
    }
  };
  auto step = [&](int kc, const uint4(&xc)[KS], uint4(&xn)[KS]) {
    lds_barrier();  // every wave is done reading the previous stage
#pragma unroll
    for (int g = 0; g < SMAX; ++g) {
      if (g < nact) {
#pragma unroll
        for (int i = 0; i < NAV; ++i) {
          const int e = tid + i * kThreads;
          *reinterpret_cast<uint4 *>(stage + g * SST + (e / (KC / 8)) * AST + 8 * (e % (KC / 8))) = ar[g][i];
        }
      }
    }
    lds_barrier();
    if (kc + KC < d_in) {
      load_a(kc + KC);
      load_x(kc + KC, xn);
    }
    if (wave_live) {
#pragma unroll
      for (int g = 0; g < SMAX; ++g) {
        if (g < nact) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
              const uint4 av =
                  *reinterpret_cast<const uint4 *>(stage + g * SST + (16 * jt + l16) * AST + 32 * ks + 8 * kg);
              acc[g][jt] = mfma32(av, xc[ks], acc[g][jt]);
            }
          }
        }
      }
    }
  };
  load_a(0);
  load_x(0, x0);
  for (int kc = 0; kc < d_in; kc += 2 * KC) {
    step(kc, x0, x1);
    if (kc + KC < d_in) step(kc + KC, x1, x0);
  }
  // acc[g][jt][q] = v_g[t_m][16 jt + 4 kg + q]: scaled and rounded once to bf16
  // it is the B operand of the expand's MFMA for this lane's row
  uint2 v[SMAX][JT];
#pragma unroll
  for (int g = 0; g < SMAX; ++g) {
    const float sc = (row_ok && g < nact) ? M.sc[m][SL ? 0 : min(g, nact - 1)] : 0.f;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const f32x4 sv = acc[g][jt] * sc;
      v[g][jt] = make_uint2(pack_bf2(sv[0], sv[1]), pack_bf2(sv[2], sv[3]));
    }
  }

  // ------------------------------------------------------------ expand --
  if constexpr (SL) {
    // stages are (slice, output block), slice-major; each stage is a whole
    // 128-output block of one slice's y, stored when the stage ends.  Each
    // slice's width, B (at the tile's adapter) and y row are taken once here
    // and picked by unrolled compares (no index known only at run time).
    int dos[SMAX], nob[SMAX];
    const uint16_t *Bb[SMAX];
    uint16_t *Yb[SMAX];
    int n_st = 0;
#pragma unroll
    for (int g = 0; g < SMAX; ++g) {
      dos[g] = 0;
#pragma unroll
      for (int q = 0; q < LORA_MAX_SLICES; ++q)  // constant indices into the argument block
        if (q == p0 + g) dos[g] = a.sd_out[q];
      const lora_problem &pg = gp[p0 + min(g, nact - 1)];
      Bb[g] = static_cast<const uint16_t *>(pg.B) + (int64_t)M.a[0] * dos[g] * R;
      Yb[g] = static_cast<uint16_t *>(pg.y) + trow * pg.ldy;
      nob[g] = g < nact ? (dos[g] + NO - 1) / NO : 0;
      n_st += nob[g];
    }
    struct StageAt {
      int g, ob, dout;
      const uint16_t *B;
      uint16_t *y;
    };
    auto stage_at = [&](int st) {
      StageAt r{0, st, dos[0], Bb[0], Yb[0]};
#pragma unroll
      for (int q = 0; q + 1 < SMAX; ++q)
        if (r.g == q && r.ob >= nob[q]) {
          r.ob -= nob[q];
          r.g = q + 1;
          r.dout = dos[q + 1];
          r.B = Bb[q + 1];
          r.y = Yb[q + 1];
        }
      r.ob *= NO;
      return r;
    };
    const int rk = M.rk[0];
    uint4 br[NBV];
    uint4 yc[OT / 2], yn[OT / 2];
    f32x4 yacc[OT];
    auto load_b = [&](const StageAt &sa) {
#pragma unroll
      for (int i = 0; i < NBV; ++i) {
        const int e = tid + i * kThreads;
        const int row = e / (R / 8), c = 8 * (e % (R / 8));
        br[i] = (sa.ob + row < sa.dout && c < rk) ? gload<uint4>(sa.B + (int64_t)(sa.ob + row) * R + c)
                                                   : make_uint4(0, 0, 0, 0);
      }
    };
    auto load_y = [&](const StageAt &sa, uint4(&yr)[OT / 2]) {
#pragma unroll
      for (int p = 0; p < OT / 2; ++p) {
        const int o = sa.ob + 32 * p + 8 * kg;
        yr[p] = (row_ok && o < sa.dout) ? gload<uint4>(sa.y + o) : make_uint4(0, 0, 0, 0);
      }
    };
    if (n_st > 0) {
      const StageAt s0 = stage_at(0);
      load_b(s0);
      load_y(s0, yc);
    }
    for (int st = 0; st < n_st; ++st) {
      const StageAt cur = stage_at(st);
      lds_barrier();  // every wave is done reading the previous stage
#pragma unroll
      for (int i = 0; i < NBV; ++i) {
        const int e = tid + i * kThreads;
        const int row = e / (R / 8);
        const int lrow = (row & ~31) | (((row >> 2) & 1) << 4) | (((row >> 3) & 3) << 2) | (row & 3);
        *reinterpret_cast<uint4 *>(stage + lrow * BST + 8 * (e % (R / 8))) = br[i];
      }
      lds_barrier();
      if (st + 1 < n_st) {
        const StageAt nx = stage_at(st + 1);
        load_b(nx);
        load_y(nx, yn);
      }
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) yacc[ot] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (wave_live) {
#pragma unroll
        for (int g = 0; g < SMAX; ++g) {
          if (g == cur.g) {
#pragma unroll
            for (int ot = 0; ot < OT; ++ot) {
#pragma unroll
              for (int jt = 0; jt < JT; ++jt) {
                const uint2 bv = *reinterpret_cast<const uint2 *>(stage + (16 * ot + l16) * BST + 16 * jt + 4 * kg);
                yacc[ot] = mfma16(bv, v[g][jt], yacc[ot]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int p = 0; p < OT / 2; ++p) {
        const int o = cur.ob + 32 * p + 8 * kg;
        if (row_ok && o < cur.dout) {
          const uint4 y0 = yc[p];
          const f32x4 lo = yacc[2 * p], hi = yacc[2 * p + 1];
          gstore(cur.y + o, make_uint4(pack_bf2(bf_lo(y0.x) + lo[0], bf_hi(y0.x) + lo[1]),
                                       pack_bf2(bf_lo(y0.y) + lo[2], bf_hi(y0.y) + lo[3]),
                                       pack_bf2(bf_lo(y0.z) + hi[0], bf_hi(y0.z) + hi[1]),
                                       pack_bf2(bf_lo(y0.w) + hi[2], bf_hi(y0.w) + hi[3])));
        }
        yc[p] = yn[p];
      }
    }
    return;
  } else {
  // stages are (output block, slot), slot-minor, as in mfma_tile
  const int n_ob = (o_hi - o_lo + NO - 1) / NO;
  const int n_st = n_ob * nact;
  uint4 br[NBV];
  uint4 yc[OT / 2], yn[OT / 2];
  f32x4 yacc[OT];
  auto load_b = [&](int st) {
    const int ob = o_lo + (st / nact) * NO, kk = st % nact;
    const uint16_t *__restrict__ Bk = static_cast<const uint16_t *>(pr.B) + (int64_t)M.a[kk] * d_out * R;
    const int rk = M.rk[kk];
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int e = tid + i * kThreads;
      const int row = e / (R / 8), c = 8 * (e % (R / 8));
      br[i] = (ob + row < o_hi && c < rk) ? gload<uint4>(Bk + (int64_t)(ob + row) * R + c) : make_uint4(0, 0, 0, 0);
    }
  };
  auto load_y = [&](int ob, uint4(&yr)[OT / 2]) {
#pragma unroll
    for (int p = 0; p < OT / 2; ++p) {
      const int o = ob + 32 * p + 8 * kg;
      yr[p] = (row_ok && o < o_hi) ? gload<uint4>(yrow + o) : make_uint4(0, 0, 0, 0);
    }
  };
  if (n_st > 0) {
    load_b(0);
    load_y(o_lo, yc);
  }
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) yacc[ot] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < n_st; ++st) {
    const int ob = o_lo + (st / nact) * NO, kk = st % nact;
    lds_barrier();  // every wave is done reading the previous stage
    // the interleaved row order of mfma_tile's expand stages (two 16-wide
    // output tiles give each lane 8 consecutive outputs of its row)
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int e = tid + i * kThreads;
      const int row = e / (R / 8);
      const int lrow = (row & ~31) | (((row >> 2) & 1) << 4) | (((row >> 3) & 3) << 2) | (row & 3);
      *reinterpret_cast<uint4 *>(stage + lrow * BST + 8 * (e % (R / 8))) = br[i];
    }
    lds_barrier();
    if (st + 1 < n_st) {
      load_b(st + 1);
      if ((st + 1) % nact == 0) load_y(ob + NO, yn);
    }
    if (wave_live) {
#pragma unroll
      for (int g = 0; g < SMAX; ++g) {
        if (g == kk) {
#pragma unroll
          for (int ot = 0; ot < OT; ++ot) {
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
              const uint2 bv = *reinterpret_cast<const uint2 *>(stage + (16 * ot + l16) * BST + 16 * jt + 4 * kg);
              yacc[ot] = mfma16(bv, v[g][jt], yacc[ot]);
            }
          }
        }
      }
    }
    if (kk == nact - 1) {
#pragma unroll
      for (int p = 0; p < OT / 2; ++p) {
        const int o = ob + 32 * p + 8 * kg;
        if (row_ok && o < o_hi) {
          const uint4 y0 = yc[p];
          const f32x4 lo = yacc[2 * p], hi = yacc[2 * p + 1];
          gstore(yrow + o, make_uint4(pack_bf2(bf_lo(y0.x) + lo[0], bf_hi(y0.x) + lo[1]),
                                      pack_bf2(bf_lo(y0.y) + lo[2], bf_hi(y0.y) + lo[3]),
                                      pack_bf2(bf_lo(y0.z) + hi[0], bf_hi(y0.z) + hi[1]),
                                      pack_bf2(bf_lo(y0.w) + hi[2], bf_hi(y0.w) + hi[3])));
        }
        yc[p] = yn[p];
      }
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) yacc[ot] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  }
}

// ---------------------------------------------------------------- kernel --
// SMAX > 1 (fused launches whose requests stack 2 .. SMAX adapters): tiles
// with several slots take mfma_tile_stacked, the others mfma_tile.  NSL: the
// output slices the build handles (LORA_MAX_SLICES for lora_apply_sliced's
// launches, 1 for all others).
template <int JT, int HS, int MODE, int SMAX, int NSL>
__device__ __forceinline__ void mfma_kernel_body(const ApplyArgs &a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Meta &M = *reinterpret_cast<Meta *>(smem);
  uint16_t *stage = reinterpret_cast<uint16_t *>(smem + kMetaBytes);
  uint16_t *vpark = reinterpret_cast<uint16_t *>(smem + kMetaBytes + MfmaCfg<JT, HS>::LDS);
  const PlanHdr ph = read_plan_header(a);
  if (!ph.ok) return;
  const int n_m64 = ph.n_m, n_ms = ph.n_ms, n_active = ph.n_active;
  const int per_tile = NSL == 1 ? a.items_m_tile : a.cmo[a.ns];  // items of one tile, over every slice
  // The plan's 48-row tiling when the 64-row items are more than the CUs (so
  // some CUs would run two and set the launch's duration) but the 48-row items
  // all fit on the chip at once: the CUs that run two then hold 96 rows
  // instead of 128.  With more items than that, 64-row tiles (their adapter
  // staging spread over more rows) are faster.
  const bool small = (int64_t)n_m64 * per_tile * a.n_problems > a.n_cu &&
                     (int64_t)n_ms * per_tile * a.n_problems <= a.mfma_slots;
  const int n_m = small ? n_ms : n_m64;
  const int4 *tiles = small ? a.tiles_ms : a.tiles_m;
  const int64_t per_grp = (int64_t)n_m * per_tile;
  walk_items(per_grp * a.n_problems, per_tile, [&](int64_t item) {
    const int g = int(item / per_grp);
    const int64_t rem = item - (int64_t)g * per_grp;
    // tiles in reverse plan order: the plan puts the requests with several
    // adapters (the longest tiles: a shrink and an expand pass per slot)
    // last, and they should start first rather than form the launch's tail
    const int tile = n_m - 1 - int(rem / per_tile);
    const Chunk c = chunk_of<NSL, 1>(a, true, int(rem % per_tile));
    const lora_problem pr = a.probs ? gload<lora_problem>(a.probs + (int64_t)g * a.ns + c.slice) : a.single;
    const int4 td = gload<int4>(tiles + tile);
    setup_rows(a, td, n_active, M);
    if (M.nact > 0 && (MODE == MODE_SHRINK || c.o_lo < c.o_hi)) {
      if constexpr (SMAX > 1) {
        if (M.nact > 1) {
          mfma_tile_stacked<JT, SMAX>(a, pr, td.z, c.o_lo, c.o_hi, c.d_out, M, stage);
          return;
        }
      }
      mfma_tile<JT, HS, MODE>(a, pr, td.z, c.o_lo, c.o_hi, c.d_out, M, stage, vpark);
    }
  }, a.mfma_uniform != 0);
}

template <int JT, int HS, int MODE, int NSL>
__global__ __launch_bounds__(kThreads) void mfma_kernel(ApplyArgs a) {
  mfma_kernel_body<JT, HS, MODE, 1, NSL>(a);
}

// The stacked-slot build, held to two waves per SIMD (two workgroups per CU):
// left to itself the compiler would give the wide stacks more registers and
// halve the occupancy.  Launched for single-slice calls only.
template <int JT, int SMAX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void mfma_stacked_kernel(ApplyArgs a) {
  mfma_kernel_body<JT, 1, MODE_FUSED, SMAX, 1>(a);
}

// Sliced launches with one slot per request and 2 .. SMAX slices a group: one
// item per row tile for all the group's slices.  When the slices read the same
// x (the intended use, checked here per group) the tile walks x once for
// every slice's intermediate; otherwise it walks it once per slice.  Held to
// two waves per SIMD like the stacked build.
template <int JT, int SMAX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void mfma_sliced_kernel(ApplyArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Meta &M = *reinterpret_cast<Meta *>(smem);
  uint16_t *stage = reinterpret_cast<uint16_t *>(smem + kMetaBytes);
  const PlanHdr ph = read_plan_header(a);
  if (!ph.ok) return;
  const int n_m64 = ph.n_m, n_ms = ph.n_ms, n_active = ph.n_active;
  // the plan's 48-row tiling under the same rule as mfma_kernel_body's
  const bool small = (int64_t)n_m64 * a.n_problems > a.n_cu && (int64_t)n_ms * a.n_problems <= a.mfma_slots;
  const int n_m = small ? n_ms : n_m64;
  const int4 *tiles = small ? a.tiles_ms : a.tiles_m;
  const int ns = a.ns;
  walk_items((int64_t)n_m * a.n_problems, 1, [&](int64_t item) {
    const int g = int(item / n_m);
    const int tile = n_m - 1 - int(item - (int64_t)g * n_m);  // longest first, as in mfma_kernel_body
    const lora_problem *gp = a.probs + (int64_t)g * ns;
    const int4 td = gload<int4>(tiles + tile);
    setup_rows(a, td, n_active, M);
    if (M.nact > 0) {
      const lora_problem q0 = gload<lora_problem>(gp);
      bool same = true;
      for (int p = 1; p < ns; ++p) {
        const lora_problem q = gload<lora_problem>(gp + p);
        same = same && q.x == q0.x && q.ldx == q0.ldx;
      }
      // one pass over every slice, or (different x) one pass per slice
      const int passes = same ? 1 : ns;
      for (int p = 0; p < passes; ++p)
        mfma_tile_stacked<JT, SMAX, true>(a, q0, td.z, 0, 0, 0, M, stage, gp, same ? 0 : p, same ? ns : 1);
    }
  }, a.mfma_uniform != 0);
}

// Launch one instantiation; the first launch lifts its dynamic-LDS limit to
// the 160 KB a gfx950 workgroup may use.
template <int JT, int HS, int M, int NSL>
hipError_t launch_one(const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  static const bool lds_limit_raised =
      raise_lds_limit(reinterpret_cast<const void *>(&mfma_kernel<JT, HS, M, NSL>), kMaxLdsBytes);
  (void)lds_limit_raised;
  hipLaunchKernelGGL((mfma_kernel<JT, HS, M, NSL>), dim3(grid), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

template <int JT, int SMAX>
hipError_t launch_sliced(const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  static const bool lds_limit_raised =
      raise_lds_limit(reinterpret_cast<const void *>(&mfma_sliced_kernel<JT, SMAX>), kMaxLdsBytes);
  (void)lds_limit_raised;
  hipLaunchKernelGGL((mfma_sliced_kernel<JT, SMAX>), dim3(grid), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

template <int JT, int SMAX>
hipError_t launch_stacked(const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  static const bool lds_limit_raised =
      raise_lds_limit(reinterpret_cast<const void *>(&mfma_stacked_kernel<JT, SMAX>), kMaxLdsBytes);
  (void)lds_limit_raised;
  hipLaunchKernelGGL((mfma_stacked_kernel<JT, SMAX>), dim3(grid), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

// Launches with several output slices are fused ones (lora_apply_sliced).
template <int JT, int HS>
hipError_t launch_jt(int mode, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  if (a.ns > 1)
    return mode == MODE_FUSED ? launch_one<JT, HS, MODE_FUSED, LORA_MAX_SLICES>(a, grid, smem, stream)
                              : hipErrorInvalidValue;
  switch (mode) {
    case MODE_FUSED: return launch_one<JT, HS, MODE_FUSED, 1>(a, grid, smem, stream);
    case MODE_SHRINK: return launch_one<JT, HS, MODE_SHRINK, 1>(a, grid, smem, stream);
    case MODE_EXPAND: return launch_one<JT, HS, MODE_EXPAND, 1>(a, grid, smem, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Meta + staging + the parked intermediate of up to `slots` slots.
template <int JT, int HS>
size_t smem_of(int slots) {
  return kMetaBytes + MfmaCfg<JT, HS>::LDS + size_t(slots) * kMfmaRows * MfmaCfg<JT, HS>::VST * 2;
}

size_t mfma_smem_bytes(int jt, int slots, bool half) {
  switch (jt) {
    case 1: return smem_of<1, 1>(slots);
    case 2: return smem_of<2, 1>(slots);
    case 4: return half ? smem_of<4, 2>(slots) : smem_of<4, 1>(slots);
    case 8: return half ? smem_of<8, 2>(slots) : smem_of<8, 1>(slots);
  }
  return 0;
}

// Half stages are built for ranks 64 and 128 only: smaller ranks park little.
bool mfma_half_available(int jt) { return jt == 4 || jt == 8; }

// The stacked-slot build: meta + the larger of the stacked A stages and the
// single-slot path's staging with one parked intermediate.
template <int JT, int SMAX>
size_t stacked_smem_of() {
  const size_t single = MfmaCfg<JT, 1>::LDS + size_t(kMfmaRows) * MfmaCfg<JT, 1>::VST * 2;
  return kMetaBytes + (StackCfg<JT, SMAX>::LDS > single ? StackCfg<JT, SMAX>::LDS : single);
}

size_t mfma_stacked_smem_bytes(int jt, int smax) {
  switch (jt * 16 + smax) {
    case 16 + 2: return stacked_smem_of<1, 2>();
    case 16 + 3: return stacked_smem_of<1, 3>();
    case 16 + 4: return stacked_smem_of<1, 4>();
    case 32 + 2: return stacked_smem_of<2, 2>();
    case 32 + 3: return stacked_smem_of<2, 3>();
    case 32 + 4: return stacked_smem_of<2, 4>();
    case 64 + 2: return stacked_smem_of<4, 2>();
    case 64 + 3: return stacked_smem_of<4, 3>();
    case 64 + 4: return stacked_smem_of<4, 4>();
    case 128 + 2: return stacked_smem_of<8, 2>();
    case 128 + 3: return stacked_smem_of<8, 3>();
    case 128 + 4: return stacked_smem_of<8, 4>();
  }
  return 0;
}

hipError_t launch_mfma_stacked(int jt, int smax, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  switch (jt * 16 + smax) {
    case 16 + 2: return launch_stacked<1, 2>(a, grid, smem, stream);
    case 16 + 3: return launch_stacked<1, 3>(a, grid, smem, stream);
    case 16 + 4: return launch_stacked<1, 4>(a, grid, smem, stream);
    case 32 + 2: return launch_stacked<2, 2>(a, grid, smem, stream);
    case 32 + 3: return launch_stacked<2, 3>(a, grid, smem, stream);
    case 32 + 4: return launch_stacked<2, 4>(a, grid, smem, stream);
    case 64 + 2: return launch_stacked<4, 2>(a, grid, smem, stream);
    case 64 + 3: return launch_stacked<4, 3>(a, grid, smem, stream);
    case 64 + 4: return launch_stacked<4, 4>(a, grid, smem, stream);
    case 128 + 2: return launch_stacked<8, 2>(a, grid, smem, stream);
    case 128 + 3: return launch_stacked<8, 3>(a, grid, smem, stream);
    case 128 + 4: return launch_stacked<8, 4>(a, grid, smem, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_sliced(int jt, int nsl, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  switch (jt * 16 + nsl) {
    case 16 + 2: return launch_sliced<1, 2>(a, grid, smem, stream);
    case 16 + 3: return launch_sliced<1, 3>(a, grid, smem, stream);
    case 16 + 4: return launch_sliced<1, 4>(a, grid, smem, stream);
    case 32 + 2: return launch_sliced<2, 2>(a, grid, smem, stream);
    case 32 + 3: return launch_sliced<2, 3>(a, grid, smem, stream);
    case 32 + 4: return launch_sliced<2, 4>(a, grid, smem, stream);
    case 64 + 2: return launch_sliced<4, 2>(a, grid, smem, stream);
    case 64 + 3: return launch_sliced<4, 3>(a, grid, smem, stream);
    case 64 + 4: return launch_sliced<4, 4>(a, grid, smem, stream);
    case 128 + 2: return launch_sliced<8, 2>(a, grid, smem, stream);
    case 128 + 3: return launch_sliced<8, 3>(a, grid, smem, stream);
    case 128 + 4: return launch_sliced<8, 4>(a, grid, smem, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma(int mode, int jt, bool half, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  switch (jt) {
    case 1: return launch_jt<1, 1>(mode, a, grid, smem, stream);
    case 2: return launch_jt<2, 1>(mode, a, grid, smem, stream);
    case 4: return half ? launch_jt<4, 2>(mode, a, grid, smem, stream) : launch_jt<4, 1>(mode, a, grid, smem, stream);
    case 8: return half ? launch_jt<8, 2>(mode, a, grid, smem, stream) : launch_jt<8, 1>(mode, a, grid, smem, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
