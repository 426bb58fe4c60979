// Apply kernels: the unmerged LoRA delta y += scale * (x A_i^T) B_i^T over the
// tiles of a plan, with three modes (fused, shrink only, expand only).
//
// "Serving several LoRAs, ControlNet and IP-Adapter", section "LoRA: merged or
// alongside": the unmerged form adds x A^T B^T to x W^T; A is r x d, B is
// d x r (here r x d_in and d_out x r).  "Exercises" (four requests): each
// group of requests that share a LoRA computes its own x A^T B^T, results go
// back to the original rows.  Comparison table, "Stacking several LoRAs":
// stacked adapters are summed, treated here as one adapter whose rank is the
// sum of the slots' ranks (the A's stacked by rows, the B's by columns).
//
// Work items.  A plan tile is a run of rows of one adapter group.  A work item
// is (problem, tile, output-column chunk); the grid walks items in an order
// that keeps every chunk of one tile, and neighbouring tiles of one adapter,
// on the same XCD (blockIdx % 8 is the XCD a workgroup is dispatched to), so
// the adapter's A and B are fetched from HBM once and re-read from that XCD's
// L2.  Every chunk recomputes the rank-r intermediate of its rows.
//
// Two tile bodies:
//   * VALU (decode / BGMV tiles, <= 16 rows, any rank, fp32 or bf16): the
//     shrink streams each adapter row of A with 16-byte loads along d_in,
//     every lane multiplies it with the matching piece of up to 8 token rows of
//     x, and a wave butterfly reduce-scatter plus an LDS sum over the four
//     waves yields the rank-r intermediate in LDS (fp32).  The expand streams
//     B rows with 16-byte loads, reduces each output over the lanes that share
//     a B row and stages the delta in LDS, so y is read and written with
//     coalesced 16-byte accesses.
//   * MFMA (prefill tiles of 64 rows, bf16, rank 16/32/64/128): wave w owns
//     rows 16w..16w+15.  Shrink: V^T = A x^T on v_mfma_f32_16x16x32_bf16 with
//     A staged through LDS (shared by the four waves) and x loaded straight
//     into operand registers; the result is scaled and rounded once to bf16
//     and kept in registers in exactly the layout the expand consumes.
//     Expand: Y^T += B V^T per 64-column chunk, B staged through LDS, y read
//     and written as 8-byte pieces of the accumulator layout.

#include "lora_internal.hpp"

namespace lora {
namespace {

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

__device__ __forceinline__ float dot2_bf(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// ----------------------------------------------------- element vector ops --
// A "vector" is 16 bytes (8 bf16 / 4 fp32) on the vector path, one element otherwise.
template <typename T, bool VEC> struct VOps;

template <> struct VOps<uint16_t, true> {
  static constexpr int E = 8;
  typedef uint4 V;
  static __device__ __forceinline__ V load(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
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
  static __device__ __forceinline__ void add_store(uint16_t *p, const float *d) {
    uint4 y = load(p);
    const float4 d0 = *reinterpret_cast<const float4 *>(d);
    const float4 d1 = *reinterpret_cast<const float4 *>(d + 4);
    uint4 o;
    o.x = pack_bf2(bf_lo(y.x) + d0.x, bf_hi(y.x) + d0.y);
    o.y = pack_bf2(bf_lo(y.y) + d0.z, bf_hi(y.y) + d0.w);
    o.z = pack_bf2(bf_lo(y.z) + d1.x, bf_hi(y.z) + d1.y);
    o.w = pack_bf2(bf_lo(y.w) + d1.z, bf_hi(y.w) + d1.w);
    *reinterpret_cast<uint4 *>(p) = o;
  }
};

template <> struct VOps<uint16_t, false> {
  static constexpr int E = 1;
  typedef uint16_t V;
  static __device__ __forceinline__ V load(const uint16_t *p) { return *p; }
  static __device__ __forceinline__ V zero() { return 0; }
  static __device__ __forceinline__ float dot(V a, V b, float acc) { return fmaf(bf_to_f(a), bf_to_f(b), acc); }
  static __device__ __forceinline__ float dotf(const float *v, V b, float acc) { return fmaf(v[0], bf_to_f(b), acc); }
  static __device__ __forceinline__ void add_store(uint16_t *p, const float *d) { *p = f_to_bf(bf_to_f(*p) + d[0]); }
};

template <> struct VOps<float, true> {
  static constexpr int E = 4;
  typedef float4 V;
  static __device__ __forceinline__ V load(const float *p) { return *reinterpret_cast<const float4 *>(p); }
  static __device__ __forceinline__ V zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ float dot(V a, V b, float acc) {
    acc = fmaf(a.x, b.x, acc); acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc); return fmaf(a.w, b.w, acc);
  }
  static __device__ __forceinline__ float dotf(const float *v, V b, float acc) {
    const float4 a = *reinterpret_cast<const float4 *>(v);
    return dot(a, b, acc);
  }
  static __device__ __forceinline__ void add_store(float *p, const float *d) {
    float4 y = load(p);
    const float4 a = *reinterpret_cast<const float4 *>(d);
    y.x += a.x; y.y += a.y; y.z += a.z; y.w += a.w;
    *reinterpret_cast<float4 *>(p) = y;
  }
};

template <> struct VOps<float, false> {
  static constexpr int E = 1;
  typedef float V;
  static __device__ __forceinline__ V load(const float *p) { return *p; }
  static __device__ __forceinline__ V zero() { return 0.f; }
  static __device__ __forceinline__ float dot(V a, V b, float acc) { return fmaf(a, b, acc); }
  static __device__ __forceinline__ float dotf(const float *v, V b, float acc) { return fmaf(v[0], b, acc); }
  static __device__ __forceinline__ void add_store(float *p, const float *d) { *p = *p + d[0]; }
};

// ------------------------------------------------------------- LDS layout --
constexpr int kMetaRows = kMfmaRows;  // rows of tile metadata
struct Meta {
  int t[kMetaRows];                    // token row
  int a[LORA_MAX_SLOTS];               // tile's adapters (compacted slot order)
  int nact;                            // valid slots
  int pad[3];
  int pos[kMetaRows][LORA_MAX_SLOTS];  // original slot index of compacted slot
  float sc[kMetaRows][LORA_MAX_SLOTS]; // scale of compacted slot
};
constexpr size_t kMetaBytes = (sizeof(Meta) + 255) & ~size_t(255);

constexpr int kAStride = 64 + 8;  // bf16 elements per staged A row (64 columns + pad)

__host__ __device__ inline size_t valu_smem(int kr_max) {
  return size_t(kRowBlock) * kr_max * 4 + size_t(kRowBlock) * kValuOutChunk * 4 + 4 * 64 * 4;
}
__host__ __device__ inline size_t mfma_smem(int r) {
  const size_t a = size_t(r) * kAStride * 2, b = size_t(64) * (r + 8) * 2;
  return a > b ? a : b;
}

// ------------------------------------------------------------ tile setup --
// Fill the tile's rows (token index, compacted slots, scales) into LDS.
__device__ void setup_rows(const ApplyArgs &a, int4 td, int n_active, Meta &M) {
  const int tid = threadIdx.x;
  const int p0 = td.x, q0 = td.y, nrows = td.z;
  if (tid < nrows) {
    const int p = p0 + tid;
    int lo = q0, hi = min(q0 + tid, n_active - 1);
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cumlen[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int s = a.sseg[lo];
    M.t[tid] = a.sst[lo] + (p - a.cumlen[lo]);
    int kk = 0;
    for (int k = 0; k < a.K; ++k) {
      const int ad = a.idx[(int64_t)s * a.K + k];
      if (ad < 0 || ad >= a.n) continue;
      M.pos[tid][kk] = k;
      M.sc[tid][kk] = a.scale ? a.scale[(int64_t)s * a.K + k] : 1.0f;
      if (tid == 0) M.a[kk] = ad;
      ++kk;
    }
    if (tid == 0) M.nact = kk;
  }
}

// Sum of one value per (lane, index) over the 64 lanes of a wave, for 64
// indices at once: a butterfly reduce-scatter, 63 exchanges in all.  Step S
// halves the values a lane holds: it keeps the half selected by lane bit S and
// adds the partner's copy of that half.  On return lane l holds the wave total
// of index l.
template <int S>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[64], int lane) {
  const bool upper = (lane & S) != 0;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const float send = upper ? v[i] : v[i + S];
    const float keep = upper ? v[i + S] : v[i];
    v[i] = keep + __shfl_xor(send, S);
  }
}

__device__ __forceinline__ float wave_reduce_scatter64(float (&v)[64]) {
  const int lane = threadIdx.x & 63;
  reduce_scatter_step<32>(v, lane);
  reduce_scatter_step<16>(v, lane);
  reduce_scatter_step<8>(v, lane);
  reduce_scatter_step<4>(v, lane);
  reduce_scatter_step<2>(v, lane);
  reduce_scatter_step<1>(v, lane);
  return v[0];
}

// ------------------------------------------------------------ VALU tile --
template <typename T, bool VEC, int MODE>
__device__ void valu_tile(const ApplyArgs &a, const lora_problem &pr, int nrows, int o_lo, int o_hi, Meta &M,
                          float *s_v, float *s_d, float *s_red) {
  typedef VOps<T, VEC> O;
  typedef typename O::V V;
  constexpr int E = O::E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r, d_in = a.d_in, d_out = a.d_out, nact = M.nact;
  const int KR = a.kr_max;
  const T *__restrict__ Ab = static_cast<const T *>(pr.A);
  const T *__restrict__ Bb = static_cast<const T *>(pr.B);
  const T *__restrict__ xb = static_cast<const T *>(pr.x);
  T *__restrict__ yb = static_cast<T *>(pr.y);

  if (MODE == MODE_SHRINK) {
    // zero the columns of empty slots of every row of the tile
    for (int w = tid; w < nrows * a.K; w += kThreads) {
      const int m = w / a.K, k = w % a.K;
      bool used = false;
      for (int kk = 0; kk < nact; ++kk) used |= (M.pos[m][kk] == k);
      if (!used) {
        float *vp = a.v + (int64_t)M.t[m] * a.ldv + (int64_t)k * r;
        for (int j = 0; j < r; ++j) vp[j] = 0.f;
      }
    }
  }

  for (int m0 = 0; m0 < nrows; m0 += kRowBlock) {
    const int nb = min(kRowBlock, nrows - m0);

    if (MODE != MODE_EXPAND) {
      // ---- shrink: s_v[m][kk*r + j] = sc * sum_c x[t_m][c] A[a_kk][j][c]
      const int nvx = d_in / E;
      const T *xrow[kRowBlock];
#pragma unroll
      for (int m = 0; m < kRowBlock; ++m) xrow[m] = xb + (int64_t)M.t[m0 + (m < nb ? m : 0)] * pr.ldx;
      for (int kk = 0; kk < nact; ++kk) {
        const T *Aa = Ab + (int64_t)M.a[kk] * r * d_in;
        for (int j0 = 0; j0 < r; j0 += 8) {
          float acc[64];
#pragma unroll
          for (int i = 0; i < 64; ++i) acc[i] = 0.f;
          for (int cv = tid; cv < nvx; cv += kThreads) {
            V xv[kRowBlock];
#pragma unroll
            for (int m = 0; m < kRowBlock; ++m) xv[m] = (m < nb) ? O::load(xrow[m] + (int64_t)cv * E) : O::zero();
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              if (j0 + jj < r) {
                const V av = O::load(Aa + (int64_t)(j0 + jj) * d_in + (int64_t)cv * E);
#pragma unroll
                for (int m = 0; m < kRowBlock; ++m)
                  if (m < nb) acc[m * 8 + jj] = O::dot(xv[m], av, acc[m * 8 + jj]);
              }
            }
          }
          const float val = wave_reduce_scatter64(acc);
          s_red[wave * 64 + lane] = val;
          __syncthreads();
          if (tid < 64) {
            const int m = tid >> 3, j = j0 + (tid & 7);
            if (m < nb && j < r) {
              float sum = (s_red[tid] + s_red[64 + tid]) + (s_red[128 + tid] + s_red[192 + tid]);
              sum *= M.sc[m0 + m][kk];
              if (MODE == MODE_SHRINK)
                a.v[(int64_t)M.t[m0 + m] * a.ldv + (int64_t)M.pos[m0 + m][kk] * r + j] = sum;
              else
                s_v[m * KR + kk * r + j] = sum;
            }
          }
          __syncthreads();
        }
      }
    } else {
      // ---- expand only: load the caller's intermediate (compacted) into LDS
      for (int w = tid; w < nb * nact * r; w += kThreads) {
        const int m = w / (nact * r), rem = w % (nact * r), kk = rem / r, j = rem % r;
        s_v[m * KR + kk * r + j] = a.v[(int64_t)M.t[m0 + m] * a.ldv + (int64_t)M.pos[m0 + m][kk] * r + j];
      }
      __syncthreads();
    }
    if (MODE == MODE_SHRINK) continue;

    // ---- expand: y[t_m][o] += sum_kk sum_j s_v[m][kk*r + j] B[a_kk][o][j]
    const int VR = r / E;  // vectors per B row
    int L = 1;
    while (L < VR && L < 64) L <<= 1;  // lanes sharing one B row (power of two)
    const int RP = kThreads / L;       // B rows per pass
    const int lr = tid & (L - 1), orow = tid / L;
    for (int ob = o_lo; ob < o_hi; ob += kValuOutChunk) {
      const int oe = min(ob + kValuOutChunk, o_hi);
      for (int o0 = ob; o0 < oe; o0 += RP) {
        const int o = o0 + orow;
        float pacc[kRowBlock];
#pragma unroll
        for (int m = 0; m < kRowBlock; ++m) pacc[m] = 0.f;
        if (o < oe) {
          for (int kk = 0; kk < nact; ++kk) {
            const T *Brow = Bb + ((int64_t)M.a[kk] * d_out + o) * r;
            for (int jv = lr; jv < VR; jv += L) {
              const V bv = O::load(Brow + jv * E);
#pragma unroll
              for (int m = 0; m < kRowBlock; ++m)
                if (m < nb) pacc[m] = O::dotf(s_v + m * KR + kk * r + jv * E, bv, pacc[m]);
            }
          }
        }
        for (int off = L >> 1; off >= 1; off >>= 1) {
#pragma unroll
          for (int m = 0; m < kRowBlock; ++m) pacc[m] += __shfl_xor(pacc[m], off);
        }
        if (lr == 0 && o < oe) {
#pragma unroll
          for (int m = 0; m < kRowBlock; ++m)
            if (m < nb) s_d[m * kValuOutChunk + (o - ob)] = pacc[m];
        }
      }
      __syncthreads();
      const int nov = (oe - ob) / E;
      for (int w = tid; w < nb * nov; w += kThreads) {
        const int m = w / nov, ov = w % nov;
        O::add_store(yb + (int64_t)M.t[m0 + m] * pr.ldy + ob + ov * E, s_d + m * kValuOutChunk + ov * E);
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------ MFMA tile --
__device__ __forceinline__ f32x4 mfma32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ f32x4 mfma16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                    0, 0);
}

// JT = rank / 16; KMAX = slots held in registers.
template <int JT, int MODE>
__device__ void mfma_tile(const ApplyArgs &a, const lora_problem &pr, int nrows, int o_lo, int o_hi, Meta &M,
                          uint16_t *stage) {
  constexpr int R = 16 * JT;
  constexpr int KMAX = (kMfmaMaxSlotRank / R) < LORA_MAX_SLOTS ? (kMfmaMaxSlotRank / R) : LORA_MAX_SLOTS;
  constexpr int NA = (R * 8 + kThreads - 1) / kThreads;  // 16-byte pieces per thread when staging A or B
  constexpr int BST = R + 8;                            // staged B row stride (elements)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  const int m = 16 * w + l16;  // this lane's tile row (operand row and output column)
  const bool row_ok = m < nrows;
  const int d_in = a.d_in, d_out = a.d_out;
  const int nact = M.nact;
  const uint16_t *__restrict__ Ab = static_cast<const uint16_t *>(pr.A);
  const uint16_t *__restrict__ Bb = static_cast<const uint16_t *>(pr.B);
  const uint16_t *__restrict__ xrow =
      static_cast<const uint16_t *>(pr.x) + (int64_t)M.t[row_ok ? m : 0] * pr.ldx;
  uint16_t *__restrict__ yrow = static_cast<uint16_t *>(pr.y) + (int64_t)M.t[row_ok ? m : 0] * pr.ldy;
  const bool wave_live = 16 * w < nrows;

  // packed bf16 intermediate: vp[kk][jt] = v[t][16 jt + 4 kg + 0..3] of compacted slot kk
  uint2 vp[KMAX][JT];

  // ---------------- shrink (or load of the intermediate) ----------------
#pragma unroll
  for (int kk = 0; kk < KMAX; ++kk) {
    if (kk >= nact) break;
    if (MODE == MODE_EXPAND) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row_ok)
          f = *reinterpret_cast<const float4 *>(a.v + (int64_t)M.t[m] * a.ldv + (int64_t)M.pos[m][kk] * R + 16 * jt +
                                                4 * kg);
        vp[kk][jt] = make_uint2(pack_bf2(f.x, f.y), pack_bf2(f.z, f.w));
      }
      continue;
    }
    const uint16_t *Aa = Ab + (int64_t)M.a[kk] * R * d_in;
    f32x4 acc[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 areg[NA];
    uint4 xreg[2];
    auto load_chunk = [&](int kc) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int e = tid + i * kThreads;
        const int row = e >> 3, cv = e & 7;
        areg[i] = make_uint4(0, 0, 0, 0);
        if (row < R && kc + cv * 8 < d_in) areg[i] = *reinterpret_cast<const uint4 *>(Aa + (int64_t)row * d_in + kc + cv * 8);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = kc + 32 * h + 8 * kg;
        xreg[h] = make_uint4(0, 0, 0, 0);
        if (row_ok && c < d_in) xreg[h] = *reinterpret_cast<const uint4 *>(xrow + c);
      }
    };
    load_chunk(0);
    for (int kc = 0; kc < d_in; kc += 64) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int e = tid + i * kThreads;
        const int row = e >> 3, cv = e & 7;
        if (row < R) *reinterpret_cast<uint4 *>(stage + row * kAStride + cv * 8) = areg[i];
      }
      const uint4 x0 = xreg[0], x1 = xreg[1];
      __syncthreads();
      if (kc + 64 < d_in) load_chunk(kc + 64);
      if (wave_live) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const uint16_t *ap = stage + (16 * jt + l16) * kAStride + 8 * kg;
          const uint4 a0 = *reinterpret_cast<const uint4 *>(ap);
          const uint4 a1 = *reinterpret_cast<const uint4 *>(ap + 32);
          acc[jt] = mfma32(a0, x0, acc[jt]);
          acc[jt] = mfma32(a1, x1, acc[jt]);
        }
      }
      __syncthreads();
    }
    // acc[jt][q] = v[t_m][16 jt + 4 kg + q] (unscaled)
    const float sc = row_ok ? M.sc[m][kk] : 0.f;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const f32x4 s = acc[jt] * sc;
      if (MODE == MODE_SHRINK) {
        if (row_ok)
          *reinterpret_cast<float4 *>(a.v + (int64_t)M.t[m] * a.ldv + (int64_t)M.pos[m][kk] * R + 16 * jt + 4 * kg) =
              make_float4(s[0], s[1], s[2], s[3]);
      } else {
        vp[kk][jt] = make_uint2(pack_bf2(s[0], s[1]), pack_bf2(s[2], s[3]));
      }
    }
  }
  if (MODE == MODE_SHRINK) {
    // zero the columns of empty slots
    for (int e = tid; e < nrows * a.K; e += kThreads) {
      const int mm = e / a.K, k = e % a.K;
      bool used = false;
      for (int kk = 0; kk < nact; ++kk) used |= (M.pos[mm][kk] == k);
      if (!used) {
        float *vq = a.v + (int64_t)M.t[mm] * a.ldv + (int64_t)k * R;
        for (int j = 0; j < R; ++j) vq[j] = 0.f;
      }
    }
    return;
  }

  // ---------------- expand ----------------
  for (int ob = o_lo; ob < o_hi; ob += 64) {
    // y pieces of this chunk: lane holds y[t][ob + 16 ot + 4 kg + 0..3]
    uint2 yold[4];
#pragma unroll
    for (int ot = 0; ot < 4; ++ot) {
      const int o = ob + 16 * ot + 4 * kg;
      yold[ot] = make_uint2(0, 0);
      if (row_ok && o < o_hi) yold[ot] = *reinterpret_cast<const uint2 *>(yrow + o);
    }
    f32x4 yacc[4];
#pragma unroll
    for (int ot = 0; ot < 4; ++ot) yacc[ot] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int kk = 0; kk < KMAX; ++kk) {
      if (kk >= nact) break;
      const uint16_t *Ba = Bb + ((int64_t)M.a[kk] * d_out + ob) * R;
      // stage B[ob .. ob+64)[0 .. R) into LDS
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int e = tid + i * kThreads;
        const int row = e / (R / 8), cv = e % (R / 8);
        if (row < 64) {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (ob + row < o_hi) v = *reinterpret_cast<const uint4 *>(Ba + (int64_t)row * R + cv * 8);
          *reinterpret_cast<uint4 *>(stage + row * BST + cv * 8) = v;
        }
      }
      __syncthreads();
      if (wave_live) {
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) {
          const uint16_t *bp = stage + (16 * ot + l16) * BST + 4 * kg;
#pragma unroll
          for (int h = 0; h < JT / 2; ++h) {
            const uint2 b0 = *reinterpret_cast<const uint2 *>(bp + 32 * h);
            const uint2 b1 = *reinterpret_cast<const uint2 *>(bp + 32 * h + 16);
            const uint4 aop = make_uint4(b0.x, b0.y, b1.x, b1.y);
            const uint2 v0 = vp[kk][2 * h], v1 = vp[kk][2 * h + 1];
            const uint4 bop = make_uint4(v0.x, v0.y, v1.x, v1.y);
            yacc[ot] = mfma32(aop, bop, yacc[ot]);
          }
          if (JT & 1) {
            const uint2 b0 = *reinterpret_cast<const uint2 *>(bp + 16 * (JT - 1));
            yacc[ot] = mfma16(b0, vp[kk][JT - 1], yacc[ot]);
          }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int ot = 0; ot < 4; ++ot) {
      const int o = ob + 16 * ot + 4 * kg;
      if (row_ok && o < o_hi) {
        const uint2 yo = yold[ot];
        const uint2 yn = make_uint2(pack_bf2(bf_lo(yo.x) + yacc[ot][0], bf_hi(yo.x) + yacc[ot][1]),
                                    pack_bf2(bf_lo(yo.y) + yacc[ot][2], bf_hi(yo.y) + yacc[ot][3]));
        *reinterpret_cast<uint2 *>(yrow + o) = yn;
      }
    }
  }
}

// ---------------------------------------------------------------- kernel --
template <typename T, bool VEC, int JT, int MODE>
__global__ __launch_bounds__(kThreads) void apply_kernel(ApplyArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  Meta &M = *reinterpret_cast<Meta *>(smem);
  unsigned char *work = smem + kMetaBytes;

  const int n_m = a.hdr[H_TILES_M], n_v = a.hdr[H_TILES_V], n_active = a.hdr[H_ACTIVE];
  const int64_t per_prob = (int64_t)n_m * a.cm + (int64_t)n_v * a.cv;
  const int64_t N = per_prob * a.n_problems;
  if (N == 0) return;
  const int xcd = blockIdx.x & 7, lb = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  const int64_t ipx = (N + 7) >> 3;

  for (int64_t i = lb; i < ipx; i += per_xcd) {
    const int64_t item = xcd * ipx + i;
    if (item >= N) break;
    const int p = int(item / per_prob);
    int64_t rem = item - (int64_t)p * per_prob;
    const bool is_m = rem < (int64_t)n_m * a.cm;
    int tile, chunk, width;
    if (is_m) {
      tile = int(rem / a.cm); chunk = int(rem % a.cm); width = a.wm;
    } else {
      rem -= (int64_t)n_m * a.cm;
      tile = int(rem / a.cv); chunk = int(rem % a.cv); width = a.wv;
    }
    const lora_problem pr = a.probs ? a.probs[p] : a.single;
    const int4 td = is_m ? a.tiles_m[tile] : a.tiles_v[tile];
    const int o_lo = chunk * width;
    const int o_hi = min(a.d_out, o_lo + width);
    setup_rows(a, td, n_active, M);
    __syncthreads();
    if (M.nact > 0 && (MODE == MODE_SHRINK || o_lo < o_hi)) {
      if constexpr (JT > 0) {
        if (is_m) {
          mfma_tile<JT, MODE>(a, pr, td.z, o_lo, o_hi, M, reinterpret_cast<uint16_t *>(work));
        } else {
          float *s_v = reinterpret_cast<float *>(work);
          valu_tile<T, VEC, MODE>(a, pr, td.z, o_lo, o_hi, M, s_v, s_v + kRowBlock * a.kr_max,
                                  s_v + kRowBlock * a.kr_max + kRowBlock * kValuOutChunk);
        }
      } else {
        float *s_v = reinterpret_cast<float *>(work);
        valu_tile<T, VEC, MODE>(a, pr, td.z, o_lo, o_hi, M, s_v, s_v + kRowBlock * a.kr_max,
                                s_v + kRowBlock * a.kr_max + kRowBlock * kValuOutChunk);
      }
    }
    __syncthreads();
  }
}

template <typename T, bool VEC, int JT, int MODE>
hipError_t launch_one(const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  hipLaunchKernelGGL((apply_kernel<T, VEC, JT, MODE>), dim3(grid), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

template <typename T, bool VEC, int JT>
hipError_t launch_mode(int mode, const ApplyArgs &a, int grid, size_t smem, hipStream_t stream) {
  switch (mode) {
    case MODE_FUSED: return launch_one<T, VEC, JT, MODE_FUSED>(a, grid, smem, stream);
    case MODE_SHRINK: return launch_one<T, VEC, JT, MODE_SHRINK>(a, grid, smem, stream);
    case MODE_EXPAND: return launch_one<T, VEC, JT, MODE_EXPAND>(a, grid, smem, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t apply_smem_bytes(int r, int kr_max, bool mfma) {
  size_t w = valu_smem(kr_max);
  if (mfma && mfma_smem(r) > w) w = mfma_smem(r);
  return kMetaBytes + w;
}

hipError_t launch_apply(int mode, int dtype, bool vec, int jt, const ApplyArgs &a, int grid, size_t smem,
                        hipStream_t stream) {
  if (dtype == LORA_F32) {
    return vec ? launch_mode<float, true, 0>(mode, a, grid, smem, stream)
               : launch_mode<float, false, 0>(mode, a, grid, smem, stream);
  }
  if (!vec) return launch_mode<uint16_t, false, 0>(mode, a, grid, smem, stream);
  switch (jt) {
    case 0: return launch_mode<uint16_t, true, 0>(mode, a, grid, smem, stream);
    case 1: return launch_mode<uint16_t, true, 1>(mode, a, grid, smem, stream);
    case 2: return launch_mode<uint16_t, true, 2>(mode, a, grid, smem, stream);
    case 4: return launch_mode<uint16_t, true, 4>(mode, a, grid, smem, stream);
    case 8: return launch_mode<uint16_t, true, 8>(mode, a, grid, smem, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
