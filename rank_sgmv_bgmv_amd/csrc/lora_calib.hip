// Gather-read probe (include/lora_calib.h): a measurement aid, not part of
// any LoRA call.  One 256-thread workgroup reads its blocks of a pool with
// 16-byte loads, eight in flight per lane (32 KB per round for the
// workgroup), a workgroup barrier between blocks, optionally reads and writes
// back a small slice of a second buffer, and XORs what it read into one word.
// Blocks of the size of one adapter's A or B, scattered over a pool, two per
// workgroup with a y-row-sized slice, reproduce the decode kernel's traffic
// without any of its arithmetic.
//
// Tile-stream probe: the traffic of the MFMA kernel's prefill tiles without
// their arithmetic -- a tile's rows of x read stage by stage, then its rows
// of y read and written back stage by stage, with a stage of A or B read
// beside each -- or the same rows of x and y streamed whole rows at a time.

#include "lora_device.hpp"
#include "lora_calib.h"

namespace lora {
namespace {

constexpr int kCalibThreads = 256;
constexpr int kCalibInFlight = 8;  // 16-byte loads per lane per round
constexpr int kCalibRound = kCalibThreads * kCalibInFlight * 16;
constexpr int kCalibRmwPiece = kCalibThreads * 16;
constexpr int kCalibRmwMax = 4;  // 16-byte pieces per lane held across the last block

__global__ __launch_bounds__(kCalibThreads) void gather_read_kernel(const unsigned char *pool, const int64_t *off,
                                                                    int bpg, int block_bytes, unsigned char *rmw,
                                                                    int rmw_bytes, uint32_t *sink) {
  __shared__ uint32_t part[kCalibThreads / 64];
  const int g = blockIdx.x;
  uint4 x = make_uint4(0, 0, 0, 0);
  uint4 keep[kCalibRmwMax];
  const int npiece = rmw ? rmw_bytes / kCalibRmwPiece : 0;
  unsigned char *mine = rmw ? rmw + (int64_t)g * rmw_bytes : nullptr;
  for (int k = 0; k < bpg; ++k) {
    if (k == bpg - 1) {
#pragma unroll
      for (int p = 0; p < kCalibRmwMax; ++p)
        if (p < npiece) keep[p] = gload_at<uint4>(mine, uint32_t((p * kCalibThreads + threadIdx.x) * 16));
    }
    const unsigned char *base = pool + gload<int64_t>(off + (int64_t)g * bpg + k);
    for (int r0 = 0; r0 < block_bytes; r0 += kCalibRound) {
      uint4 v[kCalibInFlight];
#pragma unroll
      for (int i = 0; i < kCalibInFlight; ++i)
        v[i] = gload_at<uint4>(base, uint32_t(r0 + (i * kCalibThreads + threadIdx.x) * 16));
#pragma unroll
      for (int i = 0; i < kCalibInFlight; ++i) {
        x.x ^= v[i].x;
        x.y ^= v[i].y;
        x.z ^= v[i].z;
        x.w ^= v[i].w;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < kCalibRmwMax; ++p) {
    if (p < npiece) {
      uint4 v = keep[p];
      asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));  // an opaque value: the store stays
      gstore_at(mine, uint32_t((p * kCalibThreads + threadIdx.x) * 16), v);
    }
  }
  uint32_t w = x.x ^ x.y ^ x.z ^ x.w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) w ^= __shfl_xor(w, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) gstore(sink + g, part[0] ^ part[1] ^ part[2] ^ part[3]);
}

constexpr int kTileXStage = 512;   // bytes of each row of x per shrink stage (256 bf16 columns)
constexpr int kTileYStage = 256;   // bytes of each row of y per expand stage (128 bf16 outputs)
constexpr int kTileAStage = 32768; // bytes of A per shrink stage (64 ranks x 256 columns)
constexpr int kTileBStage = 16384; // bytes of B per expand stage (128 outputs x 64 ranks)

__device__ __forceinline__ void xor_in(uint32_t &acc, const uint4 &v) { acc ^= v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kCalibThreads) void tile_stream_kernel(const unsigned char *x, unsigned char *y,
                                                                    const unsigned char *ad, int n_adapters,
                                                                    int rows, int row_bytes, int order,
                                                                    uint32_t *sink) {
  __shared__ uint32_t part[kCalibThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  const unsigned char *xb = x + (int64_t)t * rows * row_bytes;
  unsigned char *yb = y + (int64_t)t * rows * row_bytes;
  const int64_t a_bytes = (int64_t)(row_bytes / kTileXStage) * kTileAStage;
  const int64_t b_bytes = (int64_t)(row_bytes / kTileYStage) * kTileBStage;
  const unsigned char *A = ad ? ad + (int64_t)(t % n_adapters) * (a_bytes + b_bytes) : nullptr;
  const unsigned char *B = ad ? A + a_bytes : nullptr;
  uint32_t acc = 0;
  if (order == 0) {
    // lane (l16, kg) of wave w: row 16 w + l16, 16-byte pieces kg, kg + 4, ... of the row's stage
    const bool live = 16 * w + l16 < rows;
    const int64_t ro = (int64_t)(live ? 16 * w + l16 : 0) * row_bytes;
    for (int s = 0; s < row_bytes / kTileXStage; ++s) {
      uint4 v[kTileXStage / 64], a[kTileAStage / (kCalibThreads * 16)];
#pragma unroll
      for (int k = 0; k < kTileXStage / 64; ++k) v[k] = gload<uint4>(xb + ro + s * kTileXStage + 64 * k + 16 * kg);
      if (A) {
#pragma unroll
        for (int i = 0; i < kTileAStage / (kCalibThreads * 16); ++i)
          a[i] = gload<uint4>(A + (int64_t)s * kTileAStage + (i * kCalibThreads + tid) * 16);
      }
      __syncthreads();
      if (live) {
#pragma unroll
        for (int k = 0; k < kTileXStage / 64; ++k) xor_in(acc, v[k]);
      }
      if (A) {
#pragma unroll
        for (int i = 0; i < kTileAStage / (kCalibThreads * 16); ++i) xor_in(acc, a[i]);
      }
    }
    for (int s = 0; s < row_bytes / kTileYStage; ++s) {
      uint4 v[kTileYStage / 64], b[kTileBStage / (kCalibThreads * 16)];
#pragma unroll
      for (int k = 0; k < kTileYStage / 64; ++k) v[k] = gload<uint4>(yb + ro + s * kTileYStage + 64 * k + 16 * kg);
      if (B) {
#pragma unroll
        for (int i = 0; i < kTileBStage / (kCalibThreads * 16); ++i)
          b[i] = gload<uint4>(B + (int64_t)s * kTileBStage + (i * kCalibThreads + tid) * 16);
      }
      __syncthreads();
      if (B) {
#pragma unroll
        for (int i = 0; i < kTileBStage / (kCalibThreads * 16); ++i) xor_in(acc, b[i]);
      }
      if (live) {
#pragma unroll
        for (int k = 0; k < kTileYStage / 64; ++k) {
          xor_in(acc, v[k]);
          uint4 o = v[k];
          asm volatile("" : "+v"(o.x), "+v"(o.y), "+v"(o.z), "+v"(o.w));  // an opaque value: the store stays
          gstore(yb + ro + s * kTileYStage + 64 * k + 16 * kg, o);
        }
      }
    }
  } else {
    // whole rows: wave w takes rows w, w + 4, ... one after another, 1 KB per load instruction
    for (int r = w; r < rows; r += kCalibThreads / 64) {
      for (int c0 = 0; c0 < row_bytes; c0 += 8 * 1024) {
        uint4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int c = c0 + q * 1024 + lane * 16;
          v[q] = c < row_bytes ? gload<uint4>(xb + (int64_t)r * row_bytes + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) xor_in(acc, v[q]);
      }
    }
    for (int r = w; r < rows; r += kCalibThreads / 64) {
      for (int c0 = 0; c0 < row_bytes; c0 += 8 * 1024) {
        uint4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int c = c0 + q * 1024 + lane * 16;
          v[q] = c < row_bytes ? gload<uint4>(yb + (int64_t)r * row_bytes + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int c = c0 + q * 1024 + lane * 16;
          if (c < row_bytes) {
            xor_in(acc, v[q]);
            uint4 o = v[q];
            asm volatile("" : "+v"(o.x), "+v"(o.y), "+v"(o.z), "+v"(o.w));
            gstore(yb + (int64_t)r * row_bytes + c, o);
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m);
  if (lane == 0) part[w] = acc;
  __syncthreads();
  if (tid == 0) gstore(sink + t, part[0] ^ part[1] ^ part[2] ^ part[3]);
}

}  // namespace
}  // namespace lora

extern "C" lora_status lora_calib_gather_read(const void *pool, const int64_t *off, int32_t n_groups,
                                              int32_t blocks_per_group, int32_t block_bytes, void *rmw,
                                              int32_t rmw_bytes, int32_t lds_bytes, uint32_t *sink,
                                              hipStream_t stream) {
  if (!pool || !off || !sink || n_groups < 0) return LORA_EINVAL;
  if (blocks_per_group < 1 || block_bytes <= 0 || block_bytes % lora::kCalibRound != 0) return LORA_ESHAPE;
  if (rmw && (rmw_bytes <= 0 || rmw_bytes % lora::kCalibRmwPiece != 0 ||
              rmw_bytes > lora::kCalibRmwMax * lora::kCalibRmwPiece))
    return LORA_ESHAPE;
  if (lds_bytes < 0 || lds_bytes > 65536) return LORA_ESHAPE;
  if (n_groups == 0) return LORA_OK;
  static const bool lds_limit_raised =
      lora::raise_lds_limit(reinterpret_cast<const void *>(&lora::gather_read_kernel), lora::kMaxLdsBytes);
  (void)lds_limit_raised;
  hipLaunchKernelGGL(lora::gather_read_kernel, dim3(n_groups), dim3(lora::kCalibThreads), size_t(lds_bytes), stream,
                     static_cast<const unsigned char *>(pool), off, blocks_per_group, block_bytes,
                     static_cast<unsigned char *>(rmw), rmw ? rmw_bytes : 0, sink);
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_EHIP;
}

extern "C" lora_status lora_calib_tile_stream(const void *x, void *y, int32_t n_tiles, int32_t rows,
                                              int32_t row_bytes, const void *adapters, int32_t n_adapters,
                                              int32_t order, int32_t lds_bytes, uint32_t *sink,
                                              hipStream_t stream) {
  if (!x || !y || !sink || n_tiles < 0 || (adapters && n_adapters < 1)) return LORA_EINVAL;
  if (rows < 1 || rows > 64 || row_bytes < 1024 || row_bytes % 1024 != 0 || row_bytes > 65536 ||
      (order != 0 && order != 1) || lds_bytes < 0 || lds_bytes > 65536)
    return LORA_ESHAPE;
  if (n_tiles == 0) return LORA_OK;
  static const bool lds_limit_raised =
      lora::raise_lds_limit(reinterpret_cast<const void *>(&lora::tile_stream_kernel), lora::kMaxLdsBytes);
  (void)lds_limit_raised;
  hipLaunchKernelGGL(lora::tile_stream_kernel, dim3(n_tiles), dim3(lora::kCalibThreads), size_t(lds_bytes), stream,
                     static_cast<const unsigned char *>(x), static_cast<unsigned char *>(y),
                     static_cast<const unsigned char *>(adapters), n_adapters, rows, row_bytes, order, sink);
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_EHIP;
}
