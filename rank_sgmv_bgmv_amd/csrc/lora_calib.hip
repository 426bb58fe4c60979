// Gather-read probe (include/lora_calib.h): a measurement aid, not part of
// any LoRA call.  One 256-thread workgroup reads its blocks of a pool with
// 16-byte loads, eight in flight per lane (32 KB per round for the
// workgroup), a workgroup barrier between blocks, optionally reads and writes
// back a small slice of a second buffer, and XORs what it read into one word.
// Blocks of the size of one adapter's A or B, scattered over a pool, two per
// workgroup with a y-row-sized slice, reproduce the decode kernel's traffic
// without any of its arithmetic.

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
