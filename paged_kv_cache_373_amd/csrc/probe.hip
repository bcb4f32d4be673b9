// probe.hip - the benchmark's read probe, built on its own into
// libpkv_probe.so (not part of libpagedkv.so or its C ABI).
//
// A trivial read kernel that measures the streaming-read ceiling the decode
// kernels are held against: it reads whole 2 KiB tiles (one (block, head) K
// or V tile at B = 16, D = 64) in a caller-given order and does nothing with
// them but fold them into one word per thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeTileBytes = 2048;
constexpr int kProbeThreads = 256;
constexpr int kProbeTilesPerGroup = 32;  // 64 KiB per workgroup, all loads in flight at once

// Workgroup g reads tiles order[32 g .. 32 g + 31]: per step j the first 128
// threads read tile order[32 g + 2 j], the other 128 tile order[32 g + 2 j + 1],
// 16 bytes per thread, so every load instruction covers two whole tiles.
__global__ void __launch_bounds__(kProbeThreads)
    read_tiles(const u32x4_t* __restrict__ src, const int32_t* __restrict__ order,
               uint32_t* __restrict__ sink) {
  constexpr int kSteps = kProbeTilesPerGroup / 2;
  const int half = threadIdx.x >> 7;
  const int l = threadIdx.x & 127;
  const int32_t* ord = order + static_cast<size_t>(blockIdx.x) * kProbeTilesPerGroup;
  int tile[kSteps];
#pragma unroll
  for (int j = 0; j < kSteps; ++j) tile[j] = ord[2 * j + half];
  u32x4_t v[kSteps];
#pragma unroll
  for (int j = 0; j < kSteps; ++j)
    v[j] = src[static_cast<size_t>(tile[j]) * (kProbeTileBytes / 16) + l];
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kSteps; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  sink[static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = x;
}

}  // namespace

// Reads num_tiles tiles of 2048 bytes from `src` (device, 16-byte aligned),
// tile order[i] (device int32, each in range) being the i-th read, and writes
// one folded word per thread to `sink` (device, num_tiles * 8 uint32).
// num_tiles must be a positive multiple of 32.  Returns 0, -1 for an invalid
// argument (nothing enqueued) or -4 for a launch error.
extern "C" int pkv_probe_read_tiles(const void* src, const int32_t* order, int64_t num_tiles,
                                    uint32_t* sink, void* stream) {
  if (num_tiles <= 0 || num_tiles % kProbeTilesPerGroup != 0 ||
      num_tiles / kProbeTilesPerGroup > 0x7FFFFFFF)
    return -1;
  if (src == nullptr || order == nullptr || sink == nullptr ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return -1;
  const dim3 grid(static_cast<unsigned>(num_tiles / kProbeTilesPerGroup));
  read_tiles<<<grid, kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4_t*>(src), order, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
