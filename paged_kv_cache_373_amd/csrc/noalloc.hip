// noalloc.hip - pkv_paged_attention_decode_noalloc: paged decode attention
// whose split-KV scratch is a fixed device array of this library instead of
// a caller-provided workspace, for callers that cannot allocate.
//
// The array holds the same layout as a decode workspace: a leading counter
// region that must be zero when a call starts (every call leaves it zero)
// and per-piece partial results behind it.  Each device the library runs on
// has its own copy of the array, at its own address, held until the process
// ends.  The host never names the array in a kernel argument or a copy: it
// looks its device address up once per device (hipGetSymbolAddress with that
// device current) and passes that address on.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"

namespace pkv {
namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;  // PKV_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static_assert(kScratchBytes == PKV_NOALLOC_SCRATCH_BYTES, "header and library disagree");

struct DeviceScratch {
  void* ptr = nullptr;  // device address of `scratch` on this device
  size_t zeroed = 0;    // leading bytes known to be zero
};
std::mutex g_lock;
DeviceScratch g_dev[kMaxDevices];

// Zeroes words [begin, end) of a 4-byte-aligned device buffer.  A kernel of
// our own rather than a memset, so the clearing is an ordinary kernel node
// when a caller captures the call in a graph.
__global__ void zero_words(uint32_t* p, size_t begin, size_t end) {
  for (size_t i = begin + blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < end;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// The device the call's stream belongs to (the current device for the null
// stream).
hipError_t stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) return hipGetDevice(dev);
  return hipStreamGetDevice(s, dev);
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status pkv_paged_attention_decode_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* seq_lens, int32_t block_size, float scale, void* out,
    const pkv_decode_dims* dims, void* stream) {
  using namespace pkv;
  // Host checks first: nothing is looked up or enqueued for a call that
  // fails them, or whose scratch would not fit the array.
  const size_t need = pkv_decode_workspace_size(dims, block_size);
  if (need == static_cast<size_t>(-1)) return PKV_ERR_INVALID;
  if (need > kScratchBytes) return PKV_ERR_WORKSPACE;
  const size_t counters = pkv_decode_workspace_zeroed_bytes(dims, block_size);
  if (dims->num_seqs == 0) return PKV_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_tables == nullptr ||
      seq_lens == nullptr || out == nullptr)
    return PKV_ERR_INVALID;
  if (need == 0)
    return decode_entry(q, nullptr, nullptr, k_cache, v_cache, block_tables, seq_lens,
                        block_size, scale, out, dims, nullptr, 0, stream);

  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  if (stream_device(s, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> guard(g_lock);
  DeviceScratch& ds = g_dev[dev];
  if (ds.ptr == nullptr) {
    // Set-up, once per device, with that device current.
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return PKV_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return PKV_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return PKV_ERR_HIP;
    ds.ptr = p;
    ds.zeroed = 0;  // not assumed: the counters are cleared before first use
  }
  if (counters > ds.zeroed) {
    // The counter region grows over bytes an earlier call may have left
    // partial results in: clear them on the call's stream, first.
    const size_t words_begin = ds.zeroed / 4, words_end = counters / 4;
    const size_t n = words_end - words_begin;
    const unsigned blocks = static_cast<unsigned>(n < 256 * 256 ? (n + 255) / 256 : 256);
    zero_words<<<blocks, 256, 0, s>>>(static_cast<uint32_t*>(ds.ptr), words_begin, words_end);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  const pkv_status st = decode_entry(q, nullptr, nullptr, k_cache, v_cache, block_tables,
                                     seq_lens, block_size, scale, out, dims, ds.ptr,
                                     kScratchBytes, stream);
  // After the call the counter region is zero again and the bytes behind it
  // hold this call's partial results.
  if (st == PKV_OK) ds.zeroed = counters;
  return st;
}
