// Decode without allocation: pkv_decode with its workspace (the split-KV
// partials and the balanced split's tile prefix sums) in a file-scope device
// array, for callers that cannot allocate device memory.
//
// The array lives in the library's code object, so every GPU the library
// runs on holds its own copy at its own address from the first use until the
// process ends. Host code never passes the array's name to a kernel (on the
// host that name is only a stand-in, not a device address): the address is
// looked up once per device with hipGetSymbolAddress, while that device is
// current, and kept.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pkv.h"
#include "pkv_launch.h"

namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the
// first call for that device.
pkv_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return PKV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

size_t pkv_noalloc_scratch_bytes(void) { return kScratchBytes; }

pkv_status pkv_decode_noalloc(const pkv_decode_params* params, const void* q,
                              const void* key_cache, const void* value_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* out,
                              float* out_f32, void* stream) {
  if (params == nullptr) return PKV_ERR_NULL;
  // A workspace beyond the array is refused before any GPU call. For invalid
  // params decode_workspace is 0 and pkv_decode's own checks report them.
  const size_t need = pkv::decode_workspace(params);
  if (need > kScratchBytes) return PKV_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const pkv_status st = scratch_for_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  return pkv::decode_call(params, q, key_cache, value_cache, block_table, seq_lens, out, out_f32,
                          ws, need, stream);
}

}  // extern "C"
