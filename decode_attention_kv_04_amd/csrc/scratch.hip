// Static device scratch for decode_attn_run_noalloc: the split states that
// decode_attn_run keeps in a caller-provided workspace live here instead, in
// one file-scope device array per GPU, so that a caller that cannot allocate
// (code under HIP graph capture, tight serving loops) needs no workspace.
//
// The array is part of the library's code object: every GPU the library runs
// on holds its own copy, of kScratchBytes, until the process ends. On the
// host the array's name is only a stand-in for the symbol, never a device
// address: the address is looked up once per device (with that device
// current) and kept, and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "decode_attn.h"
#include "kernels.h"

static_assert(DECODE_ATTN_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[DECODE_ATTN_SCRATCH_BYTES];

namespace da {

namespace {
std::mutex g_scratch_mutex;
std::unordered_map<int, void*> g_scratch_ptr;  // device ordinal -> address of that device's array
}  // namespace

hipError_t scratch_address(int device, void** ptr) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  auto it = g_scratch_ptr.find(device);
  if (it != g_scratch_ptr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  int current = -1;
  hipError_t e = hipGetDevice(&current);
  if (e != hipSuccess) return e;
  if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (current != device) {
    const hipError_t back = hipSetDevice(current);
    if (e == hipSuccess) e = back;
  }
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[device] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace da
