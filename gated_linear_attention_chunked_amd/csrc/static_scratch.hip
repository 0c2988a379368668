// Allocation-free hybrid forward: lizard_hybrid_fwd with its scratch memory
// taken from a fixed device array instead of a caller workspace, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops).
//
// The array lives in this library's code object, so every device the library
// runs on holds its own copy, at its own address, until the process ends.  On
// the host, `scratch` names a host-side stand-in, not device memory: its device
// address is resolved once per device with hipGetSymbolAddress and only that
// pointer is ever handed to the kernels.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/lizard.h"

namespace {

// Largest forward workspace any accepted shape needs is B*H*(G-1) <= 255
// segment states of (128*128 + 128) floats, 16.06 MiB; the array leaves room
// above that.
constexpr size_t kScratchBytes = LIZARD_STATIC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of `scratch` on the current device (resolved on the first
// call for that device), or nullptr with *err set.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_err[dev];
  return g_ptr[dev];
}

}  // namespace

namespace lz {
lizard_status_t hybrid_fwd_args(const lizard_desc_t* desc, const void* q, const void* k,
                                const void* v, const void* gate, const void* meta_k,
                                const void* meta_v, const void* o, const void* ring_k,
                                const void* ring_v, const void* q_w, const void* k_w);
}

extern "C" {

lizard_status_t lizard_hybrid_fwd_static(const lizard_desc_t* desc, const void* q, const void* k,
                                         const void* v, const void* gate, const void* meta_k,
                                         const void* meta_v, const float* h0, void* o,
                                         float* lse, void* o_swa, float* hT, void* ring_k,
                                         void* ring_v, const void* q_w, const void* k_w,
                                         hipStream_t stream) {
  // every argument check of lizard_hybrid_fwd runs first, before any HIP call
  const lizard_status_t st =
      lz::hybrid_fwd_args(desc, q, k, v, gate, meta_k, meta_v, o, ring_k, ring_v, q_w, k_w);
  if (st != LIZARD_OK) return st;
  const size_t need = lizard_workspace_bytes(desc, LIZARD_OP_HYBRID_FWD);
  if (need > kScratchBytes) return LIZARD_E_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {  // problems that need no scratch never look the array up
    hipError_t e = hipSuccess;
    ws = scratch_ptr(&e);
    if (!ws) return LIZARD_E_HIP;
  }
  return lizard_hybrid_fwd(desc, q, k, v, gate, meta_k, meta_v, h0, o, lse, o_swa, hT, ring_k,
                           ring_v, q_w, k_w, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
