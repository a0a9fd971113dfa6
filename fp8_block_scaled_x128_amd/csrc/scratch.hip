// scratch.hip -- device memory the library owns statically, one copy per GPU (each device that
// loads the library's code object holds its own copy until the process ends):
//   - `scratch`: the split-K partial tiles and arrival counters of fp8gemm_nt_noalloc, the dense
//     entry point for callers that cannot allocate (code under HIP graph capture, serving loops,
//     harnesses that forbid hipMalloc);
//   - the device error word every kernel reports precondition breaks into.
// Both start at zero when the code object is loaded.  Host code never passes these arrays'
// names to a kernel or a copy: the names are host-side stand-ins, not device addresses.  The
// device addresses come from hipGetSymbolAddress, once per device with that device current
// (scratch_pointers, called by the library's per-device set-up), and only those are used.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8gemm_internal.h"

namespace fp8gemm {

// fp32 partials first, then the counters (kScratchPartialBytes is a multiple of 256)
static __device__ __align__(256) uint8_t scratch[kScratchPartialBytes + kScratchCounters * sizeof(int32_t)];
static __device__ __align__(256) int32_t device_error_word[64];

int scratch_pointers(ScratchPointers* out) {
    void* s = nullptr;
    void* e = nullptr;
    if (hipGetSymbolAddress(&s, HIP_SYMBOL(scratch)) != hipSuccess || s == nullptr) return -1;
    if (hipGetSymbolAddress(&e, HIP_SYMBOL(device_error_word)) != hipSuccess || e == nullptr) return -1;
    out->partials = static_cast<float*>(s);
    out->counters = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(s) + kScratchPartialBytes);
    out->err = static_cast<int32_t*>(e);
    return 0;
}

}  // namespace fp8gemm
