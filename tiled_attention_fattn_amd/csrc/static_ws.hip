// A library-owned device workspace for callers that cannot allocate device
// memory (work recorded under graph capture, tight serving loops, harnesses
// that forbid allocation): fattn_bwd_noalloc runs the backward with its row
// statistics in this buffer instead of a caller-supplied workspace.
//
// The buffer is a file-scope device array, so every GPU that loads the
// library's code object holds its own copy until the process ends. In host
// code the array's name is only a host-side stand-in: its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and that address, never the name, is what the kernels receive.
// Every call on one GPU shares that GPU's copy: calls that overlap on one
// GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fattn_launch.h"

namespace {

static __device__ __align__(256) char scratch[fattn::kStaticWorkspaceBytes];

std::mutex g_mu;
void* g_scratch_ptr[64];  // device address of `scratch` per device id (null: not looked up)

}  // namespace

namespace fattn {

hipError_t static_workspace(int device, void** ptr) {
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace fattn
