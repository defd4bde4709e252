// Split-KV forward for callers that cannot allocate device memory: code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
//
// fa_fwd_splitkv takes its float32 partials (one normalised O and one LSE per
// chunk and query row) from a workspace the caller allocates.  This entry
// point runs the same kernels with the partials in `scratch`, a static device
// array of FA_NOALLOC_SCRATCH_BYTES that every device the library runs on
// holds until the process ends.  It calls no hipMalloc, hipFree or other
// allocating routine.  The split kernel writes every partial it reads back
// (a chunk with no visible key for a row writes O = 0 and LSE = -inf), so the
// buffer needs no clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/fa.h"

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current.  In host code the array's name is only a
// host-side stand-in, never a device address: kernels and copies get the
// pointer returned here.
int scratch_on_current_device(void **out) {
    static std::mutex mu;
    static std::vector<void *> ptrs;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return FA_ERR_DEVICE;
        }
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_splitkv_noalloc(const fa_fwd_args *a, int num_splits) {
    const int64_t need = fa_splitkv_workspace_bytes(a, num_splits);
    // invalid arguments: fa_fwd_splitkv reports their status before any HIP call
    if (need < 0) return fa_fwd_splitkv(a, num_splits, nullptr, 0);
    if (need == 0) return FA_OK;  // empty problem
    if (need > (int64_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    void *ws = nullptr;
    const int st = scratch_on_current_device(&ws);
    if (st != FA_OK) return st;
    return fa_fwd_splitkv(a, num_splits, ws, (int64_t)FA_NOALLOC_SCRATCH_BYTES);
}
