// moe_permute_noalloc: the token-dispatch permutation for callers that
// cannot allocate device memory.  Its scratch (the entry ranks and the
// chunk histogram of the permutation kernels) is a static device array of
// this file instead of a caller workspace.
//
// In host code the array's name stands for a host-side shadow, not a device
// address, so it is never passed to a kernel or a copy: the first call on a
// device looks up that device's copy with hipGetSymbolAddress (each GPU holds
// its own copy at its own address) and every later call passes that pointer
// to the kernels exactly as moe_permute passes its workspace.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the current device's scratch, looked up once per device.
hipError_t scratch_address(void** out) {
    static DeviceSetup setup;
    long long addr = 0, unused = 0;
    const hipError_t err = device_setup(setup, addr, unused, [](int, long long& a, long long&) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || ((uintptr_t)p & 255u)) return hipErrorInvalidValue;
        a = (long long)(uintptr_t)p;
        return hipSuccess;
    });
    *out = (void*)(uintptr_t)addr;
    return err;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_permute_noalloc(const int32_t* topk_ids, const uint16_t* x, int T, int d,
                                   int E, int k, int32_t* counts, int32_t* offsets,
                                   int32_t* dest, int32_t* src, uint16_t* x_perm,
                                   uint32_t* d_flags, void* stream) {
    const int st = permute_arg_checks(topk_ids, x, T, d, E, k, counts, offsets, dest, src, x_perm);
    if (st != MOE_OK) return st;
    if (permute_workspace_bytes(T, k, E) > kScratchBytes) return MOE_ERR_SCRATCH;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
    return launch_permute(topk_ids, x, T, d, E, k, counts, offsets, dest, src, x_perm, d_flags, ws,
                          (hipStream_t)stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}
