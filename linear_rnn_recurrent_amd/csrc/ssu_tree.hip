// Tree-verify entry: dispatch on the state dtype to the per-dtype kernel files,
// and the library-owned scratch of the allocation-free variant.
#include <mutex>

#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {

// The B . C workspace of ssu_tree_verify_noalloc: one copy per device, alive
// until the process ends. Host code never uses this name as an address (on
// the host it is only a stand-in for the symbol): tree_scratch() looks the
// device address up once per device.
static __device__ __align__(256) unsigned char scratch[SSU_TREE_SCRATCH_BYTES];

hipError_t tree_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_tree(const TreeParams &p, hipStream_t stream)
{
    if (p.d.batch == 0 || p.num_nodes == 0)
        return hipSuccess;
    switch (p.d.state_dtype) {
    case kF32: return launch_tree_f32(p, stream);
    case kF16: return launch_tree_f16(p, stream);
    case kBF16: return launch_tree_bf16(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
