// Tree-verify entry: dispatch on the state dtype to the per-dtype kernel files.
#include "ssu_device.h"
#include "ssu_internal.h"

namespace ssu {

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
