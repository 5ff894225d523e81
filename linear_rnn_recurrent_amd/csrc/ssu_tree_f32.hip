// Tree-verify kernels for float state (template in ssu_tree_impl.h).
#include "ssu_tree_impl.h"

namespace ssu {

hipError_t launch_tree_f32(const TreeParams &p, hipStream_t stream)
{
    return launch_tree_state<float>(p, stream);
}

}  // namespace ssu
