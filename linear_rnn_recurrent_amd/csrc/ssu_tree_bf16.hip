// Tree-verify kernels for bf16_t state (template in ssu_tree_impl.h).
#include "ssu_tree_impl.h"

namespace ssu {

hipError_t launch_tree_bf16(const TreeParams &p, hipStream_t stream)
{
    return launch_tree_state<bf16_t>(p, stream);
}

}  // namespace ssu
