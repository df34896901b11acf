// Kernel instantiations for one element type (bf16).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(bf16, DT_BF16)
}  // namespace spt
