// Kernel instantiations for one element type (bf16) and B layout (col-major).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(bf16_col, DT_BF16, 1)
}  // namespace spt
