// Kernel instantiations for one element type (bf16) and B layout (row-major).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(bf16_row, DT_BF16, 0)
}  // namespace spt
