// Kernel instantiations for one element type (f16) and B layout (row-major).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(f16_row, DT_F16, 0)
}  // namespace spt
