// Kernel instantiations for one element type (f16) and B layout (col-major).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(f16_col, DT_F16, 1)
}  // namespace spt
