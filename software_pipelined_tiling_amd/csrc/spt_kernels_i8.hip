// Kernel instantiations for one element type (i8).
#include "spt_instances.hpp"

namespace spt {
SPT_DEFINE_TABLE(i8, DT_I8)
}  // namespace spt
