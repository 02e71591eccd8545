// Kernel instantiations: GruCell, bfloat16 projections, time blocks that
// certify each record a pass late (the long-sequence default with many
// channels), compiled with their own scheduler options (build.py).
#include "launch.hpp"

namespace pararnn {
PARARNN_DEFINE_DEFER_LAUNCHER(gru_bf16, GruCell, true)
}  // namespace pararnn
