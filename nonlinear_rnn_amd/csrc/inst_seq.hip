// Kernel instantiations: step-by-step sequential application.
#include "launch.hpp"

namespace pararnn {

hipError_t launch_sequential(bool lstm, bool bf16, hipStream_t st, const SeqArgs &a)
{
    const dim3 grid((unsigned)((a.channels + kWave - 1) / kWave)), block(kWave);
    if (!lstm && !bf16)
        hipLaunchKernelGGL((sequential_kernel<GruCell, 32, false>), grid, block, 0, st, a);
    else if (!lstm)
        hipLaunchKernelGGL((sequential_kernel<GruCell, 32, true>), grid, block, 0, st, a);
    else if (!bf16)
        hipLaunchKernelGGL((sequential_kernel<LstmCell, 16, false>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((sequential_kernel<LstmCell, 16, true>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace pararnn
