// Kernel instantiations: the standalone linear-recurrence scan.
#include "launch.hpp"

namespace pararnn {

#define PARARNN_SCAN_CASE(KK, WW)                                                               \
    case KK * 100 + WW:                                                                         \
        if (S == 1 && reverse)                                                                  \
            hipLaunchKernelGGL((scan_kernel<Map1, KK, WW, true>), grid, block, 0, st, a);       \
        else if (S == 1)                                                                        \
            hipLaunchKernelGGL((scan_kernel<Map1, KK, WW, false>), grid, block, 0, st, a);      \
        else if (reverse)                                                                       \
            hipLaunchKernelGGL((scan_kernel<Map2, KK, WW, true>), grid, block, 0, st, a);       \
        else                                                                                    \
            hipLaunchKernelGGL((scan_kernel<Map2, KK, WW, false>), grid, block, 0, st, a);      \
        break;

hipError_t launch_scan(int S, int K, int W, bool reverse, int64_t groups, hipStream_t st,
                       const ScanArgs &a)
{
    const dim3 grid((unsigned)groups), block((unsigned)(kWave * W));
    switch (K * 100 + W) {
        PARARNN_BASE_KW(PARARNN_SCAN_CASE)
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pararnn
