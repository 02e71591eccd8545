// Kernel instantiation: the input projection (MFMA GEMM).
#define PARARNN_DEFINE_PROJECT_KERNEL
#include "project.hpp"

namespace pararnn {

hipError_t launch_project(hipStream_t st, const ProjArgs &a)
{
    const int64_t groups = (int64_t)a.tiles_m * a.tiles_n * a.B;
    const bool vec = a.I % proj::kBK == 0 && a.wsm % 8 == 0 && a.xst % 8 == 0 && a.xsb % 8 == 0 &&
                     (reinterpret_cast<uintptr_t>(a.w) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.x) & 15u) == 0;
    if (vec)
        hipLaunchKernelGGL(project_kernel<true>, dim3((unsigned)groups), dim3(proj::kThreads), 0,
                           st, a);
    else
        hipLaunchKernelGGL(project_kernel<false>, dim3((unsigned)groups), dim3(proj::kThreads), 0,
                           st, a);
    return hipGetLastError();
}

}  // namespace pararnn
