// Kernel instantiation: the input projection (MFMA GEMM).
#define PARARNN_DEFINE_PROJECT_KERNEL
#include "project.hpp"

namespace pararnn {

hipError_t launch_project(hipStream_t st, const ProjArgs &a)
{
    const int64_t groups = (int64_t)a.tiles_m * a.tiles_n * a.B;
    hipLaunchKernelGGL(project_kernel, dim3((unsigned)groups), dim3(proj::kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace pararnn
