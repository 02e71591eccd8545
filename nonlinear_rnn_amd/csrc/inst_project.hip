// Kernel instantiation: the input projection (MFMA GEMM).
#define PARARNN_DEFINE_PROJECT_KERNEL
#include "project.hpp"

namespace pararnn {

hipError_t launch_project(hipStream_t st, const ProjArgs &args)
{
    ProjArgs a = args;
    const bool vec = a.I % proj::kBK == 0 && a.wsm % 8 == 0 && a.xst % 8 == 0 && a.xsb % 8 == 0 &&
                     (reinterpret_cast<uintptr_t>(a.w) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.x) & 15u) == 0;
    // the ring kernel addresses a tile's rows with 32-bit byte offsets
    const bool ring = vec && a.I % proj::kRBK == 0 && a.wsm < (int64_t(1) << 22) &&
                      a.xst < (int64_t(1) << 22);
    const int64_t bn = ring ? proj::kRBN : proj::kBN;
    const int64_t tm = (a.M + proj::kBM - 1) / proj::kBM, tn = (a.T + bn - 1) / bn;
    a.tiles_m = (int32_t)tm;
    a.tiles_n = (int32_t)tn;
    // m tiles per group: their W tiles (kBM rows x I) together about 2 MB,
    // and at least 4 so that the x tiles in flight on an XCD are shared by
    // several workgroups (measured: 1 per group re-streams x per m tile)
    const int64_t wtile = (int64_t)proj::kBM * a.I * 2;
    int64_t gm = wtile > 0 ? (int64_t(2) << 20) / wtile : tm;
    if (gm < 4) gm = 4;
    a.group_m = (int32_t)(gm > tm ? tm : gm);
    const int64_t groups = tm * tn * a.B;
    if (ring)
        hipLaunchKernelGGL(project_kernel_ring, dim3((unsigned)groups), dim3(proj::kRThreads), 0,
                           st, a);
    else if (vec)
        hipLaunchKernelGGL(project_kernel<true>, dim3((unsigned)groups), dim3(proj::kThreads), 0,
                           st, a);
    else
        hipLaunchKernelGGL(project_kernel<false>, dim3((unsigned)groups), dim3(proj::kThreads), 0,
                           st, a);
    return hipGetLastError();
}

}  // namespace pararnn
