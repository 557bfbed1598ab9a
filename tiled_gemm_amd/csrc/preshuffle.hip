// B pre-shuffle: rewrite B (N x K row-major) into MFMA operand order.
//
// The image is the byte layout (N/16, Kb/64, 4, 16, 16):(16Kb, 1024, 256, 16, 1)
// of FlyDSL's preshuffle GEMM (Kernel Authoring skill, section 6 "GEMM
// Pattern (Preshuffle)" step 1; K counted in bytes, 16-byte kpack).  The
// same five coordinates address B itself through the layout
// (N/16, Kb/64, 4, 16, 16):(16Kb, 64, 16, Kb, 1).  Both layouts come from
// the host planner; each thread moves one 16-byte chunk, computing its
// source and destination with crd2idx on them.  A wave writes one 1 KiB
// block contiguously and reads 16 rows x 64 bytes.  HBM-bound: 2 |B| bytes.
#include "device.hpp"
#include "kernels.hpp"

namespace tg {

constexpr int kShufThreads = 256;

__global__ __launch_bounds__(kShufThreads) void preshuffle_b_kernel(const PreshuffleArgs p)
{
    const int l = lane_id();
    const int w = threadIdx.x >> 6;
    const int64_t kgroups = (p.kblocks + 3) / 4;          // 4 waves -> 4 k-blocks per workgroup
    const int64_t total = (int64_t)p.nblocks * kgroups;
    for (int64_t g = blockIdx.x; g < total; g += gridDim.x) {
        const int64_t nb = g / kgroups;
        const int64_t kblk = (g - nb * kgroups) * 4 + w;
        if (kblk >= p.kblocks)
            continue;
        const int64_t crd[5] = {nb, kblk, l >> 4, l & 15, 0};
        const int64_t src = crd2idx(p.src, crd);
        const int64_t dst = crd2idx(p.dst, crd);
        const u32x4 v = *(const u32x4 *)((const uint8_t *)p.B + src);
        *(u32x4 *)((uint8_t *)p.Bs + dst) = v;
    }
}

hipError_t launch_preshuffle(const PreshuffleArgs &a, hipStream_t s)
{
    const int64_t kgroups = (a.kblocks + 3) / 4;
    const int64_t total = (int64_t)a.nblocks * kgroups;
    if (total == 0)
        return hipSuccess;
    const int grid = (int)(total < 65536 * 4 ? total : 65536 * 4);
    hipLaunchKernelGGL(preshuffle_b_kernel, dim3(grid), dim3(kShufThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace tg
