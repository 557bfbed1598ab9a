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

// Block-scale image of an MX operand (layout in BscaleArgs): thread t writes
// the 16 bytes of lane t % 64 of (row quad, group) t / 64.
__global__ __launch_bounds__(256) void bscale_image_kernel(const BscaleArgs p)
{
    const int64_t total = (int64_t)p.quads * p.groups * 64;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(t & 63);
        const int64_t qg = t >> 6;
        const int g = (int)(qg % p.groups);
        const int64_t quad = qg / p.groups;
        uint32_t word[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t row = p.form ? quad * 64 + (b >> 1) * 32 + (lane & 31) : quad * 64 + b * 16 + (lane & 15);
            uint32_t w = 0;
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) {
                // 32-element block along K
                const int64_t blk = p.form ? (int64_t)16 * g + 2 * (2 * sl + (b & 1)) + (lane >> 5)
                                           : (int64_t)(4 * g + sl) * 4 + (lane >> 4);
                const uint32_t v = (row < p.rows && blk < p.kblocks) ? p.src[row * p.kblocks + blk] : 127u;
                w |= v << (8 * sl);
            }
            word[b] = w;
        }
        *(u32x4 *)(p.dst + t * 16) = u32x4{word[0], word[1], word[2], word[3]};
    }
}

hipError_t launch_bscale_image(const BscaleArgs &a, hipStream_t s)
{
    const int64_t total = (int64_t)a.quads * a.groups * 64;
    if (total == 0)
        return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(bscale_image_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace tg
