// Split-K reduction: C = cvt(epilogue(sum_s W[s])).
//
// When a problem has too few output tiles to fill the chip (a few hundred
// rows of A against a large B), the tile kernels split K into `splits`
// slices and each slice writes its fp32 partial tile to a workspace.  This
// kernel then sums the partials of each element in slice order (so the result
// does not depend on scheduling), applies the same epilogue as the tile
// kernels -- (acc * sa(m)) * sb(n), + bias[n], activation -- and converts.
//
// Bound: HBM.  Bytes per element: 4 * splits read + out_bytes written (plus
// the epilogue vectors, which stay in cache).  Each thread handles 8
// consecutive columns of one row (N is a multiple of 16), i.e. two 16-byte
// loads per slice, coalesced across the wave.
#include "device.hpp"
#include "kernels.hpp"

#include <mutex>

namespace tg {

constexpr int kReduceThreads = 256;
constexpr int kReduceCols = 8;           // columns per thread

template <int OUT>
__global__ __launch_bounds__(kReduceThreads) void split_reduce_kernel(const SplitReduceArgs a)
{
    const size_t per_row = (size_t)a.N / kReduceCols;
    const size_t item = (size_t)blockIdx.x * kReduceThreads + threadIdx.x;
    if (item >= (size_t)a.M * per_row)
        return;
    const int row = (int)(item / per_row);
    const int col = (int)(item - (size_t)row * per_row) * kReduceCols;
    const size_t plane = (size_t)a.M * (size_t)a.N;
    const float *w = a.W + (size_t)row * a.N + col;
    f32x4 lo = *(const f32x4 *)w, hi = *(const f32x4 *)(w + 4);
    for (int s = 1; s < a.splits; ++s) {
        const float *ws = w + (size_t)s * plane;
        const f32x4 l2 = *(const f32x4 *)ws, h2 = *(const f32x4 *)(ws + 4);
        lo += l2;
        hi += h2;
    }
    const EpiView ev = epi_view(a.epi, a.M, a.N);
    const float sa = epi_row_scale(ev, row);
    float v[kReduceCols] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int t = 0; t < kReduceCols; t += 2) {
        float sb[2], bz[2];
        epi_col2(ev, col + t, sb, bz);
        v[t] = epi_apply1(ev, v[t], sa, sb[0], bz[0]);
        v[t + 1] = epi_apply1(ev, v[t + 1], sa, sb[1], bz[1]);
    }
    if constexpr (OUT == kOutF32) {
        float *c = (float *)a.C + (size_t)row * a.N + col;
        *(f32x4 *)c = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4 *)(c + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
        uint16_t *c = (uint16_t *)a.C + (size_t)row * a.N + col;
        *(u32x4 *)c = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])};
    }
}

hipError_t launch_split_reduce(const SplitReduceArgs &a, hipStream_t s)
{
    const size_t items = (size_t)a.M * (size_t)(a.N / kReduceCols);
    const size_t blocks = (items + kReduceThreads - 1) / kReduceThreads;
    if (a.out == kOutF32)
        hipLaunchKernelGGL(split_reduce_kernel<kOutF32>, dim3((unsigned)blocks), dim3(kReduceThreads), 0, s, a);
    else
        hipLaunchKernelGGL(split_reduce_kernel<kOutBf16>, dim3((unsigned)blocks), dim3(kReduceThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The library's own split-K workspace, for callers that cannot allocate
// (gemm_run_ws_noalloc): one statically sized device array, held on every
// GPU the library runs on until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory; its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever handed to kernels.  Every call on
// one GPU shares the array, so calls that overlap in time on one GPU race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void **ptr)
{
    static std::mutex mu;
    static void *addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace tg
