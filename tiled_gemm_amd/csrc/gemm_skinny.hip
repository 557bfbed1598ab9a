// Skinny GEMM (M <= 64): C = A * B^T when B is the only large operand and
// the product is bound by streaming B from HBM once.
//
// One workgroup of 8 waves owns 32 columns of C (two 16-column MFMA blocks)
// and every row.  The K range is split among the waves by interleaving
// 128-byte steps (wave w takes steps w, w+8, ...), so at any moment the
// workgroup streams one contiguous 1 KiB span of each of its 32 B rows.
// Operands go straight from global memory into VGPRs with 16-byte buffer
// loads, several steps ahead; the MFMA operand layout is the same as in the
// tiled kernel (lane l: row l % 16, K chunks l / 16 and 4 + l / 16).  The
// eight partial 16x16 tiles per output block are summed through LDS in a
// fixed wave order (deterministic), then scaled, converted and stored.
#include "device.hpp"
#include "kernels.hpp"

namespace tg {

constexpr int kSkinnyWaves = kSkinnyThreads / 64;
constexpr int kSkinnyDepth = 4;        // K steps loaded before the first is consumed

template <int MB, int ELEM, int OUT>
__global__ __launch_bounds__(kSkinnyThreads, 1) void gemm_skinny_kernel(const SkinnyArgs p)
{
    constexpr int NB = kSkinnyTileN / 16;           // column blocks per workgroup
    constexpr int ROWS = MB * 16;
    __shared__ __attribute__((aligned(16))) float red[kSkinnyWaves][ROWS][kSkinnyTileN];

    const int w = wave_id();
    const int l = lane_id();
    const int q = l >> 4, r16 = l & 15;
    const int n0 = blockIdx.x * kSkinnyTileN;
    const uint32_t kb = (uint32_t)p.kbytes;
    const int rows_b = min(p.N - n0, kSkinnyTileN);
    const auto rA = make_rsrc(p.A, (uint32_t)p.M * kb);
    const auto rB = make_rsrc((const uint8_t *)p.B + (size_t)n0 * kb, (uint32_t)rows_b * kb);
    const int nk = p.k_tiles;
    const bool ragged = p.tail_bytes != kTileKBytes;

    uint32_t voffA[MB], voffB[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
        voffA[i] = (uint32_t)(i * 16 + r16) * kb + (uint32_t)q * kChunkBytes;
#pragma unroll
    for (int j = 0; j < NB; ++j)
        voffB[j] = (uint32_t)(j * 16 + r16) * kb + (uint32_t)q * kChunkBytes;

    struct Step {
        u32x4 a[MB][2];
        u32x4 b[NB][2];
    };
    auto load = [&](int kt, Step &st) {
        const uint32_t soff = (uint32_t)kt * kTileKBytes;
        const bool part = ragged && kt == nk - 1;     // second 64 bytes absent
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            st.b[j][0] = buf_load16(rB, voffB[j], soff);
            st.b[j][1] = part ? u32x4{0, 0, 0, 0} : buf_load16(rB, voffB[j] + 64u, soff);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            st.a[i][0] = buf_load16(rA, voffA[i], soff);
            st.a[i][1] = part ? u32x4{0, 0, 0, 0} : buf_load16(rA, voffA[i] + 64u, soff);
        }
    };

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Step &st) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if constexpr (ELEM == kBf16) {
                    acc[i][j] = mfma_bf16(st.b[j][0], st.a[i][0], acc[i][j]);
                    acc[i][j] = mfma_bf16(st.b[j][1], st.a[i][1], acc[i][j]);
                } else {
                    acc[i][j] = mfma_fp8(st.b[j][0], st.b[j][1], st.a[i][0], st.a[i][1], acc[i][j]);
                }
            }
    };

    // Steps of this wave: w, w + 8, w + 16, ...  Process them in groups of
    // kSkinnyDepth: all loads of a group are issued before its MFMAs.
    Step st[kSkinnyDepth];
    for (int base = w; base < nk; base += kSkinnyDepth * kSkinnyWaves) {
#pragma unroll
        for (int d = 0; d < kSkinnyDepth; ++d) {
            const int kt = base + d * kSkinnyWaves;
            if (kt < nk)
                load(kt, st[d]);
        }
#pragma unroll
        for (int d = 0; d < kSkinnyDepth; ++d) {
            const int kt = base + d * kSkinnyWaves;
            if (kt < nk)
                compute(st[d]);
        }
    }

    // ---- cross-wave reduction in a fixed order, then the epilogue.
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[w][i * 16 + r16][j * 16 + 4 * q + v] = acc[i][j][v];
    __syncthreads();

    float sa = 1.f, sb = 1.f;
    if (p.scale != nullptr) {
        sa = p.scale[0];
        sb = p.scale[1];
    }
    constexpr int OB = OUT == kOutF32 ? 4 : 2;
    const uint32_t ldc = (uint32_t)p.N * OB;
    const auto rC = make_rsrc(p.C, (uint32_t)p.M * ldc);
    // Each thread finishes pairs of adjacent outputs.
    for (int o = threadIdx.x * 2; o < ROWS * kSkinnyTileN; o += kSkinnyThreads * 2) {
        const int row = o / kSkinnyTileN, col = o % kSkinnyTileN;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int ww = 0; ww < kSkinnyWaves; ++ww) {
            s0 += red[ww][row][col];
            s1 += red[ww][row][col + 1];
        }
        s0 = (s0 * sa) * sb;
        s1 = (s1 * sa) * sb;
        const int n = n0 + col;
        const uint32_t voff = (row < p.M && n < p.N) ? (uint32_t)row * ldc + (uint32_t)n * OB : kOobOffset;
        if constexpr (OUT == kOutF32)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__builtin_bit_cast(uint32_t, s0),
                                                        __builtin_bit_cast(uint32_t, s1)},
                                                  rC, voff, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(s0, s1), rC, voff, 0, 0);
    }
}

template <int MB, int ELEM, int OUT>
static hipError_t launch_skinny(const SkinnyArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, ELEM, OUT>), dim3(grid), dim3(kSkinnyThreads), 0, s, a);
    return hipGetLastError();
}

#define TG_SKINNY(MB, ELEM, OUT) \
    SkinnyVariant{MB, ELEM, OUT, kSkinnyWaves * MB * 16 * kSkinnyTileN * 4, &launch_skinny<MB, ELEM, OUT>}

static const SkinnyVariant kSkinny[] = {
    TG_SKINNY(1, kBf16, kOutBf16), TG_SKINNY(2, kBf16, kOutBf16), TG_SKINNY(4, kBf16, kOutBf16),
    TG_SKINNY(1, kBf16, kOutF32),  TG_SKINNY(2, kBf16, kOutF32),  TG_SKINNY(4, kBf16, kOutF32),
    TG_SKINNY(1, kFp8, kOutBf16),  TG_SKINNY(2, kFp8, kOutBf16),  TG_SKINNY(4, kFp8, kOutBf16),
};

const SkinnyVariant *skinny_variants(int *count)
{
    *count = (int)(sizeof(kSkinny) / sizeof(kSkinny[0]));
    return kSkinny;
}

}  // namespace tg
