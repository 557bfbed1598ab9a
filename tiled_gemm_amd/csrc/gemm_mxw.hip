// MX GEMM C = A * B^T (MXFP4, MXFP8) on the 32x32x64 form of gfx950's scaled MFMA,
// 256 x 256 tiles (FlyDSL "Kernel Authoring" skill, section 6 "GEMM Pattern
// (Preshuffle)": B pre-shuffled into operand order, A staged through
// XOR-swizzled LDS, LDS ping-pong; section 3 "Runtime Loops with
// Loop-Carried Values" for the load-next / compute-current loop; the "FlyDSL
// Kernel authoring guide", section 4.3 "ROCm intrinsics", for the f8f6f4
// scaled MFMA family and its E8M0 block scales).
//
// Why a second MX kernel: a lane's 16-byte e2m1 operand feeds a 32x32x64
// MFMA (131072 flops) where the 16x16x128 shape does half that, so the A
// fragment reads from LDS per flop halve; the matrix unit alone runs either
// shape at over 92% of the e2m1 peak (8 waves per CU, independent
// accumulators), but one 16-byte LDS read per 32x32x64 MFMA interleaved with
// them already caps it near 64% (one read per two MFMAs: 80-84%).  The
// 32 x 32 accumulators also let MX run on 8 waves (the 16x16x128 MX kernel
// spills there).  Per 64-element K slice a lane feeds row
// l % 32 -- e2m1: one 16-byte chunk, elements 32 (l / 32) .. +31; e4m3: chunks
// l / 32 and 2 + l / 32 of the slice -- and one scale byte, for K block
// l / 32 of the slice.
//
// Workgroup: WAVES waves side by side along N; wave w owns all 256 rows and
// the WN = 256 / WAVES columns from WN w (JB = WN / 32 blocks of 32), i.e.
// 8 x JB accumulators of 32 x 32 in AGPRs.  Main-loop step: 128 bytes of K
// (e2m1: 256 elements, four 64-element slices; e4m3: two slices).
//
//   A   global -> LDS by loads that write LDS directly, ring of 4 stages of
//       32 KiB (rows of 128 bytes, 16-byte chunks XOR-swizzled); a fragment
//       is one or two 16-byte LDS reads (row 32 i + l % 32, the chunks above).
//   B   global -> VGPRs, 4 JB 16-byte loads per lane and step, issued one
//       step ahead into two register sets renamed by unrolling.  From the
//       pre-shuffled image, chunk c of the step for column n = WN w + 32 J +
//       l % 32 is 16-row block n / 16, k-block 2 kt + c / 4, quarter c % 4,
//       row n % 16: two 512-byte runs per wave load.
//   Scales from block-scale image form 1 (one record of 1 KiB per 64-row
//       quad and 512-element group, 2 steps of e2m1 or 4 of e4m3): lane l's
//       16 bytes hold, in word 2 u + par,
//       byte b, the scale of row 32 u + l % 32 of the quad for K block
//       2 s' + l / 32 of slice s' = 2 b + par.  One 16-byte load per quad and
//       group brings a lane every scale it feeds; op_sel picks the byte.
//   Sync  one barrier per step, PD groups before its end, after an exact vmcnt
//       wait for A's next stage; every load is issued unconditionally (steps
//       past the end read out of range and return zeros, whose products are
//       zero whatever the scale).
//   Epilogue (acc * s_a) * s_b (+ bias, activation) in fp32, RNE to bf16.
#include "device.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace tg {

namespace {

constexpr int W4_BM = 256;
constexpr int W4_BN = 256;
constexpr int W4_NS = 4;                                   // LDS stages of A
constexpr int W4_STAGE = W4_BM * kTileKBytes;              // 32 KiB

template <int N>
using xc = std::integral_constant<int, N>;

// The scaled MFMA with scale byte `byte` (a constant once the loops unroll).
__device__ inline void mxw(f32x16 &acc, u32x4 x, u32x4 y, uint32_t sx, uint32_t sy, int byte)
{
    switch (byte) {
    case 0: mfma_mx4w_a<0>(acc, x, y, sx, sy); break;
    case 1: mfma_mx4w_a<1>(acc, x, y, sx, sy); break;
    case 2: mfma_mx4w_a<2>(acc, x, y, sx, sy); break;
    default: mfma_mx4w_a<3>(acc, x, y, sx, sy); break;
    }
}
__device__ inline void mxw(f32x16 &acc, i32x8 x, i32x8 y, uint32_t sx, uint32_t sy, int byte)
{
    switch (byte) {
    case 0: mfma_mx8w_a<0>(acc, x, y, sx, sy); break;
    case 1: mfma_mx8w_a<1>(acc, x, y, sx, sy); break;
    case 2: mfma_mx8w_a<2>(acc, x, y, sx, sy); break;
    default: mfma_mx8w_a<3>(acc, x, y, sx, sy); break;
    }
}

}  // namespace

template <int ELEM, bool BPRE, int WAVES, int PD>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_mxw_kernel(const TiledArgs p)
{
    constexpr bool F8 = ELEM == kMx8;
    constexpr int SLICES = F8 ? 2 : 4;                     // 64-element K slices per step
    constexpr int W4_NG = 8 * SLICES;                      // groups per step: (row block, slice)
    constexpr int SPG = 8 / SLICES;                        // steps per scale group
    constexpr int BL = F8 ? 2 : 1;                         // chunks per row and slice
    constexpr int THREADS = 64 * WAVES;
    constexpr int WN = W4_BN / WAVES;                      // columns per wave
    constexpr int JB = WN / 32;                            // 32-column blocks per wave
    constexpr int AR = W4_STAGE / (THREADS * kChunkBytes); // A loads per lane and step
    constexpr int BR = JB * SLICES * BL;                   // B loads per lane and step (4 JB)
    constexpr int SL = 5;                                  // scale loads per group
    static_assert(JB >= 1 && WN % 32 == 0, "whole 32-column blocks per wave");
    static_assert(ELEM == kMx4 || ELEM == kMx8, "MX operands");
    static_assert(PD >= 1 && PD < W4_NG / 2, "prefetch distance");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[W4_NS * W4_STAGE];

    const int w = wave_id();
    const int l = lane_id();
    const int r32 = l & 31, g = l >> 5;

    const SplitK sk = split_k_of(p);
    int tm, tn;
    tile_of_wg(sk.wg, sk.grid, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m0 = tm * W4_BM, n0 = tn * W4_BN;
    const int rows_a = min(p.M - m0, W4_BM);
    const int rows_b = min(p.N - n0, W4_BN);
    const uint32_t kb = (uint32_t)p.kbytes;
    const uint32_t kbB = (uint32_t)p.kbytes_b;
    const auto rA = make_rsrc((const uint8_t *)p.A + (size_t)m0 * kb, (uint32_t)rows_a * kb);
    const auto rB = make_rsrc((const uint8_t *)p.B + (size_t)n0 * kbB, (uint32_t)rows_b * kbB);
    const int nk = sk.nk;
    const uint32_t tail = sk.tail;

    // ---- A: load r of a step lands at byte (r * WAVES + w) * 1024 + 16 l of
    // the stage, i.e. row pc / 8, physical chunk pc % 8; the lane fetches
    // logical chunk swz_chunk(row, pc % 8).
    uint32_t voffA[AR];
    uint32_t tailA = 0;
#pragma unroll
    for (int r = 0; r < AR; ++r) {
        const int pc = (r * WAVES + w) * 64 + l;
        const int row = pc >> 3;
        const int c = swz_chunk(row, pc & 7);
        voffA[r] = (uint32_t)row * kb + (uint32_t)c * kChunkBytes;
        tailA |= ((uint32_t)(c * kChunkBytes) < tail ? 1u : 0u) << r;
    }
    // ---- B: load b = (SLICES J + s) BL + h brings chunk c of the step of
    // column WN w + 32 J + r32: e2m1 c = 2 s + g, e4m3 c = 4 s + 2 h + g.
    uint32_t voffB[BR];
    uint32_t tailB = 0;
#pragma unroll
    for (int b = 0; b < BR; ++b) {
        const int J = b / (SLICES * BL), s = (b / BL) % SLICES, h = b % BL;
        const int n = WN * w + 32 * J + r32;
        const int c = F8 ? 4 * s + 2 * h + g : 2 * s + g;
        if constexpr (BPRE)
            voffB[b] = (uint32_t)(n >> 4) * 16u * kbB + (uint32_t)(c >> 2) * 1024u +
                       (uint32_t)((c & 3) * 16 + (n & 15)) * 16u;
        else
            voffB[b] = (uint32_t)n * kbB + (uint32_t)c * kChunkBytes;
        tailB |= ((uint32_t)(c * kChunkBytes) < tail ? 1u : 0u) << b;
    }
    constexpr uint32_t kBStep = BPRE ? 2048u : (uint32_t)kTileKBytes;

    // MASK false: the caller guarantees tile kt is whole and in range.
    auto issue_a_one = [&](int kt, int r, auto mask_c) {
        uint32_t vo = voffA[r];
        if constexpr (decltype(mask_c)::value) {
            const bool beyond = kt >= nk;
            const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
            vo = keep_or_oob(!beyond & (!part | (((tailA >> r) & 1u) != 0)), vo);
        }
        buf_load16_to_lds(rA, lds + (kt % W4_NS) * W4_STAGE + (r * WAVES + w) * 1024, vo,
                          (uint32_t)kt * kTileKBytes);
        issue_fence();
    };
    u32x4 bq[2][BR];
    auto issue_b_one = [&](int kt, auto set_c, int b, auto mask_c) {
        constexpr int S = decltype(set_c)::value;
        uint32_t vo = voffB[b];
        if constexpr (decltype(mask_c)::value) {
            const bool beyond = kt >= nk;
            const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
            vo = keep_or_oob(!beyond & (!part | (((tailB >> b) & 1u) != 0)), vo);
        }
        bq[S][b] = buf_load16(rB, vo, (uint32_t)kt * kBStep);
        issue_fence();
    };

    // ---- block scales of one group (two steps), from image form 1: one
    // 16-byte record slot per lane and quad, word 2 u + par for row half u and
    // slice parity par, byte s' / 2 for slice s' of the group.  A: the four
    // quads of the tile's rows; B: the quad of the wave's columns.
    const int G = p.s_groups;
    const auto rSA = make_rsrc(p.sa_img, (uint32_t)((p.M + 63) / 64) * (uint32_t)G * 1024u);
    const auto rSB = make_rsrc(p.sb_img, (uint32_t)((p.N + 63) / 64) * (uint32_t)G * 1024u);
    const uint32_t qb = (uint32_t)((n0 + WN * w) / 64);
    const int ub0 = ((WN * w) >> 5) & 1;                  // row half of the quad of block J = 0
    // B: with one 32-column block per wave only the two words of its row half
    // are loaded (8 bytes).
    using ScB = typename std::conditional<JB == 1, u32x2, u32x4>::type;
    u32x4 scA[4], scA_n[4];
    ScB scB, scB_n;
    auto issue_scales = [&](int g2) {
        const bool in = g2 < G;              // past the last group: out of range
#pragma unroll
        for (int Q = 0; Q < 4; ++Q)
            scA_n[Q] = buf_load16(
                rSA, keep_or_oob(in, ((uint32_t)(m0 / 64 + Q) * (uint32_t)G + (uint32_t)g2) * 1024u + (uint32_t)l * 16u),
                0);
        const uint32_t ob = (qb * (uint32_t)G + (uint32_t)g2) * 1024u + (uint32_t)l * 16u;
        if constexpr (JB == 1)
            scB_n = buf_load8(rSB, keep_or_oob(in, ob + (uint32_t)ub0 * 8u), 0);
        else
            scB_n = buf_load16(rSB, keep_or_oob(in, ob), 0);
        issue_fence();
    };

    f32x16 acc[8][JB];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int J = 0; J < JB; ++J)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][J][v] = 0.f;

    // ---- fragments: group t of a step = (row block t % 8, slice t / 8).
    using FragT = typename std::conditional<F8, i32x8, u32x4>::type;
    FragT fa[W4_NG];
    auto load_frag = [&](int stage, int t) {
        const int i = t & 7, s = t >> 3;
        const int row = 32 * i + r32;
        const uint8_t *base = lds + stage * W4_STAGE + row * kTileKBytes;
        if constexpr (F8)
            fa[t] = join32(lds_load16(base + swz_chunk(row, 4 * s + g) * kChunkBytes),
                           lds_load16(base + swz_chunk(row, 4 * s + 2 + g) * kChunkBytes));
        else
            fa[t] = lds_load16(base + swz_chunk(row, 2 * s + g) * kChunkBytes);
    };

    // Load issue order per step k: the next group's scales at the start of
    // its first step (k even), B(k+1) spread over the groups before the
    // barrier, A(k+3) over the groups after it.  At the start of step k, B(k)
    // needs every load issued after it done except A(k+2): vmcnt(AR).  At
    // barrier(k), A(k+1) has two B steps, one A step and one group of
    // scales behind it.
    constexpr int kVmStart = AR;
    constexpr int kVmBar0 = 2 * BR + AR;
    static_assert(kVmBar0 + SL < 64, "vmcnt is 6 bits");
    auto wait_vm = [&](auto n_c) {
        constexpr int n = decltype(n_c)::value;
        __builtin_amdgcn_s_waitcnt((kWaitVmcnt0 & ~0xC00F) | (n & 0xF) | ((n >> 4) << 14));
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // One step; CUR: its B register set, GP: its position in the scale group.
    auto step = [&](int kt, auto cur_c, auto gp_c, auto mask_c) {
        constexpr int CUR = decltype(cur_c)::value;
        constexpr int GP = decltype(gp_c)::value;
        // scale loads behind A(k+1): one group's when step k or k-1 starts a group
        constexpr int kVmBar = kVmBar0 + SL * ((GP == 0) + ((GP - 1 + SPG) % SPG == 0));
        const int st = kt % W4_NS;
        wait_vm(xc<kVmStart>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (GP == 0) {
#pragma unroll
            for (int Q = 0; Q < 4; ++Q)
                scA[Q] = scA_n[Q];
            scB = scB_n;
            issue_scales(kt / SPG + 1);
        }
#pragma unroll
        for (int t = 0; t < W4_NG; ++t) {
            if (t < W4_NG - PD) {
#pragma unroll
                for (int b = t * BR / (W4_NG - PD); b < (t + 1) * BR / (W4_NG - PD); ++b)
                    issue_b_one(kt + 1, xc<1 - CUR>{}, b, mask_c);
            } else {
                const int go = t - (W4_NG - PD);
                if (go == 0) {
                    wait_vm(xc<kVmBar>{});
                    barrier();
                }
#pragma unroll
                for (int r = go * AR / PD; r < (go + 1) * AR / PD; ++r)
                    issue_a_one(kt + W4_NS - 1, r, mask_c);
            }
            if (t + PD < W4_NG)
                load_frag(st, t + PD);
            else
                load_frag((kt + 1) % W4_NS, t + PD - W4_NG);
            const int i = t & 7, s = t >> 3;
            const int sg = SLICES * GP + s;                  // slice of the scale group
#pragma unroll
            for (int J = 0; J < JB; ++J) {
                const int b0 = (SLICES * J + s) * BL;
                const uint32_t sx = scB[JB == 1 ? (sg & 1) : 2 * J + (sg & 1)];
                const uint32_t sy = scA[i >> 1][2 * (i & 1) + (sg & 1)];
                if constexpr (F8)
                    mxw(acc[i][J], join32(bq[CUR][b0], bq[CUR][b0 + 1]), fa[t], sx, sy, sg >> 1);
                else
                    mxw(acc[i][J], bq[CUR][b0], fa[t], sx, sy, sg >> 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- prologue: group 0's scales, A tiles 0 .. NS-2 and B(0), then the
    // first fragments.
    using masked = std::true_type;
    using unmasked = std::false_type;
    issue_scales(0);
    for (int v = 1 - W4_NS; v < 0; ++v) {
        if (v == -1) {
#pragma unroll
            for (int b = 0; b < BR; ++b)
                issue_b_one(0, xc<0>{}, b, masked{});
        }
#pragma unroll
        for (int r = 0; r < AR; ++r)
            issue_a_one(v + W4_NS - 1, r, masked{});
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 & ~0x0F00);      // vmcnt(0) lgkmcnt(0)
    barrier();
#pragma unroll
    for (int t = 0; t < PD; ++t)
        load_frag(0, t);
    // Steps run in scale groups (2 or 4 steps); a step past nk is a phantom
    // on zeros.  A group whose loads (B up to kt + SPG, A up to kt + SPG +
    // NS - 2) all cover whole, in-range tiles runs without per-lane masks.
    int kt = 0;
    const int nfull = tail == (uint32_t)kTileKBytes ? nk : nk - 1;
    auto group = [&](int k0, auto mask_c) {
        step(k0, xc<0>{}, xc<0>{}, mask_c);
        step(k0 + 1, xc<1>{}, xc<1>{}, mask_c);
        if constexpr (SPG == 4) {
            step(k0 + 2, xc<0>{}, xc<2>{}, mask_c);
            step(k0 + 3, xc<1>{}, xc<3>{}, mask_c);
        }
    };
    for (; kt + SPG + W4_NS - 2 < nfull; kt += SPG)
        group(kt, unmasked{});
    for (; kt < nk; kt += SPG)
        group(kt, masked{});
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    mfma_drain_acc(acc);

    // ---- epilogue.  Lane l of block (i, J) holds C[32 i + r32][WN w + 32 J
    // + 8 u + 4 g + j] in acc[i][J][4 u + j].  Row blocks outside, the lane's
    // column runs inside, so a wave writes adjacent pieces of a C row back to
    // back.
    const EpiView ev = epi_view(p.epi, p.M, p.N);
    const uint32_t ldc = (uint32_t)p.N * 2u;
    const auto rC = make_rsrc((uint8_t *)sk.C + (size_t)m0 * ldc, (uint32_t)rows_a * ldc);
    f32x4 sbv[JB][4], bzv[JB][4];
#pragma unroll
    for (int J = 0; J < JB; ++J)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int col = n0 + WN * w + 32 * J + 8 * u + 4 * g;
            sbv[J][u] = epi_col_scale4(ev, col);
            bzv[J][u] = epi_bias4(ev, col);
        }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 32 * i + r32;
        const float sa = epi_row_scale(ev, m0 + row);
#pragma unroll
        for (int J = 0; J < JB; ++J)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int col = n0 + WN * w + 32 * J + 8 * u + 4 * g;
                const uint32_t voff = col < p.N ? (uint32_t)row * ldc + (uint32_t)col * 2u : kOobOffset;
                const f32x4 a = f32x4{acc[i][J][4 * u], acc[i][J][4 * u + 1], acc[i][J][4 * u + 2],
                                      acc[i][J][4 * u + 3]};
                const f32x4 v = epi_apply4(ev, a, sa, sbv[J][u], bzv[J][u]);
                buf_store8(rC, u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)}, voff);
            }
    }
}

template <int ELEM, bool BPRE, int WAVES, int PD>
static hipError_t launch_mxw(const TiledArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_mxw_kernel<ELEM, BPRE, WAVES, PD>), dim3(a.grid), dim3(64 * WAVES), 0, s, a);
    return hipGetLastError();
}

#define TG_MXW(ELEM, BPRE, WAVES, PD)                                                            \
    TiledVariant{W4_BM, W4_BN, 1, WAVES, ELEM, kOutBf16, BPRE, W4_NS * W4_STAGE, W4_NS,           \
                 &launch_mxw<ELEM, BPRE, WAVES, PD>}

// The first variant of each layout is the planner's choice; the rest are
// alternatives compiled into sweep builds only.
static const TiledVariant kMxw[] = {
    TG_MXW(kMx4, true, 8, 6),
    TG_MXW(kMx4, false, 8, 6),
    TG_MXW(kMx8, true, 8, 2),     // 2 (e4m3 fragments are 8 VGPRs: deeper prefetch spills)
    TG_MXW(kMx8, false, 8, 2),
#ifdef TGEMM_SWEEP
    // alternatives (sweep builds only): prefetch distances, one wave per SIMD
    TG_MXW(kMx4, true, 8, 4),     // 4
    TG_MXW(kMx4, true, 8, 5),
    TG_MXW(kMx4, true, 8, 7),
    TG_MXW(kMx4, true, 4, 6),     // 7: one wave per SIMD
    TG_MXW(kMx4, false, 4, 6),
#endif
};

const TiledVariant *mxw_variants(int *count)
{
    *count = (int)(sizeof(kMxw) / sizeof(kMxw[0]));
    return kMxw;
}

}  // namespace tg
