// Software-pipelined GEMM C = A * B^T for 256 x 256 tiles, the kernel behind
// both layouts at large sizes (FlyDSL "Kernel Authoring" skill, section 6
// "GEMM Pattern (Preshuffle)": B pre-shuffled into MFMA operand order, A
// staged through XOR-swizzled LDS, 64-byte K micro-steps, LDS ping-pong;
// section 3 "Runtime Loops with Loop-Carried Values" for the prefetch-next /
// compute-current loop).
//
// B goes straight to VGPRs in both layouts.  Pre-shuffled, one wave load is
// one contiguous 1 KiB operand block; from the plain N x K layout, lane l
// loads the 16 bytes of row l % 16 at K chunk l / 16, i.e. 16 rows x 64
// contiguous bytes per wave load (the companion load for chunks 4..7 covers
// the other half of each 128-byte row segment).
//
// Workgroup: WAVES waves (two per SIMD at 8), 256 x 256 output tile, waves
// side by side along N (each wave owns all 256 rows and 256 / WAVES columns,
// so no B byte is loaded twice).  Main-loop step: 128 bytes of K.
//
//   A   global -> LDS by 16-byte buffer loads that write LDS directly, into a
//       ring of NS stages (NS - 2 tiles in flight beyond the one being read).
//   B   global -> VGPRs, two 16-byte loads per lane per 16-column block,
//       issued at the start of the step before its use, in two register sets
//       renamed by unrolling the loop.
//   LDS -> VGPR: the A fragments of a step form one ordered stream; each
//       fragment is requested PD groups before its MFMAs, and the first PD
//       fragments of step k+1 are requested during the last PD groups of
//       step k.
//   Sync: one barrier per step, placed PD groups before the step's end.  At
//       that point the wave waits (exact vmcnt) for A tile k+1, meets the
//       other waves, then issues A tile k+NS-1 into the stage every wave
//       finished reading in step k-1.  Every load is issued unconditionally
//       (tiles past the end read out of range and return zeros), so the
//       number of loads in flight behind any given load is fixed and the
//       vmcnt immediates are exact.
//   Epilogue as in the generic tiled kernel: (acc * s_a) * s_b, RNE to bf16,
//   buffer stores (rows past M and columns past N dropped).
#include "device.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace tg {

namespace {

constexpr int BP_BM = 256;
constexpr int BP_BN = 256;
constexpr int BP_STAGE = BP_BM * kTileKBytes;                       // 32 KiB of A per stage

template <int WGM, int WGN, int NS>
struct BpCfg {
    static constexpr int WAVES = WGM * WGN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WTM = BP_BM / WGM;                        // rows per wave
    static constexpr int WTN = BP_BN / WGN;                        // columns per wave
    static constexpr int FM = WTM / 16;                            // 16-row blocks per wave
    static constexpr int FN = WTN / 16;                            // 16-column blocks per wave
    static constexpr int AR = BP_STAGE / (THREADS * kChunkBytes);  // DMA rounds per stage
    static constexpr int LDS = NS * BP_STAGE;
    static_assert(NS >= 4, "the barrier schedule needs two stages beyond read/ready");
    static_assert(LDS <= 160 * 1024, "gfx950 LDS is 160 KiB per workgroup");
};

template <int N>
using ic = std::integral_constant<int, N>;

}  // namespace

// ELEM: kBf16 (2 x 16x16x32 per step) or kFp8 (1 x 16x16x128 per step).
// PD: fragment prefetch distance in groups.
// BPRE: B is the pre-shuffled image (true) or plain N x K (false).
// ADMA: A goes global -> LDS by the load's own LDS write (true) or through
// VGPRs: loaded at barrier(k), written with ds_write_b128 at barrier(k+1).
template <int ELEM, int OUT, bool BPRE, int WGM, int WGN, int NS, int PD, bool ADMA, bool ACCA, bool SPREAD>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_pipe_kernel(const TiledArgs p)
{
    using Cfg = BpCfg<WGM, WGN, NS>;
    constexpr int WAVES = Cfg::WAVES;
    constexpr int BP_FM = Cfg::FM, BP_FN = Cfg::FN, BP_AR = Cfg::AR;
    constexpr int BP_BR = BP_FN * (ELEM == kW4A8 ? 1 : 2);    // B loads per lane per step
    constexpr int BP_WTM = Cfg::WTM, BP_WTN = Cfg::WTN;
    // Fragment stream of one step: bf16 -> 2 sub-steps x 16 row blocks, one
    // 16-byte read each; fp8 -> 16 row blocks, two reads (chunks q, q+4).
    // WIDE: one 128-byte MFMA operand per block and step (fp8, MX e4m3);
    // otherwise two 64-byte halves (bf16, MX e2m1).
    constexpr bool WIDE = ELEM == kFp8 || ELEM == kMx8;
    constexpr bool MX = ELEM == kMx8 || ELEM == kMx4;
    // Integer operands: int8 A with int8 B (kI8) or packed int4 B (kW4A8).
    // An int4 step of B is 64 bytes per row: one 16-byte load per lane and
    // 16-column block (lane group q: values 32 q .. 32 q + 31 of the step),
    // unpacked into two int8 atom operands, half h pairing with A chunk
    // 2 q + h.
    constexpr bool INT = ELEM == kI8 || ELEM == kW4A8;
    constexpr bool W4 = ELEM == kW4A8;
    constexpr int BH = W4 ? 1 : 2;                           // B loads per block and step
    // Integer GEMMs write bf16; their fp32-output instances write split-K
    // partials (the int32 sums converted, times 1/16 for int4 B).
    constexpr int NG = WIDE ? BP_FM : 2 * BP_FM;            // groups (FN MFMAs each)
    static_assert(!MX || (ACCA && ADMA && BP_WTM % 64 == 0 && BP_WTN % 64 == 0),
                  "MX operands run on the AGPR-accumulator kernel, whole 64-row scale quads per wave");
    static_assert(PD >= 1 && PD < NG / 2, "prefetch distance");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg::LDS];

    const int w = wave_id();
    const int l = lane_id();
    const int q = l >> 4, r16 = l & 15;
    const int wm = w / WGN, wn = w % WGN;

    const SplitK sk = split_k_of(p);
    int tm, tn;
    tile_of_wg(sk.wg, sk.grid, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m0 = tm * BP_BM, n0 = tn * BP_BN;
    const int rows_a = min(p.M - m0, BP_BM);
    const int rows_b = min(p.N - n0, BP_BN);
    const uint32_t kb = (uint32_t)p.kbytes;
    const uint32_t kbB = (uint32_t)p.kbytes_b;
    // A split starts its operands' resources at its first K step (bytes of
    // that step: A 128 per row; B as kBStep below), so every step index below
    // is split-relative.  Only bf16 and fp8 plans split K: the MX scale
    // images are indexed by the absolute step.
    const uint32_t shA = (uint32_t)sk.kt0 * (uint32_t)kTileKBytes;
    const uint32_t shB =
        (uint32_t)sk.kt0 * (W4 ? (BPRE ? 1024u : 64u) : (BPRE ? 2048u : (uint32_t)kTileKBytes));
    const auto rA = make_rsrc((const uint8_t *)p.A + (size_t)m0 * kb + shA, (uint32_t)rows_a * kb - shA);
    const auto rB = make_rsrc((const uint8_t *)p.B + (size_t)n0 * kbB + shB, (uint32_t)rows_b * kbB - shB);
    const int nk = sk.nk;
    const uint32_t tail = sk.tail;

    // ---- A: global -> LDS source offsets, as in the generic kernel.
    uint32_t voffA[BP_AR];
    uint32_t tailA = 0;
#pragma unroll
    for (int r = 0; r < BP_AR; ++r) {
        const int pc = (r * WAVES + w) * 64 + l;
        const int row = pc >> 3;
        const int c = swz_chunk(row, pc & 7);
        voffA[r] = (uint32_t)row * kb + (uint32_t)c * kChunkBytes;
        tailA |= ((uint32_t)(c * kChunkBytes) < tail ? 1u : 0u) << r;
    }
    u32x4 stA[BP_AR];                           // staging (ADMA == false)
    int stA_tile = 0;
    // One A load (round r of tile kt), for the spread schedule below.
    // MASK false: the caller guarantees tile kt is whole and in range, so
    // the offsets need no per-lane selection.
    auto issue_a_one = [&](int kt, int r, auto mask_c) {
        uint32_t vo = voffA[r];
        if constexpr (decltype(mask_c)::value) {
            const bool beyond = kt >= nk;
            const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
            const bool keep = !beyond & (!part | (((tailA >> r) & 1u) != 0));
            vo = keep_or_oob(keep, vo);
        }
        buf_load16_to_lds(rA, lds + (kt % NS) * BP_STAGE + (r * WAVES + w) * 1024, vo, (uint32_t)kt * kTileKBytes);
        issue_fence();
    };
    auto issue_a = [&](int kt) {
        const bool beyond = kt >= nk;
        const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
        uint8_t *sA = lds + (kt % NS) * BP_STAGE;
        const uint32_t soff = (uint32_t)kt * kTileKBytes;
#pragma unroll
        for (int r = 0; r < BP_AR; ++r) {
            const bool keep = !beyond & (!part | (((tailA >> r) & 1u) != 0));
            const uint32_t vo = keep_or_oob(keep, voffA[r]);
            if constexpr (ADMA)
                buf_load16_to_lds(rA, sA + (r * WAVES + w) * 1024, vo, soff);
            else
                stA[r] = buf_load16(rA, vo, soff);
        }
        stA_tile = kt;
        issue_fence();
    };
    // ADMA == false: write the staged tile into its stage (lane l of round r
    // at byte (r * WAVES + w) * 1024 + 16 l, the same place the DMA writes).
    auto store_a = [&]() {
        uint8_t *sA = lds + (stA_tile % NS) * BP_STAGE;
#pragma unroll
        for (int r = 0; r < BP_AR; ++r)
            *(u32x4 *)(sA + (r * WAVES + w) * 1024 + l * 16) = stA[r];
    };

    // ---- B: n-block (wn * FN + j) of the workgroup.  Pre-shuffled: k-blocks
    // 2kt and 2kt+1 (1 KiB apart); plain: chunks q and q + 4 of row
    // 16 * nb + r16 (64 bytes apart).  Packed int4: the one k-block kt, or
    // chunk q of the row's 64 bytes of the step.
    constexpr uint32_t kBHalf = BPRE ? 1024u : 64u;
    constexpr uint32_t kBStep = W4 ? (BPRE ? 1024u : 64u) : (BPRE ? 2048u : (uint32_t)kTileKBytes);
    uint32_t voffB[BP_FN];
#pragma unroll
    for (int j = 0; j < BP_FN; ++j)
        voffB[j] = BPRE ? (uint32_t)(wn * BP_FN + j) * 16u * kbB + (uint32_t)l * 16u
                        : (uint32_t)((wn * BP_FN + j) * 16 + r16) * kbB + (uint32_t)q * kChunkBytes;
    // A half-filled last step (K bytes 0..63 valid): half 1 is the missing part.
    auto b_keep = [&](bool beyond, bool part, int h) { return !beyond & ((h == 0) | !part); };
    u32x4 bq[2][BP_FN][BH];
    auto issue_b_one = [&](int kt, auto set_c, int j, int h, auto mask_c) {
        constexpr int S = decltype(set_c)::value;
        uint32_t vo = voffB[j] + (uint32_t)h * kBHalf;
        if constexpr (decltype(mask_c)::value) {
            const bool beyond = kt >= nk;
            const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
            vo = keep_or_oob(b_keep(beyond, part, h), vo);
        }
        bq[S][j][h] = buf_load16(rB, vo, (uint32_t)kt * kBStep);
        issue_fence();
    };
    auto issue_b = [&](int kt, auto set_c) {
        constexpr int S = decltype(set_c)::value;
        const bool beyond = kt >= nk;
        const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
        const uint32_t soff = (uint32_t)kt * kBStep;
#pragma unroll
        for (int j = 0; j < BP_FN; ++j)
#pragma unroll
            for (int h = 0; h < BH; ++h)
                bq[S][j][h] = buf_load16(rB, keep_or_oob(b_keep(beyond, part, h), voffB[j] + (uint32_t)h * kBHalf),
                                         soff);
        issue_fence();
    };

    f32x4 acc[BP_FM][BP_FN];
#pragma unroll
    for (int i = 0; i < BP_FM; ++i)
#pragma unroll
        for (int j = 0; j < BP_FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- fragment stream.  Group g of a step reads A row block g % FM at
    // chunk (g / FM) * 4 + q (bf16, MX e2m1) or chunks q and q + 4 (fp8, MX
    // e4m3: the 16x16x128 e4m3 operand's own layout, in which lane group q
    // holds K bytes 16 q .. +15 and 64 + 16 q .. +15 of the slice while the
    // scale byte of lane group q serves K block q, elements 32 q .. 32 q + 31).
    using FragT = typename std::conditional<WIDE, i32x8, u32x4>::type;
    FragT fa[NG];
    auto frag_addr = [&](int stage, int g, int half) -> const uint8_t * {
        const int i = g % BP_FM;
        const int c = W4 ? 2 * q + g / BP_FM : (!WIDE ? (g / BP_FM) * 4 + q : half * 4 + q);
        const int row = wm * BP_WTM + i * 16 + r16;
        return lds + stage * BP_STAGE + row * kTileKBytes + swz_chunk(row, c) * kChunkBytes;
    };
    auto load_frag = [&](int stage, int g) {
        const u32x4 lo = lds_load16(frag_addr(stage, g, 0));
        if constexpr (WIDE)
            fa[g] = join32(lo, lds_load16(frag_addr(stage, g, 1)));
        else
            fa[g] = lo;
    };

    // ---- MX block scales (see BscaleArgs): one 16-byte load per lane brings
    // the scales of 4 row blocks for the 4 K-slices of a group; "cur" serves
    // the current group, "nxt" is loaded one group ahead.  Slices: MX e4m3 one
    // per step (4 steps per group), MX e2m1 two per step (2 steps per group).
    constexpr int SPG = ELEM == kMx8 ? 4 : 2;
    constexpr int SQA = MX ? BP_FM / 4 : 1, SQB = MX ? BP_FN / 4 : 1;
    constexpr int SL = MX ? SQA + SQB : 0;                    // scale loads per group
    u32x4 scA[SQA], scB[SQB], scA_n[SQA], scB_n[SQB];
    const int G = p.s_groups;
    const auto rSA = make_rsrc(p.sa_img, (uint32_t)((p.M + 63) / 64) * (uint32_t)G * 1024u);
    const auto rSB = make_rsrc(p.sb_img, (uint32_t)((p.N + 63) / 64) * (uint32_t)G * 1024u);
    const int qa0 = (m0 + wm * BP_WTM) / 64, qb0 = (n0 + wn * BP_WTN) / 64;
    auto issue_scales = [&](int g2) {
        const bool in = g2 < G;              // past the last group: out of range (not the next quad)
#pragma unroll
        for (int t = 0; t < SQA; ++t)
            scA_n[t] = buf_load16(rSA, keep_or_oob(in, ((uint32_t)(qa0 + t) * (uint32_t)G + (uint32_t)g2) * 1024u +
                                                           (uint32_t)l * 16u), 0);
#pragma unroll
        for (int t = 0; t < SQB; ++t)
            scB_n[t] = buf_load16(rSB, keep_or_oob(in, ((uint32_t)(qb0 + t) * (uint32_t)G + (uint32_t)g2) * 1024u +
                                                           (uint32_t)l * 16u), 0);
        issue_fence();
    };
    // The scaled MFMA on block (i, j) with the scale byte of K-slice `byte`
    // of the current group (the switch folds away: every index is a constant
    // after unrolling).
    auto mfma_mx = [&](int i, int j, auto bx, auto ay, int byte) {
        const uint32_t sx = scB[j / 4][j % 4], sy = scA[i / 4][i % 4];
        switch (byte) {
        case 0:
            if constexpr (ELEM == kMx8) mfma_mx8_a<0>(acc[i][j], bx, ay, sx, sy); else mfma_mx4_a<0>(acc[i][j], bx, ay, sx, sy);
            break;
        case 1:
            if constexpr (ELEM == kMx8) mfma_mx8_a<1>(acc[i][j], bx, ay, sx, sy); else mfma_mx4_a<1>(acc[i][j], bx, ay, sx, sy);
            break;
        case 2:
            if constexpr (ELEM == kMx8) mfma_mx8_a<2>(acc[i][j], bx, ay, sx, sy); else mfma_mx4_a<2>(acc[i][j], bx, ay, sx, sy);
            break;
        default:
            if constexpr (ELEM == kMx8) mfma_mx8_a<3>(acc[i][j], bx, ay, sx, sy); else mfma_mx4_a<3>(acc[i][j], bx, ay, sx, sy);
            break;
        }
    };
    // W4: the current step's B operands unpacked to int8 (set at step start).
    u32x4 ub[BP_FN][2];
    auto mma_group = [&](int g, auto set_c, auto gp_c) {
        constexpr int S = decltype(set_c)::value;
        constexpr int GP = decltype(gp_c)::value;            // step position in its scale group
        const int i = g % BP_FM;
#pragma unroll
        for (int j = 0; j < BP_FN; ++j) {
            if constexpr (INT) {
                const u32x4 bx = W4 ? ub[j][g / BP_FM] : bq[S][j][W4 ? 0 : g / BP_FM];
                if constexpr (ACCA)
                    mfma_i8_a(acc[i][j], bx, fa[g]);
                else
                    acc[i][j] = mfma_i8(bx, fa[g], acc[i][j]);
            } else if constexpr (ELEM == kMx8)
                mfma_mx(i, j, join32(bq[S][j][0], bq[S][j][1]), fa[g], GP);
            else if constexpr (ELEM == kMx4)
                mfma_mx(i, j, bq[S][j][g / BP_FM], fa[g], 2 * GP + g / BP_FM);
            else if constexpr (ELEM == kBf16 && ACCA)
                mfma_bf16_a(acc[i][j], bq[S][j][g / BP_FM], fa[g]);
            else if constexpr (ELEM == kBf16)
                acc[i][j] = mfma_bf16(bq[S][j][g / BP_FM], fa[g], acc[i][j]);
            else if constexpr (ACCA)
                mfma_fp8x8_a(acc[i][j], join32(bq[S][j][0], bq[S][j][1]), fa[g]);
            else
                acc[i][j] = mfma_fp8x8(join32(bq[S][j][0], bq[S][j][1]), fa[g], acc[i][j]);
        }
    };

    // Load issue order (one entry per step k):
    //   start(k):   B(k+1)                      BP_BR loads
    //   barrier(k): A tile k+NS-1 (DMA)         BP_AR loads
    // At start(k), B(k) needs the loads issued after it done except the
    // A(k+NS-2) DMA: vmcnt(AR).  At barrier(k), A tile k+1 (issued at
    // barrier(k+2-NS)) has (NS-2) B issues and (NS-3) A issues behind it.
    // With ADMA == false the A loads land in VGPRs and the compiler waits for
    // them before the ds_write; the barrier then needs no vmcnt, and the LDS
    // stores of the previous barrier are covered by waiting until at most the
    // fragment reads issued since remain (LDS operations retire in order).
    // MX: the scale loads of a group are issued at the start of its first step
    // (before that step's B loads), so they add SL loads behind A tile k+1 for
    // every group start among steps k-(NS-3) .. k.
    constexpr int kVmStart = BP_AR;
    constexpr auto scale_starts = [](int gp) {
        int n = 0;
        for (int d = 0; d <= NS - 3; ++d)
            n += (((gp - d) % SPG + SPG) % SPG) == 0;
        return n;
    };
    constexpr int kVmBarrier0 = (NS - 2) * BP_BR + (NS - 3) * BP_AR;
    static_assert(kVmBarrier0 + SL * (NS - 2) < 64, "vmcnt is 6 bits");
    constexpr int kLgkmBarrier = PD * (WIDE ? 2 : 1);
    auto wait_vm = [&](auto n_c) {
        constexpr int n = decltype(n_c)::value;
        __builtin_amdgcn_s_waitcnt((kWaitVmcnt0 & ~0xC00F) | (n & 0xF) | ((n >> 4) << 14));
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // One step.  Set CUR holds B(kt); set 1-CUR receives B(kt+1).  GP: the
    // step's position in its scale group (MX).
    auto step = [&](int kt, auto cur_c, auto gp_c, auto mask_c) {
        constexpr int CUR = decltype(cur_c)::value;
        constexpr int GP = decltype(gp_c)::value;
        constexpr int kVmBar = kVmBarrier0 + SL * scale_starts(GP);
        const int st = kt % NS;
        wait_vm(ic<kVmStart>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (W4) {
#pragma unroll
            for (int j = 0; j < BP_FN; ++j) {
                ub[j][0] = int4x32_half_to_i8(bq[CUR][j][0], 0);
                ub[j][1] = int4x32_half_to_i8(bq[CUR][j][0], 1);
            }
        }
        if constexpr (MX && GP == 0) {
#pragma unroll
            for (int t = 0; t < SQA; ++t)
                scA[t] = scA_n[t];
#pragma unroll
            for (int t = 0; t < SQB; ++t)
                scB[t] = scB_n[t];
            issue_scales(kt / SPG + 1);
        }
        if constexpr (!(SPREAD && ADMA))
            issue_b(kt + 1, ic<1 - CUR>{});
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if constexpr (SPREAD && ADMA) {
                // B(kt+1) spread over the groups before the barrier, A(kt+NS-1)
                // over the groups after it: the same issue order across the
                // barrier (so the same vmcnt counts), without bursts that
                // stall the wave at issue while the memory pipeline drains.
                if (g < NG - PD) {
#pragma unroll
                    for (int b = g * BP_BR / (NG - PD); b < (g + 1) * BP_BR / (NG - PD); ++b)
                        issue_b_one(kt + 1, ic<1 - CUR>{}, b / BH, b % BH, mask_c);
                } else {
                    const int go = g - (NG - PD);
                    if (go == 0) {
                        wait_vm(ic<kVmBar>{});
                        barrier();
                    }
#pragma unroll
                    for (int r = go * BP_AR / PD; r < (go + 1) * BP_AR / PD; ++r)
                        issue_a_one(kt + NS - 1, r, mask_c);
                }
            } else if (g == NG - PD) {
                if constexpr (ADMA) {
                    wait_vm(ic<kVmBar>{});
                    barrier();
                    issue_a(kt + NS - 1);
                } else {
                    __builtin_amdgcn_s_waitcnt((0xC07F & ~0x0F00) | (kLgkmBarrier << 8));
                    barrier();
                    store_a();                       // tile kt+NS-2, loaded at barrier(kt-1)
                    __builtin_amdgcn_sched_barrier(0);
                    issue_a(kt + NS - 1);
                }
            }
            // prefetch: group g + PD of this step, or group g + PD - NG of the next
            if (g + PD < NG)
                load_frag(st, g + PD);
            else
                load_frag((kt + 1) % NS, g + PD - NG);
            mma_group(g, ic<CUR>{}, ic<GP>{});
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- prologue: the loads of virtual steps 1-NS .. -1 (B(k+1) only for
    // k+1 >= 0, so the first barriers wait for everything), then the first
    // fragments.
    if constexpr (MX)
        issue_scales(0);
    for (int v = 1 - NS; v < 0; ++v) {
        if (v == -1)
            issue_b(0, ic<0>{});
        if constexpr (!ADMA) {
            if (v > 1 - NS) {
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                store_a();
            }
        }
        issue_a(v + NS - 1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 & ~0x0F00);      // vmcnt(0) lgkmcnt(0)
    barrier();
#pragma unroll
    for (int g = 0; g < PD; ++g)
        load_frag(0, g);
    // Steps run in pairs (MX e4m3: in fours, one scale group); steps past nk
    // are phantom steps whose operands are all out of range, i.e. zeros, and
    // add exact zeros.
    // With the spread schedule, a pair of steps whose loads (B up to kt + 2,
    // A up to kt + NS) all cover whole, in-range tiles runs without per-lane
    // masks; the remaining pairs run the masked copy.
    using masked = std::true_type;
    using unmasked = std::false_type;
    if constexpr (ELEM == kMx8) {
        for (int kt = 0; kt < nk; kt += 4) {
            step(kt, ic<0>{}, ic<0>{}, masked{});
            step(kt + 1, ic<1>{}, ic<1>{}, masked{});
            step(kt + 2, ic<0>{}, ic<2>{}, masked{});
            step(kt + 3, ic<1>{}, ic<3>{}, masked{});
        }
    } else {
        int kt = 0;
        if constexpr (SPREAD && ADMA) {
            const int nfull = tail == (uint32_t)kTileKBytes ? nk : nk - 1;   // whole steps
            for (; kt + NS < nfull; kt += 2) {
                step(kt, ic<0>{}, ic<0>{}, unmasked{});
                step(kt + 1, ic<1>{}, ic<1>{}, unmasked{});
            }
        }
        for (; kt < nk; kt += 2) {
            step(kt, ic<0>{}, ic<0>{}, masked{});
            step(kt + 1, ic<1>{}, ic<1>{}, masked{});
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if constexpr (ACCA)
        mfma_drain_acc(acc);

    // ---- epilogue: scale, bias, activation, convert, store.  Row blocks
    // outside, column blocks inside: a wave writes its adjacent pieces of
    // one C row back to back, so the L2 merges them into whole lines before
    // they go to HBM (the other order measured 1.46x the bytes of C written).
    const EpiView ev = epi_view(p.epi, p.M, p.N);
    constexpr int OB = OUT == kOutF32 ? 4 : 2;
    const uint32_t ldc = (uint32_t)p.N * OB;
    const auto rC = make_rsrc((uint8_t *)sk.C + (size_t)m0 * ldc, (uint32_t)rows_a * ldc);
    f32x4 sbv[BP_FN], bzv[BP_FN];
#pragma unroll
    for (int j = 0; j < BP_FN; ++j) {
        const int col = n0 + wn * BP_WTN + j * 16 + 4 * q;
        sbv[j] = epi_col_scale4(ev, col);
        bzv[j] = epi_bias4(ev, col);
    }
#pragma unroll
    for (int i = 0; i < BP_FM; ++i) {
        const int row = wm * BP_WTM + i * 16 + r16;
        const float sa = epi_row_scale(ev, m0 + row);
#pragma unroll
        for (int j = 0; j < BP_FN; ++j) {
            const int col = n0 + wn * BP_WTN + j * 16 + 4 * q;
            const uint32_t voff = col < p.N ? (uint32_t)row * ldc + (uint32_t)col * OB : kOobOffset;
            const f32x4 a = INT ? int_acc_to_f32(acc[i][j], W4 ? 0.0625f : 1.f) : acc[i][j];
            const f32x4 v = epi_apply4(ev, a, sa, sbv[j], bzv[j]);
            if constexpr (OUT == kOutF32)
                buf_store16(rC, __builtin_bit_cast(u32x4, v), voff);
            else
                buf_store8(rC, u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)}, voff);
        }
    }
}

template <int ELEM, int OUT, bool BPRE, int WGM, int WGN, int NS, int PD, bool ADMA, bool ACCA, bool SPREAD>
static hipError_t launch_pipe(const TiledArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_pipe_kernel<ELEM, OUT, BPRE, WGM, WGN, NS, PD, ADMA, ACCA, SPREAD>), dim3(a.grid),
                       dim3(64 * WGM * WGN), 0, s, a);
    return hipGetLastError();
}

#define TG_PIPE_S(ELEM, OUT, BPRE, WGM, WGN, NS, PD, ADMA, SPREAD)                              \
    TiledVariant{BP_BM, BP_BN, WGM, WGN, ELEM, OUT, BPRE, BpCfg<WGM, WGN, NS>::LDS, NS,          \
                 &launch_pipe<ELEM, OUT, BPRE, WGM, WGN, NS, PD, ADMA, (WGM * WGN == 4), SPREAD>}
#define TG_PIPE(ELEM, OUT, BPRE, WGM, WGN, NS, PD, ADMA) TG_PIPE_S(ELEM, OUT, BPRE, WGM, WGN, NS, PD, ADMA, false)

// The first 8-wave and the first 4-wave variant of each (elem, out, layout)
// are the ones a plan can get; sweep builds add alternatives.
static const TiledVariant kPipe[] = {
    TG_PIPE_S(kBf16, kOutBf16, true, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kBf16, kOutF32, true, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kBf16, kOutBf16, false, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kBf16, kOutF32, false, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kFp8, kOutBf16, false, 1, 8, 4, 3, true, true),
    TG_PIPE_S(kFp8, kOutBf16, true, 1, 8, 4, 3, true, true),
    // 4 waves, one per SIMD, 256 accumulators each in AGPRs
    TG_PIPE_S(kBf16, kOutBf16, true, 1, 4, 4, 12, true, true),
    TG_PIPE_S(kBf16, kOutBf16, false, 1, 4, 4, 12, true, true),
    TG_PIPE_S(kBf16, kOutF32, true, 1, 4, 4, 12, true, true),
    TG_PIPE_S(kBf16, kOutF32, false, 1, 4, 4, 12, true, true),
    TG_PIPE_S(kFp8, kOutBf16, false, 1, 4, 4, 6, true, true),
    TG_PIPE_S(kFp8, kOutBf16, true, 1, 4, 4, 6, true, true),
    // MX block-scaled operands (4 waves, AGPR accumulators)
    TG_PIPE_S(kMx8, kOutBf16, true, 1, 4, 4, 3, true, true),
    TG_PIPE_S(kMx8, kOutBf16, false, 1, 4, 4, 3, true, true),
    TG_PIPE_S(kMx4, kOutBf16, true, 1, 4, 4, 12, true, true),
    TG_PIPE_S(kMx4, kOutBf16, false, 1, 4, 4, 12, true, true),
    // integer operands: 8 waves, then 4 waves with AGPR accumulators
    TG_PIPE_S(kI8, kOutBf16, true, 1, 8, 4, 6, true, true),     // 16
    TG_PIPE_S(kI8, kOutBf16, false, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kW4A8, kOutBf16, true, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kW4A8, kOutBf16, false, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kI8, kOutBf16, true, 1, 4, 4, 12, true, true),    // 20
    TG_PIPE_S(kI8, kOutBf16, false, 1, 4, 4, 12, true, true),
    TG_PIPE_S(kW4A8, kOutBf16, true, 1, 4, 4, 12, true, true),
    TG_PIPE_S(kW4A8, kOutBf16, false, 1, 4, 4, 12, true, true),
    // fp8 and integer operands with fp32 output: the split-K partial tiles
    TG_PIPE_S(kFp8, kOutF32, false, 1, 8, 4, 3, true, true),    // 24
    TG_PIPE_S(kFp8, kOutF32, true, 1, 8, 4, 3, true, true),
    TG_PIPE_S(kI8, kOutF32, true, 1, 8, 4, 6, true, true),      // 26
    TG_PIPE_S(kI8, kOutF32, false, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kW4A8, kOutF32, true, 1, 8, 4, 6, true, true),
    TG_PIPE_S(kW4A8, kOutF32, false, 1, 8, 4, 6, true, true),
#ifdef TGEMM_SWEEP
    // alternatives (sweep builds only)
    TG_PIPE(kBf16, kOutBf16, true, 1, 8, 4, 4, true),           // 30: loads in bursts
    TG_PIPE_S(kBf16, kOutBf16, true, 1, 8, 4, 5, true, true),   // 31
    TG_PIPE_S(kBf16, kOutBf16, true, 1, 8, 4, 7, true, true),   // 32
    TG_PIPE_S(kBf16, kOutBf16, true, 1, 8, 5, 6, true, true),   // 33
    TG_PIPE_S(kFp8, kOutBf16, false, 1, 8, 4, 2, true, true),   // 34
    TG_PIPE_S(kFp8, kOutBf16, false, 1, 8, 4, 4, true, true),   // 35
    TG_PIPE(kFp8, kOutBf16, false, 1, 8, 4, 3, true),           // 36: loads in bursts
#endif
};

const TiledVariant *pipe_variants(int *count)
{
    *count = (int)(sizeof(kPipe) / sizeof(kPipe[0]));
    return kPipe;
}

}  // namespace tg
