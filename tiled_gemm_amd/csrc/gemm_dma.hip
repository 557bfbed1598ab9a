// GEMM C = A * B^T for 256 x 256 tiles with BOTH operands staged through LDS
// by the buffer loads' own LDS writes (FlyDSL "Kernel Authoring" skill,
// section 6 "GEMM Pattern (Preshuffle)": 64-byte K micro-steps, LDS
// ping-pong, XOR-swizzled tiles, B in MFMA operand order; section 3 "Runtime
// Loops with Loop-Carried Values" for the load-next / compute-current loop).
//
// Why both operands go through LDS on gfx950: a 16-byte load whose data
// returns to VGPRs costs the MFMA loop about three times what the same bytes
// cost when the load writes LDS directly (work-skipping measurements of the
// register-staged B kernel: dropping its B loads gained 22-33%, dropping the
// same number of LDS-writing A loads 8%).  The pages' preshuffle kernel keeps
// B out of LDS; here the pre-shuffled image still pays off, because a wave's
// 1 KiB operand block is contiguous both in HBM and in LDS, so B needs no
// swizzle and its fragment reads are linear.
//
// Workgroup: WGM x WGN waves over a 256 x 256 output tile (2 x 4: each wave
// 128 rows x 64 columns, 128 fp32 accumulators per lane).  Main-loop step:
// 128 bytes of K (two 16x16x32 bf16 MFMAs per 16 x 16 block, or one fp8
// 16x16x128).
//
//   LDS     two stages of 64 KiB: A (256 rows x 128 B, chunk-swizzled) and B
//           (pre-shuffled: 32 operand blocks of 1 KiB; plain: 256 rows x
//           128 B, chunk-swizzled like A).
//   DMA     step k+2 is issued right after barrier(k) into the stage step k
//           has just finished reading, spread over the last PD groups.
//   Reads   one ordered stream per step: for each half h of the step, the FN
//           B fragments, then the A fragments of the FM row blocks; each
//           read runs PD groups ahead of its MFMAs, across the step boundary.
//   Sync    one barrier per step, PD groups before its end, after
//           vmcnt(0) (step k+1 has landed) and lgkmcnt(0) (every read of the
//           stage about to be overwritten has returned).
//   Epilogue (acc * s_a) * s_b (+ bias, activation) in fp32, RNE to bf16,
//           buffer stores (rows past M and columns past N dropped).
#include "device.hpp"
#include "kernels.hpp"

namespace tg {

namespace {

constexpr int DM_BM = 256;
constexpr int DM_BN = 256;
constexpr int DM_A = DM_BM * kTileKBytes;      // 32 KiB of A per stage
constexpr int DM_B = DM_BN * kTileKBytes;      // 32 KiB of B per stage
constexpr int DM_STAGE = DM_A + DM_B;
constexpr int DM_LDS = 2 * DM_STAGE;           // 128 KiB

template <int N>
using dic = std::integral_constant<int, N>;

}  // namespace

template <int ELEM, int OUT, bool BPRE, int WGM, int WGN, int PD, bool BKN, bool AKM>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_dma_kernel(const TiledArgs p)
{
    static_assert(ELEM == kBf16 || ELEM == kFp8 || (ELEM == kI8 && OUT == kOutBf16),
                  "bf16, fp8 e4m3 or int8 operands");
    // BKN: B stored K x N (C = A * B): a step's K-rows of the tile's 256
    // columns are the B stage (bf16: 64 rows of 512 bytes, chunks swizzled by
    // bkn_swz, two 16-bit transpose reads per operand; fp8: 128 rows of 256
    // bytes, bkn8_swz, four 8-bit transpose reads per operand).
    static_assert(!BKN || !BPRE, "K x N B is not pre-shuffled");
    // AKM: A stored K x M, staged and read the same way (64 K-rows of the
    // tile's 256 rows of C per step).
    static_assert(!AKM || !BPRE, "K x M A with a plain B");
    // fp8: one 128-byte K slice per step and MFMA (16x16x128, 32 bytes per
    // lane: chunks q and q + 4 of the slice); bf16: two 64-byte halves.
    // int8 shares the fp8 staging and fragments (8-bit elements); each 32-byte
    // fragment feeds two 16x16x64 int8 MFMAs, one per 16-byte half (chunk q,
    // then chunk q + 4: the same K slots in A and in B), into int32 sums.
    constexpr bool I8 = ELEM == kI8;
    constexpr bool F8 = ELEM == kFp8 || I8;                 // 8-bit elements
    // K x N B geometry per step: bf16 64 K-rows of 512 bytes (swizzle
    // bkn_swz), fp8 128 K-rows of 256 bytes (swizzle bkn8_swz).
    constexpr int KN_ROWS = F8 ? 128 : 64;
    constexpr int KN_CPR = (F8 ? 256 : 512) / kChunkBytes;
    auto kn_swz = [](int k) { return F8 ? bkn8_swz(k) : bkn_swz(k); };
    constexpr int WAVES = WGM * WGN;
    constexpr int THREADS = 64 * WAVES;
    constexpr int WTM = DM_BM / WGM, WTN = DM_BN / WGN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int AR = DM_A / (THREADS * kChunkBytes);     // A loads per lane and step
    constexpr int BR = DM_B / (THREADS * kChunkBytes);     // B loads per lane and step
    constexpr int NL = AR + BR;
    constexpr int NG = F8 ? FM : 2 * FM;                   // groups per step: half h = g / FM (bf16)
    static_assert(WAVES == 8, "two waves per SIMD: 128 accumulators per lane in VGPRs");
    // bf16: next-step B fragments of half 0 reuse the dead registers of
    // half 0; fp8: B fragments are double-buffered by step parity on the 1 x 8
    // grid, single-buffered (SB, below) on the 2 x 4 grid.
    static_assert(PD >= 1 && (F8 ? PD < FM : PD <= FM), "prefetch distance");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[DM_LDS];

    const int w = wave_id();
    const int l = lane_id();
    const int q = l >> 4, r16 = l & 15;
    const int wm = w / WGN, wn = w % WGN;

    const SplitK sk = split_k_of(p);
    int tm, tn;
    tile_of_wg(sk.wg, sk.grid, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m0 = tm * DM_BM, n0 = tn * DM_BN;
    const int rows_a = min(p.M - m0, DM_BM);
    const int rows_b = min(p.N - n0, DM_BN);
    const uint32_t kb = (uint32_t)p.kbytes;
    const uint32_t kbB = (uint32_t)p.kbytes_b;
    const uint32_t lda = (uint32_t)p.lda_bytes;
    // A split starts its operands' resources at its first K step (kAStep /
    // kBStep bytes per step, below), so every step index is split-relative.
    // K x M A (like K x N B): per step 64 K-rows of 2-byte elements or 128 of
    // 1-byte ones, the tile's 256 rows of C each.
    constexpr int EA = F8 ? 1 : 2;                       // bytes per element of A
    const uint32_t shA = (uint32_t)sk.kt0 * (AKM ? (uint32_t)KN_ROWS * lda : (uint32_t)kTileKBytes);
    const auto rA = AKM ? make_rsrc((const uint8_t *)p.A + (size_t)m0 * EA + shA,
                                    (uint32_t)((size_t)p.K * lda - (size_t)m0 * EA - shA))
                        : make_rsrc((const uint8_t *)p.A + (size_t)m0 * kb + shA, (uint32_t)rows_a * kb - shA);
    // K x N B: the resource starts at column n0 and ends with the matrix, so
    // K-rows past K read zeros; columns past N read neighbouring data or
    // zeros and only feed columns of C that are never stored.
    const uint32_t ldb = (uint32_t)p.ldb_bytes;
    constexpr int EB = F8 ? 1 : 2;                       // bytes per element
    const uint32_t shB = (uint32_t)sk.kt0 * (BKN ? (uint32_t)KN_ROWS * ldb : (BPRE ? 2048u : (uint32_t)kTileKBytes));
    const auto rB = BKN ? make_rsrc((const uint8_t *)p.B + (size_t)n0 * EB + shB,
                                    (uint32_t)((size_t)p.K * ldb - (size_t)n0 * EB - shB))
                        : make_rsrc((const uint8_t *)p.B + (size_t)n0 * kbB + shB, (uint32_t)rows_b * kbB - shB);
    const int nk = sk.nk;
    const uint32_t tail = sk.tail;

    // ---- load sources.  Load r of a step lands at byte (r * WAVES + w) *
    // 1024 + 16 l of its operand's half of the stage.  Row-major operands:
    // that is row pc / 8, physical chunk pc % 8, so the lane fetches logical
    // chunk swz_chunk(row, pc % 8).  Pre-shuffled B: operand block u = (n
    // block u / 2, K half u % 2), 1 KiB contiguous in the image.
    uint32_t voffA[AR], voffB[BR];
    uint32_t tailA = 0, tailB = 0;
#pragma unroll
    for (int r = 0; r < AR; ++r) {
        const int pc = (r * WAVES + w) * 64 + l;
        if constexpr (AKM) {
            const int row = pc / KN_CPR;                // 32 (2-byte) or 16 (1-byte) chunks per K-row
            const int c = (pc % KN_CPR) ^ kn_swz(row);
            voffA[r] = (uint32_t)row * lda + (uint32_t)c * kChunkBytes;
            tailA |= 1u << r;                           // rows past K are out of range
        } else {
            const int row = pc >> 3;
            const int c = swz_chunk(row, pc & 7);
            voffA[r] = (uint32_t)row * kb + (uint32_t)c * kChunkBytes;
            tailA |= ((uint32_t)(c * kChunkBytes) < tail ? 1u : 0u) << r;
        }
    }
#pragma unroll
    for (int r = 0; r < BR; ++r) {
        const int u = r * WAVES + w;
        if constexpr (BKN) {
            const int pc = u * 64 + l;
            const int row = pc / KN_CPR;
            const int c = (pc % KN_CPR) ^ kn_swz(row);
            voffB[r] = (uint32_t)row * ldb + (uint32_t)c * kChunkBytes;
            tailB |= 1u << r;                           // rows past K are out of range
        } else if constexpr (BPRE) {
            voffB[r] = (uint32_t)(u >> 1) * 16u * kbB + (uint32_t)(u & 1) * 1024u + (uint32_t)l * 16u;
            tailB |= ((uint32_t)((u & 1) * 64) < tail ? 1u : 0u) << r;
        } else {
            const int pc = u * 64 + l;
            const int row = pc >> 3;
            const int c = swz_chunk(row, pc & 7);
            voffB[r] = (uint32_t)row * kbB + (uint32_t)c * kChunkBytes;
            tailB |= ((uint32_t)(c * kChunkBytes) < tail ? 1u : 0u) << r;
        }
    }
    const uint32_t kAStep = AKM ? (uint32_t)KN_ROWS * lda : (uint32_t)kTileKBytes;   // bytes of A per step
    // bytes of B per step: pre-shuffled image 2 KiB per block row, N x K 128
    // per row, K x N 64 K-rows
    const uint32_t kBStep = BKN ? (uint32_t)KN_ROWS * ldb : (BPRE ? 2048u : (uint32_t)kTileKBytes);
    // Load idx (A rounds first, then B) of step kt into stage S.  Loads past
    // the last step, and the missing half of a half-filled last step, read
    // out of range and land zeros.
    // MASK == false: the caller guarantees step kt is whole and in range, so
    // the offsets need no per-lane selection (no VALU work beside the load).
    auto issue_one = [&](int kt, auto s_c, int idx, auto mask_c) {
        constexpr int S = decltype(s_c)::value;
        if constexpr (!decltype(mask_c)::value) {
            if (idx < AR)
                buf_load16_to_lds(rA, lds + S * DM_STAGE + (idx * WAVES + w) * 1024, voffA[idx],
                                  (uint32_t)kt * kAStep);
            else
                buf_load16_to_lds(rB, lds + S * DM_STAGE + DM_A + ((idx - AR) * WAVES + w) * 1024, voffB[idx - AR],
                                  (uint32_t)kt * kBStep);
            issue_fence();
            return;
        }
        const bool beyond = kt >= nk;
        const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
        if (idx < AR) {
            const bool keep = !beyond & (!part | (((tailA >> idx) & 1u) != 0));
            buf_load16_to_lds(rA, lds + S * DM_STAGE + (idx * WAVES + w) * 1024, keep_or_oob(keep, voffA[idx]),
                              (uint32_t)kt * kAStep);
        } else {
            const int r = idx - AR;
            const bool keep = !beyond & (!part | (((tailB >> r) & 1u) != 0));
            buf_load16_to_lds(rB, lds + S * DM_STAGE + DM_A + (r * WAVES + w) * 1024, keep_or_oob(keep, voffB[r]),
                              (uint32_t)kt * kBStep);
        }
        issue_fence();
    };

    // ---- fragments.  A: row block i, half h -> logical chunk 4 h + q of row
    // wm * WTM + 16 i + r16 (fp8: chunks q and q + 4).  B: block j of the
    // wave, half h.
    // K x M A: the operand of row block i for half h, two transpose reads.
    auto akm_frag = [&](int s, int g, int h) -> u32x4 {
        const uint8_t *sA = lds + s * DM_STAGE;
        const int col = wm * WTM + (g % FM) * 16 + 4 * (r16 & 3);   // this lane's 4 source rows of C
        const int c = (col * 2) >> 4, off = (col * 2) & 15;
        u32x2 t2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int k = 32 * h + 8 * q + 4 * t + (r16 >> 2);
            t2[t] = lds_read_tr16(sA + k * 512 + ((c ^ bkn_swz(k)) << 4) + off);
        }
        return u32x4{t2[0].x, t2[0].y, t2[1].x, t2[1].y};
    };
    // 8-bit K x M A: the 32-byte operand of row block g as four 8-bit
    // transpose reads, K positions as in bkn8_frag (the rows of C play the
    // part of B's columns there).
    auto akm8_frag = [&](int s, int g) -> i32x8 {
        const uint8_t *sA = lds + s * DM_STAGE;
        const int e = r16 >> 1, b = r16 & 1;
        const int rb = wm * WTM + (g % FM) * 16 + 8 * b;        // this lane's 8 source rows of C
        const int c = rb >> 4, off = rb & 15;
        u32x2 t4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int k = (t >> 1) * 64 + 16 * q + 8 * (t & 1) + e;
            t4[t] = lds_read_tr8(sA + k * 256 + ((c ^ bkn8_swz(k)) << 4) + off);
        }
        return i32x8{(int)t4[0].x, (int)t4[0].y, (int)t4[1].x, (int)t4[1].y,
                     (int)t4[2].x, (int)t4[2].y, (int)t4[3].x, (int)t4[3].y};
    };
    auto a_addr = [&](int s, int g, int h) -> const uint8_t * {
        const int i = g % FM;
        const int row = wm * WTM + i * 16 + r16;
        return lds + s * DM_STAGE + row * kTileKBytes + swz_chunk(row, h * 4 + q) * kChunkBytes;
    };
    // K x N: the operand of column block j for half h (k = 32 h + 8 q .. + 7
    // of the step, one column per lane) as two transpose reads.
    auto bkn_frag = [&](int s, int h, int j) -> u32x4 {
        const uint8_t *sB = lds + s * DM_STAGE + DM_A;
        const int col = wn * WTN + j * 16 + 4 * (r16 & 3);    // this lane's 4 source columns
        const int c = (col * 2) >> 4, off = (col * 2) & 15;
        u32x2 t2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int k = 32 * h + 8 * q + 4 * t + (r16 >> 2);
            t2[t] = lds_read_tr16(sB + k * 512 + ((c ^ bkn_swz(k)) << 4) + off);
        }
        return u32x4{t2[0].x, t2[0].y, t2[1].x, t2[1].y};
    };
    // fp8 K x N: the 32-byte operand of column block j (this lane's column,
    // K positions 16 q .. 16 q + 15 and 64 + 16 q .. + 15 of the step, the
    // order A's two chunks give) as four 8-row transpose reads.
    auto bkn8_frag = [&](int s, int j) -> i32x8 {
        const uint8_t *sB = lds + s * DM_STAGE + DM_A;
        const int e = r16 >> 1, b = r16 & 1;
        const int cb = wn * WTN + j * 16 + 8 * b;                // this lane's 8 source columns
        const int c = cb >> 4, off = cb & 15;
        u32x2 t4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int k = (t >> 1) * 64 + 16 * q + 8 * (t & 1) + e;
            t4[t] = lds_read_tr8(sB + k * 256 + ((c ^ bkn8_swz(k)) << 4) + off);
        }
        return i32x8{(int)t4[0].x, (int)t4[0].y, (int)t4[1].x, (int)t4[1].y,
                     (int)t4[2].x, (int)t4[2].y, (int)t4[3].x, (int)t4[3].y};
    };
    auto b_addr = [&](int s, int h, int j) -> const uint8_t * {
        const int nb = wn * FN + j;
        if constexpr (BPRE)
            return lds + s * DM_STAGE + DM_A + (nb * 2 + h) * 1024 + l * 16;
        const int row = nb * 16 + r16;
        return lds + s * DM_STAGE + DM_A + row * kTileKBytes + swz_chunk(row, h * 4 + q) * kChunkBytes;
    };
    using FragT = typename std::conditional<F8, i32x8, u32x4>::type;
    // 8-bit operands on a 2 x 4 grid: two sets of the four 8-register B
    // fragments would not fit beside 128 accumulators in 256 registers, so
    // there is one set, and the last group of a step reloads fragment j from
    // the next stage right after its last MFMA (SB).
    constexpr bool SB = F8 && FN > 2;
    FragT fa[NG];
    FragT fb[SB ? 1 : 2][FN];   // bf16: [half][block]; fp8: [step parity][block]
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Reads for group t of the step held in stage s: the half's B fragments
    // first when t opens a half, then t's A fragment.
    auto b8_frag = [&](int s, int j) -> i32x8 {
        if constexpr (BKN)
            return bkn8_frag(s, j);
        else
            return join32(lds_load16(b_addr(s, 0, j)), lds_load16(b_addr(s, 1, j)));
    };
    auto load_group = [&](int s, int t) {
        if constexpr (F8) {
            if constexpr (!SB) {
                if (t == 0) {
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        fb[s][j] = b8_frag(s, j);
                }
            }
            if constexpr (AKM)
                fa[t] = akm8_frag(s, t);
            else
                fa[t] = join32(lds_load16(a_addr(s, t, 0)), lds_load16(a_addr(s, t, 1)));
        } else {
            if (t % FM == 0) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (BKN)
                        fb[t / FM][j] = bkn_frag(s, t / FM, j);
                    else
                        fb[t / FM][j] = lds_load16(b_addr(s, t / FM, j));
                }
            }
            if constexpr (AKM)
                fa[t] = akm_frag(s, t, t / FM);
            else
                fa[t] = lds_load16(a_addr(s, t, t / FM));
        }
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    auto step = [&](int kt, auto s_c, auto mask_c) {
        constexpr int S = decltype(s_c)::value;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g == NG - PD) {
                // Every read of stage S has been issued: wait for them and for
                // step kt+1's loads, meet, then refill stage S with step kt+2.
                __builtin_amdgcn_s_waitcnt(0);
                barrier();
            }
            if (g >= NG - PD) {
                const int go = g - (NG - PD);
#pragma unroll
                for (int idx = go * NL / PD; idx < (go + 1) * NL / PD; ++idx)
                    issue_one(kt + 2, s_c, idx, mask_c);
            }
            if (g + PD < NG)
                load_group(S, g + PD);
            else
                load_group(S ^ 1, g + PD - NG);
            const int i = g % FM, h = g / FM;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                constexpr int SF = SB ? 0 : S;
                if constexpr (I8) {
                    acc[i][j] = mfma_i8(lo16(fb[SF][j]), lo16(fa[g]), acc[i][j]);
                    acc[i][j] = mfma_i8(hi16(fb[SF][j]), hi16(fa[g]), acc[i][j]);
                } else if constexpr (F8) {
                    acc[i][j] = mfma_fp8x8(fb[SF][j], fa[g], acc[i][j]);
                } else {
                    acc[i][j] = mfma_bf16(fb[h][j], fa[g], acc[i][j]);
                }
                // The barrier of this step (PD groups back) has made the next
                // stage visible.
                if constexpr (SB) {
                    if (g == NG - 1) {
                        // in this order: the reload may take the registers
                        // the MFMA above has just read
                        __builtin_amdgcn_sched_barrier(0);
                        fb[0][j] = b8_frag(S ^ 1, j);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- prologue: steps 0 and 1 into stages 0 and 1, the first fragments.
#pragma unroll
    for (int idx = 0; idx < NL; ++idx)
        issue_one(0, dic<0>{}, idx, std::true_type{});
#pragma unroll
    for (int idx = 0; idx < NL; ++idx)
        issue_one(1, dic<1>{}, idx, std::true_type{});
    __builtin_amdgcn_s_waitcnt(0);
    barrier();
    if constexpr (SB) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[0][j] = b8_frag(0, j);
    }
#pragma unroll
    for (int t = 0; t < PD; ++t)
        load_group(0, t);
    // Steps run in pairs; a step past nk is a phantom whose operands are all
    // zeros (its loads read out of range), so it adds exact zeros.
    // Steps kt < nfull - 2 load whole, in-range steps (kt + 2 < nfull) and
    // run without masks; the last few steps run the masked form.
    const int nfull = tail == (uint32_t)kTileKBytes ? nk : nk - 1;
    int kt = 0;
    for (; kt + 1 < nfull - 2; kt += 2) {
        step(kt, dic<0>{}, std::false_type{});
        step(kt + 1, dic<1>{}, std::false_type{});
    }
    for (; kt < nk; kt += 2) {
        step(kt, dic<0>{}, std::true_type{});
        step(kt + 1, dic<1>{}, std::true_type{});
    }
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: row blocks outside, column blocks inside, so a wave
    // writes its adjacent pieces of one C row back to back.
    const EpiView ev = epi_view(p.epi, p.M, p.N);
    constexpr int OB = OUT == kOutF32 ? 4 : 2;
    const uint32_t ldc = (uint32_t)p.N * OB;
    const auto rC = make_rsrc((uint8_t *)sk.C + (size_t)m0 * ldc, (uint32_t)rows_a * ldc);
    f32x4 sbv[FN], bzv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WTN + j * 16 + 4 * q;
        sbv[j] = epi_col_scale4(ev, col);
        bzv[j] = epi_bias4(ev, col);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = wm * WTM + i * 16 + r16;
        const float sa = epi_row_scale(ev, m0 + row);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WTN + j * 16 + 4 * q;
            const uint32_t voff = col < p.N ? (uint32_t)row * ldc + (uint32_t)col * OB : kOobOffset;
            const f32x4 a = I8 ? int_acc_to_f32(acc[i][j], 1.f) : acc[i][j];
            const f32x4 v = epi_apply4(ev, a, sa, sbv[j], bzv[j]);
            if constexpr (OUT == kOutF32)
                buf_store16(rC, __builtin_bit_cast(u32x4, v), voff);
            else
                buf_store8(rC, u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)}, voff);
        }
    }
}

template <int ELEM, int OUT, bool BPRE, int WGM, int WGN, int PD, bool BKN, bool AKM>
static hipError_t launch_dma(const TiledArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_dma_kernel<ELEM, OUT, BPRE, WGM, WGN, PD, BKN, AKM>), dim3(a.grid),
                       dim3(64 * WGM * WGN), 0, s, a);
    return hipGetLastError();
}

#define TG_DMA(ELEM, OUT, BPRE, WGM, WGN, PD)                                                       \
    TiledVariant{DM_BM, DM_BN, WGM, WGN, ELEM, OUT, BPRE, DM_LDS, 2,                                    \
                 &launch_dma<ELEM, OUT, BPRE, WGM, WGN, PD, false, false>}
#define TG_DMA_L(OUT, WGM, WGN, PD, BKN, AKM)                                                        \
    TiledVariant{DM_BM, DM_BN, WGM, WGN, kBf16, OUT, false, DM_LDS, 2,                                  \
                 &launch_dma<kBf16, OUT, false, WGM, WGN, PD, BKN, AKM>, BKN, AKM}
#define TG_DMA_KN(OUT, WGM, WGN, PD) TG_DMA_L(OUT, WGM, WGN, PD, true, false)
#define TG_DMA_KN8E(ELEM, WGM, WGN, PD)                                                            \
    TiledVariant{DM_BM, DM_BN, WGM, WGN, ELEM, kOutBf16, false, DM_LDS, 2,                              \
                 &launch_dma<ELEM, kOutBf16, false, WGM, WGN, PD, true, false>, true, false}
#define TG_DMA_KN8(WGM, WGN, PD) TG_DMA_KN8E(kFp8, WGM, WGN, PD)
#define TG_DMA_AT8(ELEM, BKN)                                                                      \
    TiledVariant{DM_BM, DM_BN, 1, 8, ELEM, kOutBf16, false, DM_LDS, 2,                                  \
                 &launch_dma<ELEM, kOutBf16, false, 1, 8, 2, BKN, true>, BKN, true}

static const TiledVariant kDma[] = {
    TG_DMA(kBf16, kOutBf16, false, 2, 4, 6),   // B N x K
    TG_DMA(kBf16, kOutF32, false, 2, 4, 4),
    TG_DMA(kFp8, kOutBf16, false, 2, 4, 2),    // fp8, B N x K
    TG_DMA(kFp8, kOutF32, false, 2, 4, 2),
    TG_DMA(kI8, kOutBf16, false, 2, 4, 2),     // int8, B N x K
    TG_DMA_KN(kOutBf16, 2, 4, 4),              // B stored K x N
    TG_DMA_KN(kOutF32, 2, 4, 4),
    // A stored K x M: prefetch distance 2 (a K x M fragment is two transpose
    // reads and their addresses; at 4 the kernel spilled 19-38 VGPRs and ran
    // 13-17% slower)
    TG_DMA_L(kOutBf16, 2, 4, 2, false, true),  // A stored K x M, B N x K
    TG_DMA_L(kOutF32, 2, 4, 2, false, true),
    TG_DMA_L(kOutBf16, 2, 4, 2, true, true),   // A stored K x M, B K x N
    TG_DMA_L(kOutF32, 2, 4, 2, true, true),
    TG_DMA_KN8(1, 8, 3),                       // fp8, B stored K x N
    TG_DMA_KN8E(kI8, 1, 8, 3),                 // int8, B stored K x N
    // 8-bit A stored K x M (8-bit transpose reads on both operands)
    TG_DMA_AT8(kFp8, false),                   // fp8, A K x M, B N x K
    TG_DMA_AT8(kFp8, true),                    // fp8, A K x M, B K x N
    TG_DMA_AT8(kI8, false),                    // int8, A K x M, B N x K
    TG_DMA_AT8(kI8, true),                     // int8, A K x M, B K x N
#ifdef TGEMM_SWEEP
    // alternatives (sweep builds only): other prefetch distances, and
    // pre-shuffled B through LDS
    TG_DMA(kBf16, kOutBf16, false, 2, 4, 4),   // 16
    TG_DMA(kFp8, kOutBf16, false, 1, 8, 2),    // 17
    TG_DMA(kFp8, kOutBf16, true, 1, 8, 3),
    TG_DMA(kBf16, kOutBf16, true, 2, 4, 6),    // 19
    TG_DMA_KN(kOutBf16, 2, 4, 6),
    TG_DMA_KN8(1, 8, 2),                       // 21
    TG_DMA_L(kOutBf16, 2, 4, 4, false, true),  // 22: A K x M
    TG_DMA_L(kOutBf16, 2, 4, 3, false, true),
    TG_DMA_L(kOutBf16, 2, 4, 4, true, true),   // 24: A K x M, B K x N
    TG_DMA_L(kOutBf16, 2, 4, 3, true, true),
    TG_DMA_KN(kOutBf16, 2, 4, 3),              // 26: B K x N
    TG_DMA(kBf16, kOutBf16, false, 2, 4, 5),   // 27: B N x K
    TG_DMA(kFp8, kOutBf16, false, 1, 8, 3),    // 28: fp8 1 x 8
    TG_DMA(kFp8, kOutBf16, false, 2, 4, 3),
    TG_DMA(kFp8, kOutBf16, true, 2, 4, 3),     // 30: fp8 2 x 4, B pre-shuffled
#endif
};

const TiledVariant *dma_variants(int *count)
{
    *count = (int)(sizeof(kDma) / sizeof(kDma[0]));
    return kDma;
}

}  // namespace tg
