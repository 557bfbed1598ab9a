// Skinny GEMM (M <= 64): C = A * B^T when B is the only large operand and
// the product is bound by streaming B from HBM once (decode shapes).  Two
// kernels share the workgroup shape, the K split over the waves and the
// reduction: gemm_skinny_kernel below (B N x K, bf16 / fp8 / int8, both
// operands staged through LDS) and gemm_skinny_pre_kernel further down (B
// pre-shuffled, streamed straight into VGPRs; also W4A8 and MX).
//
// One workgroup owns 32 columns of C (two 16-column MFMA blocks) and every
// row.  Its WAVES waves split K: wave w takes a contiguous run of 128-byte K
// steps, and with ROTATE each workgroup starts its sweep at a different step
// (wrapping), so the concurrent loads of all workgroups spread over the rows
// instead of hitting one K offset of rows 16 KiB apart.
//
// For this shape the per-CU vector-memory path, not HBM, sets the pace when
// loads cover half cache lines, so every load here covers whole 128-byte
// lines: one wave load brings 8 rows x 128 bytes straight into LDS (the
// load's own LDS write, lane l writing bytes 16 l .. 16 l + 15 of the wave's
// 1 KiB destination), each lane choosing its source chunk so that the LDS
// image is XOR-swizzled (chunk c of row r sits at c ^ ((r >> 1) & 7), as in
// the tiled kernels); the MFMA fragments are then read with conflict-free
// 16-byte LDS reads.  Each wave owns a ring of DEPTH stages, so the loop needs
// no workgroup barrier: wait until the oldest stage has landed (vmcnt), read
// its fragments, run the MFMAs, then refill that stage with the step DEPTH
// ahead.  Steps past the wave's run read out of range, i.e. zeros, which keeps
// the number of loads in flight constant.
//
// The partial tiles of the waves are summed through LDS in a fixed wave order
// (deterministic), then scaled, converted and stored.
#include "device.hpp"
#include "kernels.hpp"

namespace tg {

constexpr int kRedPitch = kSkinnyTileN + 1;   // padded reduction row (bank spread)

// Sums the waves' partial 16 x 16 tiles through LDS in a fixed wave order
// (deterministic), then applies the epilogue and stores C.  The caller has
// drained every load that writes LDS and synchronised the workgroup.
// IUNIT = 0: fp32 accumulators.  Otherwise the accumulators hold int32 sums
// (integer MFMAs): the waves' partials are summed in int32 (exact), then
// converted to fp32 and multiplied by 1 / IUNIT (a power of two, exact).
template <int MB, int OUT, int WAVES, int IUNIT = 0>
__device__ inline void skinny_finish(const SkinnyArgs &p, const f32x4 (&acc)[MB][kSkinnyTileN / 16], uint8_t *lds,
                                     int n0)
{
    constexpr int NB = kSkinnyTileN / 16;
    constexpr int ROWS_A = MB * 16;
    const int w = wave_id();
    const int l = lane_id();
    const int q = l >> 4, r16 = l & 15;
    using RedRows = float[ROWS_A][kRedPitch];
    RedRows *red = reinterpret_cast<RedRows *>(lds);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[w][i * 16 + r16][j * 16 + 4 * q + v] = acc[i][j][v];
    __syncthreads();

    const EpiView ev = epi_view(p.epi, p.M, p.N);
    constexpr int OB = OUT == kOutF32 ? 4 : 2;
    const uint32_t ldc = (uint32_t)p.N * OB;
    const auto rC = make_rsrc(p.C, (uint32_t)p.M * ldc);
    // Each thread finishes pairs of adjacent outputs.
    for (int o = threadIdx.x * 2; o < ROWS_A * kSkinnyTileN; o += 64 * WAVES * 2) {
        const int row = o / kSkinnyTileN, col = o % kSkinnyTileN;
        float s0 = 0.f, s1 = 0.f;
        if constexpr (IUNIT != 0) {
            int32_t i0 = 0, i1 = 0;
#pragma unroll
            for (int ww = 0; ww < WAVES; ++ww) {
                i0 += __builtin_bit_cast(int32_t, red[ww][row][col]);
                i1 += __builtin_bit_cast(int32_t, red[ww][row][col + 1]);
            }
            s0 = (float)i0 * (1.f / IUNIT);
            s1 = (float)i1 * (1.f / IUNIT);
        } else {
#pragma unroll
            for (int ww = 0; ww < WAVES; ++ww) {
                s0 += red[ww][row][col];
                s1 += red[ww][row][col + 1];
            }
        }
        const int n = n0 + col;
        float sb[2], bz[2];
        epi_col2(ev, n, sb, bz);
        const float sa = epi_row_scale(ev, row);
        s0 = epi_apply1(ev, s0, sa, sb[0], bz[0]);
        s1 = epi_apply1(ev, s1, sa, sb[1], bz[1]);
        const uint32_t voffc = (row < p.M && n < p.N) ? (uint32_t)row * ldc + (uint32_t)n * OB : kOobOffset;
        if constexpr (OUT == kOutF32)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__builtin_bit_cast(uint32_t, s0),
                                                        __builtin_bit_cast(uint32_t, s1)},
                                                  rC, voffc, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(s0, s1), rC, voffc, 0, 0);
    }
}

template <int MB, int WAVES, int DEPTH>
struct SkinnyCfg {
    static constexpr int ROWS_A = MB * 16;
    static constexpr int ROWS = ROWS_A + kSkinnyTileN;      // stage rows: A rows, then B rows
    static constexpr int STAGE = ROWS * kTileKBytes;        // bytes per stage
    static constexpr int RING = DEPTH * STAGE;              // bytes per wave
    static constexpr int LOADS = ROWS / 8;                  // 1 KiB wave loads per stage
    static constexpr int RED = WAVES * ROWS_A * kRedPitch * 4;
    static constexpr int LDS = WAVES * RING > RED ? WAVES * RING : RED;
    static_assert(ROWS_A % 8 == 0, "a wave load must not mix A and B rows");
    static_assert(LDS <= 160 * 1024, "gfx950 LDS is 160 KiB per workgroup");
    static_assert((DEPTH - 1) * LOADS < 64, "vmcnt holds 6 bits");
};

template <int MB, int ELEM, int OUT, int WAVES, int DEPTH, bool ROTATE>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_skinny_kernel(const SkinnyArgs p)
{
    using Cfg = SkinnyCfg<MB, WAVES, DEPTH>;
    constexpr int NB = kSkinnyTileN / 16;
    constexpr int L = Cfg::LOADS;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg::LDS];

    const int w = wave_id();
    const int l = lane_id();
    const int q = l >> 4, r16 = l & 15;
    const int n0 = blockIdx.x * kSkinnyTileN;
    const uint32_t kb = (uint32_t)p.kbytes;
    const int rows_b = min(p.N - n0, kSkinnyTileN);
    const auto rA = make_rsrc(p.A, (uint32_t)p.M * kb);
    const auto rB = make_rsrc((const uint8_t *)p.B + (size_t)n0 * kb, (uint32_t)rows_b * kb);
    const int nk = p.k_tiles;
    const uint32_t tail = (uint32_t)p.tail_bytes;
    uint8_t *const ring = lds + w * Cfg::RING;

    // Wave load j of a stage covers stage rows 8j .. 8j + 7; lane l takes row
    // 8j + l / 8 and the logical chunk that the swizzle puts in slot l % 8.
    // Rows past M or N lie past their buffer's record count (zeros).
    uint32_t voff[L];
    uint32_t half_keep = 0;     // bit j: this lane's chunk lies in the first 64 bytes
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int row = 8 * j + (l >> 3);
        const int c = swz_chunk(row, l & 7);
        const int src_row = row < Cfg::ROWS_A ? row : row - Cfg::ROWS_A;
        voff[j] = (uint32_t)src_row * kb + (uint32_t)c * kChunkBytes;
        half_keep |= (c < kChunksPerRow / 2 ? 1u : 0u) << j;
    }

    const int per = (nk + WAVES - 1) / WAVES;
    const int first = w * per;
    const int nt = max(0, min(per, nk - first));         // this wave's steps
    const int rot = ROTATE ? (int)((blockIdx.x * 37u) % (uint32_t)max(nk, 1)) : 0;

    // Step t of this wave into ring stage s (every load is issued; the ones
    // past the run or past K in a half-filled last step are out of range).
    auto issue = [&](int t, int s) {
        int kt = first + t + rot;
        kt = kt >= nk ? kt - nk : kt;
        const bool in = t < nt;
        const bool part = (kt == nk - 1) & (tail != (uint32_t)kTileKBytes);
        const uint32_t soff = in ? (uint32_t)kt * kTileKBytes : 0u;
        uint8_t *const dst = ring + s * Cfg::STAGE;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const bool keep = in & (!part | (((half_keep >> j) & 1u) != 0));
            buf_load16_to_lds(8 * j < Cfg::ROWS_A ? rA : rB, dst + j * 1024, keep_or_oob(keep, voff[j]), soff);
        }
        issue_fence();
    };

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA operands of one stage: lane l takes row l % 16 of each 16-row
    // block and the logical chunks l / 16 and 4 + l / 16 (the tiled kernels'
    // lane/K assignment).
    auto compute = [&](int s) {
        const uint8_t *const st = ring + s * Cfg::STAGE;
        auto frag = [&](int row, int c) {
            return lds_load16(st + row * kTileKBytes + swz_chunk(row, c) * kChunkBytes);
        };
        u32x4 a[MB][2], b[NB][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
                b[j][h] = frag(Cfg::ROWS_A + j * 16 + r16, h * 4 + q);
#pragma unroll
            for (int i = 0; i < MB; ++i)
                a[i][h] = frag(i * 16 + r16, h * 4 + q);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if constexpr (ELEM == kBf16) {
                    acc[i][j] = mfma_bf16(b[j][0], a[i][0], acc[i][j]);
                    acc[i][j] = mfma_bf16(b[j][1], a[i][1], acc[i][j]);
                } else if constexpr (ELEM == kI8) {
                    acc[i][j] = mfma_i8(b[j][0], a[i][0], acc[i][j]);
                    acc[i][j] = mfma_i8(b[j][1], a[i][1], acc[i][j]);
                } else {
                    acc[i][j] = mfma_fp8x8(join32(b[j][0], b[j][1]), join32(a[i][0], a[i][1]), acc[i][j]);
                }
            }
    };

    // Waiting for the oldest stage leaves the DEPTH - 1 younger ones in flight.
    constexpr int kVm = (DEPTH - 1) * L;
    constexpr int kWaitOldest = (kWaitVmcnt0 & ~0xC00F) | (kVm & 0xF) | ((kVm >> 4) << 14);
    constexpr int kWaitLds = 0xC07F;                 // lgkmcnt(0) only
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
        issue(s, s);
    int s = 0;
    for (int t = 0; t < nt; ++t) {
        __builtin_amdgcn_s_waitcnt(kWaitOldest);
        compute(s);
        __builtin_amdgcn_s_waitcnt(kWaitLds);         // the stage's reads are done before its refill
        issue(t + DEPTH, s);
        s = s + 1 == DEPTH ? 0 : s + 1;
    }
    // Out-of-range loads still write (zeros) into LDS: drain them before the
    // ring is reused for the reduction.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 & ~0x0F00);
    __syncthreads();

    skinny_finish<MB, OUT, WAVES, ELEM == kI8 ? 1 : 0>(p, acc, lds, n0);
}

template <int MB, int ELEM, int OUT, int WAVES, int DEPTH, bool ROTATE>
static hipError_t launch_skinny(const SkinnyArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_skinny_kernel<MB, ELEM, OUT, WAVES, DEPTH, ROTATE>), dim3(grid), dim3(64 * WAVES), 0,
                       s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny GEMM with B pre-shuffled.  The pre-shuffled image stores each
// 16-column block's operand for 64 bytes of K as one contiguous 1 KiB, in
// the MFMA lane order (lane l: column l % 16, K bytes 16 (l / 16) .. +15), so
// B goes straight from HBM into VGPRs with whole-line, fully contiguous wave
// loads and never touches LDS.  Only A, which every workgroup re-reads from
// L2, is staged: whole-line LDS-writing loads into a per-wave ring, read back
// in the MFMA order like the tiled kernels' A.  The step, the K split over
// the waves, the rotation and the reduction are those of the kernel above.
// ---------------------------------------------------------------------------
template <int MB, int WAVES, int DEPTH, bool BLDS, int BH = 2>
struct SkinnyPreCfg {
    static constexpr int ROWS_A = MB * 16;
    static constexpr int ASTAGE = ROWS_A * kTileKBytes;     // A bytes per stage
    static constexpr int BL = BH * (kSkinnyTileN / 16);     // 1 KiB B loads per stage
    static constexpr int STAGE = ASTAGE + (BLDS ? BL * 1024 : 0);
    static constexpr int RING = DEPTH * STAGE;              // bytes per wave
    static constexpr int AL = ROWS_A / 8;                   // 1 KiB A loads per stage
    static constexpr int LOADS = AL + BL;
    static constexpr int RED = WAVES * ROWS_A * kRedPitch * 4;
    static constexpr int LDS = WAVES * RING > RED ? WAVES * RING : RED;
    static_assert(LDS <= 160 * 1024, "gfx950 LDS is 160 KiB per workgroup");
    static_assert((DEPTH - 1) * LOADS < 64, "vmcnt holds 6 bits");
};

template <int MB, int ELEM, int OUT, int WAVES, int DEPTH, bool BLDS, int ORD>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_skinny_pre_kernel(const SkinnyArgs p)
{
    // Packed int4 B (W4A8): one 1 KiB block per 16 columns and step, i.e. the
    // 64 B-bytes of 128 K values per row; lane group q holds values 32 q ..
    // 32 q + 31, unpacked into two int8 operands, half h pairing with A
    // chunk 2 q + h.  Otherwise two blocks (K bytes 0..63 and 64..127 of the
    // step) pairing with A chunks q and 4 + q.
    //
    // MX (MXFP8, MXFP4): the operands of the fp8 and bf16 schedules (chunks q
    // and q + 4 as one 32-byte e4m3 operand; or per 64-byte half one 16-byte
    // e2m1 operand), scaled per lane by the E8M0 bytes of the scale images:
    // one 16-byte load per lane and stage brings the scales of 4 row blocks
    // (A: the rows' quad; B: the columns' quad) for the 4 K-slices of the
    // step's group.  A group is 4 steps (MXFP8, one 128-element slice per
    // step) or 2 (MXFP4, two per step); each wave's run starts on a group and
    // the ring depth is a multiple of it, so every slice index is a constant.
    constexpr bool W4 = ELEM == kW4A8;
    constexpr bool INT = ELEM == kI8 || W4;
    constexpr bool MX = ELEM == kMx8 || ELEM == kMx4;
    constexpr int SPG = ELEM == kMx8 ? 4 : 2;                 // steps per scale group
    constexpr int BH = W4 ? 1 : 2;
    static_assert(!INT || OUT == kOutBf16, "integer GEMMs write bf16");
    static_assert(!MX || (DEPTH % SPG == 0 && ORD == 1 && !BLDS), "MX: whole scale groups per ring, runs");
    using Cfg = SkinnyPreCfg<MB, WAVES, DEPTH, BLDS, BH>;
    constexpr int NB = kSkinnyTileN / 16;
    constexpr int AL = Cfg::AL;
    constexpr int LOADS = Cfg::LOADS + (MX ? 2 : 0);
    __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg::LDS];

    const int w = wave_id();
    const int l = lane_id();
    const int q = l >> 4, r16 = l & 15;
    const int n0 = blockIdx.x * kSkinnyTileN;
    const uint32_t kb = (uint32_t)p.kbytes;
    const int rows_b = min(p.N - n0, kSkinnyTileN);
    const uint32_t kbB = (uint32_t)p.kbytes_b;
    const auto rA = make_rsrc(p.A, (uint32_t)p.M * kb);
    // The workgroup's 16-column blocks are contiguous in the image (16 * kbB
    // bytes each); a block past N lies past the record count (zeros).
    const auto rB = make_rsrc((const uint8_t *)p.B + (size_t)n0 * kbB, (uint32_t)rows_b * kbB);
    const int nk = p.k_tiles;
    const uint32_t tail = (uint32_t)p.tail_bytes;
    uint8_t *const ring = lds + w * Cfg::RING;

    // A: wave load j covers rows 8j .. 8j + 7 of the stage, as above.
    uint32_t voffA[AL];
    uint32_t half_keep = 0;
#pragma unroll
    for (int j = 0; j < AL; ++j) {
        const int row = 8 * j + (l >> 3);
        const int c = swz_chunk(row, l & 7);
        voffA[j] = (uint32_t)row * kb + (uint32_t)c * kChunkBytes;
        half_keep |= (c < kChunksPerRow / 2 ? 1u : 0u) << j;
    }

    // ORD: 0 runs of steps, rotated start; 1 runs; 2 steps w, w + WAVES, ...,
    // rotated start; 3 the same without rotation
    constexpr bool INTER = ORD >= 2;
    const int per = MX ? ((nk + WAVES - 1) / WAVES + SPG - 1) / SPG * SPG : (nk + WAVES - 1) / WAVES;
    const int first = INTER ? w : w * per;
    const int nt = INTER ? (w < nk ? (nk - w + WAVES - 1) / WAVES : 0) : max(0, min(per, nk - first));
    const int rot = (ORD == 0 || ORD == 2) ? (int)((blockIdx.x * 37u) % (uint32_t)max(nk, 1)) : 0;

    // B of one step: image blocks BH kt + h of 16-column block j.
    u32x4 bq[DEPTH][NB][BH];
    // MX: the scale words of each stage's group (A: row blocks 0..3 of quad 0;
    // B: the columns' quad, whose blocks bq0, bq0 + 1 are this workgroup's).
    u32x4 scA[DEPTH], scB[DEPTH];
    const int G = p.s_groups;
    const auto rSA = make_rsrc(p.sa_img, MX ? (uint32_t)G * 1024u : 0u);
    const auto rSB = make_rsrc(p.sb_img, MX ? (uint32_t)((p.N + 63) / 64) * (uint32_t)G * 1024u : 0u);
    const uint32_t sbase = (uint32_t)(n0 / 64) * (uint32_t)G;
    const bool bq_hi = (n0 & 32) != 0;

    // Step t of this wave into stage s.  Every load is issued; those past the
    // run, or past K in a half-filled last step, are out of range (zeros).
    auto issue = [&](int t, auto s_c) {
        constexpr int S = decltype(s_c)::value;
        int kt = first + (INTER ? WAVES * t : t) + rot;
        kt = kt >= nk ? kt - nk : kt;
        const bool in = t < nt;
        const bool part = (kt == nk - 1) & (tail != (uint32_t)kTileKBytes);
        const uint32_t soffA = in ? (uint32_t)kt * kTileKBytes : 0u;
        uint8_t *const dst = ring + S * Cfg::STAGE;
#pragma unroll
        for (int j = 0; j < AL; ++j) {
            const bool keep = in & (!part | (((half_keep >> j) & 1u) != 0));
            buf_load16_to_lds(rA, dst + j * 1024, keep_or_oob(keep, voffA[j]), soffA);
        }
        const uint32_t soffB = in ? (uint32_t)kt * (uint32_t)(BH * 1024) : 0u;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int h = 0; h < BH; ++h) {
                const bool keep = in & (!part | (h == 0));
                const uint32_t voffB =
                    keep_or_oob(keep, (uint32_t)j * 16u * kbB + (uint32_t)h * 1024u + (uint32_t)l * 16u);
                if constexpr (BLDS)
                    buf_load16_to_lds(rB, dst + Cfg::ASTAGE + (BH * j + h) * 1024, voffB, soffB);
                else
                    bq[S][j][h] = buf_load16(rB, voffB, soffB);
            }
        if constexpr (MX) {
            const uint32_t g = (uint32_t)(kt / SPG);
            const bool sin = in & ((int)g < G);
            scA[S] = buf_load16(rSA, keep_or_oob(sin, g * 1024u + (uint32_t)l * 16u), 0);
            scB[S] = buf_load16(rSB, keep_or_oob(sin, (sbase + g) * 1024u + (uint32_t)l * 16u), 0);
        }
        issue_fence();
    };

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A operands: lane l takes row l % 16 of each 16-row block and chunks
    // l / 16 (paired with K block 2 kt) and 4 + l / 16 (block 2 kt + 1).
    auto compute = [&](auto s_c) {
        constexpr int S = decltype(s_c)::value;
        const uint8_t *const st = ring + S * Cfg::STAGE;
        u32x4 a[MB][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int row = i * 16 + r16;
                const int c = W4 ? 2 * q + h : h * 4 + q;
                a[i][h] = lds_load16(st + row * kTileKBytes + swz_chunk(row, c) * kChunkBytes);
            }
        if constexpr (BLDS) {
            // the staged operand blocks are in lane order already
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int h = 0; h < BH; ++h)
                    bq[S][j][h] = lds_load16(st + Cfg::ASTAGE + (BH * j + h) * 1024 + l * 16);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            u32x4 b0, b1;
            if constexpr (W4) {
                b0 = int4x32_half_to_i8(bq[S][j][0], 0);
                b1 = int4x32_half_to_i8(bq[S][j][0], 1);
            } else {
                b0 = bq[S][j][0];
                b1 = bq[S][j][BH - 1];
            }
            uint32_t sx = 0;
            if constexpr (MX)
                sx = bq_hi ? (j ? scB[S].w : scB[S].z) : (j ? scB[S].y : scB[S].x);
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                if constexpr (MX) {
                    constexpr int GP = S % SPG;                 // the step's place in its group
                    const uint32_t sy = scA[S][i];
                    if constexpr (ELEM == kMx8) {
                        mfma_mx8_a<GP>(acc[i][j], join32(b0, b1), join32(a[i][0], a[i][1]), sx, sy);
                    } else {
                        mfma_mx4_a<2 * GP>(acc[i][j], b0, a[i][0], sx, sy);
                        mfma_mx4_a<2 * GP + 1>(acc[i][j], b1, a[i][1], sx, sy);
                    }
                } else if constexpr (ELEM == kBf16) {
                    acc[i][j] = mfma_bf16(b0, a[i][0], acc[i][j]);
                    acc[i][j] = mfma_bf16(b1, a[i][1], acc[i][j]);
                } else if constexpr (INT) {
                    acc[i][j] = mfma_i8(b0, a[i][0], acc[i][j]);
                    acc[i][j] = mfma_i8(b1, a[i][1], acc[i][j]);
                } else {
                    acc[i][j] = mfma_fp8x8(join32(b0, b1), join32(a[i][0], a[i][1]), acc[i][j]);
                }
            }
        }
    };

    // Waiting for the oldest stage leaves the DEPTH - 1 younger ones in
    // flight.  The run is rounded up to whole rings; the extra steps load and
    // multiply zeros.
    constexpr int kVm = (DEPTH - 1) * LOADS;
    static_assert(kVm < 64, "vmcnt holds 6 bits");
    constexpr int kWaitOldest = (kWaitVmcnt0 & ~0xC00F) | (kVm & 0xF) | ((kVm >> 4) << 14);
    constexpr int kWaitLds = 0xC07F;
    const int ntr = (nt + DEPTH - 1) / DEPTH * DEPTH;
    static_for<DEPTH>([&](auto s_c) { issue(decltype(s_c)::value, s_c); });
    for (int t0 = 0; t0 < ntr; t0 += DEPTH) {
        static_for<DEPTH>([&](auto s_c) {
            __builtin_amdgcn_s_waitcnt(kWaitOldest);
            compute(s_c);
            __builtin_amdgcn_s_waitcnt(kWaitLds);     // the stage's A reads are done before its refill
            issue(t0 + decltype(s_c)::value + DEPTH, s_c);
        });
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 & ~0x0F00);
    if constexpr (MX)
        mfma_drain_acc(acc);                      // the scaled MFMAs are inline assembly
    __syncthreads();
    skinny_finish<MB, OUT, WAVES, ELEM == kI8 ? 1 : (W4 ? 16 : 0)>(p, acc, lds, n0);
}

template <int MB, int ELEM, int OUT, int WAVES, int DEPTH, bool BLDS, int ORD>
static hipError_t launch_skinny_pre(const SkinnyArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_skinny_pre_kernel<MB, ELEM, OUT, WAVES, DEPTH, BLDS, ORD>), dim3(grid), dim3(64 * WAVES), 0,
                       s, a);
    return hipGetLastError();
}

#define TG_SKINNY(MB, ELEM, OUT, WAVES, DEPTH, ROTATE)                                                       \
    SkinnyVariant{MB, ELEM, OUT, WAVES, DEPTH, SkinnyCfg<MB, WAVES, DEPTH>::LDS,                             \
                  &launch_skinny<MB, ELEM, OUT, WAVES, DEPTH, ROTATE>}

#define TG_SKINNY_PRE_O(MB, ELEM, OUT, WAVES, DEPTH, BLDS, ORD)                                              \
    SkinnyVariant{MB, ELEM, OUT, WAVES, DEPTH, SkinnyPreCfg<MB, WAVES, DEPTH, BLDS, ELEM == kW4A8 ? 1 : 2>::LDS, \
                  &launch_skinny_pre<MB, ELEM, OUT, WAVES, DEPTH, BLDS, ORD>, true}
#define TG_SKINNY_PRE_L(MB, ELEM, OUT, WAVES, DEPTH, BLDS) TG_SKINNY_PRE_O(MB, ELEM, OUT, WAVES, DEPTH, BLDS, 1)
#define TG_SKINNY_PRE(MB, ELEM, OUT, WAVES, DEPTH) TG_SKINNY_PRE_L(MB, ELEM, OUT, WAVES, DEPTH, false)

// The first variant of each (rows, elem, out, B layout) is the planner's choice; the
// rest are alternatives compiled into sweep builds only.
static const SkinnyVariant kSkinny[] = {
    TG_SKINNY(1, kBf16, kOutBf16, 8, 3, true), TG_SKINNY(2, kBf16, kOutBf16, 8, 2, true),
    TG_SKINNY(4, kBf16, kOutBf16, 4, 3, true), TG_SKINNY(1, kBf16, kOutF32, 8, 3, true),
    TG_SKINNY(2, kBf16, kOutF32, 8, 2, true),  TG_SKINNY(4, kBf16, kOutF32, 4, 3, true),
    TG_SKINNY(1, kFp8, kOutBf16, 8, 3, true),  TG_SKINNY(2, kFp8, kOutBf16, 8, 2, true),
    TG_SKINNY(4, kFp8, kOutBf16, 4, 3, true),
    // B pre-shuffled (register-staged B, steps in runs, no rotation)
    TG_SKINNY_PRE(1, kBf16, kOutBf16, 12, 2), TG_SKINNY_PRE(2, kBf16, kOutBf16, 12, 2),     // 9
    TG_SKINNY_PRE(4, kBf16, kOutBf16, 8, 2),  TG_SKINNY_PRE(1, kBf16, kOutF32, 12, 2),
    TG_SKINNY_PRE(2, kBf16, kOutF32, 12, 2),  TG_SKINNY_PRE(4, kBf16, kOutF32, 8, 2),
    TG_SKINNY_PRE(1, kFp8, kOutBf16, 12, 2),  TG_SKINNY_PRE(2, kFp8, kOutBf16, 12, 2),      // 15
    TG_SKINNY_PRE(4, kFp8, kOutBf16, 8, 2),
    // integer operands: int8 with B N x K or pre-shuffled, W4A8 pre-shuffled
    TG_SKINNY(1, kI8, kOutBf16, 8, 3, true), TG_SKINNY(2, kI8, kOutBf16, 8, 2, true),          // 18
    TG_SKINNY(4, kI8, kOutBf16, 4, 3, true),
    TG_SKINNY_PRE(1, kI8, kOutBf16, 12, 2), TG_SKINNY_PRE(2, kI8, kOutBf16, 12, 2),             // 21
    TG_SKINNY_PRE(4, kI8, kOutBf16, 8, 2),
    TG_SKINNY_PRE(1, kW4A8, kOutBf16, 12, 2), TG_SKINNY_PRE(2, kW4A8, kOutBf16, 12, 2),         // 24
    TG_SKINNY_PRE(4, kW4A8, kOutBf16, 8, 2),
    // MX block-scaled operands, B pre-shuffled
    TG_SKINNY_PRE(1, kMx8, kOutBf16, 8, 4), TG_SKINNY_PRE(2, kMx8, kOutBf16, 8, 4),           // 27
    TG_SKINNY_PRE(4, kMx8, kOutBf16, 4, 4),
    TG_SKINNY_PRE(1, kMx4, kOutBf16, 12, 2), TG_SKINNY_PRE(2, kMx4, kOutBf16, 12, 2),         // 30
    TG_SKINNY_PRE(4, kMx4, kOutBf16, 8, 2),
#ifdef TGEMM_SWEEP
    // alternatives (sweep builds only) for the 32-row bf16 shape: B N x K
    TG_SKINNY(2, kBf16, kOutBf16, 8, 2, false), TG_SKINNY(2, kBf16, kOutBf16, 4, 4, true),     // 33
    TG_SKINNY(2, kBf16, kOutBf16, 2, 8, true),
    // B pre-shuffled: (waves, stages, B via LDS, order)
    TG_SKINNY_PRE_O(2, kBf16, kOutBf16, 8, 4, false, 0), TG_SKINNY_PRE(2, kBf16, kOutBf16, 8, 4),   // 36
    TG_SKINNY_PRE(2, kBf16, kOutBf16, 16, 2), TG_SKINNY_PRE(2, kBf16, kOutBf16, 12, 3),
    TG_SKINNY_PRE_L(2, kBf16, kOutBf16, 8, 2, true), TG_SKINNY_PRE_O(2, kBf16, kOutBf16, 12, 2, false, 3), // 40
    TG_SKINNY_PRE(2, kBf16, kOutBf16, 8, 3), TG_SKINNY_PRE(2, kBf16, kOutBf16, 10, 2),
    // the 64-row shape
    TG_SKINNY_PRE(4, kBf16, kOutBf16, 4, 4),                                                    // 44
#endif
};

const SkinnyVariant *skinny_variants(int *count)
{
    *count = (int)(sizeof(kSkinny) / sizeof(kSkinny[0]));
    return kSkinny;
}

}  // namespace tg
