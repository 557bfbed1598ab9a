// Tiled GEMM C = A * B^T on gfx950 MFMA, after the preshuffle GEMM pattern
// of FlyDSL's "Kernel Authoring" skill (section 6 "GEMM Pattern
// (Preshuffle)") and the kernel shape of the "Kernel authoring guide"
// (section 11: 256-thread blocks, 2-stage LDS, M at run time).
//
// One workgroup (4 waves) computes a BM x BN tile of C.  The K loop walks
// 128-byte steps (64 bf16 or 128 fp8 elements), i.e. two of the pages'
// 64-byte micro-steps:
//   * A (and B unless pre-shuffled) go global -> LDS with 16-byte buffer
//     loads that write LDS directly (no VGPR staging).  A wave writes 1 KiB
//     contiguously, so the XOR swizzle of 16-byte chunks is realised by each
//     lane choosing its source chunk.  Two LDS stages: tile k+1 is in flight
//     while tile k is consumed.  The K step advances only the scalar offset.
//   * A pre-shuffled B skips LDS: each 1 KiB block of the image is one wave's
//     B operand, loaded with one coalesced 16-byte load per lane into VGPRs,
//     one tile ahead.
//   * MFMA: bf16 16x16x32 (two per 128-byte step) or fp8 16x16x128 (one).
//     The B fragment is passed as the instruction's first operand, so each
//     lane's 4 accumulators are 4 consecutive columns of one row of C.
//   * Epilogue: (acc * s_a) * s_b in fp32, round-to-nearest-even to bf16
//     (or fp32 as is), buffer stores; rows past M and columns past N are
//     dropped by the buffer range check.
//   * B stored K x N (BKN, C = A * B, bf16): a step's 64 K-rows of the
//     tile's BN columns go to LDS by the same direct loads, rows of BN * 2
//     bytes with the 16-byte chunks XOR-swizzled by bkn_swz(k).  The MFMA
//     operand (8 consecutive k of one column per lane) comes out of LDS
//     through the gfx950 transpose read ds_read_b64_tr_b16 (FlyDSL
//     "add-target-atom-op" skill, section 1.5.2 "Shape-product invariants":
//     the copy atom ds_read_tr16_b64 spans 16 lanes; the per-lane layout
//     below was established with an in-bounds probe): within each 16-lane
//     block, lane i receives element
//     i % 4 of the 64 bits fetched by lane 4 e + i / 4, for e = 0..3.  So
//     lane 4 a + b of block q points at row k0 + a, columns c0 + 4 b .. + 3,
//     and lane i of the block ends up with rows k0 .. k0 + 3 of column
//     c0 + i.  Rows past K lie past the end of B and read as zeros.
#include "device.hpp"
#include "kernels.hpp"

namespace tg {

template <int BM, int BN, int WGM, int WGN, int ELEM, bool BPRE, int OUT, bool BKN = false>
struct TiledCfg {
    static constexpr int kWaves = 4;
    static_assert(WGM * WGN == kWaves, "4 waves per workgroup");
    static constexpr int WTM = BM / WGM;             // rows per wave
    static constexpr int WTN = BN / WGN;             // columns per wave
    static constexpr int FM = WTM / 16;              // 16x16 MFMA tiles per wave (rows)
    static constexpr int FN = WTN / 16;              // (columns)
    static constexpr int A_BYTES = BM * kTileKBytes;
    static constexpr int B_BYTES = BPRE ? 0 : BN * kTileKBytes;   // N x K: BN rows; K x N: 64 k-rows of BN * 2
    static constexpr int KN_ROW = BN * 2;                          // bytes of one K-row of a K x N tile (bf16)
    static constexpr int KN_CPR = KN_ROW / kChunkBytes;            // its 16-byte chunks
    static_assert(!BKN || (ELEM == kBf16 && !BPRE && KN_CPR >= 16), "K x N B: bf16, staged in LDS");
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int ROUND_BYTES = kTiledThreads * kChunkBytes;   // one 16B load per thread
    static constexpr int A_ROUNDS = A_BYTES / ROUND_BYTES;
    static constexpr int B_ROUNDS = B_BYTES / ROUND_BYTES;
    static_assert(A_BYTES % ROUND_BYTES == 0 && B_BYTES % ROUND_BYTES == 0, "tile / thread count");
    static_assert(LDS <= 160 * 1024, "gfx950 LDS is 160 KiB per workgroup");
};

template <int BM, int BN, int WGM, int WGN, int ELEM, bool BPRE, int OUT, bool BKN>
__global__ __launch_bounds__(kTiledThreads, 1) void gemm_tiled_kernel(const TiledArgs p)
{
    using Cfg = TiledCfg<BM, BN, WGM, WGN, ELEM, BPRE, OUT, BKN>;
    constexpr int FM = Cfg::FM, FN = Cfg::FN;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg::LDS];

    const int w = wave_id();
    const int l = lane_id();
    const int wm = w / WGN, wn = w % WGN;

    int tm, tn;
    tile_of_wg(blockIdx.x, p.grid, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_a = min(p.M - m0, BM);
    const int rows_b = min(p.N - n0, BN);
    const uint32_t kb = (uint32_t)p.kbytes;
    const auto rA = make_rsrc((const uint8_t *)p.A + (size_t)m0 * kb, (uint32_t)rows_a * kb);
    // K x N B: the resource starts at column n0 and ends with the matrix, so
    // rows past K read zeros (columns past N read neighbouring data or zeros
    // and only feed columns of C that are never stored).
    const uint32_t ldb = (uint32_t)p.ldb_bytes;
    const auto rB = BKN ? make_rsrc((const uint8_t *)p.B + (size_t)n0 * 2, (uint32_t)((size_t)p.K * ldb - (size_t)n0 * 2))
                        : make_rsrc((const uint8_t *)p.B + (size_t)n0 * kb, (uint32_t)rows_b * kb);
    const int nk = p.k_tiles;
    const uint32_t tail = (uint32_t)p.tail_bytes;

    // ---- global -> LDS source offsets (one 16-byte chunk per thread per round).
    // Round r of wave w fills LDS chunks [(4r + w) * 64, +64) of the stage;
    // chunk p sits in row p / 8 at physical slot p % 8, which holds logical
    // chunk (p % 8) ^ swz_row(row).  Bit r of the tail masks says whether the
    // chunk lies inside a partial last K step.
    uint32_t voffA[Cfg::A_ROUNDS];
    uint32_t tailA = 0, tailB = 0;
#pragma unroll
    for (int r = 0; r < Cfg::A_ROUNDS; ++r) {
        const int pc = (r * 4 + w) * 64 + l;
        const int row = pc >> 3;
        const int c = swz_chunk(row, pc & 7);
        voffA[r] = (uint32_t)row * kb + (uint32_t)c * kChunkBytes;
        tailA |= ((uint32_t)(c * kChunkBytes) < tail ? 1u : 0u) << r;
    }
    uint32_t voffB[Cfg::B_ROUNDS > 0 ? Cfg::B_ROUNDS : 1];
#pragma unroll
    for (int r = 0; r < Cfg::B_ROUNDS; ++r) {
        const int pc = (r * 4 + w) * 64 + l;
        if constexpr (BKN) {
            // physical chunk pc % CPR of K-row pc / CPR holds logical chunk
            // (pc % CPR) ^ bkn_swz(row); K tails need no mask (see rB)
            const int row = pc / Cfg::KN_CPR;
            const int c = (pc % Cfg::KN_CPR) ^ bkn_swz(row);
            voffB[r] = (uint32_t)row * ldb + (uint32_t)c * kChunkBytes;
            tailB |= 1u << r;
        } else {
            const int row = pc >> 3;
            const int c = swz_chunk(row, pc & 7);
            voffB[r] = (uint32_t)row * kb + (uint32_t)c * kChunkBytes;
            tailB |= ((uint32_t)(c * kChunkBytes) < tail ? 1u : 0u) << r;
        }
    }

    auto issue_lds = [&](int kt, int stage) {
        const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
        uint8_t *sA = lds + stage * Cfg::STAGE;
        const uint32_t soff = (uint32_t)kt * kTileKBytes;
#pragma unroll
        for (int r = 0; r < Cfg::A_ROUNDS; ++r) {
            const uint32_t vo = (!part || ((tailA >> r) & 1u)) ? voffA[r] : kOobOffset;
            buf_load16_to_lds(rA, sA + (r * 4 + w) * 1024, vo, soff);
        }
        if constexpr (!BPRE) {
            uint8_t *sB = sA + Cfg::A_BYTES;
            // K x N: a step is 64 K-rows of B
            const uint32_t soffB = BKN ? (uint32_t)kt * 64u * ldb : soff;
#pragma unroll
            for (int r = 0; r < Cfg::B_ROUNDS; ++r) {
                const uint32_t vo = (!part || ((tailB >> r) & 1u)) ? voffB[r] : kOobOffset;
                buf_load16_to_lds(rB, sB + (r * 4 + w) * 1024, vo, soffB);
            }
        }
    };

    // ---- pre-shuffled B: block (nb, kb64) at nb * 16 * kb + kb64 * 1024; lane l
    // reads its 16 bytes at + 16 * l.  Column block j of this wave is n-block
    // wn * FN + j of the workgroup.
    uint32_t voffBs[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        voffBs[j] = (uint32_t)(wn * FN + j) * 16u * kb + (uint32_t)l * 16u;

    auto load_bpre = [&](int kt, u32x4 (&bq)[FN][2]) {
        const bool part = (kt == nk - 1) && tail != (uint32_t)kTileKBytes;
        const uint32_t soff = (uint32_t)kt * 2048u;   // two 1 KiB blocks per 128-byte K step
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            bq[j][0] = buf_load16(rB, voffBs[j], soff);
            bq[j][1] = part ? u32x4{0, 0, 0, 0} : buf_load16(rB, voffBs[j] + 1024u, soff);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS byte address of logical chunk c of tile row `row` in a stage operand.
    auto lds_chunk = [&](const uint8_t *base, int row, int c) -> const uint8_t * {
        return base + row * kTileKBytes + swz_chunk(row, c) * kChunkBytes;
    };

    const int q = l >> 4;       // K slot group of this lane
    const int r16 = l & 15;     // row within a 16-row block

    // K x N B: the operand of column block j for sub-step s (k = 32 s + 8 q
    // .. + 7 of the step, one column per lane) as two transpose reads.
    auto bkn_frag = [&](const uint8_t *sB, int s, int j) -> u32x4 {
        const int col = wn * Cfg::WTN + j * 16 + 4 * (r16 & 3);      // this lane's 4 source columns
        const int c = (col * 2) >> 4, off = (col * 2) & 15;
        u32x2 h[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int k = 32 * s + 8 * q + 4 * t + (r16 >> 2);
            h[t] = lds_read_tr16(sB + k * Cfg::KN_ROW + ((c ^ bkn_swz(k)) << 4) + off);
        }
        return u32x4{h[0].x, h[0].y, h[1].x, h[1].y};
    };

    auto compute = [&](int stage, const u32x4 (&bq)[FN][2]) {
        const uint8_t *sA = lds + stage * Cfg::STAGE;
        const uint8_t *sB = sA + Cfg::A_BYTES;
        if constexpr (ELEM == kBf16) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int c = s * 4 + q;
                u32x4 bf[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (BPRE)
                        bf[j] = bq[j][s];
                    else if constexpr (BKN)
                        bf[j] = bkn_frag(sB, s, j);
                    else
                        bf[j] = lds_load16(lds_chunk(sB, wn * Cfg::WTN + j * 16 + r16, c));
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const u32x4 af = lds_load16(lds_chunk(sA, wm * Cfg::WTM + i * 16 + r16, c));
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = mfma_bf16(bf[j], af, acc[i][j]);
                }
            }
        } else {
            u32x4 blo[FN], bhi[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (BPRE) {
                    blo[j] = bq[j][0];
                    bhi[j] = bq[j][1];
                } else {
                    const int row = wn * Cfg::WTN + j * 16 + r16;
                    blo[j] = lds_load16(lds_chunk(sB, row, q));
                    bhi[j] = lds_load16(lds_chunk(sB, row, q + 4));
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * Cfg::WTM + i * 16 + r16;
                const u32x4 alo = lds_load16(lds_chunk(sA, row, q));
                const u32x4 ahi = lds_load16(lds_chunk(sA, row, q + 4));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma_fp8(blo[j], bhi[j], alo, ahi, acc[i][j]);
            }
        }
    };

    // ---- main loop.  One step: wait until the step's tile has landed and
    // every wave is done with the other stage, start the next tile into that
    // stage (and the next pre-shuffled B fragments into the other register
    // set), then run this tile's MFMAs.  Steps go in pairs so that stage and
    // register set are compile-time constants.
    u32x4 bq0[FN][2], bq1[FN][2];
    auto step = [&](int kt, int stage, const u32x4 (&cur)[FN][2], u32x4 (&nxt)[FN][2]) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (kt + 1 < nk) {
            issue_lds(kt + 1, stage ^ 1);
            if constexpr (BPRE)
                load_bpre(kt + 1, nxt);
        }
        compute(stage, cur);
    };
    if (nk > 0) {
        issue_lds(0, 0);
        if constexpr (BPRE)
            load_bpre(0, bq0);
    }
    for (int kt = 0; kt < nk; ++kt) {
        step(kt, kt & 1, bq0, bq1);
        if constexpr (BPRE) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                bq0[j][0] = bq1[j][0];
                bq0[j][1] = bq1[j][1];
            }
        }
    }

    // ---- epilogue: scale, bias, activation, convert, store.  Lane l holds
    // C[row][col .. col+3] with row = l % 16 and col = 4 * (l / 16) inside
    // each 16x16 tile.
    const EpiView ev = epi_view(p.epi, p.M, p.N);
    constexpr int OB = OUT == kOutF32 ? 4 : 2;
    const uint32_t ldc = (uint32_t)p.N * OB;
    const auto rC = make_rsrc((uint8_t *)p.C + (size_t)m0 * ldc, (uint32_t)rows_a * ldc);
    // Row blocks outside, column blocks inside: adjacent pieces of a C row
    // leave back to back and merge in the L2 into whole lines.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = wm * Cfg::WTM + i * 16 + r16;
        const float sa = epi_row_scale(ev, m0 + row);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * Cfg::WTN + j * 16 + 4 * q;
            const uint32_t voff = col < p.N ? (uint32_t)row * ldc + (uint32_t)col * OB : kOobOffset;
            const f32x4 v = epi_apply4(ev, acc[i][j], sa, epi_col_scale4(ev, col), epi_bias4(ev, col));
            if constexpr (OUT == kOutF32) {
                buf_store16(rC, __builtin_bit_cast(u32x4, v), voff);
            } else {
                buf_store8(rC, u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)}, voff);
            }
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int ELEM, bool BPRE, int OUT, bool BKN>
static hipError_t launch_tiled(const TiledArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WGM, WGN, ELEM, BPRE, OUT, BKN>), dim3(a.grid),
                       dim3(kTiledThreads), 0, s, a);
    return hipGetLastError();
}

#define TG_TILED_L(BM, BN, WGM, WGN, ELEM, BPRE, OUT, BKN)                                 \
    TiledVariant{BM, BN, WGM, WGN, ELEM, OUT, BPRE,                                         \
                 TiledCfg<BM, BN, WGM, WGN, ELEM, BPRE, OUT, BKN>::LDS, 2,                  \
                 &launch_tiled<BM, BN, WGM, WGN, ELEM, BPRE, OUT, BKN>, BKN}
#define TG_TILED(BM, BN, WGM, WGN, ELEM, BPRE, OUT) TG_TILED_L(BM, BN, WGM, WGN, ELEM, BPRE, OUT, false)

static const TiledVariant kTiled[] = {
    TG_TILED(256, 256, 2, 2, kBf16, false, kOutBf16),
    TG_TILED(256, 256, 2, 2, kBf16, false, kOutF32),
    TG_TILED(256, 256, 1, 4, kBf16, true, kOutBf16),
    TG_TILED(256, 256, 1, 4, kBf16, true, kOutF32),
    TG_TILED(256, 256, 2, 2, kFp8, false, kOutBf16),
    TG_TILED(256, 256, 1, 4, kFp8, true, kOutBf16),
    TG_TILED(128, 128, 2, 2, kBf16, false, kOutBf16),
    TG_TILED(128, 128, 2, 2, kBf16, false, kOutF32),
    TG_TILED(128, 128, 2, 2, kBf16, true, kOutBf16),
    TG_TILED(128, 128, 2, 2, kBf16, true, kOutF32),
    TG_TILED(128, 128, 2, 2, kFp8, false, kOutBf16),
    TG_TILED(128, 128, 2, 2, kFp8, true, kOutBf16),
    // B stored K x N (bf16)
    TG_TILED_L(256, 256, 2, 2, kBf16, false, kOutBf16, true),
    TG_TILED_L(256, 256, 2, 2, kBf16, false, kOutF32, true),
    TG_TILED_L(128, 128, 2, 2, kBf16, false, kOutBf16, true),
    TG_TILED_L(128, 128, 2, 2, kBf16, false, kOutF32, true),
};

const TiledVariant *tiled_variants(int *count)
{
    *count = (int)(sizeof(kTiled) / sizeof(kTiled[0]));
    return kTiled;
}

}  // namespace tg
