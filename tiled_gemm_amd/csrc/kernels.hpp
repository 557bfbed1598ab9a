// Kernel argument blocks and launcher entry points shared by the HIP kernel
// translation units and the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "layout.hpp"

namespace tg {

// kMx8 / kMx4: MX block-scaled e4m3 / e2m1 operands, one E8M0 scale per 32
// elements along K.  kI8: int8 A and B; kW4A8: int8 A, packed int4 B.
enum Elem { kBf16 = 0, kFp8 = 1, kMx8 = 2, kMx4 = 3, kI8 = 4, kW4A8 = 5 };
enum Out { kOutF32 = 0, kOutBf16 = 1 };

// Epilogue operands (device pointers): C = act((acc * s_a) * s_b + bias).
enum EpiAct { kActNone = 0, kActRelu = 1, kActSilu = 2, kActGelu = 3 };
struct EpiArgs {
    const float *sa;        // nullptr (1), one value for every row, or one per row of C
    const float *sb;        // nullptr (1), one value for every column, or one per column
    const float *bias;      // nullptr (0) or one per column
    int32_t sa_rows;        // 0: sa[0] for every row; 1: sa[row]
    int32_t sb_cols;        // 0: sb[0] for every column; 1: sb[col]
    int32_t act;            // EpiAct
};

struct TiledArgs {
    const void *A;
    const void *B;
    void *C;
    EpiArgs epi;
    int32_t M, N;
    int32_t kbytes;         // bytes of one row of A (K * elem_bytes)
    int32_t k_tiles;        // ceil(kbytes / 128)
    int32_t tail_bytes;     // valid bytes of the last K tile: 64 or 128
    int32_t grid, tiles_m, tiles_n, group_m;
    // MX operands only: the block-scale images of A and B (see
    // BscaleArgs) and their number of 4-slice groups along K.
    const uint8_t *sa_img;
    const uint8_t *sb_img;
    int32_t s_groups;
    int32_t kbytes_b;       // bytes of one row of B (kbytes, or kbytes / 2 for int4 B)
    int32_t K;              // elements along K
    int32_t ldb_bytes;      // B stored K x N: bytes of one row of B (N * elem_bytes)
    int32_t lda_bytes;      // A stored K x M: bytes of one row of A (M * elem_bytes)
    // Split K: with splits > 1 the launch has grid = tiles * splits
    // workgroups; workgroup g takes tile g % tiles and the split_steps K steps
    // starting at step (g / tiles) * split_steps (the last split: the rest),
    // and writes its fp32 partial tile to C + (g / tiles) * M * N * 4 bytes
    // with the identity epilogue.  splits == 1: the whole K, C as given.
    int32_t splits;
    int32_t split_steps;
};

// Sum of the split-K partials and the epilogue: C[m][n] = cvt(epi(sum over
// s in order of W[s][m][n])), W holding `splits` fp32 M x N matrices.
struct SplitReduceArgs {
    const float *W;
    void *C;
    EpiArgs epi;
    int32_t M, N;
    int32_t splits;
    int32_t out;            // kOutF32 or kOutBf16
};

// Block-scale image of an MX operand with R rows: the bytes
// (ceil(R / 64), G, 64, 4, 4) in row-major order -- row quad (64 rows), group
// of 4 MFMA K-slices (128 elements each), lane l, 16-row block b of the quad,
// slice s of the group -- holding the E8M0 scale of row 64 quad + 16 b + l % 16
// for the 32 elements of slice 4 g + s that lane l feeds the MFMA
// (elements 32 (l / 16) .. +31 of the slice); 127 (unit scale) past the rows
// or the blocks.  One 16-byte load per lane brings a wave the scales of 4 row
// blocks for 4 K-slices.
struct BscaleArgs {
    const uint8_t *src;     // R x (K / 32) E8M0 bytes, row-major
    uint8_t *dst;           // the image
    int32_t rows;           // R
    int32_t kblocks;        // K / 32
    int32_t groups;         // G = ceil(ceil(K / 128) / 4)
    int32_t quads;          // ceil(R / 64)
    // 0: the layout above.  1: the 32x32x64 MFMA's (MXFP4 tile kernel): word
    // w of lane l, byte b holds row 64 quad + 32 (w / 2) + l % 32, K block
    // 16 g + 2 (2 b + w % 2) + l / 32, so one 16-byte load per lane brings
    // both 32-row halves of a quad for the 8 64-element slices of a group.
    int32_t form;
};

struct SkinnyArgs {
    const void *A;
    const void *B;
    void *C;
    EpiArgs epi;
    int32_t M, N;
    int32_t kbytes;
    int32_t k_tiles;
    int32_t tail_bytes;
    int32_t kbytes_b;       // bytes of one row of B (kbytes, or kbytes / 2 for int4 B)
    // MX operands only: the block-scale images (see BscaleArgs) and their
    // number of 4-slice groups along K.
    const uint8_t *sa_img;
    const uint8_t *sb_img;
    int32_t s_groups;
};

struct PreshuffleArgs {
    const void *B;
    void *Bs;
    Layout src;             // B bytes through the 5 pre-shuffle coordinates
    Layout dst;             // the pre-shuffled image
    int32_t nblocks;        // N / 16
    int32_t kblocks;        // kbytes / 64
};

// Tiled-kernel variants compiled into the library.
struct TiledVariant {
    int bm, bn, wgm, wgn;   // output tile and wave grid (wgm x wgn waves)
    int elem, out;
    bool preshuffled;
    int lds_bytes;
    int lds_stages;         // K steps the LDS ring holds
    hipError_t (*launch)(const TiledArgs &, hipStream_t);
    bool bkn = false;       // B stored K x N
    bool akm = false;       // A stored K x M
};

struct SkinnyVariant {
    int mblocks;            // 16-row blocks of M covered (M <= 16 * mblocks)
    int elem, out;
    int waves;              // waves per workgroup, each taking a slice of K
    int stages;             // LDS stages per wave
    int lds_bytes;
    hipError_t (*launch)(const SkinnyArgs &, int grid, hipStream_t);
    bool preshuffled = false;   // B is the pre-shuffled image (register-staged B)
};

constexpr int kSkinnyTileN = 32;
constexpr int kTiledThreads = 256;

const TiledVariant *tiled_variants(int *count);
hipError_t launch_split_reduce(const SplitReduceArgs &a, hipStream_t s);
const TiledVariant *pipe_variants(int *count);
const TiledVariant *dma_variants(int *count);
const TiledVariant *mxw_variants(int *count);   // MX on the 32x32x64 scaled MFMA
const SkinnyVariant *skinny_variants(int *count);
hipError_t launch_preshuffle(const PreshuffleArgs &, hipStream_t);
hipError_t launch_bscale_image(const BscaleArgs &, hipStream_t);

// The library's static split-K workspace (gemm_run_ws_noalloc): its device
// address on the current device (looked up on the first call per device).
constexpr size_t kStaticWorkspaceBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
hipError_t static_workspace(void **ptr);

}  // namespace tg
