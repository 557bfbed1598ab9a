// C ABI of the tiled GEMM library (declared in include/tgemm.h): the host
// planner (shape validation, static tile table, layouts, raster) and the
// launchers.  Host code only; the kernels live in the .hip files.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "tgemm.h"
#include "kernels.hpp"
#include "layout.hpp"

using tg::Layout;

struct gemm_plan {
    gemm_plan_info info;
    int64_t kbytes;                    // bytes of one row of A
    int64_t kbytes_b;                  // bytes of one row of B
    int32_t k_tiles, tail_bytes;
    const tg::TiledVariant *tiled;     // kernel == 0
    const tg::SkinnyVariant *skinny;   // kernel == 1
    // Split K with a workspace (gemm_run_ws): the 256 x 256 fp32-output
    // variant, the number of K slices and the steps per slice; splits == 1
    // when splitting does not pay.
    const tg::TiledVariant *split_v;
    int32_t splits, split_steps, split_grid, split_tiles_m, split_tiles_n, split_group_m;
};

namespace {

thread_local std::string g_last_error;

// The plan's tile kernel is the 32x32x64 MX one, which reads block-scale
// image form 1.
bool wide_scales(const gemm_plan *p)
{
    int n = 0;
    const tg::TiledVariant *x = tg::mxw_variants(&n);
    return p->info.kernel == 0 && p->tiled && p->tiled >= x && p->tiled < x + n;
}

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void ok() { g_last_error.clear(); }

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxRowBytes = int64_t(1) << 23;    // 256 rows stay below 2^31 bytes of buffer range
constexpr int kLdsLimit = 160 * 1024;                   // gfx950 LDS per workgroup

bool is_mx(int dtype) { return dtype == GEMM_MXFP8_OUT_BF16 || dtype == GEMM_MXFP4_OUT_BF16; }
bool is_int(int dtype) { return dtype == GEMM_I8_OUT_BF16 || dtype == GEMM_W4A8_OUT_BF16; }
// Bits per element of A.
int elem_bits_of(int dtype)
{
    switch (dtype) {
    case GEMM_E4M3_OUT_BF16:
    case GEMM_MXFP8_OUT_BF16:
    case GEMM_I8_OUT_BF16:
    case GEMM_W4A8_OUT_BF16:
        return 8;
    case GEMM_MXFP4_OUT_BF16:
        return 4;
    default:
        return 16;
    }
}
int b_elem_bits_of(int dtype) { return dtype == GEMM_W4A8_OUT_BF16 ? 4 : elem_bits_of(dtype); }
int out_bytes_of(int dtype) { return dtype == GEMM_BF16_OUT_F32 ? 4 : 2; }
int elem_of(int dtype)
{
    switch (dtype) {
    case GEMM_E4M3_OUT_BF16:
        return tg::kFp8;
    case GEMM_MXFP8_OUT_BF16:
        return tg::kMx8;
    case GEMM_MXFP4_OUT_BF16:
        return tg::kMx4;
    case GEMM_I8_OUT_BF16:
        return tg::kI8;
    case GEMM_W4A8_OUT_BF16:
        return tg::kW4A8;
    default:
        return tg::kBf16;
    }
}
// 4-slice groups of K (one MFMA K-slice is 128 elements).
int64_t scale_groups(int64_t K) { return ((K + 127) / 128 + 3) / 4; }
int out_of(int dtype) { return dtype == GEMM_BF16_OUT_F32 ? tg::kOutF32 : tg::kOutBf16; }

// Sweep builds (-DTGEMM_SWEEP) also compile the alternative tile
// configurations of every kernel family and let TGEMM_VARIANT=<family>:<index>
// pick one of them by its index in the family's table (family: pipe, dma,
// mxw or skinny).  A default build has neither the alternatives nor this
// hook: its plans depend on the arguments of gemm_plan_create[_opt] only.
#ifdef TGEMM_SWEEP
template <typename V, typename Pred>
const V *sweep_pick(const char *family, const V *v, int n, Pred ok)
{
    const char *e = getenv("TGEMM_VARIANT");
    const size_t len = strlen(family);
    if (!e || strncmp(e, family, len) != 0 || e[len] != ':')
        return nullptr;
    const int k = atoi(e + len + 1);
    return k >= 0 && k < n && ok(v[k]) ? &v[k] : nullptr;
}
#define TG_SWEEP_PICK(FAMILY, V, N, PRED)                        \
    if (const auto *sv_ = sweep_pick(FAMILY, V, N, PRED))      \
        return sv_;
#else
#define TG_SWEEP_PICK(FAMILY, V, N, PRED)
#endif

template <typename V, typename Pred>
const V *first_of(const V *v, int n, Pred ok)
{
    for (int i = 0; i < n; ++i)
        if (ok(v[i]))
            return &v[i];
    return nullptr;
}

// Static tile table: the first entry of the chosen kernel family whose
// predicate holds.  `kc` is the caller's gemm_kernel_choice (GEMM_KERNEL_AUTO:
// the planner's own pick by shape).  force256: 256 x 256 tiles with fp32
// output (the split-K partial tiles).
const tg::TiledVariant *pick_tiled(const gemm_plan_info &I, int kc, bool force256 = false)
{
    int n = 0;
    const tg::TiledVariant *v = tg::tiled_variants(&n);
    const bool pre = I.layout == GEMM_LAYOUT_BT_PRESHUFFLED;
    const bool bkn = I.layout == GEMM_LAYOUT_BN || I.layout == GEMM_LAYOUT_AT_BN;
    const bool akm = I.layout == GEMM_LAYOUT_AT || I.layout == GEMM_LAYOUT_AT_BN;
    const int elem = elem_of(I.dtype), out = force256 ? tg::kOutF32 : out_of(I.dtype);
    const bool any256 = kc == GEMM_KERNEL_AUTO || kc == GEMM_KERNEL_TILE256;
    int nd = 0, nb = 0;
    const tg::TiledVariant *d = tg::dma_variants(&nd);
    const tg::TiledVariant *b = tg::pipe_variants(&nb);
    // A stored K x M, and 8-bit B stored K x N: only the LDS-staged 256 x 256
    // kernel reads them.
    if (akm || (bkn && (elem == tg::kFp8 || elem == tg::kI8))) {
        if (!any256)
            return nullptr;
        auto ok = [&](const tg::TiledVariant &x) {
            return x.akm == akm && x.elem == elem && x.out == out && x.bkn == bkn;
        };
        TG_SWEEP_PICK("dma", d, nd, ok)
        return first_of(d, nd, ok);
    }
    if (is_mx(I.dtype) || is_int(I.dtype)) {
        // MX and integer operands: 256 x 256 tiles at any M, N (tails are
        // masked).  MX tiles run on the 32x32x64 kernel (twice the e2m1 rate
        // of the 16x16x128 form, and 8 waves); GEMM_KERNEL_PIPE4 picks the
        // 16x16x128 form on the 4-wave pipelined kernel.  Integer tiles run on
        // the pipelined kernel, 8 waves, or 4 with GEMM_KERNEL_PIPE4.
        if (is_mx(I.dtype) && any256) {
            int nw = 0;
            const tg::TiledVariant *x = tg::mxw_variants(&nw);
            auto ok = [&](const tg::TiledVariant &y) { return y.elem == elem && y.preshuffled == pre; };
            TG_SWEEP_PICK("mxw", x, nw, ok)
            return first_of(x, nw, ok);
        }
        // int8 with B stored N x K: the LDS-staged kernel, whose loads cover
        // whole 128-byte lines of B (as for fp8); the split-K partial tiles
        // (fp32 out) stay on the pipelined kernel.
        if (elem == tg::kI8 && !pre && any256 && out == tg::kOutBf16) {
            auto ok = [&](const tg::TiledVariant &x) {
                return x.elem == elem && x.out == out && !x.preshuffled && !x.bkn && !x.akm;
            };
            TG_SWEEP_PICK("dma", d, nd, ok)
            if (const tg::TiledVariant *x = first_of(d, nd, ok))
                return x;
        }
        const int waves = kc == GEMM_KERNEL_PIPE4 ? 4 : 8;
        if (!(any256 || kc == GEMM_KERNEL_PIPE || kc == GEMM_KERNEL_PIPE4) || (is_mx(I.dtype) && waves != 4))
            return nullptr;
        auto ok = [&](const tg::TiledVariant &y) {
            return y.elem == elem && y.out == out && y.preshuffled == pre && y.wgm * y.wgn == waves;
        };
        TG_SWEEP_PICK("pipe", b, nb, ok)
        return first_of(b, nb, ok);
    }
    int tile = 0;
    if (force256 || kc == GEMM_KERNEL_TILE256 || kc == GEMM_KERNEL_PIPE || kc == GEMM_KERNEL_PIPE4 ||
        kc == GEMM_KERNEL_GENERIC_256)
        tile = 256;
    else if (kc == GEMM_KERNEL_GENERIC_128)
        tile = 128;
    else {
        const int64_t big = ((I.M + 255) / 256) * ((I.N + 255) / 256);
        tile = big >= 128 ? 256 : 128;
    }
    if (tile == 256 && any256) {
        // bf16 and fp8 with B stored N x K (bf16 also K x N): both operands
        // staged through LDS by the loads' own LDS writes (gemm_dma.hip: whole
        // 128-byte lines of B, where the register-staged kernel's MFMA lane
        // order can only load half lines; K x N through the transpose read).
        auto ok = [&](const tg::TiledVariant &x) {
            return x.elem == elem && x.out == out && x.preshuffled == pre && x.bkn == bkn && !x.akm;
        };
        TG_SWEEP_PICK("dma", d, nd, ok)
        if ((elem == tg::kBf16 || elem == tg::kFp8) && !pre)
            return first_of(d, nd, ok);
    }
    // Otherwise 256 x 256 tiles run the software-pipelined kernel (B N x K or
    // pre-shuffled, B straight to registers), 8 waves, or 4 waves with AGPR
    // accumulators for GEMM_KERNEL_PIPE4.
    if (tile == 256 && !bkn && kc != GEMM_KERNEL_GENERIC_256) {
        const int waves = kc == GEMM_KERNEL_PIPE4 ? 4 : 8;
        auto ok = [&](const tg::TiledVariant &y) {
            return y.elem == elem && y.out == out && y.preshuffled == pre && y.wgm * y.wgn == waves;
        };
        TG_SWEEP_PICK("pipe", b, nb, ok)
        return first_of(b, nb, ok);
    }
    if (kc == GEMM_KERNEL_PIPE || kc == GEMM_KERNEL_PIPE4)
        return nullptr;
    return first_of(v, n, [&](const tg::TiledVariant &x) {
        return x.bm == tile && x.bn == tile && x.elem == elem && x.out == out && x.preshuffled == pre &&
               x.bkn == bkn;
    });
}

const tg::SkinnyVariant *pick_skinny(const gemm_plan_info &I, int kc)
{
    // Skinny kernels: bf16, fp8 and int8 with B N x K or pre-shuffled; W4A8
    // and the MX formats with B pre-shuffled.  Only the planner's own choice
    // (GEMM_KERNEL_AUTO) takes them.
    const bool pre = I.layout == GEMM_LAYOUT_BT_PRESHUFFLED;
    if ((I.layout != GEMM_LAYOUT_BT && !pre) || I.M < 1 || I.M > 64 || kc != GEMM_KERNEL_AUTO ||
        ((I.dtype == GEMM_W4A8_OUT_BF16 || is_mx(I.dtype)) && !pre))
        return nullptr;
    const int mb = I.M <= 16 ? 1 : (I.M <= 32 ? 2 : 4);
    int n = 0;
    const tg::SkinnyVariant *v = tg::skinny_variants(&n);
    auto ok = [&](const tg::SkinnyVariant &x) {
        return x.mblocks == mb && x.elem == elem_of(I.dtype) && x.out == out_of(I.dtype) && x.preshuffled == pre;
    };
    TG_SWEEP_PICK("skinny", v, n, ok)
    return first_of(v, n, ok);
}

// Split K for the workspace entry point.  A problem whose 256 x 256 tiles
// number fewer than the 256 CUs (a few hundred rows against a large B) is
// bound by how fast each CU streams its tile's operands, so K is divided into
// s slices: tiles * s workgroups each write an fp32 partial tile, and a
// reduction kernel sums the slices in order and applies the epilogue.  s is
// the largest power of two with tiles * s <= 256, at least 8 K steps (1 KiB
// of K) per slice and partials no larger than B; `forced` (the caller's
// gemm_plan_options.splits) overrides it, 1 disabling the split.
void plan_split(gemm_plan *p, int kc, int forced)
{
    const gemm_plan_info &I = p->info;
    p->splits = 1;
    p->split_steps = p->k_tiles;
    const int elem = elem_of(I.dtype);
    if (kc == GEMM_KERNEL_GENERIC_128 || kc == GEMM_KERNEL_GENERIC_256)   // the generic kernel does not split
        return;
    if (I.kernel != 0 || I.M == 0 || I.N == 0 || I.K == 0 || is_mx(I.dtype) ||
        (I.layout != GEMM_LAYOUT_BT && I.layout != GEMM_LAYOUT_BT_PRESHUFFLED) ||
        I.N * 4 * 256 >= (int64_t(1) << 31))
        return;
    const int64_t tm = (I.M + 255) / 256, tn = (I.N + 255) / 256;
    const int64_t tiles = tm * tn;
    int s = 1;
    if (forced > 0) {
        s = forced;
    } else if (elem == tg::kFp8 && I.tile_m != 256) {
        // fp8 B is half the bytes, so the fp32 partials weigh twice as much:
        // measured, splitting beats the 128 x 128 tiles' plan only where that
        // plan already takes 256 x 256 tiles (M around 1024 for N = 8192).
        return;
    } else {
        // Also: the partials written and read back (s * M * N * 4 bytes) stay
        // within B's bytes (measured: W4A8 at 256 x 8192 x 8192 takes 0.0516 ms
        // with 4 slices, 0.0539 with 8).
        while (tiles * s * 2 <= 256 && p->k_tiles / (s * 2) >= 8 &&
               (int64_t)(s * 2) * I.M * 4 <= p->kbytes_b)
            s *= 2;
    }
    if (s < 2 || s > 64)
        return;
    const int per = (p->k_tiles + s - 1) / s;
    if ((int64_t)(s - 1) * per >= p->k_tiles)           // every slice non-empty
        return;
    const tg::TiledVariant *v = pick_tiled(I, kc == GEMM_KERNEL_AUTO ? GEMM_KERNEL_TILE256 : kc, true);
    // Only the pipelined and the LDS-staged kernels read the split fields.
    int np = 0, nd = 0;
    const tg::TiledVariant *pv = tg::pipe_variants(&np), *dv = tg::dma_variants(&nd);
    const bool splittable = v && ((v >= pv && v < pv + np) || (v >= dv && v < dv + nd));
    if (!splittable || v->bm != 256 || v->bn != 256 || v->lds_bytes > kLdsLimit)
        return;
    p->split_v = v;
    p->splits = s;
    p->split_steps = per;
    p->split_tiles_m = (int32_t)tm;
    p->split_tiles_n = (int32_t)tn;
    p->split_group_m = (int32_t)(tm < 4 ? tm : 4);
    p->split_grid = (int32_t)(tiles * s);
}

Layout make(std::initializer_list<int64_t> shape, std::initializer_list<int64_t> stride)
{
    Layout L{};
    L.rank = (int32_t)shape.size();
    int i = 0;
    for (int64_t s : shape)
        L.shape[i++] = s;
    i = 0;
    for (int64_t d : stride)
        L.stride[i++] = d;
    return L;
}

Layout view_of(const gemm_plan &p, int view, bool *okv)
{
    const gemm_plan_info &I = p.info;
    const int64_t Kb = p.kbytes_b;
    *okv = true;
    switch (view) {
    case GEMM_VIEW_A:
        if (I.layout == GEMM_LAYOUT_AT || I.layout == GEMM_LAYOUT_AT_BN)
            return make({I.K, I.M * I.elem_bytes}, {I.M * I.elem_bytes, 1});
        return make({I.M, p.kbytes}, {p.kbytes, 1});
    case GEMM_VIEW_B:
        if (I.layout == GEMM_LAYOUT_BN || I.layout == GEMM_LAYOUT_AT_BN)
            return make({I.K, I.N * I.elem_bytes}, {I.N * I.elem_bytes, 1});
        return make({I.N, Kb}, {Kb, 1});
    case GEMM_VIEW_B_SHUF:
        return make({I.N / 16, Kb / 64, 4, 16, 16}, {16 * Kb, 1024, 256, 16, 1});
    case GEMM_VIEW_B_SRC:
        return make({I.N / 16, Kb / 64, 4, 16, 16}, {16 * Kb, 64, 16, Kb, 1});
    case GEMM_VIEW_C:
        return make({I.M, I.N}, {I.N * I.out_bytes, I.out_bytes});
    case GEMM_VIEW_LDS_A:
        return make({I.tile_m, tg::kChunksPerRow, tg::kChunkBytes}, {tg::kTileKBytes, tg::kChunkBytes, 1});
    case GEMM_VIEW_TILE:
        return make({I.tiles_m, I.tiles_n},
                    {(int64_t)I.tile_m * I.N * I.out_bytes, (int64_t)I.tile_n * I.out_bytes});
    default:
        *okv = false;
        return Layout{};
    }
}

// gfx950 check, once per device.
int check_device()
{
    static std::mutex mu;
    static int verdict[64];   // 0 unknown, 1 ok, -1 not gfx950
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(GEMM_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64)
        return fail(GEMM_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> g(mu);
    if (verdict[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(GEMM_ERR_HIP, "hipGetDeviceProperties failed");
        verdict[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    if (verdict[dev] != 1)
        return fail(GEMM_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
    return GEMM_OK;
}

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

const char *gemm_last_error(void) { return g_last_error.c_str(); }

gemm_plan *gemm_plan_create_opt(int64_t M, int64_t N, int64_t K, int dtype, int layout,
                                const gemm_plan_options *opt)
{
    const int kc = opt ? opt->kernel : GEMM_KERNEL_AUTO;
    const int forced_splits = opt ? opt->splits : 0;
    if (kc < GEMM_KERNEL_AUTO || kc > GEMM_KERNEL_PIPE4) {
        fail(GEMM_ERR_INVALID_ARG, "unknown kernel choice %d", kc);
        return nullptr;
    }
    if (forced_splits < 0 || forced_splits > 64) {
        fail(GEMM_ERR_INVALID_ARG, "splits=%d outside 0..64", forced_splits);
        return nullptr;
    }
    if (dtype < GEMM_BF16_OUT_F32 || dtype > GEMM_W4A8_OUT_BF16) {
        fail(GEMM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
        return nullptr;
    }
    if (layout < GEMM_LAYOUT_BT || layout > GEMM_LAYOUT_AT_BN) {
        fail(GEMM_ERR_INVALID_ARG, "unknown layout %d", layout);
        return nullptr;
    }
    const bool b_kn = layout == GEMM_LAYOUT_BN || layout == GEMM_LAYOUT_AT_BN;
    const bool a_km = layout == GEMM_LAYOUT_AT || layout == GEMM_LAYOUT_AT_BN;
    const bool bf16_in = dtype == GEMM_BF16_OUT_F32 || dtype == GEMM_BF16_OUT_BF16;
    if (a_km && !bf16_in && dtype != GEMM_E4M3_OUT_BF16 && dtype != GEMM_I8_OUT_BF16) {
        fail(GEMM_ERR_UNSUPPORTED, "A stored K x M is supported for bf16, fp8 e4m3 and int8 inputs");
        return nullptr;
    }
    if (b_kn && !bf16_in && dtype != GEMM_E4M3_OUT_BF16 && dtype != GEMM_I8_OUT_BF16) {
        fail(GEMM_ERR_UNSUPPORTED, "B stored K x N is supported for bf16, fp8 e4m3 and int8 inputs");
        return nullptr;
    }
    if (M < 0 || N < 0 || K < 0) {
        fail(GEMM_ERR_INVALID_ARG, "negative size (M=%lld N=%lld K=%lld)", (long long)M, (long long)N,
             (long long)K);
        return nullptr;
    }
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) {
        fail(GEMM_ERR_UNSUPPORTED, "size above 2^30");
        return nullptr;
    }
    const int ebits = elem_bits_of(dtype), ob = out_bytes_of(dtype);
    const int64_t kbytes = K * ebits / 8;
    const int64_t kbytes_b = K * b_elem_bits_of(dtype) / 8;
    if (is_mx(dtype) && K % 32 != 0) {
        fail(GEMM_ERR_UNSUPPORTED, "K=%lld must be a multiple of 32 (MX block)", (long long)K);
        return nullptr;
    }
    if (dtype == GEMM_W4A8_OUT_BF16 && K % 128 != 0) {
        fail(GEMM_ERR_UNSUPPORTED, "K=%lld must be a multiple of 128 for W4A8 (64-byte steps of int4 B)",
             (long long)K);
        return nullptr;
    }
    if (is_int(dtype) && K >= (int64_t(1) << 17)) {
        fail(GEMM_ERR_UNSUPPORTED, "K=%lld: integer sums need K < 2^17 to stay inside int32", (long long)K);
        return nullptr;
    }
    if (N % 16 != 0) {
        fail(GEMM_ERR_UNSUPPORTED, "N=%lld must be a multiple of 16", (long long)N);
        return nullptr;
    }
    if (kbytes % 64 != 0) {
        fail(GEMM_ERR_UNSUPPORTED, "K*elem_bytes=%lld must be a multiple of 64 (64-byte K step)",
             (long long)kbytes);
        return nullptr;
    }
    if (kbytes >= kMaxRowBytes) {
        fail(GEMM_ERR_UNSUPPORTED, "K*elem_bytes=%lld must be below 2^23", (long long)kbytes);
        return nullptr;
    }
    if (N * ob * 256 >= (int64_t(1) << 31)) {
        fail(GEMM_ERR_UNSUPPORTED, "N=%lld too large for 32-bit C tile offsets", (long long)N);
        return nullptr;
    }
    if (b_kn && K * N * (ebits / 8) >= (int64_t(1) << 31)) {
        fail(GEMM_ERR_UNSUPPORTED, "B stored K x N must stay below 2^31 bytes (32-bit offsets)");
        return nullptr;
    }
    if (a_km && K * M * (ebits / 8) >= (int64_t(1) << 31)) {
        fail(GEMM_ERR_UNSUPPORTED, "A stored K x M must stay below 2^31 bytes (32-bit offsets)");
        return nullptr;
    }
    if (a_km && (M * (ebits / 8)) % 16 != 0) {
        fail(GEMM_ERR_UNSUPPORTED, "M=%lld must make the K-rows of A (K x M) whole 16-byte pieces", (long long)M);
        return nullptr;
    }
    if (is_mx(dtype)) {
        // The kernels address the block-scale images with 32-bit offsets and
        // use 2^31 as their out-of-range offset.
        const int64_t quads = ((M > N ? M : N) + 63) / 64;
        if (quads * scale_groups(K) * 1024 >= (int64_t(1) << 31)) {
            fail(GEMM_ERR_UNSUPPORTED, "MX block-scale image above 2^31 bytes (32-bit offsets)");
            return nullptr;
        }
    }
    if (M * kbytes >= (int64_t(1) << 32) && M <= 64) {
        fail(GEMM_ERR_UNSUPPORTED, "skinny A above 4 GiB");
        return nullptr;
    }

    gemm_plan *p = new (std::nothrow) gemm_plan();
    if (!p) {
        fail(GEMM_ERR_INVALID_ARG, "out of host memory");
        return nullptr;
    }
    gemm_plan_info &I = p->info;
    I.M = M;
    I.N = N;
    I.K = K;
    I.dtype = dtype;
    I.layout = layout;
    I.elem_bytes = ebits / 8;
    I.elem_bits = ebits;
    I.b_elem_bits = b_elem_bits_of(dtype);
    I.out_bytes = ob;
    p->kbytes = kbytes;
    p->kbytes_b = kbytes_b;
    p->k_tiles = (int32_t)((kbytes + tg::kTileKBytes - 1) / tg::kTileKBytes);
    p->tail_bytes = kbytes % tg::kTileKBytes ? (int32_t)(kbytes % tg::kTileKBytes) : tg::kTileKBytes;
    I.tile_k_bytes = tg::kTileKBytes;
    I.split_k = 1;

    if ((p->skinny = pick_skinny(I, kc)) != nullptr) {
        I.kernel = 1;
        I.tile_m = p->skinny->mblocks * 16;
        I.tile_n = tg::kSkinnyTileN;
        I.threads = 64 * p->skinny->waves;
        I.lds_stages = p->skinny->stages;
        I.lds_bytes = p->skinny->lds_bytes;
        I.tiles_m = 1;
        I.tiles_n = (int32_t)(N / tg::kSkinnyTileN + (N % tg::kSkinnyTileN ? 1 : 0));
        I.group_m = 1;
        I.split_k = p->skinny->waves;
        I.grid = I.tiles_n;
    } else if ((p->tiled = pick_tiled(I, kc)) != nullptr) {
        I.kernel = 0;
        I.tile_m = p->tiled->bm;
        I.tile_n = p->tiled->bn;
        I.threads = 64 * p->tiled->wgm * p->tiled->wgn;
        I.lds_bytes = p->tiled->lds_bytes;
        I.lds_stages = p->tiled->lds_stages;
        I.tiles_m = (int32_t)((M + I.tile_m - 1) / I.tile_m);
        I.tiles_n = (int32_t)((N + I.tile_n - 1) / I.tile_n);
        I.group_m = I.tile_m >= 256 ? 4 : 8;
        if (I.group_m > I.tiles_m)
            I.group_m = I.tiles_m > 0 ? I.tiles_m : 1;
        const int64_t grid = (int64_t)I.tiles_m * I.tiles_n;
        if (grid >= (int64_t(1) << 31)) {
            delete p;
            fail(GEMM_ERR_UNSUPPORTED, "too many tiles");
            return nullptr;
        }
        I.grid = (int32_t)grid;
    } else {
        delete p;
        fail(GEMM_ERR_UNSUPPORTED, "no kernel for this dtype/layout%s", kc ? " and kernel choice" : "");
        return nullptr;
    }
    if (I.lds_bytes > kLdsLimit) {
        delete p;
        fail(GEMM_ERR_UNSUPPORTED, "tile needs %d bytes of LDS (> 160 KiB)", I.lds_bytes);
        return nullptr;
    }
    plan_split(p, kc, forced_splits);
    I.ws_splits = p->splits;
    I.ws_grid = p->splits > 1 ? p->split_grid : I.grid;
    I.scale_form = wide_scales(p) ? 1 : 0;
    ok();
    return p;
}

gemm_plan *gemm_plan_create(int64_t M, int64_t N, int64_t K, int dtype, int layout)
{
    return gemm_plan_create_opt(M, N, K, dtype, layout, nullptr);
}

void gemm_plan_destroy(gemm_plan *plan) { delete plan; }

size_t gemm_preshuffled_b_bytes(const gemm_plan *plan)
{
    if (!plan || plan->info.layout == GEMM_LAYOUT_BN || plan->info.layout == GEMM_LAYOUT_AT_BN)
        return 0;
    return (size_t)plan->info.N * (size_t)plan->kbytes_b;
}

int gemm_plan_query(const gemm_plan *plan, gemm_plan_info *info)
{
    if (!plan || !info)
        return fail(GEMM_ERR_INVALID_ARG, "NULL plan or info");
    *info = plan->info;
    ok();
    return GEMM_OK;
}

int gemm_plan_layout(const gemm_plan *plan, int view, int32_t *rank, int64_t *shape, int64_t *stride)
{
    if (!plan || !rank || !shape || !stride)
        return fail(GEMM_ERR_INVALID_ARG, "NULL argument");
    bool okv = false;
    const Layout L = view_of(*plan, view, &okv);
    if (!okv)
        return fail(GEMM_ERR_INVALID_ARG, "unknown view %d", view);
    *rank = L.rank;
    for (int i = 0; i < GEMM_MAX_RANK; ++i) {
        shape[i] = i < L.rank ? L.shape[i] : 0;
        stride[i] = i < L.rank ? L.stride[i] : 0;
    }
    ok();
    return GEMM_OK;
}

int64_t gemm_layout_crd2idx(int32_t rank, const int64_t *shape, const int64_t *stride, const int64_t *crd)
{
    if (rank < 0 || rank > GEMM_MAX_RANK || (rank && (!shape || !stride || !crd))) {
        fail(GEMM_ERR_INVALID_ARG, "bad layout arguments");
        return -1;
    }
    Layout L{};
    L.rank = rank;
    for (int i = 0; i < rank; ++i) {
        if (crd[i] < 0 || crd[i] >= shape[i]) {
            fail(GEMM_ERR_INVALID_ARG, "coordinate %d = %lld outside [0, %lld)", i, (long long)crd[i],
                 (long long)shape[i]);
            return -1;
        }
        L.shape[i] = shape[i];
        L.stride[i] = stride[i];
    }
    ok();
    return tg::crd2idx(L, crd);
}

int gemm_layout_idx2crd(int32_t rank, const int64_t *shape, const int64_t *stride, int64_t idx, int64_t *crd)
{
    if (rank < 0 || rank > GEMM_MAX_RANK || (rank && (!shape || !stride || !crd)) || idx < 0)
        return fail(GEMM_ERR_INVALID_ARG, "bad layout arguments");
    Layout L{};
    L.rank = rank;
    for (int i = 0; i < rank; ++i) {
        if (shape[i] <= 0 || stride[i] < 0)
            return fail(GEMM_ERR_INVALID_ARG, "mode %d: shape must be > 0, stride >= 0", i);
        L.shape[i] = shape[i];
        L.stride[i] = stride[i];
    }
    tg::idx2crd(L, idx, crd);
    ok();
    return GEMM_OK;
}

int32_t gemm_lds_swizzle(int32_t row, int32_t chunk, int32_t chunks_per_row)
{
    if (row < 0 || chunk < 0 || chunks_per_row != tg::kChunksPerRow || chunk >= chunks_per_row) {
        fail(GEMM_ERR_INVALID_ARG, "swizzle defined for rows of %d chunks", tg::kChunksPerRow);
        return -1;
    }
    ok();
    return tg::swz_chunk(row, chunk);
}

int gemm_tile_of_workgroup(const gemm_plan *plan, int32_t wg, int32_t *tm, int32_t *tn)
{
    if (!plan || !tm || !tn || wg < 0 || wg >= plan->info.grid)
        return fail(GEMM_ERR_INVALID_ARG, "bad workgroup query");
    const gemm_plan_info &I = plan->info;
    if (I.kernel == 1) {
        *tm = 0;
        *tn = wg;
    } else {
        int a = 0, b = 0;
        tg::tile_of_wg(wg, I.grid, I.tiles_m, I.tiles_n, I.group_m, &a, &b);
        *tm = a;
        *tn = b;
    }
    ok();
    return GEMM_OK;
}

int gemm_preshuffle_b(const gemm_plan *plan, const void *B, void *B_shuf, hipStream_t stream)
{
    if (!plan)
        return fail(GEMM_ERR_INVALID_ARG, "NULL plan");
    if (plan->info.layout == GEMM_LAYOUT_BN || plan->info.layout == GEMM_LAYOUT_AT_BN)
        return fail(GEMM_ERR_INVALID_ARG, "the pre-shuffled image is made from B stored N x K");
    const size_t bytes = gemm_preshuffled_b_bytes(plan);
    if (bytes == 0) {
        ok();
        return GEMM_OK;
    }
    if (!B || !B_shuf)
        return fail(GEMM_ERR_INVALID_ARG, "NULL B or B_shuf");
    if (misaligned(B) || misaligned(B_shuf))
        return fail(GEMM_ERR_INVALID_ARG, "B and B_shuf must be 16-byte aligned");
    if (overlap(B, bytes, B_shuf, bytes))
        return fail(GEMM_ERR_INVALID_ARG, "B_shuf overlaps B");
    if (int rc = check_device())
        return rc;
    bool okv = false;
    tg::PreshuffleArgs a{};
    a.B = B;
    a.Bs = B_shuf;
    a.src = view_of(*plan, GEMM_VIEW_B_SRC, &okv);
    a.dst = view_of(*plan, GEMM_VIEW_B_SHUF, &okv);
    a.nblocks = (int32_t)(plan->info.N / 16);
    a.kblocks = (int32_t)(plan->kbytes_b / 64);
    const hipError_t e = tg::launch_preshuffle(a, stream);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "preshuffle launch: %s", hipGetErrorString(e));
    ok();
    return GEMM_OK;
}

}  // extern "C"

namespace {

int run_impl(const gemm_plan *plan, const void *A, const void *B, void *C, const tg::EpiArgs &epi,
             hipStream_t stream, const void *sa_img = nullptr, const void *sb_img = nullptr)
{
    if (!plan)
        return fail(GEMM_ERR_INVALID_ARG, "NULL plan");
    const gemm_plan_info &I = plan->info;
    if (I.M == 0 || I.N == 0) {
        ok();
        return GEMM_OK;
    }
    if (!A && I.K)
        return fail(GEMM_ERR_INVALID_ARG, "NULL A");
    if (!B && I.K)
        return fail(GEMM_ERR_INVALID_ARG, "NULL B");
    if (!C)
        return fail(GEMM_ERR_INVALID_ARG, "NULL C");
    if ((A && misaligned(A)) || (B && misaligned(B)) || misaligned(C))
        return fail(GEMM_ERR_INVALID_ARG, "A, B and C must be 16-byte aligned");
    const size_t cbytes = (size_t)I.M * I.N * I.out_bytes;
    if (overlap(C, cbytes, A, (size_t)I.M * plan->kbytes) || overlap(C, cbytes, B, (size_t)I.N * plan->kbytes_b))
        return fail(GEMM_ERR_INVALID_ARG, "C overlaps A or B");
    if (int rc = check_device())
        return rc;
    hipError_t e;
    if (I.kernel == 1) {
        tg::SkinnyArgs a{};
        a.A = A;
        a.B = B;
        a.C = C;
        a.epi = epi;
        a.M = (int32_t)I.M;
        a.N = (int32_t)I.N;
        a.kbytes = (int32_t)plan->kbytes;
        a.k_tiles = plan->k_tiles;
        a.tail_bytes = plan->tail_bytes;
        a.kbytes_b = (int32_t)plan->kbytes_b;
        a.sa_img = (const uint8_t *)sa_img;
        a.sb_img = (const uint8_t *)sb_img;
        a.s_groups = (int32_t)scale_groups(I.K);
        e = plan->skinny->launch(a, I.grid, stream);
    } else {
        tg::TiledArgs a{};
        a.A = A;
        a.B = B;
        a.C = C;
        a.epi = epi;
        a.M = (int32_t)I.M;
        a.N = (int32_t)I.N;
        a.kbytes = (int32_t)plan->kbytes;
        a.kbytes_b = (int32_t)plan->kbytes_b;
        a.K = (int32_t)I.K;
        a.ldb_bytes = (int32_t)(I.N * I.elem_bytes);
        a.lda_bytes = (int32_t)(I.M * I.elem_bytes);
        a.k_tiles = plan->k_tiles;
        a.tail_bytes = plan->tail_bytes;
        a.grid = I.grid;
        a.tiles_m = I.tiles_m;
        a.tiles_n = I.tiles_n;
        a.group_m = I.group_m;
        a.sa_img = (const uint8_t *)sa_img;
        a.sb_img = (const uint8_t *)sb_img;
        a.s_groups = (int32_t)scale_groups(I.K);
        e = plan->tiled->launch(a, stream);
    }
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    ok();
    return GEMM_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

size_t workspace_bytes(const gemm_plan *plan)
{
    if (!plan || plan->splits < 2)
        return 0;
    return (size_t)plan->splits * (size_t)plan->info.M * (size_t)plan->info.N * 4u;
}

// Split-K run: the slices' fp32 partials into W, then the ordered sum and
// the epilogue into C.  The caller has validated A, B, C and W.
int run_split(const gemm_plan *plan, const void *A, const void *B, void *C, void *W, const tg::EpiArgs &epi,
              hipStream_t stream)
{
    const gemm_plan_info &I = plan->info;
    tg::TiledArgs a{};
    a.A = A;
    a.B = B;
    a.C = W;
    a.epi = tg::EpiArgs{};                 // partials: no scaling, no bias, no activation
    a.epi.act = tg::kActNone;
    a.M = (int32_t)I.M;
    a.N = (int32_t)I.N;
    a.kbytes = (int32_t)plan->kbytes;
    a.kbytes_b = (int32_t)plan->kbytes_b;
    a.K = (int32_t)I.K;
    a.ldb_bytes = (int32_t)(I.N * I.elem_bytes);
    a.lda_bytes = (int32_t)(I.M * I.elem_bytes);
    a.k_tiles = plan->k_tiles;
    a.tail_bytes = plan->tail_bytes;
    a.grid = plan->split_grid;
    a.tiles_m = plan->split_tiles_m;
    a.tiles_n = plan->split_tiles_n;
    a.group_m = plan->split_group_m;
    a.splits = plan->splits;
    a.split_steps = plan->split_steps;
    hipError_t e = plan->split_v->launch(a, stream);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "split-K launch: %s", hipGetErrorString(e));
    tg::SplitReduceArgs r{};
    r.W = (const float *)W;
    r.C = C;
    r.epi = epi;
    r.M = (int32_t)I.M;
    r.N = (int32_t)I.N;
    r.splits = plan->splits;
    r.out = out_of(I.dtype);
    e = tg::launch_split_reduce(r, stream);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "split-K reduction launch: %s", hipGetErrorString(e));
    ok();
    return GEMM_OK;
}

// The epilogue description -> kernel arguments (GEMM_OK or an error).
int epi_from(const gemm_epilogue_args *epi, tg::EpiArgs *e)
{
    *e = tg::EpiArgs{};
    if (!epi)
        return GEMM_OK;
    if (epi->epilogue < GEMM_EPI_NONE || epi->epilogue > GEMM_EPI_BIAS_GELU)
        return fail(GEMM_ERR_INVALID_ARG, "unknown epilogue %d", (int)epi->epilogue);
    if ((epi->scale_a_per_row != 0 && epi->scale_a_per_row != 1) ||
        (epi->scale_b_per_col != 0 && epi->scale_b_per_col != 1))
        return fail(GEMM_ERR_INVALID_ARG, "scale_a_per_row and scale_b_per_col must be 0 or 1");
    const bool wants_bias = epi->epilogue != GEMM_EPI_NONE;
    if (wants_bias && !epi->bias)
        return fail(GEMM_ERR_INVALID_ARG, "the bias epilogues need a bias vector");
    if (!wants_bias && epi->bias)
        return fail(GEMM_ERR_INVALID_ARG, "bias given with GEMM_EPI_NONE");
    if ((epi->scale_a && !aligned(epi->scale_a, 4)) ||
        (epi->scale_b && !aligned(epi->scale_b, epi->scale_b_per_col ? 16 : 4)) ||
        (epi->bias && !aligned(epi->bias, 16)))
        return fail(GEMM_ERR_INVALID_ARG,
                    "scale_a must be 4-byte aligned; per-column scale_b and bias 16-byte aligned");
    e->sa = epi->scale_a;
    e->sb = epi->scale_b;
    e->bias = epi->bias;
    e->sa_rows = epi->scale_a_per_row;
    e->sb_cols = epi->scale_b_per_col;
    static const int kAct[] = {tg::kActNone, tg::kActNone, tg::kActRelu, tg::kActSilu, tg::kActGelu};
    e->act = kAct[epi->epilogue];
    return GEMM_OK;
}

int reject_mx(const gemm_plan *plan)
{
    if (plan && is_mx(plan->info.dtype))
        return fail(GEMM_ERR_INVALID_ARG, "MX plans run through gemm_run_mx (block scales)");
    return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_run(const gemm_plan *plan, const void *A, const void *B, void *C, const float *scale,
             hipStream_t stream)
{
    if (int rc = reject_mx(plan))
        return rc;
    if (scale && !aligned(scale, 4))
        return fail(GEMM_ERR_INVALID_ARG, "scale must be 4-byte aligned");
    tg::EpiArgs e{};
    e.sa = scale;
    e.sb = scale ? scale + 1 : nullptr;
    e.act = tg::kActNone;
    return run_impl(plan, A, B, C, e, stream);
}

int gemm_run_ex(const gemm_plan *plan, const void *A, const void *B, void *C, const gemm_epilogue_args *epi,
                hipStream_t stream)
{
    if (int rc = reject_mx(plan))
        return rc;
    tg::EpiArgs e;
    if (int rc = epi_from(epi, &e))
        return rc;
    return run_impl(plan, A, B, C, e, stream);
}

size_t gemm_workspace_bytes(const gemm_plan *plan) { return workspace_bytes(plan); }

int gemm_run_ws(const gemm_plan *plan, const void *A, const void *B, void *C, const gemm_epilogue_args *epi,
                void *workspace, size_t workspace_bytes_given, hipStream_t stream)
{
    if (int rc = reject_mx(plan))
        return rc;
    tg::EpiArgs e;
    if (int rc = epi_from(epi, &e))
        return rc;
    const size_t need = workspace_bytes(plan);
    if (need == 0 || !workspace || workspace_bytes_given < need)
        return run_impl(plan, A, B, C, e, stream);
    const gemm_plan_info &I = plan->info;
    if (!A || !B || !C)
        return fail(GEMM_ERR_INVALID_ARG, "NULL A, B or C");
    if (misaligned(A) || misaligned(B) || misaligned(C) || misaligned(workspace))
        return fail(GEMM_ERR_INVALID_ARG, "A, B, C and the workspace must be 16-byte aligned");
    const size_t cbytes = (size_t)I.M * I.N * I.out_bytes;
    const size_t abytes = (size_t)I.M * plan->kbytes, bbytes = (size_t)I.N * plan->kbytes_b;
    if (overlap(C, cbytes, A, abytes) || overlap(C, cbytes, B, bbytes))
        return fail(GEMM_ERR_INVALID_ARG, "C overlaps A or B");
    if (overlap(workspace, need, A, abytes) || overlap(workspace, need, B, bbytes) ||
        overlap(workspace, need, C, cbytes))
        return fail(GEMM_ERR_INVALID_ARG, "the workspace overlaps A, B or C");
    if (int rc = check_device())
        return rc;
    return run_split(plan, A, B, C, workspace, e, stream);
}

int gemm_run_ws_noalloc(const gemm_plan *plan, const void *A, const void *B, void *C,
                        const gemm_epilogue_args *epi, hipStream_t stream)
{
    static_assert(GEMM_STATIC_WORKSPACE_BYTES == tg::kStaticWorkspaceBytes, "header and library agree");
    if (int rc = reject_mx(plan))
        return rc;
    tg::EpiArgs e;
    if (int rc = epi_from(epi, &e))
        return rc;
    const size_t need = workspace_bytes(plan);
    if (need == 0)
        return run_impl(plan, A, B, C, e, stream);
    if (need > tg::kStaticWorkspaceBytes)
        return fail(GEMM_ERR_UNSUPPORTED,
                    "the plan's split-K partials need %zu bytes, more than the %zu-byte static workspace "
                    "(gemm_run_ws takes a workspace of any size)",
                    need, tg::kStaticWorkspaceBytes);
    const gemm_plan_info &I = plan->info;
    if (!A || !B || !C)
        return fail(GEMM_ERR_INVALID_ARG, "NULL A, B or C");
    if (misaligned(A) || misaligned(B) || misaligned(C))
        return fail(GEMM_ERR_INVALID_ARG, "A, B and C must be 16-byte aligned");
    const size_t cbytes = (size_t)I.M * I.N * I.out_bytes;
    if (overlap(C, cbytes, A, (size_t)I.M * plan->kbytes) || overlap(C, cbytes, B, (size_t)I.N * plan->kbytes_b))
        return fail(GEMM_ERR_INVALID_ARG, "C overlaps A or B");
    if (int rc = check_device())
        return rc;
    void *ws = nullptr;
    const hipError_t he = tg::static_workspace(&ws);
    if (he != hipSuccess || !ws)
        return fail(GEMM_ERR_HIP, "static workspace address: %s", hipGetErrorString(he));
    return run_split(plan, A, B, C, ws, e, stream);
}

size_t gemm_bscale_image_bytes(const gemm_plan *plan, int operand)
{
    if (!plan || !is_mx(plan->info.dtype) || (operand != 0 && operand != 1))
        return 0;
    const int64_t rows = operand ? plan->info.N : plan->info.M;
    return (size_t)((rows + 63) / 64) * (size_t)scale_groups(plan->info.K) * 1024u;
}

int gemm_preshuffle_bscale(const gemm_plan *plan, int operand, const void *scales, void *image, hipStream_t stream)
{
    if (!plan)
        return fail(GEMM_ERR_INVALID_ARG, "NULL plan");
    if (!is_mx(plan->info.dtype))
        return fail(GEMM_ERR_INVALID_ARG, "block scales belong to MX plans");
    if (operand != 0 && operand != 1)
        return fail(GEMM_ERR_INVALID_ARG, "operand must be 0 (A) or 1 (B)");
    const size_t bytes = gemm_bscale_image_bytes(plan, operand);
    const int64_t rows = operand ? plan->info.N : plan->info.M;
    const size_t src_bytes = (size_t)rows * (size_t)(plan->info.K / 32);
    if (bytes == 0 || src_bytes == 0) {
        ok();
        return GEMM_OK;
    }
    if (!scales || !image)
        return fail(GEMM_ERR_INVALID_ARG, "NULL scales or image");
    if (!aligned(image, 16))
        return fail(GEMM_ERR_INVALID_ARG, "image must be 16-byte aligned");
    if (overlap(scales, src_bytes, image, bytes))
        return fail(GEMM_ERR_INVALID_ARG, "image overlaps the scales");
    if (int rc = check_device())
        return rc;
    tg::BscaleArgs a{};
    a.src = (const uint8_t *)scales;
    a.dst = (uint8_t *)image;
    a.rows = (int32_t)rows;
    a.kblocks = (int32_t)(plan->info.K / 32);
    a.groups = (int32_t)scale_groups(plan->info.K);
    a.quads = (int32_t)((rows + 63) / 64);
    a.form = plan->info.scale_form;
    const hipError_t e = tg::launch_bscale_image(a, stream);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "block-scale image launch: %s", hipGetErrorString(e));
    ok();
    return GEMM_OK;
}

int gemm_run_mx(const gemm_plan *plan, const void *A, const void *A_bscale, const void *B, const void *B_bscale,
                void *C, const gemm_epilogue_args *epi, hipStream_t stream)
{
    if (!plan)
        return fail(GEMM_ERR_INVALID_ARG, "NULL plan");
    if (!is_mx(plan->info.dtype))
        return fail(GEMM_ERR_INVALID_ARG, "gemm_run_mx needs an MX plan");
    if (plan->info.M && plan->info.N && plan->info.K) {
        if (!A_bscale || !B_bscale)
            return fail(GEMM_ERR_INVALID_ARG, "NULL block-scale image");
        if (!aligned(A_bscale, 16) || !aligned(B_bscale, 16))
            return fail(GEMM_ERR_INVALID_ARG, "block-scale images must be 16-byte aligned");
    }
    tg::EpiArgs e;
    if (int rc = epi_from(epi, &e))
        return rc;
    return run_impl(plan, A, B, C, e, stream, A_bscale, B_bscale);
}

}  // extern "C"
