// Device-side building blocks for gfx950 (CDNA4): buffer resources, the MFMA
// atoms, and the fp32 -> bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "kernels.hpp"
#include "layout.hpp"

namespace tg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) void lds_void;

// Offset that lies past every buffer's record count (the planner keeps
// record counts below 2^31): a load from it returns zero and a store to it is
// dropped (buffer range checking).
constexpr uint32_t kOobOffset = 0x80000000u;

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4],
// lgkmcnt [11:8]); a field at its maximum means "do not wait on it".
constexpr int kWaitVmcnt0 = 0x0F70;

// Raw buffer resource over [base, base + bytes).  Word 3 = 0x00020000 is the
// gfx9-family default (32-bit data format, no swizzle, no stride).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

__device__ inline u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}

__device__ inline uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Compiler-only memory fence: keeps the loads issued before it ahead of the
// memory operations after it (no instruction, no wait), so a software
// pipeline's loads stay where it issues them instead of sinking towards
// their first use.
__device__ inline void issue_fence() { asm volatile("" ::: "memory"); }

// Branch-free choice of a buffer offset: `off` when `keep`, else an offset
// past the record count (which the planner keeps below 2^31).
__device__ inline uint32_t keep_or_oob(bool keep, uint32_t off)
{
    const uint32_t m = 0u - (uint32_t)keep;           // all ones when kept
    return (off & m) | (kOobOffset & ~m);
}

__device__ inline void buf_store16(__amdgpu_buffer_rsrc_t r, u32x4 v, uint32_t voff)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}

__device__ inline void buf_store8(__amdgpu_buffer_rsrc_t r, u32x2 v, uint32_t voff)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}

// 16 bytes per lane straight from global memory into LDS.  The destination
// of lane l is lds_wave_base + 16 * l: a wave writes 1 KiB contiguously, so
// any swizzle is applied on the global side (the lane picks its source).
__device__ inline void buf_load16_to_lds(__amdgpu_buffer_rsrc_t r, void *lds_wave_base,
                                         uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_wave_base, 16, voff, soff, 0, 0);
}

__device__ inline u32x4 lds_load16(const void *p) { return *(const u32x4 *)p; }

// ---------------------------------------------------------------------------
// MFMA atoms.  Both compute a 16 x 16 fp32 tile D += X * Y^T over a K slice
// of 64 bytes (bf16) or 128 bytes (fp8).  Lane l supplies row l % 16 of X and
// of Y and the K slots (l / 16) of the slice; the result lane l holds
// D[4 * (l / 16) + v][l % 16], v = 0..3.  X and Y use the same lane/K
// assignment, so any consistent placement of the K elements into the slots
// gives the same dot products.
// ---------------------------------------------------------------------------
__device__ inline f32x4 mfma_bf16(u32x4 x, u32x4 y, f32x4 acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
}

// fp8 e4m3 (format code 0 for both operands), unit E8M0 block scales (127).
__device__ inline f32x4 mfma_fp8x8(i32x8 x, i32x8 y, f32x4 acc)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, 0, 0, 0, 127, 0, 127);
}

// The 16-byte halves of a 32-byte operand.
__device__ inline u32x4 lo16(i32x8 v) { return u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]}; }
__device__ inline u32x4 hi16(i32x8 v) { return u32x4{(uint32_t)v[4], (uint32_t)v[5], (uint32_t)v[6], (uint32_t)v[7]}; }

// Two 16-byte halves as one 32-byte fp8 operand.
__device__ inline i32x8 join32(u32x4 lo, u32x4 hi)
{
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ inline f32x4 mfma_fp8(u32x4 x_lo, u32x4 x_hi, u32x4 y_lo, u32x4 y_hi, f32x4 acc)
{
    i32x8 x, y;
    x.s0 = x_lo.x; x.s1 = x_lo.y; x.s2 = x_lo.z; x.s3 = x_lo.w;
    x.s4 = x_hi.x; x.s5 = x_hi.y; x.s6 = x_hi.z; x.s7 = x_hi.w;
    y.s0 = y_lo.x; y.s1 = y_lo.y; y.s2 = y_lo.z; y.s3 = y_lo.w;
    y.s4 = y_hi.x; y.s5 = y_hi.y; y.s6 = y_hi.z; y.s7 = y_hi.w;
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, 0, 0, 0, 127, 0, 127);
}

// The same two atoms with the accumulator pinned to AGPRs (inline assembly,
// "+a"), for kernels whose accumulators fill the AGPR file (256 per lane): the
// compiler then keeps every accumulator in place across the main loop instead
// of copying between register files.  It does not know these are MFMAs and
// inserts none of the wait states around them, so the kernels using them keep
// two rules: (1) an MFMA that depends on an earlier one reads that MFMA's
// result only as its accumulator, with SrcC and vDst the very same registers
// (the case the matrix unit resolves by itself; the 8-wave 32x32x64 MX kernel
// updates an accumulator every 8 MFMAs, the others every 32 or more); (2) no
// other instruction reads or writes an accumulator until mfma_drain_acc() has
// waited out more cycles than any of these MFMAs takes to finish (its passes
// plus two) and pinned the reads behind that wait.
// v_mfma_f32_16x16x128_f8f6f4 with its default format fields is e4m3 x e4m3,
// the unscaled form of mfma_fp8x8 above.
__device__ inline void mfma_bf16_a(f32x4 &acc, u32x4 x, u32x4 y)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
}

__device__ inline void mfma_fp8x8_a(f32x4 &acc, i32x8 x, i32x8 y)
{
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
}

// MX block-scaled MFMA with the accumulator pinned to AGPRs:
// D += (X * 2^(sx - 127)) * (Y * 2^(sy - 127))^T, sx and sy byte BYTE of the
// lane's scale registers (each lane's scale covers its 32 K elements).
// mx8: e4m3 operands (8 VGPRs); mx4: e2m1 operands (4 VGPRs; format fields 4).
#define TG_MX_ASM(LO, HI, TAIL)                                                                 \
    "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" #LO "," #LO ",0] "     \
    "op_sel_hi:[" #HI "," #HI ",0]" TAIL
template <int BYTE>
__device__ inline void mfma_mx8_a(f32x4 &acc, i32x8 x, i32x8 y, uint32_t sx, uint32_t sy)
{
    static_assert(BYTE >= 0 && BYTE < 4, "scale byte");
    if constexpr (BYTE == 0)
        asm volatile(TG_MX_ASM(0, 0, "") : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else if constexpr (BYTE == 1)
        asm volatile(TG_MX_ASM(1, 0, "") : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else if constexpr (BYTE == 2)
        asm volatile(TG_MX_ASM(0, 1, "") : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else
        asm volatile(TG_MX_ASM(1, 1, "") : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
}
template <int BYTE>
__device__ inline void mfma_mx4_a(f32x4 &acc, u32x4 x, u32x4 y, uint32_t sx, uint32_t sy)
{
    static_assert(BYTE >= 0 && BYTE < 4, "scale byte");
    if constexpr (BYTE == 0)
        asm volatile(TG_MX_ASM(0, 0, " cbsz:4 blgp:4") : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else if constexpr (BYTE == 1)
        asm volatile(TG_MX_ASM(1, 0, " cbsz:4 blgp:4") : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else if constexpr (BYTE == 2)
        asm volatile(TG_MX_ASM(0, 1, " cbsz:4 blgp:4") : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else
        asm volatile(TG_MX_ASM(1, 1, " cbsz:4 blgp:4") : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
}
#undef TG_MX_ASM

// The 32x32x64 form for e2m1 operands (4 VGPRs each), accumulator in AGPRs:
// D[32 x 32] += (X * 2^(sx - 127)) * (Y * 2^(sy - 127))^T.  Lane l feeds row
// l % 32 of its operand with elements 32 (l / 32) .. +31 of the 64-element
// slice (16 bytes), and its scale byte covers those 32 elements.  Lane l
// receives D[8 u + 4 (l / 32) + j][l % 32] in accumulator element 4 u + j.
#define TG_MX32_ASM(LO, HI)                                                                     \
    "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" #LO "," #LO ",0] "     \
    "op_sel_hi:[" #HI "," #HI ",0] cbsz:4 blgp:4"
template <int BYTE>
__device__ inline void mfma_mx4w_a(f32x16 &acc, u32x4 x, u32x4 y, uint32_t sx, uint32_t sy)
{
    static_assert(BYTE >= 0 && BYTE < 4, "scale byte");
    if constexpr (BYTE == 0)
        asm volatile(TG_MX32_ASM(0, 0) : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else if constexpr (BYTE == 1)
        asm volatile(TG_MX32_ASM(1, 0) : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else if constexpr (BYTE == 2)
        asm volatile(TG_MX32_ASM(0, 1) : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else
        asm volatile(TG_MX32_ASM(1, 1) : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
}
#undef TG_MX32_ASM
// The same for e4m3 operands (8 VGPRs each): lane l feeds row l % 32 with K
// bytes 16 (l / 32) .. +15 and 32 + 16 (l / 32) .. +15 of the 64-byte slice,
// while its scale byte covers K block l / 32 (elements 32 (l / 32) .. +31).
#define TG_MX32F8_ASM(LO, HI)                                                                   \
    "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" #LO "," #LO ",0] "     \
    "op_sel_hi:[" #HI "," #HI ",0]"
template <int BYTE>
__device__ inline void mfma_mx8w_a(f32x16 &acc, i32x8 x, i32x8 y, uint32_t sx, uint32_t sy)
{
    static_assert(BYTE >= 0 && BYTE < 4, "scale byte");
    if constexpr (BYTE == 0)
        asm volatile(TG_MX32F8_ASM(0, 0) : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else if constexpr (BYTE == 1)
        asm volatile(TG_MX32F8_ASM(1, 0) : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else if constexpr (BYTE == 2)
        asm volatile(TG_MX32F8_ASM(0, 1) : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
    else
        asm volatile(TG_MX32F8_ASM(1, 1) : "+a"(acc) : "v"(x), "v"(y), "v"(sx), "v"(sy));
}
#undef TG_MX32F8_ASM

// int8 atom: D += X * Y^T over 64 int8 values per row (16 bytes per lane, the
// same lane / K slot assignment as the bf16 atom), int32 sums.  The
// accumulator travels as f32x4 storage holding the int32 bits, so the
// kernels keep one accumulator type; the epilogue converts.
__device__ inline f32x4 mfma_i8(u32x4 x, u32x4 y, f32x4 acc)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, x),
                                                                           __builtin_bit_cast(i32x4, y),
                                                                           __builtin_bit_cast(i32x4, acc), 0, 0, 0));
}

__device__ inline void mfma_i8_a(f32x4 &acc, u32x4 x, u32x4 y)
{
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
}

// Eight packed int4 values (one word: element 2t in the low nibble of byte
// t, two's complement) -> eight int8 bytes in element order, each holding 16
// times its value (the nibble moved to the high half of its byte, where the
// int8 sign bit is the int4 sign bit).  Sums of such bytes are 16 times the
// int4 sums, exactly; the caller divides by 16.
__device__ inline u32x2 int4x8_to_i8x16(uint32_t w)
{
    const uint32_t ev = (w << 4) & 0xF0F0F0F0u;    // elements 0, 2, 4, 6 in bytes 0..3
    const uint32_t od = w & 0xF0F0F0F0u;           // elements 1, 3, 5, 7
    // v_perm_b32 byte select over {od, ev}: selectors 0-3 pick bytes of ev,
    // 4-7 bytes of od.  lo = [ev0, od0, ev1, od1], hi = [ev2, od2, ev3, od3].
    return u32x2{__builtin_amdgcn_perm(od, ev, 0x05010400u), __builtin_amdgcn_perm(od, ev, 0x07030602u)};
}

// Half h (elements 16 h .. 16 h + 15) of 32 packed int4 values, as one int8
// atom operand.
__device__ inline u32x4 int4x32_half_to_i8(u32x4 w, int h)
{
    const u32x2 a = int4x8_to_i8x16(h ? w.z : w.x);
    const u32x2 b = int4x8_to_i8x16(h ? w.w : w.y);
    return u32x4{a.x, a.y, b.x, b.y};
}

// The int32 sums held in an accumulator's bits -> fp32 (nearest even), times
// `unit` (a power of two, so exact).
__device__ inline f32x4 int_acc_to_f32(f32x4 acc, float unit)
{
    const i32x4 v = __builtin_bit_cast(i32x4, acc);
    return f32x4{(float)v.x * unit, (float)v.y * unit, (float)v.z * unit, (float)v.w * unit};
}

// 64 wait states: longer than any MFMA's result latency.
__device__ inline void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory"); }

// The drain for accumulators written by the inline-assembly MFMAs above:
// wait out the MFMA latency, then pass every accumulator through an empty
// statement that claims to modify it.  The drain alone orders nothing: it
// has no register operands, so the compiler may move the epilogue's AGPR
// reads above it, right behind the MFMA that is still writing them.
template <int FM, int FN>
__device__ inline void mfma_drain_acc(f32x4 (&acc)[FM][FN])
{
    mfma_drain();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            asm volatile("" : "+a"(acc[i][j]));
}

template <int FM, int FN>
__device__ inline void mfma_drain_acc(f32x16 (&acc)[FM][FN])
{
    mfma_drain();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            asm volatile("" : "+a"(acc[i][j]));
}

// Two fp32 -> two bf16 (round to nearest even), packed low-first.
__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int N>
using ic_t = std::integral_constant<int, N>;

// ---------------------------------------------------------------------------
// Fused epilogue: z = (acc * s_a[row]) * s_b[col] (+ bias[col]), then the
// activation, in fp32.  The vectors are read through range-checked buffer
// resources, so rows past M (whose stores are dropped anyway) read zeros
// instead of memory past the caller's vectors.
// ---------------------------------------------------------------------------
struct EpiView {
    __amdgpu_buffer_rsrc_t ra, rb, rz;
    uint32_t sa_step, sb_step;   // bytes per row / column; 0 broadcasts element 0
    bool has_a, has_b, has_bias;
    int act;
};

__device__ inline EpiView epi_view(const EpiArgs &e, int M, int N)
{
    EpiView v;
    v.has_a = e.sa != nullptr;
    v.has_b = e.sb != nullptr;
    v.has_bias = e.bias != nullptr;
    v.sa_step = e.sa_rows ? 4u : 0u;
    v.sb_step = e.sb_cols ? 4u : 0u;
    v.ra = make_rsrc(e.sa, e.sa_rows ? (uint32_t)M * 4u : 4u);
    v.rb = make_rsrc(e.sb, e.sb_cols ? (uint32_t)N * 4u : 4u);
    v.rz = make_rsrc(e.bias, (uint32_t)N * 4u);
    v.act = e.act;
    return v;
}

__device__ inline float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// s_a of one row (row counted in the whole C).
__device__ inline float epi_row_scale(const EpiView &v, int row)
{
    return v.has_a ? as_f32(__builtin_amdgcn_raw_buffer_load_b32(v.ra, (uint32_t)row * v.sa_step, 0, 0)) : 1.f;
}

// s_b and bias of the 4 columns col .. col+3 (col % 4 == 0; the vectors are
// 16-byte aligned).
__device__ inline f32x4 epi_col_scale4(const EpiView &v, int col)
{
    if (!v.has_b)
        return f32x4{1.f, 1.f, 1.f, 1.f};
    if (v.sb_step == 0) {
        const float s = as_f32(__builtin_amdgcn_raw_buffer_load_b32(v.rb, 0u, 0, 0));
        return f32x4{s, s, s, s};
    }
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(v.rb, (uint32_t)col * 4u, 0, 0));
}

__device__ inline f32x4 epi_bias4(const EpiView &v, int col)
{
    if (!v.has_bias)
        return f32x4{0.f, 0.f, 0.f, 0.f};
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(v.rz, (uint32_t)col * 4u, 0, 0));
}

// The same for the 2 columns col, col+1 (col even).
__device__ inline void epi_col2(const EpiView &v, int col, float *sb, float *bz)
{
    sb[0] = sb[1] = 1.f;
    bz[0] = bz[1] = 0.f;
    if (v.has_b) {
        if (v.sb_step == 0) {
            sb[0] = sb[1] = as_f32(__builtin_amdgcn_raw_buffer_load_b32(v.rb, 0u, 0, 0));
        } else {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(v.rb, (uint32_t)col * 4u, 0, 0);
            sb[0] = as_f32(t.x);
            sb[1] = as_f32(t.y);
        }
    }
    if (v.has_bias) {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(v.rz, (uint32_t)col * 4u, 0, 0);
        bz[0] = as_f32(t.x);
        bz[1] = as_f32(t.y);
    }
}

// ReLU max(z, 0) with +0 for every z <= 0; SiLU z / (1 + e^-z); GELU by its
// definition z * Phi(z) = z / 2 * (1 + erf(z / sqrt 2)).
__device__ inline float epi_act(float z, int act)
{
    if (act == kActRelu)
        return z > 0.f ? z : 0.f;
    if (act == kActSilu)
        return z / (1.f + expf(-z));
    if (act == kActGelu)
        return 0.5f * z * (1.f + erff(z * 0.70710678118654752440f));
    return z;
}

__device__ inline float epi_apply1(const EpiView &v, float acc, float sa, float sb, float bz)
{
    float z = (acc * sa) * sb;
    if (v.has_bias)
        z = z + bz;
    return epi_act(z, v.act);
}

__device__ inline f32x4 epi_apply4(const EpiView &v, f32x4 acc, float sa, f32x4 sb, f32x4 bz)
{
    return f32x4{epi_apply1(v, acc.x, sa, sb.x, bz.x), epi_apply1(v, acc.y, sa, sb.y, bz.y),
                 epi_apply1(v, acc.z, sa, sb.z, bz.z), epi_apply1(v, acc.w, sa, sb.w, bz.w)};
}

// ---------------------------------------------------------------------------
// B stored K x N (bf16): K-rows of a tile in LDS and the gfx950 transpose read.
// ---------------------------------------------------------------------------
// XOR applied to the 16-byte chunk index of K-row k of a K x N B tile: the 4
// rows one 16-lane block reads at once (k0 .. k0+3, k0 % 4 == 0) get chunk
// pairs {c, c+1} ^ 2a, disjoint, and rows 8 apart (the next block) differ in
// bit 3 as well.  A bijection on every aligned group of 16 chunks.
__device__ inline int bkn_swz(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 64-bit LDS transpose read of 16-bit elements (ds_read_b64_tr_b16).  Within
// each 16-lane block, lane i receives element i % 4 of the 64 bits addressed
// by lane 4 e + i / 4, e = 0..3 (established with an in-bounds probe).  So if
// lane 4 a + b of a block points at K-row k0 + a, columns c0 + 4 b .. + 3,
// lane i of the block ends up with K-rows k0 .. k0 + 3 of column c0 + i.
__device__ inline u32x2 lds_read_tr16(const uint8_t *p)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)(__attribute__((address_space(3))) uint8_t *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// 64-bit LDS transpose read of 8-bit elements (ds_read_b64_tr_b8).  Within
// each 16-lane block, lane i receives, as its byte e (e = 0..7), byte i % 8 of
// the 64 bits addressed by lane 2 e + i / 8 (established with an in-bounds
// probe).  So if lane 2 e + b of a block points at K-row k0 + e, columns
// c0 + 8 b .. + 7, lane i ends up with K-rows k0 .. k0 + 7 of column c0 + i.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;
__device__ inline u32x2 lds_read_tr8(const uint8_t *p)
{
    const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2 *)(__attribute__((address_space(3))) uint8_t *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Chunk swizzle of the K-rows of an 8-bit K x N tile (rows of 256 bytes, one
// full 64-bank line each): chunk c of K-row k sits at c ^ (k & 7), so the 8
// rows one transpose read takes from a 16-lane block hit 8 different chunks.
__device__ inline int bkn8_swz(int k) { return k & 7; }

__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Split K (TiledArgs::splits): this workgroup's place in the tile raster,
// its K steps [kt0, kt0 + nk) with the valid bytes of the last one, and its
// output (C, or its fp32 partial in the workspace).
struct SplitK {
    int wg, grid;
    int kt0, nk;
    uint32_t tail;
    void *C;
};
__device__ inline SplitK split_k_of(const TiledArgs &p)
{
    SplitK s{(int)blockIdx.x, p.grid, 0, p.k_tiles, (uint32_t)p.tail_bytes, p.C};
    if (p.splits > 1) {
        const int tiles = p.grid / p.splits;
        const int sp = (int)blockIdx.x / tiles;
        s.wg = (int)blockIdx.x - sp * tiles;
        s.grid = tiles;
        s.kt0 = sp * p.split_steps;
        s.nk = min(p.split_steps, p.k_tiles - s.kt0);
        if (s.kt0 + s.nk < p.k_tiles)
            s.tail = kTileKBytes;
        s.C = (uint8_t *)p.C + (size_t)sp * (size_t)p.M * (size_t)p.N * 4u;
    }
    return s;
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), unrolled,
// so that register arrays indexed by the constant stay in registers.
template <typename F, int... I>
__device__ inline void static_for_seq(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F &&f)
{
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}
__device__ inline int lane_id() { return threadIdx.x & 63; }

}  // namespace tg
