// Device helpers shared by the gfx950 kernels: bit formats, nibble unpacking
// and the few CDNA4 instructions the kernels are built around.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------ buffer loads
// Raw buffer loads: an SGPR resource (base, size) plus a 32-bit per-lane byte
// offset and a wave-uniform SGPR byte offset.  This keeps 64-bit address
// arithmetic off the VALU, and a lane offset at or past ``bytes`` reads 0
// instead of faulting.  Word 3 of the descriptor is the raw 32-bit data
// format of the gfx9 family.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kAuxNontemporal = 2;  // stream past the caches: read once

// The base, size and SGPR offset of a buffer access are wave-uniform by
// contract; readfirstlane states it to the compiler (free when the value is
// already scalar), so descriptors never need a per-lane waterfall loop.
__device__ __forceinline__ uint32_t sgpr(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t u = ((uint64_t)sgpr((uint32_t)(b >> 32)) << 32) | sgpr((uint32_t)b);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0, (int)sgpr(bytes), kBufferWord3);
}

template <int kAux = 0>
__device__ __forceinline__ u32x4_t buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)sgpr(soff), kAux));
}

__device__ __forceinline__ uint16_t buf_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)sgpr(soff), 0);
}

// Device-coherent access (cache policy sc1): loads miss in an XCD's
// non-coherent L2 lines and stores write through, so data exchanged between
// workgroups on different XCDs needs no L2 write-back or invalidate.
constexpr int kAuxDeviceCoherent = 16;

__device__ __forceinline__ u32x4_t buf_load_b128_coherent(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t,
                              __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)sgpr(soff), kAuxDeviceCoherent));
}

__device__ __forceinline__ void buf_store_u16_coherent(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)voff, (int)sgpr(soff), kAuxDeviceCoherent);
}

// Relaxed device-scope flag access (vector loads/stores with sc1; no fences).
__device__ __forceinline__ unsigned flag_load(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ formats
__device__ __forceinline__ float f16_to_f32(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// c + a.lo * b.lo + a.hi * b.hi with bf16 pairs and an FP32 accumulator (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ------------------------------------------------------------------- INT4
// Packed INT4: bits 4j..4j+3 of a word hold the code of k = 8p + j.

// Biased bfloat16 pairs for the GEMV's dot2 path.  bf16 0x4300 is 128.0 and
// its unit in the last place is 1, so 0x4300 | q is exactly 128 + q.  Pair j
// (j = 0..3) holds (128 + q_j, 128 + q_{j+4}): nibbles j and j+4 sit 16 bits
// apart, so one mask extracts both.
//
// ``bias`` must be 0x43004300 held in a VGPR (see vgpr_const): gfx9 VOP3
// instructions take no literal operand, and with the mask in an SGPR and the
// bias in a VGPR each pair is one v_bitop3_b32 / v_and_or_b32 after the shift.
__device__ __forceinline__ void int4_word_biased_pairs(uint32_t w, uint32_t bias, uint32_t out[4]) {
    constexpr uint32_t kMask = 0x000F000Fu;
    out[0] = (w & kMask) | bias;
    out[1] = ((w >> 4) & kMask) | bias;
    out[2] = ((w >> 8) & kMask) | bias;
    out[3] = ((w >> 12) & kMask) | bias;
}

constexpr uint32_t kInt4BiasPair = 0x43004300u;  // bf16 pair (128.0, 128.0)

// A constant the compiler must keep in a VGPR and cannot fold into literals.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// x pairs matching int4_word_biased_pairs: from the eight bf16 x[8p .. 8p+7]
// held as four words (x0,x1), (x2,x3), (x4,x5), (x6,x7), build
// (x_j, x_{j+4}) for j = 0..3.
// Each output is one byte select (v_perm_b32: selector bytes 0-3 pick from
// the second operand, 4-7 from the first).
__device__ __forceinline__ void x_pairs_for_biased(const uint32_t xw[4], uint32_t out[4]) {
    out[0] = __builtin_amdgcn_perm(xw[2], xw[0], 0x05040100u);  // low halves
    out[1] = __builtin_amdgcn_perm(xw[2], xw[0], 0x07060302u);  // high halves
    out[2] = __builtin_amdgcn_perm(xw[3], xw[1], 0x05040100u);
    out[3] = __builtin_amdgcn_perm(xw[3], xw[1], 0x07060302u);
}

// FP32 dequantisation of one word, as the prefill GEMM computes it:
// out[j] = fma(q_j, s, nzs) with nzs = -z * s.  Exact: q s and z s have at
// most 15 significant bits, and their difference (q - z) s is representable,
// so the FMA's single rounding changes nothing.
__device__ __forceinline__ void int4_word_dequant_f32(uint32_t w, float s, float nzs, float out[8]) {
    uint32_t lo = w & 0x0F0F0F0Fu;         // codes of k = 8p + 0, 2, 4, 6 in bytes 0..3
    uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes of k = 8p + 1, 3, 5, 7
    // Opaque to the optimiser, so each byte converts with one v_cvt_f32_ubyte{0..3}
    // instead of a bit-field extract and a conversion.
    asm volatile("" : "+v"(lo), "+v"(hi));
    out[0] = fmaf((float)(lo & 0xFFu), s, nzs);
    out[1] = fmaf((float)(hi & 0xFFu), s, nzs);
    out[2] = fmaf((float)((lo >> 8) & 0xFFu), s, nzs);
    out[3] = fmaf((float)((hi >> 8) & 0xFFu), s, nzs);
    out[4] = fmaf((float)((lo >> 16) & 0xFFu), s, nzs);
    out[5] = fmaf((float)((hi >> 16) & 0xFFu), s, nzs);
    out[6] = fmaf((float)(lo >> 24), s, nzs);
    out[7] = fmaf((float)(hi >> 24), s, nzs);
}

// The prefill GEMM's matrix-core operand for one word: the eight dequantised
// weights of int4_word_dequant_f32, in k order, each rounded once to BF16
// (v_cvt_pk_bf16_f32, round to nearest even), two per 32-bit lane word.
__device__ __forceinline__ u32x4_t int4_word_dequant_bf16(uint32_t w, float s, float nzs) {
    float f[8];
    int4_word_dequant_f32(w, s, nzs, f);
    u32x4_t r;
    r.x = pack_bf16x2(f[0], f[1]);
    r.y = pack_bf16x2(f[2], f[3]);
    r.z = pack_bf16x2(f[4], f[5]);
    r.w = pack_bf16x2(f[6], f[7]);
    return r;
}

// ------------------------------------------------------------------- FP4
// One byte holds two E2M1 codes: low nibble = even k, high nibble = odd k.
// v_cvt_scalef32_pk_bf16_fp4 converts the two codes of byte ``sel`` to a bf16
// pair (even k in the low half).  With a scale of 1.0 the result is the exact
// E2M1 value; the real BF16 scale is applied afterwards in FP32.
template <int kSel>
__device__ __forceinline__ uint32_t fp4_byte_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, kSel));
}

__device__ __forceinline__ void fp4_word_pairs(uint32_t w, uint32_t out[4]) {
    out[0] = fp4_byte_to_bf16x2<0>(w);
    out[1] = fp4_byte_to_bf16x2<1>(w);
    out[2] = fp4_byte_to_bf16x2<2>(w);
    out[3] = fp4_byte_to_bf16x2<3>(w);
}

// -------------------------------------------------------------- reductions
// Cross-lane exchanges without LDS: DPP inside a row of 16 lanes, the gfx950
// row swaps (v_permlane16_swap, v_permlane32_swap) across rows.

// Value of lane l ^ m for an exchange across bit kOff (kOff = 1, 2, 4, 8) of
// a 16-lane row: quad_perm [1,0,3,2] (m = 1), quad_perm [2,3,0,1] (m = 2),
// row_half_mirror (m = 7) and row_ror:8 (m = 8).  Each partner differs from l
// in bit kOff and above it in nothing, which is all a butterfly over bits
// kOff, kOff / 2, ..., 1 needs: the masks stay independent, so every lane of
// the row is summed exactly once.
template <int kOff>
__device__ __forceinline__ float dpp_partner(float v) {
    constexpr int kCtrl = kOff == 1 ? 0xB1 : kOff == 2 ? 0x4E : kOff == 4 ? 0x141 : 0x128;
    static_assert(kOff == 1 || kOff == 2 || kOff == 4 || kOff == 8, "DPP exchanges stay inside a row of 16");
    const int b = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, kCtrl, 0xF, 0xF, false));
}

// For an exchange across lane bit kOff = 16 or 32: with a the value of lanes
// whose bit is clear and b of lanes whose bit is set, returns a's sum over
// the lane pair in the lanes with the bit clear and b's in the others.  The
// swap instruction exchanges b's clear-bit rows with a's set-bit rows, so
// adding its two outputs gives each lane its own pair sum.
template <int kOff>
__device__ __forceinline__ float swap_pair_sum(float a, float b) {
    static_assert(kOff == 16 || kOff == 32, "row swaps cross bit 4 or 5");
    const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
    uint32_t r0, r1;
    if constexpr (kOff == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
        r0 = r[0];
        r1 = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
        r0 = r[0];
        r1 = r[1];
    }
    // Scalars first: a bit_cast applied directly to the vector element r[1]
    // reads element 0 with this compiler.
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// Sum of v over the lane pair across bit kOff, in every lane.
template <int kOff>
__device__ __forceinline__ float pair_sum(float v) {
    if constexpr (kOff >= 16) {
        return swap_pair_sum<kOff>(v, v);
    } else {
        return v + dpp_partner<kOff>(v);
    }
}

// Reduce R per-lane values (one per row) across the 64 lanes of a wave.
// Each step halves the rows a lane carries: across lane bit kOff, lanes with
// the bit clear keep rows [0, R/2) and the others rows [R/2, R), each adding
// its partner's value of the rows it keeps.  R rows cost R - 1 + log2(64 / R)
// exchanges instead of 6 R.  On return every lane holds the total of row
// lane / (64 / R).  The summation order is fixed, so results are reproducible.
template <int R, int kOff>
struct RowReduce {
    static __device__ __forceinline__ void run(float* v, int lane) {
        if constexpr (R > 1) {
            constexpr int H = R / 2;
            const bool upper = (lane & kOff) != 0;
#pragma unroll
            for (int i = 0; i < H; ++i) {
                if constexpr (kOff >= 16) {
                    v[i] = swap_pair_sum<kOff>(v[i], v[i + H]);
                } else {
                    const float lo = pair_sum<kOff>(v[i]), hi = pair_sum<kOff>(v[i + H]);
                    v[i] = upper ? hi : lo;
                }
            }
            RowReduce<H, kOff / 2>::run(v, lane);
        } else if constexpr (kOff >= 1) {
            v[0] = pair_sum<kOff>(v[0]);
            RowReduce<1, kOff / 2>::run(v, lane);
        }
    }
};

template <int R>
__device__ __forceinline__ float reduce_rows(float (&v)[R], int lane) {
    static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "R must be a power of two");
    RowReduce<R, 32>::run(v, lane);
    return v[0];
}

}  // namespace w4
