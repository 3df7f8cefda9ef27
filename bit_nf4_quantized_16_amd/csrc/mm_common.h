// Device helpers shared by the matmul kernels: MFMA operand types, the
// per-block constant of a quantized weight, and the expansion of NF4 codes to
// bf16 (w' = bf16(fl32(T[c] * a')), the value nf4_dequantize produces).
#pragma once

#include "common.h"
#include "internal.h"

namespace qlnf4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

static __constant__ float c_nf4_mm[16] = {
    kNF4Host[0], kNF4Host[1], kNF4Host[2],  kNF4Host[3],  kNF4Host[4],  kNF4Host[5],  kNF4Host[6],  kNF4Host[7],
    kNF4Host[8], kNF4Host[9], kNF4Host[10], kNF4Host[11], kNF4Host[12], kNF4Host[13], kNF4Host[14], kNF4Host[15],
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Raw per-block constant: the E4M3 code and its group scale (double
// quantization) or the fp32 absmax itself. Loaded early, decoded late.
struct BlockConst {
    uint32_t c8;
    float s;
};

__device__ __forceinline__ BlockConst load_block_const(const NF4Dev& w, int64_t b) {
    BlockConst r;
    if (w.dq) {
        r.c8 = w.c8[b];
        r.s = w.scale[b / QL_DQ_BLOCKSIZE];
    } else {
        r.c8 = 0;
        r.s = w.absmax[b];
    }
    return r;
}

// OCP FP8 E4M3FN code -> fp32, exact, without branches (a data-dependent
// branch would make the compiler wait for every load in flight): the
// subnormal value m 2^-9 and the normal one (1 + m/8) 2^(e-7) are both formed
// and one is kept by a bit mask; the sign bit is copied last.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 0xFu, m = c & 0x7u;
    const uint32_t sub = __float_as_uint(static_cast<float>(m) * 0x1p-9f);
    const uint32_t nrm = ((e + 120u) << 23) | (m << 20);
    const uint32_t is_sub = 0u - ((e - 1u) >> 31);  // all ones when e == 0
    return __uint_as_float((sub & is_sub) | (nrm & ~is_sub) | ((c & 0x80u) << 24));
}

__device__ __forceinline__ float block_value(const BlockConst& c, int dq, float mu) {
    if (!dq) return c.s;
    const float prod = e4m3_decode(c.c8) * c.s;
    return prod + mu;
}

// Eight consecutive codes (one u32 of packed bytes, element 2j in the high
// nibble of byte j) -> eight bf16 values T[c] * a, low element first.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float a, const float* tab) {
    uint4 r;
    r.x = pack_bf16x2(tab[(w >> 4) & 15u] * a, tab[w & 15u] * a);
    r.y = pack_bf16x2(tab[(w >> 12) & 15u] * a, tab[(w >> 8) & 15u] * a);
    r.z = pack_bf16x2(tab[(w >> 20) & 15u] * a, tab[(w >> 16) & 15u] * a);
    r.w = pack_bf16x2(tab[(w >> 28) & 15u] * a, tab[(w >> 24) & 15u] * a);
    return r;
}

__device__ __forceinline__ void dequant8_f32(uint32_t w, float a, const float* tab, float* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out[2 * j] = tab[(w >> (8 * j + 4)) & 15u] * a;
        out[2 * j + 1] = tab[(w >> (8 * j)) & 15u] * a;
    }
}

// ---------------------------------------------------------------------------
// Register-only NF4 expansion. For one block (one absmax a), the sixteen
// products bf16(T[c] * a) are built once; their low bytes sit in lo[0..3]
// and their high bytes in hi[0..3] (entry c at byte c%4 of word c/4). A code
// then selects its two bytes with v_perm_b32 (8-entry byte lookup) and bit 3
// of the code picks the upper or lower half with v_bfi_b32. No LDS traffic.
// ---------------------------------------------------------------------------
struct Lut16 {
    uint32_t lo[4], hi[4];
};

__device__ __forceinline__ Lut16 make_lut(float a) {
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = pack_bf16x2(kNF4Host[2 * i] * a, kNF4Host[2 * i + 1] * a);
    Lut16 L;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        L.lo[w] = __builtin_amdgcn_perm(p[2 * w + 1], p[2 * w], 0x06040200u);
        L.hi[w] = __builtin_amdgcn_perm(p[2 * w + 1], p[2 * w], 0x07050301u);
    }
    return L;
}

// Bytes of entry (code & 7) of the lower or upper 8 entries of t, chosen per
// byte by mask (0xFF where the code is >= 8).
__device__ __forceinline__ uint32_t lut_bytes(const uint32_t (&t)[4], uint32_t sel7, uint32_t mask) {
    const uint32_t lo = __builtin_amdgcn_perm(t[1], t[0], sel7);
    const uint32_t hi = __builtin_amdgcn_perm(t[3], t[2], sel7);
    return (hi & mask) | (lo & ~mask);
}

// Eight codes (one u32 of packed bytes, element 2j in the high nibble of byte
// j) -> eight bf16 values, element 0 in the low half of .x.
__device__ __forceinline__ uint4 dequant8_lut(uint32_t w, const Lut16& L) {
    const uint32_t se = (w >> 4) & 0x07070707u;  // even elements, low 3 bits of the code
    const uint32_t so = w & 0x07070707u;         // odd elements
    // 0xFF per byte where bit 3 of the code is set. Bit 3 of the even code is
    // bit 7 of its byte (bit 7 of the odd one after << 4); v_perm selectors
    // 8..11 replicate bit 7 of bytes 1, 3 (second source) and 5, 7 (first
    // source), so the first source is the word shifted up one byte.
    const uint32_t me = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
    const uint32_t mo = __builtin_amdgcn_perm(w << 12, w << 4, 0x090B080Au);
    const uint32_t le = lut_bytes(L.lo, se, me), he = lut_bytes(L.hi, se, me);
    const uint32_t lo = lut_bytes(L.lo, so, mo), ho = lut_bytes(L.hi, so, mo);
    const uint32_t xa = __builtin_amdgcn_perm(he, le, 0x05010400u);  // e0 | e2 << 16
    const uint32_t xb = __builtin_amdgcn_perm(he, le, 0x07030602u);  // e4 | e6 << 16
    const uint32_t ya = __builtin_amdgcn_perm(ho, lo, 0x05010400u);  // e1 | e3 << 16
    const uint32_t yb = __builtin_amdgcn_perm(ho, lo, 0x07030602u);  // e5 | e7 << 16
    uint4 r;
    r.x = __builtin_amdgcn_perm(ya, xa, 0x05040100u);
    r.y = __builtin_amdgcn_perm(ya, xa, 0x07060302u);
    r.z = __builtin_amdgcn_perm(yb, xb, 0x05040100u);
    r.w = __builtin_amdgcn_perm(yb, xb, 0x07060302u);
    return r;
}

// The same eight values in the order the lookup yields them, without the
// final interleave: element slots (e0, e2, e4, e6, e1, e3, e5, e7). An MFMA
// operand in this order pairs with a B operand in the same order
// (x_slot_order), which the product does not see: only the pairing matters.
__device__ __forceinline__ uint4 dequant8_lut_slots(uint32_t w, const Lut16& L) {
    const uint32_t se = (w >> 4) & 0x07070707u;
    const uint32_t so = w & 0x07070707u;
    const uint32_t me = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
    const uint32_t mo = __builtin_amdgcn_perm(w << 12, w << 4, 0x090B080Au);
    const uint32_t le = lut_bytes(L.lo, se, me), he = lut_bytes(L.hi, se, me);
    const uint32_t lo = lut_bytes(L.lo, so, mo), ho = lut_bytes(L.hi, so, mo);
    uint4 r;
    r.x = __builtin_amdgcn_perm(he, le, 0x05010400u);  // e0 | e2 << 16
    r.y = __builtin_amdgcn_perm(he, le, 0x07030602u);  // e4 | e6 << 16
    r.z = __builtin_amdgcn_perm(ho, lo, 0x05010400u);  // e1 | e3 << 16
    r.w = __builtin_amdgcn_perm(ho, lo, 0x07030602u);  // e5 | e7 << 16
    return r;
}

// Eight consecutive bf16 values (v.x = x0 | x1 << 16, ...) -> the slot order
// of dequant8_lut_slots: (x0, x2), (x4, x6), (x1, x3), (x5, x7).
__device__ __forceinline__ uint4 x_slot_order(uint4 v) {
    uint4 r;
    r.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
    r.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
    r.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
    r.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
    return r;
}

// ---------------------------------------------------------------------------
// Operand helpers of the rank-r (LoRA) kernels.
// ---------------------------------------------------------------------------
typedef short v4i16_l __attribute__((ext_vector_type(4)));
typedef short v8i16_l __attribute__((ext_vector_type(8)));

// Rows r0 .. r0+7 of column c0 + li of a row-major bf16 LDS tile (row stride
// ld elements) as one MFMA operand of lane li of a 16-lane group: two
// ds_read_b64_tr_b16, each returning four rows of the lane's column.
__device__ __forceinline__ bf16x8_t lds_col8(const uint16_t* tile, int ld, int r0, int c0, int li) {
    const uint16_t* base = tile + (r0 + (li >> 2)) * ld + c0 + 4 * (li & 3);
    // address-space casts (not integer casts) keep the pointer's provenance,
    // so the compiler can tell these reads from direct-to-LDS loads elsewhere
    const v4i16_l lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_l*)(base));
    const v4i16_l hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_l*)(base + 4 * ld));
    const v8i16_l v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

// rowp[c .. c+8), zero for columns >= n (rows of n bf16 values).
__device__ __forceinline__ uint4 load_cols8(const uint16_t* rowp, int c, int n) {
    if ((n & 7) == 0) return c < n ? *reinterpret_cast<const uint4*>(rowp + c) : make_uint4(0, 0, 0, 0);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (c + e < n) ? rowp[c + e] : 0u;
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }

}  // namespace qlnf4
