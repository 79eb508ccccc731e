// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
//
// Matrix-core fragments.  Every contraction in the library is built from
// 16x16 output tiles of v_mfma_f32_16x16x32_bf16 (bf16 operands) or
// v_mfma_f32_16x16x4_f32 (fp32 operands), plus the 16x16x16 shapes for the
// 16-token triangular products.  For all of them lane l holds output rows
// 4*(l/16)+i (i = 0..3) of column l%16, the A operand's row l%16 and the
// B operand's column l%16; the items a lane contributes along k are paired
// identically in A and B.  The kernels rely only on that pairing, never on
// which logical k an item is: any permutation of k applied to both operands
// leaves the product unchanged.  That lets an accumulator tile (rows
// 4*(l/16)+i) serve directly as a B operand whose k index is the
// accumulator's row, with the A operand read in the matching order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// round-to-nearest-even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Storage element of a tensor: bfloat16 bit patterns or float32.
template <bool BF> struct Store;
template <> struct Store<true> { typedef uint16_t type; };
template <> struct Store<false> { typedef float type; };

__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ------------------------------------------------- 8 consecutive elements

// Raw bits of 8 consecutive storage elements, kept unconverted so a load can
// be issued early (prefetch) and converted after other work.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
    uint4 a;
    __device__ __forceinline__ void load(const uint16_t *p) { a = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void zero() { a = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void to_f32(float (&x)[8]) const {
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void to_f32(float (&x)[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

// Raw bits of 4 consecutive storage elements.
template <typename T> struct Raw4;
template <> struct Raw4<uint16_t> {
    uint2 a;
    __device__ __forceinline__ void load(const uint16_t *p) { a = *reinterpret_cast<const uint2 *>(p); }
    __device__ __forceinline__ void zero() { a = make_uint2(0, 0); }
    __device__ __forceinline__ void to_f32(float (&x)[4]) const {
        x[0] = __uint_as_float(a.x << 16);
        x[1] = __uint_as_float(a.x & 0xffff0000u);
        x[2] = __uint_as_float(a.y << 16);
        x[3] = __uint_as_float(a.y & 0xffff0000u);
    }
};
template <> struct Raw4<float> {
    float4 a;
    __device__ __forceinline__ void load(const float *p) { a = *reinterpret_cast<const float4 *>(p); }
    __device__ __forceinline__ void zero() { a = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void to_f32(float (&x)[4]) const { x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; }
};

// Store 4 consecutive values in the storage type (one 8- or 16-byte store).
__device__ __forceinline__ void store4(uint16_t *p, const float (&x)[4]) {
    const uint32_t lo = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    *reinterpret_cast<uint2 *>(p) = make_uint2(lo, hi);
}
__device__ __forceinline__ void store4(float *p, const float (&x)[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// ------------------------------------------------------ MFMA precisions


template <bool BF> struct Prec;

// bf16 operands, fp32 accumulation.
template <> struct Prec<true> {
    typedef uint16_t elem;   // LDS element
    typedef bf16x8 frag8;    // 8 k-items of a 16x16x32 operand
    typedef i16x4 frag4;     // 4 k-items of a 16x16x16 operand

    static __device__ __forceinline__ frag8 pack8(const float (&x)[8]) {
        f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
        return __builtin_convertvector(v, bf16x8);
    }
    static __device__ __forceinline__ frag8 pack8(f32x4 lo, f32x4 hi) {
        f32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_convertvector(v, bf16x8);
    }
    static __device__ __forceinline__ frag4 pack4(f32x4 x) {
        return __builtin_bit_cast(i16x4, __builtin_convertvector(x, bf16x4));
    }
    // 8 consecutive elements (16-byte aligned)
    static __device__ __forceinline__ frag8 lds8(const elem *p) { return *reinterpret_cast<const bf16x8 *>(p); }
    // 4 consecutive elements at p0 then 4 at p1 (each 8-byte aligned)
    static __device__ __forceinline__ frag8 lds4x2(const elem *p0, const elem *p1) {
        const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
        const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    static __device__ __forceinline__ frag4 lds4(const elem *p) { return *reinterpret_cast<const i16x4 *>(p); }
    static __device__ __forceinline__ void unpack8(frag8 f, float (&x)[8]) {
        const f32x8 v = __builtin_convertvector(f, f32x8);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = v[i];
    }
    static __device__ __forceinline__ void sts8(elem *p, const float (&x)[8]) {
        *reinterpret_cast<bf16x8 *>(p) = pack8(x);
    }
    static __device__ __forceinline__ elem cvt(float x) { return f32_to_bf16(x); }

    // Two-term split x = hi + lo, both bfloat16 (about 16 significant bits
    // together): hi = RNE(x); the residual x - hi is exact in float32.
    static constexpr bool SPLIT = true;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    // The residual is never fused with the product that made x (contraction off):
    // the split then does not depend on where the compiler inlines it.
    static __device__ __forceinline__ void split2(float a, float b, bf16x2 &hi, bf16x2 &lo) {
#pragma clang fp contract(off)
        hi = bf16x2{(__bf16)a, (__bf16)b};
        const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
        const float ra = a - __uint_as_float(hb << 16);
        const float rb = b - __uint_as_float(hb & 0xffff0000u);
        lo = bf16x2{(__bf16)ra, (__bf16)rb};
    }
    static __device__ __forceinline__ void split8(const float (&x)[8], frag8 &hi, frag8 &lo) {
        bf16x2 h[4], l[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) split2(x[2 * p], x[2 * p + 1], h[p], l[p]);
        hi = __builtin_shufflevector(__builtin_shufflevector(h[0], h[1], 0, 1, 2, 3),
                                     __builtin_shufflevector(h[2], h[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
        lo = __builtin_shufflevector(__builtin_shufflevector(l[0], l[1], 0, 1, 2, 3),
                                     __builtin_shufflevector(l[2], l[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    }
    static __device__ __forceinline__ void split8(f32x4 a, f32x4 b, frag8 &hi, frag8 &lo) {
        const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        split8(x, hi, lo);
    }
    static __device__ __forceinline__ void split4(f32x4 x, frag4 &hi, frag4 &lo) {
        bf16x2 h0, h1, l0, l1;
        split2(x[0], x[1], h0, l0);
        split2(x[2], x[3], h1, l1);
        hi = __builtin_bit_cast(i16x4, __builtin_shufflevector(h0, h1, 0, 1, 2, 3));
        lo = __builtin_bit_cast(i16x4, __builtin_shufflevector(l0, l1, 0, 1, 2, 3));
    }
    static __device__ __forceinline__ void split1(float x, elem &hi, elem &lo) {
        const __bf16 h = (__bf16)x;
        hi = __builtin_bit_cast(uint16_t, h);
        lo = f32_to_bf16(x - (float)h);
    }
    static __device__ __forceinline__ void split_sts8(elem *hi, elem *lo, const float (&x)[8]) {
        frag8 h, l;
        split8(x, h, l);
        *reinterpret_cast<frag8 *>(hi) = h;
        *reinterpret_cast<frag8 *>(lo) = l;
    }
    static __device__ __forceinline__ f32x4 mma32(frag8 a, frag8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(frag4 a, frag4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};

// fp32 operands and accumulation (K = 4 per instruction).
template <> struct Prec<false> {
    typedef float elem;
    struct frag8 { f32x4 a, b; };  // items 0..3 and 4..7
    typedef f32x4 frag4;

    static __device__ __forceinline__ frag8 pack8(const float (&x)[8]) {
        frag8 f;
        f.a = f32x4{x[0], x[1], x[2], x[3]};
        f.b = f32x4{x[4], x[5], x[6], x[7]};
        return f;
    }
    static __device__ __forceinline__ frag8 pack8(f32x4 x, f32x4 y) { return frag8{x, y}; }
    static __device__ __forceinline__ frag4 pack4(f32x4 x) { return x; }
    static __device__ __forceinline__ frag8 lds8(const elem *p) {
        return frag8{*reinterpret_cast<const f32x4 *>(p), *reinterpret_cast<const f32x4 *>(p + 4)};
    }
    static __device__ __forceinline__ frag8 lds4x2(const elem *p0, const elem *p1) {
        return frag8{*reinterpret_cast<const f32x4 *>(p0), *reinterpret_cast<const f32x4 *>(p1)};
    }
    static __device__ __forceinline__ frag4 lds4(const elem *p) { return *reinterpret_cast<const f32x4 *>(p); }
    static __device__ __forceinline__ void unpack8(frag8 f, float (&x)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = f.a[i]; x[4 + i] = f.b[i]; }
    }
    static __device__ __forceinline__ void sts8(elem *p, const float (&x)[8]) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4 *>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
    static __device__ __forceinline__ elem cvt(float x) { return x; }

    // float32 operands are already exact: the "high" part is the value, no low part.
    static constexpr bool SPLIT = false;
    static __device__ __forceinline__ void split8(const float (&x)[8], frag8 &hi, frag8 &) { hi = pack8(x); }
    static __device__ __forceinline__ void split8(f32x4 x, f32x4 y, frag8 &hi, frag8 &) { hi = frag8{x, y}; }
    static __device__ __forceinline__ void split4(f32x4 x, frag4 &hi, frag4 &) { hi = x; }
    static __device__ __forceinline__ void split1(float x, elem &hi, elem &) { hi = x; }
    static __device__ __forceinline__ void split_sts8(elem *hi, elem *, const float (&x)[8]) { sts8(hi, x); }
    static __device__ __forceinline__ f32x4 mma32(frag8 a, frag8 b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[i], b.a[i], c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[i], b.b[i], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f32x4 mma16(frag4 a, frag4 b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
        return c;
    }
};

// ------------------------------------------------ fp16 matrix-core operands
//
// v_mfma_f32_16x16x32_f16 / 16x16x16_f16 with fp32 accumulation: 11
// significant bits per operand, for operands bounded by the method (decayed
// L2-normalised keys and queries) or of unit scale (state, values).

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_v __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) fp16x4_v lds_fp16x4;

namespace h16 {

__device__ __forceinline__ f16x8 pack8(const float (&x)[8]) {
    const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
    return __builtin_convertvector(v, f16x8);   // v_cvt_pk_f16_f32, round to nearest even
}
__device__ __forceinline__ f16x8 pack8(f32x4 a, f32x4 b) {
    const f32x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_convertvector(v, f16x8);
}
__device__ __forceinline__ f16x4 pack4(f32x4 x) { return __builtin_convertvector(x, f16x4); }

// x = hi + lo with both parts fp16 (about 22 significant bits together).
__device__ __forceinline__ void split4(f32x4 x, f16x4 &hi, f16x4 &lo) {
    hi = __builtin_convertvector(x, f16x4);
    lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x4), f16x4);
}
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, f16x8 &hi, f16x8 &lo) {
    f16x4 ha, la, hb, lb;
    split4(a, ha, la);
    split4(b, hb, lb);
    hi = __builtin_shufflevector(ha, hb, 0, 1, 2, 3, 4, 5, 6, 7);
    lo = __builtin_shufflevector(la, lb, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4 mma32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 lds8(const _Float16 *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ f16x8 lds4x2(const _Float16 *p0, const _Float16 *p1) {
    const f16x4 a = *reinterpret_cast<const f16x4 *>(p0);
    const f16x4 b = *reinterpret_cast<const f16x4 *>(p1);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4a + b (a, b < 4) supplies an 8-byte address p(a, b); lane i of the
// group receives, as element a, the 16-bit value (i % 4) of p(a, i / 4).
// tr_offset gives the per-lane offset (in elements) that makes lane (g, i)
// (g = lane / 16, i = lane % 16) receive T[4g + a][i], a = 0..3, from a
// row-major 16-wide block T with row stride ld: an MFMA operand whose row is
// the block's column and whose k-items are the block's rows.
__device__ __forceinline__ int tr_offset(int lane, int ld) {
    return (4 * (lane >> 4) + ((lane & 15) >> 2)) * ld + 4 * (lane & 3);
}
__device__ __forceinline__ f16x4 tr4(const _Float16 *p) {
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)p));
}

}  // namespace h16

// ------------------------------------------------------------ wave tools

// Lane i of each 16-lane row receives lane i-N of the same row; lanes i < N get 0.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xF, 0xF, false));
}

// Every lane of each 16-lane row receives lane N's value of that row (DPP
// row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, true));
}

// Sixteen per-row values, one read per lane: lane i of a row holds element i
// (x = src[i]); afterwards every lane of the row holds all sixteen as four
// 4-vectors, out[j][e] = element 4j + e.  Replaces sixteen-lane-redundant
// 16-byte LDS reads by one 4-byte read and sixteen DPP broadcasts.
__device__ __forceinline__ void row_gather16(float x, f32x4 (&out)[4]) {
    out[0] = f32x4{row_bcast<0>(x), row_bcast<1>(x), row_bcast<2>(x), row_bcast<3>(x)};
    out[1] = f32x4{row_bcast<4>(x), row_bcast<5>(x), row_bcast<6>(x), row_bcast<7>(x)};
    out[2] = f32x4{row_bcast<8>(x), row_bcast<9>(x), row_bcast<10>(x), row_bcast<11>(x)};
    out[3] = f32x4{row_bcast<12>(x), row_bcast<13>(x), row_bcast<14>(x), row_bcast<15>(x)};
}

// Inclusive prefix sum over the 16 lanes of each DPP row.
__device__ __forceinline__ float row_inclusive_scan(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

// Workgroup barrier that orders LDS traffic only: outstanding global loads
// (prefetches) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's earlier LDS writes before its later LDS reads (other
// lanes of the same wave read what one lane wrote).
__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Forward substitution for the inverse of a unit lower-triangular 16x16 block,
// one column per lane: on entry lane i of each 16-lane row holds column i of
// the strictly lower part (Lc[ii] = L[ii][i]) and X = e_i; on exit X is column
// i of (I + L)^-1.  Step JJ needs L[ii][JJ] in every lane of the row: that is
// lane JJ's Lc[ii], taken by a DPP row broadcast fused into the FMA
// (v_fmac_f32 with row_newbcast:JJ).  The broadcast sources are only ever
// written by loads, never by a vector-ALU instruction, so no DPP read follows
// a VALU write of its source.
template <int JJ>
__device__ __forceinline__ void unit_lower_inverse_steps(float (&X)[16], const float (&Lc)[16]) {
    const float nx = -X[JJ];
#pragma unroll
    for (int ii = JJ + 1; ii < 16; ++ii)
        asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
            : "+v"(X[ii]) : "v"(Lc[ii]), "v"(nx), "i"(JJ));
    if constexpr (JJ + 2 < 16) unit_lower_inverse_steps<JJ + 1>(X, Lc);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Log-decay from a gate logit z: g = g_min * sigmoid(s z) with g_min = -5 and s
// the head's scale exp(A_h) ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the
// scaled-sigmoid mapping that replaced the unbounded -softplus one).  In
// [-5, 0] for every z: exp2 of a huge argument is inf and 1/inf is 0.
__device__ __forceinline__ float gate_from_logit(float z, float s) {
    constexpr float LOG2E_ = 1.4426950408889634f;
    return -5.0f * fast_rcp(1.0f + fast_exp2(-s * z * LOG2E_));
}

// Logistic sigmoid; for very negative x the exp overflows and rcp(inf) = 0.
// Workgroups are dealt to the 8 XCDs round robin (block i runs on XCD i mod 8).
// For a streaming kernel with one workgroup per item, map block i to item
// (i mod 8) n/8 + i/8, so that each XCD walks a contiguous range of the n items
// (a bijection when n is a multiple of 8; otherwise blocks keep their index).
__device__ __forceinline__ int xcd_contiguous(int block, int n) {
    return (n & 7) ? block : (block & 7) * (n >> 3) + (block >> 3);
}

__device__ __forceinline__ float sigmoid_f32(float x) {
    constexpr float LOG2E_ = 1.4426950408889634f;
    return fast_rcp(1.0f + fast_exp2(-x * LOG2E_));
}

}  // namespace kda
