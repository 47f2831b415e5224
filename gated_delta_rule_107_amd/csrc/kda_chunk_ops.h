// Device helpers of the chunk kernels (gfx950): MFMA operand policies for bf16 and float32
// storage, cross-lane (DPP) helpers, element packing and per-lane global addressing.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// ---------------------------------------------------------------- MFMA policies
// Accumulator layout (every 16x16 instruction here): lane l holds C[4*(l/16) + r][l % 16].
template <typename OpT> struct MM;

// Two floats rounded to bf16 and packed into one 32-bit register (v_cvt_pk_bf16_f32).  Four
// elements converted one by one and then reinterpreted as the MFMA's 16-bit integer operand
// compile to four single conversions and two v_perm_b32; built from two of these they take
// two conversions.
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ bf16x4 pack_bf16x4(float a, float b, float c, float d) {
    return __builtin_bit_cast(bf16x4, (u32x2){pack_bf16x2(a, b), pack_bf16x2(c, d)});
}

template <> struct MM<bf16> {
    static constexpr int KS = 32;                  // contraction per natural-order instruction
    typedef bf16x4 B16;                            // B operand for a 16-deep contraction
    static __device__ __forceinline__ B16 b16(const f32x4& x) { return pack_bf16x4(x[0], x[1], x[2], x[3]); }
    // acc += A[r0 + m][c0 + kk] * B[kk][n] over kk < 16, B given as an accumulator-layout
    // tile (rows kk = 4g + j held by lane group g)
    static __device__ __forceinline__ f32x4 k16(const bf16* A, int ld, int r0, int c0, B16 b, f32x4 acc,
                                                int lane) {
        const bf16x4 a = *reinterpret_cast<const bf16x4*>(A + (r0 + (lane & 15)) * ld + c0 + 4 * (lane >> 4));
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), acc, 0, 0, 0);
    }
    // a 16-deep A operand tile loaded once for several products (one per column group)
    typedef bf16x4 A16;
    static __device__ __forceinline__ A16 ld16(const bf16* A, int ld, int r0, int c0, int lane) {
        return *reinterpret_cast<const bf16x4*>(A + (r0 + (lane & 15)) * ld + c0 + 4 * (lane >> 4));
    }
    static __device__ __forceinline__ f32x4 mma16(const A16& a, B16 b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                         acc, 0, 0, 0);
    }
    // A R over a 16-deep contraction with R given in float32 (accumulator layout) and kept to
    // about 16 bits: R = hi + lo, both bf16, two products from the one loaded A.  Used for the
    // diagonal blocks of the WY solve, U_p = N_pp R_p, where rounding R_p to bf16 would carry
    // most of the solve's rounding error into U and the state.
    static __device__ __forceinline__ f32x4 mma16_split(const A16& a, const f32x4& R) {
        const B16 hi = b16(R);
        const B16 lo = pack_bf16x4(R[0] - (float)hi[0], R[1] - (float)hi[1], R[2] - (float)hi[2],
                                   R[3] - (float)hi[3]);
        return mma16(a, lo, mma16(a, hi, f32x4{0.f, 0.f, 0.f, 0.f}));
    }
    // the same over 32 contraction rows given as two tiles (rows c0.. and c0+16..), as a load
    // of the A operand and the product, so that callers can have several loads in flight
    typedef bf16x8 A32;
    static __device__ __forceinline__ A32 ld32(const bf16* A, int ld, int r0, int c0, int lane) {
        const bf16* p = A + (r0 + (lane & 15)) * ld + c0 + 4 * (lane >> 4);
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    static __device__ __forceinline__ f32x4 mma32(const A32& a, B16 b0, B16 b1, f32x4 acc) {
        const bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 k32(const bf16* A, int ld, int r0, int c0, B16 b0, B16 b1,
                                                f32x4 acc, int lane) {
        return mma32(ld32(A, ld, r0, c0, lane), b0, b1, acc);
    }
    // The same products transposed: acc^T += A B, i.e. lane l then holds (A B)[l % 16][4*(l/16) + r].
    // The A and B fragments of a 16x16 instruction have the same lane layout (lane l: row or
    // column l % 16, contraction block l / 16), so swapping the two operands transposes the result.
    static __device__ __forceinline__ f32x4 k16t(const bf16* A, int ld, int r0, int c0, B16 b, f32x4 acc,
                                                 int lane) {
        const bf16x4 a = ld16(A, ld, r0, c0, lane);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, b),
                                                         __builtin_bit_cast(i16x4, a), acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma32t(const A32& a, B16 b0, B16 b1, f32x4 acc) {
        const bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 k32t(const bf16* A, int ld, int r0, int c0, B16 b0, B16 b1,
                                                 f32x4 acc, int lane) {
        return mma32t(ld32(A, ld, r0, c0, lane), b0, b1, acc);
    }
    // natural order, both operands in LDS:
    // acc += (A[ra + m][k0 + kk] * fac[k0 + kk]) * Bm[rb + n][k0 + kk] over kk < 32
    static __device__ __forceinline__ f32x4 nat(const bf16* A, int lda, int ra, const bf16* Bm, int ldb,
                                                int rb, int k0, const float* fac, f32x4 acc, int lane) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(A + (ra + (lane & 15)) * lda + k0 + 8 * (lane >> 4));
        if (fac) {
            const f32x4* f4 = reinterpret_cast<const f32x4*>(fac + k0 + 8 * (lane >> 4));
            const f32x4 lo = f4[0], hi = f4[1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a[j] = (bf16)((float)a[j] * lo[j]);
                a[4 + j] = (bf16)((float)a[4 + j] * hi[j]);
            }
        }
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bm + (rb + (lane & 15)) * ldb + k0 + 8 * (lane >> 4));
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    // two products that share the right operand (an A tile and the M tile of the same
    // sub-tile pair), which is read once
    static __device__ __forceinline__ void nat2(const bf16* A1, const bf16* A2, int lda, int ra, const bf16* Bm,
                                                int ldb, int rb, int k0, const float* fac, f32x4& acc1,
                                                f32x4& acc2, int lane) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bm + (rb + (lane & 15)) * ldb + k0 + 8 * (lane >> 4));
        bf16x8 a1 = *reinterpret_cast<const bf16x8*>(A1 + (ra + (lane & 15)) * lda + k0 + 8 * (lane >> 4));
        bf16x8 a2 = *reinterpret_cast<const bf16x8*>(A2 + (ra + (lane & 15)) * lda + k0 + 8 * (lane >> 4));
        if (fac) {
            const f32x4* f4 = reinterpret_cast<const f32x4*>(fac + k0 + 8 * (lane >> 4));
            const f32x4 lo = f4[0], hi = f4[1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a1[j] = (bf16)((float)a1[j] * lo[j]);
                a1[4 + j] = (bf16)((float)a1[4 + j] * hi[j]);
                a2[j] = (bf16)((float)a2[j] * lo[j]);
                a2[4 + j] = (bf16)((float)a2[4 + j] * hi[j]);
            }
        }
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, b, acc2, 0, 0, 0);
    }
};

template <> struct MM<float> {
    static constexpr int KS = 4;
    typedef f32x4 B16;
    static __device__ __forceinline__ B16 b16(const f32x4& x) { return x; }
    // four v_mfma_f32_16x16x4_f32: step s contracts rows 4g + s (g = lane group)
    static __device__ __forceinline__ f32x4 k16(const float* A, int ld, int r0, int c0, B16 b, f32x4 acc,
                                                int lane) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(A + (r0 + (lane & 15)) * ld + c0 + 4 * (lane >> 4));
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 k32(const float* A, int ld, int r0, int c0, B16 b0, B16 b1,
                                                f32x4 acc, int lane) {
        acc = k16(A, ld, r0, c0, b0, acc, lane);
        return k16(A, ld, r0, c0 + 16, b1, acc, lane);
    }
    typedef f32x4 A16;
    static __device__ __forceinline__ A16 ld16(const float* A, int ld, int r0, int c0, int lane) {
        return *reinterpret_cast<const f32x4*>(A + (r0 + (lane & 15)) * ld + c0 + 4 * (lane >> 4));
    }
    static __device__ __forceinline__ f32x4 mma16(const A16& a, B16 b, f32x4 acc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 mma16_split(const A16& a, const f32x4& R) {
        return mma16(a, R, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    struct A32 { f32x4 lo, hi; };
    static __device__ __forceinline__ A32 ld32(const float* A, int ld, int r0, int c0, int lane) {
        const float* p = A + (r0 + (lane & 15)) * ld + c0 + 4 * (lane >> 4);
        return A32{*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 16)};
    }
    static __device__ __forceinline__ f32x4 mma32(const A32& a, B16 b0, B16 b1, f32x4 acc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[s], b0[s], acc, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[s], b1[s], acc, 0, 0, 0);
        return acc;
    }
    // transposed products (see MM<bf16>::k16t)
    static __device__ __forceinline__ f32x4 k16t(const float* A, int ld, int r0, int c0, B16 b, f32x4 acc,
                                                 int lane) {
        const f32x4 a = ld16(A, ld, r0, c0, lane);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b[s], a[s], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 mma32t(const A32& a, B16 b0, B16 b1, f32x4 acc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b0[s], a.lo[s], acc, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b1[s], a.hi[s], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 k32t(const float* A, int ld, int r0, int c0, B16 b0, B16 b1,
                                                 f32x4 acc, int lane) {
        return mma32t(ld32(A, ld, r0, c0, lane), b0, b1, acc);
    }
    static __device__ __forceinline__ f32x4 nat(const float* A, int lda, int ra, const float* Bm, int ldb,
                                                int rb, int k0, const float* fac, f32x4 acc, int lane) {
        float a = A[(ra + (lane & 15)) * lda + k0 + (lane >> 4)];
        if (fac) a *= fac[k0 + (lane >> 4)];
        const float b = Bm[(rb + (lane & 15)) * ldb + k0 + (lane >> 4)];
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void nat2(const float* A1, const float* A2, int lda, int ra, const float* Bm,
                                                int ldb, int rb, int k0, const float* fac, f32x4& acc1,
                                                f32x4& acc2, int lane) {
        const float b = Bm[(rb + (lane & 15)) * ldb + k0 + (lane >> 4)];
        float a1 = A1[(ra + (lane & 15)) * lda + k0 + (lane >> 4)];
        float a2 = A2[(ra + (lane & 15)) * lda + k0 + (lane >> 4)];
        if (fac) {
            const float f = fac[k0 + (lane >> 4)];
            a1 *= f;
            a2 *= f;
        }
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, b, acc2, 0, 0, 0);
    }
};

// ---------------------------------------------------------------- cross-lane helpers
// Within 16-lane rows: value of lane (i - N) (0 for the first N lanes of the row).
template <int N> __device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 | N, 0xF, 0xF, true));
}
// Within quads of lanes: value of lane (i ^ M), M in {1, 2}.
template <int M> __device__ __forceinline__ float quad_xor(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), M == 1 ? 0xB1 : 0x4E, 0xF, 0xF, false));
}
// Forward substitution with a unit lower-triangular 16 x 16 matrix I + L, its rows spread over
// the 16 lanes of a row: lane t holds row t of four right-hand-side columns in x and row t of
// the negated strictly lower part in nl (nl[s] = -L[t][s], zero for s >= t).  Step s adds
// nl[s] x_s to every row, with x_s (final after step s - 1) read from lane s; rows t <= s add
// zero.  On return lane t holds row t of (I + L)^-1 x.  The whole wave takes part (every lane
// active).
//
// One block of v_fmac_f32_dpp: the multiply-add takes x_s through DPP row_newbcast:s (lane s
// of the row) as its first source, which the compiler's own DPP folding cannot do for the
// three-operand FMA it selects.  A DPP read needs two wait states after the instruction that
// wrote its source: within the block four independent columns per step put three instructions
// between a column's write and its next read, and the s_nop covers the writes before it.
#define KDA_RFS_STEP(S, L)                                                         \
    "v_fmac_f32_dpp %0, %0, %" #L " row_newbcast:" #S " row_mask:0xf bank_mask:0xf\n\t" \
    "v_fmac_f32_dpp %1, %1, %" #L " row_newbcast:" #S " row_mask:0xf bank_mask:0xf\n\t" \
    "v_fmac_f32_dpp %2, %2, %" #L " row_newbcast:" #S " row_mask:0xf bank_mask:0xf\n\t" \
    "v_fmac_f32_dpp %3, %3, %" #L " row_newbcast:" #S " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void rows_forward_subst(float (&x)[4], const float (&nl)[15]) {
    asm volatile("s_nop 1\n\t"
                 KDA_RFS_STEP(0, 4) KDA_RFS_STEP(1, 5) KDA_RFS_STEP(2, 6) KDA_RFS_STEP(3, 7)
                 KDA_RFS_STEP(4, 8) KDA_RFS_STEP(5, 9) KDA_RFS_STEP(6, 10) KDA_RFS_STEP(7, 11)
                 KDA_RFS_STEP(8, 12) KDA_RFS_STEP(9, 13) KDA_RFS_STEP(10, 14) KDA_RFS_STEP(11, 15)
                 KDA_RFS_STEP(12, 16) KDA_RFS_STEP(13, 17) KDA_RFS_STEP(14, 18)
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])
                 : "v"(nl[0]), "v"(nl[1]), "v"(nl[2]), "v"(nl[3]), "v"(nl[4]), "v"(nl[5]), "v"(nl[6]),
                   "v"(nl[7]), "v"(nl[8]), "v"(nl[9]), "v"(nl[10]), "v"(nl[11]), "v"(nl[12]), "v"(nl[13]),
                   "v"(nl[14]));
}
#undef KDA_RFS_STEP
// ---------------------------------------------------------------- bounded row stores
// A raw buffer resource (byte offsets, no stride) over the `bytes` bytes from `base`: a store
// whose offset lies at or past the end is dropped by the hardware's range check, so the rows of
// a chunk past its last token need no branch.  Word 3 is the gfx9 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bounded_rsrc(void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
typedef unsigned u32ev2 __attribute__((ext_vector_type(2)));
typedef unsigned u32ev4 __attribute__((ext_vector_type(4)));
// Four consecutive output elements, one store at byte offset `off` of the resource.
template <typename OpT> struct Store4;
template <> struct Store4<bf16> {
    static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t rs, unsigned off, const f32x4& x) {
        const u32ev2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        __builtin_amdgcn_raw_buffer_store_b64(w, rs, (int)off, 0, 0);
    }
};
template <> struct Store4<float> {
    static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t rs, unsigned off, const f32x4& x) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32ev4, x), rs, (int)off, 0, 0);
    }
};
// ---------------------------------------------------------------- global addressing
// base (wave-uniform, in scalar registers) + a 32-bit byte offset per lane: the form the
// hardware's scalar-base addressing takes, with no 64-bit arithmetic per access
template <typename T> __device__ __forceinline__ T* at_bytes(T* base, unsigned byte_off) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off);
}
template <typename T> __device__ __forceinline__ const T* at_bytes(const T* base, unsigned byte_off) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

template <bool V> struct BoolC { static constexpr bool value = V; };

// ---------------------------------------------------------------- element access
template <typename OpT> struct Ld4;             // 4 consecutive elements <-> float[4]
template <> struct Ld4<bf16> {
    typedef bf16x4 V;
    static __device__ __forceinline__ void to_f(const V& v, float (&x)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
    }
    static __device__ __forceinline__ V from_f(const float (&x)[4]) { return pack_bf16x4(x[0], x[1], x[2], x[3]); }
    static __device__ __forceinline__ V zero() { return from_f({0.f, 0.f, 0.f, 0.f}); }
};
template <> struct Ld4<float> {
    typedef f32x4 V;
    static __device__ __forceinline__ void to_f(const V& v, float (&x)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = v[e];
    }
    static __device__ __forceinline__ V from_f(const float (&x)[4]) { return V{x[0], x[1], x[2], x[3]}; }
    static __device__ __forceinline__ V zero() { return V{0.f, 0.f, 0.f, 0.f}; }
};

__host__ __device__ constexpr int pair_fo_index(int p, int pp) {   // p - pp >= 2, p <= 3
    return p == 2 ? 0 : (pp == 0 ? 1 : 2);                          // (2,0) (3,0) (3,1)
}

}  // namespace kda
