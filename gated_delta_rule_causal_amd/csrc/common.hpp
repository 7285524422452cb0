// Device-side helpers shared by the gfx950 kernels: bf16 conversion, vector
// loads, wave-level reductions, and thin wrappers over the CDNA4 matrix-core
// (MFMA) builtins with the operand/accumulator lane layouts written down.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v* lds_short4_ptr;

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 / I/O
__device__ __forceinline__ float bf16_bits_to_f32(u16 b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round-to-nearest-even float -> bf16 (gfx950 has a native convert; clang
// lowers the __bf16 cast to it).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ u16 f32_to_bf16_bits(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(u16, h);
}

// Two floats as packed bf16 (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16_bits(lo)) | (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

// Activation element type tags.
struct IoF32 {
    using T = float;
    static __device__ __forceinline__ float load(const T* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void store(T* p, size_t i, float x) { p[i] = x; }
    // 4 consecutive elements (p + i must be 16-byte aligned for fp32)
    static __device__ __forceinline__ void load4(const T* p, size_t i, float* out) {
        float4 v = *reinterpret_cast<const float4*>(p + i);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
};
struct IoBF16 {
    using T = u16;
    static __device__ __forceinline__ float load(const T* p, size_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(T* p, size_t i, float x) { p[i] = f32_to_bf16_bits(x); }
    // 4 consecutive elements (p + i must be 8-byte aligned)
    static __device__ __forceinline__ void load4(const T* p, size_t i, float* out) {
        uint2 v = *reinterpret_cast<const uint2*>(p + i);
        out[0] = __uint_as_float(v.x << 16);
        out[1] = __uint_as_float(v.x & 0xffff0000u);
        out[2] = __uint_as_float(v.y << 16);
        out[3] = __uint_as_float(v.y & 0xffff0000u);
    }
};

// ------------------------------------------------------------ feature map
// elu(x) + 1: x + 1 for x > 0, exp(x) otherwise; always positive.
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// --------------------------------------------------------- wave reductions
// x plus the x of another lane of its 16-lane row chosen by a DPP control.
template <int CTRL>
__device__ __forceinline__ float dpp_sum(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of the group receives the group sum, bitwise the same in every
// lane.  Up to 16 lanes (one DPP row) the partial sums move by DPP, which
// stays in the VALU: lane pairs (quad_perm 1,0,3,2), then quad halves
// (2,3,0,1), then the mirrored quad of each 8-lane half and the mirrored half
// of the row; each step adds two equal-sized partial sums, so every lane ends
// with the same value (addition commutes).  Wider groups continue with
// cross-row shuffles.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G >= 2) x = dpp_sum<0xb1>(x);    // quad_perm [1,0,3,2]
    if constexpr (G >= 4) x = dpp_sum<0x4e>(x);    // quad_perm [2,3,0,1]
    if constexpr (G >= 8) x = dpp_sum<0x141>(x);   // row_half_mirror
    if constexpr (G >= 16) x = dpp_sum<0x140>(x);  // row_mirror
#pragma unroll
    for (int off = 16; off < G; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// ------------------------------------------------------------------ MFMA
// v_mfma_f32_16x16x32_bf16: D(16x16) += A(16x32) * B(32x16), fp32 accumulate.
// Lane l (0..63), with r = l % 16 and g = l / 16 (0..3):
//   A operand: 8 bf16 = A[row r][k = 8g .. 8g+7]
//   B operand: 8 bf16 = B[k = 8g .. 8g+7][col r]
//   C/D      : 4 fp32 = D[row 4g + i][col r], i = 0..3
// Any permutation of the K index applied identically to A and B leaves the
// product unchanged; the kernels use that to feed an accumulator tile back in
// as the B operand of the next product without moving data between lanes.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(float x0, float x1, float x2, float x3, float x4, float x5,
                                        float x6, float x7) {
    bf16x8 r;
    r[0] = f32_to_bf16(x0); r[1] = f32_to_bf16(x1); r[2] = f32_to_bf16(x2); r[3] = f32_to_bf16(x3);
    r[4] = f32_to_bf16(x4); r[5] = f32_to_bf16(x5); r[6] = f32_to_bf16(x6); r[7] = f32_to_bf16(x7);
    return r;
}
// Two accumulator tiles (4 values each) as one K=32 B/A operand in the
// permuted-K order: slots 0..3 from tile `lo`, slots 4..7 from tile `hi`.
__device__ __forceinline__ bf16x8 pack_acc_pair(f32x4 lo, f32x4 hi) {
    return pack8(lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------- small MFMA building blocks
__device__ __forceinline__ f32x4 mfma16x16x16(short4v a, short4v b, f32x4 c) {
    // v_mfma_f32_16x16x16_bf16: lane (r = l%16, g = l/16) holds A[r][4g..4g+3],
    // B[4g..4g+3][r]; the accumulator holds D[4g..4g+3][r].  K = 16 equals the
    // accumulator's row span, so an accumulator tile is directly a B operand.
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short4v to_bf16x4(f32x4 x) {
    short4v r;
    r[0] = static_cast<short>(f32_to_bf16_bits(x[0]));
    r[1] = static_cast<short>(f32_to_bf16_bits(x[1]));
    r[2] = static_cast<short>(f32_to_bf16_bits(x[2]));
    r[3] = static_cast<short>(f32_to_bf16_bits(x[3]));
    return r;
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ short4v lds_short4(const u16* p) { return *reinterpret_cast<const short4v*>(p); }

// Decode 8 packed bf16 (one uint4) to fp32.
__device__ __forceinline__ void unpack8(uint4 raw, float* x) {
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        x[j] = __uint_as_float((j & 1) ? (wds[j >> 1] & 0xffff0000u) : (wds[j >> 1] << 16));
}

// fp32 value as a bf16 pair (high part, rounded remainder).
struct Split4 {
    short4v h, l;
};

__device__ __forceinline__ Split4 split4(f32x4 x) {
    Split4 s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const u16 hb = f32_to_bf16_bits(x[e]);
        s.h[e] = static_cast<short>(hb);
        s.l[e] = static_cast<short>(f32_to_bf16_bits(x[e] - bf16_bits_to_f32(hb)));
    }
    return s;
}

// c + a b for 16x16 fp32 matrices given as bf16 pairs (hi*hi + hi*lo + lo*hi:
// about 16 significant bits).  a in operand layout, b in accumulator layout.
__device__ __forceinline__ f32x4 mm3(const Split4& a, const Split4& b, f32x4 c) {
    c = mfma16x16x16(a.l, b.h, c);
    c = mfma16x16x16(a.h, b.l, c);
    return mfma16x16x16(a.h, b.h, c);
}

// (I - N)^{-1} for a strictly lower triangular 16x16 N = -L given in the
// accumulator layout together with its transpose Nt (the operand layout of N
// is the accumulator layout of N^T).  N is nilpotent (N^16 = 0), so
//     (I - N)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8),
// built by three squarings, each folded into the running product; the
// factors are powers of one matrix and commute.  The first (largest)
// correction is formed from split bf16 pairs, the higher powers in bf16.
__device__ __forceinline__ f32x4 unit_lower_inverse(f32x4 N, f32x4 Nt, int r, int g) {
    f32x4 R = N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * g + i == r) R[i] += 1.f;
    const Split4 P = split4(N), Pt = split4(Nt);
    const f32x4 P2 = mm3(Pt, P, zero4());    // N N
    const f32x4 P2t = mm3(P, Pt, zero4());   // (N N)^T = N^T N^T
    R = mm3(split4(P2t), split4(R), R);      // R (I + N^2)
    const short4v q2 = to_bf16x4(P2), q2t = to_bf16x4(P2t);
    const f32x4 P4 = mfma16x16x16(q2t, q2, zero4());
    const f32x4 P4t = mfma16x16x16(q2, q2t, zero4());
    R = mfma16x16x16(to_bf16x4(P4t), to_bf16x4(R), R);   // R (I + N^4)
    const f32x4 P8t = mfma16x16x16(to_bf16x4(P4), to_bf16x4(P4t), zero4());
    return mfma16x16x16(to_bf16x4(P8t), to_bf16x4(R), R);   // R (I + N^8)
}


// ------------------------------------------------------------ LDS helpers

// Workgroup barrier that orders LDS accesses only.  __syncthreads also waits
// for this wave's global loads to land (its fence covers global memory); no
// kernel here communicates through global memory inside a launch, so loads
// issued ahead of time stay in flight across these barriers.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (a wave executes LDS operations in order; this keeps the compiler from
// moving them across).
__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// i reads 4 consecutive 16-bit values E[i][0..3] at its own address, and lane
// j = 4a + b receives E[a][b], E[a+4][b], E[a+8][b], E[a+12][b].
__device__ __forceinline__ short4v ds_read_tr(const u16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_ptr)(p));
}

// MFMA operand (8 values along the contraction index k) from a tile stored
// k-major, X[k][n] with row stride LD: lane (r = 4a + b, g) receives
// X[k0 + 8g + j][col(a) + b], j = 0..7, where col(a) (a multiple of 4) is the
// first of the four columns that lanes 4a..4a+3 of every group take.
template <int LD, class ColFn>
__device__ __forceinline__ bf16x8 tr_operand(const u16 (*X)[LD], int k0, ColFn col, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int c = col(i & 3);
    const short4v lo = ds_read_tr(&X[k0 + 8 * g + (i >> 2)][c]);
    const short4v hi = ds_read_tr(&X[k0 + 8 * g + 4 + (i >> 2)][c]);
    return __builtin_bit_cast(bf16x8, short8v(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
}

}  // namespace la
