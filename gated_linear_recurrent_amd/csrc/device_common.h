// Device helpers for the Liger Attention kernels on gfx950 (CDNA4, wave64).
//
// MFMA fragment conventions used throughout (16x16 output tiles):
//   accumulator (D) : lane L holds column (L & 15), rows 4*(L >> 4) + r, r = 0..3
//   operand (A or B): lane L holds row/column (L & 15) and KPL consecutive
//                     k-elements starting at KPL * (L >> 4) of a KSTEP-wide k-step
// so an MFMA computes D[m][n] += sum_k X[m][k] * Y[n][k] for two matrices that are
// both stored k-contiguous ("NT" form). bf16 uses v_mfma_f32_16x16x32_bf16
// (KSTEP 32, KPL 8); fp32 uses v_mfma_f32_16x16x4_f32 (KSTEP 4, KPL 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace liger {

typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(bf16_t, h);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = static_cast<__bf16>(lo);
    v[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// Hardware reciprocal (about 1 ulp); used where a correctly rounded division
// is not needed.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 2^x on the hardware exponential unit (inputs are already in log2 units).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// log2(sigmoid(x)) = min(x, 0)*log2(e) - log2(1 + 2^(-|x| log2(e))), never overflows.
__device__ __forceinline__ float log2_sigmoid(float x) {
    float ax = fabsf(x) * kLog2e;
    return fminf(x, 0.0f) * kLog2e - fast_log2(1.0f + fast_exp2(-ax));
}

__device__ __forceinline__ float sigmoidf_stable(float x) {
    const float e = fast_exp2(-fabsf(x) * kLog2e);
    const float s = fast_rcp(1.0f + e);
    return x >= 0.0f ? s : e * s;
}

// Storage type -> float.
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Numerator of the vector gate's 4-tap pool at channel c of a key row of D
// channels: the sum of the in-range taps c-1 .. c+2 in channel order, with
// the tap count in n. Always four independent reads with no branch: a tap
// past either edge reads channel c and is replaced by zero.
template <int D, typename T>
__device__ __forceinline__ float pool4_taps(const T* row, int c, int& n) {
    const bool hm = c > 0, h1 = c + 1 < D, h2 = c + 2 < D;
    const float tm = to_f32(row[hm ? c - 1 : c]), t0 = to_f32(row[c]);
    const float t1 = to_f32(row[h1 ? c + 1 : c]), t2 = to_f32(row[h2 ? c + 2 : c]);
    n = 1 + int(hm) + int(h1) + int(h2);
    return (((hm ? tm : 0.0f) + t0) + (h1 ? t1 : 0.0f)) + (h2 ? t2 : 0.0f);
}

// DPP lane exchanges (no LDS traffic). Row = 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16 lanes
constexpr int kDppRowShr1 = 0x111;

constexpr int kDppRowShr2 = 0x112;    // lane i <- lane i-2 within its row (0 before the row start)
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowShl1 = 0x101;    // lane i <- lane i+1 within its row (0 past the row end)
constexpr int kDppRowShl2 = 0x102;
constexpr int kDppRowShl4 = 0x104;
constexpr int kDppRowShl8 = 0x108;

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Inclusive suffix sum over aligned groups of G (32 or 64) lanes: lane l
// gets the sum of v over the lanes of its group from l on. Row shifts build
// the suffix inside each 16-lane row; the totals of the later rows of the
// group come from lane reads.
template <int G = 64>
__device__ __forceinline__ float group_suffix_sum(float v) {
    static_assert(G == 32 || G == 64, "a group is half a wave or a wave");
    v += dpp<kDppRowShl1>(v);
    v += dpp<kDppRowShl2>(v);
    v += dpp<kDppRowShl4>(v);
    v += dpp<kDppRowShl8>(v);
    const int row = (threadIdx.x & 63) >> 4;
    if constexpr (G == 64) {
        const float r1 = readlane_f(v, 16), r2 = readlane_f(v, 32), r3 = readlane_f(v, 48);
        const float r23 = r2 + r3;
        return v + (row == 0 ? r1 + r23 : row == 1 ? r23 : row == 2 ? r3 : 0.0f);
    } else {
        const float r1 = readlane_f(v, 16), r3 = readlane_f(v, 48);
        return v + (row == 0 ? r1 : row == 2 ? r3 : 0.0f);
    }
}
__device__ __forceinline__ float wave_suffix_sum(float v) { return group_suffix_sum<64>(v); }

// Inclusive prefix sum over the 64 lanes of a wave: lane l gets the sum of v
// over lanes 0 .. l (row shifts inside each 16-lane row, then the totals of
// the earlier rows from lane reads).
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v += dpp<kDppRowShr1>(v);
    v += dpp<kDppRowShr2>(v);
    v += dpp<kDppRowShr4>(v);
    v += dpp<kDppRowShr8>(v);
    const float r0 = readlane_f(v, 15), r1 = readlane_f(v, 31), r2 = readlane_f(v, 47);
    const float r01 = r0 + r1;
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row == 0 ? 0.0f : row == 1 ? r0 : row == 2 ? r01 : r01 + r2);
}

// All-reduce over aligned groups of 8 lanes.
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    return fmaxf(v, dpp<kDppHalfMirror>(v));
}
__device__ __forceinline__ float group8_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    return v + dpp<kDppHalfMirror>(v);
}

// Cross-row lane exchanges in the VALU (gfx950 v_permlane16_swap /
// v_permlane32_swap, no LDS round trip). Swapping a value with itself gives
// each lane the pair {own, lane ^ 16} (or lane ^ 32) in an order that depends
// on the lane; max and sum are commutative, so every lane of a pair ends
// with the same bits. The pair's elements are copied out as scalars before
// they are reinterpreted: a bit cast applied to an element of the returned
// vector reads element 0 whatever the index.
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    a = __uint_as_float(r0);
    b = __uint_as_float(r1);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    a = __uint_as_float(r0);
    b = __uint_as_float(r1);
}
__device__ __forceinline__ float xor16_max(float v) { float a, b; swap16(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float xor32_max(float v) { float a, b; swap32(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float xor16_sum(float v) { float a, b; swap16(v, a, b); return a + b; }
__device__ __forceinline__ float xor32_sum(float v) { float a, b; swap32(v, a, b); return a + b; }
// Reduction over the four lane groups (L >> 4) that share a fragment row.
__device__ __forceinline__ float group4_max(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float group4_sum(float v) { return xor32_sum(xor16_sum(v)); }

// Workgroup barrier that orders LDS accesses only: the fences are restricted
// to the local address space, so the barrier waits for outstanding LDS
// operations but not for global stores in flight. For kernels whose barriers
// protect LDS data only (no global value written and read back inside the
// workgroup).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- MFMA traits
template <typename OT> struct Mfma;

template <> struct Mfma<bf16_t> {
    static constexpr int KSTEP = 32;
    static constexpr int KPL = 8;
    typedef bf16x8_t frag;
    __device__ static __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // KPL contiguous elements from LDS (16 bytes).
    __device__ static __forceinline__ frag load(const bf16_t* p) {
        return *reinterpret_cast<const bf16x8_t*>(p);
    }
    __device__ static __forceinline__ frag zero() {
        uint4 z = make_uint4(0, 0, 0, 0);
        return __builtin_bit_cast(frag, z);
    }
    // Pack KPL floats (rounded to nearest even).
    __device__ static __forceinline__ frag pack(const float* x) {
        uint4 u;
        u.x = pack_bf16x2(x[0], x[1]);
        u.y = pack_bf16x2(x[2], x[3]);
        u.z = pack_bf16x2(x[4], x[5]);
        u.w = pack_bf16x2(x[6], x[7]);
        return __builtin_bit_cast(frag, u);
    }
};

template <> struct Mfma<float> {
    static constexpr int KSTEP = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    __device__ static __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ frag load(const float* p) { return *p; }
    __device__ static __forceinline__ frag zero() { return 0.0f; }
    __device__ static __forceinline__ frag pack(const float* x) { return x[0]; }
};

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Channel-major tiles ([c][64 keys]: V^T and the transposed state key operand)
// store key j at position key_pos(j): inside each 32-key group the two
// 16-key halves are interleaved in units of 4, so positions 8g .. 8g+7 of a
// group hold keys 4g..4g+3 and 16+4g..16+4g+3. One 16-byte read then yields
// the operand of a key-tile pair in the MFMA order used for the score
// matrices, and two consecutive keys (2m, 2m+1) stay adjacent.
__device__ __forceinline__ int key_pos(int j) {
    return (j & 32) | (((j & 15) >> 2) << 3) | (((j >> 4) & 1) << 2) | (j & 3);
}

// bf16 operand fragment over keys (the contraction index) from a token-major
// [key][channel] tile, read with two transposing LDS loads (ds_read_b64_tr_b16:
// in each 16-lane group, lane i supplies 4 consecutive elements of a row and
// lane 4a+b receives element b of the rows supplied by lanes a, a+4, a+8, a+12).
// Lane (n, g) gets channel c0 + n of keys kb + 4g + 0..3 and kb + 16 + 4g + 0..3,
// the key_pos order of a 32-key group used by the score operands.
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
__device__ __forceinline__ bf16x8_t load_key_frag(const bf16_t* tile, int pitch, int kb, int c0, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const bf16_t* p0 = tile + (kb + 4 * g + (i >> 2)) * pitch + c0 + 4 * (i & 3);
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p0));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p0 + 16 * pitch));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}

}  // namespace liger
