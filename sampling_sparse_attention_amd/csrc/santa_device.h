// Device helpers shared by the SANTA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace santa {

// ---------------------------------------------------------------------------
// Counter-based random numbers: Philox4x64 with 10 rounds, restated from its
// published definition (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011).  Each round multiplies counter words
// 0 and 2 by fixed odd constants (64x64 -> 128 bits), mixes the halves with
// words 1 and 3 and the round key; the key advances by a Weyl increment.
// Only output word 0 is needed here.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t philox4x64_10_word0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                        uint64_t c3, uint64_t k0, uint64_t k1) {
    constexpr uint64_t kMulA = 0xD2E7470EE14C6C93ull;
    constexpr uint64_t kMulB = 0xCA5A826395121157ull;
    constexpr uint64_t kWeylA = 0x9E3779B97F4A7C15ull;
    constexpr uint64_t kWeylB = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t hiA = __umul64hi(kMulA, c0);
        const uint64_t loA = kMulA * c0;
        const uint64_t hiB = __umul64hi(kMulB, c2);
        const uint64_t loB = kMulB * c2;
        const uint64_t n0 = hiB ^ c1 ^ k0;
        const uint64_t n2 = hiA ^ c3 ^ k1;
        c0 = n0;
        c1 = loB;
        c2 = n2;
        c3 = loA;
        k0 += kWeylA;
        k1 += kWeylB;
    }
    return c0;
}

// U[0,1) on the 2^-53 grid for draw j of query head h of sequence b:
// counter (j, h, b, 0), key (seed, 0).
__device__ __forceinline__ double uniform01(uint64_t seed, int b, int h, uint64_t j) {
    const uint64_t w = philox4x64_10_word0(j, (uint64_t)h, (uint64_t)b, 0ull, seed, 0ull);
    return (double)(w >> 11) * 0x1p-53;
}

// ---------------------------------------------------------------------------
// Cross-lane exchange inside a row of LPR lanes (LPR <= 32).  partner<K>(v)
// returns v from a lane that differs from this one in bit K of the lane index
// and agrees in all higher bits (within the row); lower bits may differ, which
// a reduce-scatter butterfly (highest bit first) does not care about.
// Distances below 16 use DPP row operations (no LDS traffic).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int K>
__device__ __forceinline__ float partner(float v) {
    if constexpr (K == 16) {
        // ds_swizzle bitmask mode: and 0x1F, or 0, xor 0x10 -> lane ^ 16 within 32
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    } else if constexpr (K == 8) {
        return dpp_f32<0x128>(v);       // row_ror:8   -> lane ^ 8 within 16
    } else if constexpr (K == 4) {
        return dpp_f32<0x141>(v);       // row_half_mirror: i <-> 7 - i within 8
    } else if constexpr (K == 2) {
        return dpp_f32<0x4E>(v);        // quad_perm(2,3,0,1)
    } else {
        static_assert(K == 1, "distance");
        return dpp_f32<0xB1>(v);        // quad_perm(1,0,3,2)
    }
}

// One reduce-scatter step over distance K: N live values per lane become N/2;
// the lane whose bit K is set keeps (and completes) the upper half.
template <int K, int N>
__device__ __forceinline__ void bfly_step(float* a, bool upper) {
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const float send = upper ? a[j] : a[j + N / 2];
        const float keep = upper ? a[j + N / 2] : a[j];
        a[j] = keep + partner<K>(send);
    }
}

// Reduce-scatter of NVP partial sums across the LPR lanes of a row: afterwards
// lane li of the row holds the complete sums of values [li*NVP/LPR, (li+1)*NVP/LPR)
// in a[0 .. NVP/LPR).  Requires NVP % LPR == 0 and every lane of the wave active.
template <int LPR, int NVP>
__device__ __forceinline__ void row_reduce_scatter(float* a, int li) {
    if constexpr (LPR >= 2) {
        constexpr int K = LPR / 2;
        bfly_step<K, NVP>(a, (li & K) != 0);
        row_reduce_scatter<K, NVP / 2>(a, li);
    }
}

// ---------------------------------------------------------------------------
// Wave-wide reductions and scans (fixed order, so every workgroup that runs
// them on the same data gets the same bits).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ double wave_inclusive_scan_f64(double v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
    }
    return v;
}

__device__ __forceinline__ int wave_inclusive_scan_i32(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
    }
    return v;
}

// Orders LDS writes of this wave before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The exponential used for every probability mass, in both kernels: the two
// passes must evaluate exp(s - m) identically for the tile sums of one pass to
// equal the prefix sums of the other.
__device__ __forceinline__ float mass_exp(float x) { return expf(x); }

// Masses inside a split are summed as 52-bit fixed point (e <= 1, so a split
// of <= 1024 keys stays below 2^62): integer sums are exact and independent of
// their order, so the score pass's tile sum l and the sample pass's prefix
// sums P_i agree to the last bit and P is exactly non-decreasing.
__device__ __forceinline__ uint64_t fixed_mass(float e) { return (uint64_t)(e * 0x1p52f); }
constexpr double kFixedUnit = 0x1p-52;

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------------------
// Element types of q / K / V.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Bf16 {
    static constexpr int bytes = 2;
    // dot product of 8 bf16 of a key row with 8 bf16 of a query (16 bytes each)
    __device__ static __forceinline__ float dot16(const uint4& k, const uint4& q, float acc) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                              __builtin_bit_cast(bf16x2_t, q.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                              __builtin_bit_cast(bf16x2_t, q.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                              __builtin_bit_cast(bf16x2_t, q.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                              __builtin_bit_cast(bf16x2_t, q.w), acc, false);
        return acc;
    }
    // the 8 elements of a 16-byte chunk, widened exactly to fp32
    __device__ static __forceinline__ void widen16(const uint4& v, float* out) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};

struct F32 {
    static constexpr int bytes = 4;
    __device__ static __forceinline__ float dot16(const uint4& k, const uint4& q, float acc) {
        acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
        acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
        acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
        acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
        return acc;
    }
    __device__ static __forceinline__ void widen16(const uint4& v, float* out) {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    }
};

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace santa
