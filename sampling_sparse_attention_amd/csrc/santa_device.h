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
// Draw j of query head h of sequence b in stream `stream` (counter word 3:
// 0 for SANTA's draws, 1 + t for tile t of S^2ANTA-flash).
__device__ __forceinline__ double uniform01(uint64_t seed, int b, int h, uint64_t j, uint64_t stream = 0) {
    const uint64_t w = philox4x64_10_word0(j, (uint64_t)h, (uint64_t)b, stream, seed, 0ull);
    return (double)(w >> 11) * 0x1p-53;
}

// ---------------------------------------------------------------------------
// Wave priority (fused kernel).  A workgroup streaming K issues ahead of a
// co-resident one that has finished its stream and runs its tail (statistics,
// merge, sampling), so the scoring between two batches of K loads, and with it
// the next batch, is not held up behind tail arithmetic: the last K stream of
// the Llama-shaped step ends about 0.5 us earlier.  Grids larger than the
// device (two-kernel path, flash) gain nothing or lose: there a finished tail
// frees its slot for the next workgroup.  Lowering the priority where it was
// never raised does nothing.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void priority_streaming() { __builtin_amdgcn_s_setprio(2); }
__device__ __forceinline__ void priority_tail() { __builtin_amdgcn_s_setprio(0); }

// ---------------------------------------------------------------------------
// Cross-lane data movement with DPP (VALU-only, no LDS traffic).
//
// dpp<CTRL, ROWS>(identity, v): v taken from the lane CTRL names, or
// `identity` where that lane does not exist or the row is masked off.
// Controls used (GFX9 DPP): row_shr:n = 0x110+n (lane i of a 16-lane row reads
// lane i-n of the same row), row_bcast:15 = 0x142 (every lane of row r reads
// lane 15 of row r-1), row_bcast:31 = 0x143 (rows 2 and 3 read lane 31),
// row_ror:8 = 0x128, row_half_mirror = 0x141, quad_perm = 0x00..0xFF.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t identity, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROWS, 0xF, false);
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f32(float identity, float v) {
    return __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(identity), __float_as_uint(v)));
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {   // identity 0
    const uint32_t lo = dpp_u32<CTRL, ROWS>(0u, (uint32_t)v);
    const uint32_t hi = dpp_u32<CTRL, ROWS>(0u, (uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {       // identity +0.0
    return __longlong_as_double((long long)dpp_u64<CTRL, ROWS>((uint64_t)__double_as_longlong(v)));
}

// Inclusive scans over the 64 lanes of a wave (Hillis-Steele inside 16-lane
// rows, then the two row broadcasts).  Every lane of the wave must be active.
// The order of operations is fixed, so identical inputs give identical bits in
// every workgroup.
__device__ __forceinline__ uint64_t wave_scan_add_u64(uint64_t x) {
    x += dpp_u64<0x111>(x);
    x += dpp_u64<0x112>(x);
    x += dpp_u64<0x114>(x);
    x += dpp_u64<0x118>(x);
    x += dpp_u64<0x142, 0xA>(x);
    x += dpp_u64<0x143, 0xC>(x);
    return x;
}

__device__ __forceinline__ double wave_scan_add_f64(double x) {
    x += dpp_f64<0x111>(x);
    x += dpp_f64<0x112>(x);
    x += dpp_f64<0x114>(x);
    x += dpp_f64<0x118>(x);
    x += dpp_f64<0x142, 0xA>(x);
    x += dpp_f64<0x143, 0xC>(x);
    return x;
}

__device__ __forceinline__ float wave_scan_max_f32(float x) {
    const float lo = -INFINITY;
    x = fmaxf(x, dpp_f32<0x111>(lo, x));
    x = fmaxf(x, dpp_f32<0x112>(lo, x));
    x = fmaxf(x, dpp_f32<0x114>(lo, x));
    x = fmaxf(x, dpp_f32<0x118>(lo, x));
    x = fmaxf(x, dpp_f32<0x142, 0xA>(lo, x));
    x = fmaxf(x, dpp_f32<0x143, 0xC>(lo, x));
    return x;
}

__device__ __forceinline__ int wave_scan_max_i32(int x) {
    const uint32_t lo = 0x80000000u;
    x = max(x, (int)dpp_u32<0x111>(lo, (uint32_t)x));
    x = max(x, (int)dpp_u32<0x112>(lo, (uint32_t)x));
    x = max(x, (int)dpp_u32<0x114>(lo, (uint32_t)x));
    x = max(x, (int)dpp_u32<0x118>(lo, (uint32_t)x));
    x = max(x, (int)dpp_u32<0x142, 0xA>(lo, (uint32_t)x));
    x = max(x, (int)dpp_u32<0x143, 0xC>(lo, (uint32_t)x));
    return x;
}

__device__ __forceinline__ int wave_scan_add_i32(int x) {
    x += (int)dpp_u32<0x111>(0u, (uint32_t)x);
    x += (int)dpp_u32<0x112>(0u, (uint32_t)x);
    x += (int)dpp_u32<0x114>(0u, (uint32_t)x);
    x += (int)dpp_u32<0x118>(0u, (uint32_t)x);
    x += (int)dpp_u32<0x142, 0xA>(0u, (uint32_t)x);
    x += (int)dpp_u32<0x143, 0xC>(0u, (uint32_t)x);
    return x;
}

// The value of lane `src` (uniform) in every lane.
__device__ __forceinline__ float lane_f32(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ int lane_i32(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int src) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double lane_f64(double v, int src) {
    return __longlong_as_double((long long)lane_u64((uint64_t)__double_as_longlong(v), src));
}

// Whole-wave reductions: the result in every lane.
__device__ __forceinline__ float wave_max_f32(float v) { return lane_f32(wave_scan_max_f32(v), 63); }
__device__ __forceinline__ int wave_max_i32(int v) { return lane_i32(wave_scan_max_i32(v), 63); }
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) { return lane_u64(wave_scan_add_u64(v), 63); }

// ---------------------------------------------------------------------------
// Reduce-scatter across the LPR lanes of a K row (LPR <= 32).  partner<K>(v)
// returns v from a lane that differs from this one in bit K of the lane index
// and agrees in all higher bits (within the row); lower bits may differ, which
// a reduce-scatter butterfly (highest bit first) does not care about.
// ---------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ float partner(float v) {
    if constexpr (K == 16) {
        // ds_swizzle bitmask mode: and 0x1F, or 0, xor 0x10 -> lane ^ 16 within 32
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    } else if constexpr (K == 8) {
        return dpp_f32<0x128>(0.0f, v);       // row_ror:8   -> lane ^ 8 within 16
    } else if constexpr (K == 4) {
        return dpp_f32<0x141>(0.0f, v);       // row_half_mirror: i <-> 7 - i within 8
    } else if constexpr (K == 2) {
        return dpp_f32<0x4E>(0.0f, v);        // quad_perm(2,3,0,1)
    } else {
        static_assert(K == 1, "distance");
        return dpp_f32<0xB1>(0.0f, v);        // quad_perm(1,0,3,2)
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

// Afterwards lane li of the row holds the complete sums of values
// [li*NVP/LPR, (li+1)*NVP/LPR) in a[0 .. NVP/LPR).  Requires NVP % LPR == 0
// and every lane of the wave active.
template <int LPR, int NVP>
__device__ __forceinline__ void row_reduce_scatter(float* a, int li) {
    if constexpr (LPR >= 2) {
        constexpr int K = LPR / 2;
        bfly_step<K, NVP>(a, (li & K) != 0);
        row_reduce_scatter<K, NVP / 2>(a, li);
    }
}

// Orders LDS writes of this wave before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The exponential used for every probability mass: the hardware base-2
// exponential of x * log2(e).  Each mass is evaluated once (the statistics and
// the in-split CDF share the fixed-point values), and a split's scale factor
// exp(m_t - M) is evaluated with the same function wherever it is used.  Its
// relative error (a few 1e-7 for |x| <= 20) is below that of the fp32 scores.
__device__ __forceinline__ float mass_exp(float x) { return __expf(x); }

// Masses inside a split are summed as 52-bit fixed point (e <= 1, so a split
// of <= 1024 keys stays below 2^62): integer sums are exact and independent of
// their order, so the prefix sums P_i are exactly non-decreasing and their
// last value is the split's total.  Conversions to fixed point round to
// nearest: for x * scale in [0, 2^52] (exact, scale a power of two), adding
// 2^52 in one FMA leaves the rounded integer in the low bits of the double
// (instead of the library's multi-step double-to-integer sequence).
__device__ __forceinline__ uint64_t fixed_round(double x, double scale) {
    return (uint64_t)__double_as_longlong(fma(x, scale, 0x1p52)) - 0x4330000000000000ull;
}
__device__ __forceinline__ uint64_t fixed_mass(float e) { return fixed_round((double)e, 0x1p52); }
// A split's mass w <= 1024 on the 2^-40 grid of the cross-split prefix
// (w * 2^40 < 2^52).
__device__ __forceinline__ uint64_t fixed40(double w) { return fixed_round(w, 0x1p40); }
__device__ __forceinline__ double fixed_to_double(uint64_t v) { return (double)v * 0x1p-52; }

// ---------------------------------------------------------------------------
// Element types of q / K / V.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Bf16 {
    static constexpr int bytes = 2;
    // element i of a bf16 array, widened exactly
    __device__ static __forceinline__ float elem(const void* base, int64_t i) {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
    }
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
    // acc[e] += w * x_e for the 8 bf16 of a 16-byte piece of a V row (exact
    // widening to fp32, element e at bits 16e of the piece)
    __device__ static __forceinline__ void axpy16(float w, const uint4& x, float* acc) {
        const uint32_t v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(w, __uint_as_float(v[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, __uint_as_float(v[i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
    }
};

struct F32 {
    static constexpr int bytes = 4;
    __device__ static __forceinline__ float elem(const void* base, int64_t i) {
        return reinterpret_cast<const float*>(base)[i];
    }
    __device__ static __forceinline__ float dot16(const uint4& k, const uint4& q, float acc) {
        acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
        acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
        acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
        acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
        return acc;
    }
    __device__ static __forceinline__ void axpy16(float w, const uint4& x, float* acc) {
        acc[0] = fmaf(w, __uint_as_float(x.x), acc[0]);
        acc[1] = fmaf(w, __uint_as_float(x.y), acc[1]);
        acc[2] = fmaf(w, __uint_as_float(x.z), acc[2]);
        acc[3] = fmaf(w, __uint_as_float(x.w), acc[3]);
    }
};

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Loads of data that one call reads once, in a stream (the keys, a stash
// slice): the nontemporal hint keeps these lines from displacing, in the L2
// caches, the lines the call reads again (records, shared value rows, code).
typedef unsigned int stream_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int stream_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint16_t load_stream(const uint16_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t load_stream(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
    const stream_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const stream_u32x2*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    const stream_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const stream_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load16_stream(const void* p) { return load_stream(reinterpret_cast<const uint4*>(p)); }

// The same hint for 16-byte stores of data written once (the stash, which the
// sample pass reads once, and the zeros that return it to zero).
typedef float stream_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(float4* p, const float4& v) {
    __builtin_nontemporal_store((stream_f32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<stream_f32x4*>(p));
}

}  // namespace santa
