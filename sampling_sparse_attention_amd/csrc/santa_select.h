// Radix selection of the k-th largest of a row of fp32 values, shared by the
// top-k comparator and the Gumbel-top-K team sampler.  The values become
// order-preserving 32-bit keys; three passes (11, 11 and 10 bits) each count,
// among the keys that match the digits fixed so far, how many fall into each
// bin of the next digit, and fix the bin that holds the k-th largest key.
#pragma once

#include "santa_device.h"

namespace santa {

constexpr int kSelectBins = 2048;

// An order-preserving key: a larger value has a larger key (-0 and +0 are
// one value, as they compare equal).
__device__ __forceinline__ uint32_t score_key(float s) {
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive sum over the workgroup of each thread's value (all NT threads
// take part); `scratch` holds 2 * NT / 64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int* scratch) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_scan_add_i32(v);
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int t = lane < NW ? scratch[lane] : 0;
        const int ti = wave_scan_add_i32(t);
        if (lane < NW) scratch[NW + lane] = ti - t;
    }
    __syncthreads();
    const int r = scratch[NW + wave] + incl - v;
    __syncthreads();        // scratch is reused by the next call
    return r;
}

// The k-th largest key (1 <= k <= n) of row[0 .. n) and how many keys equal
// to it are among the k largest (*krem_out).  Thread t reads row[i0 .. i1),
// i0 a multiple of 4 (16-byte loads; the row is 16-byte aligned).  `hist`
// holds kSelectBins uints, `scan` 2 * NT / 64 + 4 ints; NT = kSelectBins / 2.
template <int NT>
__device__ __forceinline__ uint32_t radix_kth(const float* row, int i0, int i1, int k, unsigned int* hist,
                                              int* scan, int* krem_out) {
    static_assert(2 * NT == kSelectBins, "two bins per thread");
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    int krem = k;                           // keys still to take at or below the current prefix
    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kBits[3] = {11, 11, 10};
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = kShift[pass];
        const uint32_t dmask = (1u << kBits[pass]) - 1u;
        for (int j = tid; j < kSelectBins; j += NT) hist[j] = 0u;
        __syncthreads();
        for (int i = i0; i < i1; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + i);
            const float sv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = score_key(sv[e]);
                if (i + e < i1 && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
        }
        __syncthreads();
        // thread t owns bins 2t and 2t + 1; the keys in the bins above a bin come
        // before it, so bin c holds the krem-th largest key when the count above
        // it is below krem and the count above it plus its own reaches krem
        const int c_hi = (int)hist[2 * tid + 1], c_lo = (int)hist[2 * tid];
        const int upto = block_exclusive_sum<NT>(c_hi + c_lo, scan) + c_hi + c_lo;    // bins <= 2t + 1
        if (tid == NT - 1) scan[2 * NW] = upto;                                         // all bins
        __syncthreads();
        const int suf = scan[2 * NW] - upto;                                             // bins > 2t + 1
        if (suf < krem && krem <= suf + c_hi) {
            scan[2 * NW + 1] = 2 * tid + 1;
            scan[2 * NW + 2] = krem - suf;
        } else if (suf + c_hi < krem && krem <= suf + c_hi + c_lo) {
            scan[2 * NW + 1] = 2 * tid;
            scan[2 * NW + 2] = krem - suf - c_hi;
        }
        __syncthreads();
        const uint32_t bin = (uint32_t)scan[2 * NW + 1];
        krem = scan[2 * NW + 2];
        prefix |= (bin & dmask) << shift;
        pmask |= dmask << shift;
        __syncthreads();
    }
    *krem_out = krem;
    return prefix;
}

// The value of an order-preserving key (the inverse of score_key; -0 comes
// back as +0).
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// radix_kth over keys held in registers: thread t holds keys[0 .. nvalid).
template <int NT, int VPT>
__device__ __forceinline__ uint32_t radix_kth_regs(const uint32_t (&keys)[VPT], int nvalid, int k,
                                                   unsigned int* hist, int* scan, int* krem_out) {
    static_assert(2 * NT == kSelectBins, "two bins per thread");
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    int krem = k;
    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kBits[3] = {11, 11, 10};
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = kShift[pass];
        const uint32_t dmask = (1u << kBits[pass]) - 1u;
        for (int j = tid; j < kSelectBins; j += NT) hist[j] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < VPT; ++e)
            if (e < nvalid && (keys[e] & pmask) == prefix) atomicAdd(&hist[(keys[e] >> shift) & dmask], 1u);
        __syncthreads();
        const int c_hi = (int)hist[2 * tid + 1], c_lo = (int)hist[2 * tid];
        const int upto = block_exclusive_sum<NT>(c_hi + c_lo, scan) + c_hi + c_lo;
        if (tid == NT - 1) scan[2 * NW] = upto;
        __syncthreads();
        const int suf = scan[2 * NW] - upto;
        if (suf < krem && krem <= suf + c_hi) {
            scan[2 * NW + 1] = 2 * tid + 1;
            scan[2 * NW + 2] = krem - suf;
        } else if (suf + c_hi < krem && krem <= suf + c_hi + c_lo) {
            scan[2 * NW + 1] = 2 * tid;
            scan[2 * NW + 2] = krem - suf - c_hi;
        }
        __syncthreads();
        const uint32_t bin = (uint32_t)scan[2 * NW + 1];
        krem = scan[2 * NW + 2];
        prefix |= (bin & dmask) << shift;
        pmask |= dmask << shift;
        __syncthreads();
    }
    *krem_out = krem;
    return prefix;
}

}  // namespace santa
