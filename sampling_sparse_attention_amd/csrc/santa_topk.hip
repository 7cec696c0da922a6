// Deterministic top-k attention, the biased comparator of "Stochastic Sparse
// Attention for Memory-Bound Inference" at a matched budget k = S (section 3.4;
// section 6 calls top-k attention a truncation of the value stage).  The scores
// come from the score pass's stash (the exact scores of section 2, Eq. 1); the
// selection is a radix select on them, as the second decode stage of the
// "Stratified Sparse Attention" page does: the k-th largest score is found
// digit by digit from histograms, without sorting the row.
//
// One workgroup per (sequence, query head).  A row of at most kTopkThreads *
// kTopkRegs scores is read once into registers (and its stash returned to
// zero then); a longer one is read from the stash in every pass below.
//   1. the row maximum M (for the weights exp(s - M));
//   2. three radix passes over order-preserving 32-bit keys of the scores
//      (11, 11 and 10 bits): each counts, among the keys that match the digits
//      fixed so far, how many fall into each bin of the next digit, and fixes
//      the bin that holds the k-th largest key;
//   3. one selection pass in index order: keys above the k-th largest are
//      kept, and of the keys equal to it the lowest indices (block scans give
//      every thread the number of equal and of kept keys before its chunk);
//      the kept keys are written to idx in ascending order, their weights to
//      LDS, and the stash is returned to zero;
//   4. o = sum_kept exp(s - M) v / sum_kept exp(s - M).
#include "santa_select.h"
#include "santa_split.h"

namespace santa {

constexpr int kTopkThreads = kSelectBins / 2;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkBins = kSelectBins;
constexpr int kTopkRegs = 32;           // scores per thread held in registers

// Element offset of V row `key` of KV head g of sequence b.
__device__ __forceinline__ int64_t v_row(const Params& p, int b, int g, int key) {
    int64_t off;
    if (p.page_shift < 0) {
        off = (int64_t)b * p.stride_seq + (int64_t)key * p.stride_tok;
    } else {
        int pg = p.block_table[(int64_t)b * p.pages_per_seq + (key >> p.page_shift)];
        pg = min(max(pg, 0), p.num_pages - 1);
        off = (int64_t)pg * p.stride_seq + (int64_t)(key & ((1 << p.page_shift) - 1)) * p.stride_tok;
    }
    return off + (int64_t)g * p.stride_head;
}

template <int D, typename E>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned int* hist = reinterpret_cast<unsigned int*>(smem);                  // [kTopkBins]
    int* scan = reinterpret_cast<int*>(smem + kTopkBins * 4);                   // [2 * waves + 4]
    float* kept_w = reinterpret_cast<float*>(smem + kTopkBins * 4 + 256);       // [kMaxTopk]
    int* kept_i = reinterpret_cast<int*>(smem + kTopkBins * 4 + 256 + kMaxTopk * 4);
    float* part = reinterpret_cast<float*>(smem);                               // [waves][D], after the selection
    const int bh = blockIdx.x;
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int g = hq / p.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = seq_len_of(p, b);
    float* o = p.o + (int64_t)bh * D;
    int32_t* idx = p.idx + (int64_t)bh * p.S;
    const int k = min(p.S, n);
    for (int i = k + tid; i < p.S; i += kTopkThreads) idx[i] = -1;
    if (n == 0) {
        for (int i = tid; i < D; i += kTopkThreads) o[i] = 0.0f;
        return;
    }
    float* row = p.stash + (int64_t)bh * p.stash_row;
    // thread t owns keys [i0, i1): a multiple of 4 keys, so its reads are 16-byte aligned
    const int C = ((n + kTopkThreads - 1) / kTopkThreads + 3) & ~3;
    const int i0 = min(n, tid * C), i1 = min(n, i0 + C);
    const bool regs = C <= kTopkRegs;       // the same in every thread
    float sr[kTopkRegs];
    uint32_t kr[kTopkRegs];
    if (regs) {
#pragma unroll
        for (int c = 0; c < kTopkRegs; c += 4) {
            float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            if (i0 + c < i1) {
                float4* src = reinterpret_cast<float4*>(row + i0 + c);
                v = *src;
                *src = make_float4(0.0f, 0.0f, 0.0f, 0.0f);      // the stash returns to zero
            }
            sr[c] = v.x; sr[c + 1] = v.y; sr[c + 2] = v.z; sr[c + 3] = v.w;
        }
#pragma unroll
        for (int c = 0; c < kTopkRegs; ++c) kr[c] = score_key(sr[c]);
    }

    // 1. the maximum score
    float mx = -INFINITY;
    if (regs) {
#pragma unroll
        for (int c = 0; c < kTopkRegs; ++c)
            if (i0 + c < i1) mx = fmaxf(mx, sr[c]);
    } else {
        for (int i = i0; i < i1; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + i);
            mx = fmaxf(mx, v.x);
            if (i + 1 < i1) mx = fmaxf(mx, v.y);
            if (i + 2 < i1) mx = fmaxf(mx, v.z);
            if (i + 3 < i1) mx = fmaxf(mx, v.w);
        }
    }
    mx = wave_max_f32(mx);
    if (lane == 0) reinterpret_cast<float*>(scan)[wave] = mx;
    __syncthreads();
    float M = reinterpret_cast<float*>(scan)[0];
    for (int w = 1; w < kTopkWaves; ++w) M = fmaxf(M, reinterpret_cast<float*>(scan)[w]);
    __syncthreads();

    // 2. radix passes: the k-th largest key, digit by digit from the top
    int krem = 0;
    const uint32_t prefix = regs ? radix_kth_regs<kTopkThreads, kTopkRegs>(kr, i1 - i0, k, hist, scan, &krem)
                                 : radix_kth<kTopkThreads>(row, i0, i1, k, hist, scan, &krem);
    // prefix is the k-th largest key; krem keys equal to it are kept (the lowest indices)
    const uint32_t kth = prefix;

    // 3. selection in index order
    int n_eq = 0, n_gt = 0;
    if (regs) {
#pragma unroll
        for (int c = 0; c < kTopkRegs; ++c) {
            if (i0 + c < i1) {
                n_gt += kr[c] > kth ? 1 : 0;
                n_eq += kr[c] == kth ? 1 : 0;
            }
        }
    } else {
        for (int i = i0; i < i1; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + i);
            const float sv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = score_key(sv[e]);
                if (i + e < i1) {
                    n_gt += key > kth ? 1 : 0;
                    n_eq += key == kth ? 1 : 0;
                }
            }
        }
    }
    const int eq_before = block_exclusive_sum<kTopkThreads>(n_eq, scan);
    const int take_eq = max(0, min(n_eq, krem - eq_before));
    int pos = block_exclusive_sum<kTopkThreads>(n_gt + take_eq, scan);
    float wsum = 0.0f;
    int eq_seen = 0;
    auto consider = [&](int i, float s, uint32_t key) {
        bool keep = key > kth;
        if (key == kth) {
            keep = eq_seen < take_eq;
            ++eq_seen;
        }
        if (keep && pos < k) {          // exactly k are kept; the bound only guards the writes
            const float w = __expf(s - M);
            idx[pos] = i;
            kept_i[pos] = i;
            kept_w[pos] = w;
            wsum += w;
            ++pos;
        }
    };
    if (regs) {
#pragma unroll
        for (int c = 0; c < kTopkRegs; ++c)
            if (i0 + c < i1) consider(i0 + c, sr[c], kr[c]);
    } else {
        for (int i = i0; i < i1; i += 4) {
            float4* src = reinterpret_cast<float4*>(row + i);
            const float4 v = *src;
            *src = make_float4(0.0f, 0.0f, 0.0f, 0.0f);      // the stash returns to zero
            const float sv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (i + e < i1) consider(i + e, sv[e], score_key(sv[e]));
        }
    }
    // the sum of the kept weights
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) wsum += __shfl_xor(wsum, m, 64);
    __syncthreads();
    if (lane == 0) reinterpret_cast<float*>(scan)[wave] = wsum;
    __syncthreads();
    float W = 0.0f;
    for (int w = 0; w < kTopkWaves; ++w) W += reinterpret_cast<float*>(scan)[w];

    // 4. gather: LPR lanes read a V row with 16-byte loads, RPL rows per wave-wide load
    constexpr int LPR = D * E::bytes / 16;
    constexpr int RPL = 64 / LPR;
    constexpr int ELV = 16 / E::bytes;
    const int rsub = lane / LPR, piece = lane % LPR;
    float acc[ELV];
#pragma unroll
    for (int e = 0; e < ELV; ++e) acc[e] = 0.0f;
    const char* vbase = reinterpret_cast<const char*>(p.v);
    constexpr int UL = 4;
    for (int r0 = wave * RPL; r0 < k; r0 += kTopkWaves * RPL * UL) {
        uint4 x[UL];
        float wt[UL];
#pragma unroll
        for (int u = 0; u < UL; ++u) {
            const int r = r0 + u * kTopkWaves * RPL + rsub;
            const bool ok = r < k;
            wt[u] = ok ? kept_w[r] : 0.0f;
            const int key = ok ? kept_i[r] : kept_i[0];
            x[u] = load16(vbase + (v_row(p, b, g, key) + piece * ELV) * E::bytes);
        }
#pragma unroll
        for (int u = 0; u < UL; ++u) E::axpy16(wt[u], x[u], acc);
    }
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < ELV; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
    __syncthreads();            // hist / scan are free: reuse them for the partial sums
    if (rsub == 0) {
#pragma unroll
        for (int e = 0; e < ELV; ++e) part[wave * D + piece * ELV + e] = acc[e];
    }
    __syncthreads();
    for (int c = tid; c < D; c += kTopkThreads) {
        float t = 0.0f;
        for (int w = 0; w < kTopkWaves; ++w) t += part[w * D + c];
        o[c] = t / W;
    }
}

size_t topk_lds_bytes() { return (size_t)kTopkBins * 4 + 256 + (size_t)kMaxTopk * 8; }

template <int D, typename E>
static hipError_t launch_topk_t(const Params& p, hipStream_t stream) {
    const size_t lds = topk_lds_bytes();
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(&topk_kernel<D, E>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_kernel<D, E>), dim3((unsigned)(p.B * p.Hq)), dim3(kTopkThreads), lds, stream, p);
    return hipGetLastError();
}

hipError_t launch_topk(const Params& p, int dtype, hipStream_t stream) {
    if (dtype == 0) return p.D == 64 ? launch_topk_t<64, Bf16>(p, stream) : launch_topk_t<128, Bf16>(p, stream);
    return p.D == 64 ? launch_topk_t<64, F32>(p, stream) : launch_topk_t<128, F32>(p, stream);
}

}  // namespace santa
