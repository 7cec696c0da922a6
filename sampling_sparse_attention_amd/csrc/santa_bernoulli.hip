// Bernoulli qK^T with the mean group query, combined with SANTA ("Stochastic
// Sparse Attention for Memory-Bound Inference", section 5, Eq. 5; section 5.1,
// Eq. 6; section 5.3).  The scores of a GQA group are estimated from one
// stochastic representative query: m = mean over the group of |q_h|; each
// feature i is kept by B stratified draws with probability m_i / max m
// (draw n keeps it iff (n + U_{i,n}) / B < m_i / max m, U from Philox4x64-10
// with key (seed, 1) and counter (n, i, g, b)); m_hat_i = (max m / B) count_i;
// and head h's score of key j is sum_i (m_hat_i / m_i) q_{h,i} k_{j,i}.  Only
// the kept features' key values are read, from a channel-major copy of K
// (K^T: [B, Hkv, d, tokens], tokens contiguous), so that skipping a feature
// skips its bytes.  The SANTA step that follows (statistics, global budget,
// sampling, gather of token-major V rows) is the one of the exact path.
//
//   bern_counts_kernel   the feature counts of every (sequence, KV head),
//                        written to the caller's [B, Hkv, d] array;
//   bern_fused_kernel    the fused decode kernel with the estimated scores;
//   bern_score_kernel    the score pass of the two-kernel path (the sample
//                        pass is the exact path's).
#include "santa_split.h"

namespace santa {

// The uniform of draw n of feature i of group (b, g).
__device__ __forceinline__ double bern_uniform(uint64_t seed, int b, int g, int i, int n) {
    const uint64_t w = philox4x64_10_word0((uint64_t)n, (uint64_t)i, (uint64_t)g, (uint64_t)b, seed, 1ull);
    return (double)(w >> 11) * 0x1p-53;
}

// Maximum of a double over the first `nw` waves of the workgroup (every
// thread of the workgroup calls it; the result is returned to all of them).
__device__ __forceinline__ double block_max_f64(double v, int nw, double* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    if (lane == 0 && wave < nw) lds[wave] = v;
    __syncthreads();
    double r = lds[0];
    for (int w = 1; w < nw; ++w) r = fmax(r, lds[w]);
    __syncthreads();
    return r;
}

// m_i = (1/G) sum_h |q_{h,i}| for the feature of this thread (threads < D),
// heads summed in order in fp64 (the decisions below are taken in fp64).
template <int G, typename E>
__device__ __forceinline__ double mean_abs_query(const Params& p, int b, int g, int i, float (&qv)[G]) {
    const char* qb = reinterpret_cast<const char*>(p.q) + ((int64_t)b * p.Hq + (int64_t)g * G) * p.D * E::bytes;
    double m = 0.0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        qv[h] = E::elem(qb, (int64_t)h * p.D + i);
        m += fabs((double)qv[h]);
    }
    return m / (double)G;
}

// One workgroup per (sequence, KV head) group, one thread per (feature,
// slice of draws): thread t takes feature t mod 128 and the draws
// n = t / 128, t / 128 + 8, ...; the slices' counts are summed in LDS.
constexpr int kCountThreads = 1024;
constexpr int kCountSlices = kCountThreads / 128;

template <int G, typename E>
__global__ __launch_bounds__(kCountThreads) void bern_counts_kernel(Params p) {
    __shared__ double s_m[128];
    __shared__ double s_max[kCountThreads / 64];
    __shared__ int s_cnt[kCountSlices][128];
    const int grp = blockIdx.x;
    const int b = grp / p.Hkv, g = grp - b * p.Hkv;
    const int i = threadIdx.x & 127, slice = threadIdx.x >> 7;
    double m = 0.0;
    if (slice == 0 && i < p.D) {
        float qv[G];
        m = mean_abs_query<G, E>(p, b, g, i, qv);
        s_m[i] = m;
    }
    const double top = block_max_f64(m, kCountThreads / 64, s_max);     // its barriers publish s_m
    int count = 0;
    if (i < p.D && top > 0.0) {
        const double pi = s_m[i] / top;
        for (int n = slice; n < p.bern_B; n += kCountSlices)
            if (((double)n + bern_uniform(p.seed, b, g, i, n)) / (double)p.bern_B < pi) ++count;
    }
    s_cnt[slice][i] = count;
    __syncthreads();
    if (slice == 0 && i < p.D) {
        int c = 0;
#pragma unroll
        for (int k = 0; k < kCountSlices; ++k) c += s_cnt[k][i];
        p.bern_counts[(int64_t)grp * p.D + i] = (uint8_t)c;
    }
}

// The group's kept features and, per head, their weights m_hat_i / m_i * q_{h,i}.
template <int G>
struct BernFeatures {
    int n;
    int feat[128];
    float w[G][128];
};

// Builds the kept-feature list of the item's group in `bf` (all threads call it).
template <int G, typename E, int NT>
__device__ __forceinline__ void bern_prologue(const Params& p, const Item& it, BernFeatures<G>& bf) {
    __shared__ double s_max[NT / 64];
    __shared__ int s_cnt[2];
    const int i = threadIdx.x;
    const int lane = i & 63, wave = i >> 6;
    float qv[G];
    int c = 0;
    double m = 0.0;
    if (i < p.D) {
        c = p.bern_counts[((int64_t)it.b * p.Hkv + it.g) * p.D + i];
        m = mean_abs_query<G, E>(p, it.b, it.g, i, qv);
    }
    const double top = block_max_f64(m, (p.D + 63) / 64, s_max);
    const bool keep = i < p.D && c > 0;
    const unsigned long long bal = __ballot(keep);
    if (lane == 0 && wave < 2) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    if (keep) {
        const int pos = (wave == 1 ? s_cnt[0] : 0) + __popcll(bal & ((1ull << lane) - 1ull));
        const double r = (top / (double)p.bern_B) * (double)c / m;     // m_hat_i / m_i
        bf.feat[pos] = i;
#pragma unroll
        for (int h = 0; h < G; ++h) bf.w[h][pos] = (float)(r * (double)qv[h]);
    }
    if (i == 0) bf.n = s_cnt[0] + (p.D > 64 ? s_cnt[1] : 0);
    __syncthreads();
}

// Estimated scores of the split's keys.  Every lane reads one 16-byte piece
// of a feature row per kept feature it takes: wave w covers the keys
// [w * split / NW, (w + 1) * split / NW), lane l the KPL keys from
// (l mod L) * KPL on (L lanes per row piece), and the 64 / L lane groups of a
// wave deal the kept features out round-robin (group r takes the r-th, the
// (r + 64/L)-th, ... in ascending feature order).  Each lane sums its features
// with fused multiply-adds in that order; the groups' sums are then added
// pairwise (xor butterfly, the same result in every lane of a key).
template <int G, typename E, int NT>
__device__ __forceinline__ void bern_stream(const Params& p, const Item& it, float* sc, const BernFeatures<G>& bf) {
    constexpr int NW = NT / 64;
    constexpr int KPL = 16 / E::bytes;         // keys per lane: one 16-byte load per feature row
    constexpr int UF = G * KPL >= 32 ? 4 : 8;  // features a lane has in flight at once (registers)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per_wave = p.split / NW;         // 16 .. 256 keys
    const int L = per_wave / KPL;              // lanes per row piece: 2 .. 64
    const int nfg = 64 / L;                    // feature groups of the wave
    const int fg = lane / L;
    const int lk = wave * per_wave + (lane - fg * L) * KPL;      // first local key of this lane
    const bool active = lk < it.ns;
    const bool full = lk + KPL <= it.ns;
    const char* base = reinterpret_cast<const char*>(p.kt) +
                       ((int64_t)it.b * p.kt_stride_seq + (int64_t)it.g * p.kt_stride_head + it.key0 +
                        (active ? lk : 0)) * E::bytes;
    const int64_t row_bytes = p.kt_stride_feat * E::bytes;
    float acc[G][KPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < KPL; ++j) acc[h][j] = 0.0f;
    const int nf = bf.n;
    for (int f0 = fg; f0 < nf; f0 += UF * nfg) {
        uint4 raw[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int f = f0 + u * nfg;
            raw[u] = make_uint4(0u, 0u, 0u, 0u);
            if (f < nf && active) {
                const char* row = base + (int64_t)bf.feat[f] * row_bytes;
                if (full) {
                    raw[u] = *reinterpret_cast<const uint4*>(row);
                } else {
                    // the sequence ends inside this lane's keys: element by element
                    uint32_t w4[4] = {0u, 0u, 0u, 0u};
                    for (int j = 0; lk + j < it.ns; ++j) {
                        const uint32_t bits = __float_as_uint(E::elem(row, j));
                        if constexpr (E::bytes == 2)
                            w4[j >> 1] |= (j & 1) ? (bits & 0xFFFF0000u) : (bits >> 16);
                        else
                            w4[j] = bits;
                    }
                    raw[u] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int f = f0 + u * nfg;
            const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
            float x[KPL];
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                if constexpr (E::bytes == 2)
                    x[j] = __uint_as_float((j & 1) ? (w4[j >> 1] & 0xFFFF0000u) : (w4[j >> 1] << 16));
                else
                    x[j] = __uint_as_float(w4[j]);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float wt = f < nf ? bf.w[h][f] : 0.0f;
#pragma unroll
                for (int j = 0; j < KPL; ++j) acc[h][j] = fmaf(wt, x[j], acc[h][j]);
            }
        }
    }
    for (int off = L; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < KPL; ++j) acc[h][j] += __shfl_xor(acc[h][j], off, 64);
    }
    if (fg == 0 && active) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < KPL; ++j)
                if (lk + j < it.ns) sc[h * p.split + lk + j] = acc[h][j] * p.scale;
    }
    priority_tail();
}

template <int G, typename E, int NT>
__device__ __forceinline__ void bern_scores(const Params& p, const Item& it, float* sc) {
    __shared__ BernFeatures<G> bf;
    bern_prologue<G, E, NT>(p, it, bf);
    bern_stream<G, E, NT>(p, it, sc, bf);
}

template <int G, int D, typename E, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 3)))
void bern_fused_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int item = take_item(p);
    if (item < 0) return;
    priority_streaming();
    const unsigned int err0 = p.sync->error;
    fused_item<G, D, E, NT>(p, make_item(p, item), err0, smem,
                            [&](const Item& it, float* sc, const int*) { bern_scores<G, E, NT>(p, it, sc); });
}

template <int G, int D, typename E, int NT>
__global__ __launch_bounds__(NT) void bern_score_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const Item it = make_item(p, blockIdx.x);
    if (it.ns == 0) return;
    const LdsLayout L = lds_layout(G, D, p.split, NT);
    float* sc = reinterpret_cast<float*>(smem + L.scratch);
    HeadState* hs = reinterpret_cast<HeadState*>(smem + L.heads);
    bern_scores<G, E, NT>(p, it, sc);
    __syncthreads();
    split_stats<G, NT, true>(p, it, sc, reinterpret_cast<uint64_t*>(smem + L.prefix), hs);
    __syncthreads();
    write_stash<G, NT>(p, it, sc);
}

template <int G, int D, typename E>
static const void* bern_fn(bool fused) {
    return fused ? reinterpret_cast<const void*>(&bern_fused_kernel<G, D, E, kThreads>)
                 : reinterpret_cast<const void*>(&bern_score_kernel<G, D, E, kThreads>);
}

template <int D, typename E>
static const void* bern_fn_g(int G, bool fused) {
    switch (G) {
        case 1: return bern_fn<1, D, E>(fused);
        case 2: return bern_fn<2, D, E>(fused);
        case 4: return bern_fn<4, D, E>(fused);
        case 7: return bern_fn<7, D, E>(fused);
        case 8: return bern_fn<8, D, E>(fused);
        default: return nullptr;
    }
}

static const void* bern_function(const Params& p, int dtype, bool fused) {
    if (dtype == 0) return p.D == 64 ? bern_fn_g<64, Bf16>(p.G, fused) : bern_fn_g<128, Bf16>(p.G, fused);
    return p.D == 64 ? bern_fn_g<64, F32>(p.G, fused) : bern_fn_g<128, F32>(p.G, fused);
}

static hipError_t launch_bern(const Params& p, int dtype, hipStream_t stream, bool fused) {
    const void* fn = bern_function(p, dtype, fused);
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = split_lds_bytes(p.G, p.D, p.split, kThreads);
    const hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    void* args[] = {const_cast<Params*>(&p)};
    return hipLaunchKernel(fn, dim3((unsigned)p.items), dim3(kThreads), args, lds, stream);
}

hipError_t launch_bern_fused(const Params& p, int dtype, hipStream_t stream) { return launch_bern(p, dtype, stream, true); }
hipError_t launch_bern_score(const Params& p, int dtype, hipStream_t stream) { return launch_bern(p, dtype, stream, false); }

int bern_fused_blocks_per_cu(const Params& p, int dtype) {
    const void* fn = bern_function(p, dtype, true);
    if (!fn) return 0;
    const size_t lds = split_lds_bytes(p.G, p.D, p.split, kThreads);
    if (allow_lds(fn, lds) != hipSuccess) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, lds) != hipSuccess) return 0;
    return n;
}

template <int G, typename E>
static hipError_t launch_counts_t(const Params& p, hipStream_t stream) {
    hipLaunchKernelGGL((bern_counts_kernel<G, E>), dim3((unsigned)(p.B * p.Hkv)), dim3(kCountThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename E>
static hipError_t launch_counts_e(const Params& p, hipStream_t stream) {
    switch (p.G) {
        case 1: return launch_counts_t<1, E>(p, stream);
        case 2: return launch_counts_t<2, E>(p, stream);
        case 4: return launch_counts_t<4, E>(p, stream);
        case 7: return launch_counts_t<7, E>(p, stream);
        case 8: return launch_counts_t<8, E>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bern_counts(const Params& p, int dtype, hipStream_t stream) {
    return dtype == 0 ? launch_counts_e<Bf16>(p, stream) : launch_counts_e<F32>(p, stream);
}

}  // namespace santa
