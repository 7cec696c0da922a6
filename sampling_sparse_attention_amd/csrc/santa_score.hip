// Score pass of SANTA decode ("Stochastic Sparse Attention for Memory-Bound
// Inference", §3.2, Pass 1: exact scores, a score stash, per-tile partition
// functions), and the sorted targets of multinomial sampling.
//
// Work unit: one workgroup per (sequence b, KV head g, split t of `split`
// consecutive keys).  The G query heads of the group are served from a single
// read of every K row: the pass streams K with 16-byte loads (LPR lanes per
// row), forms per-lane partial dot products for R rows x G heads with bf16
// dot2 (or fp32 FMA) instructions, and finishes them with one reduce-scatter
// across the row's lanes (DPP), so each lane ends up owning whole scores.
// Scores go to LDS, then to the stash with coalesced stores, together with the
// split statistics m = max s and l = sum exp(s - m) (exact fixed-point sum).
#include "santa_device.h"
#include "santa_internal.h"

namespace santa {

size_t score_lds_bytes(int G, int split) { return (size_t)G * split * sizeof(float); }
size_t sort_lds_bytes(int S) {
    int n = 1;
    while (n < S) n <<= 1;
    return (size_t)n * sizeof(uint64_t);
}

template <int G, int D, typename E>
__global__ __launch_bounds__(kBlock) void score_kernel(Params p) {
    constexpr int LPR = D * E::bytes / 16;        // lanes per K row (16 bytes each)
    constexpr int RPL = 64 / LPR;                 // rows per wave-wide load
    constexpr int R = 16 / RPL;                   // loads per lane per 16-row chunk
    constexpr int NV = R * G;                     // partial sums per lane
    constexpr int NVP = (NV + LPR - 1) / LPR * LPR;
    constexpr int M = NVP / LPR;                  // finished scores per lane
    static_assert(LPR >= 2 && LPR <= 32 && 16 % RPL == 0, "row shape");

    extern __shared__ float sc[];                 // [G][split]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int t = blockIdx.x % p.T;
    const int bg = blockIdx.x / p.T;
    const int g = bg % p.Hkv;
    const int b = bg / p.Hkv;
    const int n = seq_len_of(p, b);

    if (t == 0) {   // the sample pass accumulates into o
        float* o = p.o + ((int64_t)b * p.Hq + (int64_t)g * G) * D;
        for (int i = tid; i < G * D; i += kBlock) o[i] = 0.0f;
    }
    const int key0 = t * p.split;
    if (key0 >= n) return;
    const int ns = min(p.split, n - key0);

    const int c = lane / LPR;                     // which row of a wave-wide load
    const int li = lane % LPR;                    // which 16 bytes of the row
    uint4 qf[G];
    {
        const char* qb = reinterpret_cast<const char*>(p.q) +
                         (((int64_t)b * p.Hq + (int64_t)g * G) * D) * E::bytes + li * 16;
#pragma unroll
        for (int h = 0; h < G; ++h) qf[h] = load16(qb + (int64_t)h * D * E::bytes);
    }

    const char* kbase = reinterpret_cast<const char*>(p.k);
    const int nchunks = (ns + 15) >> 4;

    auto load_chunk = [&](int ch, uint4* kd) {
        const int r0 = key0 + (ch << 4);
        // a 16-row chunk never straddles a page (page_size >= 16, r0 % 16 == 0)
        const int64_t base = row_offset(p, b, g, r0);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = r * RPL + c;
            if ((ch << 4) + rr < ns) {
                kd[r] = load16(kbase + (base + (int64_t)rr * p.stride_tok) * E::bytes + li * 16);
            } else {
                kd[r] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    uint4 cur[R], nxt[R];
#pragma unroll
    for (int r = 0; r < R; ++r) nxt[r] = make_uint4(0u, 0u, 0u, 0u);
    if (wave < nchunks) load_chunk(wave, cur);
    for (int ch = wave; ch < nchunks; ch += kWaves) {
        if (ch + kWaves < nchunks) load_chunk(ch + kWaves, nxt);
        float acc[NVP];
#pragma unroll
        for (int j = 0; j < NVP; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int h = 0; h < G; ++h) acc[r * G + h] = E::dot16(cur[r], qf[h], 0.0f);
        row_reduce_scatter<LPR, NVP>(acc, li);
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const int vi = li * M + j;
            if (vi < NV) {
                const int r = vi / G;
                const int h = vi - r * G;
                const int local = (ch << 4) + r * RPL + c;
                if (local < ns) sc[h * p.split + local] = acc[j] * p.scale;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) cur[r] = nxt[r];
    }
    __syncthreads();

    for (int h = wave; h < G; h += kWaves) {
        const float* row = sc + h * p.split;
        float mx = -INFINITY;
        for (int i = lane; i < ns; i += 64) mx = fmaxf(mx, row[i]);
        mx = wave_max_f32(mx);
        uint64_t lf = 0;
        for (int i = lane; i < ns; i += 64) lf += fixed_mass(mass_exp(row[i] - mx));
        const double l = (double)wave_sum_u64(lf) * kFixedUnit;
        const int hq = g * G + h;
        float* dst = p.scores + ((int64_t)b * p.Hq + hq) * p.score_row + key0;
        for (int i = lane * 4; i < ns; i += 256) {
            if (i + 4 <= ns) {
                *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(row + i);
            } else {
                for (int e = i; e < ns; ++e) dst[e] = row[e];
            }
        }
        if (lane == 0) {
            SplitStat st;
            st.m = mx;
            st.pad = 0.0f;
            st.l = l;
            p.stats[((int64_t)b * p.Hq + hq) * p.T + t] = st;
        }
    }
}

// Multinomial targets: the S uniforms of every (sequence, query head), sorted
// ascending (bitonic sort of their 53-bit integers in LDS), stored as fp64.
__global__ __launch_bounds__(kBlock) void targets_kernel(Params p) {
    extern __shared__ uint64_t keys[];
    const int bh = blockIdx.x;
    const int b = bh / p.Hq;
    const int h = bh - b * p.Hq;
    if (seq_len_of(p, b) == 0) return;
    int N = 1;
    while (N < p.S) N <<= 1;
    for (int j = threadIdx.x; j < N; j += kBlock) {
        keys[j] = (j < p.S) ? (philox4x64_10_word0((uint64_t)j, (uint64_t)h, (uint64_t)b, 0ull,
                                                    p.seed, 0ull) >> 11)
                            : ~0ull;
    }
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < N; i += kBlock) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint64_t a = keys[i], c = keys[ixj];
                    const bool up = (i & k) == 0;
                    if ((a > c) == up) {
                        keys[i] = c;
                        keys[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    double* dst = p.targets + (int64_t)bh * p.S;
    for (int j = threadIdx.x; j < p.S; j += kBlock) dst[j] = (double)keys[j] * 0x1p-53;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int G, int D, typename E>
static hipError_t launch_score_t(const Params& p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.T));
    hipLaunchKernelGGL((score_kernel<G, D, E>), grid, dim3(kBlock), score_lds_bytes(G, p.split),
                       stream, p);
    return hipGetLastError();
}

template <int D, typename E>
static hipError_t launch_score_d(const Params& p, hipStream_t stream) {
    switch (p.G) {
        case 1: return launch_score_t<1, D, E>(p, stream);
        case 2: return launch_score_t<2, D, E>(p, stream);
        case 4: return launch_score_t<4, D, E>(p, stream);
        case 7: return launch_score_t<7, D, E>(p, stream);
        case 8: return launch_score_t<8, D, E>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_score(const Params& p, int dtype, hipStream_t stream) {
    if (dtype == 0) return p.D == 64 ? launch_score_d<64, Bf16>(p, stream)
                                     : launch_score_d<128, Bf16>(p, stream);
    return p.D == 64 ? launch_score_d<64, F32>(p, stream) : launch_score_d<128, F32>(p, stream);
}

hipError_t launch_targets(const Params& p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.B * p.Hq));
    hipLaunchKernelGGL(targets_kernel, grid, dim3(kBlock), sort_lds_bytes(p.S), stream, p);
    return hipGetLastError();
}

}  // namespace santa
