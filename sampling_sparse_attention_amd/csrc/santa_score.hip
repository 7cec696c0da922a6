// Score pass of the two-kernel path ("Stochastic Sparse Attention for
// Memory-Bound Inference", section 3.2, Pass 1: exact scores, a score stash and
// per-tile partition functions), the sorted targets of multinomial sampling,
// and the workspace clear.
#include "santa_split.h"

namespace santa {

size_t split_lds_bytes(int G, int D, int split, int nt) { return lds_layout(G, D, split, nt).total; }

size_t sort_lds_bytes(int S) {
    int n = 1;
    while (n < S) n <<= 1;
    return (size_t)n * sizeof(uint64_t);
}

// Multinomial targets: the S uniforms of (sequence, query head) bh, sorted
// ascending (bitonic sort of their 53-bit integers in `keys`, sort_lds_bytes(S)
// of LDS), stored as fp64.  Every thread of the workgroup calls it.
template <int NT>
__device__ __forceinline__ void sort_targets(const Params& p, int bh, uint64_t* keys) {
    const int b = bh / p.Hq;
    const int h = bh - b * p.Hq;
    if (seq_len_of(p, b) == 0) return;
    int N = 1;
    while (N < p.S) N <<= 1;
    for (int j = threadIdx.x; j < N; j += NT) {
        keys[j] = (j < p.S) ? (philox4x64_10_word0((uint64_t)j, (uint64_t)h, (uint64_t)b, 0ull,
                                                    p.seed, 0ull) >> 11)
                            : ~0ull;
    }
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < N; i += NT) {
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
    for (int j = threadIdx.x; j < p.S; j += NT) dst[j] = (double)keys[j] * 0x1p-53;
}

// One workgroup per (sequence, query head).
__global__ __launch_bounds__(256) void targets_kernel(Params p) {
    extern __shared__ uint64_t keys[];
    sort_targets<256>(p, blockIdx.x, keys);
}

// STATS: also the split statistics and records (the sample pass needs them;
// the top-k comparator reads only the stash).
template <int G, int D, typename E, int NT, bool STATS>
__global__ __launch_bounds__(NT) void score_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const Item at = item_coords(p, blockIdx.x);
    uint4 qf[G];
    load_q<G, D, E, NT>(p, at.b, at.g, qf);
    const Item it = make_item(p, blockIdx.x);
    if (it.ns != 0) {
        const LdsLayout L = lds_layout(G, D, p.split, NT);
        float* sc = reinterpret_cast<float*>(smem + L.scratch);
        int* pages = reinterpret_cast<int*>(smem + L.pages);
        HeadState* hs = reinterpret_cast<HeadState*>(smem + L.heads);
        load_pages<NT>(p, it, pages);
        __syncthreads();
        uint4 kd[ScoreStream<G, D, E, NT>::CB][ScoreStream<G, D, E, NT>::R];
        stream_scores<G, D, E, NT>(p, it, sc, pages, qf, kd, false);
        __syncthreads();
        if constexpr (STATS) {
            split_stats<G, NT, true>(p, it, sc, reinterpret_cast<uint64_t*>(smem + L.prefix), hs);
            __syncthreads();
        }
        write_stash<G, NT, STATS>(p, it, sc);
        if constexpr (STATS) publish_group_prefix<G, NT>(p, it);
    }
    if constexpr (STATS) {
        // the first B * Hq workgroups, dispatched first, sort the multinomial
        // targets once their own split is done, while the others stream K
        if (p.sort_in_score && blockIdx.x < p.B * p.Hq) {
            __syncthreads();        // the split's LDS is free again
            sort_targets<NT>(p, blockIdx.x, reinterpret_cast<uint64_t*>(smem));
        }
    }
}

// Zero-fills `n16` 16-byte words and `tail` further bytes.
__global__ __launch_bounds__(256) void clear_kernel(uint4* p, size_t n16, unsigned char* tail, int ntail) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_clear(void* ws, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const int ntail = (int)(bytes % 16);
    const size_t blocks = n16 ? ((n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096) : 1;
    hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint4*>(ws), n16, reinterpret_cast<unsigned char*>(ws) + n16 * 16,
                       ntail);
    return hipGetLastError();
}

template <int G, int D, typename E, bool STATS>
static hipError_t launch_score_t(const Params& p, hipStream_t stream) {
    const size_t lds = split_lds_bytes(G, D, p.split, kThreads);
    const void* fn = reinterpret_cast<const void*>(&score_kernel<G, D, E, kThreads, STATS>);
    const hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((score_kernel<G, D, E, kThreads, STATS>), dim3((unsigned)p.items), dim3(kThreads), lds,
                       stream, p);
    return hipGetLastError();
}

template <int D, typename E, bool STATS>
static hipError_t launch_score_d(const Params& p, hipStream_t stream) {
    switch (p.G) {
        case 1: return launch_score_t<1, D, E, STATS>(p, stream);
        case 2: return launch_score_t<2, D, E, STATS>(p, stream);
        case 4: return launch_score_t<4, D, E, STATS>(p, stream);
        case 7: return launch_score_t<7, D, E, STATS>(p, stream);
        case 8: return launch_score_t<8, D, E, STATS>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool STATS>
static hipError_t launch_score_s(const Params& p, int dtype, hipStream_t stream) {
    if (dtype == 0) return p.D == 64 ? launch_score_d<64, Bf16, STATS>(p, stream)
                                     : launch_score_d<128, Bf16, STATS>(p, stream);
    return p.D == 64 ? launch_score_d<64, F32, STATS>(p, stream) : launch_score_d<128, F32, STATS>(p, stream);
}

hipError_t launch_score(const Params& p, int dtype, hipStream_t stream, bool stats) {
    return stats ? launch_score_s<true>(p, dtype, stream) : launch_score_s<false>(p, dtype, stream);
}

hipError_t launch_targets(const Params& p, hipStream_t stream) {
    hipLaunchKernelGGL(targets_kernel, dim3((unsigned)((int64_t)p.B * p.Hq)), dim3(256),
                       sort_lds_bytes(p.S), stream, p);
    return hipGetLastError();
}

}  // namespace santa
