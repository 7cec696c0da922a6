// Sample pass of the two-kernel path: global partition function, per-split
// target ranges, inverse-CDF sampling and the gather-and-add of sampled V rows
// ("Stochastic Sparse Attention for Memory-Bound Inference", section 3.2 steps
// 2-3), from the score stash and statistics the score pass left in the
// workspace.  Same grid as the score pass, so a split's stash is read on the
// XCD that wrote it.
#include "santa_split.h"

namespace santa {

// Four workgroups per CU where that fits without spilling registers: the pass is
// bound by the latency of each workgroup's chain of steps, so residency is speed.
template <int G, int D, typename E, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 3)))
void sample_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const Item it = make_item(p, blockIdx.x);
    const unsigned int err0 = p.sync->error;    // nonzero: an earlier call left stale state
    if (it.n == 0) {
        if (it.t == 0) write_empty<G, D, NT>(p, it);
        return;
    }
    if (it.ns == 0) return;
    const LdsLayout L = lds_layout(G, D, p.split, NT);
    float* sc = reinterpret_cast<float*>(smem + L.scratch);
    int* pages = reinterpret_cast<int*>(smem + L.pages);
    HeadState* hs = reinterpret_cast<HeadState*>(smem + L.heads);
    __shared__ int s_fail;              // a head found records missing
    __shared__ unsigned int s_err;      // thread 0's read of the error word
    if (threadIdx.x == 0) {
        s_fail = 0;
        s_err = err0;
    }
    // the group's prefix words, in flight with the stash loads
    const uint64_t words = load_group_prefix_words<G, NT>(p, it);
    load_pages<NT>(p, it, pages);
    // the split's stash slice in 16-byte pieces, all loads issued before any
    // store; a piece that starts below ns may reach past it, but stays inside
    // the stash row (T * split scores).  The slice, which no other workgroup
    // reads, is returned to zero as it is read: the workspace may next serve a
    // problem of another layout, whose records, counts and slots can lie in
    // these bytes and must read zero
    {
        constexpr int MAXP = (G * (kMaxSplit / 4) + NT - 1) / NT;     // pieces per thread
        const int q4 = p.split / 4;
        uint4 v[MAXP];
        float4* src[MAXP];
#pragma unroll
        for (int k = 0; k < MAXP; ++k) {
            const int i = threadIdx.x + k * NT;
            const int h = i / q4;
            const int c = (i - h * q4) * 4;
            src[k] = (h < G && c < it.ns)
                         ? reinterpret_cast<float4*>(p.stash + ((int64_t)it.b * p.Hq + it.g * G + h) * p.stash_row +
                                                     it.key0 + c)
                         : nullptr;
            if (src[k]) v[k] = load_stream(reinterpret_cast<const uint4*>(src[k]));
        }
#pragma unroll
        for (int k = 0; k < MAXP; ++k) {
            if (src[k]) {
                const int i = threadIdx.x + k * NT;
                reinterpret_cast<uint4*>(sc)[i] = v[k];
                store_stream(src[k], make_float4(0.0f, 0.0f, 0.0f, 0.0f));
            }
        }
    }
    __syncthreads();
    split_stats<G, NT, false>(p, it, sc, reinterpret_cast<uint64_t*>(smem + L.prefix), hs);
    systematic_offsets<G, 0>(p, it, hs);
    __syncthreads();
    if (s_err) {                        // an earlier call left stale state
        if (it.t == 0) poison_group<G, D, NT>(p, it);
        return;
    }
    // the group's prefix comes from the score pass's last split (an earlier
    // launch): one missing now means no score pass preceded this one, which is
    // an error, not a wait
    prefix_and_sample<G, D, E, NT, true>(p, it, L, smem, 0, &s_fail, words);
    finish_output<G, D, NT>(p, it, &s_fail, true);
}

template <int G, int D, typename E>
static hipError_t launch_sample_t(const Params& p, hipStream_t stream) {
    const size_t lds = split_lds_bytes(G, D, p.split, kThreads);
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(&sample_kernel<G, D, E, kThreads>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sample_kernel<G, D, E, kThreads>), dim3((unsigned)p.items), dim3(kThreads), lds, stream, p);
    return hipGetLastError();
}

template <int D, typename E>
static hipError_t launch_sample_d(const Params& p, hipStream_t stream) {
    switch (p.G) {
        case 1: return launch_sample_t<1, D, E>(p, stream);
        case 2: return launch_sample_t<2, D, E>(p, stream);
        case 4: return launch_sample_t<4, D, E>(p, stream);
        case 7: return launch_sample_t<7, D, E>(p, stream);
        case 8: return launch_sample_t<8, D, E>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sample(const Params& p, int dtype, hipStream_t stream) {
    if (dtype == 0) return p.D == 64 ? launch_sample_d<64, Bf16>(p, stream)
                                     : launch_sample_d<128, Bf16>(p, stream);
    return p.D == 64 ? launch_sample_d<64, F32>(p, stream) : launch_sample_d<128, F32>(p, stream);
}

}  // namespace santa
