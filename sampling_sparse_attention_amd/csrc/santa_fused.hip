// Fused SANTA decode kernel: the whole step of section 3.2 of "Stochastic
// Sparse Attention for Memory-Bound Inference" (score pass, global budget,
// parallel gather) in one launch, one workgroup per work item -- (sequence,
// KV head, split) -- with each split's scores kept in LDS across the global
// step.
//
// The only wait is for the statistics of the other splits of the same
// (sequence, KV head) group.  Two ways to guarantee that every statistic a
// workgroup waits for is computed by a workgroup that runs:
//   - the device holds every workgroup of the grid at once (blockIdx gives
//     the item);
//   - tickets: each workgroup takes the next item from an atomic counter when
//     it starts, items numbered group by group, and one group's splits fit on
//     any single compute die (XCD).  A workgroup waits only for items of its
//     own group.  Once a ticket of the next group is taken, every ticket of
//     this group has been, so a workgroup that cannot be placed is kept out
//     only by workgroups of earlier groups, which finish without waiting for
//     later ones, or of this group.  A die whose slots all hold waiting
//     workgroups of one group would hold the whole group, so while tickets of
//     a group remain untaken some die that still has workgroups to start has
//     a slot that frees.  (Room for one group on the whole device is not
//     enough: the die a workgroup runs on is fixed by its index, and when
//     some dies run out of workgroups the remaining tickets can only be
//     taken on dies that one group's waiting workgroups may fill.)  The
//     groups' K streams and latency-bound tails then overlap from one group
//     to the next.
#include "santa_split.h"

namespace santa {

// KW, UL: the sampler's keys counted at once and V loads in flight per lane
template <int G, int D, typename E, int NT, int KW = 4, int UL = 8>
__device__ __forceinline__ void fused_item(const Params& p, const Item& it, const uint4 (&qf)[G],
                                           unsigned int err0, unsigned char* smem) {
    if (it.n == 0) {
        if (it.t == 0) write_empty<G, D, NT>(p, it);
        return;
    }
    if (it.ns == 0) return;
    const LdsLayout L = lds_layout(G, D, p.split, NT);
    float* sc = reinterpret_cast<float*>(smem + L.scratch);
    int* pages = reinterpret_cast<int*>(smem + L.pages);
    HeadState* hs = reinterpret_cast<HeadState*>(smem + L.heads);

    __shared__ int s_fail;              // a wait of this workgroup gave up
    if (threadIdx.x == 0) s_fail = 0;
    load_pages<NT>(p, it, pages);
    __syncthreads();
    stream_scores<G, D, E, NT>(p, it, sc, pages, qf);
    __shared__ unsigned int s_err;      // thread 0's read, the same for the whole workgroup
    if (threadIdx.x == 0) s_err = err0;
    __syncthreads();
    // an earlier call left the workspace in error: its counts and records are
    // stale, so nothing of this call can be trusted
    if (s_err) {
        if (it.t == 0) poison_group<G, D, NT>(p, it);
        return;
    }
    // each head's wave publishes its record; a reader re-reads a record until it
    // is written, so neither a workgroup barrier nor the stores' completion is
    // needed before the count at the group barrier
    split_stats<G, NT, true>(p, it, sc, reinterpret_cast<uint64_t*>(smem + L.prefix), hs);
    if (!group_barrier(p, it, [&] { systematic_offsets<G, 1>(p, it, hs); })) {
        poison_group<G, D, NT>(p, it);      // the barrier's result is the same in every thread
        return;
    }
    prefix_and_sample<G, D, E, NT, KW, UL>(p, it, L, smem, kSpinLimit, &s_fail);
    finish_output<G, D, NT>(p, it, &s_fail);
}

// Four waves per SIMD (all 1024 splits of a batch-1, 8-KV-head, 32k-token
// step resident at once) where that fits without spilling registers.
template <int G, int D, typename E, int NT, int KW = 4, int UL = 8>
__device__ __forceinline__ void fused_one(const Params& p, int item, unsigned char* smem) {
    const Item at = item_coords(p, item);
    uint4 qf[G];
    priority_streaming();
    load_q<G, D, E, NT>(p, at.b, at.g, qf);
    const unsigned int err0 = p.sync->error;    // in flight with q, used after the K stream
    fused_item<G, D, E, NT, KW, UL>(p, make_item(p, item), qf, err0, smem);
}

template <int G, int D, typename E, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 3)))
void fused_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    int item = blockIdx.x;
    if (p.use_ticket) {
        __shared__ int s_item;
        if (threadIdx.x == 0) {
            const unsigned int k =
                __hip_atomic_fetch_add(&p.sync->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // the last ticket of the launch: every other one has been taken, so
            // the counter returns to zero for the next call
            if (k == (unsigned int)p.items - 1u)
                __hip_atomic_store(&p.sync->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // a counter that did not start at zero (a workspace never cleared):
            // no item, and the call is marked failed
            if (k >= (unsigned int)p.items)
                __hip_atomic_store(&p.sync->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_item = k < (unsigned int)p.items ? (int)k : -1;
        }
        __syncthreads();
        item = s_item;
        if (item < 0) return;
    }
    fused_one<G, D, E, NT>(p, item, smem);
}

template <int G, int D, typename E>
static const void* fused_fn() {
    return reinterpret_cast<const void*>(&fused_kernel<G, D, E, kThreads>);
}

template <int D, typename E>
static const void* fused_fn_g(int G) {
    switch (G) {
        case 1: return fused_fn<1, D, E>();
        case 2: return fused_fn<2, D, E>();
        case 4: return fused_fn<4, D, E>();
        case 7: return fused_fn<7, D, E>();
        case 8: return fused_fn<8, D, E>();
        default: return nullptr;
    }
}

static const void* fused_function(const Params& p, int dtype) {
    if (dtype == 0) return p.D == 64 ? fused_fn_g<64, Bf16>(p.G) : fused_fn_g<128, Bf16>(p.G);
    return p.D == 64 ? fused_fn_g<64, F32>(p.G) : fused_fn_g<128, F32>(p.G);
}

hipError_t launch_fused(const Params& p, int dtype, hipStream_t stream) {
    const void* fn = fused_function(p, dtype);
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = split_lds_bytes(p.G, p.D, p.split, kThreads);
    const hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    void* args[] = {const_cast<Params*>(&p)};
    return hipLaunchKernel(fn, dim3((unsigned)p.items), dim3(kThreads), args, lds, stream);
}

int fused_blocks_per_cu(const Params& p, int dtype) {
    const void* fn = fused_function(p, dtype);
    if (!fn) return 0;
    const size_t lds = split_lds_bytes(p.G, p.D, p.split, kThreads);
    if (allow_lds(fn, lds) != hipSuccess) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, lds) != hipSuccess) return 0;
    return n;
}

}  // namespace santa
