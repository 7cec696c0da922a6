// Fused SANTA decode kernel: the whole step of section 3.2 of "Stochastic
// Sparse Attention for Memory-Bound Inference" (score pass, global budget,
// parallel gather) in one launch, one workgroup per work item -- (sequence,
// KV head, split) -- with each split's scores kept in LDS across the global
// step.
//
// The only wait is for the statistics of the other splits of the same
// (sequence, KV head) group; take_item (santa_split.h) says how a workgroup
// gets its item so that every statistic it waits for is computed by a
// workgroup that runs.
#include "santa_split.h"

namespace santa {

// Four waves per SIMD (all 1024 splits of a batch-1, 8-KV-head, 32k-token
// step resident at once) where that fits without spilling registers.
template <int G, int D, typename E, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 3)))
void fused_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int item = take_item(p);
    if (item < 0) return;
    const Item at = item_coords(p, item);
    uint4 qf[G];
    priority_streaming();
    load_q<G, D, E, NT>(p, at.b, at.g, qf);
    // the first K batch in flight with q and the sequence length
    uint4 kd[ScoreStream<G, D, E, NT>::CB][ScoreStream<G, D, E, NT>::R];
    const bool pre = stream_first_batch<G, D, E, NT>(p, at, kd);
    const unsigned int err0 = p.sync->error;    // in flight with q, used after the K stream
    fused_item<G, D, E, NT>(p, make_item(p, item), err0, smem,
                            [&](const Item& it, float* sc, const int* pages) {
                                stream_scores<G, D, E, NT>(p, it, sc, pages, qf, kd, pre);
                            });
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
