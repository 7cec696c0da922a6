// S^2ANTA-flash decode kernel ("Stochastic Sparse Attention for Memory-Bound
// Inference", section 3.3): every split (tile) of a sequence gets a fixed,
// uniform share of the S samples, samples it from its own softmax as if it
// held all the mass, and the tiles' partial outputs are merged with weights
// Z_t / Z.  No workgroup waits for another, so one launch of one workgroup per
// work item serves any grid size.
//
// The merge without a barrier: the first split of a (sequence, query head) to
// get there publishes its maximum score r with a compare-and-swap, and every
// split adds w_t = Z_t(r) * mean_t and w_t into fp64 accumulation slots, where
// Z_t(r) = sum_{i in t} exp(s_i - r) (its local mass times exp(m_t - r)).  The
// ratio of the sums is sum_t (Z_t / Z) mean_t for any common r; fp64 keeps
// exp(m_t - r) finite for score spreads up to about 700.  The last split to
// count itself done divides, writes o and returns the slots to zero.
#include "santa_split.h"

namespace santa {

template <int G, int D, typename E, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 3)))
void flash_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = NT / 64;
    constexpr int DA = D + 2;                  // accumulator row: D sums, the weight, padding
    const Item at = item_coords(p, blockIdx.x);
    uint4 qf[G];
    load_q<G, D, E, NT>(p, at.b, at.g, qf);
    const unsigned int err0 = p.sync->error;    // nonzero: an earlier call left stale state
    const Item it = make_item(p, blockIdx.x);
    if (it.n == 0) {
        if (it.t == 0) write_empty<G, D, NT>(p, it);
        return;
    }
    if (it.ns == 0) return;
    const LdsLayout L = lds_layout(G, D, p.split, NT);
    float* sc = reinterpret_cast<float*>(smem + L.scratch);
    int* pages = reinterpret_cast<int*>(smem + L.pages);
    HeadState* hs = reinterpret_cast<HeadState*>(smem + L.heads);
    const uint64_t* prefix = reinterpret_cast<const uint64_t*>(smem + L.prefix);

    load_pages<NT>(p, it, pages);
    __syncthreads();
    uint4 kd[ScoreStream<G, D, E, NT>::CB][ScoreStream<G, D, E, NT>::R];
    stream_scores<G, D, E, NT>(p, it, sc, pages, qf, kd, false);
    __shared__ unsigned int s_err;      // thread 0's read, the same for the whole workgroup
    if (threadIdx.x == 0) s_err = err0;
    __syncthreads();
    if (s_err) {                // the reference maxima, slots and counts are not to be trusted
        if (it.t == 0) poison_group<G, D, NT>(p, it);
        return;
    }
    split_stats<G, NT, false>(p, it, sc, reinterpret_cast<uint64_t*>(smem + L.prefix), hs);
    __syncthreads();            // the scores' LDS is reused for the sampling below

    // this tile's budget and the idx positions of its samples
    const int per = p.S / it.Tb, rem = p.S % it.Tb;
    const int n_t = per + (it.t < rem ? 1 : 0);
    const int off = it.t * per + min(it.t, rem);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    double* acc_group = p.flash_acc + ((int64_t)it.b * p.Hkv + it.g) * kFlashSlots * G * DA;
    // lane 0: publishes or reads head h's reference maximum r (returned) and
    // puts the tile's sampling state of head h into hs[h]
    auto tile_setup = [&](int h) -> float {
        const int hq = it.g * G + h;
        unsigned long long* ref = p.flash_ref + (int64_t)it.b * p.Hq + hq;
        unsigned long long seen = 0ull;
        const unsigned long long mine = (1ull << 32) | __float_as_uint(hs[h].m_t);
        __hip_atomic_compare_exchange_strong(ref, &seen, mine, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        const float r = seen == 0ull ? hs[h].m_t : __uint_as_float((uint32_t)seen);
        // the tile's own CDF: edges P_j in units of its fixed-point masses
        const double z = fixed_to_double(prefix[h * p.split + it.ns - 1]);
        hs[h].w_lo = 0.0;
        hs[h].f = 1.0;
        hs[h].inv_f = 1.0;
        hs[h].z = z;
        hs[h].u0 = p.mode == 2 ? uniform01(p.seed, it.b, hq, 0ull, (uint64_t)(1 + it.t)) : 0.0;
        hs[h].m_lo = off;
        hs[h].m_hi = off + n_t;
        hs[h].n_targets = n_t;
        hs[h].stream = 1 + it.t;
        hs[h].off = off;
        return r;
    };
    auto slot_of = [&](int h) { return acc_group + ((it.t % kFlashSlots) * G + h) * DA; };
    // the tile's weight relative to the shared reference r, and 1/S_t, applied
    // to a head's sum of rows; the compare-and-swap's result is first needed
    // here, after the gather
    auto add_tile = [&](double* slot, const HeadState& st, float r, double& w, int col, const float* vals) {
        w = st.z * exp((double)st.m_t - (double)__shfl(r, 0, 64));
        const double scale = w / (double)n_t;
#pragma unroll
        for (int e = 0; e < D / 64; ++e) unsafeAtomicAdd(slot + col + e, scale * (double)vals[e]);
    };
    int h_first = wave;
    if constexpr (G > NW) {
        // two heads on this wave with few samples each: both tiles' states
        // first, then one gather of both heads' rows
        static_assert(G <= 2 * NW, "one or two heads per wave");
        const int hA = wave, hB = wave + NW;
        if (hB < G && n_t <= kFewTargets) {
            float rA = 0.0f, rB = 0.0f;
            if (lane == 0) {
                rA = tile_setup(hA);
                rB = tile_setup(hB);
            }
            wave_lds_sync();
            const HeadState stA = hs[hA], stB = hs[hB];
            double* slotA = slot_of(hA);
            double* slotB = slot_of(hB);
            double wA = 0.0, wB = 0.0;
            sample_pair<G, D, E>(p, it, stA, hA, n_t, stB, hB, n_t, L, smem,
                                 [&](int col, const float* vals) { add_tile(slotA, stA, rA, wA, col, vals); },
                                 [&](int col, const float* vals) { add_tile(slotB, stB, rB, wB, col, vals); });
            if (lane == 0) {
                unsafeAtomicAdd(slotA + D, wA);
                unsafeAtomicAdd(slotB + D, wB);
            }
            h_first = G;
        }
    }
    for (int h = h_first; h < G; h += NW) {
        float r = 0.0f;
        if (lane == 0) r = tile_setup(h);
        wave_lds_sync();
        const HeadState st = hs[h];
        double* slot = slot_of(h);
        double w = 0.0;
        // two keys at a time and four V loads per lane in flight: this kernel holds
        // more state across the sampling, and a tile samples few rows
        sample_head<G, D, E, 2, 4>(p, it, st, h, L, smem,
                                   [&](int col, const float* vals) { add_tile(slot, st, r, w, col, vals); });
        if (lane == 0) unsafeAtomicAdd(slot + D, w);
    }

    // the last split of the (sequence, KV head) to finish divides and clears
    __shared__ int s_last;
    wait_memory();
    __syncthreads();
    unsigned int* done = p.barrier + ((int64_t)it.b * p.Hkv + it.g) * kBarrierStride + 32;
    if (threadIdx.x == 0) {
        const unsigned int prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned int)it.Tb - 1u;
    }
    __syncthreads();
    if (!s_last) return;
    unsigned long long* acc_bits = reinterpret_cast<unsigned long long*>(acc_group);
    auto load_acc = [&](int k) {
        return __longlong_as_double((long long)__hip_atomic_load(acc_bits + k, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT));
    };
    float* o = p.o + ((int64_t)it.b * p.Hq + (int64_t)it.g * G) * D;
    for (int i = threadIdx.x; i < G * D; i += NT) {
        const int h = i / D, e = i - h * D;
        double num = 0.0, den = 0.0;
#pragma unroll
        for (int k = 0; k < kFlashSlots; ++k) {
            num += load_acc((k * G + h) * DA + e);
            den += load_acc((k * G + h) * DA + D);
        }
        o[i] = (float)(num / den);
    }
    __syncthreads();            // every thread has read the slots before they are cleared
    for (int i = threadIdx.x; i < kFlashSlots * G * DA; i += NT)
        __hip_atomic_store(acc_bits + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < G)
        __hip_atomic_store(p.flash_ref + (int64_t)it.b * p.Hq + it.g * G + threadIdx.x, 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int D, typename E>
static const void* flash_fn() {
    return reinterpret_cast<const void*>(&flash_kernel<G, D, E, kThreads>);
}

template <int D, typename E>
static const void* flash_fn_g(int G) {
    switch (G) {
        case 1: return flash_fn<1, D, E>();
        case 2: return flash_fn<2, D, E>();
        case 4: return flash_fn<4, D, E>();
        case 7: return flash_fn<7, D, E>();
        case 8: return flash_fn<8, D, E>();
        default: return nullptr;
    }
}

// Workgroups of the flash kernel one compute unit holds at once (0: unknown).
int flash_blocks_per_cu(const Params& p, int dtype) {
    const void* fn = dtype == 0 ? (p.D == 64 ? flash_fn_g<64, Bf16>(p.G) : flash_fn_g<128, Bf16>(p.G))
                                : (p.D == 64 ? flash_fn_g<64, F32>(p.G) : flash_fn_g<128, F32>(p.G));
    if (!fn) return 0;
    const size_t lds = split_lds_bytes(p.G, p.D, p.split, kThreads);
    if (allow_lds(fn, lds) != hipSuccess) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, lds) != hipSuccess) return 0;
    return n;
}

template <int G, int D, typename E>
static hipError_t launch_flash_t(const Params& p, hipStream_t stream) {
    const size_t lds = split_lds_bytes(G, D, p.split, kThreads);
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(&flash_kernel<G, D, E, kThreads>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((flash_kernel<G, D, E, kThreads>), dim3((unsigned)p.items), dim3(kThreads), lds, stream, p);
    return hipGetLastError();
}

template <int D, typename E>
static hipError_t launch_flash_d(const Params& p, hipStream_t stream) {
    switch (p.G) {
        case 1: return launch_flash_t<1, D, E>(p, stream);
        case 2: return launch_flash_t<2, D, E>(p, stream);
        case 4: return launch_flash_t<4, D, E>(p, stream);
        case 7: return launch_flash_t<7, D, E>(p, stream);
        case 8: return launch_flash_t<8, D, E>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_flash(const Params& p, int dtype, hipStream_t stream) {
    if (dtype == 0) return p.D == 64 ? launch_flash_d<64, Bf16>(p, stream) : launch_flash_d<128, Bf16>(p, stream);
    return p.D == 64 ? launch_flash_d<64, F32>(p, stream) : launch_flash_d<128, F32>(p, stream);
}

}  // namespace santa
