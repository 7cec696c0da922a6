// The phases of one SANTA work item -- one (sequence b, KV head g, split t of
// `split` consecutive keys) -- shared by the fused decode kernel and by the
// two-kernel path (score pass + sample pass).
//
//   stream_scores  exact scores q_h . k_i / sqrt(d) of the split's keys for the
//                  G query heads of the group, from one read of every K row
//                  ("Stochastic Sparse Attention for Memory-Bound Inference",
//                  section 2, Eq. 1; section 3.2, Pass 1);
//   split_stats    per head: the split's maximum m_t, the fixed-point masses
//                  e_i = exp(s_i - m_t), their in-split prefix P_i and total
//                  l_t (the tile partition function of section 3.2, Pass 1),
//                  and the record (m_t, l_t) for the other workgroups of the
//                  sequence;
//   group_barrier  waits until every split of the sequence has published;
//   prefix_and_sample
//                  per head (one wave): merges the splits' statistics to a
//                  common maximum M (online softmax merge), forms the exact
//                  prefix W of split masses and the total Z (the global
//                  partition function of section 3.2, step 2) and the range of
//                  targets this split owns, then samples them by inverse CDF
//                  (section 2.1 and Appendix A.4), merging the sorted targets
//                  with the split's sorted CDF edges, and gathers-and-adds the
//                  sampled V rows with duplicates counted (section 2, Eq. 2-3).
#pragma once

#include "santa_device.h"
#include "santa_internal.h"

namespace santa {

struct Item {
    int b, g, t;   // sequence, KV head, split
    int n;         // tokens of sequence b
    int key0;      // first key of the split
    int ns;        // keys in the split (0: past the end of the sequence)
    int Tb;        // splits of sequence b
};

// Work item numbering (Params::item_order).
//   kOrderTokenBlocks (fused kernel, and flash grids larger than the device;
//     T a multiple of 8): workgroups are handed to the 8 XCDs round-robin by
//     index, so item i runs on XCD i mod 8; XCD x takes the splits t = x,
//     x + 8, ... and, for each, the B * Hkv groups one after another:
//     item = 8 * ((t / 8) * B * Hkv + b * Hkv + g) + t mod 8.
//     The KV heads of a token-major cache share every token row, so the
//     workgroups reading one stretch of rows run together on one XCD and the
//     rows are fetched together (1.4 us less K stream on the Llama-shaped
//     step than with the order below); every group still streams across the
//     whole launch, so the groups reach their barriers together at the end of
//     the K stream and their latency-bound tails run side by side.
//   kOrderHeadFastest (fused and flash kernels otherwise): item = t * B *
//     Hkv + b * Hkv + g, with the same side-by-side tails.
//   kOrderSplitFastest (two-kernel path, whose grids are larger than the
//     device): item = (b * Hkv + g) * T + t, so that a group's splits run close
//     together in time.
__device__ __forceinline__ Item item_coords(const Params& p, int item) {
    Item it;
    int grp;
    const int ng = p.B * p.Hkv;
    if (p.item_order == kOrderTokenBlocks) {
        const int x = item & 7;
        const int s8 = item >> 3;
        const int tb = s8 / ng;
        it.t = 8 * tb + x;
        grp = s8 - tb * ng;
    } else if (p.item_order == kOrderHeadFastest) {
        it.t = item / ng;
        grp = item - it.t * ng;
    } else {
        it.t = item % p.T;
        grp = item / p.T;
    }
    it.g = grp % p.Hkv;
    it.b = grp / p.Hkv;
    return it;
}

__device__ __forceinline__ Item make_item(const Params& p, int item) {
    Item it = item_coords(p, item);
    it.n = seq_len_of(p, it.b);
    it.key0 = it.t * p.split;
    it.ns = max(0, min(p.split, it.n - it.key0));
    it.Tb = (it.n + p.split - 1) / p.split;
    return it;
}

// Per query head of the work item, kept in LDS.
struct HeadState {
    double w_lo;    // mass of the sequence's splits before this one (W_t)
    double z;       // total mass Z of the sequence
    double f;       // exp(m_t - M)
    double inv_f;   // exp(M - m_t), the split's scale back to its own masses
    double u0;      // systematic offset
    float m_t;      // this split's maximum score
    float l_t;      // this split's mass, sum of exp(s_i - m_t)
    int m_lo;       // targets [m_lo, m_hi) fall into this split
    int m_hi;
    int lastpos;    // last key of positive mass in the split
    int n_targets;  // S of the target sequence (S, or the tile's budget in flash)
    int stream;     // Philox stream of its draws (0, or 1 + t in flash)
    int off;        // idx position of the sequence's first target (0, or the tile's in flash)
};

// Byte offsets of the dynamic LDS of a split workgroup.
struct LdsLayout {
    uint32_t scratch;   // scores fp32 [G][split]; after the statistics, per wave
                        // a TargetArea (merge targets and the sampled-key list)
    uint32_t prefix;    // u64 [G][split] in-split inclusive prefix of fixed-point masses
    uint32_t pages;     // int [split/16 + 1] physical pages of the split (paged caches)
    uint32_t heads;     // HeadState [G]
    uint32_t total;
};

// Per wave, for one chunk of at most kTargetChunk targets of one head.
struct TargetArea {
    double tau[kTargetChunk];      // targets scaled by Z
    int mark[kTargetChunk];        // per target: the list entry (multinomial) or the key
                                   // (stratified/systematic) whose first target it is, else
                                   // -1; the latter then holds each entry's first target
    int lkey[kTargetChunk];        // distinct sampled keys, ascending
    unsigned int lcnt[kTargetChunk];   // samples of each of them
};

__host__ __device__ inline LdsLayout lds_layout(int G, int D, int split, int nt) {
    const int nw = nt / 64;
    size_t scratch = (size_t)G * split * 4;
    if ((size_t)nw * sizeof(TargetArea) > scratch) scratch = (size_t)nw * sizeof(TargetArea);
    LdsLayout L;
    L.scratch = 0;
    L.prefix = (uint32_t)((scratch + 15) & ~(size_t)15);
    L.pages = L.prefix + (uint32_t)(G * split * 8);
    L.heads = (L.pages + (uint32_t)((split / 16 + 1) * 4) + 15) & ~15u;
    L.total = L.heads + (uint32_t)(G * sizeof(HeadState));
    return L;
}

// ---------------------------------------------------------------------------
// KV rows
// ---------------------------------------------------------------------------

// Physical pages of the split's keys (paged caches), clamped into the cache so
// that a bad table entry cannot address outside it.
template <int NT>
__device__ __forceinline__ void load_pages(const Params& p, const Item& it, int* pages) {
    if (p.page_shift < 0 || it.ns == 0) return;
    const int first = it.key0 >> p.page_shift;
    const int last = (it.key0 + it.ns - 1) >> p.page_shift;
    const int32_t* bt = p.block_table + (int64_t)it.b * p.pages_per_seq;
    for (int k = threadIdx.x; k <= last - first; k += NT) {
        const int pg = bt[first + k];
        pages[k] = min(max(pg, 0), p.num_pages - 1);
    }
}

// Element offset of key `local` of the split (KV head g included).
__device__ __forceinline__ int64_t row_offset(const Params& p, const Item& it, int local,
                                              const int* pages) {
    const int key = it.key0 + local;
    int64_t off;
    if (p.page_shift < 0) {
        off = (int64_t)it.b * p.stride_seq + (int64_t)key * p.stride_tok;
    } else {
        const int pg = pages[(key >> p.page_shift) - (it.key0 >> p.page_shift)];
        off = (int64_t)pg * p.stride_seq + (int64_t)(key & ((1 << p.page_shift) - 1)) * p.stride_tok;
    }
    return off + (int64_t)it.g * p.stride_head;
}

// ---------------------------------------------------------------------------
// Scores: stream the split's K rows once for all G heads.
// A K row of d elements is read by LPR = d*e/16 lanes with 16-byte loads; a
// wave-wide load covers RPL = 64/LPR rows, and a 16-row chunk takes R = 16/RPL
// loads per lane.  A wave issues the loads of CB chunks (16 loads per lane)
// before using any of them.  Each lane forms R*G partial dot products; a
// reduce-scatter across the row's lanes leaves every lane owning whole scores.
//
// The loads carry no branches (a row past the split re-reads the split's first
// row), and the first batch is straight-line code after the q loads, so the
// compiler waits for q and then for each chunk in turn instead of for every
// load before the first K load is even issued.
// ---------------------------------------------------------------------------
template <int G, int D, typename E, int NT>
struct ScoreStream {
    static constexpr int NW = NT / 64;
    static constexpr int LPR = D * E::bytes / 16;
    static constexpr int RPL = 64 / LPR;
    static constexpr int R = 16 / RPL;
    static constexpr int CB = (16 / R) > 0 ? 16 / R : 1;
    static constexpr int NV = R * G;
    static constexpr int NVP = (NV + LPR - 1) / LPR * LPR;
    static constexpr int M = NVP / LPR;
    static_assert(LPR >= 2 && LPR <= 32 && 16 % RPL == 0, "row shape");

    // Loads of the NC chunks base, base + NW, ... (16 rows each).
    template <int NC>
    __device__ __forceinline__ static void issue(const Params& p, const Item& it, const int* pages,
                                                 const char* kbase, int64_t first, int base, int nchunks,
                                                 int c, int li, uint4 (&kd)[NC][R]) {
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int ch = base + k * NW;
            const int r0 = ch << 4;
            // a 16-row chunk never straddles a page (pages >= 16 rows, r0 % 16 == 0)
            const int64_t off = (ch < nchunks) ? row_offset(p, it, r0, pages) : first;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int rr = r * RPL + c;
                const bool ok = ch < nchunks && r0 + rr < it.ns;
                const int64_t o = ok ? off + (int64_t)rr * p.stride_tok : first;
                kd[k][r] = load16_stream(kbase + o * E::bytes + li * 16);
            }
        }
    }

    template <int NC>
    __device__ __forceinline__ static void score(const Params& p, const Item& it, float* sc, int base,
                                                 int nchunks, int c, int li, const uint4 (&qf)[G],
                                                 const uint4 (&kd)[NC][R]) {
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int ch = base + k * NW;
            if (ch < nchunks) {
                float acc[NVP];
#pragma unroll
                for (int j = 0; j < NVP; ++j) acc[j] = 0.0f;
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[r * G + h] = E::dot16(kd[k][r], qf[h], 0.0f);
                row_reduce_scatter<LPR, NVP>(acc, li);
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    const int vi = li * M + j;
                    if (vi < NV) {
                        const int r = vi / G;
                        const int h = vi - r * G;
                        const int local = (ch << 4) + r * RPL + c;
                        if (local < it.ns) sc[h * p.split + local] = acc[j] * p.scale;
                    }
                }
            }
        }
    }
};

// This lane's 16-byte pieces of the G query rows of KV head g of sequence b
// (the piece li = lane % LPR of each row, as stream_scores consumes them).
// Issued at the start of a workgroup, before the sequence length is known, so
// that both loads share one memory round trip.
template <int G, int D, typename E, int NT>
__device__ __forceinline__ void load_q(const Params& p, int b, int g, uint4 (&qf)[G]) {
    const int li = (threadIdx.x & 63) % ScoreStream<G, D, E, NT>::LPR;
    const char* qb = reinterpret_cast<const char*>(p.q) + (((int64_t)b * p.Hq + (int64_t)g * G) * D) * E::bytes +
                     li * 16;
#pragma unroll
    for (int h = 0; h < G; ++h) qf[h] = load16(qb + (int64_t)h * D * E::bytes);
}

// The first batch of a split's K loads in a contiguous cache, issued before
// the sequence length is known: its rows are bounded by the cache's n_max rows
// instead of by the sequence (every such row is inside the cache), and the
// scores of rows past the sequence are never written.  Returns whether it
// issued them: only in the resident fused launch (a split past its sequence
// would read its batch for nothing, which in batches of short sequences costs
// more than the round trip saved) and not for paged caches, whose rows need
// the split's pages.
template <int G, int D, typename E, int NT>
__device__ __forceinline__ bool stream_first_batch(const Params& p, const Item& at,
                                                   uint4 (&kd)[ScoreStream<G, D, E, NT>::CB][ScoreStream<G, D, E, NT>::R]) {
    using SS = ScoreStream<G, D, E, NT>;
    if (p.page_shift >= 0 || p.use_ticket) return false;
    Item sp = at;
    sp.key0 = at.t * p.split;
    sp.ns = max(0, min(p.split, p.n_max - sp.key0));
    const int lane = threadIdx.x & 63;
    SS::template issue<SS::CB>(p, sp, nullptr, reinterpret_cast<const char*>(p.k), row_offset(p, sp, 0, nullptr),
                               threadIdx.x >> 6, (sp.ns + 15) >> 4, lane / SS::LPR, lane % SS::LPR, kd);
    return true;
}

// `kd`/`pre`: the first batch as stream_first_batch issued it, if it did.
template <int G, int D, typename E, int NT>
__device__ __forceinline__ void stream_scores(const Params& p, const Item& it, float* sc,
                                              const int* pages, const uint4 (&qf)[G],
                                              uint4 (&kd)[ScoreStream<G, D, E, NT>::CB][ScoreStream<G, D, E, NT>::R],
                                              bool pre) {
    using SS = ScoreStream<G, D, E, NT>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane / SS::LPR;
    const int li = lane % SS::LPR;
    const char* kbase = reinterpret_cast<const char*>(p.k);
    const int nchunks = (it.ns + 15) >> 4;
    const int64_t first = row_offset(p, it, 0, pages);

    if (!pre) SS::template issue<SS::CB>(p, it, pages, kbase, first, wave, nchunks, c, li, kd);
    SS::template score<SS::CB>(p, it, sc, wave, nchunks, c, li, qf, kd);
    for (int base = wave + SS::NW * SS::CB; base < nchunks; base += SS::NW * SS::CB) {
        SS::template issue<SS::CB>(p, it, pages, kbase, first, base, nchunks, c, li, kd);
        SS::template score<SS::CB>(p, it, sc, base, nchunks, c, li, qf, kd);
    }
    priority_tail();
}

// Record of split t of query head hq of sequence b: one 64-bit word
// (l_t bits << 32 | m_t bits), written and read as a single atomic word.  A
// split with keys has l_t >= 1 (its maximum contributes exp(0)), so a record
// is written exactly when its high half is nonzero; records are zero between
// calls.
__device__ __forceinline__ unsigned long long* record_of(const Params& p, int b, int hq, int t) {
    return p.records + ((int64_t)b * p.Hq + hq) * p.T + t;
}

// ---------------------------------------------------------------------------
// Split statistics and the in-split prefix (one wave per head).  Lane L owns
// keys [L*EPT, (L+1)*EPT), EPT = split/64 in {1, 2, 4, 8, 16}, read and
// written with vector LDS accesses.  With PUBLISH the head's wave stores its
// record as soon as m_t and l_t are known (no workgroup barrier first: a
// reader re-reads a record until it is written), then writes the prefix.
// ---------------------------------------------------------------------------
template <int G, int NT, int EPT, bool PUBLISH>
__device__ __forceinline__ void split_stats_t(const Params& p, const Item& it, const float* sc,
                                              uint64_t* prefix, HeadState* hs) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int split = EPT * 64;
    const int i0 = lane * EPT;
    const int n_own = max(0, min(EPT, it.ns - i0));    // keys of this lane inside the split
    for (int h = wave; h < G; h += NW) {
        float s[EPT];
        const float* row = sc + h * split + i0;
        if constexpr (EPT >= 4) {
#pragma unroll
            for (int k = 0; k < EPT; k += 4) {
                const float4 v = *reinterpret_cast<const float4*>(row + k);
                s[k] = v.x; s[k + 1] = v.y; s[k + 2] = v.z; s[k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < EPT; ++k) s[k] = row[k];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < EPT; ++k)
            if (k < n_own) mx = fmaxf(mx, s[k]);
        mx = wave_max_f32(mx);
        // fixed-point masses and their in-lane inclusive prefix
        uint64_t run[EPT];
        uint64_t acc = 0;
        int lastpos = -1;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const uint64_t e = (k < n_own) ? fixed_mass(mass_exp(s[k] - mx)) : 0;
            if (e) lastpos = i0 + k;
            acc += e;
            run[k] = acc;
        }
        const uint64_t incl = wave_scan_add_u64(acc);
        const uint64_t excl = incl - acc;
        const uint64_t total = lane_u64(incl, 63);
        lastpos = wave_max_i32(lastpos);
        if (lane == 0) {
            const float l = (float)fixed_to_double(total);
            hs[h].m_t = mx;
            hs[h].l_t = l;
            hs[h].lastpos = lastpos;
            if constexpr (PUBLISH) {
                const unsigned long long r = (unsigned long long)__float_as_uint(l) << 32 | __float_as_uint(mx);
                __hip_atomic_store(record_of(p, it.b, it.g * G + h, it.t), r, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        uint64_t* ph = prefix + h * split + i0;
        if constexpr (EPT >= 2) {
#pragma unroll
            for (int k = 0; k < EPT; k += 2)
                *reinterpret_cast<ulonglong2*>(ph + k) = make_ulonglong2(excl + run[k], excl + run[k + 1]);
        } else {
            ph[0] = excl + run[0];
        }
    }
}

template <int G, int NT, bool PUBLISH>
__device__ __forceinline__ void split_stats(const Params& p, const Item& it, const float* sc,
                                            uint64_t* prefix, HeadState* hs) {
    switch (p.split) {
        case 64: split_stats_t<G, NT, 1, PUBLISH>(p, it, sc, prefix, hs); break;
        case 128: split_stats_t<G, NT, 2, PUBLISH>(p, it, sc, prefix, hs); break;
        case 256: split_stats_t<G, NT, 4, PUBLISH>(p, it, sc, prefix, hs); break;
        case 512: split_stats_t<G, NT, 8, PUBLISH>(p, it, sc, prefix, hs); break;
        default: split_stats_t<G, NT, 16, PUBLISH>(p, it, sc, prefix, hs); break;
    }
}

// The systematic offsets U of the item's G heads, by the wave WAVE (lane h
// for head h); they depend on nothing the other splits compute.
template <int G, int WAVE>
__device__ __forceinline__ void systematic_offsets(const Params& p, const Item& it, HeadState* hs) {
    if (p.mode == 2 && (threadIdx.x >> 6) == WAVE) {
        const int lane = threadIdx.x & 63;
        const double u0 = uniform01(p.seed, it.b, it.g * G + (lane % G), 0ull);
        if (lane < G) hs[lane].u0 = u0;
    }
}

// ---------------------------------------------------------------------------
// Waits (one lane) until the device-coherent word *w satisfies `ready`, one
// load at a time (more loads in flight from every waiting workgroup slowed the
// memory traffic of the workgroups still streaming more than they saved).
// Returns false after kSpinLimit loads.
// ---------------------------------------------------------------------------
template <typename Ready>
__device__ __forceinline__ bool poll_until(const unsigned int* w, Ready&& ready) {
    for (int iter = 0; iter < kSpinLimit; ++iter) {
        if (ready(__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// ---------------------------------------------------------------------------
// Barrier of the Tb splits of one (sequence, KV head) in the fused kernel.
// Each split counts itself in once its records are written; the last one
// resets the count and raises the 16 flag copies; the others poll one copy
// each, so waiting adds almost no memory traffic.  The flags are cleared by
// the group's last split at the end of the call (finish_output).  `overlap()`
// runs on every thread meanwhile (thread 0 after its wait).  Returns false if
// the bounded wait gave up.
// ---------------------------------------------------------------------------
template <typename Overlap>
__device__ __forceinline__ bool group_barrier(const Params& p, const Item& it, Overlap&& overlap) {
    __shared__ int s_ok;
    if (threadIdx.x == 0) {
        unsigned int* bar = p.barrier + ((int64_t)it.b * p.Hkv + it.g) * kBarrierStride;
        int ok = 1;
        const unsigned int prev = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (unsigned int)it.Tb - 1u) {
            __hip_atomic_store(bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int c = 0; c < kFlagCopies; ++c)
                __hip_atomic_store(bar + 32 * (2 + c), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const unsigned int* flag = bar + 32 * (2 + blockIdx.x % kFlagCopies);
            if (!poll_until(flag, [](unsigned int v) { return v != 0u; })) {
                ok = 0;
                __hip_atomic_store(&p.sync->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        s_ok = ok;
    }
    overlap();      // the other waves' independent work while thread 0 waits
    __syncthreads();
    return s_ok != 0;
}

// ---------------------------------------------------------------------------
// Targets of §2 / §2.1 scaled by Z: tau_m = t_m * Z, non-decreasing in m.
//   multinomial  t_m = m-th smallest of S uniforms (sorted in the workspace);
//   stratified   t_m = (m + U_m) / S;
//   systematic   t_m = (m + U_0) / S.
// Counting and merging use this one function, so both see the same bits.
// ---------------------------------------------------------------------------
// MODE is a template argument so that no path evaluates another mode's
// targets (the compiler would otherwise compute the stratified Philox draw
// speculatively for every target).  In S^2ANTA-flash a tile's S_t targets
// are numbered off .. off + S_t - 1 in idx and drawn from the tile's stream;
// for SANTA off = 0, S_t = S and the stream is 0.
template <int MODE>
struct TargetSeq {
    const double* sorted;
    double u0;
    double z;
    double inv_s;   // 1 / S, rounded once
    uint64_t seed;
    int S, off, stream, b, hq;
    __device__ __forceinline__ double tau(int m) const {
        const int j = m - off;
        double t;
        if constexpr (MODE == 0) {
            t = sorted[m];
        } else if constexpr (MODE == 1) {
            t = ((double)j + uniform01(seed, b, hq, (uint64_t)j, (uint64_t)stream)) * inv_s;
        } else {
            t = ((double)j + u0) * inv_s;
        }
        return t * z;
    }
};

// Number of m in [0, S) with tau_m < x (tau non-decreasing in m).
template <int MODE>
__device__ __forceinline__ int count_below(const TargetSeq<MODE>& ts, double x, int lane) {
    if constexpr (MODE != 0) {
        // lane-parallel scan upward in windows of 64 targets
        for (int base = 0;; base += 64) {
            const int m = base + lane;
            const bool below = m < ts.S && ts.tau(m) < x;
            const unsigned long long bal = __ballot(below);
            if (bal != ~0ull) return base + __popcll(bal);
        }
    } else {
        // multinomial: 64-ary search over the sorted targets, one probe per lane
        int lo = 0, hi = ts.S;
        while (hi > lo) {
            const int len = hi - lo;
            const int step = (len + 63) >> 6;
            const int pos = lo + (lane + 1) * step - 1;
            const bool below = (pos < hi) && (ts.tau(pos) < x);
            const int k = __popcll(__ballot(below));
            if (step == 1) return lo + k;
            const int nlo = lo + k * step;
            hi = min(hi, lo + (k + 1) * step - 1);
            lo = nlo;
        }
        return lo;
    }
}

template <int MODE>
__device__ __forceinline__ TargetSeq<MODE> target_seq(const Params& p, int b, int hq, double z, double u0,
                                                      int n_targets = -1, int off = 0, int stream = 0) {
    TargetSeq<MODE> ts;
    ts.sorted = p.targets + ((int64_t)b * p.Hq + hq) * p.S;
    ts.seed = p.seed;
    ts.S = n_targets < 0 ? p.S : n_targets;
    ts.inv_s = n_targets < 0 ? p.inv_S : 1.0 / (double)n_targets;
    ts.off = off;
    ts.stream = stream;
    ts.b = b;
    ts.hq = hq;
    ts.u0 = u0;
    ts.z = z;
    return ts;
}

// Targets [m_lo, m_hi) of split t: those with W_t <= tau_m < W_{t+1}; the last
// split of positive mass also takes targets that round to tau >= Z.  For
// stratified and systematic targets tau_m lies in stratum m of [0, Z), so the
// count below x is within one of x * S / Z: lanes 0-31 test the 32 targets
// around that estimate for W_t, lanes 32-63 those for W_{t+1}, and one ballot
// gives both counts (a full scan covers a window that misses the boundary).
template <int MODE>
__device__ __forceinline__ void target_range(const Params& p, int b, int hq, double z, double u0,
                                             double w_lo, double w_hi, bool last, int lane,
                                             int* m_lo, int* m_hi) {
    const TargetSeq<MODE> ts = target_seq<MODE>(p, b, hq, z, u0);
    if constexpr (MODE == 0) {
        *m_lo = count_below(ts, w_lo, lane);
        *m_hi = last ? p.S : count_below(ts, w_hi, lane);
    } else {
        const bool upper = lane >= 32;
        const double x = upper ? w_hi : w_lo;
        // an estimate within far less than one target of the count: a fast reciprocal will do
        const double est = x * ((double)p.S * (double)__builtin_amdgcn_rcpf((float)z)) - (MODE == 2 ? u0 : 0.0);
        const int base = (int)ceil(fmin(fmax(est, -1.0), (double)p.S)) - 16;
        const int m = base + (lane & 31);
        // targets below index 0 do not exist: count them as below x, so that
        // the count is the index of the first target at or above x
        const bool below = m < 0 || (m < p.S && ts.tau(m) < x);
        const unsigned long long bal = __ballot(below);
        const int base_lo = __builtin_amdgcn_readlane(base, 0);
        const int base_hi = __builtin_amdgcn_readlane(base, 32);
        const uint32_t lo_bits = (uint32_t)bal, hi_bits = (uint32_t)(bal >> 32);
        int c_lo = base_lo + __popc(lo_bits);
        int c_hi = base_hi + __popc(hi_bits);
        // the window holds the boundary iff its first target is below x and its last is not
        if (!((lo_bits & 1u) && !(lo_bits >> 31))) c_lo = count_below(ts, w_lo, lane);
        if (!((hi_bits & 1u) && !(hi_bits >> 31))) c_hi = count_below(ts, w_hi, lane);
        *m_lo = c_lo;
        *m_hi = last ? p.S : c_hi;
    }
}

// idx of the chunk's na targets from the marks of the distinct-key list: target
// i belongs to the list entry with the largest mark at or below i (target 0 is
// always marked); lane l scans targets [4l, 4l + 4), so every lane stores.
__device__ __forceinline__ void write_idx_from_marks(TargetArea* ta, int na, int32_t* idx_row, int key0,
                                                     int lane) {
    static_assert(kTargetChunk <= 4 * 64, "four targets per lane");
    int v[4], run = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = lane * 4 + k;
        run = max(run, i < na ? ta->mark[i] : -1);
        v[k] = run;
    }
    int before = __shfl_up(wave_scan_max_i32(run), 1, 64);
    if (lane == 0) before = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = lane * 4 + k;
        if (i < na) idx_row[i] = key0 + ta->lkey[max(before, v[k])];
    }
    wave_lds_sync();
}

// ---------------------------------------------------------------------------
// Inverse-CDF sampling of multinomial targets (the sorted uniforms)
// [m0, m0 + na) of one head (one wave): each target tau goes to the first key
// j of the split whose upper edge C_{j+1} = W_t + exp(m_t - M) * P_j exceeds
// it (half-open intervals, Appendix A.4); a target past every edge (rounding)
// goes to the split's last key of positive mass.  Writes idx and leaves the
// distinct keys with their sample counts, ascending, in ta->lkey / ta->lcnt;
// returns how many.
//   few targets (<= 8): one at a time -- a ballot over the lanes' last edges
//     (lane l owns keys [l*ept, (l+1)*ept)) finds the lane that owns the key,
//     one LDS read per lane finds the key;
//   more: by keys, 64 at a time (lane l takes key j0 + l): each lane counts
//     the targets below its key's upper edge (+inf for the last key of
//     positive mass) by a binary search over the chunk's targets, and the
//     key holds the targets between that count and its left neighbour's.
//     Every key with targets marks its first one, and a max-scan over the
//     marks gives each target its key, so idx is written by all lanes at once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int sample_chunk_multinomial(const Params& p, const Item& it, const HeadState& st,
                                                        int hq, const uint64_t* ph, TargetArea* ta, int m0, int na,
                                                        int lane) {
    const int ns = it.ns;
    int32_t* idx_row = p.idx + ((int64_t)it.b * p.Hq + hq) * p.S + m0;
    const TargetSeq<0> ts = target_seq<0>(p, it.b, hq, st.z, st.u0, st.n_targets, st.off, st.stream);
    const int lastpos = max(st.lastpos, 0);
    auto edge = [&](int j) { return st.w_lo + st.f * fixed_to_double(ph[j]); };
    if (na <= 8) {
        const int ept = p.split >> 6;
        double my_tau = 0.0;
        if (lane < na) my_tau = ts.tau(m0 + lane);
        const int i0 = lane * ept;
        const int n_own = max(0, min(ept, ns - i0));
        const double lane_hi = n_own > 0 ? edge(i0 + n_own - 1) : INFINITY;
        int prev = -1, nlist = 0;
        for (int k = 0; k < na; ++k) {
            const double t = __shfl(my_tau, k, 64);
            // lanes whose every key's interval ends at or below t
            const int c = __popcll(__ballot(lane_hi <= t));
            int local;
            if (c * ept >= ns) {
                local = lastpos;
            } else {
                const bool le = lane < ept && c * ept + lane < ns && edge(c * ept + lane) <= t;
                local = c * ept + __popcll(__ballot(le));
            }
            if (lane == 0) {
                idx_row[k] = it.key0 + local;
                if (local == prev) {
                    ta->lcnt[nlist - 1] += 1u;
                } else {
                    ta->lkey[nlist] = local;
                    ta->lcnt[nlist] = 1u;
                }
            }
            if (local != prev) ++nlist;
            prev = local;
        }
        wave_lds_sync();
        return nlist;
    }
    for (int k = lane; k < na; k += 64) {
        ta->tau[k] = ts.tau(m0 + k);
        ta->mark[k] = -1;
    }
    wave_lds_sync();
    const double* tau = ta->tau;
    const int nkeys = min(ns, lastpos + 1);      // keys after lastpos take nothing
    const unsigned long long below = (1ull << lane) - 1ull;
    int carry = 0;          // count below the upper edge of the key before j0
    int nlist = 0;
    for (int j0 = 0; j0 < nkeys; j0 += 64) {
        const int j = j0 + lane;
        int c = na;
        if (j < lastpos) {
            const double u = edge(j);
            int lo = 0, hi = na;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (tau[mid] < u) lo = mid + 1;
                else hi = mid;
            }
            c = lo;
        }
        int first = __shfl_up(c, 1, 64);
        if (lane == 0) first = carry;
        carry = __shfl(c, 63, 64);
        const bool has = j < nkeys && c > first;
        const unsigned long long bal = __ballot(has);
        if (has) {
            const int pos = nlist + __popcll(bal & below);
            ta->lkey[pos] = j;
            ta->lcnt[pos] = (unsigned)(c - first);
            ta->mark[first] = pos;
        }
        nlist += __popcll(bal);
    }
    wave_lds_sync();
    write_idx_from_marks(ta, na, idx_row, it.key0, lane);
    return nlist;
}

// ---------------------------------------------------------------------------
// Inverse-CDF sampling of stratified or systematic targets [m0, m0 + na) of
// one head (one wave), every key at once.  Target m lies in stratum m of
// [0, Z), so the number of targets below a key's upper edge u is a closed
// form in u (u * S / Z, less the systematic offset) up to rounding, which can
// move it by one only where a target lies within about 1e-12 of u; one read
// of the targets on either side settles it.  Lane l owns keys [l*ept,
// (l+1)*ept) and counts the targets below the upper edge of each of them and
// of key l*ept - 1, KW keys at a time with their LDS reads issued together
// (the last key of positive mass counts every target, so that targets past
// all edges by rounding go to it).  Key j holds the targets between the count
// of key j-1 and its own (half-open intervals, Appendix A.4) and marks the
// first of them with its index.  Keys ascend with their targets, so a
// max-scan over the marks gives every target its key, and the marked targets,
// compacted in order, are the distinct keys; each holds the targets up to the
// next mark.
// ---------------------------------------------------------------------------
template <int MODE>
struct StrataCounter {
    const uint64_t* ph;
    const double* tau;
    double w_lo, f, s_over_z, shift;
    int m0, na, lastpos, last_key;

    // counts for keys j[0..N) (any j; keys at or past lastpos count na)
    template <int N>
    __device__ __forceinline__ void operator()(const int (&j)[N], int (&c)[N]) const {
        uint64_t pv[N];
#pragma unroll
        for (int q = 0; q < N; ++q) pv[q] = ph[min(max(j[q], 0), last_key)];
        double u[N];
        int i[N];
#pragma unroll
        for (int q = 0; q < N; ++q) {
            u[q] = w_lo + f * fixed_to_double(pv[q]);
            const double est = u[q] * s_over_z - shift;
            const double e = fmin(fmax(MODE == 2 ? ceil(est) : floor(est), (double)m0), (double)(m0 + na));
            i[q] = (int)e - m0;
        }
        double lo[N], hi[N];
#pragma unroll
        for (int q = 0; q < N; ++q) {
            lo[q] = tau[max(i[q] - 1, 0)];
            hi[q] = tau[min(i[q], na - 1)];
        }
#pragma unroll
        for (int q = 0; q < N; ++q) {
            int r = i[q];
            if (r > 0 && lo[q] >= u[q]) r -= 1;
            else if (r < na && hi[q] < u[q]) r += 1;
            c[q] = j[q] >= lastpos ? na : r;
        }
    }
};

// ---------------------------------------------------------------------------
// Inverse-CDF sampling of at most 64 targets [m0, m0 + na) of one head (one
// wave), one target per lane.  Target tau goes to the first key j of the split
// whose upper edge W_t + exp(m_t - M) * P_j exceeds it, i.e. with P_j above
// x = (tau - W_t) / exp(m_t - M) in the split's own fixed-point mass scale
// (half-open intervals, Appendix A.4); a target at or past the split's total
// (rounding) goes to the last key of positive mass.  Lane l holds P at the end
// of its block of keys [l*ept, (l+1)*ept); a ballot per target over those block
// ends finds the target's block, and one vector read of the block's prefix
// finds its key.  Targets ascend with their lanes, so the distinct keys are
// the lanes whose key differs from the lane before, compacted with a ballot;
// each holds the targets up to the next such lane.
// ---------------------------------------------------------------------------
template <int MODE>
__device__ __forceinline__ int sample_few(const Params& p, const Item& it, const HeadState& st, int hq,
                                          const uint64_t* ph, TargetArea* ta, int m0, int na, int lane) {
    int32_t* idx_row = p.idx + ((int64_t)it.b * p.Hq + hq) * p.S + m0;
    const TargetSeq<MODE> ts = target_seq<MODE>(p, it.b, hq, st.z, st.u0, st.n_targets, st.off, st.stream);
    const int ept = p.split >> 6;
    const bool active = lane < na;
    // the target in the split's fixed-point scale (P_j counts 2^-52 units)
    const double x = active ? (ts.tau(m0 + lane) - st.w_lo) * st.inv_f * 0x1p52 : 0.0;
    const double block_end = (double)ph[(lane + 1) * ept - 1];
    int block = 0;
    for (int k = 0; k < na; ++k) {
        const double xk = lane_f64(x, k);
        const int c = __popcll(__ballot(block_end <= xk));
        if (lane == k) block = c;
    }
    const int lastpos = max(st.lastpos, 0);
    int key = lastpos;
    if (active && block < 64) {
        const uint64_t* pb = ph + block * ept;
        int below = 0;
        for (int k = 0; k < ept; k += 2) {
            if (ept >= 2) {
                const ulonglong2 v2 = *reinterpret_cast<const ulonglong2*>(pb + k);
                below += ((double)v2.x <= x ? 1 : 0) + ((double)v2.y <= x ? 1 : 0);
            } else {
                below += (double)pb[0] <= x ? 1 : 0;
            }
        }
        key = min(block * ept + below, lastpos);
    }
    if (active) idx_row[lane] = it.key0 + key;
    // distinct keys: lanes whose key differs from the previous lane's
    int prev_key = __shfl_up(key, 1, 64);
    const bool head = active && (lane == 0 || key != prev_key);
    const unsigned long long heads = __ballot(head);
    if (head) {
        const int pos = __popcll(heads & ((1ull << lane) - 1ull));
        const unsigned long long after = lane == 63 ? 0ull : heads & (~0ull << (lane + 1));
        const int next = after ? __builtin_ctzll(after) : na;
        ta->lkey[pos] = key;
        ta->lcnt[pos] = (unsigned)(next - lane);
    }
    wave_lds_sync();
    return __popcll(heads);
}

template <int MODE, int KW>
__device__ __forceinline__ int sample_chunk_strata(const Params& p, const Item& it, const HeadState& st, int hq,
                                                   const uint64_t* ph, TargetArea* ta, int m0, int na, int lane) {
    static_assert(MODE == 1 || MODE == 2, "stratified or systematic targets");
    static_assert(kTargetChunk <= 4 * 64, "four targets per lane");
    int32_t* idx_row = p.idx + ((int64_t)it.b * p.Hq + hq) * p.S + m0;
    const TargetSeq<MODE> ts = target_seq<MODE>(p, it.b, hq, st.z, st.u0, st.n_targets, st.off, st.stream);
    for (int k = lane; k < na; k += 64) {
        ta->tau[k] = ts.tau(m0 + k);
        ta->mark[k] = -1;
    }
    wave_lds_sync();
    StrataCounter<MODE> cnt;
    cnt.ph = ph;
    cnt.tau = ta->tau;
    cnt.w_lo = st.w_lo;
    cnt.f = st.f;
    cnt.s_over_z = (double)ts.S / st.z;
    cnt.shift = (MODE == 2 ? st.u0 : 0.0) - (double)ts.off;
    cnt.m0 = m0;
    cnt.na = na;
    cnt.lastpos = max(st.lastpos, 0);
    cnt.last_key = p.split - 1;
    const int ept = p.split >> 6;
    const int i0 = lane * ept;
    int prev;               // count below the lower edge of the key in hand
    {
        int c1[1];
        const int j1[1] = {i0 - 1};     // the count below the block (none for lane 0)
        cnt(j1, c1);
        prev = lane == 0 ? 0 : c1[0];
    }
    for (int k0 = 0; k0 < ept; k0 += KW) {
        int c[KW], j[KW];
#pragma unroll
        for (int q = 0; q < KW; ++q) j[q] = i0 + k0 + q;
        cnt(j, c);
#pragma unroll
        for (int q = 0; q < KW; ++q) {
            if (k0 + q < ept && c[q] > prev) {
                ta->mark[prev] = j[q];
                prev = c[q];
            }
        }
    }
    wave_lds_sync();
    // lane l: targets [4l, 4l + 4)
    int mk[4], own[4], run = -1, nm = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = lane * 4 + k;
        mk[k] = i < na ? ta->mark[i] : -1;
        nm += mk[k] >= 0 ? 1 : 0;
        run = max(run, mk[k]);
        own[k] = run;
    }
    int before = __shfl_up(wave_scan_max_i32(run), 1, 64);
    if (lane == 0) before = -1;
    const int incl = wave_scan_add_i32(nm);
    const int nlist = lane_i32(incl, 63);
    int pos = incl - nm;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = lane * 4 + k;
        if (i < na) idx_row[i] = it.key0 + max(before, own[k]);
        if (mk[k] >= 0) {
            ta->lkey[pos] = mk[k];
            ta->mark[pos] = i;          // the entry's first target (marks are read above)
            ++pos;
        }
    }
    wave_lds_sync();
    for (int e = lane; e < nlist; e += 64)
        ta->lcnt[e] = (unsigned)((e + 1 < nlist ? ta->mark[e + 1] : na) - ta->mark[e]);
    wave_lds_sync();
    return nlist;
}

// ---------------------------------------------------------------------------
// Sampling and gather-and-add for one head (one wave, no workgroup barrier).
// Each distinct sampled key of a chunk of targets is gathered once, weighted
// by its sample count.  A V row is read by LPR = d*e/16 lanes with 16-byte
// loads, so one wave-wide load covers RPL = 64/LPR rows and UL loads per lane
// keep UL*RPL rows in flight; the row groups' partial sums are then combined
// across lanes.  The waves of a workgroup gather the rows of the same split
// at the same time, so a row that several heads of the group sampled is
// fetched from HBM once and served to the others from L2.
// ---------------------------------------------------------------------------
// The head's sum of count-weighted rows goes to emit(col, vals): every lane
// passes D/64 consecutive elements starting at column col, and the 64 lanes
// cover the row once.
// KW: keys whose target counts the stratified/systematic sampler evaluates at
// once; UL: V loads in flight per lane (more overlaps more memory accesses, at
// the cost of registers).
template <int G, int D, typename E, int KW = 4, int UL = 8, typename Emit>
__device__ __forceinline__ void sample_head(const Params& p, const Item& it, const HeadState& st, int h,
                                            const LdsLayout& L, unsigned char* smem, Emit&& emit) {
    constexpr int LPR = D * E::bytes / 16;      // lanes per V row
    constexpr int RPL = 64 / LPR;               // rows per wave-wide load
    constexpr int ELV = 16 / E::bytes;          // elements per lane per row
    constexpr int EL = D / 64;                  // output elements added per lane
    static_assert(RPL * LPR == 64 && ELV == EL * RPL, "row shape");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rsub = lane / LPR;
    const int piece = lane % LPR;
    const int hq = it.g * G + h;
    const uint64_t* ph = reinterpret_cast<const uint64_t*>(smem + L.prefix) + h * p.split;
    const int* pages = reinterpret_cast<const int*>(smem + L.pages);
    TargetArea* ta = reinterpret_cast<TargetArea*>(smem + L.scratch) + wave;
    const char* vbase = reinterpret_cast<const char*>(p.v);

    float acc[ELV];
#pragma unroll
    for (int e = 0; e < ELV; ++e) acc[e] = 0.0f;
    for (int m0 = st.m_lo; m0 < st.m_hi; m0 += kTargetChunk) {
        const int na = min(kTargetChunk, st.m_hi - m0);
        int nlist;
        if (p.mode == 2) nlist = na <= kFewTargets ? sample_few<2>(p, it, st, hq, ph, ta, m0, na, lane)
                                                   : sample_chunk_strata<2, KW>(p, it, st, hq, ph, ta, m0, na, lane);
        else if (p.mode == 1) nlist = na <= kFewTargets ? sample_few<1>(p, it, st, hq, ph, ta, m0, na, lane)
                                                        : sample_chunk_strata<1, KW>(p, it, st, hq, ph, ta, m0, na, lane);
        else nlist = sample_chunk_multinomial(p, it, st, hq, ph, ta, m0, na, lane);
        for (int r0 = 0; r0 < nlist; r0 += UL * RPL) {
            uint4 x[UL];
            float wgt[UL];
#pragma unroll
            for (int u = 0; u < UL; ++u) {
                // a load whose rows all lie past the list is not issued (the
                // test is the same in every lane); a row past the list within
                // an issued load re-reads the first row with weight 0
                wgt[u] = 0.0f;
                x[u] = make_uint4(0u, 0u, 0u, 0u);
                if (r0 + u * RPL < nlist) {
                    const int row = r0 + u * RPL + rsub;
                    const bool ok = row < nlist;
                    const int key = ta->lkey[ok ? row : 0];
                    wgt[u] = ok ? (float)ta->lcnt[row] : 0.0f;
                    const int64_t off = row_offset(p, it, key, pages) + piece * ELV;
                    x[u] = load16(vbase + off * E::bytes);
                }
            }
            // loads past the list were not issued: their terms are skipped too
            // (the test is the same in every lane)
#pragma unroll
            for (int u = 0; u < UL; ++u)
                if (r0 + u * RPL < nlist) E::axpy16(wgt[u], x[u], acc);
        }
        wave_lds_sync();       // the next chunk reuses the target area
    }
    // combine the RPL row groups: afterwards every lane holds its piece's sums
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < ELV; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
    // lane passes EL of its piece's ELV elements, so the 64 lanes cover the row once
    float vals[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) vals[e] = acc[rsub * EL + e];
    emit(piece * ELV + rsub * EL, vals);
}

// ---------------------------------------------------------------------------
// The Tb split records of one query head, K = 2^record_shift per lane (lane L
// holds records L*K .. L*K + K - 1): first an ordinary (cached) read -- once
// every split has counted itself in, the records are normally in place, and
// the splits' workgroups on one XCD then share its L2 copy -- then, for any
// not written yet, device-coherent re-reads until they are.  Returns false
// (and sets the error word and *fail) after `spin_limit` re-reads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool read_records(const Params& p, const unsigned long long* rec, int Tb, int K,
                                             int spin_limit, float (&mr)[kRecPerLane], float (&lr)[kRecPerLane],
                                             int* fail) {
    const int lane = threadIdx.x & 63;
    bool fresh = true;
#pragma unroll
    for (int k = 0; k < kRecPerLane; ++k) {
        const int j = lane * K + k;
        mr[k] = -INFINITY;
        lr[k] = 0.0f;
        if (k < K && j < Tb) {
            const unsigned long long r = rec[j];
            fresh &= (r >> 32) != 0;
            mr[k] = __uint_as_float((uint32_t)r);
            lr[k] = __uint_as_float((uint32_t)(r >> 32));
        }
    }
    for (int iter = 0; !__all(fresh); ++iter) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < kRecPerLane; ++k) {
            const int j = lane * K + k;
            mr[k] = -INFINITY;
            lr[k] = 0.0f;
            if (k < K && j < Tb) {
                const unsigned long long r = __hip_atomic_load(rec + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok &= (r >> 32) != 0;
                mr[k] = __uint_as_float((uint32_t)r);
                lr[k] = __uint_as_float((uint32_t)(r >> 32));
            }
        }
        if (__all(ok)) break;
        if (iter >= spin_limit) {
            if (lane == 0) {
                __hip_atomic_store(&p.sync->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                *fail = 1;
            }
            return false;       // the same in every lane of the wave
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

// The split masses w_j = l_j * exp(m_j - M) of one head as 2^-40 fixed point
// and their exact prefix: M, the total Z, the last split of positive mass,
// this lane's exclusive prefix `excl` and, per record k of the lane, the sum
// of the lane's records before it.
struct GroupPrefix {
    float M;
    uint64_t Z, excl;
    int last;
    uint64_t before[kRecPerLane];
};

__device__ __forceinline__ GroupPrefix group_prefix(const float (&mr)[kRecPerLane], const float (&lr)[kRecPerLane],
                                                    int Tb, int K) {
    const int lane = threadIdx.x & 63;
    GroupPrefix g;
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kRecPerLane; ++k) mx = fmaxf(mx, mr[k]);
    g.M = wave_max_f32(mx);
    uint64_t run = 0;
    int last = -1;
#pragma unroll
    for (int k = 0; k < kRecPerLane; ++k) {
        const int j = lane * K + k;
        uint64_t w = 0;
        if (k < K && j < Tb) {
            const double f = (double)mass_exp(mr[k] - g.M);
            w = fixed40((double)lr[k] * f);
            if (w) last = j;
        }
        g.before[k] = run;
        run += w;
    }
    const uint64_t incl = wave_scan_add_u64(run);
    g.excl = incl - run;
    g.Z = lane_u64(incl, 63);
    g.last = wave_max_i32(last);
    return g;
}

// ---------------------------------------------------------------------------
// Global partition function, this split's target range, then the head's
// sampling and gather (one wave per head, no workgroup barrier).
// Split masses w_j = l_j * exp(m_j - M) are summed as fixed point with 2^-40
// resolution, so the prefix W is exact, monotone and identical in every
// workgroup of the sequence, and the ranges [W_t, W_t+1) tile [0, Z).
// Records still missing after `spin_limit` re-reads set the error word and
// *fail (shared by the workgroup, read by finish_output after its barrier),
// and the head is skipped: nothing is computed from an incomplete set of
// records.
// ---------------------------------------------------------------------------
// The two-kernel path's group-prefix words of the heads a wave samples,
// loaded before the sample pass needs them (the score pass, an earlier launch,
// wrote them): lane 4 s + k of the wave holds, for its s-th head h = wave +
// s * NW, word k of Z = P[Tb], W_t = P[t], W_t+1 = P[t + 1] and M | last << 32
// = P[T + 1], where P is the head's [T + 2] prefix row.
template <int G, int NT>
__device__ __forceinline__ uint64_t load_group_prefix_words(const Params& p, const Item& it) {
    constexpr int NW = NT / 64;
    constexpr int HPW = (G + NW - 1) / NW;     // heads per wave, at most
    static_assert(4 * HPW <= 64, "one lane per word");
    const int lane = threadIdx.x & 63;
    const int h = (threadIdx.x >> 6) + (lane >> 2) * NW;
    if (lane >= 4 * HPW || h >= G) return 0ull;
    const unsigned long long* gp = p.gprefix + ((int64_t)it.b * p.Hq + it.g * G + h) * (p.T + 2);
    const int k = lane & 3;
    return gp[k == 0 ? it.Tb : k == 1 ? it.t : k == 2 ? it.t + 1 : p.T + 1];
}

// Sampling and gather-and-add for two heads of one wave whose target ranges
// hold at most kFewTargets targets each (groups of more heads than waves): both heads'
// distinct keys are found first (head B's kept one per lane while head A's
// fill the wave's target area), then one gather loop reads the rows of both
// lists with all their loads in flight together, so the wave waits for one
// round of V loads instead of one per head.  Per head the rows are added with
// the same count weights as sample_head; only the order of the fp32 sums of
// the second head's rows differs.  Each head with targets passes its sum to
// its emit(col, vals) as sample_head does.
template <int G, int D, typename E, int UL = 4, typename EmitA, typename EmitB>
__device__ __forceinline__ void sample_pair(const Params& p, const Item& it, const HeadState& sA, int hA, int nA,
                                            const HeadState& sB, int hB, int nB, const LdsLayout& L,
                                            unsigned char* smem, EmitA&& emitA, EmitB&& emitB) {
    constexpr int LPR = D * E::bytes / 16;
    constexpr int RPL = 64 / LPR;
    constexpr int ELV = 16 / E::bytes;
    constexpr int EL = D / 64;
    static_assert(kFewTargets <= 64 && RPL * LPR == 64 && ELV == EL * RPL, "row shape");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rsub = lane / LPR;
    const int piece = lane % LPR;
    TargetArea* ta = reinterpret_cast<TargetArea*>(smem + L.scratch) + wave;
    const int* pages = reinterpret_cast<const int*>(smem + L.pages);
    const char* vbase = reinterpret_cast<const char*>(p.v);
    auto sample_list = [&](const HeadState& st, int h, int na) -> int {
        const int hq = it.g * G + h;
        const uint64_t* ph = reinterpret_cast<const uint64_t*>(smem + L.prefix) + h * p.split;
        if (p.mode == 2) return sample_few<2>(p, it, st, hq, ph, ta, st.m_lo, na, lane);
        if (p.mode == 1) return sample_few<1>(p, it, st, hq, ph, ta, st.m_lo, na, lane);
        return sample_chunk_multinomial(p, it, st, hq, ph, ta, st.m_lo, na, lane);
    };
    // head B's distinct keys, entry j in lane j (lanes past the list hold key 0
    // with count 0: key 0 is a row of every split)
    int nlB = 0, keyB = 0;
    unsigned int cntB = 0;
    if (nB > 0) {
        nlB = sample_list(sB, hB, nB);
        if (lane < nlB) {
            keyB = ta->lkey[lane];
            cntB = ta->lcnt[lane];
        }
        wave_lds_sync();        // head A's sampling reuses the target area
    }
    const int nlA = nA > 0 ? sample_list(sA, hA, nA) : 0;
    const int ntot = nlA + nlB;
    float accA[ELV], accB[ELV];
#pragma unroll
    for (int e = 0; e < ELV; ++e) accA[e] = accB[e] = 0.0f;
    for (int r0 = 0; r0 < ntot; r0 += UL * RPL) {
        uint4 x[UL];
        float wa[UL], wb[UL];
#pragma unroll
        for (int u = 0; u < UL; ++u) {
            const int row = r0 + u * RPL + rsub;
            // head B's entry of this row from the lane holding it (every lane
            // takes part in the exchange)
            const int jb = min(max(row - nlA, 0), 63);
            const int kb = __shfl(keyB, jb, 64);
            const unsigned int cb = (unsigned int)__shfl((int)cntB, jb, 64);
            wa[u] = 0.0f;
            wb[u] = 0.0f;
            x[u] = make_uint4(0u, 0u, 0u, 0u);
            // a load whose rows all lie past both lists is not issued (the test
            // is the same in every lane); a row past them within an issued load
            // reads key 0 with weight 0
            if (r0 + u * RPL < ntot) {
                int key = kb;
                if (row < nlA) {
                    key = ta->lkey[row];
                    wa[u] = (float)ta->lcnt[row];
                } else if (row < ntot) {
                    wb[u] = (float)cb;
                }
                const int64_t off = row_offset(p, it, key, pages) + piece * ELV;
                x[u] = load16(vbase + off * E::bytes);
            }
        }
#pragma unroll
        for (int u = 0; u < UL; ++u)
            if (r0 + u * RPL < ntot) {
                E::axpy16(wa[u], x[u], accA);
                E::axpy16(wb[u], x[u], accB);
            }
    }
    wave_lds_sync();            // the target area is free again
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < ELV; ++e) {
            accA[e] += __shfl_xor(accA[e], m, 64);
            accB[e] += __shfl_xor(accB[e], m, 64);
        }
    const int col = piece * ELV + rsub * EL;
    float vals[EL];
    if (nA > 0) {
#pragma unroll
        for (int e = 0; e < EL; ++e) vals[e] = accA[rsub * EL + e];
        emitA(col, vals);
    }
    if (nB > 0) {
#pragma unroll
        for (int e = 0; e < EL; ++e) vals[e] = accB[rsub * EL + e];
        emitB(col, vals);
    }
}

// prefix_and_sample for G > NW (two heads on some waves): the same per-head
// steps, but a wave whose two heads each hold at most kFewTargets targets
// samples both before gathering their rows together (sample_pair).
template <int G, int D, typename E, int NT, bool FROM_PREFIX, int KW, int UL>
__device__ __forceinline__ void prefix_and_sample_pairs(const Params& p, const Item& it, const LdsLayout& L,
                                                        unsigned char* smem, int spin_limit, int* fail,
                                                        uint64_t words) {
    HeadState* hs = reinterpret_cast<HeadState*>(smem + L.heads);
    constexpr int NW = NT / 64;
    static_assert(G > NW && G <= 2 * NW, "one or two heads per wave");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Tb = it.Tb;
    const int ks = Tb <= 64 ? 0 : Tb <= 128 ? 1 : Tb <= 256 ? 2 : 3;
    const int K = 1 << ks;
    // head h's group prefix, target range and state; false if the head is to
    // be skipped (its records or prefix are missing: the error is set)
    auto setup = [&](int h, HeadState& st) -> bool {
        const int hq = it.g * G + h;
        const int t = it.t;
        float M;
        uint64_t W_t, W_t1, Z;
        int last;
        if constexpr (FROM_PREFIX) {
            // the score pass's last split left the group's prefix: one word each
            const int s4 = 4 * ((h - wave) / NW);
            Z = lane_u64(words, s4);
            W_t = lane_u64(words, s4 + 1);
            W_t1 = lane_u64(words, s4 + 2);
            const uint64_t ml = lane_u64(words, s4 + 3);
            M = __uint_as_float((uint32_t)ml);
            last = (int)(ml >> 32);
            if (Z == 0) {           // no score pass wrote it (Z >= 1 once one did)
                if (lane == 0) {
                    __hip_atomic_store(&p.sync->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    *fail = 1;
                }
                return false;
            }
        } else {
            float mr[kRecPerLane], lr[kRecPerLane];
            if (!read_records(p, record_of(p, it.b, hq, 0), Tb, K, spin_limit, mr, lr, fail)) return false;
            GroupPrefix gpx = group_prefix(mr, lr, Tb, K);
            M = gpx.M;
            Z = gpx.Z;
            last = gpx.last;
            const int kt = t & (K - 1);
            const int kt1 = (t + 1) & (K - 1);
            uint64_t at_t = 0, at_t1 = 0;
#pragma unroll
            for (int k = 0; k < kRecPerLane; ++k) {
                if (k == kt) at_t = gpx.before[k];
                if (k == kt1) at_t1 = gpx.before[k];
            }
            W_t = lane_u64(gpx.excl + at_t, t >> ks);
            W_t1 = (t + 1 < Tb) ? lane_u64(gpx.excl + at_t1, (t + 1) >> ks) : Z;
        }
        const double u0 = hs[h].u0;
        const double z = (double)Z * 0x1p-40;
        const double w_lo = (double)W_t * 0x1p-40;
        const double w_hi = (double)W_t1 * 0x1p-40;
        int m_lo, m_hi;
        if (p.mode == 2) target_range<2>(p, it.b, hq, z, u0, w_lo, w_hi, t == last, lane, &m_lo, &m_hi);
        else if (p.mode == 1) target_range<1>(p, it.b, hq, z, u0, w_lo, w_hi, t == last, lane, &m_lo, &m_hi);
        else target_range<0>(p, it.b, hq, z, u0, w_lo, w_hi, t == last, lane, &m_lo, &m_hi);
        // the head's state in registers (every value here is the same in all lanes)
        st = hs[h];
        st.w_lo = w_lo;
        st.z = z;
        st.f = (double)mass_exp(st.m_t - M);
        st.inv_f = (double)mass_exp(M - st.m_t);
        st.m_lo = m_lo;
        st.m_hi = max(m_hi, m_lo);
        st.n_targets = p.S;
        st.stream = 0;
        st.off = 0;
        return true;
    };
    // into accumulation slot t mod kOutSlots of the group
    auto slot_of = [&](int h) {
        return p.accum + ((((int64_t)it.b * p.Hkv + it.g) * kOutSlots + it.t % kOutSlots) * G + h) * D;
    };
    auto one_head = [&](const HeadState& st, int h) {
        float* slot = slot_of(h);
        sample_head<G, D, E, KW, UL>(p, it, st, h, L, smem, [&](int col, const float* vals) {
#pragma unroll
            for (int e = 0; e < D / 64; ++e) unsafeAtomicAdd(slot + col + e, vals[e]);
        });
    };
    const int hA = wave, hB = wave + NW;
    HeadState sA;
    const int nA = setup(hA, sA) ? sA.m_hi - sA.m_lo : 0;
    if (hB >= G) {                  // one head on this wave
        if (nA > 0) one_head(sA, hA);
        return;
    }
    HeadState sB;
    const int nB = setup(hB, sB) ? sB.m_hi - sB.m_lo : 0;
    if (nA <= kFewTargets && nB <= kFewTargets) {
        float* slotA = slot_of(hA);
        float* slotB = slot_of(hB);
        sample_pair<G, D, E>(p, it, sA, hA, nA, sB, hB, nB, L, smem,
                             [&](int col, const float* vals) {
#pragma unroll
                                 for (int e = 0; e < D / 64; ++e) unsafeAtomicAdd(slotA + col + e, vals[e]);
                             },
                             [&](int col, const float* vals) {
#pragma unroll
                                 for (int e = 0; e < D / 64; ++e) unsafeAtomicAdd(slotB + col + e, vals[e]);
                             });
    } else {
        if (nA > 0) one_head(sA, hA);
        if (nB > 0) one_head(sB, hB);
    }
}

// FROM_PREFIX: the group's prefix words come from load_group_prefix_words
// (`words`), otherwise from the split records.  Groups of more heads than
// waves take prefix_and_sample_pairs.
template <int G, int D, typename E, int NT, bool FROM_PREFIX = false, int KW = 4, int UL = 8>
__device__ __forceinline__ void prefix_and_sample(const Params& p, const Item& it, const LdsLayout& L,
                                                  unsigned char* smem, int spin_limit, int* fail,
                                                  uint64_t words = 0) {
    constexpr int NW = NT / 64;
    if constexpr (G > NW) {
        prefix_and_sample_pairs<G, D, E, NT, FROM_PREFIX, KW, UL>(p, it, L, smem, spin_limit, fail, words);
        return;
    }
    HeadState* hs = reinterpret_cast<HeadState*>(smem + L.heads);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Tb = it.Tb;
    // records per lane: the power of two K = 2^ks with 64 K >= Tb (K <= kRecPerLane)
    const int ks = Tb <= 64 ? 0 : Tb <= 128 ? 1 : Tb <= 256 ? 2 : 3;
    const int K = 1 << ks;
    for (int h = wave; h < G; h += NW) {
        const int hq = it.g * G + h;
        const int t = it.t;
        float M;
        uint64_t W_t, W_t1, Z;
        int last;
        if constexpr (FROM_PREFIX) {
            // the score pass's last split left the group's prefix: one word each
            const int s4 = 4 * ((h - wave) / NW);
            Z = lane_u64(words, s4);
            W_t = lane_u64(words, s4 + 1);
            W_t1 = lane_u64(words, s4 + 2);
            const uint64_t ml = lane_u64(words, s4 + 3);
            M = __uint_as_float((uint32_t)ml);
            last = (int)(ml >> 32);
            if (Z == 0) {           // no score pass wrote it (Z >= 1 once one did)
                if (lane == 0) {
                    __hip_atomic_store(&p.sync->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    *fail = 1;
                }
                continue;
            }
        } else {
            float mr[kRecPerLane], lr[kRecPerLane];
            if (!read_records(p, record_of(p, it.b, hq, 0), Tb, K, spin_limit, mr, lr, fail)) continue;
            GroupPrefix gpx = group_prefix(mr, lr, Tb, K);
            M = gpx.M;
            Z = gpx.Z;
            last = gpx.last;
            // W_t and W_{t+1} (exclusive prefixes of splits t and t+1)
            const int kt = t & (K - 1);
            const int kt1 = (t + 1) & (K - 1);
            uint64_t at_t = 0, at_t1 = 0;
#pragma unroll
            for (int k = 0; k < kRecPerLane; ++k) {
                if (k == kt) at_t = gpx.before[k];
                if (k == kt1) at_t1 = gpx.before[k];
            }
            W_t = lane_u64(gpx.excl + at_t, t >> ks);
            W_t1 = (t + 1 < Tb) ? lane_u64(gpx.excl + at_t1, (t + 1) >> ks) : Z;
        }

        const double u0 = hs[h].u0;
        const double z = (double)Z * 0x1p-40;
        const double w_lo = (double)W_t * 0x1p-40;
        const double w_hi = (double)W_t1 * 0x1p-40;
        int m_lo, m_hi;
        if (p.mode == 2) target_range<2>(p, it.b, hq, z, u0, w_lo, w_hi, t == last, lane, &m_lo, &m_hi);
        else if (p.mode == 1) target_range<1>(p, it.b, hq, z, u0, w_lo, w_hi, t == last, lane, &m_lo, &m_hi);
        else target_range<0>(p, it.b, hq, z, u0, w_lo, w_hi, t == last, lane, &m_lo, &m_hi);
        // the head's state in registers (every value here is the same in all lanes)
        HeadState st = hs[h];
        st.w_lo = w_lo;
        st.z = z;
        st.f = (double)mass_exp(st.m_t - M);
        st.inv_f = (double)mass_exp(M - st.m_t);
        st.m_lo = m_lo;
        st.m_hi = max(m_hi, m_lo);
        st.n_targets = p.S;
        st.stream = 0;
        st.off = 0;
        if (st.m_hi > st.m_lo) {
            // into accumulation slot t mod kOutSlots of the group
            float* slot = p.accum + ((((int64_t)it.b * p.Hkv + it.g) * kOutSlots + it.t % kOutSlots) * G + h) * D;
            sample_head<G, D, E, KW, UL>(p, it, st, h, L, smem, [&](int col, const float* vals) {
#pragma unroll
                for (int e = 0; e < D / 64; ++e) unsafeAtomicAdd(slot + col + e, vals[e]);
            });
        }
    }
}

// ---------------------------------------------------------------------------
// Two-kernel path: the last split of a (sequence, KV head) to finish the score
// pass computes the group's split-mass prefixes once, with the fused kernel's
// arithmetic (read_records, group_prefix), so that each split of the sample
// pass reads W_t, W_{t+1}, Z, M and the last split of positive mass instead of
// every record of the sequence.  The count is the group's barrier word 0,
// which the two-kernel path does not otherwise use; the last split returns it
// to zero, and the sample pass's last split clears the prefixes.
// ---------------------------------------------------------------------------
template <int G, int NT>
__device__ __forceinline__ void publish_group_prefix(const Params& p, const Item& it) {
    constexpr int NW = NT / 64;
    __shared__ int s_last;
    __syncthreads();        // the workgroup's records are stored
    if (threadIdx.x == 0) {
        unsigned int* bar = p.barrier + ((int64_t)it.b * p.Hkv + it.g) * kBarrierStride;
        const unsigned int prev = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned int)it.Tb - 1u;
        if (s_last) __hip_atomic_store(bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Tb = it.Tb;
    const int K = 1 << (Tb <= 64 ? 0 : Tb <= 128 ? 1 : Tb <= 256 ? 2 : 3);
    int fail = 0;
    for (int h = wave; h < G; h += NW) {
        const int hq = it.g * G + h;
        float mr[kRecPerLane], lr[kRecPerLane];
        // a give-up leaves the prefix at zero, which the sample pass reports
        if (!read_records(p, record_of(p, it.b, hq, 0), Tb, K, kSpinLimit, mr, lr, &fail)) continue;
        const GroupPrefix gpx = group_prefix(mr, lr, Tb, K);
        unsigned long long* gp = p.gprefix + ((int64_t)it.b * p.Hq + hq) * (p.T + 2);
#pragma unroll
        for (int k = 0; k < kRecPerLane; ++k) {
            const int j = lane * K + k;
            if (k < K && j < Tb) gp[j] = gpx.excl + gpx.before[k];
        }
        if (lane == 0) {
            gp[Tb] = gpx.Z;
            gp[p.T + 1] = (unsigned long long)__float_as_uint(gpx.M) | ((unsigned long long)(uint32_t)gpx.last << 32);
        }
    }
}

// ---------------------------------------------------------------------------
// Failed calls.  A bounded wait that gives up sets the workspace's error word;
// the splits that gave up write NaN to o and -1 to idx for their group's heads
// and stop, so the group's counts are left unfinished (the workspace needs
// santa_workspace_init).  A later call that finds the error word set at its
// start does the same for every group instead of consuming the stale state,
// and the split that would finish a group's output writes NaN if the error
// word is set by then.  The error word itself is the authoritative signal:
// a split of a group that did not wait may still have finished it first.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned int workspace_error_now(const Params& p) {
    return __hip_atomic_load(&p.sync->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int D, int NT>
__device__ __forceinline__ void poison_group(const Params& p, const Item& it) {
    float* o = p.o + ((int64_t)it.b * p.Hq + (int64_t)it.g * G) * D;
    for (int i = threadIdx.x; i < G * D; i += NT) o[i] = __builtin_nanf("");
    int32_t* idx = p.idx + ((int64_t)it.b * p.Hq + (int64_t)it.g * G) * p.S;
    for (int i = threadIdx.x; i < G * p.S; i += NT) idx[i] = -1;
}

// Waits until every memory operation this wave has issued has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

// ---------------------------------------------------------------------------
// The output of a (sequence, KV head) and the clean-up of its workspace state.
// Each split, once its additions into the accumulation slots have completed,
// counts itself done.  The last one -- every other split of the group has then
// passed the barrier and read the records and targets -- sums the kOutSlots
// slots, stores o = (1/S) * sum (Eq. 3) for the G heads, and returns to zero
// the slots, the counts, the barrier flags, the group's split records and
// (multinomial) its targets, so that a completed call leaves this state all
// zero: the next call may have another layout, whose synchronisation state
// can lie where this call's targets were.  Nothing here waits for another
// workgroup.
// ---------------------------------------------------------------------------
template <int G, int D, int NT>
__device__ __forceinline__ void finish_output(const Params& p, const Item& it, const int* fail,
                                              bool clear_prefix = false) {
    __shared__ int s_last;
    wait_memory();           // this wave's slot additions have been performed
    __syncthreads();
    if (*fail) {             // a head's wait gave up: the group is not finished
        poison_group<G, D, NT>(p, it);
        return;
    }
    unsigned int* bar = p.barrier + ((int64_t)it.b * p.Hkv + it.g) * kBarrierStride;
    if (threadIdx.x == 0) {
        const unsigned int prev = __hip_atomic_fetch_add(bar + 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned int)it.Tb - 1u;
    }
    __syncthreads();
    if (!s_last) return;
    // slot words in pairs: the 16 loads of a pair are all in flight at once
    constexpr int NP = G * D / 2;
    unsigned long long* acc =
        reinterpret_cast<unsigned long long*>(p.accum + ((int64_t)it.b * p.Hkv + it.g) * kOutSlots * G * D);
    float* o = p.o + ((int64_t)it.b * p.Hq + (int64_t)it.g * G) * D;
    // a wait of this call gave up somewhere: the output is not trusted
    const float inv_s = workspace_error_now(p) ? __builtin_nanf("") : 1.0f / (float)p.S;
    for (int i = threadIdx.x; i < NP; i += NT) {
        unsigned long long v[kOutSlots];
#pragma unroll
        for (int k = 0; k < kOutSlots; ++k)
            v[k] = __hip_atomic_load(acc + k * NP + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int k = 0; k < kOutSlots; ++k) {
            s0 += __uint_as_float((uint32_t)v[k]);
            s1 += __uint_as_float((uint32_t)(v[k] >> 32));
        }
#pragma unroll
        for (int k = 0; k < kOutSlots; ++k)
            __hip_atomic_store(acc + k * NP + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *reinterpret_cast<float2*>(o + 2 * i) = make_float2(s0 * inv_s, s1 * inv_s);
    }
    if (threadIdx.x == 0) __hip_atomic_store(bar + 32, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < kFlagCopies)
        __hip_atomic_store(bar + 32 * (2 + threadIdx.x), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = threadIdx.x; i < G * it.Tb; i += NT) {
        const int h = i / it.Tb;
        __hip_atomic_store(record_of(p, it.b, it.g * G + h, i - h * it.Tb), 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (p.mode == 0) {
        double* tg = p.targets + ((int64_t)it.b * p.Hq + (int64_t)it.g * G) * p.S;
        for (int i = threadIdx.x; i < G * p.S; i += NT) tg[i] = 0.0;
    }
    if (clear_prefix) {         // the two-kernel path's group prefixes
        unsigned long long* gp = p.gprefix + ((int64_t)it.b * p.Hq + (int64_t)it.g * G) * (p.T + 2);
        for (int i = threadIdx.x; i < G * (p.T + 2); i += NT) gp[i] = 0ull;
    }
}

// o = 0 and idx = -1 for the G heads of an empty sequence.
template <int G, int D, int NT>
__device__ __forceinline__ void write_empty(const Params& p, const Item& it) {
    float* o = p.o + ((int64_t)it.b * p.Hq + (int64_t)it.g * G) * D;
    for (int i = threadIdx.x; i < G * D; i += NT) o[i] = 0.0f;
    int32_t* idx = p.idx + ((int64_t)it.b * p.Hq + (int64_t)it.g * G) * p.S;
    for (int i = threadIdx.x; i < G * p.S; i += NT) idx[i] = -1;
}


// ---------------------------------------------------------------------------
// The score stash of the two-kernel path: the split's scaled scores from LDS
// (sc[h * split + local]) to stash row (b, g * G + h) at the split's first key,
// with coalesced 16-byte stores.
// ---------------------------------------------------------------------------
// STREAM: with the nontemporal hint (for the sample pass, which reads the
// stash once, well after; the top-k selection reads it at once and is better
// served from the caches).
template <int G, int NT, bool STREAM = true>
__device__ __forceinline__ void write_stash(const Params& p, const Item& it, const float* sc) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    for (int h = threadIdx.x >> 6; h < G; h += NW) {
        const float* row = sc + h * p.split;
        float* dst = p.stash + ((int64_t)it.b * p.Hq + it.g * G + h) * p.stash_row + it.key0;
        for (int i = lane * 4; i < it.ns; i += 256) {
            if (i + 4 <= it.ns) {
                if constexpr (STREAM)
                    store_stream(reinterpret_cast<float4*>(dst + i), *reinterpret_cast<const float4*>(row + i));
                else
                    *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(row + i);
            } else {
                for (int e = i; e < it.ns; ++e) dst[e] = row[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The work item of a fused-kernel workgroup, -1 if it has none.  A workgroup
// waits only for the statistics of the other splits of its (sequence, KV
// head) group; two ways to guarantee that every statistic a workgroup waits
// for is computed by a workgroup that runs:
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
// ---------------------------------------------------------------------------
__device__ __forceinline__ int take_item(const Params& p) {
    if (!p.use_ticket) return blockIdx.x;
    __shared__ int s_item;
    if (threadIdx.x == 0) {
        const unsigned int k = __hip_atomic_fetch_add(&p.sync->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the last ticket of the launch: every other one has been taken, so the
        // counter returns to zero for the next call
        if (k == (unsigned int)p.items - 1u)
            __hip_atomic_store(&p.sync->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // a counter that did not start at zero (a workspace never cleared): no
        // item, and the call is marked failed
        if (k >= (unsigned int)p.items)
            __hip_atomic_store(&p.sync->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_item = k < (unsigned int)p.items ? (int)k : -1;
    }
    __syncthreads();
    return s_item;
}

// ---------------------------------------------------------------------------
// One work item of the fused decode kernel: the whole step of section 3.2 of
// "Stochastic Sparse Attention for Memory-Bound Inference" (score pass, global
// budget, parallel gather) for one (sequence, KV head, split), with the
// split's scores kept in LDS across the wait for the other splits.
// stream(it, sc, pages) fills the scaled scores sc[h * split + local] of the
// item's keys for the G heads (the exact scores of Eq. 1, or an estimate of
// them); err0 is the workspace's error word as read at the start.
// ---------------------------------------------------------------------------
template <int G, int D, typename E, int NT, typename Stream>
__device__ __forceinline__ void fused_item(const Params& p, const Item& it, unsigned int err0, unsigned char* smem,
                                           Stream&& stream) {
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
    stream(it, sc, pages);
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
    prefix_and_sample<G, D, E, NT>(p, it, L, smem, kSpinLimit, &s_fail);
    finish_output<G, D, NT>(p, it, &s_fail);
}

}  // namespace santa
