// SANTA++: attention through representative keys ("SANTA++: Sampling
// Attention through Representative Keys", section 2.2-2.3, Appendix A
// Algorithms 1, 2 and 4, Appendix D).
//
// Preparation, once after prefill (pp_build_kernel, one wave per parent):
// the prompt's N keys of every (sequence, KV head) are cut into contiguous
// parents of P tokens; in each, up to R actual keys become representatives --
// the first nearest the parent's mean key, each later one the member farthest
// from its nearest representative so far -- and every member joins its
// nearest representative's team (a representative owns its own row).
// Distances are squared Euclidean, in fp64, on the keys widened exactly from
// their storage type.  The kernel writes team-ordered copies of the prompt's
// K and V rows, the representative keys and each team's first row, so that a
// team's members are one contiguous range.
//
// Decoding (three launches):
//   pp_route_kernel   one workgroup per (sequence, KV head, block of teams):
//                     the G query heads' routing logits phi = log n_g +
//                     q . l_g / sqrt(d) and Gumbel-perturbed scores Y;
//   pp_select_kernel  one workgroup per (sequence, query head): the K largest
//                     Y by radix selection (ties to the lower team index), the
//                     threshold tau = the (K+1)-th, and the corrections
//                     c_g = 1 - exp(-exp(phi_g - tau)); the last head of each
//                     GQA group to finish merges the group's selections into
//                     one read plan (each team once, with the heads that chose
//                     it and their log c_g);
//   pp_attend_kernel  NC workgroups per (sequence, KV head) read the plan's
//                     rows and the exact suffix once for the whole group and
//                     accumulate each head's online softmax over its own teams
//                     with logits s - log c_g (so 1/c_g weighs both sums of
//                     Eq. 4); the last of them merges the partial results.
#include "santa_pp.h"
#include "santa_select.h"

namespace santa {

constexpr int kPPRouteRows = 64;        // teams per route workgroup
constexpr int kPPSelectThreads = kSelectBins / 2;

__device__ __forceinline__ int64_t pp_row(const PPParams& p, int b, int g, int t) {
    return (int64_t)b * p.stride_seq + (int64_t)t * p.stride_tok + (int64_t)g * p.stride_head;
}

// ---------------------------------------------------------------------------
// Team construction
// ---------------------------------------------------------------------------
// (value, index) reductions over a wave: the smaller (larger) value, ties to
// the lower index.
__device__ __forceinline__ void wave_argmin(double& v, int& i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(v, off, 64);
        const int oi = __shfl_xor(i, off, 64);
        if (ov < v || (ov == v && oi < i)) {
            v = ov;
            i = oi;
        }
    }
}

__device__ __forceinline__ void wave_argmax(double& v, int& i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(v, off, 64);
        const int oi = __shfl_xor(i, off, 64);
        if (ov > v || (ov == v && oi < i)) {
            v = ov;
            i = oi;
        }
    }
}

// Squared distance between member rows a and b of the parent (LDS, fp32 values
// widened to fp64), features summed in order.
template <int D>
__device__ __forceinline__ double member_dist(const float* keys, int a, int b) {
    double s = 0.0;
    for (int j = 0; j < D; ++j) {
        const double t = (double)keys[a * D + j] - (double)keys[b * D + j];
        s = fma(t, t, s);
    }
    return s;
}

// One wave per (sequence, KV head, parent).
template <int D, typename E>
__global__ __launch_bounds__(64) void pp_build_kernel(PPParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* keys = reinterpret_cast<float*>(smem);                      // [P][D]
    __shared__ double mu[D];
    __shared__ int reps[kPPMaxParent];
    const int lane = threadIdx.x;
    const int nparents = (p.N + p.P - 1) / p.P;
    const int wg = blockIdx.x;
    const int u = wg % nparents;
    const int bg = wg / nparents;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    const int base = u * p.P;
    const int cs = min(p.P, p.N - base);
    const int r = min(p.R, cs);
    const char* kc = reinterpret_cast<const char*>(p.k);
    const char* vc = reinterpret_cast<const char*>(p.v);
    for (int i = 0; i < cs; ++i)
        for (int j = lane; j < D; j += 64) keys[i * D + j] = E::elem(kc, pp_row(p, b, g, base + i) + j);
    __syncthreads();
    // the parent's mean key, members summed in token order
    for (int j = lane; j < D; j += 64) {
        double s = 0.0;
        for (int i = 0; i < cs; ++i) s += (double)keys[i * D + j];
        mu[j] = s / (double)cs;
    }
    __syncthreads();
    const bool member = lane < cs;
    // first representative: nearest the mean
    double dv = INFINITY;
    if (member) {
        double s = 0.0;
        for (int j = 0; j < D; ++j) {
            const double t = (double)keys[lane * D + j] - mu[j];
            s = fma(t, t, s);
        }
        dv = s;
    }
    int di = member ? lane : 1 << 30;
    wave_argmin(dv, di);
    if (lane == 0) reps[0] = di;
    // farthest-first: the member farthest from its nearest representative
    double nearest = INFINITY;
    bool chosen = member && lane == di;
    for (int c = 1; c < r; ++c) {
        __syncthreads();
        if (member) nearest = fmin(nearest, member_dist<D>(keys, lane, reps[c - 1]));
        double fv = (member && !chosen) ? nearest : -INFINITY;
        int fi = member ? lane : 1 << 30;
        wave_argmax(fv, fi);
        if (lane == 0) reps[c] = fi;
        if (lane == fi) chosen = true;
    }
    __syncthreads();
    // assignment: the nearest representative, ties to the one chosen first;
    // each representative owns its own row
    int owner = 0;
    if (member) {
        double best = INFINITY;
        for (int c = 0; c < r; ++c) {
            const double dd = member_dist<D>(keys, lane, reps[c]);
            if (dd < best) {
                best = dd;
                owner = c;
            }
        }
        for (int c = 0; c < r; ++c)
            if (reps[c] == lane) owner = c;
    }
    // team offsets within the parent, members in token order
    int off = 0, pos = 0;
    const unsigned long long below = (1ull << lane) - 1ull;
    const int team0 = u * p.R;                   // every earlier parent is full: R teams each
    for (int c = 0; c < r; ++c) {
        const unsigned long long m = __ballot(member && owner == c);
        if (member && owner == c) pos = off + __popcll(m & below);
        if (lane == 0)
            p.team_start[((int64_t)b * p.Hkv + g) * (p.M + 1) + team0 + c] = base + off;
        off += __popcll(m);
    }
    if (lane == 0 && u == nparents - 1) p.team_start[((int64_t)b * p.Hkv + g) * (p.M + 1) + p.M] = p.N;
    // the team-ordered copies (16-byte pieces) and the representative keys
    constexpr int PIECES = D * E::bytes / 16;
    char* pk = reinterpret_cast<char*>(p.packed_k);
    char* pv = reinterpret_cast<char*>(p.packed_v);
    char* rk = reinterpret_cast<char*>(p.rep_k);
    const int64_t bg_rows = ((int64_t)b * p.Hkv + g) * p.N;
    for (int i = 0; i < cs; ++i) {
        const int dst = __shfl(pos, i, 64);
        const int64_t src = pp_row(p, b, g, base + i) * E::bytes;
        const int64_t to = (bg_rows + base + dst) * D * E::bytes;
        for (int c = lane; c < PIECES; c += 64) {
            *reinterpret_cast<uint4*>(pk + to + c * 16) = load16(kc + src + c * 16);
            *reinterpret_cast<uint4*>(pv + to + c * 16) = load16(vc + src + c * 16);
        }
    }
    if (member) p.perm[bg_rows + base + pos] = base + lane;
    for (int c = 0; c < r; ++c) {
        const int64_t src = pp_row(p, b, g, base + reps[c]) * E::bytes;
        const int64_t to = (((int64_t)b * p.Hkv + g) * p.M + team0 + c) * D * E::bytes;
        for (int e = lane; e < PIECES; e += 64) *reinterpret_cast<uint4*>(rk + to + e * 16) = load16(kc + src + e * 16);
    }
}

// ---------------------------------------------------------------------------
// Routing
// ---------------------------------------------------------------------------
__device__ __forceinline__ double pp_gumbel(uint64_t seed, int b, int h, int g) {
    const uint64_t w = philox4x64_10_word0((uint64_t)g, (uint64_t)h, (uint64_t)b, 0ull, seed, 2ull);
    const double u = ((double)(w >> 11) + 0.5) * 0x1p-53;
    return -log(-log(u));
}

template <int G, int D, typename E>
__global__ __launch_bounds__(256) void pp_route_kernel(PPParams p) {
    constexpr int LPR = D * E::bytes / 16;       // lanes per representative row
    constexpr int RPW = 64 / LPR;                // rows per wave-wide load
    static_assert(LPR >= G, "one lane of a row group per query head");
    const int nblk = (p.M + kPPRouteRows - 1) / kPPRouteRows;
    const int blk = blockIdx.x % nblk;
    const int bg = blockIdx.x / nblk;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane % LPR, rsub = lane / LPR;
    const char* qb = reinterpret_cast<const char*>(p.q) + (((int64_t)b * p.Hq + (int64_t)g * G) * D) * E::bytes + li * 16;
    uint4 qf[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qf[h] = load16(qb + (int64_t)h * D * E::bytes);
    const char* rk = reinterpret_cast<const char*>(p.rep_k) + ((int64_t)bg * p.M) * D * E::bytes + li * 16;
    const int32_t* ts = p.team_start + (int64_t)bg * (p.M + 1);
    const int t_end = min(p.M, (blk + 1) * kPPRouteRows);
    for (int t0 = blk * kPPRouteRows + wave * RPW; t0 < t_end; t0 += 4 * RPW) {
        const int t = t0 + rsub;
        const bool ok = t < t_end;
        const uint4 kv = load16(rk + (int64_t)(ok ? t : t0) * D * E::bytes);
        float dot[G];
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = E::dot16(kv, qf[h], 0.0f);
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1)
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] += __shfl_xor(dot[h], m, 64);
        if (ok && li < G) {
            float s = 0.0f;
#pragma unroll
            for (int h = 0; h < G; ++h)
                if (h == li) s = dot[h];
            const int hq = g * G + li;
            const float ph = logf((float)(ts[t + 1] - ts[t])) + s * p.scale;
            const int64_t at = ((int64_t)b * p.Hq + hq) * p.Mpad + t;
            p.phi[at] = ph;
            p.y[at] = ph + (float)pp_gumbel(p.seed, b, hq, t);
        }
    }
}

// ---------------------------------------------------------------------------
// Selection and the group's read plan
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_agent(int32_t* a, int32_t v) {
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* a, float v) {
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t* a) {
    return __hip_atomic_load(const_cast<int32_t*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* a) {
    return __hip_atomic_load(const_cast<float*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kPPSelectThreads) void pp_select_kernel(PPParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned int* hist = reinterpret_cast<unsigned int*>(smem);                  // [kSelectBins]
    int* scan = reinterpret_cast<int*>(smem + kSelectBins * 4);                  // [2 * waves + 4]
    unsigned int* maskw = reinterpret_cast<unsigned int*>(smem + kSelectBins * 4 + 256);   // [Mpad / 4]
    __shared__ int s_last, s_thr, s_total;
    const int bh = blockIdx.x;
    const int b = bh / p.Hq, hq = bh - b * p.Hq;
    const int g = hq / p.G;
    const int tid = threadIdx.x;
    const int M = p.M, K = p.K, Keff = p.Keff;
    int32_t* teams = p.teams + (int64_t)bh * (K + 1);
    float* corr = p.corr + (int64_t)bh * K;
    const float* row = p.y + (int64_t)bh * p.Mpad;
    const float* phi = p.phi + (int64_t)bh * p.Mpad;
    if (tid == 0) s_thr = 0;                 // set again below; the barriers before its reads publish it
    if (Keff == M) {
        // every team, with c = 1 (Algorithm 1, lines 4-5)
        for (int j = tid; j <= K; j += kPPSelectThreads) st_agent(teams + j, j < M ? j : -1);
        for (int j = tid; j < K; j += kPPSelectThreads) st_agent(corr + j, j < M ? 1.0f : 0.0f);
    } else {
        const int C = ((M + kPPSelectThreads - 1) / kPPSelectThreads + 3) & ~3;
        const int i0 = min(M, tid * C), i1 = min(M, i0 + C);
        int krem = 0;
        const uint32_t kth = radix_kth<kPPSelectThreads>(row, i0, i1, Keff + 1, hist, scan, &krem);
        // The Keff + 1 largest, in index order, are the keys above kth and the
        // first krem keys equal to it; the last of those (equal rank krem - 1)
        // is the threshold team, the others are the selection.
        int n_eq = 0, n_gt = 0;
        for (int i = i0; i < i1; ++i) {
            const uint32_t key = score_key(row[i]);
            n_gt += key > kth ? 1 : 0;
            n_eq += key == kth ? 1 : 0;
        }
        const int eq_before = block_exclusive_sum<kPPSelectThreads>(n_eq, scan);
        const int take_eq = max(0, min(n_eq, krem - eq_before));
        const int has_thr = (eq_before <= krem - 1 && krem - 1 < eq_before + n_eq) ? 1 : 0;
        int pos = block_exclusive_sum<kPPSelectThreads>(n_gt + take_eq - has_thr, scan);
        int eq_seen = 0;
        for (int i = i0; i < i1; ++i) {
            const uint32_t key = score_key(row[i]);
            bool keep = key > kth;
            if (key == kth) {
                if (eq_before + eq_seen == krem - 1) {
                    s_thr = i;
                    keep = false;
                } else {
                    keep = eq_seen < take_eq;
                }
                ++eq_seen;
            }
            if (keep && pos < Keff) {       // exactly Keff are kept; the bound only guards the writes
                st_agent(teams + pos, i);
                ++pos;
            }
        }
        __syncthreads();
        const int t_thr = s_thr;
        const double tau = (double)row[t_thr];
        __syncthreads();
        for (int j = tid; j < Keff; j += kPPSelectThreads) {
            const int t = ld_agent(teams + j);
            st_agent(corr + j, (float)(-expm1(-exp((double)phi[t] - tau))));      // Eq. 7
        }
        if (tid == 0) st_agent(teams + K, t_thr);
    }
    // the last head of the GQA group to finish builds the group's read plan:
    // every thread's stores are made visible before the head counts itself
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned int prev =
            __hip_atomic_fetch_add(&p.arrive[b * p.Hkv + g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned int)p.G - 1u;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (tid == 0) __hip_atomic_store(&p.arrive[b * p.Hkv + g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int MW = p.Mpad / 4;
    for (int w = tid; w < MW; w += kPPSelectThreads) maskw[w] = 0u;
    __syncthreads();
    for (int h = 0; h < p.G; ++h) {
        const int32_t* th = p.teams + ((int64_t)b * p.Hq + g * p.G + h) * (K + 1);
        for (int j = tid; j < Keff; j += kPPSelectThreads) {
            const int t = ld_agent(th + j);
            if ((unsigned int)t < (unsigned int)M) atomicOr(&maskw[t >> 2], (1u << h) << (8 * (t & 3)));
        }
    }
    __syncthreads();
    // compact the union in team order
    const int CW = (MW + kPPSelectThreads - 1) / kPPSelectThreads;
    const int w0 = min(MW, tid * CW), w1 = min(MW, w0 + CW);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) {
        const unsigned int m = maskw[w];
        cnt += ((m & 0xFFu) != 0) + ((m & 0xFF00u) != 0) + ((m & 0xFF0000u) != 0) + ((m & 0xFF000000u) != 0);
    }
    int at = block_exclusive_sum<kPPSelectThreads>(cnt, scan);
    int32_t* plan = p.plan + (int64_t)(b * p.Hkv + g) * p.PL;
    for (int w = w0; w < w1; ++w) {
        const unsigned int m = maskw[w];
        for (int e = 0; e < 4; ++e) {
            const unsigned int hm = (m >> (8 * e)) & 0xFFu;
            if (hm && at < p.PL) plan[at++] = (4 * w + e) | (int)(hm << 24);
        }
    }
    if (tid == kPPSelectThreads - 1) {
        s_total = at;
        p.plan_n[b * p.Hkv + g] = at;
    }
    __syncthreads();
    // each head's log c_g at the plan entry of its teams (binary search)
    const int total = s_total;
    float* logc = p.plan_logc + (int64_t)(b * p.Hkv + g) * p.PL * p.G;
    for (int h = 0; h < p.G; ++h) {
        const int64_t hrow = (int64_t)b * p.Hq + g * p.G + h;
        const int32_t* th = p.teams + hrow * (K + 1);
        const float* ch = p.corr + hrow * K;
        for (int j = tid; j < Keff; j += kPPSelectThreads) {
            const int t = ld_agent(th + j);
            int lo = 0, hi = total - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((plan[mid] & 0xFFFFFF) < t) lo = mid + 1;
                else hi = mid;
            }
            logc[(int64_t)lo * p.G + h] = logf(ld_agent(ch + j));
        }
    }
}

// ---------------------------------------------------------------------------
// Selected attention over the group's plan and the exact suffix
// ---------------------------------------------------------------------------
template <int G, int D, typename E>
__global__ __launch_bounds__(256) void pp_attend_kernel(PPParams p) {
    constexpr int LPR = D * E::bytes / 16;       // lanes per row
    constexpr int RPW = 64 / LPR;                // rows per wave-wide load
    constexpr int ELV = 16 / E::bytes;           // elements per lane piece
    constexpr int NG = 4 * RPW;                  // lane groups of the workgroup
    __shared__ float s_m[NG][G], s_l[NG][G];
    __shared__ float s_acc[NG][G][D];
    __shared__ int s_last;
    const int c = blockIdx.x % p.NC;
    const int bg = blockIdx.x / p.NC;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane % LPR, rsub = lane / LPR;
    const int grp = wave * RPW + rsub;
    const char* qb = reinterpret_cast<const char*>(p.q) + (((int64_t)b * p.Hq + (int64_t)g * G) * D) * E::bytes + li * 16;
    uint4 qf[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qf[h] = load16(qb + (int64_t)h * D * E::bytes);
    float m[G], l[G], acc[G][ELV];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < ELV; ++e) acc[h][e] = 0.0f;
    }
    auto consume = [&](const uint4& kv, const uint4& vv, const float (&lc)[G], unsigned int heads) {
        float dot[G];
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = E::dot16(kv, qf[h], 0.0f);
#pragma unroll
        for (int mm = 1; mm < LPR; mm <<= 1)
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] += __shfl_xor(dot[h], mm, 64);
        float vf[ELV];
#pragma unroll
        for (int e = 0; e < ELV; ++e) vf[e] = 0.0f;
        E::axpy16(1.0f, vv, vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (!((heads >> h) & 1u)) continue;
            const float x = dot[h] * p.scale - lc[h];
            const float mn = fmaxf(m[h], x);
            const float so = __expf(m[h] - mn);
            const float pe = __expf(x - mn);
            l[h] = l[h] * so + pe;
#pragma unroll
            for (int e = 0; e < ELV; ++e) acc[h][e] = acc[h][e] * so + pe * vf[e];
            m[h] = mn;
        }
    };
    // plan entries of this chunk: lane group grp takes the entries grp, grp + NG, ...
    const int U = p.plan_n[bg];
    const int e0 = (int)((int64_t)U * c / p.NC), e1 = (int)((int64_t)U * (c + 1) / p.NC);
    const int32_t* plan = p.plan + (int64_t)bg * p.PL;
    const float* logc = p.plan_logc + (int64_t)bg * p.PL * G;
    const int32_t* ts = p.team_start + (int64_t)bg * (p.M + 1);
    const char* pk = reinterpret_cast<const char*>(p.packed_k) + ((int64_t)bg * p.N) * D * E::bytes + li * 16;
    const char* pv = reinterpret_cast<const char*>(p.packed_v) + ((int64_t)bg * p.N) * D * E::bytes + li * 16;
    for (int e = e0 + grp; e < e1; e += NG) {
        const int ent = plan[e];
        const int t = ent & 0xFFFFFF;
        const unsigned int heads = (unsigned int)ent >> 24;
        float lc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) lc[h] = ((heads >> h) & 1u) ? logc[(int64_t)e * G + h] : 0.0f;
        const int r0 = ts[t], r1 = ts[t + 1];
        for (int rr = r0; rr < r1; ++rr) {
            const uint4 kv = load16(pk + (int64_t)rr * D * E::bytes);
            const uint4 vv = load16(pv + (int64_t)rr * D * E::bytes);
            consume(kv, vv, lc, heads);
        }
    }
    // the exact suffix: rows N .. seq_len - 1 of the token-major cache, weight 1 for every head
    const int n = min(max(p.seq_lens[b], p.N), p.n_max);
    const int ns = n - p.N;
    if (ns > 0) {
        const int s0 = p.N + (int)((int64_t)ns * c / p.NC), s1 = p.N + (int)((int64_t)ns * (c + 1) / p.NC);
        float zero[G];
#pragma unroll
        for (int h = 0; h < G; ++h) zero[h] = 0.0f;
        const char* kc = reinterpret_cast<const char*>(p.k) + li * 16;
        const char* vc = reinterpret_cast<const char*>(p.v) + li * 16;
        for (int i = s0 + grp; i < s1; i += NG) {
            const int64_t off = pp_row(p, b, g, i) * E::bytes;
            consume(load16(kc + off), load16(vc + off), zero, (1u << G) - 1u);
        }
    }
    // merge the lane groups of the workgroup
    if (li == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            s_m[grp][h] = m[h];
            s_l[grp][h] = l[h];
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < ELV; ++e) s_acc[grp][h][li * ELV + e] = acc[h][e];
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * (D + 2); idx += 256) {
        const int h = idx / (D + 2), col = idx - h * (D + 2);
        float mx = -INFINITY;
        for (int q = 0; q < NG; ++q) mx = fmaxf(mx, s_m[q][h]);
        float val = 0.0f;
        for (int q = 0; q < NG; ++q) {
            const float w = s_m[q][h] == -INFINITY ? 0.0f : __expf(s_m[q][h] - mx);
            val += w * (col == 0 ? 0.0f : col == 1 ? s_l[q][h] : s_acc[q][h][col - 2]);
        }
        if (col == 0) val = mx;
        st_agent(p.part + (((int64_t)b * p.Hq + g * G + h) * p.NC + c) * (D + 2) + col, val);
    }
    // the last chunk of the group merges the chunks
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned int prev = __hip_atomic_fetch_add(&p.done[bg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned int)p.NC - 1u;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (threadIdx.x == 0) __hip_atomic_store(&p.done[bg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int h = idx / D, col = idx - h * D;
        const float* pr = p.part + (((int64_t)b * p.Hq + g * G + h) * p.NC) * (D + 2);
        float mx = -INFINITY;
        for (int q = 0; q < p.NC; ++q) mx = fmaxf(mx, ld_agent(pr + q * (D + 2)));
        float ls = 0.0f, as = 0.0f;
        for (int q = 0; q < p.NC; ++q) {
            const float mq = ld_agent(pr + q * (D + 2));
            const float w = mq == -INFINITY ? 0.0f : __expf(mq - mx);
            ls += w * ld_agent(pr + q * (D + 2) + 1);
            as += w * ld_agent(pr + q * (D + 2) + 2 + col);
        }
        p.o[((int64_t)b * p.Hq + g * G + h) * D + col] = ls > 0.0f ? as / ls : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, typename E>
static hipError_t launch_build_t(const PPParams& p, hipStream_t stream) {
    const int nparents = (p.N + p.P - 1) / p.P;
    const size_t lds = (size_t)p.P * D * 4;
    hipLaunchKernelGGL((pp_build_kernel<D, E>), dim3((unsigned)(p.B * p.Hkv * nparents)), dim3(64), lds, stream, p);
    return hipGetLastError();
}

hipError_t launch_pp_build(const PPParams& p, int dtype, hipStream_t stream) {
    if (dtype == 0) return p.D == 64 ? launch_build_t<64, Bf16>(p, stream) : launch_build_t<128, Bf16>(p, stream);
    return p.D == 64 ? launch_build_t<64, F32>(p, stream) : launch_build_t<128, F32>(p, stream);
}

template <int G, int D, typename E>
static hipError_t launch_decode_t(const PPParams& p, hipStream_t stream) {
    const int nblk = (p.M + kPPRouteRows - 1) / kPPRouteRows;
    hipLaunchKernelGGL((pp_route_kernel<G, D, E>), dim3((unsigned)(p.B * p.Hkv * nblk)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)kSelectBins * 4 + 256 + (size_t)p.Mpad;
    e = allow_lds(reinterpret_cast<const void*>(&pp_select_kernel), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pp_select_kernel, dim3((unsigned)(p.B * p.Hq)), dim3(kPPSelectThreads), lds, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pp_attend_kernel<G, D, E>), dim3((unsigned)(p.B * p.Hkv * p.NC)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, typename E>
static hipError_t launch_decode_d(const PPParams& p, hipStream_t stream) {
    switch (p.G) {
        case 1: return launch_decode_t<1, D, E>(p, stream);
        case 2: return launch_decode_t<2, D, E>(p, stream);
        case 4: return launch_decode_t<4, D, E>(p, stream);
        case 7: return launch_decode_t<7, D, E>(p, stream);
        case 8: return launch_decode_t<8, D, E>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_pp_decode(const PPParams& p, int dtype, hipStream_t stream) {
    if (dtype == 0) return p.D == 64 ? launch_decode_d<64, Bf16>(p, stream) : launch_decode_d<128, Bf16>(p, stream);
    return p.D == 64 ? launch_decode_d<64, F32>(p, stream) : launch_decode_d<128, F32>(p, stream);
}

}  // namespace santa
