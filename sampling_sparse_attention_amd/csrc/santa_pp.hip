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
// Decoding (four launches; the launch boundaries order every exchange, so
// no kernel waits on another workgroup or fences):
//   pp_route_kernel   one workgroup per (sequence, KV head, block of teams):
//                     the G query heads' routing logits phi = log n_g +
//                     q . l_g / sqrt(d) and Gumbel-perturbed scores Y (and the
//                     block's words of the group's selection mask cleared);
//   pp_select_kernel  one workgroup per (sequence, query head): the K largest
//                     Y by radix selection (ties to the lower team index), the
//                     threshold tau = the (K+1)-th, and the corrections
//                     c_g = 1 - exp(-exp(phi_g - tau)); each head marks its
//                     teams in the group's mask (a byte of head bits per team);
//   pp_attend_kernel  NC workgroups per (sequence, KV head) compact the mask
//                     into the group's read plan (each team once, with the
//                     heads that chose it), read their share of its rows and
//                     of the exact suffix once for the whole group, and
//                     accumulate each head's online softmax over its own teams
//                     with logits s - log c_g (so 1/c_g weighs both sums of
//                     Eq. 4);
//   pp_reduce_kernel  one workgroup per query head merges the partial results.
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

// One workgroup per (sequence, KV head, block of kPPRouteRows teams): every
// wave issues all its representative-row loads first, the workgroup draws the
// block's Gumbel variates while they are in flight, then the dot products.
template <int G, int D, typename E>
__global__ __launch_bounds__(256) void pp_route_kernel(PPParams p) {
    constexpr int LPR = D * E::bytes / 16;       // lanes per representative row
    constexpr int RPW = 64 / LPR;                // rows per wave-wide load
    constexpr int ITER = kPPRouteRows / (4 * RPW);
    static_assert(LPR >= G, "one lane of a row group per query head");
    static_assert(ITER * 4 * RPW == kPPRouteRows, "rows per workgroup");
    __shared__ float s_gum[kPPRouteRows][G];
    __shared__ float s_logn[kPPRouteRows];
    const int nblk = (p.M + kPPRouteRows - 1) / kPPRouteRows;
    const int blk = blockIdx.x % nblk;
    const int bg = blockIdx.x / nblk;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane % LPR, rsub = lane / LPR;
    const int t_base = blk * kPPRouteRows;
    const int t_end = min(p.M, t_base + kPPRouteRows);
    const char* qb = reinterpret_cast<const char*>(p.q) + (((int64_t)b * p.Hq + (int64_t)g * G) * D) * E::bytes + li * 16;
    uint4 qf[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qf[h] = load16(qb + (int64_t)h * D * E::bytes);
    const char* rk = reinterpret_cast<const char*>(p.rep_k) + ((int64_t)bg * p.M) * D * E::bytes + li * 16;
    uint4 kd[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int t = t_base + it * 4 * RPW + wave * RPW + rsub;
        kd[it] = load16_stream(rk + (int64_t)(t < t_end ? t : t_base) * D * E::bytes);
    }
    const int32_t* ts = p.team_start + (int64_t)bg * (p.M + 1);
    // this block's words of the group's selection mask start the call at zero
    // (kPPRouteRows is a multiple of 4: the blocks' words do not overlap)
    if (threadIdx.x < kPPRouteRows / 4 && t_base + 4 * (int)threadIdx.x < p.Mpad)
        p.mask[(int64_t)bg * (p.Mpad / 4) + t_base / 4 + threadIdx.x] = 0u;
    for (int pr = threadIdx.x; pr < kPPRouteRows * G; pr += 256) {
        const int tl = pr / G, h = pr - tl * G;
        if (t_base + tl < t_end) s_gum[tl][h] = (float)pp_gumbel(p.seed, b, g * G + h, t_base + tl);
    }
    if (threadIdx.x < kPPRouteRows && t_base + (int)threadIdx.x < t_end) {
        const int t = t_base + threadIdx.x;
        s_logn[threadIdx.x] = logf((float)(ts[t + 1] - ts[t]));
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int tl = it * 4 * RPW + wave * RPW + rsub;
        const int t = t_base + tl;
        float dot[G];
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = E::dot16(kd[it], qf[h], 0.0f);
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1)
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] += __shfl_xor(dot[h], m, 64);
        if (t < t_end && li < G) {
            float sv = 0.0f;
#pragma unroll
            for (int h = 0; h < G; ++h)
                if (h == li) sv = dot[h];
            const float ph = s_logn[tl] + sv * p.scale;
            const int64_t at = ((int64_t)b * p.Hq + g * G + li) * p.Mpad + t;
            p.phi[at] = ph;
            p.y[at] = ph + s_gum[tl][li];
        }
    }
}

// ---------------------------------------------------------------------------
// Selection and the group's read plan
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mark_team(unsigned int* mask, int t, unsigned int bit) {
    __hip_atomic_fetch_or(mask + (t >> 2), bit << (8 * (t & 3)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kPPRegVals = 16;      // scores per thread held in registers (M <= 16384)
constexpr int kPPStage = 1024;      // kept teams staged in LDS before their corrections

// A kept team: its slot in the output, its correction (Eq. 7, fp64), its log c
// for the attention and its bit in the group's mask.
__device__ __forceinline__ void keep_team(const PPParams& p, int32_t* teams, float* corr, float* lc,
                                          unsigned int* mask, unsigned int bit, int pos, int t, float phi,
                                          double tau) {
    const double c = -expm1(-exp((double)phi - tau));
    teams[pos] = t;
    corr[pos] = (float)c;
    lc[t] = (float)log(c);
    mark_team(mask, t, bit);
}

__global__ __launch_bounds__(kPPSelectThreads) void pp_select_kernel(PPParams p) {
    constexpr int NT = kPPSelectThreads;
    __shared__ unsigned int hist[kSelectBins];
    __shared__ int scan[2 * (NT / 64) + 4];
    __shared__ int s_team[kPPStage];
    __shared__ float s_phi[kPPStage];
    const int bh = blockIdx.x;
    const int b = bh / p.Hq, hq = bh - b * p.Hq;
    const int g = hq / p.G, h = hq - g * p.G;
    const int tid = threadIdx.x;
    const int M = p.M, K = p.K, Keff = p.Keff;
    int32_t* teams = p.teams + (int64_t)bh * (K + 1);
    float* corr = p.corr + (int64_t)bh * K;
    const float* yrow = p.y + (int64_t)bh * p.Mpad;
    const float* prow = p.phi + (int64_t)bh * p.Mpad;
    float* lc = p.logc + (int64_t)bh * p.Mpad;
    unsigned int* mask = p.mask + (int64_t)(b * p.Hkv + g) * (p.Mpad / 4);
    const unsigned int bit = 1u << h;
    if (Keff == M) {
        // every team, with c = 1 (Algorithm 1, lines 4-5)
        for (int j = tid; j <= K; j += NT) teams[j] = j < M ? j : -1;
        for (int j = tid; j < K; j += NT) corr[j] = j < M ? 1.0f : 0.0f;
        for (int t = tid; t < M; t += NT) {
            lc[t] = 0.0f;
            mark_team(mask, t, bit);
        }
    } else if (M <= NT * kPPRegVals) {
        // the row in registers: thread t holds teams [16t, 16t + 16)
        const int i0 = tid * kPPRegVals;
        const int nvalid = max(0, min(kPPRegVals, M - i0));
        uint32_t key[kPPRegVals];
        float ph[kPPRegVals];
#pragma unroll
        for (int j = 0; j < kPPRegVals / 4; ++j) {
            float4 yv = make_float4(0.f, 0.f, 0.f, 0.f), pv = yv;
            if (i0 + 4 * j < p.Mpad) {
                yv = *reinterpret_cast<const float4*>(yrow + i0 + 4 * j);
                pv = *reinterpret_cast<const float4*>(prow + i0 + 4 * j);
            }
            key[4 * j] = score_key(yv.x);
            key[4 * j + 1] = score_key(yv.y);
            key[4 * j + 2] = score_key(yv.z);
            key[4 * j + 3] = score_key(yv.w);
            ph[4 * j] = pv.x;
            ph[4 * j + 1] = pv.y;
            ph[4 * j + 2] = pv.z;
            ph[4 * j + 3] = pv.w;
        }
        int krem = 0;
        const uint32_t kth = radix_kth_regs<NT, kPPRegVals>(key, nvalid, Keff + 1, hist, scan, &krem);
        // the Keff + 1 largest, in index order, are the keys above kth and the
        // first krem keys equal to it; the last of those (equal rank krem - 1) is
        // the threshold team, whose score is kth's value
        const double tau = (double)key_value(kth);
        int n_eq = 0, n_gt = 0;
#pragma unroll
        for (int e = 0; e < kPPRegVals; ++e) {
            if (e < nvalid) {
                n_gt += key[e] > kth ? 1 : 0;
                n_eq += key[e] == kth ? 1 : 0;
            }
        }
        const int eq_before = block_exclusive_sum<NT>(n_eq, scan);
        const int take_eq = max(0, min(n_eq, krem - eq_before));
        const int has_thr = (eq_before <= krem - 1 && krem - 1 < eq_before + n_eq) ? 1 : 0;
        int pos = block_exclusive_sum<NT>(n_gt + take_eq - has_thr, scan);
        int eq_seen = 0;
        const bool staged = Keff <= kPPStage;
#pragma unroll
        for (int e = 0; e < kPPRegVals; ++e) {
            if (e >= nvalid) continue;
            bool keep = key[e] > kth;
            if (key[e] == kth) {
                if (eq_before + eq_seen == krem - 1) {
                    teams[K] = i0 + e;
                    keep = false;
                } else {
                    keep = eq_seen < take_eq;
                }
                ++eq_seen;
            }
            if (keep && pos < Keff) {
                if (staged) {
                    s_team[pos] = i0 + e;
                    s_phi[pos] = ph[e];
                    ++pos;
                } else {
                    keep_team(p, teams, corr, lc, mask, bit, pos++, i0 + e, ph[e], tau);
                }
            }
        }
        if (staged) {
            // the corrections one kept team per thread, instead of once per
            // register slot in every wave that keeps a team there
            __syncthreads();
            for (int j = tid; j < Keff; j += NT) keep_team(p, teams, corr, lc, mask, bit, j, s_team[j], s_phi[j], tau);
        }
    } else {
        // long rows: the same from memory
        const int C = ((M + NT - 1) / NT + 3) & ~3;
        const int i0 = min(M, tid * C), i1 = min(M, i0 + C);
        int krem = 0;
        const uint32_t kth = radix_kth<NT>(yrow, i0, i1, Keff + 1, hist, scan, &krem);
        const double tau = (double)key_value(kth);
        int n_eq = 0, n_gt = 0;
        for (int i = i0; i < i1; ++i) {
            const uint32_t kk = score_key(yrow[i]);
            n_gt += kk > kth ? 1 : 0;
            n_eq += kk == kth ? 1 : 0;
        }
        const int eq_before = block_exclusive_sum<NT>(n_eq, scan);
        const int take_eq = max(0, min(n_eq, krem - eq_before));
        const int has_thr = (eq_before <= krem - 1 && krem - 1 < eq_before + n_eq) ? 1 : 0;
        int pos = block_exclusive_sum<NT>(n_gt + take_eq - has_thr, scan);
        int eq_seen = 0;
        for (int i = i0; i < i1; ++i) {
            const uint32_t kk = score_key(yrow[i]);
            bool keep = kk > kth;
            if (kk == kth) {
                if (eq_before + eq_seen == krem - 1) {
                    teams[K] = i;
                    keep = false;
                } else {
                    keep = eq_seen < take_eq;
                }
                ++eq_seen;
            }
            if (keep && pos < Keff) keep_team(p, teams, corr, lc, mask, bit, pos++, i, prow[i], tau);
        }
    }
}

// ---------------------------------------------------------------------------
// Selected attention over the group's plan and the exact suffix
// ---------------------------------------------------------------------------
constexpr int kPPEntryBlock = 256;      // plan entries staged in LDS at a time
constexpr int kPPRowsInFlight = 4;      // rows a lane group loads before consuming them

template <int G, int D, typename E>
__global__ __launch_bounds__(256) void pp_attend_kernel(PPParams p) {
    constexpr int LPR = D * E::bytes / 16;       // lanes per row
    constexpr int RPW = 64 / LPR;                // rows per wave-wide load
    constexpr int ELV = 16 / E::bytes;           // elements per lane piece
    constexpr int NG = 4 * RPW;                  // lane groups of the workgroup
    constexpr int UL = kPPRowsInFlight;
    constexpr int EB = kPPEntryBlock;
    __shared__ int s_team[EB], s_first[EB], s_mask[EB], s_pref[EB + 1];
    __shared__ float s_lc[EB][G];
    __shared__ float s_m[NG][G], s_l[NG][G], s_w[NG][G], s_mx[G];
    __shared__ float s_acc[NG][G][D];
    __shared__ int s_scan[2 * 4 + 4];
    __shared__ int s_U;
    const int c = blockIdx.x % p.NC;
    const int bg = blockIdx.x / p.NC;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
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
    auto consume = [&](const uint4& kv, const uint4& vv, const float* lc, unsigned int heads) {
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
            const float x = dot[h] * p.scale - (lc ? lc[h] : 0.0f);
            const float mn = fmaxf(m[h], x);
            const float so = __expf(m[h] - mn);
            const float pe = __expf(x - mn);
            l[h] = l[h] * so + pe;
#pragma unroll
            for (int e = 0; e < ELV; ++e) acc[h][e] = acc[h][e] * so + pe * vf[e];
            m[h] = mn;
        }
    };
    // The group's read plan is its selection mask, compacted in team order: the
    // heads' marks are complete (the selection is an earlier launch); every
    // chunk counts the selected teams and takes its share of them.
    const unsigned int* mask = p.mask + (int64_t)bg * (p.Mpad / 4);
    const int MW = p.Mpad / 4;
    const int CW = (MW + 255) / 256;
    const int w0 = min(MW, tid * CW), w1 = min(MW, w0 + CW);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) {
        const unsigned int mw = mask[w];
        cnt += ((mw & 0xFFu) != 0) + ((mw & 0xFF00u) != 0) + ((mw & 0xFF0000u) != 0) + ((mw & 0xFF000000u) != 0);
    }
    const int at = block_exclusive_sum<256>(cnt, s_scan);
    if (tid == 255) s_U = at + cnt;
    __syncthreads();
    const int U = s_U;
    const int e0 = (int)((int64_t)U * c / p.NC), e1 = (int)((int64_t)U * (c + 1) / p.NC);
    const int32_t* ts = p.team_start + (int64_t)bg * (p.M + 1);
    const char* pk = reinterpret_cast<const char*>(p.packed_k) + ((int64_t)bg * p.N) * D * E::bytes + li * 16;
    const char* pv = reinterpret_cast<const char*>(p.packed_v) + ((int64_t)bg * p.N) * D * E::bytes + li * 16;
    for (int eb = e0; eb < e1; eb += EB) {
        // stage EB entries: team, heads, first row, log c per head, and the row prefix
        const int ne = min(EB, e1 - eb);
        if (cnt > 0 && at < eb + ne && at + cnt > eb) {
            int pos = at;
            for (int w = w0; w < w1; ++w) {
                const unsigned int mw = mask[w];
                for (int e = 0; e < 4; ++e) {
                    const unsigned int hm = (mw >> (8 * e)) & 0xFFu;
                    if (!hm) continue;
                    if (pos >= eb && pos < eb + ne) {
                        s_team[pos - eb] = 4 * w + e;
                        s_mask[pos - eb] = (int)hm;
                    }
                    ++pos;
                }
            }
        }
        __syncthreads();
        int sz = 0;
        if (tid < ne) {
            const int t = s_team[tid];
            const unsigned int heads = (unsigned int)s_mask[tid];
            const int r0 = ts[t];
            sz = ts[t + 1] - r0;
            s_first[tid] = r0;
#pragma unroll
            for (int h = 0; h < G; ++h)
                s_lc[tid][h] = ((heads >> h) & 1u) ? p.logc[((int64_t)b * p.Hq + g * G + h) * p.Mpad + t] : 0.0f;
        }
        const int pre = block_exclusive_sum<256>(sz, s_scan);
        if (tid < ne) s_pref[tid] = pre;
        if (tid == ne - 1) s_pref[ne] = pre + sz;
        __syncthreads();
        const int total = s_pref[ne];
        // rows of the staged entries, lane group grp taking rows grp, grp + NG, ...
        for (int r0 = grp; r0 < total; r0 += NG * UL) {
            uint4 kv[UL], vv[UL];
            int ei[UL];
#pragma unroll
            for (int u = 0; u < UL; ++u) {
                const int r = r0 + u * NG;
                const int rr = r < total ? r : 0;
                int lo = 0, hi = ne - 1;                   // the entry holding row rr
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_pref[mid] <= rr) lo = mid;
                    else hi = mid - 1;
                }
                ei[u] = r < total ? lo : -1;
                const int64_t row = s_first[lo] + (rr - s_pref[lo]);
                kv[u] = load16_stream(pk + row * D * E::bytes);
                vv[u] = load16_stream(pv + row * D * E::bytes);
            }
#pragma unroll
            for (int u = 0; u < UL; ++u)
                if (ei[u] >= 0) consume(kv[u], vv[u], s_lc[ei[u]], (unsigned int)s_mask[ei[u]]);
        }
        __syncthreads();
    }
    // the exact suffix: rows N .. seq_len - 1 of the token-major cache, weight 1 for every head
    const int n = min(max(p.seq_lens[b], p.N), p.n_max);
    const int ns = n - p.N;
    if (ns > 0) {
        const int s0 = p.N + (int)((int64_t)ns * c / p.NC), s1 = p.N + (int)((int64_t)ns * (c + 1) / p.NC);
        const char* kc = reinterpret_cast<const char*>(p.k) + li * 16;
        const char* vc = reinterpret_cast<const char*>(p.v) + li * 16;
        for (int i0 = s0 + grp; i0 < s1; i0 += NG * UL) {
            uint4 kv[UL], vv[UL];
#pragma unroll
            for (int u = 0; u < UL; ++u) {
                const int i = i0 + u * NG < s1 ? i0 + u * NG : s0;
                const int64_t off = pp_row(p, b, g, i) * E::bytes;
                kv[u] = load16_stream(kc + off);
                vv[u] = load16_stream(vc + off);
            }
#pragma unroll
            for (int u = 0; u < UL; ++u)
                if (i0 + u * NG < s1) consume(kv[u], vv[u], nullptr, (1u << G) - 1u);
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
    if (tid < G) {
        float mx = -INFINITY;
        for (int q = 0; q < NG; ++q) mx = fmaxf(mx, s_m[q][tid]);
        s_mx[tid] = mx;
    }
    __syncthreads();
    if (tid < NG * G) {
        const int q = tid / G, h = tid - q * G;
        s_w[q][h] = s_m[q][h] == -INFINITY ? 0.0f : __expf(s_m[q][h] - s_mx[h]);
    }
    __syncthreads();
    for (int idx = tid; idx < G * (D + 2); idx += 256) {
        const int h = idx / (D + 2), col = idx - h * (D + 2);
        float val = s_mx[h];
        if (col > 0) {
            val = 0.0f;
            for (int q = 0; q < NG; ++q) val += s_w[q][h] * (col == 1 ? s_l[q][h] : s_acc[q][h][col - 2]);
        }
        p.part[(((int64_t)b * p.Hq + g * G + h) * p.NC + c) * (D + 2) + col] = val;
    }
}

// The chunks' partial results of one query head, brought to a common scale and
// divided (Eq. 4: o = U_hat / Z_hat): thread col of a D-thread workgroup.
template <int D>
__global__ __launch_bounds__(D) void pp_reduce_kernel(PPParams p) {
    const int bh = blockIdx.x;
    const int col = threadIdx.x;
    const float* pr = p.part + (int64_t)bh * kPPChunks * (D + 2);
    float mq[kPPChunks], lq[kPPChunks], aq[kPPChunks];
#pragma unroll
    for (int q = 0; q < kPPChunks; ++q) {
        mq[q] = pr[q * (D + 2)];
        lq[q] = pr[q * (D + 2) + 1];
        aq[q] = pr[q * (D + 2) + 2 + col];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < kPPChunks; ++q) mx = fmaxf(mx, mq[q]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int q = 0; q < kPPChunks; ++q) {
        const float w = mq[q] == -INFINITY ? 0.0f : __expf(mq[q] - mx);
        L += w * lq[q];
        A += w * aq[q];
    }
    p.o[(int64_t)bh * D + col] = L > 0.0f ? A / L : 0.0f;
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
    hipLaunchKernelGGL(pp_select_kernel, dim3((unsigned)(p.B * p.Hq)), dim3(kPPSelectThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pp_attend_kernel<G, D, E>), dim3((unsigned)(p.B * p.Hkv * p.NC)), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pp_reduce_kernel<D>), dim3((unsigned)(p.B * p.Hq)), dim3(D), 0, stream, p);
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
