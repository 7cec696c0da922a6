// Sample pass of SANTA decode: global partition function, per-split sample
// budget, inverse-CDF sampling and the gather-and-add of sampled V rows
// ("Stochastic Sparse Attention for Memory-Bound Inference", §3.2 steps 2-3;
// estimator §2, Eq. 3; strata and shared offset §2.1; inverse CDF Appendix A.4).
//
// One workgroup per (sequence b, KV head g, split t), the same grid as the
// score pass so that a split's stashed scores are read on the XCD that wrote
// them.  For each of its G query heads (one wave per head):
//
//  A. From the split statistics of all splits of the head: M = max m_j,
//     w_j = l_j exp(m_j - M), fp64 prefix W_j and Z = W_T.  Every workgroup of
//     the head runs this identical fixed-order computation, so all agree on the
//     bits of every W_j.  Split t owns the targets tau_m = t_m * Z with
//     W_t <= tau_m < W_{t+1} (the last split of positive mass also owns targets
//     that round to >= Z): the proportional budget of §3.2, exact per target.
//     The index range [m_lo, m_hi) of those targets is found with a 64-ary
//     search over the non-decreasing target sequence.
//  B. In-split CDF: e_i = exp(s_i - m_t) as 52-bit fixed point, prefix sums in
//     exact integer arithmetic (order-free, hence monotone and deterministic),
//     boundaries C_{i+1} = W_t + exp(m_t - M) * P_i in LDS.
//  C. Merge path of the split's sorted targets against the sorted boundaries:
//     target tau gets the key j with C_j <= tau < C_{j+1}; it is written to idx
//     and counted in an LDS histogram (per head, per key).
//  D. The union over the G heads of keys with a count (each distinct V row once).
//  E. Gather-and-add: each distinct row is read once (16-byte loads) and added
//     with weight count_h to head h's fp32 accumulator; the per-split partial
//     sum, times 1/S, is added atomically into o.
#include "santa_device.h"
#include "santa_internal.h"

namespace santa {

namespace {

struct HeadInfo {
    double w_lo;      // mass below this split (W_t)
    double z;         // total mass Z
    double f;         // exp(m_t - M)
    double u0;        // systematic offset
    float m_t;        // this split's maximum score
    int m_lo, m_hi;   // targets [m_lo, m_hi) fall into this split
    int pad;
};

struct TargetSeq {
    const double* sorted;   // multinomial: sorted uniforms of this head
    double u0;
    uint64_t seed;
    int mode, S, b, hq;
    // t_m of §2 / §2.1: sorted uniform, (m + U_m) / S or (m + U) / S
    __device__ __forceinline__ double at(int m) const {
        if (mode == 0) return sorted[m];
        const double u = (mode == 1) ? uniform01(seed, b, hq, (uint64_t)m) : u0;
        return ((double)m + u) / (double)S;
    }
};

// Number of m in [0, S) with t_m * z < x (t_m non-decreasing in m).  Whole
// wave; each round probes 64 evenly spaced positions.
__device__ int count_below(const TargetSeq& ts, double z, double x, int lane) {
    int lo = 0, hi = ts.S;              // answer in [lo, hi]
    while (hi > lo) {
        const int len = hi - lo;
        const int step = (len + 63) >> 6;
        const int pos = lo + (lane + 1) * step - 1;
        const bool below = (pos < hi) && (ts.at(pos) * z < x);
        const int k = __popcll(__ballot(below));
        if (step == 1) return lo + k;
        const int nlo = lo + k * step;
        hi = min(hi, lo + (k + 1) * step - 1);
        lo = nlo;
    }
    return lo;
}

struct SampleLayout {
    size_t cdf, tau, red, cnt, rows, info, misc, total;
};

__host__ __device__ inline SampleLayout sample_layout(int G, int D, int split) {
    SampleLayout L;
    const size_t cdf_bytes = (size_t)kWaves * split * sizeof(double);
    const size_t tau_bytes = (size_t)kWaves * kTargetChunk * sizeof(double);
    const size_t red_bytes = (size_t)kWaves * G * D * sizeof(float);
    L.cdf = 0;
    L.tau = cdf_bytes;
    L.red = 0;                                         // reuses cdf/tau after the merge
    size_t region = cdf_bytes + tau_bytes;
    if (red_bytes > region) region = red_bytes;
    L.cnt = region;
    L.rows = L.cnt + (size_t)G * split * sizeof(uint32_t);
    L.info = (L.rows + (size_t)split * sizeof(int) + 15) & ~(size_t)15;
    L.misc = L.info + (size_t)G * sizeof(HeadInfo);
    L.total = L.misc + 16;
    return L;
}

}  // namespace

size_t sample_lds_bytes(int G, int D, int split) { return sample_layout(G, D, split).total; }

template <int G, int D, typename E>
__global__ __launch_bounds__(kBlock) void sample_kernel(Params p) {
    constexpr int LPR = D * E::bytes / 16;
    constexpr int RPL = 64 / LPR;
    constexpr int EPL = 16 / E::bytes;

    extern __shared__ __align__(16) unsigned char smem[];
    const SampleLayout L = sample_layout(G, D, p.split);
    double* cdf_all = reinterpret_cast<double*>(smem + L.cdf);
    double* tau_all = reinterpret_cast<double*>(smem + L.tau);
    float* red = reinterpret_cast<float*>(smem + L.red);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(smem + L.cnt);
    int* rows = reinterpret_cast<int*>(smem + L.rows);
    HeadInfo* info = reinterpret_cast<HeadInfo*>(smem + L.info);
    int* misc = reinterpret_cast<int*>(smem + L.misc);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int t = blockIdx.x % p.T;
    const int bg = blockIdx.x / p.T;
    const int g = bg % p.Hkv;
    const int b = bg / p.Hkv;
    const int n = seq_len_of(p, b);

    if (n == 0) {          // empty sequence: o stays 0, idx = -1
        if (t == 0) {
            int32_t* dst = p.idx + ((int64_t)b * p.Hq + (int64_t)g * G) * p.S;
            for (int i = tid; i < G * p.S; i += kBlock) dst[i] = -1;
        }
        return;
    }
    const int Tb = (n + p.split - 1) / p.split;
    if (t >= Tb) return;
    const int key0 = t * p.split;
    const int ns = min(p.split, n - key0);

    for (int i = tid; i < G * p.split; i += kBlock) cnt[i] = 0u;
    if (tid == 0) misc[0] = 0;

    // ---- A: global partition function and this split's target range ------
    for (int h = wave; h < G; h += kWaves) {
        const int hq = g * G + h;
        const SplitStat* st = p.stats + ((int64_t)b * p.Hq + hq) * p.T;
        float mx = -INFINITY;
        for (int j = lane; j < Tb; j += 64) mx = fmaxf(mx, st[j].m);
        const float M = wave_max_f32(mx);
        double carry = 0.0, w_lo = 0.0, w_hi = 0.0, f_t = 0.0;
        int last = -1;
        for (int j0 = 0; j0 < Tb; j0 += 64) {
            const int j = j0 + lane;
            double w = 0.0, f = 0.0;
            if (j < Tb) {
                const SplitStat s = st[j];
                f = exp((double)s.m - (double)M);
                w = s.l * f;
            }
            if (w > 0.0) last = j;
            const double incl = carry + wave_inclusive_scan_f64(w, lane);   // W_{j+1}
            if (j == t) {
                w_hi = incl;
                f_t = f;
            }
            if (j == t - 1) w_lo = incl;
            carry = __shfl(incl, 63, 64);
        }
        last = wave_max_i32(last);
        w_hi = __shfl(w_hi, t & 63, 64);
        f_t = __shfl(f_t, t & 63, 64);
        w_lo = (t == 0) ? 0.0 : __shfl(w_lo, (t - 1) & 63, 64);
        const double z = carry;

        TargetSeq ts;
        ts.sorted = p.targets + ((int64_t)b * p.Hq + hq) * p.S;
        ts.seed = p.seed;
        ts.mode = p.mode;
        ts.S = p.S;
        ts.b = b;
        ts.hq = hq;
        ts.u0 = (p.mode == 2) ? uniform01(p.seed, b, hq, 0ull) : 0.0;
        const int m_lo = count_below(ts, z, w_lo, lane);
        const int m_hi = (t == last) ? p.S : count_below(ts, z, w_hi, lane);
        if (lane == 0) {
            HeadInfo hi;
            hi.w_lo = w_lo;
            hi.z = z;
            hi.f = f_t;
            hi.u0 = ts.u0;
            hi.m_t = st[t].m;
            hi.m_lo = m_lo;
            hi.m_hi = max(m_hi, m_lo);
            hi.pad = 0;
            info[h] = hi;
        }
    }
    __syncthreads();
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) any |= info[h].m_hi > info[h].m_lo;
    if (!any) return;      // no sample lands in this split: its V rows are never read

    // ---- B + C: in-split CDF and merge-path sampling, one wave per head ----
    const int ept = p.split >> 6;          // keys per lane in the scan (<= 16)
    for (int h = wave; h < G; h += kWaves) {
        const HeadInfo hi = info[h];
        if (hi.m_hi <= hi.m_lo) continue;
        const int hq = g * G + h;
        double* cdf = cdf_all + wave * p.split;
        double* tau = tau_all + wave * kTargetChunk;
        const float* srow = p.scores + ((int64_t)b * p.Hq + hq) * p.score_row + key0;

        uint64_t part[16];
        uint64_t run = 0;
        int lastpos = -1;
        for (int k = 0; k < 16; ++k) {
            if (k < ept) {
                const int i = lane * ept + k;
                uint64_t e = 0;
                if (i < ns) {
                    e = fixed_mass(mass_exp(srow[i] - hi.m_t));
                    if (e) lastpos = i;
                }
                run += e;
                part[k] = run;
            }
        }
        // exclusive prefix of the lane totals (exact integer scan)
        uint64_t incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint64_t y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        const uint64_t excl = incl - run;
        const double scale = hi.f * kFixedUnit;
        for (int k = 0; k < 16; ++k) {
            if (k < ept) {
                const int i = lane * ept + k;
                if (i < ns) cdf[i] = hi.w_lo + scale * (double)(excl + part[k]);
            }
        }
        lastpos = wave_max_i32(lastpos);

        TargetSeq ts;
        ts.sorted = p.targets + ((int64_t)b * p.Hq + hq) * p.S;
        ts.seed = p.seed;
        ts.mode = p.mode;
        ts.S = p.S;
        ts.b = b;
        ts.hq = hq;
        ts.u0 = hi.u0;
        int32_t* idx_row = p.idx + ((int64_t)b * p.Hq + hq) * p.S;
        uint32_t* cnt_h = cnt + h * p.split;
        for (int m0 = hi.m_lo; m0 < hi.m_hi; m0 += kTargetChunk) {
            const int na = min(kTargetChunk, hi.m_hi - m0);
            for (int k = lane; k < na; k += 64) tau[k] = ts.at(m0 + k) * hi.z;
            wave_lds_sync();
            // merge path: lane takes an equal share of the merged sequence
            // (boundaries before targets on ties, so a target equal to C_j
            // lands on key j: half-open intervals)
            const int total = na + ns;
            const int per = (total + 63) >> 6;
            const int d0 = min(lane * per, total);
            const int d1 = min(d0 + per, total);
            int lo = max(0, d0 - ns), up = min(d0, na);
            while (lo < up) {
                const int mid = (lo + up) >> 1;
                if (tau[mid] < cdf[d0 - 1 - mid]) lo = mid + 1;
                else up = mid;
            }
            int i = lo, j = d0 - lo;
            for (int d = d0; d < d1; ++d) {
                if (i < na && (j >= ns || tau[i] < cdf[j])) {
                    // j = number of boundaries <= tau: key j, or past the
                    // split's last boundary (rounding): last key of positive mass
                    const int local = (j < ns) ? j : max(lastpos, 0);
                    idx_row[m0 + i] = key0 + local;
                    atomicAdd(&cnt_h[local], 1u);
                    ++i;
                } else {
                    ++j;
                }
            }
            wave_lds_sync();
        }
    }
    __syncthreads();

    // ---- D: distinct rows over the G heads ---------------------------------
    for (int i = tid; i < ns; i += kBlock) {
        bool used = false;
#pragma unroll
        for (int h = 0; h < G; ++h) used |= cnt[h * p.split + i] != 0u;
        if (used) rows[atomicAdd(&misc[0], 1)] = i;
    }
    __syncthreads();

    // ---- E: gather-and-add ---------------------------------------------------
    const int nr = misc[0];
    const int c = lane / LPR;
    const int li = lane % LPR;
    const int slot = wave * RPL + c;
    constexpr int kSlots = kWaves * RPL;
    float acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    const char* vbase = reinterpret_cast<const char*>(p.v);
    for (int k = slot; k < nr; k += kSlots) {
        const int local = rows[k];
        const uint4 raw = load16(vbase + row_offset(p, b, g, key0 + local) * E::bytes + li * 16);
        float x[EPL];
        E::widen16(raw, x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float w = (float)cnt[h * p.split + local];
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w, x[e], acc[h][e]);
        }
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);
    if (c == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) red[(wave * G + h) * D + li * EPL + e] = acc[h][e];
    }
    __syncthreads();
    const float inv_s = 1.0f / (float)p.S;
    float* o = p.o + ((int64_t)b * p.Hq + (int64_t)g * G) * D;
    for (int i = tid; i < G * D; i += kBlock) {
        const int h = i / D;
        if (info[h].m_hi > info[h].m_lo) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += red[w * G * D + i];
            unsafeAtomicAdd(o + i, s * inv_s);
        }
    }
}

template <int G, int D, typename E>
static hipError_t launch_sample_t(const Params& p, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.T));
    hipLaunchKernelGGL((sample_kernel<G, D, E>), grid, dim3(kBlock),
                       sample_lds_bytes(G, D, p.split), stream, p);
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
