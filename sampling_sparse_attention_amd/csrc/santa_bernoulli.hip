// Bernoulli qK^T with the mean group query, combined with SANTA ("Stochastic
// Sparse Attention for Memory-Bound Inference", section 5, Eq. 5; section 5.1,
// Eq. 6; section 5.3).  The scores of a GQA group are estimated from one
// stochastic representative query: m = mean over the group of |q_h|; each
// feature i is kept by B stratified draws with probability m_i / max m
// (draw n keeps it iff (n + U_{i,n}) / B < m_i / max m, U from Philox4x64-10
// with key (seed, 1) and counter (n, i, g, b)); m_hat_i = (max m / B) count_i;
// and head h's score of key j is sum_i (m_hat_i / m_i) q_{h,i} k_{j,i}.  Only
// the kept features' key values are read, from a channel-major copy of K
// (K^T: [B, Hkv, d, tokens], tokens contiguous), so that skipping a feature
// skips its bytes.  The SANTA step that follows (statistics, global budget,
// sampling, gather of token-major V rows) is the one of the exact path.
//
// Every workgroup derives its group's feature counts itself (a few Philox
// draws per feature, see bern_count); the first split of each group writes
// them to the caller's [B, Hkv, d] array.
//
//   bern_fused_kernel    the fused decode kernel with the estimated scores;
//   bern_score_kernel    the score pass of the two-kernel path (the sample
//                        pass is the exact path's).
#include <type_traits>

#include "santa_split.h"

namespace santa {

// The uniform of draw n of feature i of group (b, g).
__device__ __forceinline__ double bern_uniform(uint64_t seed, int b, int g, int i, int n) {
    const uint64_t w = philox4x64_10_word0((uint64_t)n, (uint64_t)i, (uint64_t)g, (uint64_t)b, seed, 1ull);
    return (double)(w >> 11) * 0x1p-53;
}

// Maximum of a double over the first `nw` waves of the workgroup (every
// thread of the workgroup calls it; the result is returned to all of them).
__device__ __forceinline__ double block_max_f64(double v, int nw, double* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    if (lane == 0 && wave < nw) lds[wave] = v;
    __syncthreads();
    double r = lds[0];
    for (int w = 1; w < nw; ++w) r = fmax(r, lds[w]);
    __syncthreads();
    return r;
}

// m_i = (1/G) sum_h |q_{h,i}| for the feature of this thread (threads < D),
// heads summed in order in fp64 (the decisions below are taken in fp64).
template <int G, typename E>
__device__ __forceinline__ double mean_abs_query(const Params& p, int b, int g, int i, float (&qv)[G]) {
    const char* qb = reinterpret_cast<const char*>(p.q) + ((int64_t)b * p.Hq + (int64_t)g * G) * p.D * E::bytes;
    double m = 0.0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        qv[h] = E::elem(qb, (int64_t)h * p.D + i);
        m += fabs((double)qv[h]);
    }
    return m / (double)G;
}

// How many of the B stratified draws keep a feature of keep probability pi:
// draw n keeps it iff (n + U_n) / B < pi, in fp64.  Whatever U in [0, 1) is,
// the rounded (n + U) / B lies in [fl(n / B), fl((n + 1) / B)] (rounding is
// monotone and n + 1 is exact), so draw n is kept for certain when
// fl((n + 1) / B) < pi and never when fl(n / B) >= pi; only the other draws
// need their uniform.  With n0 = floor(B pi) (B <= 64, so 1/B dwarfs the
// rounding) every draw below n0 - 1 is certain and every draw above n0 + 1
// impossible, so three draws are looked at; and at most one of them needs its
// uniform (if fl(n / B) < pi <= fl((n + 1) / B), draw n + 1 is impossible and
// draw n - 1 certain), so every lane computes at most one Philox block, all
// lanes at once.  Dividing by a power-of-two B is a multiplication by its
// exact reciprocal.
__device__ __forceinline__ int bern_count(double pi, int B, uint64_t seed, int b, int g, int i) {
    if (!(pi > 0.0)) return 0;
    const double Bd = (double)B;
    const bool pow2 = (B & (B - 1)) == 0;
    const double invB = 1.0 / Bd;
    auto over_b = [&](double x) { return pow2 ? x * invB : x / Bd; };
    const int n0 = min((int)floor(Bd * pi), B);
    int c = max(n0 - 1, 0);
    int un = -1;                                    // the draw that needs its uniform, if any
#pragma unroll
    for (int k = -1; k <= 1; ++k) {
        const int n = n0 + k;
        if (n < 0 || n >= B) continue;
        if (over_b((double)(n + 1)) < pi) ++c;
        else if (!(over_b((double)n) >= pi)) un = n;
    }
    if (un >= 0 && over_b((double)un + bern_uniform(seed, b, g, i, un)) < pi) ++c;
    return c;
}

// The group's kept features and, per head, their weights m_hat_i / m_i * q_{h,i}.
template <int G>
struct BernFeatures {
    int n;
    int feat[128];
    float w[G][128];
};

// Builds the kept-feature list of the item's group in `bf` (all threads call
// it); the group's first split also writes the feature counts.
template <int G, typename E, int NT>
__device__ __forceinline__ void bern_prologue(const Params& p, const Item& it, BernFeatures<G>& bf) {
    __shared__ double s_max[NT / 64];
    __shared__ int s_cnt[2];
    const int i = threadIdx.x;
    const int lane = i & 63, wave = i >> 6;
    float qv[G];
    double m = 0.0;
    if (i < p.D) m = mean_abs_query<G, E>(p, it.b, it.g, i, qv);
    const double top = block_max_f64(m, (p.D + 63) / 64, s_max);
    int c = 0;
    if (i < p.D && top > 0.0) c = bern_count(m / top, p.bern_B, p.seed, it.b, it.g, i);
    if (i < p.D && it.t == 0) p.bern_counts[((int64_t)it.b * p.Hkv + it.g) * p.D + i] = (uint8_t)c;
    const bool keep = i < p.D && c > 0;
    const unsigned long long bal = __ballot(keep);
    if (lane == 0 && wave < 2) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    if (keep) {
        const int pos = (wave == 1 ? s_cnt[0] : 0) + __popcll(bal & ((1ull << lane) - 1ull));
        const double r = (top / (double)p.bern_B) * (double)c / m;     // m_hat_i / m_i
        bf.feat[pos] = i;
#pragma unroll
        for (int h = 0; h < G; ++h) bf.w[h][pos] = (float)(r * (double)qv[h]);
    }
    if (i == 0) bf.n = s_cnt[0] + (p.D > 64 ? s_cnt[1] : 0);
    __syncthreads();
}

// A piece of KPL consecutive elements of a feature row, as one load.
template <int BYTES> struct PieceOf;
template <> struct PieceOf<2> { using T = uint16_t; };
template <> struct PieceOf<4> { using T = uint32_t; };
template <> struct PieceOf<8> { using T = uint2; };
template <> struct PieceOf<16> { using T = uint4; };

template <typename E, int KPL, typename P>
__device__ __forceinline__ void unpack_piece(const P& v, float (&x)[KPL]) {
    if constexpr (E::bytes == 2) {
        if constexpr (KPL == 1) {
            x[0] = __uint_as_float((uint32_t)v << 16);
        } else if constexpr (KPL == 2) {
            x[0] = __uint_as_float(v << 16);
            x[1] = __uint_as_float(v & 0xFFFF0000u);
        } else if constexpr (KPL == 4) {
            x[0] = __uint_as_float(v.x << 16);
            x[1] = __uint_as_float(v.x & 0xFFFF0000u);
            x[2] = __uint_as_float(v.y << 16);
            x[3] = __uint_as_float(v.y & 0xFFFF0000u);
        } else {
            x[0] = __uint_as_float(v.x << 16);
            x[1] = __uint_as_float(v.x & 0xFFFF0000u);
            x[2] = __uint_as_float(v.y << 16);
            x[3] = __uint_as_float(v.y & 0xFFFF0000u);
            x[4] = __uint_as_float(v.z << 16);
            x[5] = __uint_as_float(v.z & 0xFFFF0000u);
            x[6] = __uint_as_float(v.w << 16);
            x[7] = __uint_as_float(v.w & 0xFFFF0000u);
        }
    } else {
        if constexpr (KPL == 1) {
            x[0] = __uint_as_float(v);
        } else if constexpr (KPL == 2) {
            x[0] = __uint_as_float(v.x);
            x[1] = __uint_as_float(v.y);
        } else {
            x[0] = __uint_as_float(v.x);
            x[1] = __uint_as_float(v.y);
            x[2] = __uint_as_float(v.z);
            x[3] = __uint_as_float(v.w);
        }
    }
}

// Estimated scores of the split's keys.  Wave w covers the keys
// [w * split / NW, (w + 1) * split / NW), lane l the KPL keys from l * KPL on,
// and every wave reads the kept feature rows one after the other: one load
// per lane and feature, the whole wave on the same row, so that the feature
// index and the G weights are the same in every lane (they are taken from
// one lane into scalar registers) and the vector registers hold the loads in
// flight, UF features' worth (about 128 bytes per lane).  The loads carry no
// branches, so that they all stay in flight: a batch past the last kept
// feature repeats that feature with weight 0, a lane past the split's keys
// re-reads the split's first piece, and a piece that the sequence ends inside
// is read whole (it ends within the row: pieces are KPL-aligned and the row
// stride is a multiple of KPL elements); the scores of keys past the end are
// never written.  Each key's score is the fp32 fused multiply-add sum of its
// kept features in ascending order.
template <int G, typename E, int NT, int KPL>
__device__ __forceinline__ void bern_stream(const Params& p, const Item& it, float* sc, const BernFeatures<G>& bf) {
    constexpr int NW = NT / 64;
    constexpr int PB = KPL * E::bytes;                         // bytes per load
    constexpr int UF = PB >= 16 ? 8 : PB >= 8 ? 16 : 32;        // features in flight
    static_assert(UF <= 64, "one lane per feature of a batch");
    using Piece = typename PieceOf<PB>::T;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per_wave = p.split / NW;                         // 16 .. 256 keys
    const int lk = wave * per_wave + lane * KPL;               // first local key of this lane
    const bool active = lane * KPL < per_wave && lk < it.ns;
    const char* gbase = reinterpret_cast<const char*>(p.kt) +
                        ((int64_t)it.b * p.kt_stride_seq + (int64_t)it.g * p.kt_stride_head + it.key0) * E::bytes;
    const int lane_off = (active ? lk : 0) * E::bytes;
    const int64_t row_bytes = p.kt_stride_feat * E::bytes;
    float acc[G][KPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < KPL; ++j) acc[h][j] = 0.0f;
    const int nf = bf.n;
    for (int f0 = 0; f0 < nf; f0 += UF) {
        // lane u < UF holds the index and weights of feature f0 + u (the last
        // kept feature with weight 0 past the end)
        const int fl = min(f0 + lane, nf - 1);
        const bool real = lane < UF && f0 + lane < nf;
        const int my_feat = bf.feat[fl];
        float my_w[G];
#pragma unroll
        for (int h = 0; h < G; ++h) my_w[h] = real ? bf.w[h][fl] : 0.0f;
        Piece raw[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int feat = __builtin_amdgcn_readlane(my_feat, u);
            raw[u] = load_stream(reinterpret_cast<const Piece*>(gbase + (int64_t)feat * row_bytes + lane_off));
        }
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            float x[KPL];
            unpack_piece<E, KPL>(raw[u], x);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w[h]), u));
#pragma unroll
                for (int j = 0; j < KPL; ++j) acc[h][j] = fmaf(wt, x[j], acc[h][j]);
            }
        }
    }
    if (active) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < KPL; ++j)
                if (lk + j < it.ns) sc[h * p.split + lk + j] = acc[h][j] * p.scale;
    }
    priority_tail();
}

// Estimated scores of the split's keys, whole feature rows at a time, for
// splits of KB * 64 * PK keys (PK = 16 / element bytes keys per lane, KB in
// {1, 2, 4}).  One 16-byte load per lane reads PK keys of a feature row, one
// wave-wide load 64 * PK keys; wave w reads key block w mod KB of the kept
// features f = w / KB + j * F (F = NW / KB feature groups), so every wave
// streams its own features over its own keys with full 16-byte loads.  Feature
// index and weights come from one lane into scalar registers, as above, and
// the loads carry no branches (padding repeats the last kept feature with
// weight 0; a lane past the split's keys re-reads the split's first piece; a
// piece that the sequence ends inside is read whole, within the row).  Each
// group's sum is the fp32 fused multiply-add sum of its features in ascending
// order; the F group sums of a key are then added pairwise ((g0 + g1) + (g2 +
// g3)) through LDS, before the scale.
template <int G, typename E, int NT>
__device__ __forceinline__ void bern_stream_rows(const Params& p, const Item& it, float* sc, float* part,
                                                 const BernFeatures<G>& bf) {
    constexpr int NW = NT / 64;
    constexpr int PK = 16 / E::bytes;                          // keys per lane
    constexpr int WK = 64 * PK;                                // keys per wave-wide load
    constexpr int UF = G <= 4 ? 16 : 8;                        // features in flight
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int KB = p.split / WK;                               // 1, 2 or 4
    const int F = NW / KB;
    const int kb = wave % KB, fg = wave / KB;
    const int lk = kb * WK + lane * PK;                        // first local key of this lane
    const bool active = lk < it.ns;
    const char* gbase = reinterpret_cast<const char*>(p.kt) +
                        ((int64_t)it.b * p.kt_stride_seq + (int64_t)it.g * p.kt_stride_head + it.key0) * E::bytes;
    const int lane_off = (active ? lk : 0) * E::bytes;        // the split's first piece is in the row
    const int64_t row_bytes = p.kt_stride_feat * E::bytes;
    float acc[G][PK];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < PK; ++j) acc[h][j] = 0.0f;
    const int nf = bf.n;
    for (int f0 = fg; f0 < nf; f0 += UF * F) {
        // lane u < UF holds the index and weights of feature f0 + u * F
        const int fi = f0 + lane * F;
        const bool real = lane < UF && fi < nf;
        const int fl = real ? fi : nf - 1;
        const int my_feat = bf.feat[fl];
        float my_w[G];
#pragma unroll
        for (int h = 0; h < G; ++h) my_w[h] = real ? bf.w[h][fl] : 0.0f;
        uint4 raw[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int feat = __builtin_amdgcn_readlane(my_feat, u);
            raw[u] = load16_stream(gbase + (int64_t)feat * row_bytes + lane_off);
        }
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            float x[PK];
            unpack_piece<E, PK>(raw[u], x);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w[h]), u));
#pragma unroll
                for (int j = 0; j < PK; ++j) acc[h][j] = fmaf(wt, x[j], acc[h][j]);
            }
        }
    }
    priority_tail();
    // group sums to LDS: part[(fg * G + h) * split + key]
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float4* dst = reinterpret_cast<float4*>(part + (fg * G + h) * p.split + lk);
#pragma unroll
        for (int j = 0; j < PK; j += 4) dst[j / 4] = make_float4(acc[h][j], acc[h][j + 1], acc[h][j + 2], acc[h][j + 3]);
    }
    __syncthreads();
    // pairwise sums of the F groups, (h, key) values spread over the workgroup
    constexpr int MAXV = G * 1024 / NT;
    const int nv = G * p.split;
    float v[MAXV];
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int i = threadIdx.x + k * NT;
        float s = 0.0f;
        if (i < nv) {
            const int st = nv;                                 // stride between groups
            if (F == 4) s = (part[i] + part[i + st]) + (part[i + 2 * st] + part[i + 3 * st]);
            else if (F == 2) s = part[i] + part[i + st];
            else s = part[i];
        }
        v[k] = s * p.scale;
    }
    __syncthreads();        // sc may overlap the group sums
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int i = threadIdx.x + k * NT;
        if (i < nv) {
            const int h = i / p.split, key = i - h * p.split;
            if (key < it.ns) sc[i] = v[k];
        }
    }
}

// Keys per lane of a split: a wave covers split / 4 of them, 64 lanes; 0 for
// the whole-row stream (bern_stream_rows) where the split is 1, 2 or 4 times
// the keys of a wave-wide 16-byte load.
inline int bern_kpl(int split, int elem_bytes) {
    const int wk = 64 * 16 / elem_bytes;
    if (split >= wk && (split / wk == 1 || split / wk == 2 || split / wk == 4)) return 0;
    const int per_lane = split / (kThreads / 64) / 64;
    return per_lane >= 4 ? 4 : per_lane >= 2 ? 2 : 1;
}

// LDS of a Bernoulli workgroup: the split layout, or, if larger, the group
// sums of the whole-row stream (F * G * split = NW * 64 * PK * G floats),
// which overlap the layout during the stream.
inline size_t bern_lds_bytes(const Params& p, int elem_bytes) {
    const size_t base = split_lds_bytes(p.G, p.D, p.split, kThreads);
    if (bern_kpl(p.split, elem_bytes) != 0) return base;
    const size_t rows = (size_t)(kThreads / 64) * 64 * (16 / elem_bytes) * p.G * sizeof(float);
    return rows > base ? rows : base;
}

template <int G, int D, typename E, int NT, int KPL>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 3)))
void bern_fused_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ BernFeatures<G> bf;
    const int item = take_item(p);
    if (item < 0) return;
    priority_streaming();
    const unsigned int err0 = p.sync->error;
    const Item it = make_item(p, item);
    // splits with keys need the feature list; the first split of every group,
    // keys or not, writes the counts
    if (it.ns > 0 || it.t == 0) bern_prologue<G, E, NT>(p, it, bf);
    fused_item<G, D, E, NT>(p, it, err0, smem, [&](const Item& at, float* sc, const int*) {
        if constexpr (KPL == 0) bern_stream_rows<G, E, NT>(p, at, sc, reinterpret_cast<float*>(smem), bf);
        else bern_stream<G, E, NT, KPL>(p, at, sc, bf);
    });
}

template <int G, int D, typename E, int NT, int KPL>
__global__ __launch_bounds__(NT) void bern_score_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ BernFeatures<G> bf;
    const Item it = make_item(p, blockIdx.x);
    if (it.ns == 0 && it.t != 0) return;
    bern_prologue<G, E, NT>(p, it, bf);
    if (it.ns == 0) return;
    const LdsLayout L = lds_layout(G, D, p.split, NT);
    float* sc = reinterpret_cast<float*>(smem + L.scratch);
    HeadState* hs = reinterpret_cast<HeadState*>(smem + L.heads);
    if constexpr (KPL == 0) bern_stream_rows<G, E, NT>(p, it, sc, reinterpret_cast<float*>(smem), bf);
    else bern_stream<G, E, NT, KPL>(p, it, sc, bf);
    __syncthreads();
    split_stats<G, NT, true>(p, it, sc, reinterpret_cast<uint64_t*>(smem + L.prefix), hs);
    __syncthreads();
    write_stash<G, NT>(p, it, sc);
    publish_group_prefix<G, NT>(p, it);
}

template <int G, int D, typename E, int KPL>
static const void* bern_fn(bool fused) {
    return fused ? reinterpret_cast<const void*>(&bern_fused_kernel<G, D, E, kThreads, KPL>)
                 : reinterpret_cast<const void*>(&bern_score_kernel<G, D, E, kThreads, KPL>);
}

template <int G, int D, typename E>
static const void* bern_fn_k(int kpl, bool fused) {
    return kpl == 0 ? bern_fn<G, D, E, 0>(fused)
         : kpl == 4 ? bern_fn<G, D, E, 4>(fused) : kpl == 2 ? bern_fn<G, D, E, 2>(fused) : bern_fn<G, D, E, 1>(fused);
}

template <int D, typename E>
static const void* bern_fn_g(int G, int kpl, bool fused) {
    switch (G) {
        case 1: return bern_fn_k<1, D, E>(kpl, fused);
        case 2: return bern_fn_k<2, D, E>(kpl, fused);
        case 4: return bern_fn_k<4, D, E>(kpl, fused);
        case 7: return bern_fn_k<7, D, E>(kpl, fused);
        case 8: return bern_fn_k<8, D, E>(kpl, fused);
        default: return nullptr;
    }
}

static const void* bern_function(const Params& p, int dtype, bool fused) {
    const int kpl = bern_kpl(p.split, dtype == 0 ? 2 : 4);
    if (dtype == 0) return p.D == 64 ? bern_fn_g<64, Bf16>(p.G, kpl, fused) : bern_fn_g<128, Bf16>(p.G, kpl, fused);
    return p.D == 64 ? bern_fn_g<64, F32>(p.G, kpl, fused) : bern_fn_g<128, F32>(p.G, kpl, fused);
}

static hipError_t launch_bern(const Params& p, int dtype, hipStream_t stream, bool fused) {
    const void* fn = bern_function(p, dtype, fused);
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = bern_lds_bytes(p, dtype == 0 ? 2 : 4);
    const hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    void* args[] = {const_cast<Params*>(&p)};
    return hipLaunchKernel(fn, dim3((unsigned)p.items), dim3(kThreads), args, lds, stream);
}

hipError_t launch_bern_fused(const Params& p, int dtype, hipStream_t stream) { return launch_bern(p, dtype, stream, true); }
hipError_t launch_bern_score(const Params& p, int dtype, hipStream_t stream) { return launch_bern(p, dtype, stream, false); }

int bern_fused_blocks_per_cu(const Params& p, int dtype) {
    const void* fn = bern_function(p, dtype, true);
    if (!fn) return 0;
    const size_t lds = bern_lds_bytes(p, dtype == 0 ? 2 : 4);
    if (allow_lds(fn, lds) != hipSuccess) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, lds) != hipSuccess) return 0;
    return n;
}

}  // namespace santa
