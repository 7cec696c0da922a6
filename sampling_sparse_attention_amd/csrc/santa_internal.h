// Internal launch interface of libsanta: the host-validated parameter block
// handed by value to every kernel, and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace santa {

// Per split of a query head: maximum scaled score and sum of exp(s - m).
struct __align__(16) SplitStat {
    float m;
    float pad;
    double l;
};

constexpr int kBlock = 256;          // threads per workgroup (4 waves of 64)
constexpr int kWaves = kBlock / 64;
constexpr int kTargetChunk = 256;    // targets per merge-path pass of one wave
constexpr int kMaxSplit = 1024;
constexpr int kMaxSamples = 65535;
constexpr int kMaxSortSamples = 8192;

struct Params {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* seq_lens;
    const int32_t* block_table;   // null when contiguous
    float* o;
    int32_t* idx;
    float* scores;                // [B, Hq, score_row]
    SplitStat* stats;             // [B, Hq, T]
    double* targets;              // [B, Hq, S] (multinomial only)
    int64_t stride_seq;           // elements
    int64_t stride_tok;
    int64_t stride_head;
    int64_t score_row;            // floats per (b, h) row of the score stash (T * split)
    uint64_t seed;
    float scale;                  // 1 / sqrt(d)
    int32_t B, Hq, Hkv, G, D;
    int32_t n_max;
    int32_t page_shift;           // log2(page_size); -1 when contiguous
    int32_t pages_per_seq;
    int32_t num_pages;
    int32_t split;                // keys per split, multiple of 64
    int32_t T;                    // splits per sequence: ceil(n_max / split)
    int32_t S;
    int32_t mode;
};

// Bytes of dynamic LDS each kernel needs.
size_t score_lds_bytes(int G, int split);
size_t sample_lds_bytes(int G, int D, int split);
size_t sort_lds_bytes(int S);

hipError_t launch_targets(const Params& p, hipStream_t stream);
hipError_t launch_score(const Params& p, int dtype, hipStream_t stream);
hipError_t launch_sample(const Params& p, int dtype, hipStream_t stream);

// Element offset of row (token i, KV head g) of sequence b; page entries are
// clamped into the cache so that a bad table cannot address outside it.
__device__ __forceinline__ int64_t row_offset(const Params& p, int b, int g, int i) {
    int64_t off;
    if (p.page_shift < 0) {
        off = (int64_t)b * p.stride_seq + (int64_t)i * p.stride_tok;
    } else {
        int pg = p.block_table[(int64_t)b * p.pages_per_seq + (i >> p.page_shift)];
        pg = min(max(pg, 0), p.num_pages - 1);
        off = (int64_t)pg * p.stride_seq + (int64_t)(i & ((1 << p.page_shift) - 1)) * p.stride_tok;
    }
    return off + (int64_t)g * p.stride_head;
}

// Number of valid tokens of sequence b.
__device__ __forceinline__ int seq_len_of(const Params& p, int b) {
    return min(max(p.seq_lens[b], 0), p.n_max);
}

}  // namespace santa
