// Internal launch interface of libsanta: the host-validated parameter block
// handed by value to every kernel, the workspace layout and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace santa {

constexpr int kMaxSplit = 1024;
constexpr int kRecPerLane = 8;           // split records per lane when a wave merges a sequence's splits
constexpr int kMaxSplitsPerSeq = 64 * kRecPerLane;   // T: splits of one sequence
constexpr int kMaxSamples = 65535;
constexpr int kMaxSortSamples = 8192;
constexpr int kTargetChunk = 256;        // targets one wave places per pass
constexpr int kFewTargets = 32;          // up to this many targets of a chunk: one target per lane
constexpr int kSpinLimit = 1 << 21;      // polls of a bounded wait (about 1 us each)

// Workspace state word (first kSyncBytes bytes of the workspace): the error
// word, nonzero once a bounded wait gave up (the outputs of that call are
// invalid and the workspace needs santa_workspace_init).  Every other byte of
// the workspace is zero between calls: a record or flag that is nonzero was
// written by the current call.
struct SyncWords {
    unsigned int error;
    unsigned int pad0[31];
    unsigned int ticket;          // fused kernel with tickets: items handed out so far this call
    unsigned int pad1[31];
};
constexpr size_t kSyncBytes = sizeof(SyncWords);

// Per (sequence, KV head) synchronisation lines (128 bytes each), all zero
// between calls:
//   line 0 word 0: splits that have published their records this call (the
//                  last one resets it);
//   line 1 word 0: splits that have added their output this call (the last one
//                  finishes the output and resets it);
//   lines 2 .. 1+kFlagCopies: copies of a flag raised to 1 once all splits
//                  published (a waiting workgroup polls copy
//                  blockIdx % kFlagCopies, so no line is polled by many).
constexpr int kFlagCopies = 16;
constexpr int kBarrierLines = 2 + kFlagCopies;
constexpr int kBarrierStride = 32 * kBarrierLines;   // 32-bit words per (sequence, KV head)

// Partial outputs: each split adds its per-head sums into accumulation slot
// (split % kOutSlots) of its (sequence, KV head), so few additions meet on one
// word; the last split to finish sums the slots into o and clears them.
constexpr int kOutSlots = 8;
// S^2ANTA-flash's fp64 slots: fewer than the fused kernel's, since its last
// split reads and clears twice the bytes per slot (Llama-shaped step: 29.6 us
// with 8, 28.2 us with 4, 32.7 us with 2)
constexpr int kFlashSlots = 4;

// Orders of the work items (sequence, KV head, split) over the workgroup indices.
constexpr int kOrderSplitFastest = 0;
constexpr int kOrderHeadFastest = 1;
constexpr int kOrderTokenBlocks = 2;      // needs T % 8 == 0

struct Params {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* seq_lens;
    const int32_t* block_table;   // null when contiguous
    float* o;
    int32_t* idx;
    SyncWords* sync;
    unsigned long long* records;  // [B, Hq, T] words: l bits << 32 | m bits (0: not written yet)
    unsigned long long* gprefix;  // two-kernel path: [B * Hq][T + 2] split-mass prefixes W_t, Z, then M | last << 32
    unsigned int* barrier;        // [B * Hkv] x kBarrierStride words: counts, flags
    float* accum;                 // [B * Hkv][kOutSlots][G * D] partial outputs (zero between calls)
    double* flash_acc;            // S^2ANTA-flash: [B * Hkv][kFlashSlots][G][D + 2] weighted sums, weight
    unsigned long long* flash_ref;   // S^2ANTA-flash: [B, Hq] reference maximum (1 << 32 | bits), 0 unset
    float* stash;                 // [B, Hq, T * split] scaled scores (two-kernel path)
    double* targets;              // [B, Hq, S] sorted uniforms (multinomial only)
    int64_t stride_seq;           // elements
    int64_t stride_tok;
    int64_t stride_head;
    int64_t stash_row;            // floats per (b, h) row of the stash (T * split)
    uint64_t seed;
    double inv_S;                 // 1 / S
    float scale;                  // 1 / sqrt(d)
    int32_t B, Hq, Hkv, G, D;
    int32_t n_max;
    int32_t page_shift;           // log2(page_size); -1 when contiguous
    int32_t pages_per_seq;
    int32_t num_pages;
    int32_t split;                // keys per split, multiple of 64
    int32_t T;                    // splits per sequence: ceil(n_max / split)
    int32_t items;                // B * Hkv * T work items (one workgroup each)
    int32_t item_order;           // kOrder*: how a workgroup index maps to (b, g, t)
    int32_t use_ticket;           // fused kernel: items taken in start order from sync->ticket
    int32_t sort_in_score;        // multinomial, two-kernel path: the score pass's first B * Hq
                                  // workgroups sort the targets (no separate launch)
    int32_t S;
    int32_t mode;
    // Bernoulli qK^T: K transposed ([B, Hkv, d, tokens], tokens contiguous), the
    // number of Bernoulli draws, and the feature counts [B, Hkv, d]
    const void* kt;
    int64_t kt_stride_seq;
    int64_t kt_stride_head;
    int64_t kt_stride_feat;
    int32_t bern_B;
    uint8_t* bern_counts;
};

// Dynamic LDS bytes of the split kernels for a group size, head dim, split and
// block size.
size_t split_lds_bytes(int G, int D, int split, int nt);
size_t sort_lds_bytes(int S);

// Number of threads per workgroup of the split kernels.
constexpr int kThreads = 256;

hipError_t launch_targets(const Params& p, hipStream_t stream);
// stats = false: scores to the stash only (no split statistics or records)
hipError_t launch_score(const Params& p, int dtype, hipStream_t stream, bool stats = true);
hipError_t launch_topk(const Params& p, int dtype, hipStream_t stream);
// Bernoulli qK^T: the feature counts, then the fused kernel (grid p.items, items
// by ticket when p.use_ticket) or the score pass of the two-kernel path
hipError_t launch_bern_fused(const Params& p, int dtype, hipStream_t stream);
hipError_t launch_bern_score(const Params& p, int dtype, hipStream_t stream);
int bern_fused_blocks_per_cu(const Params& p, int dtype);
constexpr int kMaxBernoulli = 64;        // Bernoulli draws per feature
constexpr int kMaxTopk = 8192;           // largest k of the top-k comparator
hipError_t launch_sample(const Params& p, int dtype, hipStream_t stream);
hipError_t launch_fused(const Params& p, int dtype, hipStream_t stream);
hipError_t launch_clear(void* ws, size_t bytes, hipStream_t stream);
hipError_t launch_flash(const Params& p, int dtype, hipStream_t stream);
// Workgroups of the fused kernel one compute unit can hold at once (0 on error).
int fused_blocks_per_cu(const Params& p, int dtype);
int flash_blocks_per_cu(const Params& p, int dtype);
// Bytes of LDS one workgroup may use on gfx950.
constexpr size_t kLdsPerWorkgroup = 163840;

// Lets kernel `fn` be launched with `bytes` of dynamic LDS (needed above 64 KiB).
inline hipError_t allow_lds(const void* fn, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Number of valid tokens of sequence b.
__device__ __forceinline__ int seq_len_of(const Params& p, int b) {
    return min(max(p.seq_lens[b], 0), p.n_max);
}

}  // namespace santa
