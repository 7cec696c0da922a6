// C ABI of libsanta: host-side validation, workspace layout, path choice and
// kernel dispatch.  Every check runs on the host before anything is enqueued;
// the library keeps no state between calls apart from a per-thread error
// message.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "santa.h"
#include "santa_internal.h"
#include "santa_pp.h"

namespace {

thread_local char g_error[512] = "";

santa_status fail(santa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return st;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

bool split_fits(int G, int D, int split) {
    return santa::split_lds_bytes(G, D, split, santa::kThreads) <= santa::kLdsPerWorkgroup;
}

// Default keys per split: 512, halved while the step would have fewer than
// kTargetItems work items (about two per compute unit, so that the K stream
// keeps HBM busy), doubled while a sequence would need more than
// kMaxSplitsPerSeq splits, and halved until the split's LDS fits.  Larger
// splits mean fewer workgroups repeating the same cross-split work after the
// K stream.  Measured: batch-1, 32/8-head, 32k-token step 26.3 us at 512 keys
// against 27.7 at 256 and 30.8 at 1024; 64 x 32/8 heads at 32k (fused kernel
// with tickets) 931 us at 512 against 1252 at 256 and 970 at 1024; 4 x 28/4
// heads at 128k (score and sample passes) 262 us at 512 against 340 at 256.
// The rule reads only the shape, so the workspace size does not depend on the
// device.
constexpr int64_t kTargetItems = 512;

int default_split(const santa_shape& s, int G) {
    const int64_t groups = (int64_t)s.batch * s.num_kv_heads;
    auto splits = [&](int split) { return ((int64_t)s.max_seq_len + split - 1) / split; };
    int split = 512;
    while (split > 64 && groups * splits(split) < kTargetItems) split >>= 1;
    while (split < santa::kMaxSplit && splits(split) > santa::kMaxSplitsPerSeq) split <<= 1;
    while (split > 64 && !split_fits(G, s.head_dim, split)) split >>= 1;
    return split;
}

struct Plan {
    int G, split, T, elem_bytes;
    santa_workspace_layout layout;
};

santa_status make_plan(const santa_shape* s, int32_t S, int32_t mode, Plan* plan) {
    if (!s) return fail(SANTA_STATUS_INVALID_ARGUMENT, "shape is NULL");
    if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "batch, num_q_heads and num_kv_heads must be >= 1");
    if (s->num_q_heads % s->num_kv_heads)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                    s->num_q_heads, s->num_kv_heads);
    const int G = s->num_q_heads / s->num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 7 && G != 8)
        return fail(SANTA_STATUS_UNSUPPORTED, "group size %d not built (1, 2, 4, 7, 8)", G);
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(SANTA_STATUS_UNSUPPORTED, "head_dim %d not built (64, 128)", s->head_dim);
    if (s->dtype != SANTA_DTYPE_BF16 && s->dtype != SANTA_DTYPE_F32)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "unknown dtype %d", s->dtype);
    if (s->max_seq_len < 1) return fail(SANTA_STATUS_INVALID_ARGUMENT, "max_seq_len must be >= 1");
    if ((int64_t)s->max_seq_len > (int64_t)santa::kMaxSplit * santa::kMaxSplitsPerSeq)
        return fail(SANTA_STATUS_UNSUPPORTED, "max_seq_len %d above %d", s->max_seq_len,
                    santa::kMaxSplit * santa::kMaxSplitsPerSeq);
    const int eb = s->dtype == SANTA_DTYPE_BF16 ? 2 : 4;
    if (s->page_size != 0) {
        if (s->page_size < 16 || !is_pow2(s->page_size) || s->page_size > (1 << 20))
            return fail(SANTA_STATUS_INVALID_ARGUMENT, "page_size %d is not a power of two in [16, 2^20]",
                        s->page_size);
        const int64_t need = ((int64_t)s->max_seq_len + s->page_size - 1) / s->page_size;
        if (s->pages_per_seq < need)
            return fail(SANTA_STATUS_INVALID_ARGUMENT, "pages_per_seq %d < ceil(max_seq_len / page_size) = %lld",
                        s->pages_per_seq, (long long)need);
        if (s->num_pages < 1) return fail(SANTA_STATUS_INVALID_ARGUMENT, "num_pages must be >= 1");
    }
    if (s->kv_stride_tok < 1 || s->kv_stride_seq < 0 || s->kv_stride_head < 0)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "KV strides must be non-negative (token stride >= 1)");
    if ((s->kv_stride_tok * eb) % 16 || (s->kv_stride_seq * eb) % 16 || (s->kv_stride_head * eb) % 16)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "KV strides must keep every row 16-byte aligned");
    if (mode < SANTA_MODE_MULTINOMIAL || mode > SANTA_MODE_SYSTEMATIC)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "unknown sampling mode %d", mode);
    if (S < 1) return fail(SANTA_STATUS_INVALID_ARGUMENT, "num_samples must be >= 1 (got %d)", S);
    if (S > santa::kMaxSamples)
        return fail(SANTA_STATUS_UNSUPPORTED, "num_samples %d above %d", S, santa::kMaxSamples);
    if (mode == SANTA_MODE_MULTINOMIAL && S > santa::kMaxSortSamples)
        return fail(SANTA_STATUS_UNSUPPORTED, "multinomial sampling supports num_samples <= %d",
                    santa::kMaxSortSamples);
    int split = s->split_size;
    if (split == 0) {
        split = default_split(*s, G);
    } else if (split < 64 || split > santa::kMaxSplit || (split & (split - 1))) {
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "split_size %d is not a power of two in [64, %d]",
                    split, santa::kMaxSplit);
    }
    if (!split_fits(G, s->head_dim, split))
        return fail(SANTA_STATUS_UNSUPPORTED, "split_size %d needs more than %zu bytes of LDS for group %d",
                    split, santa::kLdsPerWorkgroup, G);
    const int64_t T = ((int64_t)s->max_seq_len + split - 1) / split;
    if (T > santa::kMaxSplitsPerSeq)
        return fail(SANTA_STATUS_UNSUPPORTED, "split_size %d gives %lld splits per sequence (at most %d)",
                    split, (long long)T, santa::kMaxSplitsPerSeq);
    if ((int64_t)s->batch * s->num_kv_heads * T >= (1ll << 31) || (int64_t)s->batch * s->num_q_heads >= (1ll << 31))
        return fail(SANTA_STATUS_UNSUPPORTED, "problem too large for one launch");

    plan->G = G;
    plan->split = split;
    plan->T = (int)T;
    plan->elem_bytes = eb;
    santa_workspace_layout& L = plan->layout;
    const size_t rows = (size_t)s->batch * s->num_q_heads;
    L.split_size = split;
    L.num_splits = (int32_t)T;
    L.sync_offset = 0;
    L.barrier_offset = align256(santa::kSyncBytes);
    L.accum_offset = align256(L.barrier_offset + (size_t)s->batch * s->num_kv_heads * santa::kBarrierStride * 4);
    L.flash_offset = align256(L.accum_offset + (size_t)s->batch * s->num_q_heads * santa::kOutSlots *
                                                   s->head_dim * sizeof(float));
    // flash region: reference maxima [B, Hq] u64, then (256-aligned) the fp64
    // accumulators [B, Hkv, kFlashSlots, G, d + 2]
    L.records_offset = align256(L.flash_offset + align256(rows * sizeof(unsigned long long)) +
                                (size_t)s->batch * s->num_q_heads * santa::kFlashSlots * (s->head_dim + 2) *
                                    sizeof(double));
    // split records [B, Hq, T], then the group prefixes [B, Hq, T + 2]
    L.stash_offset = align256(L.records_offset + rows * (size_t)T * 8 + rows * (size_t)(T + 2) * 8);
    L.stash_row_bytes = (size_t)T * split * sizeof(float);
    L.targets_offset = align256(L.stash_offset + rows * L.stash_row_bytes);
    const size_t targets = mode == SANTA_MODE_MULTINOMIAL ? rows * (size_t)S * sizeof(double) : 0;
    L.total_bytes = align256(L.targets_offset + targets);
    return SANTA_STATUS_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

santa_status make_params(const santa_shape* s, const void* q, const void* k, const void* v,
                         const int32_t* seq_lens, const int32_t* block_table, int32_t S, int32_t mode,
                         uint64_t seed, float* o, int32_t* idx, void* ws, size_t ws_bytes,
                         santa::Params* p, Plan* plan) {
    santa_status st = make_plan(s, S, mode, plan);
    if (st != SANTA_STATUS_OK) return st;
    if (!q || !k || !v || !seq_lens || !o || !idx || !ws)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "a required pointer is NULL");
    if ((s->page_size != 0) != (block_table != nullptr))
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "block_table must be given exactly when page_size > 0");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "q, k_cache and v_cache must be 16-byte aligned");
    if (!aligned(o, 16) || !aligned(idx, 4) || !aligned(seq_lens, 4) ||
        (block_table && !aligned(block_table, 4)))
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "o must be 16-byte and idx/seq_lens/block_table 4-byte aligned");
    if (!aligned(ws, 256)) return fail(SANTA_STATUS_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (ws_bytes < plan->layout.total_bytes)
        return fail(SANTA_STATUS_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes,
                    plan->layout.total_bytes);

    const santa_workspace_layout& L = plan->layout;
    char* w = static_cast<char*>(ws);
    p->q = q;
    p->k = k;
    p->v = v;
    p->seq_lens = seq_lens;
    p->block_table = block_table;
    p->o = o;
    p->idx = idx;
    p->sync = reinterpret_cast<santa::SyncWords*>(w + L.sync_offset);
    p->records = reinterpret_cast<unsigned long long*>(w + L.records_offset);
    p->gprefix = p->records + (size_t)s->batch * s->num_q_heads * plan->T;
    p->barrier = reinterpret_cast<unsigned int*>(w + L.barrier_offset);
    p->accum = reinterpret_cast<float*>(w + L.accum_offset);
    p->flash_ref = reinterpret_cast<unsigned long long*>(w + L.flash_offset);
    p->flash_acc = reinterpret_cast<double*>(w + L.flash_offset + align256((size_t)s->batch * s->num_q_heads * 8));
    p->stash = reinterpret_cast<float*>(w + L.stash_offset);
    p->targets = reinterpret_cast<double*>(w + L.targets_offset);
    p->stride_seq = s->kv_stride_seq;
    p->stride_tok = s->kv_stride_tok;
    p->stride_head = s->kv_stride_head;
    p->stash_row = (int64_t)plan->T * plan->split;
    p->seed = seed;
    p->scale = (float)(1.0 / __builtin_sqrt((double)s->head_dim));
    p->inv_S = 1.0 / (double)S;
    p->B = s->batch;
    p->Hq = s->num_q_heads;
    p->Hkv = s->num_kv_heads;
    p->G = plan->G;
    p->D = s->head_dim;
    p->n_max = s->max_seq_len;
    p->page_shift = -1;
    if (s->page_size) {
        int sh = 0;
        while ((1 << sh) < s->page_size) ++sh;
        p->page_shift = sh;
    }
    p->pages_per_seq = s->pages_per_seq;
    p->num_pages = s->num_pages;
    p->split = plan->split;
    p->T = plan->T;
    p->items = (int32_t)((int64_t)s->batch * s->num_kv_heads * plan->T);
    p->item_order = santa::kOrderSplitFastest;
    p->use_ticket = 0;
    p->sort_in_score = 0;
    p->kt = nullptr;
    p->kt_stride_seq = p->kt_stride_head = p->kt_stride_feat = 0;
    p->bern_B = 0;
    p->bern_counts = nullptr;
    p->S = S;
    p->mode = mode;
    return SANTA_STATUS_OK;
}

santa_status hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return SANTA_STATUS_OK;
    return fail(SANTA_STATUS_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

// How santa_decode runs a problem: 1 = the fused kernel, every workgroup
// resident at once; 3 = the fused kernel with tickets (items taken in start
// order), when one group's splits fit on a single compute die (XCD); 2 =
// score pass + sample pass; 0 = unknown (HIP error).  The fused kernel's
// workgroups wait for the other splits of their group.
int choose_path(const santa::Params& p, int dtype, bool bernoulli = false) {
    int dev = 0, cus = 0, xccs = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xccs < 1) xccs = 1;
    const int per_cu = bernoulli ? santa::bern_fused_blocks_per_cu(p, dtype) : santa::fused_blocks_per_cu(p, dtype);
    if (per_cu <= 0) return 0;
    if ((int64_t)per_cu * cus >= (int64_t)p.items) return 1;
    return (int64_t)per_cu * (cus / xccs) >= (int64_t)p.T ? 3 : 2;
}

enum Stage { kScore = 1, kSample = 2, kDecode = 3 };

santa_status run(int stages, const santa_shape* s, const void* q, const void* k, const void* v,
                 const int32_t* seq_lens, const int32_t* block_table, int32_t S, int32_t mode,
                 uint64_t seed, float* o, int32_t* idx, void* ws, size_t ws_bytes, void* stream,
                 uint32_t flags = 0) {
    santa::Params p;
    Plan plan;
    santa_status st = make_params(s, q, k, v, seq_lens, block_table, S, mode, seed, o, idx, ws,
                                  ws_bytes, &p, &plan);
    if (st != SANTA_STATUS_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int path = 2;
    if (stages == kDecode && !(flags & SANTA_FLAG_TWO_KERNEL)) {
        path = choose_path(p, s->dtype);
        if (path == 0) return fail(SANTA_STATUS_HIP_ERROR, "querying the device for the launch plan failed");
    }
    if ((stages & kScore) && mode == SANTA_MODE_MULTINOMIAL) {
        // the two-kernel path's score pass sorts the targets itself when its grid
        // has a workgroup per (sequence, query head) and their LDS holds the sort
        if (path == 2 && (int64_t)p.items >= (int64_t)p.B * p.Hq &&
            santa::sort_lds_bytes(S) <= santa::split_lds_bytes(p.G, p.D, p.split, santa::kThreads)) {
            p.sort_in_score = 1;
        } else {
            st = hip_check(santa::launch_targets(p, hs), "launching the target sort");
            if (st != SANTA_STATUS_OK) return st;
        }
    }
    if (path == 1 || path == 3) {
        if (path == 1) {
            p.item_order = p.T % 8 == 0 ? santa::kOrderTokenBlocks : santa::kOrderHeadFastest;
        } else {
            p.item_order = santa::kOrderSplitFastest;     // group by group, in ticket order
            p.use_ticket = 1;
        }
        st = hip_check(santa::launch_fused(p, s->dtype, hs), "launching the fused decode kernel");
        if (st != SANTA_STATUS_OK) return st;
    } else {
        if (stages & kScore) {
            st = hip_check(santa::launch_score(p, s->dtype, hs), "launching the score pass");
            if (st != SANTA_STATUS_OK) return st;
        }
        if (stages & kSample) {
            st = hip_check(santa::launch_sample(p, s->dtype, hs), "launching the sample pass");
            if (st != SANTA_STATUS_OK) return st;
        }
    }
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

// ---------------------------------------------------------------------------
// The workspace of santa_decode_noalloc: one array per device, a part of the
// library's code object (no allocation call).  In host code `scratch` only
// names the symbol; its device address comes from hipGetSymbolAddress, once
// per device, and is what every kernel and the clear receive.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocBytes = SANTA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};     // device address of `scratch` per device
bool g_scratch_clear[kMaxDevices] = {};    // its zero fill has been enqueued

// The current device's scratch address, looked up once per device; with
// `clear`, the first call on a device also enqueues its zero fill on `stream`
// (the workspace protocol needs all zero before a first call).
santa_status noalloc_scratch(bool clear, hipStream_t stream, void** out) {
    int dev = 0;
    santa_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st != SANTA_STATUS_OK) return st;
    if (dev < 0 || dev >= kMaxDevices) return fail(SANTA_STATUS_UNSUPPORTED, "device %d above %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        st = hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (st != SANTA_STATUS_OK) return st;
        if (!ptr || !aligned(ptr, 256))
            return fail(SANTA_STATUS_HIP_ERROR, "the scratch array has no usable device address");
        g_scratch_ptr[dev] = ptr;
    }
    if (clear && !g_scratch_clear[dev]) {
        st = hip_check(santa::launch_clear(g_scratch_ptr[dev], kNoAllocBytes, stream), "clearing the scratch array");
        if (st != SANTA_STATUS_OK) return st;
        g_scratch_clear[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    return SANTA_STATUS_OK;
}


// ---------------------------------------------------------------------------
// SANTA++
// ---------------------------------------------------------------------------
int64_t pp_teams(int64_t N, int64_t P, int64_t R) {
    if (N < 1 || P < 1 || R < 1 || R > P || P % R) return -1;
    return (N / P) * R + (N % P ? std::min<int64_t>(R, N % P) : 0);
}

struct PPLayout {
    size_t y, phi, logc, mask, part, total;
};

PPLayout pp_layout(const santa_shape& s, int64_t M) {
    const int64_t Mpad = (M + 3) & ~int64_t(3);
    const int64_t groups = (int64_t)s.batch * s.num_kv_heads;
    const int64_t rows = (int64_t)s.batch * s.num_q_heads;
    PPLayout L;
    size_t at = 0;
    auto take = [&](size_t bytes) { const size_t r = at; at = align256(at + bytes); return r; };
    L.y = take(rows * Mpad * 4);
    L.phi = take(rows * Mpad * 4);
    L.logc = take(rows * Mpad * 4);
    L.mask = take(groups * Mpad);
    L.part = take(rows * santa::kPPChunks * (int64_t)(s.head_dim + 2) * 4);
    L.total = at;
    return L;
}

// Shape, prompt and team checks shared by the SANTA++ entry points.
santa_status pp_check(const santa_shape* s, int32_t N, int32_t P, int32_t R, int* G, int64_t* M) {
    Plan plan;
    santa_status st = make_plan(s, 1, SANTA_MODE_SYSTEMATIC, &plan);
    if (st != SANTA_STATUS_OK) return st;
    if (s->page_size != 0) return fail(SANTA_STATUS_UNSUPPORTED, "SANTA++ reads a contiguous cache (page_size must be 0)");
    if (P < 1 || P > santa::kPPMaxParent || R < 1 || R > P || P % R)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "need 1 <= R <= P <= %d with P divisible by R (P %d, R %d)",
                    santa::kPPMaxParent, P, R);
    if (N < 1 || N > s->max_seq_len)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "prompt length %d not in [1, max_seq_len %d]", N, s->max_seq_len);
    const int64_t m = pp_teams(N, P, R);
    if (m > santa::kPPMaxTeams)
        return fail(SANTA_STATUS_UNSUPPORTED, "%lld teams, at most %d", (long long)m, santa::kPPMaxTeams);
    *G = plan.G;
    *M = m;
    return SANTA_STATUS_OK;
}

santa_status pp_table_check(const santa_pp_table* t) {
    if (!t || !t->packed_k || !t->packed_v || !t->rep_k || !t->team_start || !t->perm)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "a team-table pointer is NULL");
    if (!aligned(t->packed_k, 16) || !aligned(t->packed_v, 16) || !aligned(t->rep_k, 16) ||
        !aligned(t->team_start, 4) || !aligned(t->perm, 4))
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "team-table arrays must be 16-byte (rows) or 4-byte (indices) aligned");
    return SANTA_STATUS_OK;
}

void pp_fill(santa::PPParams* p, const santa_shape* s, int G, int32_t N, int32_t P, int32_t R, int64_t M,
             const santa_pp_table* t) {
    *p = santa::PPParams{};
    p->B = s->batch;
    p->Hq = s->num_q_heads;
    p->Hkv = s->num_kv_heads;
    p->G = G;
    p->D = s->head_dim;
    p->N = N;
    p->P = P;
    p->R = R;
    p->M = (int)M;
    p->Mpad = (int)((M + 3) & ~int64_t(3));
    p->n_max = s->max_seq_len;
    p->stride_seq = s->kv_stride_seq;
    p->stride_tok = s->kv_stride_tok;
    p->stride_head = s->kv_stride_head;
    p->packed_k = t->packed_k;
    p->packed_v = t->packed_v;
    p->rep_k = t->rep_k;
    p->team_start = t->team_start;
    p->perm = t->perm;
    p->scale = (float)(1.0 / __builtin_sqrt((double)s->head_dim));
    p->NC = santa::kPPChunks;
}

}  // namespace

extern "C" {

size_t santa_noalloc_scratch_bytes(void) { return kNoAllocBytes; }

santa_status santa_noalloc_init(void* stream) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    void* ptr = nullptr;
    santa_status st = noalloc_scratch(false, hs, &ptr);
    if (st != SANTA_STATUS_OK) return st;
    st = hip_check(santa::launch_clear(ptr, kNoAllocBytes, hs), "clearing the scratch array");
    if (st != SANTA_STATUS_OK) return st;
    {
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
            std::lock_guard<std::mutex> lock(g_scratch_mu);
            g_scratch_clear[dev] = true;
        }
    }
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_decode_noalloc(const santa_shape* shape, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                                  int32_t num_samples, int32_t mode, uint64_t seed, float* o, int32_t* idx,
                                  void* stream) {
    // the size check first, so that a problem too large is refused before the
    // device is touched
    Plan plan;
    santa_status st = make_plan(shape, num_samples, mode, &plan);
    if (st != SANTA_STATUS_OK) return st;
    if (plan.layout.total_bytes > kNoAllocBytes)
        return fail(SANTA_STATUS_WORKSPACE_TOO_SMALL,
                    "santa_decode_noalloc: the problem needs %zu bytes of workspace, the scratch array holds %zu "
                    "(use santa_decode with a workspace)",
                    plan.layout.total_bytes, kNoAllocBytes);
    void* ws = nullptr;
    st = noalloc_scratch(true, static_cast<hipStream_t>(stream), &ws);
    if (st != SANTA_STATUS_OK) return st;
    return run(kDecode, shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o, idx, ws,
               kNoAllocBytes, stream);
}

santa_status santa_noalloc_status(void* stream, uint32_t* error_word) {
    void* ws = nullptr;
    santa_status st = noalloc_scratch(false, static_cast<hipStream_t>(stream), &ws);
    if (st != SANTA_STATUS_OK) return st;
    return santa_workspace_status(ws, kNoAllocBytes, stream, error_word);
}


int32_t santa_abi_version(void) { return SANTA_ABI_VERSION; }

const char* santa_status_string(santa_status status) {
    switch (status) {
        case SANTA_STATUS_OK: return "ok";
        case SANTA_STATUS_INVALID_ARGUMENT: return "invalid argument";
        case SANTA_STATUS_UNSUPPORTED: return "unsupported";
        case SANTA_STATUS_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SANTA_STATUS_HIP_ERROR: return "HIP error";
    }
    return "unknown status";
}

const char* santa_last_error(void) { return g_error; }

santa_status santa_workspace_layout_query(const santa_shape* shape, int32_t num_samples, int32_t mode,
                                          santa_workspace_layout* out) {
    if (!out) return fail(SANTA_STATUS_INVALID_ARGUMENT, "out is NULL");
    Plan plan;
    santa_status st = make_plan(shape, num_samples, mode, &plan);
    if (st != SANTA_STATUS_OK) return st;
    *out = plan.layout;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_workspace_size(const santa_shape* shape, int32_t num_samples, int32_t mode,
                                  size_t* bytes) {
    if (!bytes) return fail(SANTA_STATUS_INVALID_ARGUMENT, "bytes is NULL");
    Plan plan;
    santa_status st = make_plan(shape, num_samples, mode, &plan);
    if (st != SANTA_STATUS_OK) return st;
    *bytes = plan.layout.total_bytes;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace) return fail(SANTA_STATUS_INVALID_ARGUMENT, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(SANTA_STATUS_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (workspace_bytes < santa::kSyncBytes)
        return fail(SANTA_STATUS_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs at least %zu",
                    workspace_bytes, santa::kSyncBytes);
    santa_status st = hip_check(santa::launch_clear(workspace, workspace_bytes, static_cast<hipStream_t>(stream)),
                                "launching the workspace clear");
    if (st != SANTA_STATUS_OK) return st;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

int32_t santa_decode_path(const santa_shape* shape, int32_t num_samples, int32_t mode) {
    santa::Params p;
    Plan plan;
    santa_status st = make_plan(shape, num_samples, mode, &plan);
    if (st != SANTA_STATUS_OK) return -(int32_t)st;
    p.G = plan.G;
    p.D = shape->head_dim;
    p.split = plan.split;
    p.T = plan.T;
    p.items = (int32_t)((int64_t)shape->batch * shape->num_kv_heads * plan.T);
    const int path = choose_path(p, shape->dtype);
    if (path == 0) {
        fail(SANTA_STATUS_HIP_ERROR, "querying the device for the launch plan failed");
        return -(int32_t)SANTA_STATUS_HIP_ERROR;
    }
    g_error[0] = '\0';
    return path;
}

santa_status santa_decode(const santa_shape* shape, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                          int32_t num_samples, int32_t mode, uint64_t seed, float* o, int32_t* idx,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return run(kDecode, shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o,
               idx, workspace, workspace_bytes, stream);
}

santa_status santa_decode_flash(const santa_shape* shape, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                                int32_t num_samples, int32_t mode, uint64_t seed, float* o, int32_t* idx,
                                void* workspace, size_t workspace_bytes, void* stream) {
    santa::Params p;
    Plan plan;
    santa_status st = make_params(shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed, o,
                                  idx, workspace, workspace_bytes, &p, &plan);
    if (st != SANTA_STATUS_OK) return st;
    if (mode == SANTA_MODE_MULTINOMIAL)
        return fail(SANTA_STATUS_UNSUPPORTED, "santa_decode_flash samples stratified or systematic (mode 1 or 2)");
    if (num_samples < plan.T)
        return fail(SANTA_STATUS_UNSUPPORTED,
                    "santa_decode_flash needs a sample for every tile: num_samples %d < %d splits",
                    num_samples, plan.T);
    // The workgroups running together read the K rows of all KV heads of one
    // range of tokens, which lie together in the token-major cache
    // (split-fastest measured 10-40 % slower).  A grid larger than the device,
    // with T a multiple of 8, also keeps all KV heads of a split on one XCD
    // (ragged 16-sequence batch: 154 -> 144 us); a resident grid keeps the
    // head-fastest order, whose finishing times varied less from run to run
    // (Llama-shaped step: 29.7 us against 29.7 or 31 us).
    int dev = 0, cus = 0;
    const int per_cu = santa::flash_blocks_per_cu(p, shape->dtype);
    if (per_cu <= 0 || hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(SANTA_STATUS_HIP_ERROR, "querying the device for the launch plan failed");
    const bool resident = (int64_t)per_cu * cus >= (int64_t)p.items;
    p.item_order = !resident && p.T % 8 == 0 ? santa::kOrderTokenBlocks : santa::kOrderHeadFastest;
    st = hip_check(santa::launch_flash(p, shape->dtype, static_cast<hipStream_t>(stream)),
                   "launching the flash decode kernel");
    if (st != SANTA_STATUS_OK) return st;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_decode_topk(const santa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, const int32_t* block_table, int32_t k, float* o,
                               int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
    santa::Params p;
    Plan plan;
    santa_status st = make_params(shape, q, k_cache, v_cache, seq_lens, block_table, k, SANTA_MODE_SYSTEMATIC, 0,
                                  o, idx, workspace, workspace_bytes, &p, &plan);
    if (st != SANTA_STATUS_OK) return st;
    if (k > santa::kMaxTopk)
        return fail(SANTA_STATUS_UNSUPPORTED, "santa_decode_topk keeps at most %d keys (k = %d)", santa::kMaxTopk, k);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    st = hip_check(santa::launch_score(p, shape->dtype, hs, false), "launching the score pass");
    if (st != SANTA_STATUS_OK) return st;
    st = hip_check(santa::launch_topk(p, shape->dtype, hs), "launching the top-k selection");
    if (st != SANTA_STATUS_OK) return st;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_decode_bernoulli(const santa_shape* shape, const void* q, const void* k_t,
                                    const santa_kt_layout* kt, const void* v_cache, const int32_t* seq_lens,
                                    int32_t num_samples, int32_t mode, uint64_t seed, int32_t num_bernoulli,
                                    float* o, int32_t* idx, uint8_t* feature_counts, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    santa::Params p;
    Plan plan;
    santa_status st = make_params(shape, q, k_t, v_cache, seq_lens, nullptr, num_samples, mode, seed, o, idx,
                                  workspace, workspace_bytes, &p, &plan);
    if (st != SANTA_STATUS_OK) return st;
    if (!kt || !feature_counts) return fail(SANTA_STATUS_INVALID_ARGUMENT, "kt layout or feature_counts is NULL");
    if (shape->page_size != 0)
        return fail(SANTA_STATUS_UNSUPPORTED, "santa_decode_bernoulli reads a contiguous K^T (page_size must be 0)");
    if (num_bernoulli < 1 || num_bernoulli > santa::kMaxBernoulli)
        return fail(SANTA_STATUS_UNSUPPORTED, "num_bernoulli %d not in [1, %d]", num_bernoulli, santa::kMaxBernoulli);
    const int64_t eb = plan.elem_bytes;
    if (kt->stride_feat < shape->max_seq_len || kt->stride_seq < 0 || kt->stride_head < 0)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "K^T rows must hold max_seq_len tokens (stride_feat %lld < %d)",
                    (long long)kt->stride_feat, shape->max_seq_len);
    if ((kt->stride_feat * eb) % 16 || (kt->stride_seq * eb) % 16 || (kt->stride_head * eb) % 16)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "K^T strides must keep every row 16-byte aligned");
    p.kt = k_t;
    p.kt_stride_seq = kt->stride_seq;
    p.kt_stride_head = kt->stride_head;
    p.kt_stride_feat = kt->stride_feat;
    p.bern_B = num_bernoulli;
    p.bern_counts = feature_counts;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int path = choose_path(p, shape->dtype, true);
    if (path == 0) return fail(SANTA_STATUS_HIP_ERROR, "querying the device for the launch plan failed");
    if (mode == SANTA_MODE_MULTINOMIAL) {
        st = hip_check(santa::launch_targets(p, hs), "launching the target sort");
        if (st != SANTA_STATUS_OK) return st;
    }
    if (path == 1 || path == 3) {
        if (path == 1) {
            p.item_order = p.T % 8 == 0 ? santa::kOrderTokenBlocks : santa::kOrderHeadFastest;
        } else {
            p.item_order = santa::kOrderSplitFastest;
            p.use_ticket = 1;
        }
        st = hip_check(santa::launch_bern_fused(p, shape->dtype, hs), "launching the fused Bernoulli kernel");
    } else {
        st = hip_check(santa::launch_bern_score(p, shape->dtype, hs), "launching the Bernoulli score pass");
        if (st == SANTA_STATUS_OK)
            st = hip_check(santa::launch_sample(p, shape->dtype, hs), "launching the sample pass");
    }
    if (st != SANTA_STATUS_OK) return st;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_decode_args(const santa_args* a, void* stream) {
    if (!a) return fail(SANTA_STATUS_INVALID_ARGUMENT, "args is NULL");
    if (a->flags & ~(uint32_t)SANTA_FLAG_TWO_KERNEL)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "unknown flags 0x%x", a->flags);
    switch (a->algorithm) {
        case SANTA_ALGO_PROP:
            return run(kDecode, &a->shape, a->q, a->k_cache, a->v_cache, a->seq_lens, a->block_table,
                       a->num_samples, a->mode, a->seed, a->o, a->idx, a->workspace, a->workspace_bytes, stream,
                       a->flags);
        case SANTA_ALGO_FLASH:
            return santa_decode_flash(&a->shape, a->q, a->k_cache, a->v_cache, a->seq_lens, a->block_table,
                                      a->num_samples, a->mode, a->seed, a->o, a->idx, a->workspace,
                                      a->workspace_bytes, stream);
    }
    return fail(SANTA_STATUS_INVALID_ARGUMENT, "unknown algorithm %d", a->algorithm);
}

santa_status santa_workspace_status(const void* workspace, size_t workspace_bytes, void* stream,
                                    uint32_t* error_word) {
    if (!workspace || !error_word) return fail(SANTA_STATUS_INVALID_ARGUMENT, "workspace or error_word is NULL");
    if (!aligned(workspace, 256)) return fail(SANTA_STATUS_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (workspace_bytes < santa::kSyncBytes)
        return fail(SANTA_STATUS_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs at least %zu",
                    workspace_bytes, santa::kSyncBytes);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint32_t word = 0;
    santa_status st = hip_check(hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, hs),
                                "reading the workspace's error word");
    if (st != SANTA_STATUS_OK) return st;
    st = hip_check(hipStreamSynchronize(hs), "waiting for the stream");
    if (st != SANTA_STATUS_OK) return st;
    *error_word = word;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_score_pass(const santa_shape* shape, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                              int32_t num_samples, int32_t mode, uint64_t seed, float* o, int32_t* idx,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return run(kScore, shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed,
               o, idx, workspace, workspace_bytes, stream);
}

santa_status santa_sample_pass(const santa_shape* shape, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                               int32_t num_samples, int32_t mode, uint64_t seed, float* o, int32_t* idx,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return run(kSample, shape, q, k_cache, v_cache, seq_lens, block_table, num_samples, mode, seed,
               o, idx, workspace, workspace_bytes, stream);
}


int32_t santa_pp_num_teams(int32_t N, int32_t P, int32_t R) {
    const int64_t m = pp_teams(N, P, R);
    return m < 0 || m > INT32_MAX ? -1 : (int32_t)m;
}

santa_status santa_pp_build(const santa_shape* shape, const void* k_cache, const void* v_cache, int32_t N,
                            int32_t P, int32_t R, const santa_pp_table* table, void* stream) {
    int G = 0;
    int64_t M = 0;
    santa_status st = pp_check(shape, N, P, R, &G, &M);
    if (st != SANTA_STATUS_OK) return st;
    if (!k_cache || !v_cache) return fail(SANTA_STATUS_INVALID_ARGUMENT, "k_cache or v_cache is NULL");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "k_cache and v_cache must be 16-byte aligned");
    st = pp_table_check(table);
    if (st != SANTA_STATUS_OK) return st;
    santa::PPParams p;
    pp_fill(&p, shape, G, N, P, R, M, table);
    p.k = k_cache;
    p.v = v_cache;
    st = hip_check(santa::launch_pp_build(p, shape->dtype, static_cast<hipStream_t>(stream)), "launching the team build");
    if (st != SANTA_STATUS_OK) return st;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_pp_workspace_size(const santa_shape* shape, int32_t N, int32_t P, int32_t R, int32_t K,
                                     size_t* bytes) {
    int G = 0;
    int64_t M = 0;
    santa_status st = pp_check(shape, N, P, R, &G, &M);
    if (st != SANTA_STATUS_OK) return st;
    if (K < 1) return fail(SANTA_STATUS_INVALID_ARGUMENT, "the team count K must be >= 1 (got %d)", K);
    if (!bytes) return fail(SANTA_STATUS_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = pp_layout(*shape, M).total;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

santa_status santa_pp_decode(const santa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, int32_t N, int32_t P, int32_t R, const santa_pp_table* table,
                             int32_t K, uint64_t seed, float* o, int32_t* teams, float* corr, void* workspace,
                             size_t workspace_bytes, void* stream) {
    int G = 0;
    int64_t M = 0;
    santa_status st = pp_check(shape, N, P, R, &G, &M);
    if (st != SANTA_STATUS_OK) return st;
    if (K < 1) return fail(SANTA_STATUS_INVALID_ARGUMENT, "the team count K must be >= 1 (got %d)", K);
    if (!q || !k_cache || !v_cache || !seq_lens || !o || !teams || !corr || !workspace)
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "a required pointer is NULL");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
        !aligned(seq_lens, 4) || !aligned(teams, 4) || !aligned(corr, 4))
        return fail(SANTA_STATUS_INVALID_ARGUMENT, "q, the caches and o must be 16-byte, the index arrays 4-byte aligned");
    if (!aligned(workspace, 256)) return fail(SANTA_STATUS_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    st = pp_table_check(table);
    if (st != SANTA_STATUS_OK) return st;
    const int64_t Keff = std::min<int64_t>(K, M);
    const PPLayout L = pp_layout(*shape, M);
    if (workspace_bytes < L.total)
        return fail(SANTA_STATUS_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    santa::PPParams p;
    pp_fill(&p, shape, G, N, P, R, M, table);
    char* w = static_cast<char*>(workspace);
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.seq_lens = seq_lens;
    p.seed = seed;
    p.K = K;
    p.Keff = (int)Keff;
    p.o = o;
    p.teams = teams;
    p.corr = corr;
    p.y = reinterpret_cast<float*>(w + L.y);
    p.phi = reinterpret_cast<float*>(w + L.phi);
    p.logc = reinterpret_cast<float*>(w + L.logc);
    p.mask = reinterpret_cast<unsigned int*>(w + L.mask);
    p.part = reinterpret_cast<float*>(w + L.part);
    st = hip_check(santa::launch_pp_decode(p, shape->dtype, static_cast<hipStream_t>(stream)),
                   "launching the SANTA++ decode");
    if (st != SANTA_STATUS_OK) return st;
    g_error[0] = '\0';
    return SANTA_STATUS_OK;
}

}  // extern "C"
