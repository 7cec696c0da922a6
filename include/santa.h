/*
 * santa.h -- C ABI of the SANTA decode-step attention library (libsanta.so).
 *
 * SANTA ("Stochastic Sparse Attention for Memory-Bound Inference", Lee et al.)
 * replaces the value stage of decode attention by sampling:
 *
 *   s_i = q . k_i / sqrt(d)              exact scores over the whole cache (§2, Eq. 1)
 *   p   = softmax(s)                     the post-softmax row as a categorical law (§2)
 *   i_1..i_S ~ p                         multinomial (i.i.d.), stratified or
 *                                        systematic draws (§2, Eq. 3; §2.1)
 *   o   = (1/S) * sum_s v_{i_s}          gather-and-add of only the sampled V rows
 *                                        (§2, Eq. 2-3), an unbiased estimate of A V
 *                                        (Appendix A.1, A.4)
 *
 * The library computes this for one decode step of a batch of sequences with
 * grouped-query attention (G = Hq / Hkv query heads share one KV head), on one
 * gfx950 GPU.  It follows the proportional-allocation kernel strategy of §3.2
 * (exact tile statistics, a global partition function, then a parallel gather
 * in which each tile draws exactly the samples that fall into its share of the
 * probability mass).
 *
 * Sampling conventions (the pages leave these open):
 *   - uniforms: U = (w0 >> 11) * 2^-53, w0 = word 0 of Philox4x64-10 (Salmon
 *     et al., SC 2011) with key (seed, 0) and counter (j, h, b, 0) for draw j
 *     of query head h of sequence b;
 *   - targets: multinomial sorts U_0..U_{S-1}; stratified t_m = (m + U_m) / S;
 *     systematic t_m = (m + U_0) / S;
 *   - key i is chosen for target t iff F(i) <= t < F(i+1), F the CDF of p
 *     (Appendix A.4); a target at or past F(n) takes the last key of positive
 *     mass;
 *   - idx lists the S chosen logical token positions in ascending target
 *     order; a sequence of length 0 gives o = 0 and idx = -1.
 *
 * Ownership and execution: the caller allocates and owns every buffer (all
 * device pointers below point to device memory on the current HIP device).
 * The library never allocates device memory and never synchronises; every
 * kernel is enqueued on the given stream (NULL: the default stream), so calls
 * can be captured into a HIP graph.  Host-side argument checks happen before
 * anything is enqueued; on any non-OK status nothing was enqueued.  Errors
 * raised while kernels run surface at the caller's next synchronisation.
 *
 * State: the library keeps none between calls on the host.  A workspace must
 * be all zero before its first call (santa_workspace_init, or any zero fill).
 * Every completed call leaves it all zero again (except for the error word
 * after a failed wait), the score stash and the multinomial targets included,
 * so one workspace large enough for each of them serves calls of any shapes,
 * modes and sample counts in any order (one problem's stash can lie where
 * another's counts and records are).  The two-kernel path
 * counts as one call from the start of santa_score_pass to the end of the
 * santa_sample_pass that follows it.  Calls that share a workspace must not
 * overlap (same stream, or ordered by events).
 *
 * Failed waits: the kernels that wait for other workgroups bound every wait
 * (about two seconds).  A wait that gives up sets the workspace's error word
 * (byte 0), and the workgroups that gave up write NaN to o and -1 to idx for
 * their (sequence, KV head) group; the call still returns SANTA_STATUS_OK,
 * because the failure happens after it returned.  Every later call on that
 * workspace finds the word set and writes NaN / -1 for every group instead of
 * computing, until santa_workspace_init clears it.  santa_workspace_status
 * reads the word; it is the authoritative signal that a call's outputs are
 * invalid (a group whose own splits did not wait may still hold finite values).
 *
 * Device residency: santa_decode's fused paths (santa_decode_path() == 1 or 3)
 * have the workgroups of one (sequence, KV head) wait for each other, which is
 * safe only while the device can hold every workgroup of the launch at once
 * (path 1), or every workgroup of one group on each compute die (path 3).
 * The library checks that from the occupancy of an otherwise idle device.  A
 * kernel running on the same device at the same time (another stream, another
 * process) can keep workgroups from being placed until the waits give up.
 * Callers that share the device with concurrent kernels pass
 * SANTA_FLAG_TWO_KERNEL to santa_decode_args; the two-kernel path and
 * santa_decode_flash never wait for a workgroup that has not started.
 */
#ifndef SANTA_H
#define SANTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SANTA_ABI_VERSION 4

typedef enum santa_status {
    SANTA_STATUS_OK = 0,
    SANTA_STATUS_INVALID_ARGUMENT = 1,     /* null pointer, bad size, misaligned buffer */
    SANTA_STATUS_UNSUPPORTED = 2,          /* valid but not built: head_dim, group size, S range */
    SANTA_STATUS_WORKSPACE_TOO_SMALL = 3,
    SANTA_STATUS_HIP_ERROR = 4             /* a HIP launch failed; see santa_last_error() */
} santa_status;

/* Sampling rules (§2 and §2.1). */
enum {
    SANTA_MODE_MULTINOMIAL = 0,   /* S i.i.d. draws from p (SANTA) */
    SANTA_MODE_STRATIFIED = 1,    /* one independent draw per stratum [m/S, (m+1)/S) (S2ANTA-strat) */
    SANTA_MODE_SYSTEMATIC = 2     /* one offset shared by all strata (S2ANTA-sys) */
};

/* Element type of q, K and V. */
enum {
    SANTA_DTYPE_BF16 = 0,
    SANTA_DTYPE_F32 = 1
};

/*
 * Problem shape and KV-cache layout.
 *
 * q is [batch, num_q_heads, head_dim], dense.  Query head h reads KV head
 * h / G.  Row (token i, KV head g) of a cache lives at element offset
 *   contiguous (page_size == 0):  b * kv_stride_seq + i * kv_stride_tok + g * kv_stride_head
 *   paged      (page_size  > 0):  P * kv_stride_seq + (i % page_size) * kv_stride_tok
 *                                 + g * kv_stride_head,
 *                                 P = block_table[b * pages_per_seq + i / page_size]
 * and holds head_dim contiguous elements.  K and V share the layout.  Every
 * row must start on a 16-byte boundary.  A contiguous cache holds the rows of
 * tokens 0 .. max_seq_len - 1 of every sequence: the score pass may read K
 * rows past a sequence's length (their scores are never used).
 */
typedef struct santa_shape {
    int32_t batch;            /* B >= 1 */
    int32_t num_q_heads;      /* Hq >= 1 */
    int32_t num_kv_heads;     /* Hkv >= 1, Hq % Hkv == 0, G = Hq / Hkv in {1, 2, 4, 7, 8} */
    int32_t head_dim;         /* d in {64, 128} */
    int32_t max_seq_len;      /* n_max >= 1; seq_lens are clamped to [0, n_max] on the device */
    int32_t page_size;        /* 0: contiguous cache; else a power of two >= 16 */
    int32_t pages_per_seq;    /* paged: row length of block_table, >= ceil(n_max / page_size) */
    int32_t num_pages;        /* paged: pages in each cache; table entries are clamped to [0, num_pages) */
    int32_t dtype;            /* SANTA_DTYPE_* of q, K and V */
    int32_t split_size;       /* keys per split of the score pass: 0 (library default) or a
                                 power of two in [64, 1024] */
    int64_t kv_stride_seq;    /* elements between sequences (contiguous) or pages (paged) */
    int64_t kv_stride_tok;    /* elements between consecutive tokens */
    int64_t kv_stride_head;   /* elements between KV heads */
} santa_shape;

/*
 * Workspace layout (byte offsets into the caller's workspace, 256-byte aligned):
 *   sync     barrier_offset bytes at the start: a 32-bit error word (byte 0)
 *            that becomes nonzero if a bounded wait of a call gave up (that
 *            call's outputs are invalid; santa_workspace_init clears it), and
 *            at byte 128 the item counter of the fused kernel's path 3;
 *   barrier  [B, Hkv] x 18 lines of 128 bytes: per (sequence, KV head) the
 *            counts of its splits that have published their records and that
 *            have added their output in the current call, and 16 copies of a
 *            flag raised once all of them published;
 *   accum    fp32 [B, Hkv, 8, G, d]: partial outputs, added by the splits of a
 *            (sequence, KV head) into slot (split % 8) and summed into o by
 *            the last of them;
 *   flash    santa_decode_flash only: per (sequence, query head) a 64-bit
 *            reference maximum, then (256-byte aligned) fp64 accumulators
 *            [B, Hkv, 4, G, d + 2] of weighted tile means and weights;
 *   records  [B, Hq, num_splits] x 8 bytes: per split the maximum score m and
 *            l = sum exp(s_i - m) (the tile partition functions of section 3.2,
 *            Pass 1) as one word, fp32 l in the high and fp32 m in the low half
 *            (l >= 1 for a split with keys, so 0 means not written yet); then
 *            [B, Hq, num_splits + 2] x 8 bytes of the two-kernel path: the
 *            exclusive prefix W_t of the split masses (2^-40 fixed point),
 *            the total Z after the sequence's last split, and at the end the
 *            maximum M (fp32, low half) and the last split of positive mass
 *            (high half), written by the last split of the score pass;
 *   stash    fp32 [B, Hq, num_splits * split_size]: scaled scores s_i (the
 *            "score stash" of section 3.2, Pass 1), written by
 *            santa_score_pass and read (and cleared) by santa_sample_pass; row
 *            b*Hq+h starts at stash_offset + (b*Hq+h) * stash_row_bytes;
 *   targets  fp64 [B, Hq, S]: sorted multinomial targets (mode 0 only, else
 *            empty).
 * All of it except the error word is zero between calls.
 */
typedef struct santa_workspace_layout {
    size_t total_bytes;
    size_t sync_offset;
    size_t barrier_offset;
    size_t accum_offset;
    size_t flash_offset;
    size_t records_offset;
    size_t stash_offset;
    size_t stash_row_bytes;
    size_t targets_offset;
    int32_t split_size;
    int32_t num_splits;       /* ceil(n_max / split_size) */
} santa_workspace_layout;

/* Version of this ABI (SANTA_ABI_VERSION of the built library). */
int32_t santa_abi_version(void);

/* Human-readable name of a status code; never NULL. */
const char* santa_status_string(santa_status status);

/* Detail of the last non-OK status returned on this host thread ("" if none). */
const char* santa_last_error(void);

/*
 * Workspace layout for a problem.  Host-only arithmetic: touches no device.
 * Returns INVALID_ARGUMENT / UNSUPPORTED for shapes santa_decode would reject.
 */
santa_status santa_workspace_layout_query(const santa_shape* shape, int32_t num_samples,
                                          int32_t mode, santa_workspace_layout* out);

/* Bytes of workspace santa_decode needs (the total_bytes of the layout). */
santa_status santa_workspace_size(const santa_shape* shape, int32_t num_samples, int32_t mode,
                                  size_t* bytes);

/*
 * Zero-fills a workspace (workspace_bytes bytes, 256-byte aligned) with a
 * kernel on `stream`; required once before the first call on a workspace.
 */
santa_status santa_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * How santa_decode will run this problem on the current device: 1 = one fused
 * kernel (score pass, global budget and gather in one launch), used when the
 * device holds one workgroup per work item (sequence, KV head, split) at
 * once; 3 = the same fused kernel when only the splits of one (sequence, KV
 * head) fit at once on a single compute die (XCD): workgroups then take their
 * work items from a counter in the workspace in the order they start, group
 * by group; 2 = the score pass
 * followed by the sample pass otherwise.  Returns the negated santa_status on
 * error.  Queries the HIP runtime, touches no memory.
 */
int32_t santa_decode_path(const santa_shape* shape, int32_t num_samples, int32_t mode);

/*
 * One SANTA decode step.
 *
 *   q            [B, Hq, d] dtype, device
 *   k_cache      K rows, dtype, device, layout as in santa_shape
 *   v_cache      V rows, same layout
 *   seq_lens     [B] int32, device: n_b, the number of valid tokens of sequence b
 *   block_table  [B, pages_per_seq] int32, device; NULL iff page_size == 0
 *   num_samples  S, 1 <= S <= 65536 (multinomial: S <= 8192); may exceed n_b
 *   mode         SANTA_MODE_*
 *   seed         key word 0 of the Philox generator
 *   o            [B, Hq, d] fp32, device, output: the SANTA estimate (Eq. 3)
 *   idx          [B, Hq, S] int32, device, output: sampled token positions
 *   workspace    device scratch of at least santa_workspace_size() bytes,
 *                256-byte aligned, initialised once by santa_workspace_init
 *   stream       hipStream_t to enqueue on (NULL: default stream)
 *
 * The result is a deterministic function of the inputs and seed except for
 * the order of the fp32 additions that form o.
 */
santa_status santa_decode(const santa_shape* shape, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* seq_lens,
                          const int32_t* block_table, int32_t num_samples, int32_t mode,
                          uint64_t seed, float* o, int32_t* idx, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * The two halves of santa_decode, for per-stage checks and timing.  Calling
 * santa_score_pass then santa_sample_pass on one stream with the same
 * arguments is exactly santa_decode.
 *
 * santa_score_pass: the score pass of section 3.2, Pass 1 -- fills the
 *   workspace's stash and records (and, for multinomial sampling, the sorted
 *   targets).  Reads q, K, seq_lens, block_table.
 * santa_sample_pass: global partition function, budget allocation and
 *   parallel gather (section 3.2 steps 2-3) -- writes idx and o.  Reads the
 *   workspace written by santa_score_pass, V, seq_lens, block_table.  It must
 *   directly follow santa_score_pass with the same arguments on the same
 *   workspace; without that call's records it sets the error word.
 * santa_decode runs either these two kernels or the fused kernel with the same
 * results (santa_decode_path says which).
 */
/*
 * S^2ANTA-flash (section 3.3 of "Stochastic Sparse Attention for Memory-Bound
 * Inference"): the same arguments and outputs as santa_decode, computed
 * without the global budget.  The splits of santa_workspace_layout_query are
 * the tiles: the T_b tiles of sequence b share the num_samples samples, tile
 * t taking floor(num_samples / T_b) plus one for t < num_samples mod T_b
 * (idx holds them tile by tile, each tile's in ascending target order); each
 * tile samples by the given rule from its own softmax (Philox stream 1 + t,
 * draw j at counter (j, h, b, 1 + t)), and
 *     o = sum_t (Z_t / Z) * (1/S_t) * sum_j V[idx_tj],
 * with Z_t the tile's partition function.  mode must be
 * SANTA_MODE_STRATIFIED or SANTA_MODE_SYSTEMATIC and num_samples at least the
 * number of splits (else SANTA_STATUS_UNSUPPORTED).  No workgroup waits for
 * another, so every problem size runs as one kernel.  The weights are summed
 * in fp64 relative to one split's maximum score, which needs the maximum
 * scores of a sequence's tiles to lie within about 700 of each other.
 */
santa_status santa_decode_flash(const santa_shape* shape, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                                int32_t num_samples, int32_t mode, uint64_t seed, float* o, int32_t* idx,
                                void* workspace, size_t workspace_bytes, void* stream);

santa_status santa_score_pass(const santa_shape* shape, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* seq_lens,
                              const int32_t* block_table, int32_t num_samples, int32_t mode,
                              uint64_t seed, float* o, int32_t* idx, void* workspace,
                              size_t workspace_bytes, void* stream);

santa_status santa_sample_pass(const santa_shape* shape, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* seq_lens,
                               const int32_t* block_table, int32_t num_samples, int32_t mode,
                               uint64_t seed, float* o, int32_t* idx, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Deterministic top-k attention, the biased comparator the SANTA page measures
 * SANTA against at a matched budget k = S (section 3.4; section 6): the exact
 * scores of every key (Eq. 1, the score pass), the min(k, n_b) keys with the
 * largest scores (lower token index first among equal scores, found by a radix
 * select on the score stash), and attention renormalised over them,
 *     o = sum_{i kept} exp(s_i) v_i / sum_{i kept} exp(s_i).
 * idx [B, Hq, k] lists the kept token positions in ascending order, padded
 * with -1 when n_b < k; a sequence of length 0 gives o = 0.  Arguments as for
 * santa_decode (k in place of num_samples, no mode or seed); the workspace is
 * santa_workspace_size(shape, k, SANTA_MODE_SYSTEMATIC) bytes (its score
 * stash is used and returned to zero).  1 <= k <= 8192 (else
 * SANTA_STATUS_UNSUPPORTED).  Two launches: the score pass, then one
 * workgroup per (sequence, query head).
 */
santa_status santa_decode_topk(const santa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, const int32_t* block_table, int32_t k, float* o,
                               int32_t* idx, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Layout of K transposed (channel-major), for santa_decode_bernoulli: element
 * (sequence b, KV head g, feature i, token j) at
 *   b * stride_seq + g * stride_head + i * stride_feat + j
 * (tokens contiguous; every row 16-byte aligned; stride_feat >= max_seq_len).
 * Elements of a row past its sequence's length, below stride_feat, may be
 * read and do not affect the result.
 */
typedef struct santa_kt_layout {
    int64_t stride_seq;
    int64_t stride_head;
    int64_t stride_feat;
} santa_kt_layout;

/*
 * Bernoulli qK^T with the mean group query, combined with SANTA (section 5,
 * Eq. 5; section 5.1, Eq. 6; section 5.3).  The scores are estimated rather
 * than exact: for every (sequence b, KV head g) group,
 *   m_i      = (1/G) sum_h |q_{h,i}|                 (the mean group query)
 *   count_i  = #{n < B : (n + U_{i,n}) / B < m_i / max_j m_j}
 *              (B stratified Bernoulli draws; U from Philox4x64-10 with key
 *              (seed, 1) and counter (n, i, g, b); decided in fp64)
 *   s_hat_hj = sum_i ((max_j m_j / B) count_i / m_i) q_{h,i} k_{j,i}
 * and SANTA then samples from softmax(s_hat / sqrt(d)) exactly as
 * santa_decode does (same num_samples, mode and seed conventions).  Only the
 * features with count_i > 0 are read from K^T, so skipped features cost no
 * bytes; feature_counts [B, Hkv, d] (uint8, device) receives count_i.
 * Arithmetic of s_hat: the weights (max m / B) count_i / m_i q_{h,i} are
 * formed in fp64 and rounded once to fp32; the kept features, in ascending
 * order, are dealt round-robin to F groups (F = 1, 2 or 4, fixed by the
 * element size and the split), each group sums its terms by fp32 fused
 * multiply-adds in that order, the group sums are added pairwise, and the
 * result is multiplied by the fp32 1/sqrt(d).
 *
 *   shape        sizes and the layout of v_cache (contiguous: page_size 0)
 *   k_t, kt      K transposed and its layout (santa_kt_layout)
 *   v_cache      token-major V as in santa_decode
 *   num_bernoulli B, 1 <= B <= 64
 * Workspace: santa_workspace_size(shape, num_samples, mode) bytes.  Runs the
 * fused kernel (or the score and sample passes) chosen as for santa_decode;
 * every workgroup derives its group's counts itself.
 */
santa_status santa_decode_bernoulli(const santa_shape* shape, const void* q, const void* k_t,
                                    const santa_kt_layout* kt, const void* v_cache, const int32_t* seq_lens,
                                    int32_t num_samples, int32_t mode, uint64_t seed, int32_t num_bernoulli,
                                    float* o, int32_t* idx, uint8_t* feature_counts, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * SANTA++: attention through representative keys ("SANTA++: Sampling
 * Attention through Representative Keys", section 2.2-2.3; Appendix A,
 * Algorithms 1, 2 and 4; Appendix D).
 *
 * After prefill, the N prompt keys of every (sequence, KV head) are cut into
 * contiguous parents of P tokens (Algorithm 4).  In each parent, up to R
 * actual keys become representatives: the first is the member nearest the
 * parent's mean key, each later one the member farthest from its nearest
 * representative so far (ties to the lower token index); every member joins
 * its nearest representative's team (ties to the earlier representative) and
 * each representative owns its own row (Algorithm 2).  Distances are squared
 * Euclidean in fp64 on the keys as stored.  Teams are numbered parent by
 * parent, in the order their representatives were chosen; members keep token
 * order.  A parent of c tokens holds min(R, c) teams, so there are
 * M = (N / P) R + min(R, N mod P) teams (santa_pp_num_teams).
 *
 * Team table (caller-owned device arrays, written by santa_pp_build and read
 * by santa_pp_decode; B, Hkv, d from the shape, dtype of the caches):
 *   packed_k, packed_v  [B, Hkv, N, d]  the prompt rows in team order (team
 *                       g's members are rows team_start[g] .. team_start[g+1]-1)
 *   rep_k               [B, Hkv, M, d]  the representative keys
 *   team_start          [B, Hkv, M + 1] int32
 *   perm                [B, Hkv, N]     int32: token index of each packed row
 * Limits: 1 <= R <= P <= 64, P divisible by R, 1 <= N <= max_seq_len,
 * M <= 131072; contiguous caches only (page_size 0).
 */
typedef struct santa_pp_table {
    void* packed_k;
    void* packed_v;
    void* rep_k;
    int32_t* team_start;
    int32_t* perm;
} santa_pp_table;

/* M for a prompt of N tokens, parents of P and at most R teams each; -1 if the
 * parameters are invalid (R > P, P not divisible by R, N < 1). */
int32_t santa_pp_num_teams(int32_t N, int32_t P, int32_t R);

/* Builds the team table from the first N rows of every sequence of the
 * token-major k_cache / v_cache (layout of shape).  Asynchronous on stream. */
santa_status santa_pp_build(const santa_shape* shape, const void* k_cache, const void* v_cache, int32_t N,
                            int32_t P, int32_t R, const santa_pp_table* table, void* stream);

/* Workspace bytes of santa_pp_decode for K teams per query head (any
 * contents: every call overwrites what it reads). */
santa_status santa_pp_workspace_size(const santa_shape* shape, int32_t N, int32_t P, int32_t R, int32_t K,
                                     size_t* bytes);

/*
 * One SANTA++ decode step (Algorithm 1 for every query head; section 2.3).
 * For query head h of sequence b (KV head g = h / G):
 *   phi_t = log n_t + q . l_t / sqrt(d)                     (Eq. 3, fp32)
 *   Y_t   = phi_t + G_t, G_t = -log(-log U), U = ((w0 >> 11) + 1/2) 2^-53,
 *           w0 word 0 of Philox4x64-10 with key (seed, 2) and counter
 *           (t, h, b, 0)                                    (fp64, added in fp32)
 *   the K teams of largest Y (ties to the lower team index) and tau, the
 *   (K+1)-th largest; c_t = 1 - exp(-exp(phi_t - tau))      (Eq. 7, fp64)
 *   o = U_hat / Z_hat over the suffix rows N .. seq_len-1 of the caches
 *   (weight 1) and every member of the selected teams (weight 1 / c_t),
 *   exponentials of s = q . k / sqrt(d)                     (Eq. 4, fp32)
 * K >= M selects every team with c = 1 (dense attention).  The heads of a GQA
 * group read the union of their teams once (Appendix D); a row of a team that
 * several heads chose is loaded once and weighed per head.
 *
 *   q         [B, Hq, d]; k_cache, v_cache token-major, for the suffix rows;
 *   seq_lens  [B] int32 device: prompt + generated rows (below N counts as N)
 *   o         [B, Hq, d] fp32
 *   teams     [B, Hq, K + 1] int32: the selected teams in ascending order, then
 *             the threshold team (-1 entries past min(K, M) and for K >= M)
 *   corr      [B, Hq, K] fp32: c_t of teams[j] (1 for K >= M)
 * Workspace: santa_pp_workspace_size bytes, 256-byte aligned.  Four launches
 * on stream (routing, selection, attention over the group's union, merge);
 * calls that share a workspace must not overlap.
 */
santa_status santa_pp_decode(const santa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, int32_t N, int32_t P, int32_t R, const santa_pp_table* table,
                             int32_t K, uint64_t seed, float* o, int32_t* teams, float* corr, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Algorithms of santa_args. */
enum {
    SANTA_ALGO_PROP = 0,    /* santa_decode: exact global budget (section 3.2, S2ANTA-prop) */
    SANTA_ALGO_FLASH = 1    /* santa_decode_flash: uniform tile budgets (section 3.3) */
};

/* Flags of santa_args. */
enum {
    SANTA_FLAG_TWO_KERNEL = 1u   /* SANTA_ALGO_PROP: never the fused kernel (see Device residency) */
};

/*
 * Every argument of one decode step in one struct; the fields mean exactly
 * what the arguments of the same names of santa_decode mean.
 */
typedef struct santa_args {
    santa_shape shape;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* seq_lens;
    const int32_t* block_table;
    int32_t num_samples;
    int32_t mode;
    uint64_t seed;
    float* o;
    int32_t* idx;
    void* workspace;
    size_t workspace_bytes;
    int32_t algorithm;      /* SANTA_ALGO_* */
    uint32_t flags;         /* SANTA_FLAG_* (0: santa_decode's own path choice) */
} santa_args;

/*
 * One decode step from a santa_args: santa_decode (SANTA_ALGO_PROP, honouring
 * SANTA_FLAG_TWO_KERNEL) or santa_decode_flash (SANTA_ALGO_FLASH), with their
 * statuses.  Unknown algorithms or flags give SANTA_STATUS_INVALID_ARGUMENT.
 */
santa_status santa_decode_args(const santa_args* args, void* stream);

/*
 * Reads the workspace's error word (nonzero: a bounded wait of a call that
 * used this workspace gave up, see Failed waits) into *error_word.  It waits
 * for the work already enqueued on `stream` (a host synchronisation, unlike
 * every other call of this library).
 */
santa_status santa_workspace_status(const void* workspace, size_t workspace_bytes, void* stream,
                                    uint32_t* error_word);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): santa_decode
 * without a workspace argument.  Its workspace is a 64 MiB array that is part
 * of the library's code object (SANTA_NOALLOC_SCRATCH_BYTES, held by every
 * device the library runs on until the process ends); these calls allocate
 * nothing.  Everything else is santa_decode's: the same kernels, path choice,
 * arguments (minus workspace and workspace_bytes) and results.
 *
 *   - A problem whose santa_workspace_size exceeds the array returns
 *     SANTA_STATUS_WORKSPACE_TOO_SMALL before touching the device (the
 *     Llama-3.1-8B-shaped 32k step needs 4.8 MiB; batch 4 of 28/4 heads at
 *     128k tokens about 60 MiB).
 *   - All calls on one device share that device's array, and its state
 *     carries from call to call exactly as santa_decode's workspace does: a
 *     completed call leaves it zero.  Calls that overlap on one device (two
 *     streams, two threads without ordering) race on it; order them.
 *   - The array must be zero before the first call: santa_noalloc_init clears
 *     it on `stream` (call it once per device before capturing a graph, and
 *     again after santa_noalloc_status reports a failed wait); otherwise the
 *     first santa_decode_noalloc on a device enqueues that clear itself.
 */
#define SANTA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Bytes of the no-allocation scratch array (SANTA_NOALLOC_SCRATCH_BYTES). */
size_t santa_noalloc_scratch_bytes(void);

/* Zero-fills the current device's scratch array on `stream` (a kernel, no allocation). */
santa_status santa_noalloc_init(void* stream);

/* santa_decode on the current device's scratch array (see above). */
santa_status santa_decode_noalloc(const santa_shape* shape, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                                  int32_t num_samples, int32_t mode, uint64_t seed, float* o, int32_t* idx,
                                  void* stream);

/* santa_workspace_status of the current device's scratch array (synchronises `stream`). */
santa_status santa_noalloc_status(void* stream, uint32_t* error_word);

#ifdef __cplusplus
}
#endif

#endif /* SANTA_H */
