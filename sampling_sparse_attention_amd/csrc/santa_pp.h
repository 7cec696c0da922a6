// Parameters and launchers of the SANTA++ kernels (santa_pp.hip).
#pragma once

#include "santa_internal.h"

namespace santa {

constexpr int kPPMaxParent = 64;        // one wave per parent
constexpr int kPPMaxTeams = 131072;     // the selection's union mask is one LDS byte per team
constexpr int kPPChunks = 16;           // attend workgroups per (sequence, KV head)

struct PPParams {
    int B, Hq, Hkv, G, D;
    int N, P, R, M, Mpad, K, Keff, PL, NC;
    int n_max;
    const void* q;
    const void* k;                 // token-major caches (prompt rows for the build, suffix rows for decoding)
    const void* v;
    int64_t stride_seq, stride_tok, stride_head;
    const int32_t* seq_lens;
    void* packed_k;                // [B, Hkv, N, D]
    void* packed_v;
    void* rep_k;                   // [B, Hkv, M, D]
    int32_t* team_start;           // [B, Hkv, M + 1]
    int32_t* perm;                 // [B, Hkv, N]
    uint64_t seed;
    float scale;
    float* o;                      // [B, Hq, D]
    int32_t* teams;                // [B, Hq, K + 1]
    float* corr;                   // [B, Hq, K]
    unsigned int* arrive;          // [B * Hkv]
    unsigned int* done;            // [B * Hkv]
    float* y;                      // [B, Hq, Mpad]
    float* phi;                    // [B, Hq, Mpad]
    int32_t* plan;                 // [B, Hkv, PL]: team | heads << 24
    float* plan_logc;              // [B, Hkv, PL, G]
    int32_t* plan_n;               // [B, Hkv]
    float* part;                   // [B, Hq, NC, D + 2]
};

hipError_t launch_pp_build(const PPParams& p, int dtype, hipStream_t stream);
hipError_t launch_pp_decode(const PPParams& p, int dtype, hipStream_t stream);

}  // namespace santa
