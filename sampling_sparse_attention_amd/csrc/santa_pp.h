// Parameters and launchers of the SANTA++ kernels (santa_pp.hip).
#pragma once

#include "santa_internal.h"

namespace santa {

constexpr int kPPMaxParent = 64;        // one wave per parent
constexpr int kPPMaxTeams = 131072;     // the selection's union mask is one LDS byte per team
constexpr int kPPChunks = 32;           // attend workgroups per (sequence, KV head)

struct PPParams {
    int B, Hq, Hkv, G, D;
    int N, P, R, M, Mpad, K, Keff, NC;
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
    float* y;                      // [B, Hq, Mpad]
    float* phi;                    // [B, Hq, Mpad]
    float* logc;                   // [B, Hq, Mpad]: log c_g of the head's selected teams
    unsigned int* mask;            // [B, Hkv, Mpad / 4]: per team, a byte of the heads that chose it
    float* part;                   // [B, Hq, NC, D + 2]
};

hipError_t launch_pp_build(const PPParams& p, int dtype, hipStream_t stream);
hipError_t launch_pp_decode(const PPParams& p, int dtype, hipStream_t stream);

}  // namespace santa
