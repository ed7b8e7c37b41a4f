// fa_internal.h -- launch interface between the C ABI layer (fa_api.hip) and
// the kernel files.  Host-side only; the arguments have been validated by the
// caller, so launchers only pick an instance and a grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
    const void *Q, *K, *V;
    void *O;
    float *L;
    int64_t B, H, Nq, Nk, d;
    float scale;
    int causal;
    int64_t kv_block;  // fp32 path: keys per online-softmax step
    int64_t q_start;   // causal: query row i sits at key position q_start + i
};

struct BwdArgs {
    const void *Q, *K, *V, *O, *dO;
    const float *L;
    void *dQ, *dK, *dV;
    float *D;   // workspace [B][H][Nq]: rowsum(dO * O)
    float *L2;  // workspace [B][H][Nq]: L * log2(e)
    int64_t B, H, Nq, Nk, d;
    float scale;
    int causal;
    int64_t q_start;  // causal: query row i sits at key position q_start + i
};

struct DecodeArgs {
    const void *Q, *K, *V;
    float *part_m, *part_l, *part_o;
    int64_t B, H, Nq, Nk, d, n_split;
    float scale;
    int causal;       // query row i sees keys 0 .. q_start + i only
    int64_t q_start;
};

struct MergeArgs {
    const float *part_m, *part_l, *part_o;
    void *O;
    float *L;
    int64_t rows, d, n_split;
    int out_bf16;
};

// Debug build (FA_STATS=1): event counters of the bf16 kernels, one array per
// source file, indexed by fa_stat (include/fa_stats.h).
#ifndef FA_STATS
#define FA_STATS 0
#endif
constexpr int kStatCount = 8;
#if FA_STATS
hipError_t stats_fwd(unsigned long long *host, bool reset);  // copy out, or zero
hipError_t stats_bwd(unsigned long long *host, bool reset);
void fwd_bf16_tile(int64_t d, bool workgroup, int64_t *rows, int64_t *cols);
void bwd_bf16_tiles(int64_t d, int causal, int64_t *kv_rows, int64_t *kv_cols, int64_t *q_rows,
                    int64_t *q_cols);
#endif

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s);
hipError_t launch_decode_split_bf16(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_split_f32(const DecodeArgs &a, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t s);
hipError_t launch_merge_states(const MergeArgs &a, hipStream_t s);

}  // namespace fa
