// decode.hip -- split-KV decoding (Flash-Decoding) and the merge of
// (m, l, o) states.
//
// Pass 1 (decode_split_kernel): one workgroup per (query row, split).  The
// split's keys are streamed once from HBM: d/8 lanes hold one key row
// (16 bytes each), so a wave instruction covers 64*8/d whole rows and every
// load is a contiguous 1 KiB.  Each lane group keeps its own running
// (m, l, o[8]) over the keys it visits; groups and waves are merged through
// LDS at the end with the merge rule.  Nothing here is a dense contraction
// (one query row), so it runs on the vector ALUs; the bound is HBM bandwidth.
// Source: flash_decode and state_of_scores (attention_kernels.py): split
// bounds, per-split summaries, and the empty split as the identity.  With
// the causal offset, row i of the Nq new tokens sees keys 0 .. q_start + i
// (the mask of standard_attention), so a split can be empty for some rows.
//
// Pass 2 (merge_states_kernel): one workgroup per row folds the n_split
// summaries with merge_states (attention_kernels.py): largest m, rebase both
// sides, base 0 when every m is -inf; then O = o / l and L = m + log l.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kUnroll = 4;

// Sum over aligned groups of G lanes (G in {8, 16}) with DPP row permutes;
// every lane of the group receives the group total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
    if (G == 16)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
    return v;
}

// q . k over this lane's 8 columns (packed bf16 words), fp32 accumulation.
__device__ __forceinline__ float dot8(const u32x4 &q, const u32x4 &k) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        s = fmaf(bf16_lo(q[w]), bf16_lo(k[w]), s);
        s = fmaf(bf16_hi(q[w]), bf16_hi(k[w]), s);
    }
    return s;
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_o, int64_t Nq, int64_t Nk, int64_t n_split, float c, int causal,
    int64_t qoff) {
    constexpr int LPK = D / 8;       // lanes per key row
    constexpr int KPI = 64 / LPK;    // key rows per wave instruction
    constexpr int NG = kDecWaves * KPI;  // lane groups per workgroup
    __shared__ float sm[NG], sl[NG];
    __shared__ float so[NG][D + 1];

    const int64_t item = blockIdx.x;
    const int64_t row = item / n_split, split = item % n_split;
    const int64_t bh = row / Nq;
    const int64_t j0 = Nk * split / n_split;
    int64_t j1 = Nk * (split + 1) / n_split;
    // causal over the new tokens: row i (of Nq) sees keys 0 .. qoff + i
    if (causal && qoff + row % Nq + 1 < j1) j1 = qoff + row % Nq + 1;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int grp = lane / LPK, sub = lane % LPK;
    const int g = wave * KPI + grp;  // this lane group's id in the workgroup

    const u32x4 q = *(const u32x4 *)(Q + row * D + sub * 8);
    const uint16_t *Kh = K + bh * Nk * D + sub * 8;
    const uint16_t *Vh = V + bh * Nk * D + sub * 8;

    float m = -INFINITY, l = 0.f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;

    // lane group g visits keys j0 + g, j0 + g + NG, ...
    for (int64_t jb = j0 + g; jb < j1; jb += (int64_t)NG * kUnroll) {
        u32x4 kr[kUnroll], vr[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = jb + (int64_t)u * NG;
            ok[u] = j < j1;
            const int64_t jj = ok[u] ? j : jb;  // stay in bounds
            kr[u] = __builtin_nontemporal_load((const u32x4 *)(Kh + jj * D));
            vr[u] = __builtin_nontemporal_load((const u32x4 *)(Vh + jj * D));
        }
        float s[kUnroll];
        float smax = -INFINITY;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            s[u] = group_sum<LPK>(dot8(q, kr[u])) * c;
            if (!ok[u]) s[u] = -INFINITY;
            smax = fmaxf(smax, s[u]);
        }
        const float m_new = fmaxf(m, smax);  // finite: key jb is always valid
        const float alpha = fast_exp2(m - m_new);
        float p[kUnroll];
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            p[u] = fast_exp2(s[u] - m_new);
            psum += p[u];
        }
        l = l * alpha + psum;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                o[2 * w] = fmaf(p[u], bf16_lo(vr[u][w]), o[2 * w]);
                o[2 * w + 1] = fmaf(p[u], bf16_hi(vr[u][w]), o[2 * w + 1]);
            }
        }
        m = m_new;
    }

    if (sub == 0) {
        sm[g] = m;
        sl[g] = l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) so[g][sub * 8 + e] = o[e];
    __syncthreads();

    // fold the NG lane-group states; m stays in base-2 scaled units here
    float M = -INFINITY;
    for (int t = 0; t < NG; ++t) M = fmaxf(M, sm[t]);
    const float base = (M == -INFINITY) ? 0.f : M;
    float* pm = part_m + row * n_split + split;
    float* pl = part_l + row * n_split + split;
    float* po = part_o + (row * n_split + split) * D;
    for (int col = threadIdx.x; col < D; col += kDecThreads) {
        float acc = 0.f;
        for (int t = 0; t < NG; ++t) acc = fmaf(so[t][col], fast_exp2(sm[t] - base), acc);
        po[col] = acc;
    }
    if (threadIdx.x == 0) {
        float lt = 0.f;
        for (int t = 0; t < NG; ++t) lt = fmaf(sl[t], fast_exp2(sm[t] - base), lt);
        *pm = M * kLn2;  // natural-log units: max of scale * q . k
        *pl = lt;
    }
}

constexpr int kMergeThreads = 128;

template <bool kBf16Out>
__global__ __launch_bounds__(kMergeThreads) void merge_states_kernel(
    const float *__restrict__ part_m, const float *__restrict__ part_l,
    const float *__restrict__ part_o, void *__restrict__ O, float *__restrict__ L, int64_t d,
    int64_t n_split) {
    const int64_t row = blockIdx.x;
    const float *pm = part_m + row * n_split;
    const float *pl = part_l + row * n_split;
    const float *po = part_o + row * n_split * d;
    float M = -INFINITY;
    for (int64_t s = 0; s < n_split; ++s) M = fmaxf(M, pm[s]);
    const float base = (M == -INFINITY) ? 0.f : M;
    float l = 0.f;
    for (int64_t s = 0; s < n_split; ++s) l = fmaf(pl[s], fast_exp2((pm[s] - base) * kLog2e), l);
    const float inv = 1.f / l;
    for (int64_t col = threadIdx.x; col < d; col += kMergeThreads) {
        float acc = 0.f;
        for (int64_t s = 0; s < n_split; ++s)
            acc = fmaf(po[s * d + col], fast_exp2((pm[s] - base) * kLog2e), acc);
        const float out = acc * inv;
        if (kBf16Out) {
            uint32_t w = pack_bf16x2(out, 0.f);
            ((uint16_t *)O)[row * d + col] = (uint16_t)(w & 0xffffu);
        } else {
            ((float *)O)[row * d + col] = out;
        }
    }
    if (threadIdx.x == 0) L[row] = M + logf(l);
}

}  // namespace

hipError_t launch_decode_split_bf16(const DecodeArgs &a, hipStream_t s) {
    const int64_t rows = a.B * a.H * a.Nq;
    const dim3 grid((unsigned)(rows * a.n_split));
    const float c = a.scale * kLog2e;
    if (a.d == 128)
        hipLaunchKernelGGL(decode_split_kernel<128>, grid, dim3(kDecThreads), 0, s,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           a.part_m, a.part_l, a.part_o, a.Nq, a.Nk, a.n_split, c, a.causal,
                           a.q_start);
    else
        hipLaunchKernelGGL(decode_split_kernel<64>, grid, dim3(kDecThreads), 0, s,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           a.part_m, a.part_l, a.part_o, a.Nq, a.Nk, a.n_split, c, a.causal,
                           a.q_start);
    return hipGetLastError();
}

hipError_t launch_merge_states(const MergeArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)a.rows);
    if (a.out_bf16)
        hipLaunchKernelGGL(merge_states_kernel<true>, grid, dim3(kMergeThreads), 0, s, a.part_m,
                           a.part_l, a.part_o, a.O, a.L, a.d, a.n_split);
    else
        hipLaunchKernelGGL(merge_states_kernel<false>, grid, dim3(kMergeThreads), 0, s, a.part_m,
                           a.part_l, a.part_o, a.O, a.L, a.d, a.n_split);
    return hipGetLastError();
}

}  // namespace fa
