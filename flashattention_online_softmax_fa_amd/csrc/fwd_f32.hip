// fwd_f32.hip -- fp32 attention forward and split-KV decoding on the vector
// ALUs, any 1 <= d <= 128, with a run-time online-softmax step of kv_block
// keys.
//
// One wave per query row.  Each step scores kv_block keys (lane t scores keys
// t, t+64, ...), takes the step maximum with a wave reduction, rescales the
// running denominator and accumulator by exp2(m_old - m_new) (zero on the
// first step, where m_old = -inf), and adds the step's exp2 weights times V
// (lane c owns output columns c and c+64).  One division at the end, and the
// natural-log L = (m + log2 l) * ln 2.
// Source: tiled (lab.py) and TiledAttention (model.py); flash_forward
// (attention_kernels.py) for the base-e statistics.  Scores are kept in base 2
// (scale * log2 e folded into one multiplier), which is the same recurrence.
//
// The fp32 decoding pass runs the same loop over one split's keys and writes
// the split's unnormalised state (m, l, o) instead of O and L.
// Source: flash_decode and state_of_scores (attention_kernels.py).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxStep = 256;  // 4 keys per lane

// Online-softmax state of one query row over keys [kbeg, kend) of one head,
// walked in steps of `step` keys: base-2 maximum m (of c * q.k), denominator
// l, and the unnormalised accumulator (lane c owns columns c and c + 64).
// An empty range leaves m = -inf, l = 0, acc = 0.
struct RowState {
    float m, l, acc0, acc1;
};

__device__ RowState row_state(const float *__restrict__ q, const float *__restrict__ Kh,
                              const float *__restrict__ Vh, int64_t kbeg, int64_t kend, int d,
                              float c, int step, int lane) {
    RowState st{-INFINITY, 0.f, 0.f, 0.f};
    for (int64_t start = kbeg; start < kend; start += step) {
        const int nb = (int)((start + step < kend ? start + step : kend) - start);
        float s[4];
        float bmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = lane + 64 * u;
            s[u] = -INFINITY;
            if (t < nb) {
                const float *k = Kh + (start + t) * d;
                float dot = 0.f;
                for (int cc = 0; cc < d; ++cc) dot = fmaf(q[cc], k[cc], dot);
                s[u] = dot * c;
            }
            bmax = fmaxf(bmax, s[u]);
        }
        bmax = wave_max(bmax);
        const float m_new = fmaxf(st.m, bmax);
        const float alpha = fast_exp2(st.m - m_new);  // exp2(-inf) = 0 on the first step
        float p[4], psum = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            p[u] = fast_exp2(s[u] - m_new);  // masked keys: exp2(-inf) = 0
            psum += p[u];
        }
        psum = wave_sum(psum);
        st.l = st.l * alpha + psum;
        st.acc0 *= alpha;
        st.acc1 *= alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            for (int t = 0; t < 64; ++t) {
                const int j = 64 * u + t;
                if (j >= nb) break;
                const float pj = __shfl(p[u], t);
                const float *v = Vh + (start + j) * d;
                if (lane < d) st.acc0 = fmaf(pj, v[lane], st.acc0);
                if (lane + 64 < d) st.acc1 = fmaf(pj, v[lane + 64], st.acc1);
            }
        }
        st.m = m_new;
    }
    return st;
}

__global__ __launch_bounds__(256) void fwd_f32_kernel(const float *__restrict__ Q,
                                                      const float *__restrict__ K,
                                                      const float *__restrict__ V,
                                                      float *__restrict__ O, float *__restrict__ L,
                                                      int64_t rows, int64_t Nq, int64_t Nk, int d,
                                                      float c, int causal, int64_t qoff,
                                                      int step) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row >= rows) return;  // wave-uniform; the kernel has no block barrier
    const int64_t bh = row / Nq, i = row % Nq;
    // causal: keys 0 .. qoff + i are visible (qoff >= 0, so at least key 0)
    const int64_t nvis = causal ? (qoff + i + 1 < Nk ? qoff + i + 1 : Nk) : Nk;
    const RowState st =
        row_state(Q + row * d, K + bh * Nk * d, V + bh * Nk * d, 0, nvis, d, c, step, lane);
    const float inv = 1.f / st.l;
    if (lane < d) O[row * d + lane] = st.acc0 * inv;
    if (lane + 64 < d) O[row * d + lane + 64] = st.acc1 * inv;
    if (lane == 0) L[row] = (st.m + log2f(st.l)) * kLn2;
}

// Split-KV decoding in fp32: one wave per (query row, split); the state of
// the split's visible keys, m in natural-log units (the scale applied).
__global__ __launch_bounds__(256) void decode_split_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ part_m, float *__restrict__ part_l, float *__restrict__ part_o,
    int64_t items, int64_t Nq, int64_t Nk, int d, int64_t n_split, float c, int causal,
    int64_t qoff) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
    if (item >= items) return;  // wave-uniform
    const int64_t row = item / n_split, split = item % n_split;
    const int64_t bh = row / Nq, i = row % Nq;
    const int64_t j0 = Nk * split / n_split;
    int64_t j1 = Nk * (split + 1) / n_split;
    if (causal && qoff + i + 1 < j1) j1 = qoff + i + 1;
    const RowState st =
        row_state(Q + row * d, K + bh * Nk * d, V + bh * Nk * d, j0, j1, d, c, 64, lane);
    float *po = part_o + item * d;
    if (lane < d) po[lane] = st.acc0;
    if (lane + 64 < d) po[lane + 64] = st.acc1;
    if (lane == 0) {
        part_m[item] = st.m * kLn2;  // -inf for an empty split
        part_l[item] = st.l;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t s) {
    const int64_t rows = a.B * a.H * a.Nq;
    const int64_t blocks = (rows + kWaves - 1) / kWaves;
    int step = (int)(a.kv_block > 0 ? a.kv_block : 64);
    if (step > kMaxStep) step = kMaxStep;
    hipLaunchKernelGGL(fwd_f32_kernel, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s,
                       (const float *)a.Q, (const float *)a.K, (const float *)a.V, (float *)a.O,
                       a.L, rows, a.Nq, a.Nk, (int)a.d, a.scale * kLog2e, a.causal, a.q_start,
                       step);
    return hipGetLastError();
}

hipError_t launch_decode_split_f32(const DecodeArgs &a, hipStream_t s) {
    const int64_t items = a.B * a.H * a.Nq * a.n_split;
    const int64_t blocks = (items + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(decode_split_f32_kernel, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s,
                       (const float *)a.Q, (const float *)a.K, (const float *)a.V, a.part_m,
                       a.part_l, a.part_o, items, a.Nq, a.Nk, (int)a.d, a.n_split,
                       a.scale * kLog2e, a.causal, a.q_start);
    return hipGetLastError();
}

}  // namespace fa
