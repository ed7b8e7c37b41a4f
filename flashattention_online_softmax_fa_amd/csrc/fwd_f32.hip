// fwd_f32.hip -- fp32 attention forward on the vector ALUs, any 1 <= d <= 128,
// with a run-time online-softmax step of kv_block keys.
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
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxStep = 256;  // 4 keys per lane

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
    const float *q = Q + row * d;
    const float *Kh = K + bh * Nk * d;
    const float *Vh = V + bh * Nk * d;
    // causal: keys 0 .. qoff + i are visible (qoff >= 0, so at least key 0)
    const int64_t nvis = causal ? (qoff + i + 1 < Nk ? qoff + i + 1 : Nk) : Nk;

    float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int64_t start = 0; start < nvis; start += step) {
        const int nb = (int)((start + step < nvis ? start + step : nvis) - start);
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
        const float m_new = fmaxf(m, bmax);
        const float alpha = fast_exp2(m - m_new);  // exp2(-inf) = 0 on the first step
        float p[4], psum = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            p[u] = fast_exp2(s[u] - m_new);  // masked keys: exp2(-inf) = 0
            psum += p[u];
        }
        psum = wave_sum(psum);
        l = l * alpha + psum;
        acc0 *= alpha;
        acc1 *= alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            for (int t = 0; t < 64; ++t) {
                const int j = 64 * u + t;
                if (j >= nb) break;
                const float pj = __shfl(p[u], t);
                const float *v = Vh + (start + j) * d;
                if (lane < d) acc0 = fmaf(pj, v[lane], acc0);
                if (lane + 64 < d) acc1 = fmaf(pj, v[lane + 64], acc1);
            }
        }
        m = m_new;
    }
    const float inv = 1.f / l;
    if (lane < d) O[row * d + lane] = acc0 * inv;
    if (lane + 64 < d) O[row * d + lane + 64] = acc1 * inv;
    if (lane == 0) L[row] = (m + log2f(l)) * kLn2;
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

}  // namespace fa
