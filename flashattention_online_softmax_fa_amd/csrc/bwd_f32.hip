// bwd_f32.hip -- fp32 attention backward on the vector ALUs, any 1 <= d <= 128.
//
// Source: flash_backward (attention_kernels.py): D = rowsum(dO * O); P is
// recomputed from the stored L as exp(S - L); dV += P^T dO, dP = dO V^T,
// dS = P * (dP - D), dK += scale dS^T Q, dQ += scale dS K.  The mask is the
// causal one of standard_attention with query row i at key position
// q_start + i.
//
// Three launches, all fp32, no atomics (deterministic):
//   bwd_f32_pre   one wave per query row: D and L2 = L * log2(e);
//   bwd_f32_dq    one wave per query row: lane t scores keys t, t+64, ... of
//                 each 64-key step, then the step's dS weights times K are
//                 added with lane c owning dQ columns c and c + 64;
//   bwd_f32_dkdv  one wave per key row, the same with the roles of queries and
//                 keys exchanged (the queries that can see the key).
// This path is for exact checks at small sizes (it recomputes every score
// twice and reads K, V, Q, dO through the cache); the bf16 path is the fast
// one.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;

__global__ __launch_bounds__(256) void bwd_f32_pre(const float *__restrict__ O,
                                                   const float *__restrict__ dO,
                                                   const float *__restrict__ L,
                                                   float *__restrict__ Dv, float *__restrict__ L2,
                                                   int64_t rows, int d) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row >= rows) return;  // wave-uniform
    float s = 0.f;
    for (int c = lane; c < d; c += 64) s = fmaf(O[row * d + c], dO[row * d + c], s);
    s = wave_sum(s);
    if (lane == 0) {
        Dv[row] = s;
        L2[row] = L[row] * kLog2e;
    }
}

__device__ __forceinline__ float dot_row(const float *__restrict__ a, const float *__restrict__ b,
                                         int d) {
    float s = 0.f;
    for (int c = 0; c < d; ++c) s = fmaf(a[c], b[c], s);
    return s;
}

__global__ __launch_bounds__(256) void bwd_f32_dq(const float *__restrict__ Q,
                                                  const float *__restrict__ K,
                                                  const float *__restrict__ V,
                                                  const float *__restrict__ dO,
                                                  const float *__restrict__ L2,
                                                  const float *__restrict__ Dv,
                                                  float *__restrict__ dQ, int64_t rows,
                                                  int64_t Nq, int64_t Nk, int d, float scale,
                                                  float c, int causal, int64_t qoff) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row >= rows) return;  // wave-uniform
    const int64_t bh = row / Nq, i = row % Nq;
    const float *q = Q + row * d, *g = dO + row * d;
    const float *Kh = K + bh * Nk * d, *Vh = V + bh * Nk * d;
    const float l2 = L2[row], dd = Dv[row];
    const int64_t nvis = causal ? (qoff + i + 1 < Nk ? qoff + i + 1 : Nk) : Nk;
    float acc0 = 0.f, acc1 = 0.f;
    for (int64_t start = 0; start < nvis; start += 64) {
        const int nb = (int)(start + 64 < nvis ? 64 : nvis - start);
        float ds = 0.f;
        if (lane < nb) {
            const int64_t j = start + lane;
            const float p = fast_exp2(fmaf(dot_row(q, Kh + j * d, d), c, -l2));
            ds = p * (dot_row(g, Vh + j * d, d) - dd);
        }
        for (int t = 0; t < nb; ++t) {
            const float w = __shfl(ds, t);
            const float *k = Kh + (start + t) * d;
            if (lane < d) acc0 = fmaf(w, k[lane], acc0);
            if (lane + 64 < d) acc1 = fmaf(w, k[lane + 64], acc1);
        }
    }
    if (lane < d) dQ[row * d + lane] = scale * acc0;
    if (lane + 64 < d) dQ[row * d + lane + 64] = scale * acc1;
}

__global__ __launch_bounds__(256) void bwd_f32_dkdv(const float *__restrict__ Q,
                                                    const float *__restrict__ K,
                                                    const float *__restrict__ V,
                                                    const float *__restrict__ dO,
                                                    const float *__restrict__ L2,
                                                    const float *__restrict__ Dv,
                                                    float *__restrict__ dK, float *__restrict__ dV,
                                                    int64_t keys, int64_t Nq, int64_t Nk, int d,
                                                    float scale, float c, int causal,
                                                    int64_t qoff) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t key = (int64_t)blockIdx.x * kWaves + wave;
    if (key >= keys) return;  // wave-uniform
    const int64_t bh = key / Nk, j = key % Nk;
    const float *k = K + key * d, *v = V + key * d;
    const float *Qh = Q + bh * Nq * d, *dOh = dO + bh * Nq * d;
    const float *L2h = L2 + bh * Nq, *Dh = Dv + bh * Nq;
    // causal: query i sees key j iff j <= qoff + i
    const int64_t i0 = causal ? (j - qoff > 0 ? j - qoff : 0) : 0;
    float dk0 = 0.f, dk1 = 0.f, dv0 = 0.f, dv1 = 0.f;
    for (int64_t start = i0; start < Nq; start += 64) {
        const int nb = (int)(start + 64 < Nq ? 64 : Nq - start);
        float p = 0.f, ds = 0.f;
        if (lane < nb) {
            const int64_t i = start + lane;
            p = fast_exp2(fmaf(dot_row(Qh + i * d, k, d), c, -L2h[i]));
            ds = p * (dot_row(dOh + i * d, v, d) - Dh[i]);
        }
        for (int t = 0; t < nb; ++t) {
            const float wp = __shfl(p, t), wd = __shfl(ds, t);
            const float *qi = Qh + (start + t) * d, *gi = dOh + (start + t) * d;
            if (lane < d) {
                dv0 = fmaf(wp, gi[lane], dv0);
                dk0 = fmaf(wd, qi[lane], dk0);
            }
            if (lane + 64 < d) {
                dv1 = fmaf(wp, gi[lane + 64], dv1);
                dk1 = fmaf(wd, qi[lane + 64], dk1);
            }
        }
    }
    if (lane < d) {
        dK[key * d + lane] = scale * dk0;
        dV[key * d + lane] = dv0;
    }
    if (lane + 64 < d) {
        dK[key * d + lane + 64] = scale * dk1;
        dV[key * d + lane + 64] = dv1;
    }
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t s) {
    const int64_t rows = a.B * a.H * a.Nq, keys = a.B * a.H * a.Nk;
    const int d = (int)a.d;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL(bwd_f32_pre, dim3((unsigned)((rows + kWaves - 1) / kWaves)),
                       dim3(64 * kWaves), 0, s, (const float *)a.O, (const float *)a.dO, a.L,
                       a.D, a.L2, rows, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_f32_dq, dim3((unsigned)((rows + kWaves - 1) / kWaves)),
                       dim3(64 * kWaves), 0, s, (const float *)a.Q, (const float *)a.K,
                       (const float *)a.V, (const float *)a.dO, a.L2, a.D, (float *)a.dQ, rows,
                       a.Nq, a.Nk, d, a.scale, c, a.causal, a.q_start);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_f32_dkdv, dim3((unsigned)((keys + kWaves - 1) / kWaves)),
                       dim3(64 * kWaves), 0, s, (const float *)a.Q, (const float *)a.K,
                       (const float *)a.V, (const float *)a.dO, a.L2, a.D, (float *)a.dK,
                       (float *)a.dV, keys, a.Nq, a.Nk, d, a.scale, c, a.causal, a.q_start);
    return hipGetLastError();
}

}  // namespace fa
