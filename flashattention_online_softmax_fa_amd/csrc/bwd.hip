// bwd.hip -- attention backward on bf16 matrix cores (gfx950), d in {64, 128}.
//
// Source: flash_backward (attention_kernels.py): D = rowsum(dO * O) first;
// then every key/value tile is independent and walks the query tiles that
// can see it, recomputing P = exp(S - L) from the stored L, and forms
//     dV_j += P^T dO_i,  dP = dO_i V_j^T,  dS = P * (dP - D_i),
//     dK_j += scale dS^T Q_i,  dQ_i += scale dS K_j,
// where the dQ contributions of all key tiles are summed with atomic adds.
//
// Three launches on the caller's stream:
//   bwd_pre_kernel     D = rowsum(dO * O) in fp32 and dQ_acc = 0;
//   bwd_main_kernel    one workgroup per (batch*head, 128-key tile), 4 waves of
//                      32 keys; K and V of the wave stay in registers;
//   dq_convert_kernel  dQ = bf16(dQ_acc).
//
// Layout choices (v_mfma_f32_32x32x16_bf16, C[m][n] with lane = n):
//   S = Q K^T and dP = dO V^T put one KEY per lane (16 queries per lane), so
//   P and dS in registers are directly the B operands of dV^T = dO^T P and
//   dK^T = Q^T dS.  The transposed operands dO^T and Q^T are read from the
//   row-major LDS tiles with ds_read_b64_tr_b16: within each 16-lane group,
//   lane i receives element i%4 of the 8-byte pieces addressed by lanes
//   i/4 + 4t (t = 0..3), so lanes that address a 4-row x 16-column block
//   receive its columns.  dS goes through LDS once, [key][query], for
//   dQ = dS K, whose output has one d column per lane and makes the atomic
//   adds contiguous.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kKW = 32;               // keys per wave
constexpr int kBC = kWaves * kKW;     // keys per workgroup
constexpr int kThreads = kWaves * 64;

// Transposed read of a 4-row x 16-column block of a row-major bf16 LDS tile
// whose top-left element is `base`: lane i of each 16-lane group receives the
// 4 elements of column i.  `s` is the lane's index within its group.
__device__ __forceinline__ u32x2 tr_read(const uint16_t *base, int stride, int s) {
    const uint16_t *p = base + (s >> 2) * stride + 4 * (s & 3);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ bf16x8 join(u32x2 a, u32x2 b) {
    const u32x4 w = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, w);
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) (fp32), and zero the fp32 dQ accumulator.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t *__restrict__ O,
                                                      const uint16_t *__restrict__ dO,
                                                      float *__restrict__ Dv,
                                                      float *__restrict__ dQacc, int64_t rows) {
    constexpr int LPR = D / 8;  // lanes per row (16-byte chunks)
    const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = chunk / LPR;
    const int sub = (int)(chunk % LPR);
    float s = 0.f;
    if (row < rows) {
        const u32x4 o = *(const u32x4 *)(O + row * D + sub * 8);
        const u32x4 g = *(const u32x4 *)(dO + row * D + sub * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            s = fmaf(bf16_lo(o[w]), bf16_lo(g[w]), s);
            s = fmaf(bf16_hi(o[w]), bf16_hi(g[w]), s);
        }
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        *(f32x4 *)(dQacc + row * D + sub * 8) = z;
        *(f32x4 *)(dQacc + row * D + sub * 8 + 4) = z;
    }
    // sum over the LPR lanes of the row (aligned groups of 8 or 16 lanes)
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
    if (row < rows && sub == 0) Dv[row] = s;
}

// ---------------------------------------------------------------------------
// dQ = bf16(dQ_acc), 8 elements per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dq_convert_kernel(const float *__restrict__ acc,
                                                         uint16_t *__restrict__ dQ, int64_t n8) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4 a = *(const f32x4 *)(acc + i * 8);
    const f32x4 b = *(const f32x4 *)(acc + i * 8 + 4);
    const u32x4 w = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                     pack_bf16x2(b[2], b[3])};
    *(u32x4 *)(dQ + i * 8) = w;
}

// ---------------------------------------------------------------------------
// Main backward kernel.
// ---------------------------------------------------------------------------
template <int D>
struct BwdTile {
    static constexpr int QB = D == 64 ? 2 : 1;  // 32-query blocks per query tile
    static constexpr int BR = 32 * QB;          // queries per query tile
    static constexpr int RS = D + 8;            // row stride of Q, dO, K tiles in LDS
    static constexpr int SS = BR + 8;           // row stride of the dS tile
    static constexpr int QCH = BR * D / 8 / kThreads;  // 16-byte chunks per thread per tensor
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void bwd_main_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ L, const float *__restrict__ Dv, float *__restrict__ dQacc,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int64_t Nq, int64_t Nk, int nkt,
    float scale, float c) {
    using T = BwdTile<D>;
    constexpr int QB = T::QB, BR = T::BR, RS = T::RS, SS = T::SS;
    __shared__ __attribute__((aligned(16))) uint16_t sK[kBC * RS];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[BR * RS];
    __shared__ __attribute__((aligned(16))) uint16_t sdO[BR * RS];
    __shared__ __attribute__((aligned(16))) uint16_t sdS[kBC * SS];
    __shared__ __attribute__((aligned(16))) float sL[BR];
    __shared__ __attribute__((aligned(16))) float sD[BR];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 5, lr = lane & 31, s16 = lane & 15, G = lane >> 4;
    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = lid / nkt;
    const int kt = (int)(lid % nkt);  // causal: low key tiles see the most queries; go first
    const int64_t k0 = (int64_t)kt * kBC;
    const int64_t kw0 = k0 + wave * kKW;
    const int64_t mykey = kw0 + lr;
    const uint16_t *Qh = Q + bh * Nq * D;
    const uint16_t *dOh = dO + bh * Nq * D;
    const uint16_t *Kh = K + bh * Nk * D;
    const uint16_t *Vh = V + bh * Nk * D;
    const float *Lh = L + bh * Nq;
    const float *Dh = Dv + bh * Nq;
    float *dQh = dQacc + bh * Nq * D;

    // K and V of this wave's keys as B operands of S = Q K^T and dP = dO V^T.
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (mykey < Nk) {
            a = *(const u32x4 *)(Kh + mykey * D + ds * 16 + g * 8);
            b = *(const u32x4 *)(Vh + mykey * D + ds * 16 + g * 8);
        }
        kf[ds] = __builtin_bit_cast(bf16x8, a);
        vf[ds] = __builtin_bit_cast(bf16x8, b);
    }
    // the workgroup's K tile in LDS, row-major, for dQ = dS K
    for (int cidx = tid; cidx < kBC * D / 8; cidx += kThreads) {
        const int row = cidx / (D / 8), col = cidx % (D / 8);
        const int64_t key = k0 + row;
        const u32x4 w = key < Nk ? *(const u32x4 *)(Kh + key * D + col * 8)
                                 : u32x4{0u, 0u, 0u, 0u};
        *(u32x4 *)(&sK[row * RS + col * 8]) = w;
    }

    f32x16 dvacc[D / 32], dkacc[D / 32];
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dvacc[b][r] = 0.f;
            dkacc[b][r] = 0.f;
        }

    // query tiles that can see this key tile
    const int nqt = (int)((Nq + BR - 1) / BR);
    const int it0 = CAUSAL ? (int)(k0 / BR) : 0;

    u32x4 qreg[T::QCH], oreg[T::QCH];
    float lreg = 0.f, dreg = 0.f;
    auto load_q = [&](int it) {
        const int64_t q0 = (int64_t)it * BR;
#pragma unroll
        for (int u = 0; u < T::QCH; ++u) {
            const int cidx = tid + kThreads * u;
            const int row = cidx / (D / 8), col = cidx % (D / 8);
            const int64_t q = q0 + row;
            qreg[u] = q < Nq ? *(const u32x4 *)(Qh + q * D + col * 8) : u32x4{0u, 0u, 0u, 0u};
            oreg[u] = q < Nq ? *(const u32x4 *)(dOh + q * D + col * 8) : u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < BR) {
            const int64_t q = q0 + tid;
            // a padded query row gets L = +inf, so its P is exactly 0
            lreg = q < Nq ? Lh[q] * kLog2e : INFINITY;
            dreg = q < Nq ? Dh[q] : 0.f;
        }
    };
    auto store_q = [&]() {
#pragma unroll
        for (int u = 0; u < T::QCH; ++u) {
            const int cidx = tid + kThreads * u;
            const int row = cidx / (D / 8), col = cidx % (D / 8);
            *(u32x4 *)(&sQ[row * RS + col * 8]) = qreg[u];
            *(u32x4 *)(&sdO[row * RS + col * 8]) = oreg[u];
        }
        if (tid < BR) {
            sL[tid] = lreg;
            sD[tid] = dreg;
        }
    };

    if (it0 < nqt) {
        load_q(it0);
        store_q();
    }
    __syncthreads();

    // dQ output block of this wave: (query block, 32-column block)
    const int oqb = D == 64 ? (wave >> 1) : 0;
    const int odb = D == 64 ? (wave & 1) : wave;

    for (int it = it0; it < nqt; ++it) {
        const int64_t q0 = (int64_t)it * BR;
        if (it + 1 < nqt) load_q(it + 1);
        const bool active = mykey - lr < Nk && (!CAUSAL || q0 + BR - 1 >= kw0);
        if (active) {
            // ---- S = Q K^T and dP = dO V^T (lane: key lr; register r: query
            //      8*(r/4) + 4g + r%4 of the 32-query block)
            f32x16 sacc[QB], pacc[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[qb][r] = 0.f;
                    pacc[qb][r] = 0.f;
                }
#pragma unroll
                for (int ds = 0; ds < D / 16; ++ds) {
                    const int off = (qb * 32 + lr) * RS + ds * 16 + g * 8;
                    const bf16x8 aq = *(const bf16x8 *)(&sQ[off]);
                    const bf16x8 ao = *(const bf16x8 *)(&sdO[off]);
                    sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[ds], sacc[qb], 0, 0,
                                                                       0);
                    pacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[ds], pacc[qb], 0, 0,
                                                                       0);
                }
            }
            // ---- P = exp2(S c - L log2 e), dS = P (dP - D)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int qi = qb * 32 + 8 * r4 + 4 * g;
                    const f32x4 lv = *(const f32x4 *)(&sL[qi]);
                    const f32x4 dv = *(const f32x4 *)(&sD[qi]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        float p = fast_exp2(fmaf(sacc[qb][r], c, -lv[e]));
                        if (mykey >= Nk || (CAUSAL && mykey > q0 + qi + e)) p = 0.f;
                        sacc[qb][r] = p;
                        pacc[qb][r] = p * (pacc[qb][r] - dv[e]);
                    }
                }
            }
            // ---- bf16 B operands: k-step kq (16 queries) = registers 8h..8h+7 of block kq/2
            bf16x8 pb[BR / 16], sb[BR / 16];
#pragma unroll
            for (int kq = 0; kq < BR / 16; ++kq) {
                const int qb = kq >> 1, h = kq & 1;
                const u32x4 wp = {pack_bf16x2(sacc[qb][8 * h + 0], sacc[qb][8 * h + 1]),
                                  pack_bf16x2(sacc[qb][8 * h + 2], sacc[qb][8 * h + 3]),
                                  pack_bf16x2(sacc[qb][8 * h + 4], sacc[qb][8 * h + 5]),
                                  pack_bf16x2(sacc[qb][8 * h + 6], sacc[qb][8 * h + 7])};
                const u32x4 ws = {pack_bf16x2(pacc[qb][8 * h + 0], pacc[qb][8 * h + 1]),
                                  pack_bf16x2(pacc[qb][8 * h + 2], pacc[qb][8 * h + 3]),
                                  pack_bf16x2(pacc[qb][8 * h + 4], pacc[qb][8 * h + 5]),
                                  pack_bf16x2(pacc[qb][8 * h + 6], pacc[qb][8 * h + 7])};
                pb[kq] = __builtin_bit_cast(bf16x8, wp);
                sb[kq] = __builtin_bit_cast(bf16x8, ws);
                // dS to LDS as [key][query] for dQ = dS K
                const int kr = wave * kKW + lr;
                *(u32x2 *)(&sdS[kr * SS + kq * 16 + 4 * g]) = u32x2{ws[0], ws[1]};
                *(u32x2 *)(&sdS[kr * SS + kq * 16 + 8 + 4 * g]) = u32x2{ws[2], ws[3]};
            }
            // ---- dV^T += dO^T P and dK^T += Q^T dS.  A operand: lane holds column
            //      d = 32b + lane%32 at the 8 queries of its k-slots; slot (g, e) is
            //      query 8*(e/4) + 4g + e%4 of the step, matching P's registers.
#pragma unroll
            for (int b = 0; b < D / 32; ++b) {
                const int col = b * 32 + 16 * (G & 1);
#pragma unroll
                for (int kq = 0; kq < BR / 16; ++kq) {
                    const int r0 = kq * 16 + 4 * g;
                    const bf16x8 ao = join(tr_read(&sdO[r0 * RS + col], RS, s16),
                                           tr_read(&sdO[(r0 + 8) * RS + col], RS, s16));
                    const bf16x8 aq = join(tr_read(&sQ[r0 * RS + col], RS, s16),
                                           tr_read(&sQ[(r0 + 8) * RS + col], RS, s16));
                    dvacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb[kq], dvacc[b], 0, 0,
                                                                       0);
                    dkacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[kq], dkacc[b], 0, 0,
                                                                       0);
                }
            }
        } else {
            // keys of an idle wave add nothing to dQ
            const int kr = wave * kKW + lr;
#pragma unroll
            for (int kq = 0; kq < BR / 16; ++kq) {
                *(u32x2 *)(&sdS[kr * SS + kq * 16 + 4 * g]) = u32x2{0u, 0u};
                *(u32x2 *)(&sdS[kr * SS + kq * 16 + 8 + 4 * g]) = u32x2{0u, 0u};
            }
        }
        __syncthreads();  // dS complete; Q/dO tile no longer read
        if (it + 1 < nqt) store_q();
        // ---- dQ (32 queries x 32 columns per wave) += scale * dS K over the 128 keys.
        //      k-slot (g, e) is key 16*ks + 8g + e in both operands.
        {
            f32x16 qacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) qacc[r] = 0.f;
            const int qcol = oqb * 32 + 16 * (G & 1);
            const int dcol = odb * 32 + 16 * (G & 1);
#pragma unroll
            for (int ks = 0; ks < kBC / 16; ++ks) {
                const int r0 = ks * 16 + 8 * g;
                const bf16x8 a = join(tr_read(&sdS[r0 * SS + qcol], SS, s16),
                                      tr_read(&sdS[(r0 + 4) * SS + qcol], SS, s16));
                const bf16x8 b = join(tr_read(&sK[r0 * RS + dcol], RS, s16),
                                      tr_read(&sK[(r0 + 4) * RS + dcol], RS, s16));
                qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, qacc, 0, 0, 0);
            }
            // lane: column odb*32 + lr; register r: query 8*(r/4) + 4g + r%4 of block oqb
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t q = q0 + oqb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (q < Nq) atomicAdd(dQh + q * D + odb * 32 + lr, scale * qacc[r]);
            }
        }
        __syncthreads();  // next Q/dO tile visible; dS reads done
    }

    // ---- epilogue: dK = scale * dK_acc, dV = dV_acc (lane: key lr; register r:
    //      column 32b + 8*(r/4) + 4g + r%4)
    if (mykey < Nk) {
        uint16_t *dKr = dK + (bh * Nk + mykey) * D;
        uint16_t *dVr = dV + (bh * Nk + mykey) * D;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int col = b * 32 + 8 * t + 4 * g;
                const u32x2 wk = {pack_bf16x2(scale * dkacc[b][4 * t], scale * dkacc[b][4 * t + 1]),
                                  pack_bf16x2(scale * dkacc[b][4 * t + 2],
                                              scale * dkacc[b][4 * t + 3])};
                const u32x2 wv = {pack_bf16x2(dvacc[b][4 * t], dvacc[b][4 * t + 1]),
                                  pack_bf16x2(dvacc[b][4 * t + 2], dvacc[b][4 * t + 3])};
                *(u32x2 *)(dKr + col) = wk;
                *(u32x2 *)(dVr + col) = wv;
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_main(const BwdArgs &a, hipStream_t s) {
    const int nkt = (int)((a.Nk + kBC - 1) / kBC);
    const dim3 grid((unsigned)(a.B * a.H * nkt));
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, s,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (const uint16_t *)a.dO, a.L, a.D, a.dQacc, (uint16_t *)a.dK,
                       (uint16_t *)a.dV, a.Nq, a.Nk, nkt, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s) {
    const int64_t rows = a.B * a.H * a.Nq;
    const int64_t chunks = rows * (a.d / 8);
    const dim3 pre_grid((unsigned)((chunks + 255) / 256));
    if (a.d == 128)
        hipLaunchKernelGGL(bwd_pre_kernel<128>, pre_grid, dim3(256), 0, s, (const uint16_t *)a.O,
                           (const uint16_t *)a.dO, a.D, a.dQacc, rows);
    else
        hipLaunchKernelGGL(bwd_pre_kernel<64>, pre_grid, dim3(256), 0, s, (const uint16_t *)a.O,
                           (const uint16_t *)a.dO, a.D, a.dQacc, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.d == 128)
        e = a.causal ? launch_main<128, true>(a, s) : launch_main<128, false>(a, s);
    else
        e = a.causal ? launch_main<64, true>(a, s) : launch_main<64, false>(a, s);
    if (e != hipSuccess) return e;
    const int64_t n8 = rows * a.d / 8;
    hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       a.dQacc, (uint16_t *)a.dQ, n8);
    return hipGetLastError();
}

}  // namespace fa
