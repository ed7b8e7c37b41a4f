// fwd_bf16.hip -- attention forward on bf16 matrix cores (gfx950), d in {64, 128}.
//
// Source: flash_forward (attention_kernels.py): every query tile is
// independent; it keeps a running row maximum m, denominator l and an
// unnormalised accumulator on chip while it walks the key/value tiles,
// rescales them by exp(m_old - m_new) when the maximum grows, skips key
// tiles that lie entirely after its last query under the causal mask,
// divides once at the end and writes L = m + log l.
//
// Work split.  One workgroup (4 waves) per (batch*head, 128-query tile); each
// wave owns 32 queries.  Key/value tiles of 64 keys are staged in LDS, double
// buffered, one barrier per tile; the next tile's HBM loads are issued before
// the current tile is computed and written to LDS after it.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16).  The wave computes the
// transposed score block S^T = K Q^T, so each lane's 16 accumulator values
// belong to ONE query (lane % 32) and 16 keys; the row maximum and sum are
// per-lane work plus one exchange with lane ^ 32.  Those same registers,
// rounded to bf16, are directly the B operand of O^T += V^T P^T; V^T comes from
// LDS, where V is stored transposed (and key-permuted to match the order in
// which P sits in the registers) when the tile is staged.  Q stays in
// registers as the B operand of every score product.
//
// Softmax statistics are kept in base 2: scores are multiplied by
// scale*log2(e) inside the exponent's FMA, and L is converted back to the
// natural logarithm at the end.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kQW = 32;                // queries per wave
constexpr int kBR = kWaves * kQW;      // queries per workgroup
constexpr int kBC = 64;                // keys per tile
constexpr int kThreads = kWaves * 64;

template <int D>
struct Tile {
    static constexpr int KS = D + 8;   // K row stride in LDS (elements); 16-byte rows, bank shift 4
    static constexpr int VS = kBC + 8; // V^T row stride (elements)
    static constexpr int KCH = kBC * D / 8 / kThreads;       // 16-byte K chunks per thread
    static constexpr int VTASKS = (kBC / 4) * (D / 8);        // 4-key x 8-column V blocks
};

// Position of key k (k % 4 == 0, 0 <= k < kBC) in a V^T row: within each group
// of 16 keys, keys 0-3, 8-11 come first and 4-7, 12-15 second -- the order in
// which lane halves 0 and 1 hold P in the S^T accumulator.  16-byte chunks
// are XOR-swizzled by row to spread the transposing stores over LDS banks.
__device__ __forceinline__ int vt_offset(int row, int k, int VS) {
    const int kk = k & 15;
    const int p = (k & ~15) + ((kk >> 2) & 1) * 8 + (kk >> 3) * 4;
    const int chunk = (p >> 3) ^ ((row >> 3) & 7);
    return row * VS + chunk * 8 + (p & 7);
}

template <int D, bool CAUSAL, bool POS_SCALE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ L, int64_t Nq,
    int64_t Nk, int nqt, float c) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBC * T::KS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * T::VS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 5, lr = lane & 31;
    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t bh = lid / nqt;
    int qt = (int)(lid % nqt);
    if (CAUSAL) qt = nqt - 1 - qt;  // heaviest query tiles first
    const int64_t q0 = (int64_t)qt * kBR;
    const int64_t qw0 = q0 + wave * kQW;
    const int64_t qrow = qw0 + lr;
    const uint16_t *Qh = Q + bh * Nq * D;
    const uint16_t *Kh = K + bh * Nk * D;
    const uint16_t *Vh = V + bh * Nk * D;

    int64_t nkt = (Nk + kBC - 1) / kBC;
    if (CAUSAL) {
        const int64_t qlast = (q0 + kBR < Nq ? q0 + kBR : Nq) - 1;
        const int64_t lim = qlast / kBC + 1;
        nkt = nkt < lim ? nkt : lim;
    }
    const int64_t qw_last = (qw0 + kQW - 1 < Nq - 1) ? qw0 + kQW - 1 : Nq - 1;

    // Q fragments: B operand of S^T = K Q^T (lane: query lr, 8 columns per 16-step)
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qrow < Nq) w = *(const u32x4 *)(Qh + qrow * D + ds * 16 + g * 8);
        qf[ds] = __builtin_bit_cast(bf16x8, w);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
    float m = -INFINITY, l = 0.f;

    u32x4 kreg[T::KCH];
    u32x4 vreg[4];
    const int vdoct = tid % (D / 8), vquad = tid / (D / 8);

    auto load_tile = [&](int64_t j) {
        const int64_t kv0 = j * kBC;
#pragma unroll
        for (int u = 0; u < T::KCH; ++u) {
            const int cidx = tid + kThreads * u;
            const int row = cidx / (D / 8), col = cidx % (D / 8);
            const int64_t key = kv0 + row;
            kreg[u] = key < Nk ? *(const u32x4 *)(Kh + key * D + col * 8) : u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < T::VTASKS) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t key = kv0 + 4 * vquad + u;
                vreg[u] = key < Nk ? *(const u32x4 *)(Vh + key * D + vdoct * 8)
                                   : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < T::KCH; ++u) {
            const int cidx = tid + kThreads * u;
            const int row = cidx / (D / 8), col = cidx % (D / 8);
            *(u32x4 *)(&sK[buf][row * T::KS + col * 8]) = kreg[u];
        }
        if (tid < T::VTASKS) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // column 2w: low halves of the four key rows; column 2w+1: high halves
                const u32x2 lo = {(vreg[0][w] & 0xffffu) | (vreg[1][w] << 16),
                                  (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16)};
                const u32x2 hi = {(vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u),
                                  (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u)};
                const int r0 = vdoct * 8 + 2 * w;
                *(u32x2 *)(&sV[buf][vt_offset(r0, 4 * vquad, T::VS)]) = lo;
                *(u32x2 *)(&sV[buf][vt_offset(r0 + 1, 4 * vquad, T::VS)]) = hi;
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int64_t j = 0; j < nkt; ++j) {
        const int buf = (int)(j & 1);
        if (j + 1 < nkt) load_tile(j + 1);
        const int64_t kv0 = j * kBC;
        const bool active = qw0 < Nq && (!CAUSAL || kv0 <= qw_last);
        if (active) {
            // ---- S^T = K_j Q^T
            f32x16 sacc[kBC / 32];
#pragma unroll
            for (int kb = 0; kb < kBC / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
                for (int ds = 0; ds < D / 16; ++ds) {
                    const bf16x8 a = *(const bf16x8 *)(&sK[buf][(kb * 32 + lr) * T::KS +
                                                               ds * 16 + g * 8]);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sacc[kb], 0, 0,
                                                                       0);
                }
            }
            if (!POS_SCALE) {
#pragma unroll
                for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[kb][r] *= c;
            }
            // ---- mask: keys past Nk, and keys after the query under causal
            const bool need_mask = (kv0 + kBC > Nk) || (CAUSAL && kv0 + kBC - 1 > qw0);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                        if (key >= Nk || (CAUSAL && key > qrow)) sacc[kb][r] = -INFINITY;
                    }
            }
            // ---- online softmax (base 2)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m, POS_SCALE ? mx * c : mx);
            const float mref = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m - mref);
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < kBC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(POS_SCALE ? fmaf(sacc[kb][r], c, -mref)
                                                        : sacc[kb][r] - mref);
                    sacc[kb][r] = p;
                    lsum += p;
                }
            l = l * alpha + lsum;  // per-lane partial: this lane's 32 of the tile's 64 keys
            if (__any(m_new != m)) {
#pragma unroll
                for (int b = 0; b < D / 32; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
            }
            m = m_new;
            // ---- P^T as bf16 B operands: k-step ks uses registers 8h..8h+7 of block ks/2
            bf16x8 pf[kBC / 16];
#pragma unroll
            for (int ks = 0; ks < kBC / 16; ++ks) {
                const int kb = ks >> 1, h = ks & 1;
                const u32x4 w = {pack_bf16x2(sacc[kb][8 * h + 0], sacc[kb][8 * h + 1]),
                                 pack_bf16x2(sacc[kb][8 * h + 2], sacc[kb][8 * h + 3]),
                                 pack_bf16x2(sacc[kb][8 * h + 4], sacc[kb][8 * h + 5]),
                                 pack_bf16x2(sacc[kb][8 * h + 6], sacc[kb][8 * h + 7])};
                pf[ks] = __builtin_bit_cast(bf16x8, w);
            }
            // ---- O^T += V_j^T P^T
#pragma unroll
            for (int b = 0; b < D / 32; ++b) {
                const int row = b * 32 + lr;
#pragma unroll
                for (int ks = 0; ks < kBC / 16; ++ks) {
                    const int chunk = (ks * 2 + g) ^ ((row >> 3) & 7);
                    const bf16x8 a = *(const bf16x8 *)(&sV[buf][row * T::VS + chunk * 8]);
                    oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], oacc[b], 0, 0, 0);
                }
            }
        }
        if (j + 1 < nkt) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: one division, natural-log L
    const float l_tot = l + __shfl_xor(l, 32);
    if (qrow < Nq) {
        const float inv = 1.f / l_tot;
        uint16_t *orow = O + (bh * Nq + qrow) * D;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x2 w = {pack_bf16x2(oacc[b][4 * t] * inv, oacc[b][4 * t + 1] * inv),
                                 pack_bf16x2(oacc[b][4 * t + 2] * inv, oacc[b][4 * t + 3] * inv)};
                *(u32x2 *)(orow + b * 32 + 8 * t + 4 * g) = w;
            }
        if (g == 0) L[bh * Nq + qrow] = (m + log2f(l_tot)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_d(const FwdArgs &a, hipStream_t s) {
    const int nqt = (int)((a.Nq + kBR - 1) / kBR);
    const dim3 grid((unsigned)(a.B * a.H * nqt));
    const float c = a.scale * kLog2e;
    if (a.scale > 0.f)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, true>), grid, dim3(kThreads), 0, s,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (uint16_t *)a.O, a.L, a.Nq, a.Nk, nqt, c);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false>), grid, dim3(kThreads), 0, s,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (uint16_t *)a.O, a.L, a.Nq, a.Nk, nqt, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
    if (a.d == 128) return a.causal ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
    return a.causal ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace fa
