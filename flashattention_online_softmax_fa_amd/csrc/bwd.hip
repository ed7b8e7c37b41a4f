// bwd.hip -- attention backward on bf16 matrix cores (gfx950), d in {64, 128}.
//
// Source: flash_backward (attention_kernels.py): D = rowsum(dO * O) first;
// then P = exp(S - L) is recomputed tile by tile from the stored L, and
//     dV_j += P^T dO_i,  dP = dO_i V_j^T,  dS = P * (dP - D_i),
//     dK_j += scale dS^T Q_i,  dQ_i += scale dS K_j.
// The page sums dQ across key tiles with atomic adds.  Here the atomics are
// replaced by a second, query-major pass that recomputes S and dP for its
// own query tile and accumulates dQ in registers: on this chip fp32 atomics
// from many workgroups travel to the memory fabric (about 0.55 GB of atomic
// traffic per call at 2 x 16 heads x 4096 tokens), which costs more than
// recomputing two of the five products.  The result is also deterministic.
//
// Two launches on the caller's stream:
//   bwd_dq_kernel    one workgroup per (batch*head, 32*W-query tile), W waves
//                    of 32 queries, Q and dO in registers; K and V tiles of the key
//                    tiles its queries can see stream through an LDS ring.  It
//                    also forms D = rowsum(dO * O) and L2 = L * log2(e) of its
//                    queries and writes -D and L2 to the workspace;
//   bwd_dkdv_kernel  one workgroup per (batch*head, key tile), W waves of 32
//                    keys, K and V in registers; Q, dO, L2 and -D tiles of the
//                    query tiles that can see its keys stream through an LDS ring
//                    (by default bwd_dkdv_pipe_kernel, the same work software-
//                    pipelined over 32-query tiles: eight waves at d = 64, four
//                    at d = 128).
// Both passes start the dP accumulators from -D, so that the products leave
// dP - D and dS = P (dP - D) takes one multiply.
// Both rings are filled with global_load_lds_dwordx4 into row-major,
// chunk-swizzled tiles (see fa_device.h); a ring of 2*GR slots takes one
// barrier per GR tiles (GR tiles computed on while the next GR are in flight).
// With eight waves the two waves of a SIMD take turns issuing both their
// shares of the loads (FA_BWD_DMA_ALT), as in the forward.
//
// Layouts (v_mfma_f32_32x32x16_bf16, C[m][n] with lane = n):
//   dkdv: S = Q K^T and dP = dO V^T put one KEY per lane, so P and dS are
//         directly the B operands of dV^T = dO^T P and dK^T = Q^T dS, with dO^T
//         and Q^T read transposed from the row-major tiles.
//   dq:   S^T = K Q^T and dP^T = V dO^T put one QUERY per lane, so dS^T is
//         directly the B operand of dQ^T = K^T dS^T (K^T read transposed), and
//         L2, D are per-lane scalars.
#include "fa_device.h"
#include "fa_internal.h"

#include <type_traits>

// 1: at each barrier of a pass with eight waves, only one wave of each SIMD's
// pair (waves w and w ^ 4) issues the next group's ring loads, for both,
// alternating between the two from one barrier to the next: its partner
// computes meanwhile instead of queueing for the loads.
#ifndef FA_BWD_DMA_ALT
#define FA_BWD_DMA_ALT 1
#endif
// Instruction-interleaving strategy the compiler applies to a pipelined
// dK/dV step and to a dQ tile (__builtin_amdgcn_iglp_opt), -1 for none:
// 0 and 2 measured 0.6 % and 0.3 % faster per backward than none
#ifndef FA_BWD_IGLP
#define FA_BWD_IGLP 0
#endif
#ifndef FA_BWD_DQ_IGLP
#define FA_BWD_DQ_IGLP 2
#endif
// with FA_BWD_DMA_ALT: wave priority of the loading wave until the next
// barrier (s_setprio), so that it catches up with its partner (1.5 %)
#ifndef FA_BWD_PRIO
#define FA_BWD_PRIO 1
#endif

namespace fa {
namespace {


#if FA_STATS
__device__ unsigned long long g_bwd_stats[kStatCount];
#endif

// Eight fp32 accumulator registers r0..r0+7 -> bf16x8 (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const f32x16 &v, int r0) {
    const u32x4 w = {pack_bf16x2(v[r0 + 0], v[r0 + 1]), pack_bf16x2(v[r0 + 2], v[r0 + 3]),
                     pack_bf16x2(v[r0 + 4], v[r0 + 5]), pack_bf16x2(v[r0 + 6], v[r0 + 7])};
    return __builtin_bit_cast(bf16x8, w);
}

// Two transposed reads (rows 4g.. and 8 + 4g.. of a 16-row step) -> bf16x8.
// `off` is tr_off<ROWB>(lane, b, 0); the rows 8 further down start at
// (off ^ 32) + 8 * ROWB, since both swizzles satisfy swz(r + 8) = swz(r) ^ 2.
template <int ROWB>
__device__ __forceinline__ bf16x8 tr_pair(const uint8_t *base, int off) {
    const u32x2 lo = tr_read(base + off), hi = tr_read(base + ((off ^ 32) + 8 * ROWB));
    const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, w);
}

// 16-byte row chunk `col8` of row `row` (< rows), or zeros past the end; the
// address is clamped so the load itself is always in bounds.
__device__ __forceinline__ u32x4 load_row16(const uint16_t *base, int64_t row, int64_t rows,
                                            int D, int col8) {
    const int64_t r = row < rows ? row : rows - 1;
    const u32x4 w = *(const u32x4 *)(base + r * D + col8 * 8);
    return row < rows ? w : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// dK, dV: key-major.
// ---------------------------------------------------------------------------
template <int D, int BR_, int GR_, int KB_, int W_>
struct DkdvCfg {
    static constexpr int W = W_;                   // waves per workgroup
    static constexpr int BR = BR_;                 // queries per tile
    static constexpr int QB = BR / 32;             // 32-query blocks per tile
    static constexpr int KB = KB_;                 // 32-key blocks per wave
    static constexpr int KEYS = 32 * KB * W;       // keys per workgroup
    static constexpr int CH = D / 8, ROWB = D * 2;
    static constexpr int TILEB = BR * ROWB;        // one Q or dO tile
    static constexpr int VECB = 256;               // one L2 or D slice (64 lanes x 4 B)
    static constexpr int STAGEB = 2 * TILEB + 2 * VECB;
    static constexpr int GR = GR_;                 // query tiles per LDS barrier
    static constexpr int ST = 2 * GR;              // ring slots: GR in use, GR in flight
    static constexpr int IPW = TILEB / 1024 / W;
    static constexpr int RPI = 1024 / ROWB;
    static_assert(IPW >= 1 && IPW * W * 1024 == TILEB && BR <= 64, "dkdv tile");
    static_assert(W == 4 || W == 8, "4 or 8 waves");
};

template <int D, int BR, int GR, int KB, int W, bool CAUSAL>
__global__ __launch_bounds__(W * 64)
__attribute__((amdgpu_waves_per_eu(D == 64 && KB == 1 ? 2 : 1, KB == 1 ? 2 : 1)))
void bwd_dkdv_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
                     const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
                     const float *__restrict__ L2, const float *__restrict__ Dv,
                     uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int64_t Nq, int64_t Nk,
                     int64_t qoff, int nkt, uint32_t group, float scale, float c) {
    using T = DkdvCfg<D, BR, GR, KB, W>;
    constexpr int ST = T::ST;
    constexpr int QB = T::QB, ROWB = T::ROWB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * T::STAGEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 5, lr = lane & 31;
    const TileId tid_ = tile_order(blockIdx.x, gridDim.x / (uint32_t)nkt, (uint32_t)nkt, group);
    const int64_t bh = tid_.head;
    const int kt = (int)tid_.rank;  // causal: early keys are seen by the most queries
    const int64_t k0 = (int64_t)kt * T::KEYS;
    const int64_t kw0 = k0 + wave * 32 * KB;  // key block kb of this wave: kw0 + 32kb + lane%32
    constexpr int KW = 32 * KB;                // keys per wave
    const uint16_t *Qh = Q + bh * Nq * D;
    const uint16_t *dOh = dO + bh * Nq * D;
    const float *L2h = L2 + bh * Nq;
    const float *Dh = Dv + bh * Nq;

    // K and V of this wave's keys: B operands of S = Q K^T and dP = dO V^T
    bf16x8 kf[KB][D / 16], vf[KB][D / 16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const int64_t key = kw0 + 32 * kb + lr;
            kf[kb][ds] = __builtin_bit_cast(bf16x8, load_row16(K + bh * Nk * D, key, Nk, D, ds * 2 + g));
            vf[kb][ds] = __builtin_bit_cast(bf16x8, load_row16(V + bh * Nk * D, key, Nk, D, ds * 2 + g));
        }

    // ring loads: this lane fills chunk `lane` of its IPW 1 KiB blocks of the
    // Q and dO tiles (row (wave*IPW + u)*RPI + lane/CH of the tile, logical
    // chunk (lane % CH) ^ swz(row)); waves 0 and 1 also fill the L2 and D slices
    //      (with FA_BWD_DMA_ALT, also those of the partner wave w ^ 4)
    constexpr bool ALT = FA_BWD_DMA_ALT && W == 8 && GR > 1;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t owner_u[2] = {wave_u, wave_u ^ 4u};
    auto ld_row = [&](int o, int u) { return ((int)owner_u[o] * T::IPW + u) * T::RPI + lane / T::CH; };
    uint32_t ld_off[2][T::IPW];  // byte offset of this lane's load within a tile
#pragma unroll
    for (int o = 0; o < (ALT ? 2 : 1); ++o)
#pragma unroll
        for (int u = 0; u < T::IPW; ++u)
            ld_off[o][u] = (uint32_t)chunk_off<ROWB>(ld_row(o, u), lane % T::CH);
    // the loads of wave owner_u[o] for query tile it into stage st; LDS
    // destinations as scalar byte addresses: that wave's first block in the
    // stage, and its L2 / D slice (waves 0 and 1)
    auto issue_as = [&](int it, int st, int o) {
        const uint32_t ow = owner_u[o];
        const int64_t q0 = (int64_t)it * BR;
        const uint32_t qb = lds_addr(smem) + ow * (T::IPW * 1024) + st * T::STAGEB;
        const uint32_t ob = qb + T::TILEB;
        const uint32_t vb = lds_addr(smem) + 2 * T::TILEB + ow * T::VECB + st * T::STAGEB;
        if (q0 + 64 <= Nq) {  // every row and vector lane below in range: scalar bases
            const uint8_t *qs = (const uint8_t *)(Qh + q0 * D);
            const uint8_t *os = (const uint8_t *)(dOh + q0 * D);
#pragma unroll
            for (int u = 0; u < T::IPW; ++u) {
                dma16_s(qs, ld_off[o][u], qb + u * 1024);
                dma16_s(os, ld_off[o][u], ob + u * 1024);
            }
            if (ow < 2) dma4((ow == 0 ? L2h : Dh) + q0 + lane, vb);
            return;
        }
#pragma unroll
        for (int u = 0; u < T::IPW; ++u) {
            const int row = ld_row(o, u);
            const int64_t q = q0 + row < Nq ? q0 + row : Nq - 1;  // past the end: masked later
            const uint8_t *src = (const uint8_t *)(Qh + q * D) + (ld_off[o][u] - row * ROWB);
            const uint8_t *srco = (const uint8_t *)(dOh + q * D) + (ld_off[o][u] - row * ROWB);
            dma16(src, qb + u * 1024);
            dma16(srco, ob + u * 1024);
        }
        if (ow < 2) {
            int64_t q = q0 + lane;
            q = q < Nq ? q : Nq - 1;
            dma4((ow == 0 ? L2h : Dh) + q, vb);
        }
    };
    auto issue = [&](int it, int st) { issue_as(it, st, 0); };

    int roff[D / 16], toff[D / 32];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) roff[ds] = chunk_off<ROWB>(lr, 2 * ds + g);
#pragma unroll
    for (int b = 0; b < D / 32; ++b) toff[b] = tr_off<ROWB>(lane, b, 0);

    f32x16 dvacc[KB][D / 32], dkacc[KB][D / 32];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dvacc[kb][b][r] = 0.f;
                dkacc[kb][b][r] = 0.f;
            }

    // One query tile against this wave's keys; MASKED instances handle the
    // causal diagonal and the ragged ends, the rest carry no mask code.
    auto tile = [&](const uint8_t *qt, int64_t q0, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const uint8_t *ot = qt + T::TILEB;
        const float *lt = (const float *)(ot + T::TILEB);
        const float *dt = lt + T::VECB / 4;

        // ---- S = Q K^T and dP = dO V^T (lane: key lr of block kb; register r:
        //      query 8*(r/4) + 4g + r%4 of the 32-query block); each Q and dO
        //      fragment read from LDS serves the KB key blocks
        f32x16 sacc[QB][KB], pacc[QB][KB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.f;
            // dP starts from -D of its queries, so that the products leave
            // dP - D (register r: query 8*(r/4) + 4g + r%4 of the block)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 nd = *(const f32x4 *)(dt + qb * 32 + 8 * r4 + 4 * g);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) pacc[qb][kb][4 * r4 + e] = nd[e];
            }
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds) {
                const int off = qb * 32 * ROWB + roff[ds];
                const bf16x8 aq = *(const bf16x8 *)(qt + off);
                const bf16x8 ao = *(const bf16x8 *)(ot + off);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kb][ds], sacc[qb][kb], 0, 0, 0);
                    pacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[kb][ds], pacc[qb][kb], 0, 0, 0);
                }
            }
        }
        // ---- P = exp2(S c - L2), dS = P (dP - D); masked tiles zero the pairs
        //      past Nq, past Nk, and (causal) where the key comes after the query:
        //      query offset o in the tile is visible to key block kb iff
        //      lo[kb] <= o <= hi[kb]
        int lo[KB], hi[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            lo[kb] = 0;
            hi[kb] = BR - 1;
            if (MASKED) {
                const int64_t key = kw0 + 32 * kb + lr;
                int64_t lo64 = CAUSAL ? key - qoff - q0 : 0;
                int64_t hi64 = Nq - 1 - q0;
                if (key >= Nk) hi64 = -1;
                lo[kb] = (int)(lo64 < 0 ? 0 : (lo64 > BR ? BR : lo64));
                hi[kb] = (int)(hi64 > BR - 1 ? BR - 1 : (hi64 < -1 ? -1 : hi64));
            }
        }
        auto probs = [&](int qb) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int qi = qb * 32 + 8 * r4 + 4 * g;
                const f32x4 lv = *(const f32x4 *)(lt + qi);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        float p = fast_exp2(fmaf(sacc[qb][kb][r], c, -lv[e]));
                        if (MASKED && (qi + e < lo[kb] || qi + e > hi[kb])) p = 0.f;
                        sacc[qb][kb][r] = p;
                        pacc[qb][kb][r] = p * pacc[qb][kb][r];
                    }
            }
        };
        // ---- dV^T += dO^T P and dK^T += Q^T dS.  B operand (k-step kq of 16
        //      queries) = registers 8h..8h+7 of block kq/2, so k-slot (g, e) is
        //      query 8*(e/4) + 4g + e%4 of the step; the transposed A operand is
        //      read in the same slot order and serves the KB key blocks.  Each
        //      query block's P and dS are formed right before its two k-steps,
        //      so that its products overlap the next block's vector work (3.5 %
        //      faster at d = 128 than forming all of them first; equal at 64).
#pragma unroll
        for (int kq = 0; kq < BR / 16; ++kq) {
            if (kq % 2 == 0) probs(kq / 2);
            bf16x8 pb[KB], sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                pb[kb] = pack8(sacc[kq >> 1][kb], 8 * (kq & 1));
                sb[kb] = pack8(pacc[kq >> 1][kb], 8 * (kq & 1));
            }
#pragma unroll
            for (int b = 0; b < D / 32; ++b) {
                const int off = kq * 16 * ROWB;
                const bf16x8 ao = tr_pair<ROWB>(ot + off, toff[b]);
                const bf16x8 aq = tr_pair<ROWB>(qt + off, toff[b]);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    dvacc[kb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb[kb], dvacc[kb][b], 0, 0, 0);
                    dkacc[kb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[kb], dkacc[kb][b], 0, 0, 0);
                }
            }
        }
    };

#if FA_STATS
    uint32_t st_tiles = 0;
#endif
    // query tiles that can see this key tile (causal: query q sees keys
    // 0 .. q + qoff)
    const int nqt = (int)((Nq + BR - 1) / BR);
    const int it0 = CAUSAL ? (int)(k0 - qoff > 0 ? (k0 - qoff) / BR : 0) : 0;
#pragma unroll
    for (int t = 0; t < GR; ++t)
        if (it0 + t < nqt) issue(it0 + t, t);

    for (int it = it0; it < nqt; ++it) {
        const int idx = it - it0;
        // one barrier per GR query tiles: tiles idx .. idx+GR-1 (issued at the
        // previous barrier, the only loads in flight) have landed and become
        // visible, the slots of tiles idx-GR .. idx-1 are free, and tiles
        // idx+GR .. idx+2GR-1 are issued into them
        if (idx % GR == 0) {
            wait_vm<0>();
            lds_barrier();
            if (!ALT || ((idx / GR) & 1) == (int)(wave_u >> 2)) {
#pragma unroll
                for (int t = GR; t < 2 * GR; ++t)
                    if (it + t < nqt) {
                        issue_as(it + t, (idx + t) % ST, 0);
                        if (ALT) issue_as(it + t, (idx + t) % ST, 1);
                    }
            }
        }
        const int64_t q0 = (int64_t)it * BR;
        const int64_t q_last = (q0 + BR < Nq ? q0 + BR : Nq) - 1;  // last real query of the tile
        const bool active = kw0 < Nk && (!CAUSAL || q_last + qoff >= kw0);
        if (!active) continue;
#if FA_STATS
        ++st_tiles;
#endif
        const uint8_t *qt = smem + (idx % ST) * T::STAGEB;
        // the mask is needed on the causal diagonal and at the ragged ends only
        const bool need_mask =
            (q0 + BR > Nq) || (kw0 + KW > Nk) || (CAUSAL && q0 + qoff < kw0 + KW - 1);
        if (need_mask)
            tile(qt, q0, std::true_type{});
        else
            tile(qt, q0, std::false_type{});
    }

#if FA_STATS
    if (lane == 0 && kw0 < Nk) atomicAdd(&g_bwd_stats[3], (unsigned long long)st_tiles);
#endif
    // ---- epilogue: dK = scale * dK_acc, dV = dV_acc, each 32-key block
    //      through 4 KiB of LDS per tensor (store_rows_staged); every wave is
    //      past its last ring read at the barrier, so the ring holds the stages
    static_assert(ST * T::STAGEB >= W * 8192, "the ring holds the output stages");
    wait_vm<0>();
    lds_barrier();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        store_rows_staged<D>(smem + wave * 8192, dkacc[kb], scale, dK + bh * Nk * D, kw0 + 32 * kb, Nk, lane);
        store_rows_staged<D>(smem + wave * 8192 + 4096, dvacc[kb], 1.f, dV + bh * Nk * D, kw0 + 32 * kb, Nk,
                             lane);
    }
}

// ---------------------------------------------------------------------------
// dK, dV: key-major and software-pipelined over 32-query tiles (d = 64).
// ---------------------------------------------------------------------------
// Each wave owns 32 keys (K and V in registers) and walks the query tiles that
// see them; step t forms S and dP of tile t+1 on the matrix cores while its
// vector work turns tile t's S and dP into P and dS, then accumulates dV and
// dK with tile t.  The two sets of tiles alternate between register sets, so
// every stretch of the step has both matrix and vector work in the same wave.
// The eight waves of a workgroup share one LDS ring of Q, dO, L2 and -D tiles:
// a ring of 2*GR + 1 slots with one barrier per GR tiles (the barrier
// publishes tiles t+1 .. t+GR and frees the slots of t-GR .. t-1).
template <int D, int GR_, int W_, int KB_ = 1>
struct DkdvPipeCfg {
    static constexpr int W = W_;                   // waves per workgroup
    static constexpr int KB = KB_;                 // 32-key blocks per wave
    static constexpr int BR = 32;                  // queries per tile
    static constexpr int KEYS = 32 * KB * W;       // keys per workgroup
    static constexpr int CH = D / 8, ROWB = D * 2;
    static constexpr int TILEB = BR * ROWB;        // one Q or dO tile
    static constexpr int NB = TILEB / 1024;        // 1 KiB blocks per tile
    static constexpr int RPI = 1024 / ROWB;        // rows per 1 KiB block
    static constexpr int VECB = 256;               // one L2 or -D slice (64 lanes x 4 B)
    static constexpr int STAGEB = 2 * TILEB + 2 * VECB;
    static constexpr int GR = GR_;                 // query tiles per LDS barrier
    static constexpr int ST = 2 * GR + 1;          // ring slots
    static constexpr int LPW = 2 * NB / W;         // 1 KiB loads per wave per tile
    static_assert(LPW >= 1 && LPW * W == 2 * NB, "the tile's loads split evenly over the waves");
    static_assert(GR >= 1 && ST * STAGEB <= 160 * 1024, "ring fits the 160 KiB LDS");
};

template <int D, int GR, int W, int KB, bool CAUSAL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(W / 4, W / 4)))
void bwd_dkdv_pipe_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
                          const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
                          const float *__restrict__ L2, const float *__restrict__ Dv,
                          uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int64_t Nq,
                          int64_t Nk, int64_t qoff, int nkt, uint32_t group, float scale, float c) {
    using T = DkdvPipeCfg<D, GR, W, KB>;
    constexpr int ST = T::ST, ROWB = T::ROWB, BR = T::BR;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * T::STAGEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int g = lane >> 5, lr = lane & 31;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const TileId tid_ = tile_order(blockIdx.x, gridDim.x / (uint32_t)nkt, (uint32_t)nkt, group);
    const int64_t bh = tid_.head;
    const int64_t k0 = (int64_t)tid_.rank * T::KEYS;  // causal: early keys are seen by the most queries
    const int64_t kw0 = k0 + 32 * KB * (int64_t)wave_u;  // key block kb of this wave: kw0 + 32kb + lane%32
    const uint16_t *Qh = uniform_ptr(Q + bh * Nq * D);
    const uint16_t *dOh = uniform_ptr(dO + bh * Nq * D);
    const float *L2h = uniform_ptr(L2 + bh * Nq);
    const float *Dh = uniform_ptr(Dv + bh * Nq);

    // K and V of this wave's keys: B operands of S = Q K^T and dP = dO V^T
    // (each Q and dO fragment read from LDS serves the KB key blocks)
    bf16x8 kf[KB][D / 16], vf[KB][D / 16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const int64_t key = kw0 + 32 * kb + lr;
            kf[kb][ds] = __builtin_bit_cast(bf16x8, load_row16(K + bh * Nk * D, key, Nk, D, ds * 2 + g));
            vf[kb][ds] = __builtin_bit_cast(bf16x8, load_row16(V + bh * Nk * D, key, Nk, D, ds * 2 + g));
        }

    // ---- ring loads: load j of a tile fills 1 KiB block j of the stage (Q
    //      blocks, then dO blocks); this lane writes chunk `lane` of the block,
    //      i.e. row (j % NB)*RPI + lane/CH of its tile with logical chunk
    //      (lane % CH) ^ swz(row).  Loads 0 and 1 also fill the L2 and -D
    //      slices.  Wave w owns loads LPW*w .. LPW*w + LPW-1 (one at d = 64
    //      with eight waves, four at d = 128 with four); with FA_BWD_DMA_ALT
    //      (eight waves) wave w also issues the load of its partner w ^ 4, one
    //      barrier in two.
    constexpr bool ALT = FA_BWD_DMA_ALT && W == 8;
    constexpr int LPW = T::LPW, NO = ALT ? 2 : LPW;
    static_assert(!ALT || LPW == 1, "partner loads with one load per wave");
    uint32_t owner_u[NO], ld_off[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) {
        owner_u[o] = ALT ? (o == 0 ? wave_u : wave_u ^ 4u) : wave_u * LPW + o;
        ld_off[o] = (uint32_t)chunk_off<ROWB>((int)(owner_u[o] % T::NB) * T::RPI + lane / T::CH,
                                              lane % T::CH);
    }
    // (scalar bases at the tile and 32-bit lane offsets; rows and vector
    // lanes past Nq re-read row Nq-1, masked later)
    auto issue_as = [&](int it, int st, int o) __attribute__((always_inline)) {
        const uint32_t j = owner_u[o];
        const int64_t q0 = (int64_t)it * BR;
        const uint32_t sb = lds_addr(smem) + st * T::STAGEB;
        const uint16_t *src = (j < (uint32_t)T::NB ? Qh : dOh) + q0 * D;
        const uint32_t vb = sb + 2 * T::TILEB + j * T::VECB;  // j = 0: L2, j = 1: -D
        const float *vsrc = (j == 0 ? L2h : Dh) + q0;
        if (q0 + 64 <= Nq) {  // every row and vector lane below in range
            dma16_s(src, ld_off[o], sb + j * 1024);
            if (j < 2) dma4_s(vsrc, 4u * (uint32_t)lane, vb);
            return;
        }
        const int last = (int)(Nq - 1 - q0);  // last row of the tile in range
        const int row = (int)(j % T::NB) * T::RPI + lane / T::CH;
        const int rr = row < last ? row : last;
        dma16_s(src, ld_off[o] + (uint32_t)((rr - row) * ROWB), sb + j * 1024);
        if (j < 2) dma4_s(vsrc, 4u * (uint32_t)(lane < last ? lane : last), vb);
    };

    int roff[D / 16], toff[D / 32];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) roff[ds] = chunk_off<ROWB>(lr, 2 * ds + g);
#pragma unroll
    for (int b = 0; b < D / 32; ++b) toff[b] = tr_off<ROWB>(lane, b, 0);

    f32x16 dvacc[KB][D / 32], dkacc[KB][D / 32];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dvacc[kb][b][r] = 0.f;
                dkacc[kb][b][r] = 0.f;
            }

    // S = Q K^T and dP - D = dO V^T - D of the tile in slot st (key block kb:
    // lane: key 32kb + lr; register r: query 8*(r/4) + 4g + r%4 of the tile)
    using Set = f32x16[KB];
    auto sdp = [&](int st, Set &sa, Set &pa) __attribute__((always_inline)) {
        const uint8_t *qt = smem + st * T::STAGEB;
        const uint8_t *ot = qt + T::TILEB;
        const float *dt = (const float *)(ot + T::TILEB) + T::VECB / 4;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sa[kb][r] = 0.f;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 nd = *(const f32x4 *)(dt + 8 * r4 + 4 * g);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) pa[kb][4 * r4 + e] = nd[e];
        }
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const bf16x8 aq = *(const bf16x8 *)(qt + roff[ds]);
            const bf16x8 ao = *(const bf16x8 *)(ot + roff[ds]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kb][ds], sa[kb], 0, 0, 0);
                pa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[kb][ds], pa[kb], 0, 0, 0);
            }
        }
    };
    // P = exp2(S c - L2), dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS
    // with the tile in slot st.  MASKED instances: query offset 8*(r/4) + 4g +
    // r%4 of register r is visible to this lane's key iff lo <= 8*(r/4) + r%4
    // <= hi (lo and hi less 4g, so that the offsets compared are constants)
    auto finish = [&](int st, int64_t q0, Set &sa, Set &pa, auto masked)
                      __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        const uint8_t *qt = smem + st * T::STAGEB;
        const uint8_t *ot = qt + T::TILEB;
        const float *lt = (const float *)(ot + T::TILEB);
        int lo[KB], hi[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            lo[kb] = 0;
            hi[kb] = BR - 1;
            if (MASKED) {
                const int64_t key = kw0 + 32 * kb + lr;
                int64_t lo64 = CAUSAL ? key - qoff - q0 : 0;
                int64_t hi64 = Nq - 1 - q0;
                if (key >= Nk) hi64 = -1;
                lo[kb] = (int)(lo64 < 0 ? 0 : (lo64 > BR ? BR : lo64)) - 4 * g;
                hi[kb] = (int)(hi64 > BR - 1 ? BR - 1 : (hi64 < -1 ? -1 : hi64)) - 4 * g;
            }
        }
        // k-step kq of the products takes queries 16kq .. 16kq+15: registers
        // 8kq .. 8kq+7 (k-slot (g, e) is query 8*(e/4) + 4g + e%4 of the step),
        // and the transposed operands are read in the same slot order
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
            for (int r4 = 2 * kq; r4 < 2 * kq + 2; ++r4) {
                const f32x4 lv = *(const f32x4 *)(lt + 8 * r4 + 4 * g);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        float p = fast_exp2(fmaf(sa[kb][r], c, -lv[e]));
                        if (MASKED && (8 * r4 + e < lo[kb] || 8 * r4 + e > hi[kb])) p = 0.f;
                        sa[kb][r] = p;
                        pa[kb][r] = p * pa[kb][r];
                    }
            }
            bf16x8 pb[KB], sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                pb[kb] = pack8(sa[kb], 8 * kq);
                sb[kb] = pack8(pa[kb], 8 * kq);
            }
#pragma unroll
            for (int b = 0; b < D / 32; ++b) {
                const bf16x8 ao = tr_pair<ROWB>(ot + kq * 16 * ROWB, toff[b]);
                const bf16x8 aq = tr_pair<ROWB>(qt + kq * 16 * ROWB, toff[b]);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    dvacc[kb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb[kb], dvacc[kb][b], 0, 0, 0);
                    dkacc[kb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[kb], dkacc[kb][b], 0, 0, 0);
                }
            }
        }
    };

    // query tiles that see this workgroup's keys (causal: query q sees keys
    // 0 .. q + qoff) and the ones that see this wave's: from its on; tiles
    // before ifull cross the causal diagonal, tiles from pend on are ragged
    const int nqt = (int)((Nq + BR - 1) / BR);
    const int it0 = CAUSAL ? (int)(k0 - qoff > 0 ? (k0 - qoff) / BR : 0) : 0;
    int its = it0, ifull = it0;
    if (CAUSAL) {
        const int64_t a = kw0 - qoff - (BR - 1);  // first query tile whose last query sees kw0
        if (a > 0 && (a + BR - 1) / BR > its) its = (int)((a + BR - 1) / BR);
        const int64_t f = kw0 + 32 * KB - 1 - qoff;  // first tile whose first query sees every key
        ifull = f > 0 ? (int)((f + BR - 1) / BR) : 0;
        if (ifull < its) ifull = its;
    }
    if (kw0 >= Nk) its = ifull = nqt;     // no keys: ring steps only
    // keys after the last query's (causal): no query sees them, and the walk
    // above would still take the ragged last tile, whose rows past Nq it counts
    if (CAUSAL && kw0 > Nq - 1 + qoff) its = ifull = nqt;
    if (kw0 + 32 * KB > Nk) ifull = nqt;   // ragged keys: every tile is masked
    const int pend = (int)(Nq / BR);       // tiles before pend have no ragged queries

    auto ring = [&](int idx) __attribute__((always_inline)) {
        if (idx % GR != 0) return;
        wait_vm<0>();
        lds_barrier();
        if (ALT && FA_BWD_PRIO) __builtin_amdgcn_s_setprio(0);
        if (ALT && ((idx / GR) & 1) != (int)(wave_u >> 2)) return;
#pragma unroll
        for (int t = GR + 1; t <= 2 * GR; ++t)
            if (it0 + idx + t < nqt) {
#pragma unroll
                for (int o = 0; o < NO; ++o) issue_as(it0 + idx + t, (idx + t) % ST, o);
            }
        // the loading wave is behind its partner: let it catch up
        if (ALT && FA_BWD_PRIO) __builtin_amdgcn_s_setprio(FA_BWD_PRIO);
    };

#if FA_STATS
    uint32_t st_tiles = 0;
#endif
    Set s0, p0, s1, p1;
#pragma unroll
    for (int t = 0; t <= GR; ++t)
        if (it0 + t < nqt) {
#pragma unroll
            for (int o = 0; o < LPW; ++o) issue_as(it0 + t, t, o);  // own loads only
        }
    wait_vm<0>();
    lds_barrier();

    const std::integral_constant<bool, false> plain;
    const std::integral_constant<bool, true> generic;
    // a step without pipelining, for the tiles on the causal diagonal, the
    // ragged ends and the steps before this wave's first tile
    auto gstep = [&](int it) __attribute__((always_inline)) {
        const int idx = it - it0;
        ring(idx);
        if (it < its) return;
#if FA_STATS
        ++st_tiles;
#endif
        sdp(idx % ST, s0, p0);
        const int64_t q0 = (int64_t)it * BR;
        if (it < ifull || it >= pend)
            finish(idx % ST, q0, s0, p0, generic);
        else
            finish(idx % ST, q0, s0, p0, plain);
    };
    int it = it0;
    for (; it < nqt && it < ifull; ++it) gstep(it);
    // pipelined steps over unmasked tiles (tile it is visible here: published
    // by the last barrier, or by the one before the loop)
    if (it + 2 < nqt && it + 1 < pend) sdp((it - it0) % ST, s0, p0);
    for (; it + 2 < nqt && it + 1 < pend; it += 2) {  // tiles it, it+1 unmasked; sets alternate
        const int idx = it - it0;
#if FA_STATS
        st_tiles += 2;
#endif
        ring(idx);
        if constexpr (FA_BWD_IGLP >= 0) __builtin_amdgcn_iglp_opt(FA_BWD_IGLP);
        sdp((idx + 1) % ST, s1, p1);
        finish(idx % ST, (int64_t)it * BR, s0, p0, plain);
        ring(idx + 1);
        if constexpr (FA_BWD_IGLP >= 0) __builtin_amdgcn_iglp_opt(FA_BWD_IGLP);
        sdp((idx + 2) % ST, s0, p0);
        finish((idx + 1) % ST, (int64_t)(it + 1) * BR, s1, p1, plain);
    }
    for (; it < nqt; ++it) gstep(it);

#if FA_STATS
    if (lane == 0 && kw0 < Nk) atomicAdd(&g_bwd_stats[3], (unsigned long long)st_tiles);
#endif
    // ---- epilogue: dK = scale * dK_acc, dV = dV_acc through 4 KiB of LDS per
    //      tensor (store_rows_staged); every wave is past its last ring read at
    //      the barrier, so the ring holds the stages
    static_assert(ST * T::STAGEB >= W * 8192, "the ring holds the output stages");
    wait_vm<0>();
    lds_barrier();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        store_rows_staged<D>(smem + wave_u * 8192, dkacc[kb], scale, dK + bh * Nk * D, kw0 + 32 * kb, Nk, lane);
        store_rows_staged<D>(smem + wave_u * 8192 + 4096, dvacc[kb], 1.f, dV + bh * Nk * D, kw0 + 32 * kb,
                             Nk, lane);
    }
}

// ---------------------------------------------------------------------------
// dQ: query-major.
// ---------------------------------------------------------------------------
#ifndef FA_BWD_DQ_WPE  // waves per SIMD of the dQ pass
#define FA_BWD_DQ_WPE 2
#endif

template <int D, int BC_, int GR_, int W_, int QB_>
struct DqCfg {
    static constexpr int W = W_;                    // waves per workgroup
    static constexpr int QB = QB_;                  // 32-query blocks per wave
    static constexpr int QW = 32 * QB;              // queries per wave
    static constexpr int BR = QW * W;               // queries per workgroup
    static constexpr int BC = BC_;                  // keys per tile
    static constexpr int CH = D / 8, ROWB = D * 2;
    static constexpr int TILEB = BC * ROWB;
    static constexpr int GR = GR_;                  // key tiles per LDS barrier
    static constexpr int ST = 2 * GR;               // ring slots: GR in use, GR in flight
    static constexpr int IPW = TILEB / 1024 / W;
    static constexpr int RPI = 1024 / ROWB;
    static_assert(IPW >= 1 && IPW * W * 1024 == TILEB, "dq tile");
    static_assert(W == 4 || W == 8, "4 or 8 waves");
};

template <int D, int BC, int GR, int W, int QB, bool CAUSAL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(D == 64 ? FA_BWD_DQ_WPE : 3 - QB, D == 64 ? FA_BWD_DQ_WPE : 3 - QB)))
void bwd_dq_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
                   const uint16_t *__restrict__ V, const uint16_t *__restrict__ O,
                   const uint16_t *__restrict__ dO, const float *__restrict__ L,
                   float *__restrict__ L2, float *__restrict__ Dv,
                   uint16_t *__restrict__ dQ, int64_t Nq, int64_t Nk, int64_t qoff, int nqt,
                   uint32_t group, float scale, float c) {
    using T = DqCfg<D, BC, GR, W, QB>;
    constexpr int ST = T::ST;
    constexpr int ROWB = T::ROWB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * 2 * T::TILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, lr = lane & 31;
    const TileId tid_ = tile_order(blockIdx.x, gridDim.x / (uint32_t)nqt, (uint32_t)nqt, group);
    const int64_t bh = tid_.head;
    const int qt = CAUSAL ? nqt - 1 - (int)tid_.rank : (int)tid_.rank;  // causal: late queries see the most keys
    const int64_t q0 = (int64_t)qt * T::BR;
    const int64_t qw0 = q0 + wave * T::QW;  // query block qb of this wave: qw0 + 32qb + lane%32
    const uint16_t *Kh = K + bh * Nk * D;
    const uint16_t *Vh = V + bh * Nk * D;

    int64_t nkt = (Nk + BC - 1) / BC;
    if (CAUSAL) {
        const int64_t qlast = (q0 + T::BR < Nq ? q0 + T::BR : Nq) - 1;
        const int64_t lim = (qlast + qoff) / BC + 1;
        nkt = nkt < lim ? nkt : lim;
    }
    const int64_t qw_last = (qw0 + T::QW - 1 < Nq - 1) ? qw0 + T::QW - 1 : Nq - 1;

    // Q and dO of this lane's queries (one per 32-query block): B operands of
    // S^T = K Q^T and dP^T = V dO^T; each K and V fragment read from LDS
    // serves the QB blocks
    bf16x8 qf[QB][D / 16], of[QB][D / 16];
    float l2[QB];
    f32x16 nd[QB];  // -D of this lane's query in every register: dP^T starts from it
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int64_t qrow = qw0 + 32 * qb + lr;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            qf[qb][ds] = __builtin_bit_cast(bf16x8, load_row16(Q + bh * Nq * D, qrow, Nq, D, ds * 2 + g));
            of[qb][ds] = __builtin_bit_cast(bf16x8, load_row16(dO + bh * Nq * D, qrow, Nq, D, ds * 2 + g));
        }
        // D = rowsum(dO * O) and L2 = L * log2(e) of this query: the lane holds
        // half of the row (chunks 2ds + g), lane ^ 32 the other half.  The
        // dK/dV pass, launched after this one, reads both from the workspace.
        const int64_t qc = qrow < Nq ? qrow : Nq - 1;
        float dsum = 0.f;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const u32x4 o = load_row16(O + bh * Nq * D, qrow, Nq, D, ds * 2 + g);
            const u32x4 w = __builtin_bit_cast(u32x4, of[qb][ds]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dsum = fmaf(bf16_lo(o[e]), bf16_lo(w[e]), dsum);
                dsum = fmaf(bf16_hi(o[e]), bf16_hi(w[e]), dsum);
            }
        }
        dsum += __shfl_xor(dsum, 32);
        const float lrow = L[bh * Nq + qc];
        if (g == 0 && qrow < Nq) {
            L2[bh * Nq + qc] = lrow * kLog2e;
            Dv[bh * Nq + qc] = -dsum;
        }
        l2[qb] = qrow < Nq ? lrow * kLog2e : INFINITY;  // padded row: P = 0
#pragma unroll
        for (int r = 0; r < 16; ++r) nd[qb][r] = qrow < Nq ? -dsum : 0.f;
    }

    constexpr bool ALT = FA_BWD_DMA_ALT && W == 8 && GR > 1;
    const int owner[2] = {wave, wave ^ 4};  // this wave and, with ALT, its partner
    auto ld_row = [&](int o, int u) { return (owner[o] * T::IPW + u) * T::RPI + lane / T::CH; };
    uint32_t ld_off[2][T::IPW];  // byte offset of this lane's load within a tile
#pragma unroll
    for (int o = 0; o < (ALT ? 2 : 1); ++o)
#pragma unroll
        for (int u = 0; u < T::IPW; ++u)
            ld_off[o][u] = (uint32_t)chunk_off<ROWB>(ld_row(o, u), lane % T::CH);
    // the loads of wave owner[o] for key tile j into stage st
    auto issue_as = [&](int64_t j, int st, int o) {
        const int64_t kv0 = j * BC;
        uint8_t *kb = smem + st * 2 * T::TILEB;
        uint8_t *vb = kb + T::TILEB;
        if (kv0 + BC <= Nk) {  // whole tile in range: scalar bases
            const uint8_t *ks = (const uint8_t *)(Kh + kv0 * D);
            const uint8_t *vs = (const uint8_t *)(Vh + kv0 * D);
#pragma unroll
            for (int u = 0; u < T::IPW; ++u) {
                const int blk = owner[o] * T::IPW + u;
                dma16_s(ks, ld_off[o][u], kb + blk * 1024);
                dma16_s(vs, ld_off[o][u], vb + blk * 1024);
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < T::IPW; ++u) {
            const int row = ld_row(o, u);
            const int64_t key = kv0 + row < Nk ? kv0 + row : Nk - 1;  // past the end: masked
            const uint32_t col = ld_off[o][u] - row * ROWB;
            const int blk = owner[o] * T::IPW + u;
            dma16((const uint8_t *)(Kh + key * D) + col, kb + blk * 1024);
            dma16((const uint8_t *)(Vh + key * D) + col, vb + blk * 1024);
        }
    };
    auto issue = [&](int64_t j, int st) { issue_as(j, st, 0); };
    int koff[D / 16], toff[D / 32];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) koff[ds] = chunk_off<ROWB>(lr, 2 * ds + g);
#pragma unroll
    for (int b = 0; b < D / 32; ++b) toff[b] = tr_off<ROWB>(lane, b, 0);

    f32x16 acc[QB][D / 32];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][b][r] = 0.f;
#if FA_STATS
    uint32_t st_tiles = 0;
#endif

    // One key tile against this wave's queries; MASKED instances handle the
    // causal diagonal and the ragged end, the rest carry no mask code.
    auto tile = [&](int64_t j, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const int64_t kv0 = j * BC;
        const uint8_t *kt = smem + (j % ST) * 2 * T::TILEB;
#if FA_STATS
        ++st_tiles;
#endif
        const uint8_t *vt = kt + T::TILEB;

        // The tile is walked one 32-key block at a time (scores, vector work,
        // dQ products), so that only one block's scores are live.
        if constexpr (FA_BWD_DQ_IGLP >= 0) __builtin_amdgcn_iglp_opt(FA_BWD_DQ_IGLP);
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) {
            // ---- S^T = K Q^T, dP^T = V dO^T (lane: query lr of block qb;
            //      register r: key 8*(r/4) + 4g + r%4 of the 32-key block)
            f32x16 sacc[QB], pacc[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[qb][r] = 0.f;
                pacc[qb] = nd[qb];  // the products leave dP^T - D
            }
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds) {
                const int off = kb * 32 * ROWB + koff[ds];
                const bf16x8 ak = *(const bf16x8 *)(kt + off);
                const bf16x8 av = *(const bf16x8 *)(vt + off);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[qb][ds], sacc[qb], 0, 0, 0);
                    pacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, of[qb][ds], pacc[qb], 0, 0, 0);
                }
            }
            // ---- P = exp2(S c - L2), dS = P (dP - D), both per lane; masked
            //      tiles zero the keys past Nk and after the query
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                int lim = 32;
                if (MASKED) {
                    const int64_t qrow = qw0 + 32 * qb + lr;
                    const int64_t kb0 = kv0 + kb * 32;
                    int64_t lim64 = Nk - 1 - kb0;  // last visible key offset in the block
                    if (CAUSAL && qrow + qoff - kb0 < lim64) lim64 = qrow + qoff - kb0;
                    lim = (int)(lim64 < -1 ? -1 : (lim64 > 32 ? 32 : lim64)) - 4 * g;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(fmaf(sacc[qb][r], c, -l2[qb]));
                    if (MASKED && 8 * (r >> 2) + (r & 3) > lim) p = 0.f;
                    pacc[qb][r] = p * pacc[qb][r];
                }
            }
            // ---- dQ^T += K^T dS^T.  B operand (k-step h of 16 keys) = registers
            //      8h..8h+7: k-slot (g, e) is key 8*(e/4) + 4g + e%4 of the step;
            //      K^T is read transposed in the same slot order and serves the
            //      QB blocks.
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8 sb[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sb[qb] = pack8(pacc[qb], 8 * h);
#pragma unroll
                for (int b = 0; b < D / 32; ++b) {
                    const bf16x8 a = tr_pair<ROWB>(kt + (2 * kb + h) * 16 * ROWB, toff[b]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        acc[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[qb], acc[qb][b], 0, 0, 0);
                }
            }
        }
    };
    // ring step j: tile j has landed and is visible to every wave (a barrier
    // every GR tiles publishes the next GR tiles and refills the slots of the
    // previous GR)
    auto ring = [&](int64_t j) {
        if (j % GR != 0) return;  // one barrier per GR tiles, as in the dK/dV pass
        wait_vm<0>();
        lds_barrier();
        if (ALT && FA_BWD_PRIO) __builtin_amdgcn_s_setprio(0);
        if (ALT && ((j / GR) & 1) != (wave >> 2)) return;
#pragma unroll
        for (int t = GR; t < 2 * GR; ++t)
            if (j + t < nkt) {
                issue_as(j + t, (int)((j + t) % ST), 0);
                if (ALT) issue_as(j + t, (int)((j + t) % ST), 1);
            }
        // the loading wave is behind its partner: let it catch up
        if (ALT && FA_BWD_PRIO) __builtin_amdgcn_s_setprio(FA_BWD_PRIO);
    };
    // leading tiles with every key visible to every query of this wave
    int64_t nfull = 0;
    if (qw0 < Nq) {
        nfull = Nk / BC;
        if (CAUSAL && (qw0 + qoff + 1) / BC < nfull) nfull = (qw0 + qoff + 1) / BC;
        if (nfull > nkt) nfull = nkt;
    }

#pragma unroll
    for (int t = 0; t < GR; ++t)
        if (t < nkt) issue(t, t);
    int64_t j = 0;
    for (; j < nfull; ++j) {
        ring(j);
        tile(j, std::false_type{});
    }
    for (; j < nkt; ++j) {
        ring(j);
        const bool active = qw0 < Nq && (!CAUSAL || j * BC <= qw_last + qoff);
        if (active) tile(j, std::true_type{});
    }

#if FA_STATS
    if (lane == 0 && qw0 < Nq) atomicAdd(&g_bwd_stats[4], (unsigned long long)st_tiles);
#endif
    // ---- epilogue: dQ = scale * acc through 4 KiB of LDS (store_rows_staged);
    //      every wave is past its last ring read at the barrier, so the ring
    //      holds the stages
    static_assert(ST * 2 * T::TILEB >= W * 4096, "the ring holds the output stages");
    wait_vm<0>();
    lds_barrier();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
        store_rows_staged<D>(smem + wave * 4096, acc[qb], scale, dQ + bh * Nq * D, qw0 + 32 * qb, Nq, lane);
}

// Tile configurations (chosen by measurement on MI355X).
#ifndef FA_BWD_DKDV_BR64
#define FA_BWD_DKDV_BR64 64
#define FA_BWD_DQ_BC64 128
#endif
// d = 64: both passes on eight waves (one workgroup per CU, one ring feeding
// both waves of each SIMD), the dK/dV pass with one barrier per four query
// tiles and the dQ pass with one per two key tiles: 4 % and 2 % faster per
// backward than four waves and a barrier per tile.  (The dQ pass fits eight
// waves because it walks each key tile one 32-key block at a time.)  Two
// query blocks per dQ wave halve its LDS reads but measured 20 % slower.
// Limited to three or four waves per SIMD the dQ pass fits 127-161 registers
// without spills (four-wave workgroups, 32- or 64-key tiles), but ran 1-3 %
// slower per backward at 2 x 16 heads x 4096 and 4 x 16 heads x 2048 causal.
#ifndef FA_BWD_W_DKDV64  // waves per workgroup, d = 64
#define FA_BWD_W_DKDV64 8
#define FA_BWD_W_DQ64 8
#endif
#ifndef FA_BWD_DQ_QB128  // the same at d = 128 (2: one wave per SIMD)
#define FA_BWD_DQ_QB128 1
#endif
#ifndef FA_BWD_DQ_QB64  // 32-query blocks per wave of the dQ pass, d = 64
#define FA_BWD_DQ_QB64 1
#endif
#ifndef FA_BWD_GR_DKDV64  // tiles per LDS barrier, d = 64
#define FA_BWD_GR_DKDV64 4
#define FA_BWD_GR_DQ64 2
#endif
// d = 128, dQ pass: eight waves (one or two barriers per tile, 32- or 64-key
// tiles) measured 4-5 % slower per backward than four waves with 32-key
// tiles at 16 heads x 4096 and 2 x 16 heads x 2048 causal.  With the
// pipelined dK/dV pass, 64-key tiles on four waves (two 32-key blocks per
// tile, the vector work of one beside the products of the next) are 1 %
// faster at 32 heads x 8192 causal and 16 x 4 heads x 2048, level at
// 2 x 16 heads x 4096 causal.
#ifndef FA_BWD_W_DQ128  // waves per workgroup and keys per tile of the dQ pass, d = 128
#define FA_BWD_W_DQ128 4
#define FA_BWD_DQ_BC128 64
#endif
#ifndef FA_BWD_GR_DKDV128  // tiles per LDS barrier, d = 128 (one workgroup of four waves per CU)
#define FA_BWD_GR_DKDV128 1
#define FA_BWD_GR_DQ128 1
#endif
#ifndef FA_BWD_DKDV_KB64  // 32-key blocks per wave in the dK/dV pass, d = 64
#define FA_BWD_DKDV_KB64 1
#endif
#ifndef FA_BWD_DKDV_PIPE  // 1: d = 64 runs the software-pipelined dK/dV pass
#define FA_BWD_DKDV_PIPE 1
#endif
#ifndef FA_BWD_GR_PIPE  // its query tiles per LDS barrier
#define FA_BWD_GR_PIPE 8
#endif
// the same at d = 128 (query tiles per barrier: 4, a 9-slot ring of 16.5 KiB stages)
#ifndef FA_BWD_DKDV_PIPE128
#define FA_BWD_DKDV_PIPE128 1
#endif
// d = 64: waves per workgroup and 32-key blocks per wave of the pipelined
// pass (8 and 1: two waves per SIMD; 4 and 2: one wave per SIMD whose Q and
// dO fragments each serve two key blocks)
#ifndef FA_BWD_PIPE_W64
#define FA_BWD_PIPE_W64 8
#define FA_BWD_PIPE_KB64 1
#endif
#ifndef FA_BWD_GR_PIPE128
#define FA_BWD_GR_PIPE128 4
#endif

template <int D, bool CAUSAL>
struct DkdvChoice {
    // Two 32-key blocks per wave halve the LDS reads per product, but need more
    // than 256 registers, so one wave per SIMD and 32-query tiles; measured
    // 1.3x slower at 2 x 16 heads x 4096 causal (the compiler moves the score
    // tiles between the two register files on every tile).  With one block the
    // non-causal d = 64 instance keeps 32-query tiles: with 64 it needs more
    // than 256 registers.
    static constexpr int KB = D == 64 ? FA_BWD_DKDV_KB64 : 1;
    static constexpr int BR = KB == 2 ? 32 : (D == 64 && CAUSAL ? FA_BWD_DKDV_BR64 : 32);
    // d = 128 needs more than 256 registers (one wave per SIMD): four waves;
    // so does a 32-query tile, whose 4 KiB do not split over eight waves
    static constexpr int W = D == 64 && BR == 64 ? FA_BWD_W_DKDV64 : 4;
    static constexpr int GR = D == 64 ? FA_BWD_GR_DKDV64 : FA_BWD_GR_DKDV128;
    using Cfg = DkdvCfg<D, BR, GR, KB, W>;
};

template <int D>
struct DqChoice {
    static constexpr int BC = D == 64 ? FA_BWD_DQ_BC64 : FA_BWD_DQ_BC128;
    static constexpr int W = D == 64 ? FA_BWD_W_DQ64 : FA_BWD_W_DQ128;
    static constexpr int GR = D == 64 ? FA_BWD_GR_DQ64 : FA_BWD_GR_DQ128;
    static constexpr int QB = D == 64 ? FA_BWD_DQ_QB64 : FA_BWD_DQ_QB128;
    using Cfg = DqCfg<D, BC, GR, W, QB>;
};

template <int D, bool CAUSAL>
hipError_t launch_main(const BwdArgs &a, hipStream_t s) {
    using C = DkdvChoice<D, CAUSAL>;
    using QC = DqChoice<D>;
    // the dQ pass first: it also writes -D and L2, which the dK/dV pass reads
    const int nqt = (int)((a.Nq + QC::Cfg::BR - 1) / QC::Cfg::BR);
    hipLaunchKernelGGL((bwd_dq_kernel<D, QC::BC, QC::GR, QC::W, QC::QB, CAUSAL>),
                       dim3((unsigned)(a.B * a.H * nqt)), dim3(QC::W * 64), 0, s,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (const uint16_t *)a.O, (const uint16_t *)a.dO, a.L, a.L2, a.D,
                       (uint16_t *)a.dQ, a.Nq, a.Nk, a.q_start, nqt, tile_group(a.B * a.H),
                       a.scale, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (D == 64 ? FA_BWD_DKDV_PIPE : FA_BWD_DKDV_PIPE128) {
        // d = 128: four waves (one per SIMD: K, V, both accumulators and two
        // score sets take more than 256 registers)
        constexpr int PW = D == 64 ? FA_BWD_PIPE_W64 : 4, PG = D == 64 ? FA_BWD_GR_PIPE : FA_BWD_GR_PIPE128;
        constexpr int PK = D == 64 ? FA_BWD_PIPE_KB64 : 1;
        using P = DkdvPipeCfg<D, PG, PW, PK>;
        const int nkt = (int)((a.Nk + P::KEYS - 1) / P::KEYS);
        hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<D, PG, PW, PK, CAUSAL>),
                           dim3((unsigned)(a.B * a.H * nkt)), dim3(PW * 64), 0, s,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (const uint16_t *)a.dO, a.L2, a.D, (uint16_t *)a.dK, (uint16_t *)a.dV,
                           a.Nq, a.Nk, a.q_start, nkt, tile_group(a.B * a.H), a.scale,
                           a.scale * kLog2e);
    } else {
        const int nkt = (int)((a.Nk + C::Cfg::KEYS - 1) / C::Cfg::KEYS);
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, C::BR, C::GR, C::KB, C::W, CAUSAL>),
                           dim3((unsigned)(a.B * a.H * nkt)), dim3(C::W * 64), 0, s,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (const uint16_t *)a.dO, a.L2, a.D, (uint16_t *)a.dK, (uint16_t *)a.dV,
                           a.Nq, a.Nk, a.q_start, nkt, tile_group(a.B * a.H), a.scale,
                           a.scale * kLog2e);
    }
    return hipGetLastError();
}

}  // namespace

#if FA_STATS
hipError_t stats_bwd(unsigned long long *host, bool reset) {
    if (reset) {
        static const unsigned long long zero[kStatCount] = {};
        return hipMemcpyToSymbol(HIP_SYMBOL(g_bwd_stats), zero, sizeof(zero));
    }
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_bwd_stats), kStatCount * sizeof(*host));
}

void bwd_bf16_tiles(int64_t d, int causal, int64_t *kv_rows, int64_t *kv_cols, int64_t *q_rows,
                    int64_t *q_cols) {
    *kv_rows = d == 64 ? (causal ? 32 * DkdvChoice<64, true>::KB : 32 * DkdvChoice<64, false>::KB) : 32;
    *kv_cols = d == 64 ? (causal ? DkdvChoice<64, true>::BR : DkdvChoice<64, false>::BR) : 32;
    if (d == 64 && FA_BWD_DKDV_PIPE) {
        *kv_rows = 32 * FA_BWD_PIPE_KB64;
        *kv_cols = 32;
    }
    *q_rows = 32 * (d == 64 ? FA_BWD_DQ_QB64 : FA_BWD_DQ_QB128);
    *q_cols = d == 64 ? FA_BWD_DQ_BC64 : FA_BWD_DQ_BC128;
}
#endif

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s) {
    if (a.d == 128)
        return a.causal ? launch_main<128, true>(a, s) : launch_main<128, false>(a, s);
    return a.causal ? launch_main<64, true>(a, s) : launch_main<64, false>(a, s);
}

}  // namespace fa
