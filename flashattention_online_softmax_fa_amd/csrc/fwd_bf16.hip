// fwd_bf16.hip -- attention forward on bf16 matrix cores (gfx950), d in {64, 128}.
//
// Source: flash_forward (attention_kernels.py): every query tile is
// independent; it keeps a running row maximum m, denominator l and an
// unnormalised accumulator on chip while it walks the key/value tiles,
// rescales them when the maximum grows, skips key tiles that lie entirely
// after its last query under the causal mask, divides once at the end and
// writes L = m + log l.
//
// Work split.  One workgroup (W waves) per (batch*head, query tile); each
// wave owns 32*QB queries, whose Q rows stay in registers.  Key/value tiles of
// BC keys stream from HBM straight into an LDS ring of STAGES slots with
// global_load_lds_dwordx4 (no register staging); the loads of a tile are split
// over the waves, each waiting on its own load counter.  With eight waves the
// two waves of a SIMD (w and w ^ 4) take turns, one barrier to the next, to
// issue both their shares: issued by every wave right after the barrier, the
// loads queue in the CU's one address unit while the SIMDs idle, and a
// per-wave timeline put that queueing at 15 % of the d = 128 key loop.  One
// barrier per GR tiles both
// publishes the next GR tiles and frees the GR slots read in the steps before
// it, which are refilled right away (so GR tiles are in flight while GR are
// computed on; fewer barriers per key: d = 64 takes GR = 4 with a 16-slot
// ring, d = 128 GR = 2 with 8 slots, 2.5 % and 4 % faster than one barrier per
// tile, and 3-7 % faster than GR = 8 (17 slots) and GR = 4 (9 slots)).
//
// Software pipeline.  Step t exponentiates the scores of tile t while the
// matrix cores compute the scores of tile t+1, and accumulates O with tile
// t's values one query block at a time, right after that block's
// exponentials; the scores of consecutive tiles alternate between two
// register sets.  Leading tiles that need no mask for any of the wave's rows run a
// mask-free loop; the rest (the ragged end of the keys, the causal diagonal,
// and the idle steps of waves whose rows end earlier) run a generic one.
// Mask-free steps do not reduce the tile maximum before exponentiating: they
// exponentiate against the reference maximum and raise it only when the
// resulting sums show a score more than about 20 (base 2) above it, which
// keeps the row-max reductions off the common path.
//
// LDS layout.  K and V tiles are row-major (one key per row, 16-byte chunks).
// Chunks are XOR-swizzled per row (swz in fa_device.h) so that both access
// patterns below are free of bank conflicts: 16 lanes reading the same chunk
// of 16 consecutive rows, and 16 lanes reading 32 bytes of 4 consecutive rows.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, C[m][n] with lane = n).  The
// wave computes S^T = K Q^T, so each lane's 16 accumulator values belong to
// one query (lane % 32) and 16 keys; row max and sum are per-lane work.  Those
// registers, rounded to bf16, are the B operand of O^T += V^T P^T.  V^T is
// read from the row-major V tile with ds_read_b64_tr_b16 (within each 16-lane
// group, lane i receives element i%4 of the 8-byte pieces addressed by lanes
// i/4 + 4t, so lanes addressing a 4-row x 16-column block get its columns).
//
// Softmax statistics are base 2 with scale*log2(e) folded into the exponent's
// FMA; L is converted back to the natural logarithm at the end.
#include "fa_device.h"
#include "fa_internal.h"
#include "fwd128_step.inc"

#include <type_traits>

#ifndef FA_FWD_W64
#define FA_FWD_W64 2
#define FA_FWD_W128 2
#endif
#ifndef FA_FWD_QB64
#define FA_FWD_QB64 2
#define FA_FWD_BC64 32
#define FA_FWD_ST64 16
#define FA_FWD_QB128 1
#define FA_FWD_BC128 32
#define FA_FWD_ST128 8
#endif
#ifndef FA_FWD_WG64  // waves per workgroup
#define FA_FWD_WG64 8
#endif
#ifndef FA_FWD_WG128
#define FA_FWD_WG128 8
#endif
#ifndef FA_FWD_LAZY  // 1: mask-free steps skip the tile maximum (see step())
#define FA_FWD_LAZY 1
#endif
#ifndef FA_FWD_GR64  // key tiles per LDS barrier (the ring depth must be >= 2 * this + 1)
#define FA_FWD_GR64 4
#define FA_FWD_GR128 2
#endif
// 1: at each barrier only one wave of each SIMD's pair (waves w and w ^ 4)
// issues the group's ring loads, for both waves, alternating between the two
// from one barrier to the next
#ifndef FA_FWD_DMA_ALT
#define FA_FWD_DMA_ALT 1
#endif
// Instruction-interleaving strategy the compiler applies to a step
// (__builtin_amdgcn_iglp_opt; 2 is its pattern for matrix products mixed
// with exponentials), -1 for none: 0.7 % faster at d = 64 with 0 and 0.8 %
// at causal d = 128 with 2 than without
#ifndef FA_FWD_IGLP64
#define FA_FWD_IGLP64 0
#endif
#ifndef FA_FWD_IGLP128
#define FA_FWD_IGLP128 2
#endif
// 1: the mask-free steps of the d = 128 forward (one 32-query block per wave,
// 32-key tiles, 8 ring slots) run the generated assembly of fwd128_step.inc,
// with its own instruction order and the first K fragments of each step read
// by the step before (1.5 % faster than the compiler's step at causal d = 128)
#ifndef FA_FWD_ASM128
#define FA_FWD_ASM128 1
#endif
// with FA_FWD_DMA_ALT: wave priority of the loading wave until the next
// barrier (s_setprio), so that it catches up with its partner: 1.5 % faster
// at causal d = 128, level at d = 64
#ifndef FA_FWD_PRIO
#define FA_FWD_PRIO 1
#endif

namespace fa {
namespace {

constexpr float kMargin = 8.f;  // base-2 headroom before the reference max is raised

#if FA_STATS
__device__ unsigned long long g_fwd_stats[kStatCount];
#endif

// D: head dimension; QB: 32-query blocks per wave (each K / V^T fragment read
// from LDS feeds QB matrix-core products); BC: keys per tile; W: waves per
// workgroup.  With W = 8 the two waves that share a SIMD belong to the same
// workgroup and keep pace through its barriers, and each K/V tile is streamed
// into LDS once per CU; with W = 4 two workgroups share each CU, each with its
// own ring, and the older one is issued first, so the younger one ends a
// single-round launch alone.  W = 8 is kept: measured faster by 1-2 % at
// d = 64 and, where the ring's LDS traffic per matrix-core product is twice
// as large, by 6 % at d = 128 without the causal mask and 2 % with it.
template <int D, int QB, int BC_, int STAGES_, int W_, int G_>
struct Tile {
    static constexpr int G = G_;                     // key tiles per LDS barrier
    static constexpr int W = W_;
    static constexpr int BC = BC_;
    static constexpr int QW = 32 * QB;               // queries per wave
    static constexpr int BR = W * QW;                // queries per workgroup
    static constexpr int CH = D / 8;                 // 16-byte chunks per row
    static constexpr int ROWB = D * 2;               // bytes per row
    static constexpr int TILEB = BC * ROWB;          // bytes of one K or V tile
    static constexpr int NB = TILEB / 1024;          // 1 KiB blocks per K or V tile
    static constexpr int STAGES = STAGES_;           // LDS ring depth
    static constexpr int LPW = 2 * NB / W;           // 1 KiB loads per wave per tile (K and V)
    static constexpr int RPI = 1024 / ROWB;          // rows per 1 KiB load
    static_assert(LPW >= 1 && LPW * W == 2 * NB, "K and V tiles split evenly over the waves");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "tiles per barrier");
    static_assert(STAGES >= (G == 1 ? 3 : 2 * G + 1) && STAGES <= 20, "ring depth");
    static_assert(STAGES * 2 * TILEB + W * 4096 <= 160 * 1024, "ring and O stages fit the 160 KiB LDS");
    static_assert(BC % 32 == 0, "32-key blocks");
    static_assert(W == 4 || W == 8, "4 or 8 waves");
};

template <int D, int QB, int BC, int ST, int W, int GR, bool CAUSAL, bool POS_SCALE>
__global__ __launch_bounds__(W * 64)
__attribute__((amdgpu_waves_per_eu(D * QB >= 256 ? 1 : (W == 8 ? 2 : (D == 64 ? FA_FWD_W64 : FA_FWD_W128)), 4)))
void fwd_bf16_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
                     const uint16_t *__restrict__ V, uint16_t *__restrict__ O,
                     float *__restrict__ L, int64_t Nq, int64_t Nk, int64_t qoff, int nqt,
                     uint32_t group, float c) {
    using T = Tile<D, QB, BC, ST, W, GR>;
    constexpr int S = T::STAGES;
    constexpr int KB = BC / 32;  // 32-key blocks per tile
    // the generated mask-free step (fwd128_step.inc) for this configuration
    constexpr bool ASM = FA_FWD_ASM128 && D == 128 && QB == 1 && BC == 32 && S == 8 && W == 8 && POS_SCALE;
    // Ring lead: the loads issued at the barrier of step t are for tiles
    // t+LEAD+1 .. t+LEAD+GR.  LEAD = GR publishes tile t+1 by step t; the
    // generated step also reads part of tile t+2 in step t, which takes
    // LEAD = 2 GR (the slots of tiles t-GR .. t-1, refilled at that barrier,
    // then hold tiles t+LEAD+1 .. t+LEAD+GR, so S >= LEAD + GR + 2).
    constexpr int LEAD = ASM ? 2 * GR : GR;
    static_assert(GR == 1 || S >= LEAD + GR + 2, "ring depth for the lead");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * 2 * T::TILEB];
    __shared__ __attribute__((aligned(16))) uint8_t ostage[W * 4096];  // per-wave O staging

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, lr = lane & 31, s16 = lane & 15, G = lane >> 4;
    const int xaddr = (lane ^ 32) << 2;  // ds_bpermute address of the other half of the row
    const TileId tid_ = tile_order(blockIdx.x, gridDim.x / (uint32_t)nqt, (uint32_t)nqt, group);
    const int64_t bh = tid_.head;
    const int qt = CAUSAL ? nqt - 1 - (int)tid_.rank : (int)tid_.rank;  // causal: late queries see the most keys
    const int64_t q0 = (int64_t)qt * T::BR;
    const int64_t qw0 = q0 + wave * T::QW;  // query block qb of this wave: qw0 + 32qb + lane%32
    const uint16_t *Kh = K + bh * Nk * D;
    const uint16_t *Vh = V + bh * Nk * D;

    // Key tiles walked by the workgroup (every wave takes part in every ring
    // step), by this wave (nkt_w), and the leading ones that need no mask for
    // any row of this wave (nfull).  Under causal, query row q sees keys
    // 0 .. q + qoff.
    int nkt = (int)((Nk + BC - 1) / BC);
    if (CAUSAL) {
        const int64_t qlast = (q0 + T::BR < Nq ? q0 + T::BR : Nq) - 1;
        const int64_t lim = (qlast + qoff) / BC + 1;
        nkt = nkt < lim ? nkt : (int)lim;
    }
    const int64_t qw_last = (qw0 + T::QW - 1 < Nq - 1) ? qw0 + T::QW - 1 : Nq - 1;
    int nkt_w = 0, nfull = 0;
    if (qw0 < Nq) {
        nkt_w = nkt;
        if (CAUSAL && (qw_last + qoff) / BC + 1 < nkt_w) nkt_w = (int)((qw_last + qoff) / BC + 1);
        int64_t f = Nk / BC;
        if (CAUSAL && (qw0 + qoff + 1) / BC < f) f = (qw0 + qoff + 1) / BC;
        nfull = (int)(f < nkt_w ? f : nkt_w);
    }

    // ---- ring loads: load j = wave * LPW + u of a step fills 1 KiB block j % NB
    //      of the K (j < NB) or V tile; this lane writes LDS chunk `lane` of the
    //      block with logical chunk (lane % CH) ^ f(row) of that row
    //      (and, with FA_FWD_DMA_ALT, the same for the partner wave w ^ 4)
    constexpr bool ALT = FA_FWD_DMA_ALT && W == 8 && GR > 1;
    const int partner = wave ^ 4;
    int ld_row[2][T::LPW], ld_off[2][T::LPW];
#pragma unroll
    for (int o = 0; o < (ALT ? 2 : 1); ++o)
#pragma unroll
        for (int u = 0; u < T::LPW; ++u) {
            const int row = (((o ? partner : wave) * T::LPW + u) % T::NB) * T::RPI + lane / T::CH;
            ld_row[o][u] = row;
            ld_off[o][u] = chunk_off<T::ROWB>(row, lane % T::CH);
        }
    // the loads of wave `owner` (0: this wave, 1: its partner) for tile t into slot st
    auto issue_as = [&](int t, int st, int owner) {
        const int64_t kv0 = (int64_t)t * BC;
        const uint8_t *kt = (const uint8_t *)(Kh + kv0 * D);
        const uint8_t *vt = (const uint8_t *)(Vh + kv0 * D);
        const bool full = kv0 + BC <= Nk;
        const int ow = owner ? partner : wave;
#pragma unroll
        for (int u = 0; u < T::LPW; ++u) {
            const int j = ow * T::LPW + u;  // wave-uniform
            const bool is_v = j >= T::NB;
            const uint8_t *src = is_v ? vt : kt;
            // V follows K in the slot (ASM: K tiles of all slots, then V tiles)
            uint8_t *dst = ASM ? smem + (is_v ? S * T::TILEB + (j - T::NB) * 1024 : j * 1024) + st * T::TILEB
                               : smem + st * 2 * T::TILEB + j * 1024;
            if (full) {
                dma16_s(src, (uint32_t)ld_off[owner][u], dst);
            } else {  // rows past Nk re-read the last key; they are masked
                const int64_t key = kv0 + ld_row[owner][u];
                const int64_t back = key < Nk ? 0 : (key - (Nk - 1)) * T::ROWB;
                dma16(src + ld_off[owner][u] - back, dst);
            }
        }
    };
    auto issue = [&](int t, int st) { issue_as(t, st, 0); };
    // wait until at most n ring steps of this wave's loads are still in flight
    auto wait_pending = [&](int n) { wait_steps<T::LPW, S - 2>(n); };

    // ---- per-lane constants of the LDS reads (byte offsets within a tile;
    //      with the generated d = 128 step, LDS addresses, which it takes in
    //      fixed registers)
    const int lbase = ASM ? (int)lds_addr(smem) : 0;
    // K (A operand of S^T): row kb*32 + lr, logical chunk 2*ds + g
    int koff[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) koff[ds] = lbase + chunk_off<T::ROWB>(lr, 2 * ds + g);
    // V^T (A operand of O^T, transposed read): rows 16ks + 8h + 4g + (lane%16)/4,
    // columns 32b + 16*((lane/16)%2) + 4*(lane%4)
    int voff[D / 32][2];
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
        voff[b][0] = lbase + tr_off<T::ROWB>(lane, b, 0);
        voff[b][1] = lbase + tr_off<T::ROWB>(lane, b, 1);
        if constexpr (ASM) {  // the V tiles start S * TILEB up
            voff[b][0] += S * T::TILEB;
            voff[b][1] += S * T::TILEB;
        }
    }
    // Where the K and V tiles of ring slot st start: K then V in each slot, or,
    // with the generated step, the K tiles of all slots in the first half of
    // the ring and the V tiles in the second (every read then reaches its
    // slot with a 16-bit immediate)
    auto koff_of = [&](int st) { return ASM ? st * T::TILEB : st * 2 * T::TILEB; };
    auto voff_of = [&](int st) { return ASM ? st * T::TILEB : st * 2 * T::TILEB + T::TILEB; };
    // LDS byte at tile offset `off` of the slot at `slot_off` (ASM: `off` holds the address)
    typedef __attribute__((address_space(3))) uint8_t lds_byte;
    auto at = [&](int slot_off, int off) __attribute__((always_inline)) -> const uint8_t * {
        if constexpr (ASM)
            return (const uint8_t *)(const lds_byte *)(uintptr_t)(uint32_t)(off + slot_off);
        else
            return smem + slot_off + off;
    };

    // ---- Q fragments: B operands of S^T = K Q^T (lane: query lr of each block)
    bf16x8 qf[QB][D / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int64_t qrow = qw0 + 32 * qb + lr;
        const int64_t qr = qrow < Nq ? qrow : Nq - 1;
        const uint16_t *qp = Q + (bh * Nq + qr) * D + g * 8;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const u32x4 w = *(const u32x4 *)(qp + ds * 16);
            qf[qb][ds] = __builtin_bit_cast(bf16x8, qrow < Nq ? w : u32x4{0u, 0u, 0u, 0u});
        }
    }

#if FA_STATS
    uint32_t st_resc = 0;  // rows of this lane (g == 0) whose accumulator was rescaled
#endif
    f32x16 oacc[QB][D / 32];
    f32x16 sacc[QB][KB], snxt[QB][KB];  // scores of the current and the next tile
    // m: reference maximum; l0 + l1: this lane's half of the row sum, in two
    // chains; mt: this lane's maximum of the next tile's scores (base 2)
    float m[QB], l0[QB], l1[QB], mt[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        l0[qb] = 0.f;
        l1[qb] = 0.f;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][b][r] = 0.f;
    }

    // S^T = K_t Q^T from ring slot st; each K fragment serves all QB query blocks
    auto scores = [&](int st, f32x16 (&acc)[QB][KB]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            bf16x8 a[D / 16];
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds)
                a[ds] = *(const bf16x8 *)at(koff_of(st) + kb * 32 * T::ROWB, koff[ds]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[qb][kb][r] = 0.f;
#pragma unroll
                for (int ds = 0; ds < D / 16; ++ds)
                    acc[qb][kb] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ds], qf[qb][ds], acc[qb][kb], 0, 0, 0);
            }
        }
        if (!POS_SCALE)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[qb][kb][r] *= c;
    };
    // Mask keys past Nk, and keys after the query under causal.  Key offset of
    // register r in this lane: kb*32 + 8*(r/4) + 4g + r%4.
    auto mask = [&](int t, f32x16 (&acc)[QB][KB]) {
        const int64_t kv0 = (int64_t)t * BC;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int64_t qrow = qw0 + 32 * qb + lr;
            const bool need = (kv0 + BC > Nk) || (CAUSAL && kv0 + BC - 1 > qw0 + 32 * qb + qoff);
            if (need) {
                int64_t lim64 = Nk - 1 - kv0;  // last visible key offset
                if (CAUSAL && qrow + qoff - kv0 < lim64) lim64 = qrow + qoff - kv0;
                const int lim = (int)(lim64 < -1 ? -1 : (lim64 > BC ? BC : lim64)) - 4 * g;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) acc[qb][kb][r] = -INFINITY;
            }
        }
    };
    // this lane's maximum over its half of each query row of the tile, base 2
    auto tile_max = [&](const f32x16 (&acc)[QB][KB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float v = fmaxf(acc[qb][0][0], acc[qb][0][1]);
#pragma unroll
            for (int i = 2; i < 16 * KB; i += 2)  // pairs fold into three-way maxima
                v = fmaxf(fmaxf(v, acc[qb][i / 16][i % 16]), acc[qb][i / 16][i % 16 + 1]);
            mt[qb] = POS_SCALE ? v * c : v;
        }
    };
    // Keep a value computed where it is written: the compiler would otherwise
    // sink the row sums and maxima past the next barrier, out of the block
    // where they overlap the matrix-core work.
    auto pin = [](float &x) { __asm__ volatile("" : "+v"(x)); };

    // One step of the walk over key tiles, software-pipelined: exponentiate
    // tile t (scores in cur), compute the scores of tile t+1 into nxt
    // meanwhile, and accumulate O with tile t's values.  `generic` steps mask
    // tile t+1 where needed and handle a wave's last tile.
    // raise the reference maximum of query block qb to the row maximum of the
    // tile whose lane maxima are in mt[qb] where that exceeds it by more than
    // kMargin, rescaling the row's accumulator and sum
    auto raise = [&](int qb) {
        // the other half of the row is in lane ^ 32
        const float mj = fmaxf(mt[qb], __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                                xaddr, __builtin_bit_cast(int, mt[qb]))));
        const bool grow = mj > m[qb] + kMargin;  // same in both lanes of the row
        const float m_new = grow ? mj : m[qb];
        const float alpha = fast_exp2(m[qb] - m_new);  // 0 on the first tile, else <= 1
#if FA_STATS
        if (grow && m[qb] > -INFINITY && g == 0 && qw0 + 32 * qb + lr < Nq) ++st_resc;
#endif
        l0[qb] *= alpha;
        l1[qb] *= alpha;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][b][r] *= alpha;
        m[qb] = m_new;
    };
    // P^T of query block qb of the tile in cur as bf16 B operands (k-step ks
    // uses registers 8h..8h+7 of block ks/2, so k-slot (g, e) is key
    // 8*(e/4) + 4g + e%4 of the step); the probabilities are summed into s0, s1
    auto probs = [&](int qb, const f32x16 (&cur)[QB][KB], bf16x8 (&pf)[QB][BC / 16], float &s0,
                     float &s1) {
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks) {
            const int kb = ks >> 1, h = ks & 1;
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                p[e] = fast_exp2(POS_SCALE ? fmaf(cur[qb][kb][8 * h + e], c, -m[qb])
                                           : cur[qb][kb][8 * h + e] - m[qb]);
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                s0 += p[e];
                s1 += p[e + 1];
            }
            const u32x4 w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                             pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
            pf[qb][ks] = __builtin_bit_cast(bf16x8, w);
        }
    };
    // A operand of O^T += V_u^T P^T for k-step ks and rows 32b.. of V_u^T, read
    // transposed from the row-major V tile in the k-slot order of P^T
    auto vfrag = [&](int u, int ks, int b) {
        const int so = voff_of(u % S) + ks * 16 * T::ROWB;
        const u32x2 lo = tr_read(at(so, voff[b][0])), hi = tr_read(at(so, voff[b][1]));
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        return __builtin_bit_cast(bf16x8, w);
    };
    auto step = [&](int t, f32x16 (&cur)[QB][KB], f32x16 (&nxt)[QB][KB], auto generic) {
        constexpr bool GEN = decltype(generic)::value;
        constexpr int IGLP = D == 64 ? FA_FWD_IGLP64 : FA_FWD_IGLP128;
        if constexpr (IGLP >= 0) __builtin_amdgcn_iglp_opt(IGLP);
        // ---- online softmax (base 2).  m is a reference maximum: O = acc / l
        //      and L = m + log2 l do not depend on which reference is used, so
        //      it is raised (and the accumulator and sum rescaled) only when
        //      the exponentials would otherwise grow large.  Generic steps
        //      (with FA_FWD_LAZY = 0, every step) compare the tile maximum with
        //      m + kMargin before exponentiating; mask-free steps skip the tile
        //      maximum, exponentiate against m and check the sums afterwards.
        constexpr bool LAZY = FA_FWD_LAZY && !GEN;
        if constexpr (!LAZY) {
            if constexpr (FA_FWD_LAZY) tile_max(cur);  // else computed by the previous step
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                if (__any(mt[qb] > m[qb] + kMargin)) raise(qb);
        }
        const bool next = GEN ? t + 1 < nkt_w : true;
        if (!GEN || next) scores((t + 1) % S, nxt);

        // ---- per query block: probabilities, then O^T += V_t^T P^T at once, so
        //      that one block's products overlap the next block's exponentials
        //      (1.8 % faster at d = 64 than all products after all blocks).  The
        //      V^T fragments are read once and serve every block.
        bf16x8 pf[QB][BC / 16];
        bf16x8 va[BC / 16][D / 32];
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
            for (int b = 0; b < D / 32; ++b) va[ks][b] = vfrag(t, ks, b);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if constexpr (LAZY) {
                // Exponents against the current reference.  Every probability
                // is <= the larger of its lane's two sums, so sums <= 2^24 keep
                // P, O and l far from fp32 overflow; otherwise (an infinite sum
                // included) raise the reference to the row maximum of the tile
                // and exponentiate again.  Rare: it takes a score more than 20
                // above the reference in base 2.
                float s0 = 0.f, s1 = 0.f;
                probs(qb, cur, pf, s0, s1);
                if (__any(!(fmaxf(s0, s1) <= 0x1p24f))) {
                    float v = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) v = fmaxf(v, cur[qb][kb][r]);
                    mt[qb] = POS_SCALE ? v * c : v;
                    raise(qb);
                    s0 = 0.f;
                    s1 = 0.f;
                    probs(qb, cur, pf, s0, s1);
                }
                l0[qb] += s0;
                l1[qb] += s1;
            } else {
                probs(qb, cur, pf, l0[qb], l1[qb]);
            }
#pragma unroll
            for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
                for (int b = 0; b < D / 32; ++b)
                    oacc[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks][b], pf[qb][ks],
                                                                          oacc[qb][b], 0, 0, 0);
        }
        if (!GEN || next) {
            if (GEN && t + 1 >= nfull) mask(t + 1, nxt);
            if (!FA_FWD_LAZY) tile_max(nxt);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            pin(l0[qb]);
            pin(l1[qb]);
            if (!FA_FWD_LAZY) pin(mt[qb]);
        }
    };
    // ring step t: tile t+1 (keys of the next scores) has landed and is visible
    // to every wave, the slot read in step t-1 is free, and it is refilled
    auto ring = [&](int t) {
        if constexpr (GR > 1) {
            // one barrier per GR steps: at t = 0 (mod GR), tiles t+1 .. t+GR
            // (issued at the barrier of step t-GR, the only loads in flight) have
            // landed and become visible, the slots of tiles t-GR .. t-1 are free,
            // and tiles t+GR+1 .. t+2GR are issued into them
            if (t % GR != 0) return;
            wait_vm<0>();
            lds_barrier();
            if constexpr (ALT) {
                // one wave of each SIMD's pair loads for both, in turn: its
                // partner computes meanwhile instead of queueing for the loads
                if (FA_FWD_PRIO) __builtin_amdgcn_s_setprio(0);
                if (((t / GR) & 1) != (wave >> 2)) return;
#pragma unroll
                for (int j = LEAD + 1; j <= LEAD + GR; ++j)
                    if (t + j < nkt) {
                        issue_as(t + j, (t + j) % S, 0);
                        issue_as(t + j, (t + j) % S, 1);
                    }
                // the loading wave is behind its partner: let it catch up
                if (FA_FWD_PRIO) __builtin_amdgcn_s_setprio(FA_FWD_PRIO);
                return;
            }
#pragma unroll
            for (int j = LEAD + 1; j <= LEAD + GR; ++j)
                if (t + j < nkt) issue(t + j, (t + j) % S);
        } else {
            if (t + 1 < nkt) {
                const int ahead = nkt - t - 2;  // tiles after t+1 already issued, at most S-3
                wait_pending(ahead < S - 3 ? ahead : S - 3);
            }
            lds_barrier();
            if (t + S - 1 < nkt) issue(t + S - 1, (t + S - 1) % S);
        }
    };

    constexpr int PRO = GR > 1 ? LEAD + 1 : S - 1;  // tiles issued before the loop
#pragma unroll
    for (int t = 0; t < PRO; ++t)
        if (t < nkt) issue(t, t);
    if (nkt > 0) {
        if constexpr (ASM) {  // tiles 0 and 1 have landed
            const int rest = (nkt < PRO ? nkt : PRO) - 2;
            wait_steps<T::LPW, PRO - 2>(rest < 0 ? 0 : rest);
        } else {  // tile 0 has landed
            wait_steps<T::LPW, PRO - 1>(nkt - 1 < PRO - 1 ? nkt - 1 : PRO - 1);
        }
        lds_barrier();
        if (nkt_w > 0) {
            scores(0, sacc);
            if (nfull == 0) mask(0, sacc);
            tile_max(sacc);
            if (FA_FWD_LAZY)  // the reference starts at tile 0's row maximum (finite:
                              // every row sees key 0)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) raise(qb);
        }
    }
    const std::integral_constant<bool, false> plain;
    const std::integral_constant<bool, true> generic;
    int t = 0;
    if constexpr (ASM) {
        // The generated step (fwd128_step.inc) with this kernel's state in the
        // registers it names.  It checks nothing itself: as in the generic
        // steps, the tile maximum it leaves in mt is compared with the
        // reference before the next step, which raises it in C++ (rare).  The
        // accumulators are read by vector code only after a fence that gives
        // the step's last products time to land.
        // K fragments 0-3 of tile t+1, read by the step before (for the first
        // step, here: tiles 0 and 1 have landed)
        u32x4 kf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i] = *(const u32x4 *)at(koff_of(1), koff[i]);
        auto fence = [&]() __attribute__((always_inline)) {
            __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                             : "+{v[32:47]}"(oacc[0][0]), "+{v[48:63]}"(oacc[0][1]),
                               "+{v[64:79]}"(oacc[0][2]), "+{v[80:95]}"(oacc[0][3]));
        };
#define FA_ASM_STEP(U)                                                                            \
    __asm__ volatile(FA_FWD128_STEP_##U                                                           \
                     : "+{v[32:47]}"(oacc[0][0]), "+{v[48:63]}"(oacc[0][1]),                      \
                       "+{v[64:79]}"(oacc[0][2]), "+{v[80:95]}"(oacc[0][3]),                      \
                       "+{v[96:111]}"(sacc[0][0]), "+{v[112:127]}"(snxt[0][0]),                   \
                       "+{v184}"(l0[0]), "+{v185}"(l1[0]), "={v204}"(mt[0]),                      \
                       "+{v[128:131]}"(kf[0]), "+{v[132:135]}"(kf[1]), "+{v[136:139]}"(kf[2]),    \
                       "+{v[140:143]}"(kf[3])                                                     \
                     : [c] "s"(c), "{v[0:3]}"(qf[0][0]), "{v[4:7]}"(qf[0][1]),                    \
                       "{v[8:11]}"(qf[0][2]), "{v[12:15]}"(qf[0][3]), "{v[16:19]}"(qf[0][4]),     \
                       "{v[20:23]}"(qf[0][5]), "{v[24:27]}"(qf[0][6]), "{v[28:31]}"(qf[0][7]),    \
                       "{v186}"(negm), "{v187}"(koff[0]), "{v188}"(koff[1]), "{v189}"(koff[2]),   \
                       "{v190}"(koff[3]), "{v191}"(koff[4]), "{v192}"(koff[5]), "{v193}"(koff[6]), \
                       "{v194}"(koff[7]), "{v195}"(voff[0][0]), "{v196}"(voff[0][1]), "{v197}"(voff[1][0]), \
                       "{v198}"(voff[1][1]), "{v199}"(voff[2][0]), "{v200}"(voff[2][1]), "{v201}"(voff[3][0]), \
                       "{v202}"(voff[3][1])                                                          \
                     : FA_ASM_TEMPS "v203", "memory")
        // one asm step per ring slot, so that each has its slot in its
        // immediates and the state stays in its registers from step to step
        auto astep = [&](auto U) __attribute__((always_inline)) {
            if (__any(mt[0] > m[0] + kMargin)) {
                fence();
                raise(0);
            }
            const float negm = -m[0];
            constexpr int u = decltype(U)::value;
            if constexpr (u == 0) FA_ASM_STEP(0);
            else if constexpr (u == 1) FA_ASM_STEP(1);
            else if constexpr (u == 2) FA_ASM_STEP(2);
            else if constexpr (u == 3) FA_ASM_STEP(3);
            else if constexpr (u == 4) FA_ASM_STEP(4);
            else if constexpr (u == 5) FA_ASM_STEP(5);
            else if constexpr (u == 6) FA_ASM_STEP(6);
            else FA_ASM_STEP(7);
        };
#undef FA_ASM_STEP
        for (; t + S < nfull; t += S) {  // tiles t .. t+8 need no mask; t = 0 (mod 8)
            const int tb = t & ~(S - 1);   // t, with its low bits visible to the compiler
            ring(tb);
            astep(std::integral_constant<int, 0>());
            ring(tb + 1);
            astep(std::integral_constant<int, 1>());
            ring(tb + 2);
            astep(std::integral_constant<int, 2>());
            ring(tb + 3);
            astep(std::integral_constant<int, 3>());
            ring(tb + 4);
            astep(std::integral_constant<int, 4>());
            ring(tb + 5);
            astep(std::integral_constant<int, 5>());
            ring(tb + 6);
            astep(std::integral_constant<int, 6>());
            ring(tb + 7);
            astep(std::integral_constant<int, 7>());
        }
        fence();
    }
    for (; t + 2 < nfull; t += 2) {  // tiles t .. t+2 need no mask; scores alternate
        ring(t);
        step(t, sacc, snxt, plain);
        ring(t + 1);
        step(t + 1, snxt, sacc, plain);
    }
    for (; t < nkt; ++t) {
        ring(t);
        if (t < nkt_w) {
            step(t, sacc, snxt, generic);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sacc[qb][kb] = snxt[qb][kb];
        }
    }
    wait_vm<0>();

    // ---- epilogue: one division, natural-log L.  A lane holds 4-value pieces
    // of one query's O row (column lr of O^T), so O leaves through this wave's
    // own 4 KiB of LDS, 32 rows x 64 columns at a time: each global store then
    // writes 8 rows x 128 contiguous bytes instead of 32 rows x 16 bytes.
    // Row r's 16-byte chunk c sits at chunk c ^ (r % 8) of its 128 bytes.
    uint8_t *stg = ostage + wave * 4096;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int64_t qrow = qw0 + 32 * qb + lr;
        const float lh = l0[qb] + l1[qb];
        const float l_tot = lh + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                     xaddr, __builtin_bit_cast(int, lh)));
        const float inv = 1.f / l_tot;
        if (qrow < Nq && g == 0) L[bh * Nq + qrow] = (m[qb] + log2f(l_tot)) * kLn2;
#pragma unroll
        for (int h = 0; h < D / 64; ++h) {
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    const int b = 2 * h + b2;
                    const u32x2 w = {
                        pack_bf16x2(oacc[qb][b][4 * t4] * inv, oacc[qb][b][4 * t4 + 1] * inv),
                        pack_bf16x2(oacc[qb][b][4 * t4 + 2] * inv, oacc[qb][b][4 * t4 + 3] * inv)};
                    *(u32x2 *)(stg + lr * 128 + (((4 * b2 + t4) ^ (lr & 7)) << 4) + 8 * g) = w;
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 8 * i + (lane >> 3), ch = lane & 7;
                const u32x4 w = *(const u32x4 *)(stg + r * 128 + ((ch ^ (r & 7)) << 4));
                const int64_t orow = qw0 + 32 * qb + r;
                if (orow < Nq) *(u32x4 *)(O + (bh * Nq + orow) * D + 64 * h + 8 * ch) = w;
            }
            // the next piece overwrites the stage only after these reads
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
#if FA_STATS
    {
        int r = (int)st_resc;
        for (int o = 32; o > 0; o >>= 1) r += __shfl_xor(r, o);
        if (lane == 0) {
            if (qw0 < Nq) {
                const int nk_all = (int)((Nk + BC - 1) / BC);
                atomicAdd(&g_fwd_stats[0], (unsigned long long)nkt_w);
                atomicAdd(&g_fwd_stats[1], (unsigned long long)(nk_all - nkt_w));
            }
            atomicAdd(&g_fwd_stats[2], (unsigned long long)r);
        }
    }
#endif
}

template <int D, int QB, int BC, int ST, int W, int G, bool CAUSAL>
hipError_t launch_d(const FwdArgs &a, hipStream_t s) {
    using T = Tile<D, QB, BC, ST, W, G>;
    const int nqt = (int)((a.Nq + T::BR - 1) / T::BR);
    const dim3 grid((unsigned)(a.B * a.H * nqt));
    const float c = a.scale * kLog2e;
    const uint32_t group = tile_group(a.B * a.H);
    if (a.scale > 0.f)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BC, ST, W, G, CAUSAL, true>), grid, dim3(W * 64), 0, s,
                           (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (uint16_t *)a.O, a.L, a.Nq, a.Nk, a.q_start, nqt, group, c);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, BC, ST, W, G, CAUSAL, false>), grid, dim3(W * 64), 0,
                           s, (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                           (uint16_t *)a.O, a.L, a.Nq, a.Nk, a.q_start, nqt, group, c);
    return hipGetLastError();
}

// Tile configurations (chosen by measurement on MI355X).
constexpr int kQB64 = FA_FWD_QB64, kBC64 = FA_FWD_BC64, kST64 = FA_FWD_ST64, kWG64 = FA_FWD_WG64;
constexpr int kQB128 = FA_FWD_QB128, kBC128 = FA_FWD_BC128, kST128 = FA_FWD_ST128,
              kWG128 = FA_FWD_WG128;
constexpr int kGR64 = FA_FWD_GR64, kGR128 = FA_FWD_GR128;

}  // namespace

#if FA_STATS
hipError_t stats_fwd(unsigned long long *host, bool reset) {
    if (reset) {
        static const unsigned long long zero[kStatCount] = {};
        return hipMemcpyToSymbol(HIP_SYMBOL(g_fwd_stats), zero, sizeof(zero));
    }
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_fwd_stats), kStatCount * sizeof(*host));
}

void fwd_bf16_tile(int64_t d, bool workgroup, int64_t *rows, int64_t *cols) {
    using T128 = Tile<128, kQB128, kBC128, kST128, kWG128, kGR128>;
    using T64 = Tile<64, kQB64, kBC64, kST64, kWG64, kGR64>;
    *rows = d == 128 ? (workgroup ? T128::BR : T128::QW) : (workgroup ? T64::BR : T64::QW);
    *cols = d == 128 ? kBC128 : kBC64;
}
#endif

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
    if (a.d == 128)
        return a.causal ? launch_d<128, kQB128, kBC128, kST128, kWG128, kGR128, true>(a, s)
                        : launch_d<128, kQB128, kBC128, kST128, kWG128, kGR128, false>(a, s);
    return a.causal ? launch_d<64, kQB64, kBC64, kST64, kWG64, kGR64, true>(a, s)
                    : launch_d<64, kQB64, kBC64, kST64, kWG64, kGR64, false>(a, s);
}

}  // namespace fa
