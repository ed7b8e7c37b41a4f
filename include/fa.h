/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention library, libfa.so.
 *
 * Exact scaled-dot-product attention computed without materialising the
 * N x N score or probability matrices.  For every batch b, head h and query
 * row i:
 *
 *     S_ij = scale * sum_c Q_ic K_jc          (scores of the visible keys)
 *     O_i  = sum_j softmax_j(S_i.) V_j          (attention output)
 *     L_i  = log sum_j exp(S_ij)                (natural-log log-sum-exp)
 *
 * With `causal` set, key j is visible to query i iff j <= i (top-left
 * alignment; every query sees key 0, so no row is ever empty).
 *
 * Sources: attention_kernels.py (CMU 15-779 lecture 5): the notation block at
 * the top of the file, standard_attention, flash_forward, flash_backward,
 * flash_decode, merge_states; lab.py (hs-black FlashAttention post): dense,
 * tiled, backward.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.     Q, O, dO, dQ are [B][H][Nq][d]; K, V, dK, dV are [B][H][Nk][d];
 *             all contiguous with d fastest.  L and D are [B][H][Nq] fp32.
 * Pointers.   Device pointers (memory of the GPU current on the calling
 *             thread).  bf16 buffers must be 16-byte aligned, fp32 buffers
 *             4-byte aligned.  Inputs and outputs must not overlap.
 * Ownership.  The caller allocates and frees every buffer, workspaces
 *             included.  The library never allocates, frees or synchronises
 *             (fa_bwd_noalloc uses a fixed array inside the library instead
 *             of a workspace; see there).
 * Streams.    `stream` is a hipStream_t (NULL = the default stream).  Every
 *             call only enqueues work on it and returns; results are ready
 *             when the stream reaches that point.
 * Errors.     Arguments are checked before anything is enqueued; a rejected
 *             call returns FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED and
 *             launches nothing.  A failed launch returns FA_ERR_HIP.  Faults
 *             inside kernels surface at the caller's next synchronisation.
 *             No call keeps state between calls; calls are thread-safe
 *             (except that fa_bwd_noalloc calls on one GPU share its array).
 * Precision.  FA_BF16 inputs are multiplied on bf16 matrix cores with fp32
 *             accumulation; softmax statistics, L, D and partial states are
 *             fp32; bf16 outputs are rounded to nearest even.  FA_F32 runs
 *             in fp32 throughout.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, size < 1, bad scale, ... */
    FA_ERR_UNSUPPORTED = 2, /* valid request outside what is built (d, dtype)   */
    FA_ERR_HIP = 3,         /* the HIP runtime refused a launch                  */
    FA_STATUS_INT = 0x7fffffff /* not a status: makes every int a valid value    */
} fa_status;

typedef enum fa_dtype {
    FA_F32 = 0,  /* IEEE binary32 */
    FA_BF16 = 1, /* bfloat16      */
    FA_DTYPE_INT = 0x7fffffff /* not a dtype: makes every int a valid value (rejected) */
} fa_dtype;

/*
 * fa_fwd -- attention forward: O and L from Q, K, V.
 * Source: flash_forward (attention_kernels.py): query tiles are independent;
 * each walks the key/value tiles keeping a running maximum m, denominator l
 * and unnormalised accumulator on chip, rescales them when m grows, divides
 * once at the end and writes L = m + log l.  Fully masked key tiles are
 * skipped under `causal`.
 *   dt      FA_BF16: Q, K, V, O bf16, d in {64, 128}.
 *           FA_F32:  Q, K, V, O fp32, 1 <= d <= 128.
 *   O       output [B][H][Nq][d], dtype dt.  L output [B][H][Nq] fp32.
 *   scale   finite score scale (1/sqrt(d) is the usual choice).
 *   causal  0 or 1.
 */
fa_status fa_fwd(fa_dtype dt, const void *Q, const void *K, const void *V, void *O, float *L,
                 int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                 int causal, void *stream);

/*
 * fa_fwd_offset -- causal forward with the queries placed at key positions
 * q_start .. q_start + Nq - 1: key j is visible to query row i iff
 * j <= q_start + i.  q_start = Nk - Nq aligns the last query with the last key
 * (bottom-right causal: a chunk of new tokens attending to a cache that ends
 * with them); q_start = 0 is fa_fwd with causal = 1.
 * Source: standard_attention and flash_forward (attention_kernels.py), whose
 * causal mask compares absolute positions q_start + i and j, and skips key
 * tiles that start after the tile's last absolute query position.
 *   q_start  0 <= q_start <= 2^40 (every row then sees key 0); larger values
 *            than Nk - 1 leave every key visible.  Other arguments as fa_fwd.
 */
fa_status fa_fwd_offset(fa_dtype dt, const void *Q, const void *K, const void *V, void *O,
                        float *L, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                        float scale, int64_t q_start, void *stream);

/*
 * fa_fwd_blocked -- fp32 forward whose online-softmax step is exactly
 * `kv_block` keys (1 <= kv_block <= 256), for checking block-size invariance.
 * Source: TiledAttention (model.py) and tiled (lab.py): the result does not
 * depend on the block size.  Same arguments as fa_fwd with dt = FA_F32.
 */
fa_status fa_fwd_blocked(fa_dtype dt, const void *Q, const void *K, const void *V, void *O,
                         float *L, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                         float scale, int causal, int64_t kv_block, void *stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs: the row
 * sums D = rowsum(dO * O) (the bf16 kernels store -D) and L * log2(e), each
 * [B][H][Nq] fp32 rounded up to 256 bytes.  Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(fa_dtype dt, int64_t B, int64_t H, int64_t Nq, int64_t d);

/*
 * fa_bwd -- attention backward: dQ, dK, dV of the scalar <O, dO>.
 * Source: flash_backward (attention_kernels.py): D = rowsum(dO * O); key/value
 * tiles are independent; each walks the query tiles, recomputes
 * P = exp(S - L) from the stored L, forms dV += P^T dO, dP = dO V^T,
 * dS = P * (dP - D), dK += scale dS^T Q and dQ += scale dS K.  dK and dV
 * are accumulated per key tile; dQ is accumulated per query tile by a
 * second pass that recomputes S and dP (no atomic additions), so the
 * result is deterministic.
 *   dt         FA_BF16: bf16 tensors on matrix cores, d in {64, 128}.
 *              FA_F32:  fp32 tensors on the vector ALUs, 1 <= d <= 128 (meant
 *              for exact checks at small sizes).
 *   dQ, dK, dV have the dtype of Q.
 *   O, L       the forward's outputs for the same Q, K, V, scale, causal.
 *   dO         upstream gradient [B][H][Nq][d] bf16.
 *   dQ, dK, dV outputs, fully overwritten.
 *   workspace  device buffer of at least fa_bwd_workspace_size() bytes,
 *              256-byte aligned; its contents on entry do not matter.
 */
fa_status fa_bwd(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                 const float *L, const void *dO, void *dQ, void *dK, void *dV, void *workspace,
                 size_t ws_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                 float scale, int causal, void *stream);

/*
 * fa_bwd_offset -- backward of fa_fwd_offset: the same causal mask with
 * query row i at key position q_start + i.  Key tiles that no query can see
 * get dK = dV = 0.
 * Source: flash_backward (attention_kernels.py) with the mask of
 * standard_attention at offset q_start.
 *   q_start  as fa_fwd_offset; O and L must come from fa_fwd_offset with the
 *            same q_start.  Other arguments, workspace included, as fa_bwd.
 */
fa_status fa_bwd_offset(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                        const float *L, const void *dO, void *dQ, void *dK, void *dV,
                        void *workspace, size_t ws_bytes, int64_t B, int64_t H, int64_t Nq,
                        int64_t Nk, int64_t d, float scale, int64_t q_start, void *stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument and no allocation of any kind.  The
 * backward's workspace (D and L * log2(e)) lives instead in a fixed array of
 * FA_NOALLOC_SCRATCH_BYTES bytes of device memory inside the library, one per
 * GPU, held until the process ends.
 *   Arguments and results as fa_bwd (causal: 0 or 1, top-left).
 *   Limit: fa_bwd_workspace_size(dt, B, H, Nq, d) must not exceed
 *   FA_NOALLOC_SCRATCH_BYTES, i.e. B * H * Nq <= 2^21 query rows; larger
 *   calls return FA_ERR_INVALID_ARG and launch nothing.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a
 *   GPU (other streams or threads, before the previous call has finished)
 *   race and give wrong results.  Calls in order on one stream are safe; the
 *   array needs no clearing (every value read is written first in the call).
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
fa_status fa_bwd_noalloc(fa_dtype dt, const void *Q, const void *K, const void *V,
                         const void *O, const float *L, const void *dO, void *dQ, void *dK,
                         void *dV, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                         float scale, int causal, void *stream);

/*
 * fa_decode_split -- first pass of split-KV decoding (Flash-Decoding).
 * Source: flash_decode and state_of_scores (attention_kernels.py): the keys
 * are cut into n_split contiguous splits, split s holding keys
 * [floor(Nk*s/n_split), floor(Nk*(s+1)/n_split)); each split is summarised
 * independently as (m, l, o) with m = max score, l = sum exp(s - m),
 * o = sum exp(s - m) V (unnormalised).  An empty split (n_split > Nk) gives
 * (-inf, 0, 0).  No causal mask (see fa_decode_split_offset).
 *   dt      FA_BF16: d = 128 or 64.  FA_F32: 1 <= d <= 128 (vector ALUs).
 *           Q [B][H][Nq][d], K, V [B][H][Nk][d].
 *   part_m, part_l  outputs [B][H][Nq][n_split] fp32 (m in natural-log units,
 *                   i.e. the scale is applied).
 *   part_o          output [B][H][Nq][n_split][d] fp32.
 *   n_split >= 1.
 */
fa_status fa_decode_split(fa_dtype dt, const void *Q, const void *K, const void *V,
                          float *part_m, float *part_l, float *part_o, int64_t B, int64_t H,
                          int64_t Nq, int64_t Nk, int64_t d, int64_t n_split, float scale,
                          void *stream);

/*
 * fa_decode_split_offset -- fa_decode_split for Nq new tokens that attend
 * causally: query row i sits at key position q_start + i and sees keys
 * 0 .. q_start + i only (q_start = Nk - Nq: the tokens are the last Nq keys
 * of the cache).  A split with no visible key for a row gives (-inf, 0, 0)
 * for that row; merging it changes nothing.
 * Source: flash_decode (attention_kernels.py) with the causal mask of
 * standard_attention at offset q_start.
 *   q_start  0 <= q_start <= 2^40.  Other arguments as fa_decode_split.
 */
fa_status fa_decode_split_offset(fa_dtype dt, const void *Q, const void *K, const void *V,
                                 float *part_m, float *part_l, float *part_o, int64_t B,
                                 int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t n_split,
                                 float scale, int64_t q_start, void *stream);

/*
 * fa_merge_states -- second pass: fold n_split states per row with the merge
 * rule and normalise.
 * Source: merge_states (attention_kernels.py): m = max(m_a, m_b); both sides
 * are rebased onto m (onto 0 when both are -inf, so empty merged with empty
 * stays empty); O = o / l, L = m + log l.
 *   part_m, part_l [B][H][Nq][n_split], part_o [B][H][Nq][n_split][d], fp32.
 *   O  output [B][H][Nq][d] with dtype dt (FA_BF16 or FA_F32).  L output fp32.
 *   Any 1 <= d <= 512.  A row whose states are all empty gets O = NaN and
 *   L = -inf (no key was seen).
 */
fa_status fa_merge_states(fa_dtype dt, const float *part_m, const float *part_l,
                          const float *part_o, void *O, float *L, int64_t B, int64_t H,
                          int64_t Nq, int64_t d, int64_t n_split, void *stream);

/* Human-readable name of a status code (static string). */
const char *fa_status_str(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
