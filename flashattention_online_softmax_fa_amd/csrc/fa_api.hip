// fa_api.hip -- the C ABI (include/fa.h): argument checks, then one launcher
// per call.  Nothing is enqueued unless every check passes.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/fa.h"
#include "../../include/fa_stats.h"
#include "fa_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return p != nullptr && ((uintptr_t)p % a) == 0; }

// All sizes >= 1 and every element count used below fits comfortably in int64.
bool sizes_ok(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return false;
    int64_t bh, x;
    if (__builtin_mul_overflow(B, H, &bh)) return false;
    const int64_t n = Nq > Nk ? Nq : Nk;
    if (__builtin_mul_overflow(bh, n, &x)) return false;
    if (__builtin_mul_overflow(x, d, &x)) return false;
    return x < (int64_t(1) << 60);
}

size_t elem_size(fa_dtype dt) { return dt == FA_BF16 ? 2 : 4; }

bool dtype_ok(fa_dtype dt) { return dt == FA_F32 || dt == FA_BF16; }

constexpr int64_t kMaxGrid = 2147483647;

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Largest accepted query offset of the causal mask; keeps q_start + Nq far
// from int64 overflow in the kernels' tile arithmetic.
constexpr int64_t kMaxQStart = int64_t(1) << 40;

fa_status fwd_common(fa_dtype dt, const void *Q, const void *K, const void *V, void *O, float *L,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                     int causal, int64_t q_start, int64_t kv_block, void *stream) {
    if (!dtype_ok(dt)) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, Nq, Nk, d)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (q_start < 0 || q_start > kMaxQStart) return FA_ERR_INVALID_ARG;
    const uintptr_t al = dt == FA_BF16 ? 16 : 4;
    if (!aligned(Q, al) || !aligned(K, al) || !aligned(V, al) || !aligned(O, al) ||
        !aligned(L, 4))
        return FA_ERR_INVALID_ARG;
    fa::FwdArgs a{Q, K, V, O, L, B, H, Nq, Nk, d, scale, causal, kv_block, q_start};
    if (dt == FA_F32) {
        if (d > 128) return FA_ERR_UNSUPPORTED;
        if ((B * H * Nq + 3) / 4 > kMaxGrid) return FA_ERR_UNSUPPORTED;
        return hip_status(fa::launch_fwd_f32(a, (hipStream_t)stream));
    }
    if (kv_block != 0) return FA_ERR_UNSUPPORTED;  // the bf16 path has fixed tiles
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (B * H * ((Nq + 63) / 64) > kMaxGrid) return FA_ERR_UNSUPPORTED;
    return hip_status(fa::launch_fwd_bf16(a, (hipStream_t)stream));
}

fa_status bwd_common(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                     const float *L, const void *dO, void *dQ, void *dK, void *dV,
                     void *workspace, size_t ws_bytes, int64_t B, int64_t H, int64_t Nq,
                     int64_t Nk, int64_t d, float scale, int causal, int64_t q_start,
                     void *stream);

fa_status bwd_noalloc_common(fa_dtype dt, const void *Q, const void *K, const void *V,
                             const void *O, const float *L, const void *dO, void *dQ, void *dK,
                             void *dV, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                             float scale, int causal, void *stream);

fa_status decode_common(fa_dtype dt, const void *Q, const void *K, const void *V, float *part_m,
                        float *part_l, float *part_o, int64_t B, int64_t H, int64_t Nq,
                        int64_t Nk, int64_t d, int64_t n_split, float scale, int causal,
                        int64_t q_start, void *stream) {
    if (!dtype_ok(dt)) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, Nq, Nk, d)) return FA_ERR_INVALID_ARG;
    if (n_split < 1 || n_split > (int64_t(1) << 20)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (q_start < 0 || q_start > kMaxQStart) return FA_ERR_INVALID_ARG;
    const uintptr_t al = dt == FA_BF16 ? 16 : 4;
    if (!aligned(Q, al) || !aligned(K, al) || !aligned(V, al) || !aligned(part_m, 4) ||
        !aligned(part_l, 4) || !aligned(part_o, 4))
        return FA_ERR_INVALID_ARG;
    if (B * H * Nq > kMaxGrid / n_split) return FA_ERR_UNSUPPORTED;
    fa::DecodeArgs a{Q, K, V, part_m, part_l, part_o, B, H, Nq, Nk, d, n_split, scale, causal,
                     q_start};
    if (dt == FA_F32) {
        if (d > 128) return FA_ERR_UNSUPPORTED;
        return hip_status(fa::launch_decode_split_f32(a, (hipStream_t)stream));
    }
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    return hip_status(fa::launch_decode_split_bf16(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

fa_status fa_fwd(fa_dtype dt, const void *Q, const void *K, const void *V, void *O, float *L,
                 int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                 int causal, void *stream) {
    return fwd_common(dt, Q, K, V, O, L, B, H, Nq, Nk, d, scale, causal, 0, 0, stream);
}

fa_status fa_fwd_offset(fa_dtype dt, const void *Q, const void *K, const void *V, void *O,
                        float *L, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                        float scale, int64_t q_start, void *stream) {
    return fwd_common(dt, Q, K, V, O, L, B, H, Nq, Nk, d, scale, 1, q_start, 0, stream);
}

fa_status fa_fwd_blocked(fa_dtype dt, const void *Q, const void *K, const void *V, void *O,
                         float *L, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                         float scale, int causal, int64_t kv_block, void *stream) {
    if (dt != FA_F32) return dt == FA_BF16 ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG;
    if (kv_block < 1 || kv_block > 256) return FA_ERR_INVALID_ARG;
    return fwd_common(dt, Q, K, V, O, L, B, H, Nq, Nk, d, scale, causal, 0, kv_block, stream);
}

size_t fa_bwd_workspace_size(fa_dtype dt, int64_t B, int64_t H, int64_t Nq, int64_t d) {
    if (!dtype_ok(dt) || !sizes_ok(B, H, Nq, 1, d)) return 0;
    (void)d;
    const size_t rows = (size_t)(B * H * Nq);
    return 2 * ((rows * 4 + 255) / 256 * 256);
}

fa_status fa_bwd(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                 const float *L, const void *dO, void *dQ, void *dK, void *dV, void *workspace,
                 size_t ws_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                 float scale, int causal, void *stream) {
    return bwd_common(dt, Q, K, V, O, L, dO, dQ, dK, dV, workspace, ws_bytes, B, H, Nq, Nk, d,
                      scale, causal, 0, stream);
}

fa_status fa_bwd_offset(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                        const float *L, const void *dO, void *dQ, void *dK, void *dV,
                        void *workspace, size_t ws_bytes, int64_t B, int64_t H, int64_t Nq,
                        int64_t Nk, int64_t d, float scale, int64_t q_start, void *stream) {
    return bwd_common(dt, Q, K, V, O, L, dO, dQ, dK, dV, workspace, ws_bytes, B, H, Nq, Nk, d,
                      scale, 1, q_start, stream);
}

fa_status fa_bwd_noalloc(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                         const float *L, const void *dO, void *dQ, void *dK, void *dV, int64_t B,
                         int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                         void *stream) {
    return bwd_noalloc_common(dt, Q, K, V, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal,
                              stream);
}

}  // extern "C"

namespace {

// Every check of a backward call that does not involve the workspace; no HIP
// call is made.
fa_status bwd_check(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                    const float *L, const void *dO, void *dQ, void *dK, void *dV, int64_t B,
                    int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                    int64_t q_start) {
    if (!dtype_ok(dt)) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, Nq, Nk, d)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (q_start < 0 || q_start > kMaxQStart) return FA_ERR_INVALID_ARG;
    const uintptr_t al = dt == FA_BF16 ? 16 : 4;
    if (!aligned(Q, al) || !aligned(K, al) || !aligned(V, al) || !aligned(O, al) ||
        !aligned(dO, al) || !aligned(dQ, al) || !aligned(dK, al) || !aligned(dV, al) ||
        !aligned(L, 4))
        return FA_ERR_INVALID_ARG;
    if (dt == FA_F32) {
        if (d > 128) return FA_ERR_UNSUPPORTED;
        if ((B * H * Nq + 3) / 4 > kMaxGrid || (B * H * Nk + 3) / 4 > kMaxGrid)
            return FA_ERR_UNSUPPORTED;
        return FA_OK;
    }
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (B * H * ((Nk + 63) / 64) > kMaxGrid || B * H * ((Nq + 63) / 64) > kMaxGrid)
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// Checked arguments and a workspace of fa_bwd_workspace_size() bytes at
// `workspace`: enqueue the backward.
fa_status bwd_launch(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                     const float *L, const void *dO, void *dQ, void *dK, void *dV,
                     void *workspace, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                     float scale, int causal, int64_t q_start, void *stream) {
    const size_t half = fa_bwd_workspace_size(dt, B, H, Nq, d) / 2;
    fa::BwdArgs a{Q,  K,  V,  O,  dO, L,  dQ, dK, dV, (float *)workspace,
                  (float *)((char *)workspace + half), B, H, Nq, Nk, d, scale, causal, q_start};
    if (dt == FA_F32) return hip_status(fa::launch_bwd_f32(a, (hipStream_t)stream));
    return hip_status(fa::launch_bwd_bf16(a, (hipStream_t)stream));
}

fa_status bwd_common(fa_dtype dt, const void *Q, const void *K, const void *V, const void *O,
                     const float *L, const void *dO, void *dQ, void *dK, void *dV,
                     void *workspace, size_t ws_bytes, int64_t B, int64_t H, int64_t Nq,
                     int64_t Nk, int64_t d, float scale, int causal, int64_t q_start,
                     void *stream) {
    const fa_status st = bwd_check(dt, Q, K, V, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d, scale,
                                   causal, q_start);
    if (st != FA_OK) return st;
    if (!aligned(workspace, 256)) return FA_ERR_INVALID_ARG;
    if (ws_bytes < fa_bwd_workspace_size(dt, B, H, Nq, d)) return FA_ERR_INVALID_ARG;
    return bwd_launch(dt, Q, K, V, O, L, dO, dQ, dK, dV, workspace, B, H, Nq, Nk, d, scale,
                      causal, q_start, stream);
}

}  // namespace

// ---------------------------------------------------------------------------
// The backward's workspace (D and L * log2(e), 8 bytes per query row) in a
// fixed array of device memory, for fa_bwd_noalloc.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` only
// names the variable: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch; only
// that address is ever passed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

fa_status scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return FA_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FA_OK;
}

fa_status bwd_noalloc_common(fa_dtype dt, const void *Q, const void *K, const void *V,
                             const void *O, const float *L, const void *dO, void *dQ, void *dK,
                             void *dV, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                             float scale, int causal, void *stream) {
    fa_status st = bwd_check(dt, Q, K, V, O, L, dO, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal,
                             0);
    if (st != FA_OK) return st;
    if (fa_bwd_workspace_size(dt, B, H, Nq, d) > (size_t)FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_INVALID_ARG;
    void *ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != FA_OK) return st;
    return bwd_launch(dt, Q, K, V, O, L, dO, dQ, dK, dV, ws, B, H, Nq, Nk, d, scale, causal, 0,
                      stream);
}

}  // namespace

extern "C" {

fa_status fa_decode_split(fa_dtype dt, const void *Q, const void *K, const void *V,
                          float *part_m, float *part_l, float *part_o, int64_t B, int64_t H,
                          int64_t Nq, int64_t Nk, int64_t d, int64_t n_split, float scale,
                          void *stream) {
    return decode_common(dt, Q, K, V, part_m, part_l, part_o, B, H, Nq, Nk, d, n_split, scale, 0,
                         0, stream);
}

fa_status fa_decode_split_offset(fa_dtype dt, const void *Q, const void *K, const void *V,
                                 float *part_m, float *part_l, float *part_o, int64_t B,
                                 int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t n_split,
                                 float scale, int64_t q_start, void *stream) {
    return decode_common(dt, Q, K, V, part_m, part_l, part_o, B, H, Nq, Nk, d, n_split, scale, 1,
                         q_start, stream);
}

fa_status fa_merge_states(fa_dtype dt, const float *part_m, const float *part_l,
                          const float *part_o, void *O, float *L, int64_t B, int64_t H,
                          int64_t Nq, int64_t d, int64_t n_split, void *stream) {
    if (!dtype_ok(dt)) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, Nq, 1, d)) return FA_ERR_INVALID_ARG;
    if (n_split < 1 || n_split > (int64_t(1) << 20)) return FA_ERR_INVALID_ARG;
    if (!aligned(part_m, 4) || !aligned(part_l, 4) || !aligned(part_o, 4) ||
        !aligned(O, elem_size(dt)) || !aligned(L, 4))
        return FA_ERR_INVALID_ARG;
    if (d > 512) return FA_ERR_UNSUPPORTED;
    if (B * H * Nq > kMaxGrid) return FA_ERR_UNSUPPORTED;
    fa::MergeArgs a{part_m, part_l, part_o, O, L, B * H * Nq, d, n_split, dt == FA_BF16};
    return hip_status(fa::launch_merge_states(a, (hipStream_t)stream));
}

#if FA_STATS
fa_status fa_stats_reset(void) {
    if (hipDeviceSynchronize() != hipSuccess) return FA_ERR_HIP;
    if (fa::stats_fwd(nullptr, true) != hipSuccess || fa::stats_bwd(nullptr, true) != hipSuccess)
        return FA_ERR_HIP;
    return FA_OK;
}

fa_status fa_stats_read(uint64_t *out) {
    if (out == nullptr) return FA_ERR_INVALID_ARG;
    if (hipDeviceSynchronize() != hipSuccess) return FA_ERR_HIP;
    unsigned long long f[fa::kStatCount], b[fa::kStatCount];
    if (fa::stats_fwd(f, false) != hipSuccess || fa::stats_bwd(b, false) != hipSuccess)
        return FA_ERR_HIP;
    for (int i = 0; i < fa::kStatCount; ++i) out[i] = f[i] + b[i];
    return FA_OK;
}

fa_status fa_stats_tile(int kind, fa_dtype dt, int64_t d, int causal, int64_t *rows,
                        int64_t *cols) {
    if (rows == nullptr || cols == nullptr || kind < 0 || kind > 3) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (dt != FA_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    if (kind == 0 || kind == 3) {
        fa::fwd_bf16_tile(d, kind == 3, rows, cols);
    } else {
        int64_t kr, kc, qr, qc;
        fa::bwd_bf16_tiles(d, causal, &kr, &kc, &qr, &qc);
        *rows = kind == 1 ? kr : qr;
        *cols = kind == 1 ? kc : qc;
    }
    return FA_OK;
}
#endif

const char *fa_status_str(fa_status s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        default: break;
    }
    return "FA_ERR_UNKNOWN";
}

}  // extern "C"
