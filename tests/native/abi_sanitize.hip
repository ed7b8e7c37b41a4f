// Host-only check of the C ABI's argument layer (fa_api.hip) under
// AddressSanitizer and UndefinedBehaviorSanitizer: the kernel launchers are
// replaced by stubs that record what they were asked to launch, so every
// entry point runs its checks and its dispatch on the CPU.  Valid calls must
// reach exactly one launcher with the caller's sizes and the workspace split
// into its two halves; invalid ones must return an error and launch nothing.
// Prints "ok" or the first failure.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "../../include/fa.h"
#include "../../flashattention_online_softmax_fa_amd/csrc/fa_internal.h"

namespace {
int g_launches = 0;
fa::BwdArgs g_bwd{};
fa::FwdArgs g_fwd{};
fa::DecodeArgs g_dec{};
fa::MergeArgs g_merge{};
}  // namespace

namespace fa {
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t) { ++g_launches; g_fwd = a; return hipSuccess; }
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t) { ++g_launches; g_fwd = a; return hipSuccess; }
hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t) { ++g_launches; g_bwd = a; return hipSuccess; }
hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t) { ++g_launches; g_bwd = a; return hipSuccess; }
hipError_t launch_decode_split_bf16(const DecodeArgs &a, hipStream_t) { ++g_launches; g_dec = a; return hipSuccess; }
hipError_t launch_decode_split_f32(const DecodeArgs &a, hipStream_t) { ++g_launches; g_dec = a; return hipSuccess; }
hipError_t launch_merge_states(const MergeArgs &a, hipStream_t) { ++g_launches; g_merge = a; return hipSuccess; }
}  // namespace fa

static int fails = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::printf("line %d: %s\n", __LINE__, #cond);                  \
            ++fails;                                                        \
        }                                                                   \
    } while (0)

int main() {
    // fake, 256-byte aligned addresses: nothing is dereferenced on the host
    void *P = (void *)(uintptr_t)0x10000000;
    float *Pf = (float *)P;
    const int64_t B = 2, H = 3, Nq = 100, Nk = 77;

    // forward: valid bf16 and fp32 calls reach one launcher each
    g_launches = 0;
    EXPECT(fa_fwd(FA_BF16, P, P, P, P, Pf, B, H, Nq, Nk, 64, 0.125f, 1, nullptr) == FA_OK);
    EXPECT(g_launches == 1 && g_fwd.B == B && g_fwd.Nq == Nq && g_fwd.Nk == Nk && g_fwd.causal == 1);
    EXPECT(fa_fwd_offset(FA_BF16, P, P, P, P, Pf, B, H, Nq, Nk, 128, 0.1f, 5, nullptr) == FA_OK);
    EXPECT(g_launches == 2 && g_fwd.q_start == 5);
    EXPECT(fa_fwd_blocked(FA_F32, P, P, P, P, Pf, B, H, Nq, Nk, 16, 0.25f, 0, 7, nullptr) == FA_OK);
    EXPECT(g_launches == 3 && g_fwd.kv_block == 7);
    // forward: rejected calls launch nothing
    EXPECT(fa_fwd(FA_BF16, nullptr, P, P, P, Pf, B, H, Nq, Nk, 64, 0.125f, 0, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(FA_BF16, (char *)P + 8, P, P, P, Pf, B, H, Nq, Nk, 64, 0.125f, 0, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(FA_BF16, P, P, P, P, Pf, B, H, Nq, Nk, 64, NAN, 0, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(FA_BF16, P, P, P, P, Pf, B, H, Nq, Nk, 96, 0.1f, 0, nullptr) == FA_ERR_UNSUPPORTED);
    EXPECT(fa_fwd(FA_BF16, P, P, P, P, Pf, INT64_MAX, H, Nq, Nk, 64, 0.1f, 0, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_offset(FA_BF16, P, P, P, P, Pf, B, H, Nq, Nk, 64, 0.1f, -1, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_blocked(FA_F32, P, P, P, P, Pf, B, H, Nq, Nk, 16, 0.1f, 0, 0, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(g_launches == 3);

    // backward: the workspace holds D then L * log2(e), each rounded up to 256 B
    const size_t ws = fa_bwd_workspace_size(FA_BF16, B, H, Nq, 64);
    EXPECT(ws == 2 * ((size_t)(B * H * Nq * 4 + 255) / 256 * 256));
    EXPECT(fa_bwd(FA_BF16, P, P, P, P, Pf, P, P, P, P, P, ws, B, H, Nq, Nk, 64, 0.125f, 1,
                  nullptr) == FA_OK);
    EXPECT(g_launches == 4 && (char *)g_bwd.D == (char *)P && (char *)g_bwd.L2 == (char *)P + ws / 2);
    EXPECT(fa_bwd_offset(FA_F32, P, P, P, P, Pf, P, P, P, P, P, ws, B, H, Nq, Nk, 32, 0.2f, 3,
                         nullptr) == FA_OK);
    EXPECT(g_launches == 5 && g_bwd.q_start == 3 && g_bwd.causal == 1);
    EXPECT(fa_bwd(FA_BF16, P, P, P, P, Pf, P, P, P, P, P, ws - 1, B, H, Nq, Nk, 64, 0.125f, 1,
                  nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_bwd(FA_BF16, P, P, P, P, Pf, P, P, P, P, (char *)P + 128, ws, B, H, Nq, Nk, 64,
                  0.125f, 1, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_bwd(FA_BF16, P, P, P, P, Pf, nullptr, P, P, P, P, ws, B, H, Nq, Nk, 64, 0.125f, 1,
                  nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(g_launches == 5);
    // the no-allocation backward rejects bad arguments and oversized calls
    // before it looks up its array (which needs a GPU, absent here)
    EXPECT(fa_bwd_noalloc(FA_BF16, P, P, P, P, Pf, P, nullptr, P, P, B, H, Nq, Nk, 64, 0.1f, 1,
                          nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_bwd_noalloc(FA_BF16, P, P, P, P, Pf, P, P, P, P, 1, 1, (1 << 21) + 1, Nk, 64, 0.1f,
                          1, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(g_launches == 5);

    // decoding and merge
    EXPECT(fa_decode_split(FA_BF16, P, P, P, Pf, Pf, Pf, B, H, 1, Nk, 128, 16, 0.1f, nullptr) == FA_OK);
    EXPECT(g_launches == 6 && g_dec.n_split == 16 && g_dec.causal == 0);
    EXPECT(fa_decode_split_offset(FA_F32, P, P, P, Pf, Pf, Pf, B, H, 4, Nk, 64, 3, 0.1f, 70,
                                  nullptr) == FA_OK);
    EXPECT(g_launches == 7 && g_dec.causal == 1 && g_dec.q_start == 70);
    EXPECT(fa_decode_split(FA_BF16, P, P, P, Pf, Pf, Pf, B, H, 1, Nk, 128, 0, 0.1f, nullptr) == FA_ERR_INVALID_ARG);
    EXPECT(fa_merge_states(FA_BF16, Pf, Pf, Pf, P, Pf, B, H, 1, 128, 16, nullptr) == FA_OK);
    EXPECT(g_launches == 8 && g_merge.rows == B * H && g_merge.out_bf16 == 1);
    EXPECT(fa_merge_states(FA_F32, Pf, Pf, Pf, P, Pf, B, H, 1, 513, 16, nullptr) == FA_ERR_UNSUPPORTED);
    EXPECT(g_launches == 8);
    EXPECT(fa_status_str((fa_status)7) != nullptr);

    if (fails) return 1;
    std::printf("ok\n");
    return 0;
}
