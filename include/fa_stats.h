/*
 * fa_stats.h -- event counters of the debug build libfa_stats.so.
 *
 * libfa_stats.so is libfa.so compiled with FA_STATS=1: the same entry points
 * (include/fa.h), whose bf16 forward and backward kernels also count the
 * events below into device-side counters, one atomic addition per wave when
 * it finishes.  The release library libfa.so exports none of these calls.
 *
 * Source: flash_forward and flash_backward (attention_kernels.py), which
 * record the same quantities in a stats dict:
 *   FA_STAT_FWD_TILES     (query block, key tile) pairs computed;
 *   FA_STAT_FWD_SKIPPED   pairs skipped under causal because the key tile
 *                         starts after the block's last query position;
 *   FA_STAT_FWD_RESCALES  (query row, key tile) pairs in which the running
 *                         maximum was raised and the accumulator rescaled (the
 *                         page counts every increase of the maximum; these
 *                         kernels raise it only when the tile maximum exceeds
 *                         it by more than 2^8 (tiles that need a mask) or a
 *                         lane's sum of the tile's probabilities exceeds 2^24
 *                         (the rest), so the count is at most the page's and
 *                         equals it when every increase is larger than 2^28);
 *   FA_STAT_BWD_KV_TILES  (key block, query tile) pairs computed by the
 *                         key-major dK/dV pass;
 *   FA_STAT_BWD_Q_TILES   (query block, key tile) pairs computed by the
 *                         query-major dQ pass;
 *   FA_STAT_DQ_ATOMIC_ADDS  dQ elements added atomically: always 0 here (dQ
 *                         is accumulated in registers by the query-major
 *                         pass, not with atomic additions).
 * A "block" is the rows (or keys) one wavefront owns; fa_stats_tile reports
 * its size and the key (or query) tile size, so that the counts can be
 * checked against the page's skip rule at the same shape.
 */
#ifndef FA_STATS_H
#define FA_STATS_H

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_stat {
    FA_STAT_FWD_TILES = 0,
    FA_STAT_FWD_SKIPPED = 1,
    FA_STAT_FWD_RESCALES = 2,
    FA_STAT_BWD_KV_TILES = 3,
    FA_STAT_BWD_Q_TILES = 4,
    FA_STAT_DQ_ATOMIC_ADDS = 5,
    FA_STAT_COUNT = 8 /* length of the counter array (two spare slots) */
} fa_stat;

/* Zero every counter.  Synchronous: waits for the current device. */
fa_status fa_stats_reset(void);

/* Copy the FA_STAT_COUNT counters into host memory `out` (caller-owned).
 * Synchronous: waits for all work on the current device first. */
fa_status fa_stats_read(uint64_t *out);

/* Block shapes of the counted kernels for (dt, d, causal):
 *   kind 0: forward       -> *rows = query rows per block, *cols = keys per tile;
 *   kind 1: dK/dV pass    -> *rows = keys per block, *cols = queries per tile;
 *   kind 2: dQ pass       -> *rows = query rows per block, *cols = keys per tile;
 *   kind 3: forward       -> *rows = query rows per workgroup (the query tile
 *                            that streams K and V once), *cols = keys per tile.
 * FA_ERR_INVALID_ARG for another kind; FA_ERR_UNSUPPORTED unless dt = FA_BF16
 * and d in {64, 128}. */
fa_status fa_stats_tile(int kind, fa_dtype dt, int64_t d, int causal, int64_t *rows,
                        int64_t *cols);

#ifdef __cplusplus
}
#endif

#endif /* FA_STATS_H */
