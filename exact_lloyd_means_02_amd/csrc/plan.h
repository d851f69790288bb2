// Analytic tile plan for the gfx950 kernels (host only).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/flashkm.h"

namespace fkm {

// gfx950 resources the plan is derived from.
struct Gfx950 {
    static constexpr int cus = 256;
    static constexpr int simds_per_cu = 4;
    static constexpr int lds_bytes_per_cu = 160 * 1024;
    static constexpr int vgprs_per_lane = 512;       // arch + acc, per SIMD lane
    static constexpr int l2_bytes_per_xcd = 4 << 20;
    static constexpr int target_waves_per_simd = 2;  // lets one wave's compares overlap another's MFMA
};

// Kernel-side constants the plan and the launchers agree on.
constexpr int ASSIGN_WAVES = 4;          // waves per assign workgroup
constexpr int SPLITD_KB = 4;             // split-D: 32-centroid tiles per register group
constexpr int SORT_TILE = 4096;          // keys per sort workgroup (scatter: 8 waves x 8 rounds x 64)
constexpr int SORT_MAX_BITS = 10;        // <= 1024 bins per counting pass (LDS: 8 x bins x 2 B + 2 x bins x 4 B + 32 KiB tile)
constexpr int SORT_INLINE_TILES = 64;    // tiles per problem up to which every scatter workgroup reads the table
constexpr int SORT_MAX_TABLE = 1 << 24;  // bins x tiles entries per problem in one pass's table
constexpr int UPD_VPL_MAX = 4;           // 16-byte (or scalar) vectors per lane per row in the update

struct AssignCfg {
    int path;      // 0 small-D, 1 split-D
    int d_pad;
    int pb;        // point blocks per wave
    int tps;       // tiles per LDS stage (small-D)
    int bd;        // split-D chunk of D
    int block_n;
    int lds;
    int vgpr;
    int nsplit;    // workgroups per point tile, each scanning a share of the centroid stages
};

// Buffers of a K-split assign (AssignCfg::nsplit > 1): one 64-bit (score, index) key per point,
// all ones between launches, and the points' squared norms.
struct AssignSplit {
    int nsplit = 1;
    unsigned long long *packed = nullptr;
    float *xn = nullptr;
};

struct SortCfg {
    int bits, passes, ntiles, bins;
};

struct UpdCfg {
    int rows;      // sorted rows per wave chunk
    int vec;       // elements per vector
    int lanes;     // lanes per row (power of two)
    int groups;    // rows per step = 64 / lanes
    int vpl;       // vectors per lane per row within one column block
    int ncb;       // column blocks
    int cb_elems;  // elements per column block
    int64_t nch;   // chunks per problem
};

// Prepared centroids (assign layout) that an update refreshes from the new centroids, or
// all-null for no refresh.
struct UpdRefresh {
    void *cprep = nullptr;
    float *cnh = nullptr;
    int DP = 0, KT = 0;
    int zero_norm = 0;  // similarity metrics: refreshed norm terms are 0
};

// Memory of one update launch: each cluster's first sorted position [B][K] (from the arg-sort
// or the update's prologue), the arrival counters (zero on entry, left zero) and scratch for
// partial records and shift partials.
struct UpdMem {
    const int32_t *offs = nullptr;
    int32_t *ctr = nullptr;
    void *scratch = nullptr;
    // the batch size the update's chunk plan is made for (0: the launch's own); a launch over part
    // of a batch then chunks (and adds) each problem as the whole batch's launch would.  At least
    // the launch's problem count, so the chunks are no shorter and the counters and scratch sized
    // for the launch suffice.
    int64_t plan_B = 0;
};

AssignCfg plan_assign(int dt, int64_t B, int64_t N, int64_t D, int64_t K);
SortCfg plan_sort(int64_t N, int64_t K);
UpdCfg plan_update(int dt, int64_t B, int64_t N, int64_t D, int64_t K);

// Small-D register tile chosen for (dtype, padded D); shared with the kernel templates.
constexpr int small_d_pb(int dt, int dp) { return dt == 0 ? (dp <= 32 ? 2 : 1) : (dp <= 128 ? 2 : 1); }
// Tiles per LDS stage: 2 when a tile's 32 centroid rows span at least two 16-byte groups
// per lane half (D*s >= 64 bytes), else 4, so one stage is at least 4 KiB (one 16-byte copy
// per lane of every wave); 1 for rows of 512 bytes or more (fp32 D = 128, 2-byte D = 256),
// where one tile is 16 KiB and three such stages let three workgroups share a CU's LDS.
// Three stages rotate in LDS.
constexpr int small_d_tps(int dt, int dp) {
    return dp * (dt == 0 ? 4 : 2) >= 512 ? 1 : (dp * (dt == 0 ? 4 : 2) >= 64 ? 2 : 4);
}
constexpr int SMALL_D_STAGES = 3;
constexpr int splitd_bd(int dt) { return dt == 0 ? 16 : 32; }

// Largest D handled by the small-D path (x tile kept in registers).
constexpr int small_d_max(int dt) { return dt == 0 ? 128 : 256; }

// 32-centroid tiles per problem in the prepared layout: padded to whole LDS stages of the small-D
// kernel (small_d_tps tiles at the padded D), or to the split-D kernel's register group of
// SPLITD_KB tiles; padding tiles score +inf.  (A multiple of 4 for every D doubled the scan at
// K <= 64 where stages hold 2 tiles: 4 tiles for 2 of real centroids.)
inline int assign_tiles(int dt, int64_t D, int64_t K) {
    int mult = SPLITD_KB;
    if (D <= small_d_max(dt)) {
        int dp = dt == 0 ? 8 : 16;
        while (dp < D) dp <<= 1;
        mult = small_d_tps(dt, dp);
    }
    const int64_t t = (K + 31) / 32;
    return (int)((t + mult - 1) / mult * mult);
}

}  // namespace fkm
