// Analytic tile plan (paper summary, "Key claims": a cache-aware heuristic picks the kernel
// configuration from on-chip sizes and (N, K, D, B) instead of an exhaustive autotune).
//
// Everything here is arithmetic on gfx950 resource sizes; nothing is timed.
//
// Assign, small-D path (x tile kept in VGPRs for the whole centroid scan):
//   * D is padded to DP in {16,...,512} (2-byte types) or {8,...,256} (fp32): the MFMA k-step
//     is 16 (bf16/fp16 32x32x16) or 2 (fp32 32x32x2), and each lane holds half of every row.
//   * VGPRs per lane ~= PB * (x: DP*s/8 + accumulators 16 + best 16) + fragment ring (<= 8)
//     + ~24 (the tile's norms load into an accumulator set).  PB (32-point blocks per wave)
//     is 2 up to 256-byte rows, else 1: at most 168 registers, so three waves share a SIMD and
//     the fold of one wave runs beside the MFMAs of the others.
//   * Centroid stages of 2 tiles (4 for D*s < 64 B, 1 for D*s >= 512 B) rotate through three
//     LDS buffers, filled by direct global->LDS copies two stages ahead of use: ~49 KiB per
//     workgroup, so three workgroups (12 waves) fit a CU's 160 KiB.
//   * Every workgroup re-reads all K centroids from L2: the arithmetic intensity of that
//     stream is 2*block_n*D FLOP per D*s bytes = block_n FLOP/B (bf16), >= 128 for
//     block_n >= 128, above what L2 must feed MFMA (~2.5 PF / ~40 TB/s ~= 64 FLOP/B).
//   * Workgroups of one problem are mapped onto one XCD so its centroids (K*D*s bytes,
//     256 KiB at K=1024, D=128, bf16) stay in that XCD's 4 MiB L2.
//   * The grid must fill the chip: three workgroups per CU (the VGPR budget above) is 768
//     workgroup slots.  When B * ceil(N / block_n) falls short of them, the centroid tiles are
//     split over nsplit workgroups per point tile, each scanning a contiguous share; their
//     picks merge through a 64-bit atomic minimum of (score, index) keys, and a small kernel
//     writes the labels.  A workgroup has a fixed cost of about six tiles' worth of time (point
//     tile load, pipeline fill, epilogue: measured from the efficiency at 32 and at 128 tiles
//     per workgroup), and the merge adds a launch, so a share keeps at least 32 tiles (1024
//     centroids): below that the fixed costs eat the gain.  Within that floor the split goes as
//     far as it can (at most 8): shorter shares also shorten the tail of the last round.
// Assign, split-D path (D above the register budget, README "Large-D and dtype support"):
//   * point block of 128 (4 waves x 32), 4 centroid tiles (128 centroids) of accumulators per
//     wave, D streamed through LDS in chunks of 32 (2-byte) / 16 (fp32) elements so one stage
//     of x chunk + centroid chunk is 16 KiB, double buffered: 32 KiB of LDS and at most 168
//     registers, so three waves share a SIMD (chunks twice as wide held 64 KiB and 178 registers,
//     two waves per SIMD, and ran 2% slower at D = 1024 fp32).
// Arg-sort: counting passes over digits of the cluster id; one pass when the per-problem
//   table (bins x tiles of 4096 keys) stays <= 2^24 entries and bins <= 1024 (LDS of a scatter
//   workgroup: 8 waves x bins 16-bit counters, 2 x bins offsets, the 32 KiB staged tile); otherwise
//   balanced multi-pass LSD digits.
// Update: rows are gathered with 16-byte vector loads when D allows; a row is covered by a
//   power-of-two number of lanes so one wave load instruction moves 64 x 16 B from 64/lanes
//   rows; each wave takes `rows` consecutive sorted positions, sized so ~8 waves per SIMD
//   are in flight over the whole launch.
#include "plan.h"

#include <stdlib.h>

#include <algorithm>

namespace fkm {

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int pow2_ceil(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

static int log2_floor(int64_t v) {
    int r = -1;
    while (v > 0) { v >>= 1; ++r; }
    return r;
}

// FLASHKM_ASSIGN_SPLIT=n (n >= 1) replaces the planned split of the small-D assign (a measuring
// knob for comparing the plan with other splits; any n gives the same results).
static int split_override() {
    const char *e = getenv("FLASHKM_ASSIGN_SPLIT");
    return e ? atoi(e) : 0;
}

AssignCfg plan_assign(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    AssignCfg c{};
    c.nsplit = 1;
    const int s = dt == 0 ? 4 : 2;
    const int dmin = dt == 0 ? 8 : 16;
    if (D <= small_d_max(dt)) {
        int dp = dmin;
        while (dp < D) dp <<= 1;
        c.path = 0;
        c.d_pad = dp;
        c.pb = small_d_pb(dt, dp);
        c.tps = small_d_tps(dt, dp);
        c.bd = 0;
        c.block_n = ASSIGN_WAVES * c.pb * 32;
        c.lds = SMALL_D_STAGES * (c.tps * 32 * dp * s + c.tps * 32 * 4) + ASSIGN_WAVES * 8;
        // per point block: x (dp*s/8), accumulators (16), best tile copy (16); then the fragment
        // ring (at most 2 groups of 4) and addressing / fold temporaries (~24)
        const int qg = dp * s / 32;
        c.vgpr = c.pb * (dp * s / 8 + 32) + (qg >= 4 ? 2 : qg) * 4 + 24;
        const int64_t slots = (int64_t)Gfx950::cus * 3;
        const int64_t wgs = B * cdiv(N, c.block_n);
        const int KT = assign_tiles(dt, D, K);
        const int nst = KT / c.tps;
        int ns = 1;
        if (wgs < slots) ns = std::max(1, std::min(8, KT / 32));
        if (split_override() > 0) ns = std::max(1, std::min(split_override(), nst));
        c.nsplit = ns;
    } else {
        const int bd = splitd_bd(dt);
        c.path = 1;
        c.d_pad = (int)((D + bd - 1) / bd * bd);
        c.pb = 1;
        c.tps = SPLITD_KB;
        c.bd = bd;
        c.block_n = ASSIGN_WAVES * 32;
        c.lds = 2 * (c.block_n * bd * s + SPLITD_KB * 32 * bd * s) + SPLITD_KB * 32 * 4;
        c.vgpr = SPLITD_KB * 16 + 16 + 32 + 16 + 48;
    }
    return c;
}

SortCfg plan_sort(int64_t N, int64_t K) {
    SortCfg c{};
    const int kbits = std::max(1, log2_floor(std::max<int64_t>(1, K - 1)) + 1);
    c.ntiles = (int)cdiv(N, SORT_TILE);
    int bmax = log2_floor(std::max<int64_t>(1, SORT_MAX_TABLE / c.ntiles));
    bmax = std::max(1, std::min(SORT_MAX_BITS, bmax));
    c.passes = (kbits + bmax - 1) / bmax;
    c.bits = (kbits + c.passes - 1) / c.passes;
    c.bins = 1 << c.bits;
    return c;
}

UpdCfg plan_update(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    UpdCfg c{};
    const int s = dt == 0 ? 4 : 2;
    const int v16 = 16 / s;
    c.vec = (D % v16 == 0) ? v16 : 1;
    const int64_t nvec = D / c.vec;
    c.lanes = std::min(64, pow2_ceil(nvec));
    c.groups = 64 / c.lanes;
    const int64_t vpl_all = cdiv(nvec, c.lanes);
    c.vpl = (int)std::min<int64_t>(UPD_VPL_MAX, pow2_ceil(vpl_all));
    c.cb_elems = c.lanes * c.vpl * c.vec;
    c.ncb = (int)cdiv(D, c.cb_elems);
    // About 4 waves per SIMD over the whole launch, which at the kernel's occupancy (6 waves per
    // SIMD at 2-byte D = 128) runs in one round: fewer, longer chunks amortise each wave's start (its
    // id window and the ids at its chunk edges) and its edge work.  Rounded to the nearest power of
    // two.  Measured update times against the chunk length (MI355X): B=32 N=65536 K=1024, 101 us at
    // 512 rows against 110 at 256 (8 waves per SIMD), 109 at 768 and 112 at 1024; B=32 N=75600
    // K=1000, 125 us at 512 against 141 at 1024; one 2^24-point problem, K=64, 747 us at 4096 against
    // 778 at 2048.
    const int64_t target_waves = (int64_t)Gfx950::cus * Gfx950::simds_per_cu * 4;
    int64_t rows = (B * N) / std::max<int64_t>(1, target_waves / c.ncb);
    rows = std::max<int64_t>(64, std::min<int64_t>(4096, rows));
    int64_t p2 = pow2_ceil(rows);
    if (p2 - rows > rows - p2 / 2) p2 /= 2;
    // A chunk between a quarter of the mean segment (N / K) and twice it: the wave that owns a
    // segment cut by its chunk's end walks on to the segment's end, up to a segment's length past
    // its chunk, which unbalances the waves; such chunks are halved (one 2^24-point problem with
    // K = 4096: 811 us at 2048 rows, 852 at 4096).
    const int64_t mean_seg = N / std::max<int64_t>(1, K);
    if (p2 > mean_seg / 4 && p2 <= 2 * mean_seg) p2 = std::max<int64_t>(64, p2 / 2);
    c.rows = (int)p2;
    c.nch = cdiv(N, c.rows);
    return c;
}

}  // namespace fkm
