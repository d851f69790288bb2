// FlashAssign on gfx950: centroid preparation, small-D and split-D assign kernels.
//
// Method (paper summary, "Method"; paper digest, "核心方法" and "方法步骤详情" step (1)):
// points are tiled, centroids are scanned tile by tile, each tile's block of scores is
// computed on chip and folded into a running (min, index) per point; the N x K matrix of
// distances is never written.  The decomposition ||x-c||^2 = ||x||^2 + ||c||^2 - 2 x.c
// (paper digest, "核心方法") means the arg-min only needs ||c||^2 - 2 x.c.
//
// gfx950 mapping:
//   * v_mfma_f32_32x32x16_{bf16,f16} (fp32: v_mfma_f32_32x32x2_f32).  Operand A = 32
//     centroids, operand B = 32 points, so each lane's 16 accumulators hold 16 centroid
//     scores of ONE point: the arg-min runs inside the lane, with one cross-lane merge per
//     point at the very end.
//   * Scores are halved: the accumulator starts at ||c~||^2/2 and A holds -c~ (negation is
//     exact), so acc = ||c~||^2/2 - x.c~ = (||c~||^2 - 2 x.c~)/2 with no add per score and
//     no risk of overflowing -2c~ in fp16.  Halving commutes with rounding, so comparisons
//     are those of the full scores.
//   * Per 32-centroid tile and lane: one min over the 16 scores (eight 3-input minima), one
//     compare with the running min, and a copy of the tile's 16 scores when it improves
//     (eight 64-bit moves under the mask of improving lanes).  The slot
//     inside the winning tile is found once at the end by equality with the running min.
//     Result: the exact arg-min of the fp32 scores with ties to the lowest index (strict
//     '<' over tiles in increasing order, lowest slot, lexicographic lane merge).
//   * Centroid tiles are pre-laid-out in "MFMA-fragment" order (see prep kernel) so a stage
//     is one contiguous copy and each A fragment is one conflict-free 16-byte LDS read per
//     lane; stages rotate through three LDS buffers, filled by direct global->LDS copies
//     (buffer loads into LDS, addressed from scalar registers) two stages ahead of their use.
#include "common.h"
#include "plan.h"

namespace fkm {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Clock stamps of the assign kernels' phases, for the phase probe (probe_assign_clock.hip, which
// defines FKM_CLOCK_STAMPS); compiled out of the library.  Thread 0 of workgroup w writes
// fkm_stamps[w]: [0] start, [1] scan start (point tile and first stages in; split-D: the first
// chunk pair in), [2] scan end, [3] end (shader clock, s_memtime), [4] start and [5] end (the
// 100 MHz real-time counter), [6] the HW_ID hardware register at the start (which CU of the XCD,
// SIMD and wave slot thread 0 runs on).
#ifdef FKM_CLOCK_STAMPS
constexpr int FKM_STAMP_WGS = 1 << 14;
__device__ unsigned long long fkm_stamps[FKM_STAMP_WGS][8];
#define FKM_STAMP(i)                                                                      \
    do {                                                                                  \
        if (threadIdx.x == 0 && blockIdx.x < (unsigned)FKM_STAMP_WGS)                     \
            fkm_stamps[blockIdx.x][i] = __builtin_amdgcn_s_memtime();                      \
    } while (0)
#define FKM_RSTAMP(i)                                                                     \
    do {                                                                                  \
        if (threadIdx.x == 0 && blockIdx.x < (unsigned)FKM_STAMP_WGS)                     \
            fkm_stamps[blockIdx.x][i] = __builtin_amdgcn_s_memrealtime();                  \
    } while (0)
// hwreg(HW_REG_HW_ID = 4, offset 0, 32 bits)
#define FKM_HWSTAMP(i)                                                                    \
    do {                                                                                  \
        if (threadIdx.x == 0 && blockIdx.x < (unsigned)FKM_STAMP_WGS)                     \
            fkm_stamps[blockIdx.x][i] = (unsigned)__builtin_amdgcn_s_getreg(4 | (31 << 11)); \
    } while (0)
#else
#define FKM_STAMP(i) \
    do {             \
    } while (0)
#define FKM_RSTAMP(i) \
    do {              \
    } while (0)
#define FKM_HWSTAMP(i) \
    do {               \
    } while (0)
#endif

// ------------------------------------------------------------------------------------------
// Centroid preparation.
//   cprep (per problem, tile t of 32 centroids, group q < DP/(2*VW), lane l = i + 32h):
//     16 bytes = -c~[32t+i][(2q+h)*VW + e], e < VW  (VW = 8 for 2-byte types, 4 for fp32)
//   The contraction index is split so that the two lane halves (h) of one MFMA step hold
//   adjacent 16-byte pieces of a row: the point rows are then read 32 contiguous bytes at a
//   time (the same map is used for x, and only its consistency between A and B matters).
//   cnh[b][k] = ||c~_k||^2 / 2 in fp32 (+inf for the padding rows k >= K)
// c~ = dtype(c) with round-to-nearest-even.  Zero padding for d >= D and k >= K.
// ------------------------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void prep_centroids_kernel(const float *__restrict__ C, u32x4 *__restrict__ cprep,
                                                             float *__restrict__ cnh, int K, int D, int DP,
                                                             int KT, int zero_norm) {
    constexpr int S = DT == DT_F32 ? 4 : 2;
    constexpr int VW = 16 / S;
    const int QG = DP / (2 * VW);
    const int bt = blockIdx.x;  // b * KT + t
    const int b = bt / KT, t = bt - b * KT;
    const int i = threadIdx.x >> 3, part = threadIdx.x & 7;
    const int k = t * 32 + i;
    const bool valid_k = k < K;
    const float *row = C + ((size_t)b * K + (valid_k ? k : 0)) * D;
    float ss = 0.f;
    const int groups = DP / VW;
    for (int g = part; g < groups; g += 8) {
        const int d0 = g * VW;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            const int d = d0 + e;
            float v = (valid_k && d < D) ? row[d] : 0.f;
            uint32_t bits;
            float r;
            if constexpr (DT == DT_F32) {
                r = v;
                bits = __float_as_uint(-r);
            } else if constexpr (DT == DT_F16) {
                const uint32_t hb = f32_to_f16_bits(v);
                r = f16_bits_to_f32(hb);
                bits = hb ^ 0x8000u;  // exact negation
            } else {
                const uint32_t bb = f32_to_bf16_bits(v);
                r = bf16_bits_to_f32(bb);
                bits = bb ^ 0x8000u;
            }
            ss += r * r;
            if constexpr (S == 4) {
                w[e] = bits;
            } else {
                w[e >> 1] |= (bits & 0xFFFFu) << ((e & 1) * 16);
            }
        }
        const int h = (d0 / VW) & 1;
        const int q = d0 / (2 * VW);
        const size_t off = (((size_t)b * KT + t) * QG + q) * 64 + i + 32 * h;
        cprep[off] = u32x4{w[0], w[1], w[2], w[3]};
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    if (part == 0) cnh[(size_t)b * KT * 32 + k] = valid_k ? (zero_norm ? 0.f : 0.5f * ss) : __builtin_inff();
}

// ------------------------------------------------------------------------------------------
// shared pieces of the assign kernels
// ------------------------------------------------------------------------------------------
// One 16-byte group of a point row: elements d0 .. d0+VW-1 (zeros past D or past N).
template <int DT>
__device__ inline u32x4 load_x_group(const void *x, size_t row_elem0, int d0, int D, bool valid_pt) {
    constexpr int S = DT == DT_F32 ? 4 : 2;
    constexpr int VW = 16 / S;
    if (!valid_pt || d0 >= D) return u32x4{0u, 0u, 0u, 0u};
    if ((D % VW) == 0) {
        return *(const u32x4 *)((const char *)x + (row_elem0 + d0) * S);
    }
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < VW; ++e) {
        const int d = d0 + e;
        if (d < D) {
            if constexpr (S == 4) {
                w[e] = ((const uint32_t *)x)[row_elem0 + d];
            } else {
                w[e >> 1] |= (uint32_t)((const uint16_t *)x)[row_elem0 + d] << ((e & 1) * 16);
            }
        }
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Raw buffer descriptor over `bytes` bytes at `base` (fourth word: 32-bit data format, the
// value gfx9-family parts expect for untyped loads).  Built in scalar registers.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Copy 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): lane l
// reads the buffer at byte voff + soff (voff per lane, soff wave-uniform) and the wave's 64
// lanes fill the 1 KiB at `lds` (wave-uniform), lane l at bytes [16 l, 16 l + 16).  The
// buffer form keeps all address arithmetic in scalar registers.
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// acc += A(32 centroids) x B(32 points) over one 16-byte group per lane.
template <int DT>
__device__ inline f32x16 mfma_group(const u32x4 &a, const u32x4 &bx, f32x16 acc) {
    if constexpr (DT == DT_BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bx),
                                                       acc, 0, 0, 0);
    } else if constexpr (DT == DT_F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, bx),
                                                      acc, 0, 0, 0);
    } else {
        const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, bx);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[0], bf[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[1], bf[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[2], bf[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[3], bf[3], acc, 0, 0, 0);
        return acc;
    }
}

// acc + a.lo^2 + a.hi^2 for a word holding two 2-byte values (v_dot2_f32_{bf16,f16}).
template <int DT>
__device__ inline float dot2_self(uint32_t w, float acc) {
    if constexpr (DT == DT_BF16) {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w), __builtin_bit_cast(b2, w), acc, false);
    } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), __builtin_bit_cast(h2, w), acc, false);
    }
}

// Running arg-min state of one lane for one 32-point block.
struct ArgminState {
    float run_min;
    int run_tile;
    f32x16 best;
};

__device__ inline void argmin_init(ArgminState &s) {
    s.run_min = __builtin_inff();
    s.run_tile = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s.best[r] = __builtin_inff();
}

// Fold one tile's 16 scores (this lane's rows of the tile) into the running state.
__device__ inline void argmin_fold(ArgminState &s, const f32x16 &acc, int tile) {
    // eight three-input minima: five over triples, two over their results and the last
    // score, one over those two
    const float t0 = fminf(fminf(acc[0], acc[1]), acc[2]), t1 = fminf(fminf(acc[3], acc[4]), acc[5]);
    const float t2 = fminf(fminf(acc[6], acc[7]), acc[8]), t3 = fminf(fminf(acc[9], acc[10]), acc[11]);
    const float t4 = fminf(fminf(acc[12], acc[13]), acc[14]);
    const float u0 = fminf(fminf(t0, t1), t2), u1 = fminf(fminf(t3, t4), acc[15]);
    const float m = fminf(u0, u1);
    const bool imp = m < s.run_min;
    s.run_min = imp ? m : s.run_min;
    s.run_tile = imp ? tile : s.run_tile;
    // copy the tile's scores where the lane improved: eight 64-bit moves under the lane mask
    // (instead of sixteen selects).  Every accumulator register was already read by the
    // minima above, so the MFMA results are complete here.
    typedef unsigned long long u64x8 __attribute__((ext_vector_type(8)));
    const unsigned long long mask = __builtin_amdgcn_ballot_w64(imp);
    u64x8 bb = __builtin_bit_cast(u64x8, s.best);
    const u64x8 aa = __builtin_bit_cast(u64x8, acc);
    unsigned long long b0 = bb[0], b1 = bb[1], b2 = bb[2], b3 = bb[3], b4 = bb[4], b5 = bb[5], b6 = bb[6], b7 = bb[7];
    unsigned long long sv;
    asm volatile(
        "s_and_saveexec_b64 %0, %17\n\t"
        "v_mov_b64 %1, %9\n\t"
        "v_mov_b64 %2, %10\n\t"
        "v_mov_b64 %3, %11\n\t"
        "v_mov_b64 %4, %12\n\t"
        "v_mov_b64 %5, %13\n\t"
        "v_mov_b64 %6, %14\n\t"
        "v_mov_b64 %7, %15\n\t"
        "v_mov_b64 %8, %16\n\t"
        "s_mov_b64 exec, %0"
        : "=&s"(sv), "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3), "+v"(b4), "+v"(b5), "+v"(b6), "+v"(b7)
        : "v"(aa[0]), "v"(aa[1]), "v"(aa[2]), "v"(aa[3]), "v"(aa[4]), "v"(aa[5]), "v"(aa[6]), "v"(aa[7]), "s"(mask)
        : "scc");
    bb = u64x8{b0, b1, b2, b3, b4, b5, b6, b7};
    s.best = __builtin_bit_cast(f32x16, bb);
}

// The value held by lane l ^ 32 (the lane of the same point that holds the other 16 rows of
// each tile).  v_permlane32_swap trades lanes 32-63 of its first operand with lanes 0-31 of its
// second; with both operands v, the second result holds the upper half's values in lanes 0-31
// and the first the lower half's in lanes 32-63.  A VALU exchange, no LDS round trip.
__device__ inline uint32_t partner32(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ inline float partner32(float v) { return __uint_as_float(partner32(__float_as_uint(v))); }

// Resolve the winning centroid of this lane and merge with the partner lane (lane ^ 32, same
// point, the other 16 rows of every tile): the point's least (half) score and its lowest index.
// Accumulator r of lane (j, h) holds row 8*(r/4) + 4*h + (r%4) of the 32-centroid tile (MFMA
// 32x32 output layout).
__device__ inline void argmin_resolve(const ArgminState &s, int h, float &sc, int &k) {
    int slot = 15;
#pragma unroll
    for (int r = 15; r >= 0; --r) slot = (s.best[r] == s.run_min) ? r : slot;
    k = s.run_tile * 32 + 8 * (slot >> 2) + 4 * h + (slot & 3);
    sc = s.run_min;
    const float osc = partner32(sc);
    const int ok = (int)partner32((uint32_t)k);
    if (osc < sc || (osc == sc && ok < k)) {
        sc = osc;
        k = ok;
    }
}

// A (score, index) pair as one 64-bit key whose unsigned order is (score, then index): the fp32
// bits mapped to an order-preserving unsigned integer in the high word, the index in the low
// word.  The least key over several partial scans is the least score with the lowest index.
__device__ inline unsigned long long argmin_key(float sc, int k) {
    uint32_t u = __float_as_uint(sc);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 32) | (uint32_t)k;
}
__device__ inline float argmin_key_score(unsigned long long key) {
    uint32_t u = (uint32_t)(key >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(u);
}

// Write the merged pick of this lane (see argmin_resolve).
// xnorm == NULL: the point's squared norm is `own_norm` (computed by the caller).
__device__ inline float argmin_finish(const ArgminState &s, int h, bool write, int64_t out_i, int32_t *out_a,
                                      float *out_d, const float *xnorm, bool want_d, float own_norm = 0.f) {
    float sc;
    int k;
    argmin_resolve(s, h, sc, k);
    float d = 0.f;
    if (write) {
        out_a[out_i] = k;
        if (want_d) {
            d = (xnorm ? xnorm[out_i] : own_norm) + 2.0f * sc;  // squared distance to the chosen centroid
            if (out_d) out_d[out_i] = d;
        }
    }
    return d;
}

// A double moved across lanes by the DPP pattern CTRL (both 32-bit halves alike).
template <int CTRL>
__device__ inline double dpp_f64(double v) {
    const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
__device__ inline double readlane_f64(double v, int l) {
    const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Sum of the wave's point distances in fp64, fixed order; lane 0 writes it to dst[wave] (dst:
// the workgroup's ASSIGN_WAVES partials).  Within each row of 16 lanes the partner of a step is
// fixed by a DPP pattern (lane ^ 1, lane ^ 2, the other quad of the half-row, the other half of
// the row), so every lane of a row ends with the row's sum; the four row sums are then added in
// row order.  No LDS traffic and no workgroup barrier: a wave that finishes its scan early
// leaves without waiting for the others.  Feeds the per-iteration inertia without a pass over
// min_dist.
__device__ inline void wave_inertia(double v, double *dst) {
    v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_f64<0x141>(v);  // row_half_mirror
    v += dpp_f64<0x140>(v);  // row_mirror
    const double t = ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
    if ((threadIdx.x & 63) == 0) dst[threadIdx.x >> 6] = t;
}

// s_waitcnt immediate that waits until at most n vector-memory loads are outstanding and all
// LDS operations are done (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4]
// in bits 15:14).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | (0 << 8) | (((n >> 4) & 3) << 14); }

// Workgroup barrier that leaves newer global->LDS copies in flight: this wave's LDS traffic
// and all but its `n` youngest vector-memory loads are complete before the s_barrier.  The
// empty asm statements keep the compiler from moving memory operations across it.
template <int n>
__device__ inline void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(n));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------------------------------
// Small-D assign: each wave keeps PB blocks of 32 points in VGPRs (B operand) for the whole
// scan; centroid tiles stream through LDS in stages of two tiles, three buffers deep.
// grid = B * ceil(N / block_n) workgroups of 256 threads.
//
// Per tile the wave issues PB x QG MFMAs, then folds the tile's scores into its running
// arg-min; at least three waves share a SIMD (at most 168 registers), so one wave's fold runs
// beside the others' MFMAs.  Around them:
//   * the A fragments are read from LDS ahead of use through a 2-group register ring (each
//     slot refilled right after its last MFMA);
//   * the tile's centroid norms are read into an accumulator set just before its MFMAs;
//   * stage s+2 is copied global->LDS while stage s is consumed; a barrier in the middle of
//     each stage publishes stage s+1 before the first fragment of it is read.
// ------------------------------------------------------------------------------------------
//
// K split (nsplit > 1, for grids too small to fill the chip): the workgroups of one point tile
// scan disjoint ranges of centroid stages, and each point's pick leaves as an argmin_key through a
// 64-bit atomic minimum into `packed` (the least key: the least score, ties to the lowest index,
// the same pick as one scan of all stages).  The workgroup of the first range also writes the
// points' squared norms to xn_out (when distances are wanted); split_finish_kernel turns the keys
// into labels, distances and inertia partials.
template <int DT, int DP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void assign_small_d_kernel(
    const void *__restrict__ x, const u32x4 *__restrict__ cprep, const float *__restrict__ cnh,
    const float *__restrict__ xnorm, int32_t *__restrict__ out_a, float *__restrict__ out_d,
    double *__restrict__ wg_inertia, int N, int D, int KT, int wgs_per_b, int nsplit,
    unsigned long long *__restrict__ packed, float *__restrict__ xn_out) {
    constexpr int S = DT == DT_F32 ? 4 : 2;
    constexpr int VW = 16 / S;
    constexpr int QG = DP / (2 * VW);
    constexpr int PB = small_d_pb(DT, DP);
    constexpr int TILE_U4 = QG * 64;
    constexpr int TPS = small_d_tps(DT, DP);  // tiles per stage: at least 4 KiB, one per wave-copy
    static_assert(TPS == (QG >= 16 ? 1 : (QG >= 2 ? 2 : 4)), "stage size");
    constexpr int STAGE_U4 = TPS * TILE_U4;
    constexpr int PF = STAGE_U4 / 256;  // 1 KiB copy instructions per wave per stage
    constexpr int NCOPY = PF + 1;       // ... plus one for the stage's norms
    static_assert(STAGE_U4 % 256 == 0, "stage must split evenly over 4 waves");

    // Three distinct LDS buffers: the compiler can then tell that the reads of one buffer
    // never alias the global->LDS copies into another.
    __shared__ u32x4 s_c0[STAGE_U4], s_c1[STAGE_U4], s_c2[STAGE_U4];
    __shared__ __attribute__((aligned(16))) float s_n0[TPS * 32], s_n1[TPS * 32], s_n2[TPS * 32];

    FKM_RSTAMP(4);
    FKM_HWSTAMP(6);
    FKM_STAMP(0);
    // consecutive logical workgroups (one XCD) take the K ranges of a point tile, then the next tile
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int per_b = wgs_per_b * nsplit;
    const int b = wg / per_b;
    const int rb = wg - b * per_b;
    const int tn = rb / nsplit;
    const int sp = rb - tn * nsplit;
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index is uniform: held in a scalar register, the copy addresses derived from it
    // (global source bases and LDS destinations) stay scalar too
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, h = lane >> 5;
    const int pbase = tn * (ASSIGN_WAVES * PB * 32) + w * PB * 32;

    // The wave's point rows.  Read straight into the MFMA layout, every load instruction touches
    // 32 rows (32 bytes of each); staged through LDS instead, every copy instruction moves 1 KiB
    // of contiguous rows, and the tile arrives in about half the time.  The staging uses two of
    // the centroid stage buffers before the centroid pipeline needs them: a 32-point block per
    // wave at a time (when four of them fit in two stage buffers and rows are whole 16-byte
    // groups).  In LDS the 16-byte groups of row r are stored XOR-swizzled by r, so that the
    // MFMA-layout reads (32 rows, one group each) spread over the banks.
    u32x4 xr[PB][QG];
    constexpr int XROWB = DP * S;        // bytes of a padded row in LDS
    constexpr int XBLK = 32 * XROWB;     // bytes of one wave's 32-point block
    constexpr bool XDMA_FITS = 4 * XBLK <= 2 * STAGE_U4 * 16 && XBLK % 1024 == 0;
    const bool xdma = XDMA_FITS && (D % VW) == 0;
    if (!xdma) {
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            const int pt = pbase + p * 32 + j;
            const bool vp = pt < N;
            const size_t row0 = ((size_t)b * N + (vp ? pt : 0)) * D;
#pragma unroll
            for (int q = 0; q < QG; ++q) xr[p][q] = load_x_group<DT>(x, row0, (2 * q + h) * VW, D, vp);
        }
    }

    const u32x4 *cb = cprep + (size_t)b * KT * TILE_U4;
    const float *nb = cnh + (size_t)b * KT * 32;
    const int nst_all = KT / TPS;  // KT is a multiple of 4
    // this workgroup's stages [s_beg, nst)
    const int s_beg = sp * nst_all / nsplit;
    const int nst = (sp + 1) * nst_all / nsplit;
    const bool split = packed != nullptr;
    const bool want_d = split ? (xn_out != nullptr && sp == 0) : (out_d != nullptr || wg_inertia != nullptr);

    // Global -> LDS copy of stage st (TPS tiles and their norms).  Every wave issues exactly
    // NCOPY copy instructions, so it can wait for an older stage with a fixed count.  The
    // descriptors are based at the stage, so every offset is small; each lane's offset is the
    // constant 16 * lane, and each 1 KiB piece adds a scalar offset.
    const int lane_off = lane * 16;
    auto stage_copy = [&](int st, u32x4 *__restrict__ sc, float *__restrict__ sn) {
        const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(cb + (size_t)st * STAGE_U4, STAGE_U4 * 16);
#pragma unroll
        for (int r = 0; r < PF; ++r) {
            const int chunk = r * ASSIGN_WAVES + w;
            lds_dma16(rc, lane_off, chunk * 1024, sc + chunk * 64);
        }
        if (lane < 2 * TPS) lds_dma16(buffer_rsrc(nb + (size_t)st * TPS * 32, TPS * 32 * 4), lane_off, w * TPS * 32, sn + w * TPS * 8);
    };

    ArgminState st[PB];
#pragma unroll
    for (int p = 0; p < PB; ++p) argmin_init(st[p]);

    // A fragments: group q of the tile being multiplied lives in slot q % FR.  A slot is
    // refilled right after group q's MFMAs with group q + FR: of the same tile while there is
    // one, else of the next tile.  A ring of 2 groups (8 registers) leaves room for three waves
    // per SIMD at 2-byte D = 128 (168 registers): 3.7% faster there than a ring of 4 at two
    // waves per SIMD, and 13% faster at 2-byte D = 64 than a ring of 4.
    constexpr int FR = QG >= 4 ? 2 : QG;
    static_assert(QG % FR == 0, "fragment ring");
    u32x4 f[FR];
    f32x16 acc[PB];
    // The tile's half-norms (this lane's 16 rows) go into the last accumulator set, which the
    // first MFMA of every point block takes as its C operand: no registers of their own.
    auto load_norms = [&](const float *sn, int tt) {
        const float *nrm = sn + tt * 32 + 4 * h;
        const f32x4 c0 = *(const f32x4 *)(nrm + 0), c1 = *(const f32x4 *)(nrm + 8);
        const f32x4 c2 = *(const f32x4 *)(nrm + 16), c3 = *(const f32x4 *)(nrm + 24);
        acc[PB - 1] = f32x16{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3],
                             c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
    };
    // One tile (its norms already in acc[PB - 1]): multiply f into acc while refilling f with
    // the following fragments, each right after its last use, then fold the tile's scores.
    // One accumulator set: the fold of one wave overlaps the MFMAs of the other waves of the
    // SIMD (two accumulator sets alternating inside a wave measured 2-3% slower: the extra 32
    // registers cost more than the overlap gains).  After the last tile the refills read a
    // stale (in-bounds) buffer and are never used: no branches here.
    auto step = [&](int tile, const u32x4 *__restrict__ csc, int ctt, const u32x4 *__restrict__ nsc, int ntt) {
#pragma unroll
        for (int q = 0; q < QG; ++q) {
#pragma unroll
            for (int p = 0; p < PB; ++p) acc[p] = mfma_group<DT>(f[q % FR], xr[p][q], q == 0 ? acc[PB - 1] : acc[p]);
            if (q + FR < QG) f[q % FR] = csc[ctt * TILE_U4 + (q + FR) * 64 + lane];
            else f[q % FR] = nsc[ntt * TILE_U4 + (q + FR - QG) * 64 + lane];
        }
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            argmin_fold(st[p], acc[p], tile);
            // the fold completes here: left free to sink into the next tile it would keep a
            // second accumulator set live
            asm volatile("" : "+v"(st[p].best), "+v"(st[p].run_min), "+v"(st[p].run_tile));
        }
    };
    // Stage s lives in X; stage s+1 in Y (copied earlier); stage s+2 is copied into Z.  With a
    // whole tile of fragments in flight (FR == QG) the last step of a stage reads only Y, so Z
    // (stage s-1's buffer) is free from the start of stage s and the copy goes first.  With a
    // ring (FR < QG) the last step of stage s-1 still read Z after its mid-stage barrier, so the
    // copy waits for this stage's mid-stage barrier, which every wave passes only after it.
    // The buffer pointers are __restrict__: the alias scopes this gives the LDS reads and the
    // global->LDS copies let the compiler wait for a copy only where its buffer is read, not
    // before every LDS read after it (which would stall each stage on the newest copy).
    auto run_stage = [&](int s, u32x4 *__restrict__ xc, float *__restrict__ xn_, u32x4 *__restrict__ yc,
                         float *__restrict__ yn, u32x4 *__restrict__ zc, float *__restrict__ zn) {
        const bool copy2 = s + 2 < nst;
        constexpr bool early = FR == QG;
        if (early && copy2) stage_copy(s + 2, zc, zn);
        const int t0 = TPS * s;
#pragma unroll
        for (int i = 0; i + 1 < TPS; ++i) {
            load_norms(xn_, i);
            step(t0 + i, xc, i, xc, i + 1);  // refills from this stage
        }
        // the last tile's norms are read before the barrier, after which a faster wave may
        // already copy into this buffer
        load_norms(xn_, TPS - 1);
        const bool more = s + 1 < nst;
        if (more) {
            // stage s+1 landed (this wave), then published
            if (early && copy2) stage_barrier<NCOPY>();
            else stage_barrier<0>();
        }
        if (!early && copy2) stage_copy(s + 2, zc, zn);
        step(t0 + TPS - 1, xc, TPS - 1, yc, 0);  // last tile; refills from the next stage
    };

    // prologue: stages s_beg and s_beg + 1 in flight, the first published, its first tile loaded
    if (xdma) {
        // the point blocks through LDS (waves 0, 1 in buffer 1, waves 2, 3 in buffer 2) while
        // stage s_beg is copied into buffer 0; stage s_beg + 1 follows once every wave has read
        // its points
        constexpr int NI = XBLK / 1024;    // copy instructions per block
        constexpr int CPR = XROWB / 16;    // 16-byte groups per padded row
        constexpr int SWM = (CPR < 8 ? CPR : 8) - 1;
        u32x4 *xst = (w < 2 ? s_c1 : s_c2) + (w & 1) * (XBLK / 16);
        auto x_copy = [&](int p) {
            const int row0 = pbase + p * 32;
            // the block's rows only: rows past N are outside the buffer and read as zeros.  The
            // clamp compiles to a vector instruction; read back into a scalar register, the
            // descriptor stays scalar (else every copy below becomes a loop over lane values)
            const int nbytes = __builtin_amdgcn_readfirstlane(max(0, min(32, N - row0)) * D * S);
            const __amdgpu_buffer_rsrc_t rx =
                buffer_rsrc((const char *)x + ((size_t)b * N + min(row0, N)) * D * S, nbytes);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int b0 = i * 1024 + lane * 16;
                const int r = b0 / XROWB, c = (b0 % XROWB) / 16;
                const int cg = c ^ (r & SWM);
                // groups past D (padding) take an offset outside the buffer
                const int voff = cg * VW < D ? r * D * S + cg * 16 : 0x40000000;
                lds_dma16(rx, voff, 0, xst + i * 64);
            }
        };
        auto x_read = [&](int p) {
            const bool vp = pbase + p * 32 + j < N;
#pragma unroll
            for (int q = 0; q < QG; ++q) {
                const int c = 2 * q + h;
                const u32x4 v = xst[j * CPR + (c ^ (j & SWM))];
                xr[p][q] = (vp && c * VW < D) ? v : u32x4{0u, 0u, 0u, 0u};
            }
        };
        x_copy(0);
        stage_copy(s_beg, s_c0, s_n0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(NCOPY));  // this wave's block landed
        asm volatile("" ::: "memory");
        x_read(0);
#pragma unroll
        for (int p = 1; p < PB; ++p) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));  // the reads of the previous block
            asm volatile("" ::: "memory");
            x_copy(p);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
            asm volatile("" ::: "memory");
            x_read(p);
        }
        stage_barrier<63>();  // every wave's point reads done: buffers 1 and 2 are free
        if (nst > s_beg + 1) {
            stage_copy(s_beg + 1, s_c1, s_n1);
            stage_barrier<NCOPY>();
        } else {
            stage_barrier<0>();
        }
    } else {
        stage_copy(s_beg, s_c0, s_n0);
        if (nst > s_beg + 1) {
            stage_copy(s_beg + 1, s_c1, s_n1);
            stage_barrier<NCOPY>();
        } else {
            stage_barrier<0>();
        }
    }
#pragma unroll
    for (int q = 0; q < FR; ++q) f[q] = s_c0[q * 64 + lane];

    FKM_STAMP(1);
    for (int s0 = s_beg; s0 < nst; s0 += 3) {
        run_stage(s0, s_c0, s_n0, s_c1, s_n1, s_c2, s_n2);
        if (s0 + 1 < nst) run_stage(s0 + 1, s_c1, s_n1, s_c2, s_n2, s_c0, s_n0);
        if (s0 + 2 < nst) run_stage(s0 + 2, s_c2, s_n2, s_c0, s_n0, s_c1, s_n1);
    }

    FKM_STAMP(2);
    double dsum = 0.0;
#pragma unroll
    for (int p = 0; p < PB; ++p) {
        const int pt = pbase + p * 32 + j;
        // without given point norms: ||x||^2 from the point's registers (this lane's half of the
        // row, then the partner lane's), in fp32
        float own = 0.f;
        if (want_d && !xnorm) {
#pragma unroll
            for (int q = 0; q < QG; ++q) {
                if constexpr (DT == DT_F32) {
                    float fx[VW];
                    widen16<DT>(__builtin_bit_cast(uint4, xr[p][q]), fx);
#pragma unroll
                    for (int e = 0; e < VW; ++e) own += fx[e] * fx[e];
                } else {
                    // two squares per instruction (exact products, fp32 sum), no widening
#pragma unroll
                    for (int e = 0; e < 4; ++e) own = dot2_self<DT>(xr[p][q][e], own);
                }
            }
            own += partner32(own);
        }
        if (split) {
            float sc;
            int k;
            argmin_resolve(st[p], h, sc, k);
            if (h == 0 && pt < N) {
                atomicMin(packed + (size_t)b * N + pt, argmin_key(sc, k));
                if (want_d) xn_out[(size_t)b * N + pt] = own;
            }
        } else {
            dsum += argmin_finish(st[p], h, h == 0 && pt < N, (int64_t)b * N + pt, out_a, out_d, xnorm, want_d, own);
        }
    }
    if (!split && wg_inertia) wave_inertia(dsum, wg_inertia + ((size_t)b * wgs_per_b + tn) * ASSIGN_WAVES);
    FKM_STAMP(3);
    FKM_RSTAMP(5);
}

// After a K-split assign: each point's least key -> label (and distance xn + 2 score), with the
// threads laid out as the assign workgroup's lanes (PB blocks of 32 points per wave, lanes h == 0
// write), so the per-tile inertia partials add the same terms in the same order as the unsplit
// kernel.  Resets the keys to all ones for the next use.
template <int PB>
__global__ __launch_bounds__(256) void split_finish_kernel(unsigned long long *__restrict__ packed,
                                                           const float *__restrict__ xn, int32_t *__restrict__ out_a,
                                                           float *__restrict__ out_d, double *__restrict__ wg_inertia,
                                                           int N, int wgs_per_b) {
    const int b = blockIdx.x / wgs_per_b, tn = blockIdx.x - b * wgs_per_b;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int j = lane & 31, h = lane >> 5;
    const int pbase = tn * (ASSIGN_WAVES * PB * 32) + w * PB * 32;
    const bool want_d = out_d != nullptr || wg_inertia != nullptr;
    double dsum = 0.0;
#pragma unroll
    for (int p = 0; p < PB; ++p) {
        const int pt = pbase + p * 32 + j;
        if (h == 0 && pt < N) {
            const size_t i = (size_t)b * N + pt;
            const unsigned long long key = packed[i];
            packed[i] = ~0ull;
            out_a[i] = (int32_t)(uint32_t)key;
            if (want_d) {
                const float d = (xn ? xn[i] : 0.f) + 2.0f * argmin_key_score(key);
                if (out_d) out_d[i] = d;
                dsum += d;
            }
        }
    }
    if (wg_inertia) wave_inertia(dsum, wg_inertia + ((size_t)b * wgs_per_b + tn) * ASSIGN_WAVES);
}

// ------------------------------------------------------------------------------------------
// Split-D assign (README, "Large-D and dtype support": outer K loop, inner D loop, the
// (points x centroids) accumulator held in registers across the D loop).  Workgroup = 128
// points (4 waves x 32); register group = SPLITD_KB tiles (128 centroids); D streamed in
// chunks of BD elements: x chunk and centroid chunk staged together in LDS, double buffered.
// ------------------------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void assign_split_d_kernel(const void *__restrict__ x,
                                                             const u32x4 *__restrict__ cprep,
                                                             const float *__restrict__ cnh,
                                                             const float *__restrict__ xnorm,
                                                             int32_t *__restrict__ out_a, float *__restrict__ out_d,
                                                             double *__restrict__ wg_inertia,
                                                             int N, int D, int DP, int KT, int wgs_per_b) {
    constexpr int S = DT == DT_F32 ? 4 : 2;
    constexpr int VW = 16 / S;
    constexpr int BD = splitd_bd(DT);
    constexpr int QC = BD / (2 * VW);         // 16-byte groups per lane per chunk (= 4)
    constexpr int KB = SPLITD_KB;
    constexpr int XU4 = ASSIGN_WAVES * QC * 64;  // x chunk words
    constexpr int CU4 = KB * QC * 64;            // centroid chunk words
    constexpr int PFX = XU4 / 256, PFC = CU4 / 256;
    static_assert(XU4 % 256 == 0 && CU4 % 256 == 0, "chunks split evenly");

    __shared__ u32x4 s_x[2][XU4];
    __shared__ u32x4 s_c[2][CU4];

    FKM_RSTAMP(4);
    FKM_HWSTAMP(6);
    FKM_STAMP(0);
    const int QG = DP / (2 * VW);
    const int NC = DP / BD;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int b = wg / wgs_per_b;
    const int tn = wg - b * wgs_per_b;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = lane >> 5;
    const int pbase = tn * (ASSIGN_WAVES * 32);
    const int ngroups = (KT + KB - 1) / KB;
    const int nstage = ngroups * NC;
    const u32x4 *cb = cprep + (size_t)b * KT * QG * 64;
    const float *nb = cnh + (size_t)b * KT * 32;

    u32x4 pfx[PFX], pfc[PFC];
    auto gload = [&](int s) {
        const int g = s / NC, dc = s - g * NC;
#pragma unroll
        for (int r = 0; r < PFX; ++r) {
            const int i = tid + r * 256;
            const int pb = i / (QC * 64), rem = i - pb * (QC * 64);
            const int q = rem >> 6, ln = rem & 63;
            const int pt = pbase + pb * 32 + (ln & 31);
            const bool vp = pt < N;
            const int d0 = dc * BD + (2 * q + (ln >> 5)) * VW;
            pfx[r] = load_x_group<DT>(x, ((size_t)b * N + (vp ? pt : 0)) * D, d0, D, vp);
        }
#pragma unroll
        for (int r = 0; r < PFC; ++r) {
            const int i = tid + r * 256;
            const int t = i / (QC * 64), rem = i - t * (QC * 64);
            const int q = rem >> 6, ln = rem & 63;
            const int tile = g * KB + t;
            pfc[r] = tile < KT ? cb[((size_t)tile * QG + dc * QC + q) * 64 + ln] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto swrite = [&](int buf) {
#pragma unroll
        for (int r = 0; r < PFX; ++r) s_x[buf][tid + r * 256] = pfx[r];
#pragma unroll
        for (int r = 0; r < PFC; ++r) s_c[buf][tid + r * 256] = pfc[r];
    };

    ArgminState st;
    argmin_init(st);
    f32x16 acc[KB];

    gload(0);
    swrite(0);
    __syncthreads();
    FKM_STAMP(1);
    for (int s = 0; s < nstage; ++s) {
        const int buf = s & 1;
        const int g = s / NC, dc = s - g * NC;
        if (s + 1 < nstage) gload(s + 1);
        if (dc == 0) {
#pragma unroll
            for (int t = 0; t < KB; ++t) {
                const int tile = g * KB + t;
                const int tl = tile < KT ? tile : 0;
                const float *nrm = nb + (size_t)tl * 32 + 4 * h;
                const f32x4 c0 = *(const f32x4 *)(nrm + 0), c1 = *(const f32x4 *)(nrm + 8);
                const f32x4 c2 = *(const f32x4 *)(nrm + 16), c3 = *(const f32x4 *)(nrm + 24);
                acc[t] = f32x16{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3],
                                c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
            }
        }
#pragma unroll
        for (int q = 0; q < QC; ++q) {
            const u32x4 xb = s_x[buf][(w * QC + q) * 64 + lane];
#pragma unroll
            for (int t = 0; t < KB; ++t) acc[t] = mfma_group<DT>(s_c[buf][(t * QC + q) * 64 + lane], xb, acc[t]);
        }
        if (dc == NC - 1) {
#pragma unroll
            for (int t = 0; t < KB; ++t) {
                const int tile = g * KB + t;
                if (tile < KT) argmin_fold(st, acc[t], tile);
            }
        }
        if (s + 1 < nstage) swrite(buf ^ 1);
        __syncthreads();
    }
    FKM_STAMP(2);
    const int pt = pbase + w * 32 + (lane & 31);
    const float d = argmin_finish(st, h, h == 0 && pt < N, (int64_t)b * N + pt, out_a, out_d, xnorm,
                                  out_d != nullptr || wg_inertia != nullptr);
    if (wg_inertia) wave_inertia((double)d, wg_inertia + ((size_t)b * wgs_per_b + tn) * ASSIGN_WAVES);
    FKM_STAMP(3);
    FKM_RSTAMP(5);
}

// ------------------------------------------------------------------------------------------
// host launchers
// ------------------------------------------------------------------------------------------
#if !defined(FKM_ASSIGN_D64_UNIT) && !defined(FKM_ASSIGN_D128_UNIT)
// zero_norm: the similarity metrics (dot product, cosine) score -x.c~ alone, so the norm
// terms of the real rows are 0 (the padding rows keep +inf).
hipError_t launch_prep_centroids(int dt, const float *C, void *cprep, float *cnh, int B, int K, int D, int DP,
                                 hipStream_t stream, int zero_norm) {
    const int KT = assign_tiles(dt, D, K);
    dim3 grid(B * KT), block(256);
    if (dt == DT_F32)
        prep_centroids_kernel<DT_F32><<<grid, block, 0, stream>>>(C, (u32x4 *)cprep, cnh, K, D, DP, KT, zero_norm);
    else if (dt == DT_F16)
        prep_centroids_kernel<DT_F16><<<grid, block, 0, stream>>>(C, (u32x4 *)cprep, cnh, K, D, DP, KT, zero_norm);
    else
        prep_centroids_kernel<DT_BF16><<<grid, block, 0, stream>>>(C, (u32x4 *)cprep, cnh, K, D, DP, KT, zero_norm);
    return hipGetLastError();
}
#endif

template <int DT, int DP>
static hipError_t launch_small(const void *x, const void *cprep, const float *cnh, const float *xn, int32_t *a,
                               float *md, double *wgi, int B, int N, int D, int K, const AssignSplit &sp,
                               hipStream_t stream) {
    constexpr int PB = small_d_pb(DT, DP);
    const int KT = assign_tiles(DT, D, K);
    const int bn = ASSIGN_WAVES * PB * 32;
    const int wpb = (N + bn - 1) / bn;
    if (sp.nsplit <= 1) {
        assign_small_d_kernel<DT, DP><<<dim3(B * wpb), dim3(256), 0, stream>>>(
            x, (const u32x4 *)cprep, cnh, xn, a, md, wgi, N, D, KT, wpb, 1, nullptr, nullptr);
        return hipGetLastError();
    }
    // the keys hold all ones on entry (the previous finish, or the caller's fill, left them so)
    const bool want_d = md != nullptr || wgi != nullptr;
    float *xn_out = (want_d && !xn) ? sp.xn : nullptr;
    assign_small_d_kernel<DT, DP><<<dim3(B * wpb * sp.nsplit), dim3(256), 0, stream>>>(
        x, (const u32x4 *)cprep, cnh, xn, a, md, wgi, N, D, KT, wpb, sp.nsplit, sp.packed, xn_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    split_finish_kernel<PB><<<dim3(B * wpb), dim3(256), 0, stream>>>(sp.packed, xn ? xn : xn_out, a, md, wgi, N,
                                                                     wpb);
    return hipGetLastError();
}

// The 2-byte instances at padded D = 64 and D = 128 are compiled in files of their own
// (k_assign_d64.hip and k_assign_d128.hip: this file with FKM_ASSIGN_D64_UNIT or
// FKM_ASSIGN_D128_UNIT defined), each under the compiler scheduling strategy that runs it fastest:
// at D = 64 the default one, 8% faster (K = 1024; 2% at K = 32768) than the memory-clause strategy
// the other instances take; at D = 128 the iterative ILP one, about 0.6% faster per launch and 1% per
// fit iteration at the headline shape (four same-box A/B pairs), which would make the split-D
// kernel 18% slower.
hipError_t launch_small_2byte_d64(int dt, const void *x, const void *cprep, const float *cnh, const float *xn,
                                  int32_t *a, float *md, double *wgi, int B, int N, int D, int K,
                                  const AssignSplit &sp, hipStream_t s);
hipError_t launch_small_2byte_d128(int dt, const void *x, const void *cprep, const float *cnh, const float *xn,
                                   int32_t *a, float *md, double *wgi, int B, int N, int D, int K,
                                   const AssignSplit &sp, hipStream_t s);
#if defined(FKM_ASSIGN_D64_UNIT)
hipError_t launch_small_2byte_d64(int dt, const void *x, const void *cprep, const float *cnh, const float *xn,
                                  int32_t *a, float *md, double *wgi, int B, int N, int D, int K,
                                  const AssignSplit &sp, hipStream_t s) {
    if (dt == DT_F16) return launch_small<DT_F16, 64>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
    if (dt == DT_BF16) return launch_small<DT_BF16, 64>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
    return hipErrorInvalidValue;
}
#elif defined(FKM_ASSIGN_D128_UNIT)
hipError_t launch_small_2byte_d128(int dt, const void *x, const void *cprep, const float *cnh, const float *xn,
                                   int32_t *a, float *md, double *wgi, int B, int N, int D, int K,
                                   const AssignSplit &sp, hipStream_t s) {
    if (dt == DT_F16) return launch_small<DT_F16, 128>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
    if (dt == DT_BF16) return launch_small<DT_BF16, 128>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
    return hipErrorInvalidValue;
}
#else
template <int DT>
static hipError_t launch_small_dt(int DP, const void *x, const void *cprep, const float *cnh, const float *xn,
                                  int32_t *a, float *md, double *wgi, int B, int N, int D, int K,
                                  const AssignSplit &sp, hipStream_t s) {
    if constexpr (DT == DT_F32) {
        switch (DP) {
            case 8: return launch_small<DT, 8>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
            case 16: return launch_small<DT, 16>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
            case 32: return launch_small<DT, 32>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
            case 64: return launch_small<DT, 64>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
            case 128: return launch_small<DT, 128>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
        }
    } else {
        switch (DP) {
            case 16: return launch_small<DT, 16>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
            case 32: return launch_small<DT, 32>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
            case 64: return launch_small_2byte_d64(DT, x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
            case 128: return launch_small_2byte_d128(DT, x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
            case 256: return launch_small<DT, 256>(x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
        }
    }
    return hipErrorInvalidValue;
}

// wgi (optional): per-wave fp64 sums of the chosen distances, [B][assign_wgs_per_problem][ASSIGN_WAVES].
// xn: point norms for the distances (md / wgi); the small-D kernel computes them itself when NULL.
// sp: the K split (small-D path; nsplit 1 = one scan of all centroids per point tile).
hipError_t launch_assign(int dt, const AssignCfg &cfg, const void *x, const void *cprep, const float *cnh,
                         const float *xn, int32_t *a, float *md, double *wgi, int B, int N, int D, int K,
                         hipStream_t s, const AssignSplit &sp) {
    if (cfg.path == 0) {
        if (dt == DT_F32) return launch_small_dt<DT_F32>(cfg.d_pad, x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
        if (dt == DT_F16) return launch_small_dt<DT_F16>(cfg.d_pad, x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
        return launch_small_dt<DT_BF16>(cfg.d_pad, x, cprep, cnh, xn, a, md, wgi, B, N, D, K, sp, s);
    }
    const int KT = assign_tiles(dt, D, K);
    const int bn = ASSIGN_WAVES * 32;
    const int wpb = (N + bn - 1) / bn;
    dim3 grid(B * wpb), block(256);
    if (dt == DT_F32)
        assign_split_d_kernel<DT_F32><<<grid, block, 0, s>>>(x, (const u32x4 *)cprep, cnh, xn, a, md, wgi, N, D,
                                                             cfg.d_pad, KT, wpb);
    else if (dt == DT_F16)
        assign_split_d_kernel<DT_F16><<<grid, block, 0, s>>>(x, (const u32x4 *)cprep, cnh, xn, a, md, wgi, N, D,
                                                             cfg.d_pad, KT, wpb);
    else
        assign_split_d_kernel<DT_BF16><<<grid, block, 0, s>>>(x, (const u32x4 *)cprep, cnh, xn, a, md, wgi, N, D,
                                                              cfg.d_pad, KT, wpb);
    return hipGetLastError();
}
#endif  // FKM_ASSIGN_D64_UNIT / FKM_ASSIGN_D128_UNIT

}  // namespace fkm
