// Phase probe of the FlashAssign kernels: the kernel the plan picks (small-D or split-D) built with
// FKM_CLOCK_STAMPS, launched on a synthetic problem of the given shape, and every workgroup's clock
// stamps summarised:
//   * the shader clock during the workgroups (s_memtime cycles over the 100 MHz real-time counter);
//   * per workgroup, cycles from start to the scan (point tile in, first centroid stages in), in the
//     scan (per 32-centroid tile too), and from the scan's end to the workgroup's end, split into the
//     workgroups of the first round (started in the launch's first 2 us) and the later ones;
//   * the launch time and its fraction of the nominal MFMA peak of the dtype (2.5 PFLOP/s bf16/fp16,
//     157.3 TFLOP/s fp32), and of that peak at the measured clock;
//   * per CU, the share of time with 0..3 of its workgroups resident and in their scan, and the gaps
//     between successive workgroup starts on a CU.
// A measuring tool, not part of the library; built by build.py beside libflashkm.so and run by
// `bench.py --clock-probe`.  Usage: probe_assign_clock [B N D K [dtype: bf16|f16|f32 [extra LDS]]]
// `extra LDS` (bytes of dynamic LDS per workgroup, 2-byte types at padded D = 128 only) lowers the
// number of workgroups that share a CU: with 20000 two fit, with 40000 one (one wave per SIMD).
#define FKM_CLOCK_STAMPS 1
#include "k_assign.hip"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#define CK(x)                                                                              \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
            std::exit(1);                                                                  \
        }                                                                                  \
    } while (0)

// host rounding of fp32 to the 2-byte types, nearest even (finite inputs)
static uint16_t host_to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static uint16_t host_to_f16(float f) {
    const _Float16 h = (_Float16)f;
    uint16_t u;
    std::memcpy(&u, &h, 2);
    return u;
}

static double pct(std::vector<double> v, double q) {
    if (v.empty()) return 0.0;
    std::sort(v.begin(), v.end());
    return v[std::min(v.size() - 1, (size_t)(q * v.size()))];
}

int main(int argc, char **argv) {
    using namespace fkm;
    const int B = argc > 4 ? std::atoi(argv[1]) : 32, N = argc > 4 ? std::atoi(argv[2]) : 65536;
    const int D = argc > 4 ? std::atoi(argv[3]) : 128, K = argc > 4 ? std::atoi(argv[4]) : 1024;
    const std::string dts = argc > 5 ? std::string(argv[5]) : std::string("bf16");
    const int dyn = argc > 6 ? std::atoi(argv[6]) : 0;
    const int dt = dts == "f16" ? DT_F16 : (dts == "f32" ? DT_F32 : DT_BF16);
    const int es = dt == DT_F32 ? 4 : 2;
    const double peak = dt == DT_F32 ? 157.3e12 : 2.5e15;
    const AssignCfg cfg = plan_assign(dt, B, N, D, K);
    if (B < 1 || N < 1 || D < 1 || K < 1 || cfg.nsplit != 1) {
        std::printf("the probe covers plans without a K split\n");
        return 2;
    }
    if (dyn != 0 && (dyn < 0 || dyn > 100000 || dt == DT_F32 || cfg.path != 0 || cfg.d_pad != 128)) {
        std::printf("extra LDS: 0 .. 100000 bytes, 2-byte types at padded D = 128 only\n");
        return 2;
    }
    auto kern = dt == DT_F16 ? assign_small_d_kernel<DT_F16, 128> : assign_small_d_kernel<DT_BF16, 128>;
    if (dyn > 0) CK(hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, dyn));
    const int KT = assign_tiles(dt, D, K);
    const int wpb = (N + cfg.block_n - 1) / cfg.block_n;
    const long nwg = (long)B * wpb;
    if (nwg > FKM_STAMP_WGS) {
        std::printf("the probe records at most %d workgroups (this shape has %ld)\n", FKM_STAMP_WGS, nwg);
        return 2;
    }
    std::printf("shape B=%d N=%d D=%d K=%d %s, %s kernel: %ld workgroups of %d points, %d centroid tiles each\n", B, N,
                D, K, dts.c_str(), cfg.path == 0 ? "small-D" : "split-D", nwg, cfg.block_n, KT);
    if (dyn > 0) std::printf("extra dynamic LDS per workgroup: %d bytes\n", dyn);
    // points ~ N(0, 1) rounded to the dtype, centroids ~ N(0, 1) in fp32
    std::mt19937 rng(20260309);
    std::normal_distribution<float> nd(0.f, 1.f);
    std::vector<uint16_t> hx(dt == DT_F32 ? 0 : (size_t)B * N * D);
    std::vector<float> hxf(dt == DT_F32 ? (size_t)B * N * D : 0);
    for (auto &v : hx) v = dt == DT_F16 ? host_to_f16(nd(rng)) : host_to_bf16(nd(rng));
    for (auto &v : hxf) v = nd(rng);
    std::vector<float> hc((size_t)B * K * D);
    for (auto &v : hc) v = nd(rng);
    void *x, *cprep;
    float *C, *cnh;
    int32_t *a;
    double *wgi;
    CK(hipMalloc(&x, (size_t)B * N * D * es));
    if (dt == DT_F32) CK(hipMemcpy(x, hxf.data(), hxf.size() * 4, hipMemcpyHostToDevice));
    else CK(hipMemcpy(x, hx.data(), hx.size() * 2, hipMemcpyHostToDevice));
    CK(hipMalloc(&C, hc.size() * 4));
    CK(hipMemcpy(C, hc.data(), hc.size() * 4, hipMemcpyHostToDevice));
    CK(hipMalloc(&cprep, (size_t)B * KT * 32 * cfg.d_pad * es));
    CK(hipMalloc(&cnh, (size_t)B * KT * 32 * 4));
    CK(hipMalloc(&a, (size_t)B * N * 4));
    CK(hipMalloc(&wgi, (size_t)B * wpb * ASSIGN_WAVES * 8));  // per-wave inertia partials
    CK(launch_prep_centroids(dt, C, cprep, cnh, B, K, D, cfg.d_pad, 0, 0));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    // the launches of the fit's form (point norms from registers, inertia partials); about 40 ms of
    // load first so that the clocks have settled, then the recorded launch
    float ms = 0.f;
    const long reps = std::max(20L, (long)(0.04 * peak * 0.5 / (2.0 * B * N * (double)K * D)));
    for (long it = 0; it < reps; ++it) {
        CK(hipEventRecord(e0));
        // the 2-byte D = 128 instance of this file (the library's is built in a unit of its own, with
        // no stamps) and the extra-LDS runs launch `kern` directly, as launch_assign would
        const bool own = dyn > 0 || (cfg.path == 0 && dt != DT_F32 && cfg.d_pad == 128);
        if (!own) {
            CK(launch_assign(dt, cfg, x, cprep, cnh, nullptr, a, nullptr, wgi, B, N, D, K, 0, AssignSplit{}));
        } else {  // the same launch as launch_assign's, with the extra LDS (if any)
            kern<<<dim3(B * wpb), dim3(256), dyn, 0>>>(x, (const u32x4 *)cprep, cnh, nullptr, a, nullptr, wgi, N, D,
                                                       KT, wpb, 1, nullptr, nullptr);
            CK(hipGetLastError());
        }
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        CK(hipEventElapsedTime(&ms, e0, e1));
    }
    std::vector<unsigned long long> s((size_t)nwg * 8);
    CK(hipMemcpyFromSymbol(s.data(), HIP_SYMBOL(fkm_stamps), s.size() * 8));
    unsigned long long r0 = ~0ull, r1 = 0;
    for (long w = 0; w < nwg; ++w) {
        r0 = std::min(r0, s[w * 8 + 4]);
        r1 = std::max(r1, s[w * 8 + 5]);
    }
    std::vector<double> clk, pro1, pro2, scan, epi, dur;
    for (long w = 0; w < nwg; ++w) {
        const unsigned long long *t = &s[w * 8];
        const double rt = (double)(t[5] - t[4]);  // 10 ns units
        if (rt > 0) clk.push_back((double)(t[3] - t[0]) / rt * 100.0);
        const double start_us = (t[4] - r0) / 100.0;
        (start_us < 2.0 ? pro1 : pro2).push_back((double)(t[1] - t[0]));
        scan.push_back((double)(t[2] - t[1]));
        epi.push_back((double)(t[3] - t[2]));
        dur.push_back(rt / 100.0);
    }
    const double flop = 2.0 * B * N * (double)K * D;
    std::printf("recorded launch: %.1f us, %.1f%% of the %s MFMA peak %.1f TFLOP/s (%ld launches of load before it)\n",
                ms * 1e3, flop / (ms * 1e-3) / peak * 100.0, dts.c_str(), peak / 1e12, reps - 1);
    const double mhz = pct(clk, 0.5);
    std::printf("shader clock during the workgroups: median %.0f MHz (p10 %.0f, p90 %.0f); at the median the\n"
                "  MFMA peak is %.1f TFLOP/s and the launch runs at %.1f%% of it\n",
                mhz, pct(clk, 0.1), pct(clk, 0.9), peak * mhz / 2400.0 / 1e12,
                flop / (ms * 1e-3) / (peak * mhz / 2400.0) * 100.0);
    std::printf("workgroup duration: p50 %.2f us (min %.2f, max %.2f); span of the stamps %.1f us\n", pct(dur, 0.5),
                pct(dur, 0.0), pct(dur, 1.0), (r1 - r0) / 100.0);
    std::printf("shader cycles per workgroup (p10 / p50 / p90):\n");
    std::printf("  to the scan, first round (%4zu wgs): %8.0f %8.0f %8.0f\n", pro1.size(), pct(pro1, 0.1), pct(pro1, 0.5),
                pct(pro1, 0.9));
    std::printf("  to the scan, later     (%5zu wgs): %8.0f %8.0f %8.0f\n", pro2.size(), pct(pro2, 0.1), pct(pro2, 0.5),
                pct(pro2, 0.9));
    std::printf("  scan                                 %8.0f %8.0f %8.0f   (per centroid tile %.0f at p50)\n",
                pct(scan, 0.1), pct(scan, 0.5), pct(scan, 0.9), pct(scan, 0.5) / KT);
    std::printf("  after the scan                       %8.0f %8.0f %8.0f\n", pct(epi, 0.1), pct(epi, 0.5),
                pct(epi, 0.9));
    // Per CU: how many of its resident workgroups are in their scan at each instant.  A workgroup's CU
    // is its XCD (workgroups go to the XCDs round-robin, so blockIdx mod 8) with the SE, SH and CU
    // fields of HW_ID; shader-clock stamps are put on the real-time axis by each workgroup's own
    // start/end pair.  Measured from the launch's first start to its last start (before the drain).
    {
        struct Ev { double t; int res, scan; };
        std::vector<std::vector<Ev>> ev(8 * 256);
        double t_last_start = 0;
        for (long w = 0; w < nwg; ++w) {
            const unsigned long long *t = &s[w * 8];
            if (t[5] <= t[4] || t[3] <= t[0]) continue;
            const unsigned hw = (unsigned)t[6];
            const int key = (int)(w % 8) * 256 + (int)((hw >> 8) & 0xFFu);
            const double a = (double)(t[4] - r0), rt = (double)(t[5] - t[4]), mt = (double)(t[3] - t[0]);
            const double s1 = a + (double)(t[1] - t[0]) / mt * rt, s2 = a + (double)(t[2] - t[0]) / mt * rt;
            ev[key].push_back({a, +1, 0});
            ev[key].push_back({s1, 0, +1});
            ev[key].push_back({s2, 0, -1});
            ev[key].push_back({a + rt, -1, 0});
            t_last_start = std::max(t_last_start, a);
        }
        double busy[5] = {0, 0, 0, 0, 0}, resw[5] = {0, 0, 0, 0, 0}, total = 0;
        int cus = 0;
        std::vector<double> gaps;
        for (auto &e : ev) {
            if (e.empty()) continue;
            ++cus;
            std::sort(e.begin(), e.end(), [](const Ev &x, const Ev &y) { return x.t < y.t; });
            int res = 0, sc = 0;
            double prev = 0, last_start = -1;
            for (const Ev &x : e) {
                const double t1 = std::min(x.t, t_last_start);
                if (t1 > prev) {
                    busy[std::min(sc, 4)] += t1 - prev;
                    resw[std::min(res, 4)] += t1 - prev;
                    total += t1 - prev;
                }
                prev = std::max(prev, t1);
                if (x.res > 0) {
                    if (last_start >= 0) gaps.push_back((x.t - last_start) / 100.0);
                    last_start = x.t;
                }
                res += x.res;
                sc += x.scan;
            }
        }
        std::printf("per CU (%d CUs seen), time from the first start to the last start:\n", cus);
        std::printf("  workgroups resident:  0: %4.1f%%  1: %4.1f%%  2: %4.1f%%  3: %4.1f%%  4+: %4.1f%%\n",
                    100 * resw[0] / total, 100 * resw[1] / total, 100 * resw[2] / total, 100 * resw[3] / total,
                    100 * resw[4] / total);
        std::printf("  workgroups scanning:  0: %4.1f%%  1: %4.1f%%  2: %4.1f%%  3: %4.1f%%  4+: %4.1f%%\n",
                    100 * busy[0] / total, 100 * busy[1] / total, 100 * busy[2] / total, 100 * busy[3] / total,
                    100 * busy[4] / total);
        std::printf("  gap between successive workgroup starts on a CU (us): p10 %.2f p25 %.2f p50 %.2f p75 %.2f "
                    "p90 %.2f\n",
                    pct(gaps, 0.1), pct(gaps, 0.25), pct(gaps, 0.5), pct(gaps, 0.75), pct(gaps, 0.9));
    }
    if (cfg.path == 0 && dt != DT_F32) {
        const int mf = cfg.pb * (cfg.d_pad / 16);  // 32x32x16 MFMAs per tile and wave
        std::printf("  (a tile's MFMA work per wave: %d MFMAs of 32 cycles = %d cycles; three waves per SIMD: %d)\n",
                    mf, mf * 32, 3 * mf * 32);
    }
    return 0;
}
