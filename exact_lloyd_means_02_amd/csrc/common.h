// Internal helpers shared by the gfx950 kernels and the host layer of libflashkm.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fkm {

enum Dt : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int NUM_XCD = 8;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

__host__ __device__ inline int elem_bytes(int dt) { return dt == DT_F32 ? 4 : 2; }

// ------------------------------------------------------------------------------------------
// scalar conversions (device)
// ------------------------------------------------------------------------------------------
__device__ inline float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bfloat16 bits, nearest with ties to even (inputs are finite).
__device__ inline uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ inline float f16_bits_to_f32(uint32_t h) {
    union { uint16_t u; _Float16 f; } v;
    v.u = (uint16_t)h;
    return (float)v.f;
}

__device__ inline uint32_t f32_to_f16_bits(float f) {
    union { uint16_t u; _Float16 h; } v;
    v.h = (_Float16)f;  // round to nearest even
    return v.u;
}

// Load element `i` of a row stored in dtype DT and widen to float.
template <int DT>
__device__ inline float load_elem(const void *base, size_t i) {
    if constexpr (DT == DT_F32) {
        return ((const float *)base)[i];
    } else if constexpr (DT == DT_F16) {
        return f16_bits_to_f32(((const uint16_t *)base)[i]);
    } else {
        return bf16_bits_to_f32(((const uint16_t *)base)[i]);
    }
}

// 16-byte load marked nontemporal, for data a kernel reads once: the caches are told not to
// keep it, and a stream of such row loads runs faster than plain loads.
__device__ inline uint4 load16_nt(const void *p) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u t = __builtin_nontemporal_load((const v4u *)p);
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Widen a 16-byte vector holding 8 (2-byte types) or 4 (fp32) elements.
template <int DT>
__device__ inline void widen16(const uint4 &v, float *out) {
    if constexpr (DT == DT_F32) {
        out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == DT_F16) {
                out[2 * i] = f16_bits_to_f32(w[i] & 0xFFFFu);
                out[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
            } else {
                out[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
                out[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
            }
        }
    }
}

// Workgroups are dispatched round-robin over the XCDs (blockIdx % 8).  Map the
// physical id to a logical id so that consecutive logical ids land on the same
// XCD and share its L2 (e.g. all point tiles of one problem read the same
// centroids).  Bijective for any grid size.
__device__ inline int xcd_remap(int p, int grid) {
    const int q = grid / NUM_XCD, r = grid % NUM_XCD;
    const int x = p % NUM_XCD;
    const int start = x * q + (x < r ? x : r);
    return start + p / NUM_XCD;
}

// The same partition of logical ids over XCDs as xcd_remap, walked backwards in time: the
// first workgroups an XCD runs take the end of its range.  A kernel launched after one that
// used xcd_remap over the same data then starts on what the earlier kernel touched last
// (still in the memory-side cache) and ends on what the next such kernel reads first.
__device__ inline int xcd_remap_rev(int p, int grid) {
    const int q = grid / NUM_XCD, r = grid % NUM_XCD;
    const int x = p % NUM_XCD;
    const int start = x * q + (x < r ? x : r);
    const int count = q + (x < r ? 1 : 0);
    return start + count - 1 - p / NUM_XCD;
}

__device__ inline uint64_t lanemask_lt() {
    const int lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace fkm
