// Device helpers shared by the gfx950 kernels of libmoegmm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moegmm.h"

#define MOE_DEVICE __device__ __forceinline__

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxExperts = 1024;

MOE_DEVICE float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
MOE_DEVICE float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
MOE_DEVICE float bf16_to_f32(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Two fp32 values -> packed bf16 (lo in bits 0..15), round to nearest even,
// NaN stays a (quiet) NaN: one v_cvt_pk_bf16_f32 on gfx950.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
MOE_DEVICE uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// sigma(g) = 1 / (1 + e^-g), the gate of SiLU(g) = g * sigma(g) ("MegaMoE",
// activation formulas).
MOE_DEVICE float silu_sigmoid(float g) { return 1.0f / (1.0f + __expf(-g)); }

// Vector loads/stores of 16 bytes.
MOE_DEVICE u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
MOE_DEVICE void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Wave64 helpers.
MOE_DEVICE int lane_id() { return __lane_id(); }

// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024, a
// multiple of 64).  `scratch` needs blockDim.x/64 ints of LDS.  Returns the
// exclusive prefix; *total receives the block sum.
template <typename T>
MOE_DEVICE T block_exclusive_scan(T v, T* scratch, T* total) {
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    T incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        T t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
    }
    if (lane == 63) scratch[wid] = incl;
    __syncthreads();
    T wave_off = 0, sum = 0;
    for (int i = 0; i < nw; ++i) {
        T s = scratch[i];
        if (i < wid) wave_off += s;
        sum += s;
    }
    __syncthreads();
    *total = sum;
    return wave_off + incl - v;
}

// Per-expert row ranges from a device group_list, clamped so that every range
// lies inside [0, M_cap).  A negative count or a running sum above M_cap sets
// MOE_DEVERR_GROUP_LIST (reported by block 0 only).  Fills, for e < E:
//   s_off[e] (first row), s_cnt[e] (clamped count); returns R = sum of counts.
// Must be called by all threads of the block; E <= kMaxExperts and
// blockDim.x >= 256 (so that a thread owns at most 4 experts).  s_scan needs
// blockDim.x/64 int64 of LDS.
MOE_DEVICE int load_group_ranges(const int64_t* __restrict__ group_list, int E, int64_t M_cap,
                                 int* s_off, int* s_cnt, int64_t* s_scan, int32_t* dev_err) {
    // each thread owns up to 4 consecutive experts
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per;
    int64_t local[4] = {0, 0, 0, 0};
    int bad = 0;
    int64_t lsum = 0;
    for (int i = 0; i < per && i < 4; ++i) {
        int e = e0 + i;
        int64_t n = (e < E) ? group_list[e] : 0;
        if (n < 0) { bad = 1; n = 0; }
        if (n > M_cap) { bad = 1; n = M_cap; }
        local[i] = n;
        lsum += n;
    }
    // counts are clamped to M_cap < 2^31 each; at most 4 per thread, so the
    // int64 scan cannot overflow.
    int64_t total = 0;
    int64_t run = block_exclusive_scan<int64_t>(lsum, s_scan, &total);
    for (int i = 0; i < per && i < 4; ++i) {
        int e = e0 + i;
        if (e >= E) break;
        int64_t n = local[i];
        int64_t lo = run < M_cap ? run : M_cap;
        int64_t hi = run + n;
        if (hi > M_cap) { bad = 1; hi = M_cap; }
        s_off[e] = (int)lo;
        s_cnt[e] = (int)(hi - lo);
        run += n;
    }
    if (bad && dev_err != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
        atomicOr(dev_err, MOE_DEVERR_GROUP_LIST);
    __syncthreads();
    int R = total > M_cap ? (int)M_cap : total;
    return R;
}
