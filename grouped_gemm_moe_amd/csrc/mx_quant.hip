// Row-wise MX quantisation (E4M3 codes, E8M0 scales, groups of 32) on gfx950:
// Q_MX of the "MegaMoE" A8W8-FP scenario, for activations and for preparing
// MXFP8 weights ([E*N][K] rows).  The conversion rules are in mx.h.
//
// Four lanes own one group (16 bytes of bf16 each, so a wave's loads and
// stores are contiguous); the group maximum meets over the quad with two xor
// shuffles.  Scale row padding (bytes past ceil(K/32)) is left untouched.
#include "launch.h"
#include "mx.h"

namespace moegmm {

namespace {

constexpr int kQThreads = 256;

__global__ __launch_bounds__(kQThreads) void mx_quantize_kernel(const uint16_t* __restrict__ x,
                                                                int64_t rows, int64_t K, int64_t ld_s,
                                                                uint8_t* __restrict__ q,
                                                                uint8_t* __restrict__ s) {
    const int64_t cpr = K / 8;  // 16-byte pieces per row (4 per group)
    const int64_t total = rows * cpr;
    // every lane runs the same number of iterations (the quad maximum needs all four lanes)
    const int64_t stride = (int64_t)gridDim.x * kQThreads;
    const int64_t iters = (total + stride - 1) / stride;
    int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
    for (int64_t it = 0; it < iters; ++it, i += stride) {
        const bool ok = i < total;  // whole quads agree: total % 4 == 0
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (ok) v = ld16(x + i * 8);
        float f[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            f[2 * c] = bf16_lo(v[c]);
            f[2 * c + 1] = bf16_hi(v[c]);
        }
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(f[c]));
        amax = quad_max(amax);
        const uint32_t sb = mx_scale_byte(amax);
        const float inv = mx_inv_scale(sb);
        if (ok) {
            u32x2_t o;
            o[0] = e4m3_pack4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
            o[1] = e4m3_pack4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
            *reinterpret_cast<u32x2_t*>(q + i * 8) = o;
            const int64_t r = i / cpr, c = i - r * cpr;
            if ((c & 3) == 0) s[r * ld_s + (c >> 2)] = (uint8_t)sb;
        }
    }
}

}  // namespace

hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ld_s, uint8_t* q,
                              uint8_t* s, hipStream_t stream) {
    const int64_t total = rows * (K / 8);
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + kQThreads - 1) / kQThreads;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)blocks), dim3(kQThreads), 0, stream, x,
                       rows, K, ld_s, q, s);
    return hipGetLastError();
}

}  // namespace moegmm
