// SwiGLU, its backward, and the probs-weighted unpermute for gfx950.
//
// SwiGLU follows "MegaMoE" (activation formulas: sigma(z) = 1/(1+e^-z),
// SiLU(z) = z*sigma(z), A = SiLU(G) * U with the clamp unset), with G the
// first I and U the last I columns of the gate_up output ("NPU Training
// Operators - GMM", section "Qwen3.5 MoE 路径": one gate_up GMM, then a
// SwiGLU split).  The backward is derived by calculus (not on the pages).
//
// The unpermute follows "MegaMoE" (A16W16 Token Combine: each token sums its
// top-k expert rows weighted by the gate weights, in token order) and the
// MoeTokenPermuteWithRoutingMapGrad article (section 6.2: per output token,
// walk the top-k slots, skip -1, accumulate in FP32, cast back once).  Each
// token is owned by one workgroup and summed in ascending k, so the result is
// deterministic with no atomics.
//
// The same per-token walk, with unit weights, is the permute backward: the
// article's token gradient (section 2.3) adds every permuted row's gradient
// back onto the token it was copied from.  The backward of the weighted
// unpermute is the derivative of the Token Combine formula:
//   dy_perm[row(t,k)] = probs[t,k] * dout[t],
//   dprobs[t,k]       = <dout[t], y_perm[row(t,k)]>   (0 for a masked slot),
// both from one pass over a token's rows, the dot products reduced in a fixed
// order (lane shuffles, then the waves in order), so again deterministic.
//
// All are HBM-bound streams: 16-byte loads and stores, fp32 math.
#include "common.h"
#include "launch.h"
#include "swiglu.h"

namespace moegmm {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGrid = 2048;

// Rows r < R (R from group_list), 8 columns of the I outputs per work item.
__global__ __launch_bounds__(kThreads) void swiglu_kernel(const bf16_t* __restrict__ h,
                                                          const int64_t* __restrict__ group_list,
                                                          int E, int64_t M_cap, int64_t I,
                                                          bf16_t* __restrict__ a) {
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int64_t s_scan[kThreads / 64];
    const int R = load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, nullptr);
    const int64_t cpr = I / 8;
    const int64_t items = (int64_t)R * cpr;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < items;
         u += (int64_t)gridDim.x * kThreads) {
        const int64_t r = u / cpr, c = u - r * cpr;
        const bf16_t* hr = h + r * 2 * I;
        st16(a + r * I + c * 8, swiglu8(ld16(hr + c * 8), ld16(hr + I + c * 8)));
    }
}

// dh may be h itself (in place): a thread reads G, U and dA of its 8
// columns before it writes dG and dU to the same places, and no other thread
// touches them -- so h and dh carry no restrict.
__global__ __launch_bounds__(kThreads) void swiglu_bwd_kernel(
    const bf16_t* __restrict__ da, const bf16_t* h, const int64_t* __restrict__ group_list,
    int E, int64_t M_cap, int64_t I, bf16_t* dh) {
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int64_t s_scan[kThreads / 64];
    const int R = load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, nullptr);
    const int64_t cpr = I / 8;
    const int64_t items = (int64_t)R * cpr;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < items;
         u += (int64_t)gridDim.x * kThreads) {
        const int64_t r = u / cpr, c = u - r * cpr;
        const bf16_t* hr = h + r * 2 * I;
        const u32x4_t g = ld16(hr + c * 8);
        const u32x4_t up = ld16(hr + I + c * 8);
        const u32x4_t d = ld16(da + r * I + c * 8);
        u32x4_t og, ou;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float gv[2] = {bf16_lo(g[q]), bf16_hi(g[q])};
            float uv[2] = {bf16_lo(up[q]), bf16_hi(up[q])};
            float dv[2] = {bf16_lo(d[q]), bf16_hi(d[q])};
            float rg[2], ru[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float s = silu_sigmoid(gv[t]);
                rg[t] = dv[t] * uv[t] * s * (1.0f + gv[t] * (1.0f - s));
                ru[t] = dv[t] * gv[t] * s;
            }
            og[q] = pack_bf16x2(rg[0], rg[1]);
            ou[q] = pack_bf16x2(ru[0], ru[1]);
        }
        bf16_t* dr = dh + r * 2 * I;
        st16(dr + c * 8, og);
        st16(dr + I + c * 8, ou);
    }
}

// One workgroup per token; the row ids and gate weights of the token's top_k
// slots are read once into LDS.  Each thread owns 8 columns per pass.
constexpr int kMaxTopK = 32;

__global__ __launch_bounds__(kThreads) void unpermute_kernel(
    const bf16_t* __restrict__ y_perm, const int32_t* __restrict__ row_id_map,
    const float* __restrict__ probs, int64_t T, int top_k, int64_t H, bf16_t* __restrict__ out,
    int32_t* dev_err) {
    __shared__ int32_t s_row[kMaxTopK];
    __shared__ float s_p[kMaxTopK];
    const int64_t t = blockIdx.x;
    const int64_t S = T * top_k;
    if (threadIdx.x < top_k) {
        int32_t r = row_id_map[t * top_k + threadIdx.x];
        if (r < -1 || r >= S) {
            if (dev_err) atomicOr(dev_err, MOE_DEVERR_ROW_MAP);
            r = -1;
        }
        s_row[threadIdx.x] = r;
        s_p[threadIdx.x] = probs ? probs[t * top_k + threadIdx.x] : 1.0f;  // no probs: plain sum
    }
    __syncthreads();
    for (int64_t c0 = (int64_t)threadIdx.x * 8; c0 < H; c0 += kThreads * 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        // the rows of up to 8 slots in flight together, then added in
        // ascending k (a few tokens per call leave most CUs idle, so the
        // load latency is what a token costs)
        for (int k0 = 0; k0 < top_k; k0 += 8) {
            u32x4_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t r = k0 + j < top_k ? s_row[k0 + j] : -1;
                v[j] = r >= 0 ? ld16(y_perm + (int64_t)r * H + c0) : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t r = k0 + j < top_k ? s_row[k0 + j] : -1;
                if (r < 0) continue;
                const float p = s_p[k0 + j];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    acc[2 * d] = __builtin_fmaf(p, bf16_lo(v[j][d]), acc[2 * d]);
                    acc[2 * d + 1] = __builtin_fmaf(p, bf16_hi(v[j][d]), acc[2 * d + 1]);
                }
            }
        }
        u32x4_t o;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(acc[2 * d], acc[2 * d + 1]);
        st16(out + t * H + c0, o);
    }
}

// One workgroup per token; KMAX >= top_k is a compile-time bound so the
// per-slot partial dot products stay in registers.
template <int KMAX>
__global__ __launch_bounds__(kThreads) void unpermute_bwd_kernel(
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ y_perm,
    const int32_t* __restrict__ row_id_map, const float* __restrict__ probs, int64_t T, int top_k,
    int64_t H, bf16_t* __restrict__ dy_perm, float* __restrict__ dprobs, int32_t* dev_err) {
    __shared__ int32_t s_row[KMAX];
    __shared__ float s_p[KMAX];
    __shared__ float s_red[kThreads / 64][KMAX];
    const int64_t t = blockIdx.x;
    const int64_t S = T * top_k;
    if (threadIdx.x < KMAX) {
        int32_t r = -1;
        float p = 0.f;
        if ((int)threadIdx.x < top_k) {
            r = row_id_map[t * top_k + threadIdx.x];
            if (r < -1 || r >= S) {
                if (dev_err) atomicOr(dev_err, MOE_DEVERR_ROW_MAP);
                r = -1;
            }
            p = probs[t * top_k + threadIdx.x];
        }
        s_row[threadIdx.x] = r;
        s_p[threadIdx.x] = p;
    }
    __syncthreads();
    float part[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) part[k] = 0.f;
    for (int64_t c0 = (int64_t)threadIdx.x * 8; c0 < H; c0 += kThreads * 8) {
        const u32x4_t g = ld16(dout + t * H + c0);
        float gv[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            gv[2 * d] = bf16_lo(g[d]);
            gv[2 * d + 1] = bf16_hi(g[d]);
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int32_t r = s_row[k];
            if (r < 0) continue;
            const u32x4_t y = ld16(y_perm + (int64_t)r * H + c0);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                part[k] = __builtin_fmaf(gv[2 * d], bf16_lo(y[d]), part[k]);
                part[k] = __builtin_fmaf(gv[2 * d + 1], bf16_hi(y[d]), part[k]);
            }
            const float p = s_p[k];
            u32x4_t o;
#pragma unroll
            for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(p * gv[2 * d], p * gv[2 * d + 1]);
            st16(dy_perm + (int64_t)r * H + c0, o);
        }
    }
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        float v = part[k];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) s_red[wid][k] = v;
    }
    __syncthreads();
    if ((int)threadIdx.x < top_k) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) sum += s_red[w][threadIdx.x];
        dprobs[t * top_k + threadIdx.x] = s_row[threadIdx.x] >= 0 ? sum : 0.f;
    }
}

int64_t elementwise_grid(int64_t M_cap, int64_t I) {
    int64_t items = M_cap * (I / 8);
    int64_t g = (items + kThreads - 1) / kThreads;
    if (g > kMaxGrid) g = kMaxGrid;
    return g < 1 ? 1 : g;
}

}  // namespace

hipError_t launch_swiglu(const uint16_t* h, const int64_t* group_list, int64_t E, int64_t M_cap,
                         int64_t I, uint16_t* a, hipStream_t stream) {
    if (M_cap == 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)elementwise_grid(M_cap, I)), dim3(kThreads), 0,
                       stream, h, group_list, (int)E, M_cap, I, a);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* da, const uint16_t* h, const int64_t* group_list,
                             int64_t E, int64_t M_cap, int64_t I, uint16_t* dh,
                             hipStream_t stream) {
    if (M_cap == 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)elementwise_grid(M_cap, I)), dim3(kThreads),
                       0, stream, da, h, group_list, (int)E, M_cap, I, dh);
    return hipGetLastError();
}

hipError_t launch_unpermute(const uint16_t* y_perm, const int32_t* row_id_map, const float* probs,
                            int64_t T, int64_t top_k, int64_t H, uint16_t* out, int32_t* dev_err,
                            hipStream_t stream) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)T), dim3(kThreads), 0, stream, y_perm,
                       row_id_map, probs, T, (int)top_k, H, out, dev_err);
    return hipGetLastError();
}

hipError_t launch_permute_bwd(const uint16_t* dx_perm, const int32_t* row_id_map, int64_t T,
                              int64_t top_k, int64_t H, uint16_t* dx, int32_t* dev_err,
                              hipStream_t stream) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)T), dim3(kThreads), 0, stream, dx_perm,
                       row_id_map, nullptr, T, (int)top_k, H, dx, dev_err);
    return hipGetLastError();
}

hipError_t launch_unpermute_bwd(const uint16_t* dout, const uint16_t* y_perm,
                                const int32_t* row_id_map, const float* probs, int64_t T,
                                int64_t top_k, int64_t H, uint16_t* dy_perm, float* dprobs,
                                int32_t* dev_err, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const dim3 grid((unsigned)T), block(kThreads);
#define MOE_UNPERMUTE_BWD(KMAX)                                                                 \
    hipLaunchKernelGGL(unpermute_bwd_kernel<KMAX>, grid, block, 0, stream, dout, y_perm,        \
                       row_id_map, probs, T, (int)top_k, H, dy_perm, dprobs, dev_err)
    if (top_k <= 1) MOE_UNPERMUTE_BWD(1);
    else if (top_k <= 2) MOE_UNPERMUTE_BWD(2);
    else if (top_k <= 4) MOE_UNPERMUTE_BWD(4);
    else if (top_k <= 8) MOE_UNPERMUTE_BWD(8);
    else if (top_k <= 16) MOE_UNPERMUTE_BWD(16);
    else MOE_UNPERMUTE_BWD(32);
#undef MOE_UNPERMUTE_BWD
    return hipGetLastError();
}

}  // namespace moegmm
