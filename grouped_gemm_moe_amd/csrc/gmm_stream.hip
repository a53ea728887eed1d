// Decode-shaped grouped matmul forward for gfx950: weight streaming.
//
// Same operation as gmm_fwd ("NPU Training Operators - GMM", section 算子语义:
// y[rows_e] = x[rows_e] @ w[e] over the row ranges of group_list), for calls
// where experts own a few rows each.  There the work is reading each active
// expert's weights once from HBM; an MFMA tile would sit mostly idle on
// padding rows, so the products run on the vector ALUs in fp32 while 16-byte
// weight loads stream through every CU.
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "launch.h"

namespace moegmm {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Block = (expert e, slice of COLS columns).  A wave holds 64/(COLS/8)
// k-groups of COLS/8 column lanes; a lane owns 8 columns and walks k-chunks
// of 8 rows, so each step is eight 16-byte weight loads feeding 8x8xROWS fp32
// FMAs.  The expert's rows are staged in LDS (bf16) kStreamRows at a time,
// one pass over the weights per group of rows.  Partial sums meet first
// across the k-groups of a wave (shuffles), then across waves in LDS, always
// in the same order.
//
// SWIGLU: the gate_up forward (N = 2I) fused with SwiGLU.  The block's
// column lanes are split in two halves: the first streams gate columns
// c0 .. c0+COLS/2-1, the second the up columns I+c0 .. of the same outputs,
// and the epilogue writes a = SiLU(G) * U for COLS/2 output columns (and,
// when h is given, G and U too).
// ---------------------------------------------------------------------------
#ifndef MOEGMM_STREAM_COLS
#define MOEGMM_STREAM_COLS 256
#endif
constexpr int kStreamCols = MOEGMM_STREAM_COLS;
#ifndef MOEGMM_STREAM_UNROLL
#define MOEGMM_STREAM_UNROLL 2
#endif
constexpr int kStreamRows = 4;
constexpr int kWaves = kThreads / 64;

template <int COLS, int ROWS>
MOE_DEVICE void stream_rows(const bf16_t* __restrict__ We, const bf16_t* xs, int K, int N, int kg,
                            float (&acc)[kStreamRows][8]) {
    constexpr int kGroups = (64 / (COLS / 8)) * kWaves;
#pragma unroll MOEGMM_STREAM_UNROLL
    for (int k = kg * 8; k < K; k += 8 * kGroups) {
        u32x4_t wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[j] = ld16(We + (int64_t)(k + j) * N);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + r * K + k);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t xp = xv[j >> 1];
                const float xf = (j & 1) ? bf16_hi(xp) : bf16_lo(xp);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t wp = wv[j][c >> 1];
                    const float wf = (c & 1) ? bf16_hi(wp) : bf16_lo(wp);
                    acc[r][c] = __builtin_fmaf(xf, wf, acc[r][c]);
                }
            }
        }
    }
}

template <int COLS, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void gmm_stream_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, const int64_t* __restrict__ group_list,
    int E, int64_t M_cap, int K, int N, bf16_t* __restrict__ Y, bf16_t* __restrict__ Hout,
    int32_t* dev_err) {
    constexpr int kLanes = COLS / 8;          // column lanes of one k-group
    constexpr int kGPW = 64 / kLanes;         // k-groups per wave
    constexpr int kOutCols = SWIGLU ? COLS / 2 : COLS;  // output columns per block
    extern __shared__ __attribute__((aligned(16))) char dsmem[];
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int64_t s_scan[kThreads / 64];
    __shared__ float red[kWaves][kStreamRows][COLS];
    bf16_t* xs = reinterpret_cast<bf16_t*>(dsmem);  // [kStreamRows][K]

    load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, dev_err);
    const int Nout = SWIGLU ? N / 2 : N;  // output columns
    const int NB = (Nout + kOutCols - 1) / kOutCols;
    const int e = blockIdx.x / NB, nb = blockIdx.x % NB;
    const int off = s_off[e], cnt = s_cnt[e];
    if (cnt == 0) return;  // uniform

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int cl = lane % kLanes;
    const int kg = wid * kGPW + lane / kLanes;
    // the output column of this lane's 8 columns, and its weight column
    const int ocol = nb * kOutCols + (SWIGLU ? cl % (kLanes / 2) : cl) * 8;
    const int col = SWIGLU && cl >= kLanes / 2 ? Nout + ocol : ocol;
    const bool col_ok = ocol < Nout;
    const bf16_t* We = W + (int64_t)e * K * N + col;

    for (int r0 = 0; r0 < cnt; r0 += kStreamRows) {
        const int rows = cnt - r0 < kStreamRows ? cnt - r0 : kStreamRows;
        const int cpr = K / 8;
        for (int u = threadIdx.x; u < kStreamRows * cpr; u += kThreads) {
            const int r = u / cpr, c = u % cpr;
            u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
            if (r < rows) v = ld16(X + (int64_t)(off + r0 + r) * K + c * 8);
            *reinterpret_cast<u32x4_t*>(xs + r * K + c * 8) = v;
        }
        __syncthreads();

        float acc[kStreamRows][8];
#pragma unroll
        for (int r = 0; r < kStreamRows; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
        if (col_ok) {
            if (rows == 1) stream_rows<COLS, 1>(We, xs, K, N, kg, acc);
            else if (rows == 2) stream_rows<COLS, 2>(We, xs, K, N, kg, acc);
            else stream_rows<COLS, 4>(We, xs, K, N, kg, acc);  // a third row is zero-padded
        }
        // k-groups of this wave, then waves, in a fixed order
#pragma unroll
        for (int o = kLanes; o < 64; o <<= 1)
#pragma unroll
            for (int r = 0; r < kStreamRows; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[r][c] += __shfl_xor(acc[r][c], o, 64);
        if (lane < kLanes) {
#pragma unroll
            for (int r = 0; r < kStreamRows; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) red[wid][r][cl * 8 + c] = acc[r][c];
        }
        __syncthreads();
        if constexpr (SWIGLU) {
            // 4 output columns per thread (as many threads as the plain
            // epilogue uses): gate sums from columns j, up sums from
            // kOutCols + j of the block's partials
            constexpr int kQuads = kOutCols / 4;
            if (threadIdx.x < kStreamRows * kQuads) {
                const int r = threadIdx.x / kQuads, c4 = threadIdx.x % kQuads;
                const int gcol = nb * kOutCols + c4 * 4;
                if (r < rows && gcol < Nout) {
                    float gs[4], us[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) gs[c] = us[c] = 0.f;
#pragma unroll
                    for (int w = 0; w < kWaves; ++w)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            gs[c] += red[w][r][c4 * 4 + c];
                            us[c] += red[w][r][kOutCols + c4 * 4 + c];
                        }
                    const int64_t orow = off + r0 + r;
                    u32x2_t o;
                    o[0] = pack_bf16x2(gs[0] * silu_sigmoid(gs[0]) * us[0], gs[1] * silu_sigmoid(gs[1]) * us[1]);
                    o[1] = pack_bf16x2(gs[2] * silu_sigmoid(gs[2]) * us[2], gs[3] * silu_sigmoid(gs[3]) * us[3]);
                    *reinterpret_cast<u32x2_t*>(Y + orow * Nout + gcol) = o;
                    if (Hout) {
                        u32x2_t og, ou;
                        og[0] = pack_bf16x2(gs[0], gs[1]);
                        og[1] = pack_bf16x2(gs[2], gs[3]);
                        ou[0] = pack_bf16x2(us[0], us[1]);
                        ou[1] = pack_bf16x2(us[2], us[3]);
                        *reinterpret_cast<u32x2_t*>(Hout + orow * N + gcol) = og;
                        *reinterpret_cast<u32x2_t*>(Hout + orow * N + Nout + gcol) = ou;
                    }
                }
            }
        } else if (threadIdx.x < kStreamRows * kLanes) {
            const int r = threadIdx.x / kLanes, c8 = threadIdx.x % kLanes;
            const int gcol = nb * COLS + c8 * 8;
            if (r < rows && gcol < N) {
                float sum[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) sum[c] = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w)
#pragma unroll
                    for (int c = 0; c < 8; ++c) sum[c] += red[w][r][c8 * 8 + c];
                u32x4_t o;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(sum[2 * c], sum[2 * c + 1]);
                st16(Y + (int64_t)(off + r0 + r) * N + gcol, o);
            }
        }
        __syncthreads();
    }
}

}  // namespace

GmmVariant forced_gmm_variant() {
    const char* v = getenv("MOEGMM_FORCE_VARIANT");
    if (v == nullptr) return kVariantAuto;
    if (strcmp(v, "tile") == 0) return kVariantTile;
    if (strcmp(v, "stream") == 0) return kVariantStream;
    return kVariantAuto;
}

bool gmm_stream_applies(int64_t E, int64_t M_cap, int64_t K) {
    // the staged x rows keep the kernel's total LDS (at most 24 KiB static)
    // within 64 KiB
    const bool fits = K * kStreamRows * 2 <= 32 * 1024;
    switch (forced_gmm_variant()) {
        case kVariantTile: return false;
        case kVariantStream: return fits;
        default: break;
    }
    // a few rows per expert on average
    return M_cap <= 8 * E && fits;
}

hipError_t launch_gmm_stream(const uint16_t* x, const uint16_t* w, const int64_t* group_list,
                             int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* y,
                             int32_t* dev_err, hipStream_t stream) {
    const int64_t NB = (N + kStreamCols - 1) / kStreamCols;
    const size_t shmem = (size_t)K * kStreamRows * 2;
    hipLaunchKernelGGL((gmm_stream_kernel<kStreamCols, false>), dim3((unsigned)(E * NB)), dim3(kThreads),
                       shmem, stream, x, w, group_list, (int)E, M_cap, (int)K, (int)N, y, nullptr,
                       dev_err);
    return hipGetLastError();
}

hipError_t launch_gmm_stream_swiglu(const uint16_t* x, const uint16_t* w1,
                                    const int64_t* group_list, int64_t E, int64_t M_cap,
                                    int64_t K, int64_t I, uint16_t* a, uint16_t* h,
                                    int32_t* dev_err, hipStream_t stream) {
    const int64_t NB = (I + kStreamCols / 2 - 1) / (kStreamCols / 2);
    const size_t shmem = (size_t)K * kStreamRows * 2;
    hipLaunchKernelGGL((gmm_stream_kernel<kStreamCols, true>), dim3((unsigned)(E * NB)), dim3(kThreads),
                       shmem, stream, x, w1, group_list, (int)E, M_cap, (int)K, (int)(2 * I), a, h,
                       dev_err);
    return hipGetLastError();
}

}  // namespace moegmm
