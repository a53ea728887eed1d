// Decode-shaped grouped matmul forward for gfx950: weight streaming.
//
// Same operation as gmm_fwd ("NPU Training Operators - GMM", section 算子语义:
// y[rows_e] = x[rows_e] @ w[e] over the row ranges of group_list), for calls
// where experts own a few rows each.  There the work is reading each active
// expert's weights once from HBM; an MFMA tile would sit mostly idle on
// padding rows, so the products run on the vector ALUs in fp32 while 16-byte
// weight loads stream through every CU.
#include "common.h"
#include "launch.h"

namespace moegmm {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Decode-shaped forward: weight streaming.  Block = (expert e, 256-column
// slice).  256 threads = 8 k-groups x 32 column lanes; lane owns 8 columns,
// k-group g walks k-chunks of 8 starting at 8g with stride 64.  Rows of the
// expert are processed kStreamRows at a time (one weight pass each), staged in
// LDS as bf16; partial sums over k-groups meet in LDS.
// ---------------------------------------------------------------------------
constexpr int kStreamCols = 256;
constexpr int kStreamRows = 4;
constexpr int kStreamKGroups = kThreads / 32;

__global__ __launch_bounds__(kThreads) void gmm_stream_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, const int64_t* __restrict__ group_list,
    int E, int64_t M_cap, int K, int N, bf16_t* __restrict__ Y, int32_t* dev_err) {
    extern __shared__ __attribute__((aligned(16))) char dsmem[];
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int64_t s_scan[kThreads / 64];
    __shared__ float red[kStreamKGroups][kStreamRows][kStreamCols];
    bf16_t* xs = reinterpret_cast<bf16_t*>(dsmem);  // [kStreamRows][K]

    load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, dev_err);
    const int NB = (N + kStreamCols - 1) / kStreamCols;
    const int e = blockIdx.x / NB, nb = blockIdx.x % NB;
    const int off = s_off[e], cnt = s_cnt[e];
    if (cnt == 0) return;  // uniform

    const int kg = threadIdx.x >> 5, cl = threadIdx.x & 31;
    const int col = nb * kStreamCols + cl * 8;
    const bool col_ok = col < N;
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
#pragma unroll 2
            for (int k = kg * 8; k < K; k += 8 * kStreamKGroups) {
                u32x4_t wv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) wv[j] = ld16(We + (int64_t)(k + j) * N);
#pragma unroll
                for (int r = 0; r < kStreamRows; ++r) {
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
#pragma unroll
        for (int r = 0; r < kStreamRows; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) red[kg][r][cl * 8 + c] = acc[r][c];
        __syncthreads();
        // 4 rows x 32 chunks of 8 columns; fixed summation order over k-groups
        if (threadIdx.x < kStreamRows * (kStreamCols / 8)) {
            const int r = threadIdx.x / (kStreamCols / 8);
            const int c8 = threadIdx.x % (kStreamCols / 8);
            const int gcol = nb * kStreamCols + c8 * 8;
            if (r < rows && gcol < N) {
                float s[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) s[c] = 0.f;
                for (int g = 0; g < kStreamKGroups; ++g)
#pragma unroll
                    for (int c = 0; c < 8; ++c) s[c] += red[g][r][c8 * 8 + c];
                u32x4_t o;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(s[2 * c], s[2 * c + 1]);
                st16(Y + (int64_t)(off + r0 + r) * N + gcol, o);
            }
        }
        __syncthreads();
    }
}


}  // namespace

bool gmm_stream_applies(int64_t E, int64_t M_cap, int64_t K) {
    // a few rows per expert on average, and the staged x rows keep the
    // kernel's total LDS (40 KiB static) within 64 KiB
    return M_cap <= 8 * E && K * kStreamRows * 2 <= 24 * 1024;
}

hipError_t launch_gmm_stream(const uint16_t* x, const uint16_t* w, const int64_t* group_list,
                             int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* y,
                             int32_t* dev_err, hipStream_t stream) {
    const int64_t NB = (N + kStreamCols - 1) / kStreamCols;
    const size_t shmem = (size_t)K * kStreamRows * 2;
    hipLaunchKernelGGL(gmm_stream_kernel, dim3((unsigned)(E * NB)), dim3(kThreads), shmem, stream, x,
                       w, group_list, (int)E, M_cap, (int)K, (int)N, y, dev_err);
    return hipGetLastError();
}

}  // namespace moegmm
