// Decode-shaped grouped matmul forward for gfx950: weight streaming.
//
// Same operation as gmm_fwd ("NPU Training Operators - GMM", section 算子语义:
// y[rows_e] = x[rows_e] @ w[e] over the row ranges of group_list), for calls
// where experts own a few rows each.  There the work is reading each active
// expert's weights once from HBM; an MFMA tile would sit mostly idle on
// padding rows, so the products run on the vector ALUs in fp32 while 16-byte
// weight loads stream through every CU.
//
// Schedule.  A sub-unit is (expert e, group of kStreamRows of its rows, slice
// of 256 weight columns), one block each, dispatched by the hardware as CUs
// free up.  An expert with more rows than a group owns several sub-units per
// slice, which stream the same weight slice side by side on different CUs
// (its second pass mostly from L2) instead of one block walking its groups
// in turn: with one block per (expert, slice), a decode step where one
// expert held 48 more rows than the rest took 2.5x as long.
//
// The decode layer forward of moe_decode_fwd uses a routed form of the
// gate_up launch: every block counts the expert histogram of topk_ids and
// ranks its own expert's slots, so no permute launch runs before it.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "launch.h"
#include "route.h"
#include "swiglu.h"

namespace moegmm {

namespace {

constexpr int kThreads = 256;
static_assert(kThreads == kRouteThreads, "the routing helpers assume this block size");
constexpr int kStreamCols = 256;  // weight columns per sub-unit
constexpr int kStreamRows = 4;    // expert rows per sub-unit
constexpr int kWaves = kThreads / 64;
constexpr int kLanes = kStreamCols / 8;      // column lanes of one k-group (8 columns each)
constexpr int kGroupsPerWave = 64 / kLanes;  // k-groups per wave
constexpr int kGroups = kGroupsPerWave * kWaves;

// k-chunk iterations per unrolled loop body: 1 measured fastest (decode
// gate_up 180 us; 2: 189 us; 3 and 4: 181-183 us)
#ifndef MOEGMM_STREAM_UNROLL
#define MOEGMM_STREAM_UNROLL 1
#endif

// Bytes of the staged rows' LDS region, which the k-group partial sums
// reuse (so at least their size), rounded to 16; then the expert tables.
constexpr size_t kRedBytes = (size_t)kWaves * kStreamRows * kStreamCols * sizeof(float);
__host__ __device__ inline size_t stream_rows_bytes(int64_t K) {
    const size_t rows = (size_t)K * kStreamRows * 2;
    const size_t b = rows > kRedBytes ? rows : kRedBytes;
    return (b + 15) / 16 * 16;
}
size_t stream_lds_bytes(int64_t K, int64_t E) { return stream_rows_bytes(K) + 3 * (size_t)E * sizeof(int); }

// acc += x rows (LDS, [kStreamRows][K]) times the lane's 8 weight columns;
// k-group kg takes reduction rows 8*kg + 64*i .. +7.
template <int ROWS>
MOE_DEVICE void stream_rows(const bf16_t* __restrict__ We, const bf16_t* xs, int K, int N, int kg,
                            float (&acc)[kStreamRows][8]) {
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

// s_su[e] = first sub-unit of expert e (ceil(n_e / kStreamRows) * NB of them
// per expert); returns the total.  All threads; ends with a barrier.
MOE_DEVICE int sub_unit_starts(const int* s_cnt, int E, int NB, int* s_su, int64_t* s_scan) {
    const int per = (E + kThreads - 1) / kThreads;
    const int e0 = threadIdx.x * per;
    int64_t mine = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) mine += (int64_t)((s_cnt[e0 + i] + kStreamRows - 1) / kStreamRows) * NB;
    int64_t total;
    int64_t run = block_exclusive_scan<int64_t>(mine, s_scan, &total);
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) {
            s_su[e0 + i] = (int)run;
            run += (int64_t)((s_cnt[e0 + i] + kStreamRows - 1) / kStreamRows) * NB;
        }
    __syncthreads();
    return (int)total;
}

// Block = one sub-unit.  A wave holds kGroupsPerWave k-groups of kLanes
// column lanes; a lane owns 8 columns and walks k-chunks of 8 rows, so each
// step is eight 16-byte weight loads feeding 8 x 8 x ROWS fp32 FMAs.  The
// group's rows are staged in LDS (bf16).  Partial sums meet first across
// the k-groups of a wave (shuffles), then across waves in LDS, always in the
// same order.
//
// SWIGLU: the gate_up forward (N = 2I) fused with SwiGLU.  The sub-unit's
// column lanes are split in two halves: the first streams gate columns
// c0 .. c0+127, the second the up columns I+c0 .. of the same outputs, and
// the epilogue writes a = SiLU(G) * U for 128 output columns (and, when h is
// given, G and U too).
//
// slot (nullable): X is the token matrix [nslots / top_k, K] and row r of the
// grouped operand is token slot[r] / top_k; an entry outside [0, nslots)
// stages a zero row and sets MOE_DEVERR_SLOT.
//
// SWIGLU_IN: the down GMM on SwiGLU(X): X is H [M_cap, 2K] and the staged
// rows are A = SiLU(G) * U of its halves, rounded as the swiglu kernel
// rounds them; Hout, when given, receives A [M_cap, K] (from the sub-units
// of the first column slice).
//
// ROUTE (plain gate_up, X the token matrix): the group ranges and the rows'
// slots come from ra.ids (route_group_ranges, route_rows) instead of
// group_list and slot; the blocks of the first column slice write
// sorted_slot and row_id_map for their rows, and the grid's last block the
// call outputs (route_call_outputs).
template <bool SWIGLU, bool SWIGLU_IN = false, bool ROUTE = false>
__global__ __launch_bounds__(kThreads) void gmm_stream_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, const int64_t* __restrict__ group_list,
    int E, int64_t M_cap, int K, int N, bf16_t* __restrict__ Y, bf16_t* __restrict__ Hout,
    int32_t* dev_err, const int32_t* __restrict__ slot, int top_k, int nslots, const RouteArgs ra) {
    static_assert(!ROUTE || (!SWIGLU && !SWIGLU_IN), "the routed form is the plain gate_up");
    __shared__ int s_rows[kStreamRows];
    constexpr int kOutCols = SWIGLU ? kStreamCols / 2 : kStreamCols;  // output columns per sub-unit
    // Dynamic LDS (stream_lds_bytes): the staged rows, whose space the
    // k-group partial sums reuse once every wave has left the streaming loop,
    // then the per-expert tables, sized by E -- so that four workgroups fit
    // a CU even for K = 2048.
    extern __shared__ __attribute__((aligned(16))) char dsmem[];
    __shared__ int64_t s_scan[kThreads / 64];
    bf16_t* xs = reinterpret_cast<bf16_t*>(dsmem);  // [kStreamRows][K]
    float(*red)[kStreamRows][kStreamCols] = reinterpret_cast<float(*)[kStreamRows][kStreamCols]>(dsmem);
    int* s_off = reinterpret_cast<int*>(dsmem + stream_rows_bytes(K));
    int* s_cnt = s_off + E;
    int* s_su = s_cnt + E;

    if constexpr (ROUTE) {
        const bool last = blockIdx.x == gridDim.x - 1;
        route_group_ranges(ra.ids, nslots, E, s_off, s_cnt, s_scan, dev_err, last);
        if (last) route_call_outputs(ra, E, nslots, s_cnt);
    } else {
        load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, dev_err);
    }
    const int Nout = SWIGLU ? N / 2 : N;
    const int NB = (Nout + kOutCols - 1) / kOutCols;
    const int SU = sub_unit_starts(s_cnt, E, NB, s_su, s_scan);
    const int su = blockIdx.x;
    if (su >= SU) return;  // uniform; past this call's sub-units
    // sub-unit -> (expert, row group, slice)
    int lo = 0, hi = E - 1;  // last expert whose first sub-unit is <= su
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_su[mid] <= su) lo = mid; else hi = mid - 1;
    }
    const int e = lo, r_in = su - s_su[e];
    const int g = r_in / NB, nb = r_in % NB;
    const int off = s_off[e] + g * kStreamRows;
    const int rows = s_cnt[e] - g * kStreamRows < kStreamRows ? s_cnt[e] - g * kStreamRows : kStreamRows;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int cl = lane % kLanes;
    const int kg = wid * kGroupsPerWave + lane / kLanes;
    // this lane's 8 weight columns: output columns ocol.., weight column col
    const int ocol = nb * kOutCols + (SWIGLU ? cl % (kLanes / 2) : cl) * 8;
    const int col = SWIGLU && cl >= kLanes / 2 ? Nout + ocol : ocol;
    const bool col_ok = ocol < Nout;
    const bf16_t* We = W + (int64_t)e * K * N + col;

    if constexpr (ROUTE) {
        route_rows(ra.ids, nslots, e, g * kStreamRows, rows, s_rows, s_scan);
        if (nb == 0 && tid < rows) {
            ra.sorted_slot[off + tid] = s_rows[tid];
            ra.row_id_map[s_rows[tid]] = off + tid;
        }
    }

    // source row of each staged row (-1: zeros)
    int src[kStreamRows];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kStreamRows; ++r) {
        src[r] = r < rows ? off + r : -1;
        if constexpr (ROUTE) src[r] = r < rows ? s_rows[r] / top_k : -1;
        if (slot && r < rows) {
            const int s = slot[off + r];
            const bool ok = s >= 0 && s < nslots;
            src[r] = ok ? s / top_k : -1;
            bad |= !ok;
        }
    }
    if (bad && tid == 0 && dev_err) atomicOr(dev_err, MOE_DEVERR_SLOT);
    const int cpr = K / 8;
    for (int u = tid; u < kStreamRows * cpr; u += kThreads) {
        const int r = u / cpr, c = u % cpr;
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (SWIGLU_IN) {
            if (src[r] >= 0) {
                const bf16_t* hr = X + (int64_t)src[r] * 2 * K;
                v = swiglu8(ld16(hr + c * 8), ld16(hr + K + c * 8));
                if (Hout && nb == 0) st16(Hout + (int64_t)src[r] * K + c * 8, v);
            }
        } else {
            if (src[r] >= 0) v = ld16(X + (int64_t)src[r] * K + c * 8);
        }
        *reinterpret_cast<u32x4_t*>(xs + r * K + c * 8) = v;
    }
    __syncthreads();

    float acc[kStreamRows][8];
#pragma unroll
    for (int r = 0; r < kStreamRows; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
    if (col_ok) {
        if (rows == 1) stream_rows<1>(We, xs, K, N, kg, acc);
        else if (rows == 2) stream_rows<2>(We, xs, K, N, kg, acc);
        else stream_rows<4>(We, xs, K, N, kg, acc);  // a third row is zero-padded
    }
    // k-groups of this wave, then waves, in a fixed order
#pragma unroll
    for (int o = kLanes; o < 64; o <<= 1)
#pragma unroll
        for (int r = 0; r < kStreamRows; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[r][c] += __shfl_xor(acc[r][c], o, 64);
    __syncthreads();  // every wave is done reading the staged rows, whose space red takes
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
        if (tid < kStreamRows * kQuads) {
            const int r = tid / kQuads, c4 = tid % kQuads;
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
                const int64_t orow = off + r;
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
    } else if (tid < kStreamRows * kLanes) {
        const int r = tid / kLanes, c8 = tid % kLanes;
        const int gcol = nb * kStreamCols + c8 * 8;
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
            st16(Y + (int64_t)(off + r) * N + gcol, o);
        }
    }
}

// Sub-units at most: sum over experts of ceil(n_e / kStreamRows) groups of
// rows, <= M_cap / kStreamRows + E, times the slices.  N = weight columns.
int64_t max_sub_units(int64_t E, int64_t M_cap, int64_t N) {
    const int64_t NB = (N + kStreamCols - 1) / kStreamCols;
    return ((M_cap + kStreamRows - 1) / kStreamRows + E) * NB;
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
    // the staged x rows keep the kernel's LDS at most 64 KiB
    const bool fits = K * kStreamRows * 2 <= 32 * 1024;
    switch (forced_gmm_variant()) {
        case kVariantTile: return false;
        case kVariantStream: return fits && M_cap <= (int64_t(1) << 16);  // grid well within 2^31 blocks
        default: break;
    }
    // a few rows per expert on average
    return M_cap <= 8 * E && fits;
}

static hipError_t launch_stream(bool swiglu, const uint16_t* x, const uint16_t* w, const int64_t* group_list,
                                int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* y, uint16_t* h,
                                int32_t* dev_err, hipStream_t stream, const GatherRows& g) {
    const size_t shmem = stream_lds_bytes(K, E);
    const int64_t blocks = max_sub_units(E, M_cap, N);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    // blocks past the call's sub-units exit at once
    const dim3 grid((unsigned)blocks);
    if (swiglu)
        hipLaunchKernelGGL(gmm_stream_kernel<true>, grid, dim3(kThreads), shmem, stream, x, w, group_list,
                           (int)E, M_cap, (int)K, (int)N, y, h, dev_err, g.slot, (int)g.top_k,
                           (int)g.nslots, RouteArgs{});
    else
        hipLaunchKernelGGL(gmm_stream_kernel<false>, grid, dim3(kThreads), shmem, stream, x, w, group_list,
                           (int)E, M_cap, (int)K, (int)N, y, nullptr, dev_err, g.slot, (int)g.top_k,
                           (int)g.nslots, RouteArgs{});
    return hipGetLastError();
}

hipError_t launch_gmm_stream(const uint16_t* x, const uint16_t* w, const int64_t* group_list,
                             int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* y,
                             int32_t* dev_err, hipStream_t stream, const GatherRows& g) {
    return launch_stream(false, x, w, group_list, E, M_cap, K, N, y, nullptr, dev_err, stream, g);
}

hipError_t launch_stream_swiglu_in(const uint16_t* h, const uint16_t* w2, const int64_t* group_list,
                                   int64_t E, int64_t M_cap, int64_t I, int64_t N, uint16_t* a, uint16_t* y,
                                   int32_t* dev_err, hipStream_t stream) {
    const size_t shmem = stream_lds_bytes(I, E);
    const int64_t blocks = max_sub_units(E, M_cap, N);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gmm_stream_kernel<false, true>), dim3((unsigned)blocks), dim3(kThreads), shmem, stream,
                       h, w2, group_list, (int)E, M_cap, (int)I, (int)N, y, a, dev_err, nullptr, 1, 0,
                       RouteArgs{});
    return hipGetLastError();
}

bool decode_fwd_applies(int64_t T, int64_t top_k, int64_t H, int64_t I, int64_t E) {
    const int64_t S = T * top_k;
    // both GMMs stage 4 rows of their reduction dim in at most 32 KiB; the
    // routing scans every slot in each block, so the slots stay few
    return S <= 8 * E && S <= 16384 && H * kStreamRows * 2 <= 32 * 1024 && I * kStreamRows * 2 <= 32 * 1024;
}

hipError_t launch_gmm_stream_route(const uint16_t* x, const int32_t* ids, int64_t T, int64_t top_k,
                                   const uint16_t* w1, int64_t E, int64_t K, int64_t N, uint16_t* h,
                                   int32_t* row_id_map, int32_t* sorted_slot, int64_t* tokens_per_expert,
                                   int32_t* dev_err, hipStream_t stream) {
    const int64_t S = T * top_k;
    RouteArgs ra;
    ra.ids = ids;
    ra.row_id_map = row_id_map;
    ra.sorted_slot = sorted_slot;
    ra.tokens_per_expert = tokens_per_expert;
    const int64_t blocks = max_sub_units(E, S, N);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gmm_stream_kernel<false, false, true>), dim3((unsigned)blocks), dim3(kThreads),
                       stream_lds_bytes(K, E), stream, x, w1, nullptr, (int)E, S, (int)K, (int)N, h, nullptr,
                       dev_err, nullptr, (int)top_k, (int)S, ra);
    return hipGetLastError();
}

hipError_t launch_gmm_stream_swiglu(const uint16_t* x, const uint16_t* w1,
                                    const int64_t* group_list, int64_t E, int64_t M_cap,
                                    int64_t K, int64_t I, uint16_t* a, uint16_t* h,
                                    int32_t* dev_err, hipStream_t stream, const GatherRows& g) {
    return launch_stream(true, x, w1, group_list, E, M_cap, K, 2 * I, a, h, dev_err, stream, g);
}

}  // namespace moegmm
