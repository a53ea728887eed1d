// Grouped matmul (GMM) kernels for gfx950: forward, input gradient and
// weight gradient over per-expert row ranges.
//
// What is computed ("NPU Training Operators - GMM", section 算子语义): for
// every expert e with n_e rows starting at off_e (exclusive cumulative sum of
// group_list, an empty expert owning an empty range),
//   forward       y[rows_e]  = x[rows_e] @ w[e]
//   input grad    dx[rows_e] = dy[rows_e] @ w[e]^T
//   weight grad   dw[e]      = x[rows_e]^T @ dy[rows_e]   (0 when n_e == 0)
//
// The kernels run on the MFMA tile engine of gmm_engine.h (operand staging,
// LDS ring, fragments, epilogues).
#include "gmm_engine.h"
#include "launch.h"
#include "moegmm.h"

namespace moegmm {

namespace {

// ---------------------------------------------------------------------------
// Row-grouped GEMM, three modes:
//   kFwd:    A = x [M_cap, K] (reduction-contiguous, ld K), B(q, j) = w[e][q][j]
//            (outer-contiguous, ld N); out y [M_cap, N]; reduction K.
//   kDx:     A = dy [M_cap, N] (ld N), B(q, j) = w[e][j][q] (reduction-
//            contiguous, ld N); out dx [M_cap, K]; reduction N.
//   kSwiGLU: the gate_up forward with N = 2I fused with SwiGLU: a tile covers
//            kBN/2 output columns c of a [M_cap, I], reading gate columns c
//            and up columns I + c of w[e]; optionally h [M_cap, 2I] too.
//
// Persistent workgroups, a multiple of 8 (workgroup b runs on XCD b % 8).
// XCD x owns a contiguous eighth of the logical tile order (expert, row tile,
// column tile), and its P workgroups take that range's tiles c, c + P,
// c + 2P, ...  The tiles an XCD runs at one time are then consecutive in that
// order and start together, so the row and weight panels they share come into
// its L2 once; with one workgroup per tile they started wherever a CU freed
// up.  Each workgroup reads group_list and builds the schedule once.
// ---------------------------------------------------------------------------
enum RowsMode { kFwd = 0, kDx = 1, kSwiGLU = 2 };

// Tile queue of the weight gradient, in the caller's workspace: one counter
// per XCD and a count of finished workgroups, 128 bytes apart.  The last
// workgroup to finish puts them back to zero, so the workspace is
// zero-filled again when the kernel ends.
constexpr int kQueueStride = 32;  // uint32 per slot
constexpr int kQueueWords = 9 * kQueueStride;
static_assert(kQueueWords * sizeof(uint32_t) == MOE_GMM_QUEUE_BYTES, "queue size in the header");

// GATHER (kFwd, kSwiGLU): A is the token matrix [nslots / top_k, K] and row r
// of the grouped operand is token slot[r] / top_k (RowGather); a separate
// instantiation, so the plain kernels carry none of it.
template <int MODE, bool GATHER = false>
__global__ __launch_bounds__(kThreads, kOccupancy) void gmm_rows_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, const int64_t* __restrict__ group_list,
    int E, int64_t M_cap, int K, int N, bf16_t* __restrict__ Y, bf16_t* __restrict__ Hout,
    int32_t* dev_err, const int32_t* __restrict__ slot, int top_k, int nslots) {
    constexpr bool IS_DX = MODE == kDx;
    constexpr int kCols = MODE == kSwiGLU ? kBN / 2 : kBN;  // output columns per tile
    // room for the ring of tall tiles (tall_tile_at)
    __shared__ __attribute__((aligned(1024))) bf16_t smem[kSmemTallElems];
    __shared__ int64_t s_scan[kThreads / 64];
    __shared__ int s_off[kMaxExperts], s_cnt[kMaxExperts], s_tst[kMaxExperts];
    const int Ncols = IS_DX ? K : (MODE == kSwiGLU ? N / 2 : N);  // output columns
    const int Kred = IS_DX ? N : K;                                 // reduction length
    const int NT = (Ncols + kCols - 1) / kCols;
    // the gather arguments pass through LDS so that they are read at each
    // tile's start rather than held in scalar registers across its steps
    __shared__ const int32_t* s_slot;
    __shared__ int32_t* s_err;
    __shared__ int s_gather[2];
    if (GATHER && threadIdx.x == 0) {
        s_slot = slot;
        s_err = dev_err;
        s_gather[0] = top_k;
        s_gather[1] = nslots;
    }
    load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, dev_err);
    // the plain forward and the input gradient run half-height tiles for an
    // expert's last <= 128 rows (MixedTile); the SwiGLU epilogue assumes
    // 256 x 256 tiles
    // 256 x 256 tiles, and only where that lowers the tile count of the
    // busiest workgroup (this schedule is static: a somewhat dearer half
    // tile that does not remove a tile round only lengthens it)
    // (and, like the SwiGLU forward, tall last tiles), whichever lowers the
    // round count more; tall tiles first where both tie
    constexpr bool kHalfTiles = MODE != kSwiGLU;
    const int NTH = (Ncols + kHN - 1) / kHN;
    int ntiles = (MODE == kSwiGLU ? tall_tile_starts(s_cnt, E, s_tst, s_scan)
                                  : row_tile_starts<kBM>(s_cnt, E, s_tst, s_scan)) * NT;
    bool use_half = false, use_tall = MODE == kSwiGLU;
    if constexpr (kHalfTiles) {
        const int per_wg = gridDim.x >> 3;
        const auto rounds = [&](int n) { return ((n + 7) / 8 + per_wg - 1) / per_wg; };
        const int nmixed = mixed_tile_count(s_cnt, E, NT, NTH, s_scan);
        const int ntall = tall_tile_count(s_cnt, E, s_scan) * NT;
        if (rounds(ntall) < rounds(ntiles) && rounds(ntall) <= rounds(nmixed)) {
            use_tall = true;
            ntiles = tall_tile_starts(s_cnt, E, s_tst, s_scan) * NT;
        } else if (rounds(nmixed) < rounds(ntiles)) {
            use_half = true;
            ntiles = mixed_tile_starts(s_cnt, E, NT, NTH, s_tst, s_scan);
        }
    }
    const XcdRange xr = xcd_range(blockIdx.x & 7, ntiles);
    for (int j = blockIdx.x >> 3; j < xr.count; j += gridDim.x >> 3) {
        int e, row0, rows_valid, nt;
        bool half = false;
        if (kHalfTiles && use_half) {
            const MixedTile mt = mixed_tile_at(s_off, s_cnt, s_tst, E, NT, xr.first + j);
            e = mt.e, row0 = mt.row0, rows_valid = mt.rows_valid, nt = mt.nt, half = mt.half;
        } else {
            const RowTile rt = use_tall ? tall_tile_at(s_off, s_cnt, s_tst, E, NT, xr.first + j)
                                        : row_tile_at<kBM>(s_off, s_cnt, s_tst, E, NT, xr.first + j);
            e = rt.e, row0 = rt.row0, rows_valid = rt.rows_valid, nt = rt.nt;
        }
        const int n0 = __builtin_amdgcn_readfirstlane(nt * (half ? kHN : kCols));

        const int64_t lda = IS_DX ? N : K;
        const bf16_t* We = W + (int64_t)e * K * N;
        const int cols_left = Ncols - n0;
        const bf16_t* a_base = GATHER ? A : A + (int64_t)row0 * lda;
        const RowGather ga{GATHER ? s_slot + row0 : nullptr, GATHER ? s_gather[0] : 1, GATHER ? s_gather[1] : 0,
                           GATHER ? s_err : nullptr};
        if constexpr (MODE == kSwiGLU) {
            bf16_t* y = Y + (int64_t)row0 * Ncols + n0;
            bf16_t* h = Hout ? Hout + (int64_t)row0 * N + n0 : nullptr;
            const int tile_cols = 2 * cols_left < kBN ? 2 * cols_left : kBN;
            auto st = [&](const auto& eng) { eng.store_swiglu(y, Ncols, h, N, Ncols, rows_valid, cols_left, smem); };
            if (rows_valid > kBM)
                gemm_tile<kTallM, kBN, kWM, kWN, true, false, kNST, kSmemTallElems>(
                    a_base, lda, rows_valid, We + n0, N, cols_left, Ncols, Kred, rows_valid, tile_cols, smem, st, ga);
            else
                gemm_tile<kBM, kBN, kWM, kWN, true, false>(a_base, lda, rows_valid, We + n0, N, cols_left, Ncols,
                                                          Kred, rows_valid, tile_cols, smem, st, ga);
        } else {
            bf16_t* y = Y + (int64_t)row0 * Ncols + n0;
            const bf16_t* b_base = IS_DX ? We + (int64_t)n0 * N : We + n0;
            auto st = [&](const auto& eng) { eng.store(y, Ncols, rows_valid, cols_left, smem); };
            if (half)
                gemm_tile<kHM, kHN, kHWM, kHWN, true, IS_DX, kHNST>(a_base, lda, rows_valid, b_base, N, cols_left,
                                                                    0, Kred, rows_valid, cols_left, smem, st, ga);
            else if (rows_valid > kBM)
                gemm_tile<kTallM, kBN, kWM, kWN, true, IS_DX, kNST, kSmemTallElems>(
                    a_base, lda, rows_valid, b_base, N, cols_left, 0, Kred, rows_valid, cols_left, smem, st, ga);
            else
                gemm_tile<kBM, kBN, kWM, kWN, true, IS_DX>(a_base, lda, rows_valid, b_base, N, cols_left, 0, Kred,
                                                          rows_valid, cols_left, smem, st, ga);
        }
        __syncthreads();  // every wave is done with its epilogue image before the next tile's copies
    }
}

// ---------------------------------------------------------------------------
// Weight gradient: dw[e] = x[rows_e]^T @ dy[rows_e].  Tiles (expert, k-tile,
// n-tile), experts in descending row count (ties by index) so the longest
// reductions start first.  Both operands are outer-contiguous; the reduction
// runs over the expert's rows, zero-filled past its last row.  Empty experts
// write zeros.
//
// Persistent workgroups (a multiple of 8, at most one per CU) take tiles from
// a queue.  Tile t belongs to XCD t % 8 (workgroup b runs on XCD b % 8), so
// each XCD has its own counter and, with KT*NT % 8 == 0, takes one kx x (8/kx)
// rectangle of every expert's (k-tile, n-tile) grid: its L2 then streams a
// few x and dy panels rather than nearly all of them.  A workgroup computes
// the schedule once and fetches its next tile while the current one runs;
// the per-tile cost of a fresh workgroup (group_list read, ranking, launch)
// matters here because most experts' tiles are short.
// ---------------------------------------------------------------------------
// Weight-gradient schedule, computed once per workgroup: s_order[r] = the
// expert of rank r (descending row count, ties by index) and the tile grid.
struct DwSched {
    int KT, NT, per_e, kx;  // kx: rectangle of kx k-tile bands x (8/kx) n-tile bands, or 0
};

MOE_DEVICE DwSched dw_schedule(const int* s_cnt, int E, int K, int N, int* s_order) {
    for (int e = threadIdx.x; e < E; e += kThreads) {
        const int c = s_cnt[e];
        int r = 0;
        for (int f = 0; f < E; ++f) {
            const int cf = s_cnt[f];
            r += (cf > c) || (cf == c && f < e);
        }
        s_order[r] = e;
    }
    DwSched ds;
    ds.KT = (K + kBM - 1) / kBM;
    ds.NT = (N + kBN - 1) / kBN;
    ds.per_e = ds.KT * ds.NT;
    ds.kx = 0;
    if (ds.per_e % 8 == 0) {
        int best = 0x7fffffff;
        for (int c = 1; c <= 8; c *= 2) {
            const int ny = 8 / c;
            if (ds.KT % c == 0 && ds.NT % ny == 0 && ds.KT / c + ds.NT / ny < best) {
                best = ds.KT / c + ds.NT / ny;
                ds.kx = c;
            }
        }
    }
    __syncthreads();
    return ds;
}

// Weight-gradient tile t (XCD t % 8): dw[e][k0.., n0..] over the expert's rows.
MOE_DEVICE void dw_tile(int t, const DwSched& ds, const int* s_off, const int* s_cnt, const int* s_order,
                        const bf16_t* __restrict__ X, const bf16_t* __restrict__ DY, int K, int N,
                        bf16_t* __restrict__ DW, bf16_t* smem) {
    const int rank = t / ds.per_e, rem = t % ds.per_e;
    int kt_out, nt;
    if (ds.kx) {
        const int ny = 8 / ds.kx, KTr = ds.KT / ds.kx, NTr = ds.NT / ny;
        const int x = rem & 7, p = rem >> 3;
        kt_out = (x / ny) * KTr + p / NTr;
        nt = (x % ny) * NTr + p % NTr;
    } else {
        kt_out = rem / ds.NT;
        nt = rem % ds.NT;
    }
    const int e = __builtin_amdgcn_readfirstlane(s_order[rank]);
    const int k0 = kt_out * kBM, n0 = nt * kBN;
    const int off = __builtin_amdgcn_readfirstlane(s_off[e]);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[e]);
    const int rows_valid = K - k0 < kBM ? K - k0 : kBM;
    const int cols_valid = N - n0 < kBN ? N - n0 : kBN;
    bf16_t* out = DW + ((int64_t)e * K + k0) * N + n0;
    if (cnt == 0) {
        constexpr int CPR = kBN / 8;
        for (int u = threadIdx.x; u < kBM * CPR; u += kThreads) {
            const int row = u / CPR, c = u % CPR;
            if (row < rows_valid && c * 8 < cols_valid)
                st16(out + (int64_t)row * N + c * 8, u32x4_t{0u, 0u, 0u, 0u});
        }
        return;
    }
    gemm_tile<kBM, kBN, kWM, kWN, false, false>(
        X + (int64_t)off * K + k0, K, rows_valid, DY + (int64_t)off * N + n0, N, cols_valid, 0, cnt,
        rows_valid, cols_valid, smem,
        [&](const auto& eng) { eng.store(out, N, rows_valid, cols_valid, smem); });
}

// Every counter fetch of the calling workgroup has returned; the last
// workgroup to get here resets the queue for the next call.  Thread 0 only.
MOE_DEVICE void queue_release(uint32_t* queue) {
    __threadfence();
    if (atomicAdd(queue + 8 * kQueueStride, 1u) == gridDim.x - 1) {
        for (int x = 0; x < 8; ++x) atomicExch(queue + x * kQueueStride, 0u);
        atomicExch(queue + 8 * kQueueStride, 0u);
    }
}

__global__ __launch_bounds__(kThreads, 1) void gmm_dw_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ DY, const int64_t* __restrict__ group_list,
    int E, int64_t M_cap, int K, int N, bf16_t* __restrict__ DW, uint32_t* __restrict__ queue,
    int32_t* dev_err) {
    __shared__ __attribute__((aligned(1024))) bf16_t smem[kSmemElems];
    __shared__ int64_t s_scan[kThreads / 64];
    __shared__ int s_off[kMaxExperts], s_cnt[kMaxExperts], s_order[kMaxExperts];
    __shared__ uint32_t s_next;

    load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, dev_err);
    const DwSched ds = dw_schedule(s_cnt, E, K, N, s_order);
    const int total = E * ds.per_e;
    const int xcd = blockIdx.x & 7, wg_per_xcd = gridDim.x >> 3;
    const uint32_t mine = (uint32_t)((total - xcd + 7) / 8);  // tiles 8j + xcd, j < mine
    uint32_t* ctr = queue + xcd * kQueueStride;
    // Queue positions are unsigned and bounded by `mine` before use: a
    // workspace that was not zero-filled gives skipped or repeated tiles,
    // never an index outside the tile grid.
    uint32_t j = blockIdx.x >> 3;  // first tile static, later ones from the counter
    while (j < mine) {
        uint32_t nj = 0;
        if (threadIdx.x == 0) nj = (uint32_t)wg_per_xcd + atomicAdd(ctr, 1u);
        dw_tile(8 * (int)j + xcd, ds, s_off, s_cnt, s_order, X, DY, K, N, DW, smem);
        if (threadIdx.x == 0) s_next = nj;
        __syncthreads();  // the ring and the output image are free again
        j = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_next);
    }
    if (threadIdx.x == 0) queue_release(queue);
}

// ---------------------------------------------------------------------------
// Weight gradient with the row reduction split, for calls whose tile grid
// (E * KT * NT tiles) cannot fill the CUs -- one large dense expert, or a
// few experts with small K and N.  Two launches:
//   1. work item (tile t, chunk c) reduces chunk c of the expert's rows and
//      stores its fp32 partial in the caller's workspace (a tile whose
//      expert has one chunk writes its output directly);
//   2. eight workgroups per split tile add the tile's partials in chunk
//      order and write it as bf16 -- so the result does not depend on
//      where or when the chunks ran.
// Chunks have at least kMinChunkRows rows: an expert with few rows gets
// fewer chunks.  Partials keep the accumulator layout (4 consecutive columns
// of accumulator (i, j), group g, of wave w, lane l, as the float4 at
// ((w * TM*TN + i * TN + j) * 4 + g) * 64 + l), so every load and store of
// them moves 1 KiB per wave instruction.
// ---------------------------------------------------------------------------
constexpr int kTileFloats = kBM * kBN;
constexpr int kMinChunkRows = 256;  // shorter chunks would be mostly prologue and epilogue
constexpr int kReducePieces = 8;    // workgroups per tile in the reduction
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN, kTM = kWTM / 32, kTN = kWTN / 32;

// Chunk rows and chunk count of an expert with cnt rows, split at most S ways.
struct DwChunks {
    int rows, count;
};
MOE_DEVICE DwChunks dw_chunks(int cnt, int S) {
    int cr = (cnt + S - 1) / S;
    cr = (cr + BK - 1) / BK * BK;
    if (cr < kMinChunkRows) cr = kMinChunkRows;
    return DwChunks{cr, (cnt + cr - 1) / cr};
}

__global__ __launch_bounds__(kThreads, 1) void gmm_dw_split_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ DY, const int64_t* __restrict__ group_list,
    int E, int64_t M_cap, int K, int N, bf16_t* __restrict__ DW, int S, float* __restrict__ part,
    int32_t* dev_err) {
    __shared__ __attribute__((aligned(1024))) bf16_t smem[kSmemElems];
    __shared__ int64_t s_scan[kThreads / 64];
    __shared__ int s_off[kMaxExperts], s_cnt[kMaxExperts];

    load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, dev_err);
    const int KT = (K + kBM - 1) / kBM, NT = (N + kBN - 1) / kBN;
    const int t = blockIdx.x / S, c = blockIdx.x % S;
    const int e = t / (KT * NT), rem = t % (KT * NT);
    const int k0 = (rem / NT) * kBM, n0 = (rem % NT) * kBN;
    const int off = s_off[e], cnt = s_cnt[e];
    const int rows_valid = K - k0 < kBM ? K - k0 : kBM;
    const int cols_valid = N - n0 < kBN ? N - n0 : kBN;
    bf16_t* out = DW + ((int64_t)e * K + k0) * N + n0;
    if (cnt == 0) {  // exact zeros, written by chunk 0
        if (c != 0) return;
        constexpr int CPR = kBN / 8;
        for (int u = threadIdx.x; u < kBM * CPR; u += kThreads) {
            const int row = u / CPR, cc = u % CPR;
            if (row < rows_valid && cc * 8 < cols_valid)
                st16(out + (int64_t)row * N + cc * 8, u32x4_t{0u, 0u, 0u, 0u});
        }
        return;
    }
    const DwChunks ch = dw_chunks(cnt, S);
    if (c >= ch.count) return;  // uniform
    const int r0 = c * ch.rows, rl = cnt - r0 < ch.rows ? cnt - r0 : ch.rows;
    float* slot = part + ((int64_t)t * S + c) * kTileFloats;
    gemm_tile<kBM, kBN, kWM, kWN, false, false>(
        X + (int64_t)(off + r0) * K + k0, K, rows_valid, DY + (int64_t)(off + r0) * N + n0, N, cols_valid, 0, rl,
        rows_valid, cols_valid, smem, [&](const auto& eng) {
            if (ch.count == 1) {
                eng.store(out, N, rows_valid, cols_valid, smem);
                return;
            }
            static_assert(std::remove_reference_t<decltype(eng)>::TM == kTM &&
                              std::remove_reference_t<decltype(eng)>::TN == kTN, "tile shape");
            const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
            f32x4_t* p = reinterpret_cast<f32x4_t*>(slot) + wid * (kTM * kTN * 4 * 64) + lane;
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        p[((i * kTN + j) * 4 + g) * 64] = f32x4_t{eng.acc[i][j][4 * g], eng.acc[i][j][4 * g + 1],
                                                                  eng.acc[i][j][4 * g + 2], eng.acc[i][j][4 * g + 3]};
        });
}

// Reduction of the split tiles: workgroup (tile t, piece p) takes float4s
// [p, p + 1) * 2048 of each of the tile's partials, adds them in chunk
// order and writes its 4 bf16 columns per float4.
constexpr int kReduceThreads = 256;
__global__ __launch_bounds__(kReduceThreads) void gmm_dw_reduce_kernel(
    const int64_t* __restrict__ group_list, int E, int64_t M_cap, int K, int N, bf16_t* __restrict__ DW, int S,
    const float* __restrict__ part) {
    __shared__ int64_t s_scan[kReduceThreads / 64];
    __shared__ int s_off[kMaxExperts], s_cnt[kMaxExperts];
    load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, nullptr);
    const int KT = (K + kBM - 1) / kBM, NT = (N + kBN - 1) / kBN;
    const int t = blockIdx.x / kReducePieces, piece = blockIdx.x % kReducePieces;
    const int e = t / (KT * NT), rem = t % (KT * NT);
    const int cnt = s_cnt[e];
    if (cnt == 0) return;
    const DwChunks ch = dw_chunks(cnt, S);
    if (ch.count == 1) return;  // written by its only chunk
    const int k0 = (rem / NT) * kBM, n0 = (rem % NT) * kBN;
    const int rows_valid = K - k0 < kBM ? K - k0 : kBM;
    const int cols_valid = N - n0 < kBN ? N - n0 : kBN;
    bf16_t* out = DW + ((int64_t)e * K + k0) * N + n0;
    constexpr int kF4 = kTileFloats / 4, kPer = kF4 / kReducePieces / kReduceThreads;
    const f32x4_t* base = reinterpret_cast<const f32x4_t*>(part + (int64_t)t * S * kTileFloats);
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
        const int u = piece * (kF4 / kReducePieces) + it * kReduceThreads + threadIdx.x;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        for (int cc = 0; cc < ch.count; ++cc) v += base[(int64_t)cc * kF4 + u];
        // float4 u of the accumulator layout -> (row, 4 columns) of the tile
        const int lane = u & 63, g = (u >> 6) & 3, ij = (u >> 8) % (kTM * kTN), w = (u >> 8) / (kTM * kTN);
        const int i = ij / kTN, j = ij % kTN;
        const int row = (w / kWN) * kWTM + i * 32 + (lane & 31);
        const int col = (w % kWN) * kWTN + j * 32 + 8 * g + 4 * (lane >> 5);
        if (row < rows_valid && col < cols_valid) {
            u32x2_t pk;
            pk[0] = pack_bf16x2(v[0], v[1]);
            pk[1] = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<u32x2_t*>(out + (int64_t)row * N + col) = pk;
        }
    }
}

// ---------------------------------------------------------------------------
// Both gradients of one grouped matmul in one launch: dx = dy @ w[e]^T (row
// tiles, as gmm_rows_kernel<kDx>) and dw[e] = x^T @ dy (as gmm_dw_kernel).
// Each XCD's queue hands out its share of the input-gradient tiles first (a
// contiguous eighth of the row-tile order, so neighbouring tiles share an
// L2) and then its weight-gradient tiles.  The many short weight-gradient
// tiles fill the CUs that the input gradient's last, partial round of long
// tiles leaves idle, which two separate launches cannot do.
// ---------------------------------------------------------------------------
//
// SWIGLU_BWD: the input gradient is dA of the down GMM and its tiles go out
// through the SwiGLU backward (Engine::store_swiglu_bwd): dH = [dG | dU]
// from dA and H = [G | U] ([M_cap, 2K]) is written instead of dA.
template <bool SWIGLU_BWD>
__global__ __launch_bounds__(kThreads, 1) void gmm_bwd_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ DY, const bf16_t* __restrict__ W,
    const int64_t* __restrict__ group_list, int E, int64_t M_cap, int K, int N,
    bf16_t* __restrict__ DX, bf16_t* __restrict__ DW, const bf16_t* Hin, bf16_t* DH,
    uint32_t* __restrict__ queue, int32_t* dev_err) {
    __shared__ __attribute__((aligned(1024))) bf16_t smem[kSmemElems];
    __shared__ int64_t s_scan[kThreads / 64];
    __shared__ int s_off[kMaxExperts], s_cnt[kMaxExperts], s_order[kMaxExperts], s_tst[kMaxExperts];
    __shared__ uint32_t s_next;

    load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, dev_err);
    const DwSched ds = dw_schedule(s_cnt, E, K, N, s_order);
    const int NTx = (K + kBN - 1) / kBN;  // dx has K columns
    const int nx = mixed_tile_starts(s_cnt, E, NTx, (K + kHN - 1) / kHN, s_tst, s_scan);
    const int xcd = blockIdx.x & 7, wg_per_xcd = gridDim.x >> 3;
    // this XCD's input-gradient tiles: [x0, x0 + nxx) of the row-tile order
    const XcdRange xr = xcd_range(xcd, nx);
    const int x0 = xr.first, nxx = xr.count;
    const int mine_w = (E * ds.per_e - xcd + 7) / 8;
    const uint32_t items = (uint32_t)(nxx + mine_w);
    uint32_t* ctr = queue + xcd * kQueueStride;
    // unsigned queue positions, bounded before use (see gmm_dw_kernel)
    uint32_t j = blockIdx.x >> 3;
    while (j < items) {
        uint32_t nj = 0;
        if (threadIdx.x == 0) nj = (uint32_t)wg_per_xcd + atomicAdd(ctr, 1u);
        if (j < (uint32_t)nxx) {
            const MixedTile mt = mixed_tile_at(s_off, s_cnt, s_tst, E, NTx, x0 + (int)j);
            const int row0 = mt.row0, rows_valid = mt.rows_valid;
            const int n0 = __builtin_amdgcn_readfirstlane(mt.nt * (mt.half ? kHN : kBN));
            const int cols_left = K - n0;
            const bf16_t* We = W + (int64_t)mt.e * K * N;
            auto st = [&](const auto& eng) {
                if constexpr (SWIGLU_BWD) {
                    const int64_t o = (int64_t)row0 * 2 * K + n0;
                    eng.store_swiglu_bwd(DH + o, Hin + o, 2 * K, K, rows_valid, cols_left, smem);
                } else {
                    eng.store(DX + (int64_t)row0 * K + n0, K, rows_valid, cols_left, smem);
                }
            };
            if (mt.half)
                gemm_tile<kHM, kHN, kHWM, kHWN, true, true, kHNST>(DY + (int64_t)row0 * N, N, rows_valid,
                                                                   We + (int64_t)n0 * N, N, cols_left, 0, N,
                                                                   rows_valid, cols_left, smem, st);
            else
                gemm_tile<kBM, kBN, kWM, kWN, true, true>(DY + (int64_t)row0 * N, N, rows_valid,
                                                          We + (int64_t)n0 * N, N, cols_left, 0, N, rows_valid,
                                                          cols_left, smem, st);
        } else {
            dw_tile(8 * ((int)j - nxx) + xcd, ds, s_off, s_cnt, s_order, X, DY, K, N, DW, smem);
        }
        if (threadIdx.x == 0) s_next = nj;
        __syncthreads();  // the ring and the output image are free again
        j = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_next);
    }
    if (threadIdx.x == 0) queue_release(queue);
}

}  // namespace

int num_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Chunks per tile of the split weight gradient: 1 (no split) when the tile
// grid has at least half a workgroup per CU, else enough chunks to give
// every CU about one work item -- at most 32, and no more than chunks of
// kMinChunkRows rows that M_cap rows could fill.
static int dw_split_chunks(int64_t E, int64_t M_cap, int64_t K, int64_t N) {
    const int64_t tiles = E * ((K + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const int64_t cus = num_cus();
    if (tiles * 2 > cus) return 1;
    int64_t S = cus / tiles;
    if (S > 32) S = 32;
    const int64_t fill = (M_cap + kMinChunkRows - 1) / kMinChunkRows;
    if (S > fill) S = fill;
    return S < 2 ? 1 : (int)S;
}

// Workspace of the weight-gradient calls: the tile queue (kQueueWords; it
// must start zero-filled and is left so), then, for gmm_bwd_weight on a
// grid it splits, the fp32 partials (chunks x tiles x kBM x kBN) from byte
// kPartOffset on, scratch whose contents do not matter between calls.
constexpr size_t kPartOffset = 2048;
size_t gmm_workspace_bytes(int64_t E, int64_t M_cap, int64_t K, int64_t N, int op) {
    if (op == MOE_GMM_OP_BWD) return kQueueWords * sizeof(uint32_t);
    if (op != MOE_GMM_OP_BWD_WEIGHT) return 0;
    const int S = dw_split_chunks(E, M_cap, K, N);
    if (S == 1) return kQueueWords * sizeof(uint32_t);
    const int64_t tiles = E * ((K + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    return kPartOffset + (size_t)tiles * S * kTileFloats * sizeof(float);
}

hipError_t launch_gmm_fwd(const uint16_t* x, const uint16_t* w, const int64_t* group_list,
                          int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* y, void*,
                          int32_t* dev_err, hipStream_t stream, const GatherRows& g) {
    if (M_cap == 0) return hipSuccess;
    if (gmm_stream_applies(E, M_cap, K))
        return launch_gmm_stream(x, w, group_list, E, M_cap, K, N, y, dev_err, stream, g);
    const int64_t grid = num_cus() / 8 * 8;  // persistent, see gmm_rows_kernel
    if (g.slot)
        hipLaunchKernelGGL((gmm_rows_kernel<kFwd, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, x,
                           w, group_list, (int)E, M_cap, (int)K, (int)N, y, nullptr, dev_err, g.slot,
                           (int)g.top_k, (int)g.nslots);
    else
        hipLaunchKernelGGL(gmm_rows_kernel<kFwd>, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, w,
                           group_list, (int)E, M_cap, (int)K, (int)N, y, nullptr, dev_err, nullptr, 1, 0);
    return hipGetLastError();
}

hipError_t launch_gmm_bwd_input(const uint16_t* dy, const uint16_t* w, const int64_t* group_list,
                                int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dx,
                                void*, int32_t* dev_err, hipStream_t stream) {
    if (M_cap == 0) return hipSuccess;
    const int64_t grid = num_cus() / 8 * 8;  // persistent, see gmm_rows_kernel
    hipLaunchKernelGGL(gmm_rows_kernel<kDx>, dim3((unsigned)grid), dim3(kThreads), 0, stream, dy, w,
                       group_list, (int)E, M_cap, (int)K, (int)N, dx, nullptr, dev_err, nullptr, 1, 0);
    return hipGetLastError();
}

hipError_t launch_gmm_bwd_weight(const uint16_t* x, const uint16_t* dy, const int64_t* group_list,
                                 int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dw,
                                 void* ws, int32_t* dev_err, hipStream_t stream) {
    const int64_t tiles = E * ((K + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const int S = dw_split_chunks(E, M_cap, K, N);
    if (S > 1) {
        float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + kPartOffset);
        hipLaunchKernelGGL(gmm_dw_split_kernel, dim3((unsigned)(tiles * S)), dim3(kThreads), 0, stream, x, dy,
                           group_list, (int)E, M_cap, (int)K, (int)N, dw, S, part, dev_err);
        hipLaunchKernelGGL(gmm_dw_reduce_kernel, dim3((unsigned)(tiles * kReducePieces)), dim3(kReduceThreads), 0,
                           stream, group_list, (int)E, M_cap, (int)K, (int)N, dw, S, part);
        return hipGetLastError();
    }
    const int64_t need = (tiles + 7) / 8 * 8;
    int64_t grid = num_cus() / 8 * 8;
    if (grid > need) grid = need;
    hipLaunchKernelGGL(gmm_dw_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, dy,
                       group_list, (int)E, M_cap, (int)K, (int)N, dw, static_cast<uint32_t*>(ws),
                       dev_err);
    return hipGetLastError();
}

hipError_t launch_gmm_bwd(const uint16_t* x, const uint16_t* dy, const uint16_t* w,
                          const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K, int64_t N,
                          uint16_t* dx, uint16_t* dw, void* ws, int32_t* dev_err, hipStream_t stream) {
    hipLaunchKernelGGL(gmm_bwd_kernel<false>, dim3((unsigned)(num_cus() / 8 * 8)), dim3(kThreads), 0,
                       stream, x, dy, w, group_list, (int)E, M_cap, (int)K, (int)N, dx, dw, nullptr,
                       nullptr, static_cast<uint32_t*>(ws), dev_err);
    return hipGetLastError();
}

hipError_t launch_gmm_bwd_swiglu(const uint16_t* x, const uint16_t* dy, const uint16_t* w,
                                 const uint16_t* h, const int64_t* group_list, int64_t E, int64_t M_cap,
                                 int64_t K, int64_t N, uint16_t* dh, uint16_t* dw, void* ws,
                                 int32_t* dev_err, hipStream_t stream) {
    hipLaunchKernelGGL(gmm_bwd_kernel<true>, dim3((unsigned)(num_cus() / 8 * 8)), dim3(kThreads), 0,
                       stream, x, dy, w, group_list, (int)E, M_cap, (int)K, (int)N, nullptr, dw, h, dh,
                       static_cast<uint32_t*>(ws), dev_err);
    return hipGetLastError();
}

hipError_t launch_gmm_fwd_swiglu(const uint16_t* x, const uint16_t* w1, const int64_t* group_list,
                                 int64_t E, int64_t M_cap, int64_t K, int64_t I, uint16_t* a,
                                 uint16_t* h, void*, int32_t* dev_err, hipStream_t stream,
                                 const GatherRows& g) {
    if (M_cap == 0) return hipSuccess;
    if (gmm_stream_applies(E, M_cap, K))
        return launch_gmm_stream_swiglu(x, w1, group_list, E, M_cap, K, I, a, h, dev_err, stream, g);
    const int64_t grid = num_cus() / 8 * 8;  // persistent, see gmm_rows_kernel
    if (g.slot)
        hipLaunchKernelGGL((gmm_rows_kernel<kSwiGLU, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           x, w1, group_list, (int)E, M_cap, (int)K, (int)(2 * I), a, h, dev_err, g.slot,
                           (int)g.top_k, (int)g.nslots);
    else
        hipLaunchKernelGGL(gmm_rows_kernel<kSwiGLU>, dim3((unsigned)grid), dim3(kThreads), 0, stream, x,
                           w1, group_list, (int)E, M_cap, (int)K, (int)(2 * I), a, h, dev_err, nullptr, 1, 0);
    return hipGetLastError();
}

}  // namespace moegmm
