// MXFP8 grouped matmul kernels for gfx950 (the A8W8-FP variant of the
// expert block).
//
// What is computed ("MegaMoE", A8W8-FP scenario): operands are MX-quantised
// in groups of 32 along the reduction dimension -- E4M3 codes plus one E8M0
// scale per group -- and the matmul dequantises inside:
//   gmm_mx        y[rows_e]  = DQ(x[rows_e]) @ DQ(w[e])^T          (bf16 out)
//   gmm_mx_swiglu [G | U]    = DQ(x[rows_e]) @ DQ(w1[e])^T,
//                 A = SiLU(G) * U,  (aq, as) = Q_MX(A)     (MX out, for GMM2)
// Weights are stored reduction-contiguous, w[e] as [N][K] codes with scales
// [N][ld] (the parameter table of that scenario gives the hidden size as the
// last dimension of weight1); x is [M][K] codes with scales [M][ld].  Scale
// rows are padded to a multiple of 16 bytes; bytes past ceil(K/32) are never
// used.  For gmm_mx_swiglu, w1[e] holds the I gate rows, then the I up rows.
//
// Design: the bf16 tile engine (gmm_engine.h) carries over with fp8 bytes in
// place of bf16 pairs.  A 64-byte LDS row of one stage holds 64 reduction
// elements -- two MX groups -- and feeds one v_mfma_scale_f32_32x32x64_f8f6f4
// per fragment pair: lane l holds half of each of the two groups of row
// l%32 (two ds_read_b128) and passes the scale byte of group l/32 to the
// MFMA, which applies both operands' 2^(s-127) to the exact fp8 products.  So a stage
// moves the same bytes as a bf16 stage and the MFMAs take the same time, for
// twice the flops.  Scales travel HBM -> LDS as their own 16-byte-per-lane DMA
// (one instruction per wave every 8 steps covers 16 groups of all 256 A rows
// and 256 B rows) into a two-slot ring beside the operand ring.
#include "gmm_engine.h"
#include "launch.h"
#include "route.h"
#include "mx.h"

namespace moegmm {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));

MOE_DEVICE u32x8_t u32x8_t_of(u32x4_t lo, u32x4_t hi) {
    return u32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

static_assert(BK == 32, "an MX stage is 64 bytes: two scale groups");
static_assert(kThreads == kBM + kBN, "one scale row per thread");
constexpr int kStepsPerScaleLoad = 8;                    // 16 groups of 32 = 8 steps of 64
constexpr int kScaleSlot = (kBM + kBN) * 16;             // bytes per scale slot

// ---------------------------------------------------------------------------
// Scale rows HBM -> LDS.  Thread t < kBM loads 16 scale bytes of A row t,
// thread kBM + t those of B row t (with the gate/up pairing of Dma::init);
// LDS slot layout: [kBM A rows][16] then [kBN B rows][16].
// ---------------------------------------------------------------------------
struct ScaleDma {
    uint32_t off;
    bool ok;

    // gather.slot: A row t is token gather.slot[t] / top_k (RowGather; the
    // code DMA reports bad entries, this one just loads no scales for them)
    MOE_DEVICE void init(int64_t ld_a, int a_olim, int64_t ld_b, int b_olim, int b_pair,
                         const RowGather& gather) {
        const int t = threadIdx.x;
        if (t < kBM) {
            off = (uint32_t)(t * ld_a);
            ok = t < a_olim;
            if (gather.slot && ok) {
                const int sl = gather.slot[t];
                ok = sl >= 0 && sl < gather.nslots;
                off = ok ? (uint32_t)((int64_t)(sl / gather.top_k) * ld_a) : 0u;
            }
        } else {
            const int o = t - kBM;
            int vo = o, go = o;
            if (b_pair > 0) {
                vo = (o >> 6) * 32 + (o & 31);
                go = ((o >> 5) & 1) * b_pair + vo;
            }
            off = (uint32_t)(go * ld_b);
            ok = vo < b_olim;
        }
    }
    // group g: scale bytes 16g .. 16g+15 of every row; nblocks = ceil(K/32)
    MOE_DEVICE void issue(const uint8_t* a_sc, const uint8_t* b_sc, int g, int nblocks,
                          uint8_t* slot) const {
        const int wid = wave_id();
        const uint8_t* base = (wid < kBM / 64 ? a_sc : b_sc) + 16 * g;
        const uint32_t v = ok && 16 * g < nblocks ? off : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base), (LDS_AS void*)(slot + wid * 1024),
                                                 16, v, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// The MX engine: the bf16 engine's accumulators and epilogues, fed by scaled
// fp8 MFMAs.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN>
struct EngineMx : Engine<BM, BN, WM, WN, true, true> {
    using Base = Engine<BM, BN, WM, WN, true, true>;
    static constexpr int TM = Base::TM, TN = Base::TN, WTM = Base::WTM, WTN = Base::WTN;
    static_assert(TM % 2 == 0, "fragments are read in two halves");

    // The operand layout of the 32x32x64 fp8 MFMA: lane l holds row l%32,
    // reduction elements 16*(l/32) .. +15 in its first four registers and
    // 32 + 16*(l/32) .. +15 in the last four; the scale lane l passes is
    // that of group l/32 of its row (elements 32*(l/32) .. +31), which lanes
    // l and l^32 share.  So lane l reads logical 16-byte chunks l/32 and
    // l/32 + 2 of the 64-byte stage row -- the chunks the bf16 engine reads
    // for its two 16-deep sub-steps.
    static MOE_DEVICE void frag(i32x8_t& v, const bf16_t* lds, int o0) {
        const int lane = threadIdx.x & 63;
        const int o = o0 + (lane & 31);
        const int c = lane >> 5;
        const int sw = swz_k(o);
        u32x4_t lo, hi;
        asm volatile("ds_read_b128 %0, %1" : "=v"(lo) : "v"(lds_addr(lds + o * BK + ((c ^ sw) << 3))));
        asm volatile("ds_read_b128 %0, %1"
                     : "=v"(hi)
                     : "v"(lds_addr(lds + o * BK + (((c + 2) ^ sw) << 3))));
        v = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    static MOE_DEVICE void scale(uint32_t& s, const uint8_t* sl, int o0, int kb) {
        const int o = o0 + (threadIdx.x & 31);
        asm volatile("ds_read_u8 %0, %1" : "=v"(s) : "v"(lds_addr(sl + o * 16 + kb)));
    }

    // One 64-element step.  kb: this lane's group within the scale slot;
    // kb_ok false for a group past ceil(K/32) (its codes are zero; its scale
    // byte, padding, is replaced by 2^0).  NA: the wave's 32-row fragments
    // with valid rows; the others skip their reads and MFMAs (every hook
    // still runs).
    template <int NA = TM, class Hook>
    MOE_DEVICE void compute(const bf16_t* la, const bf16_t* lb, const uint8_t* sla, const uint8_t* slb,
                            int kb, bool kb_ok, Hook& hook) {
        static_assert(NA >= 1 && NA <= TM, "active fragments");
        const int wid = threadIdx.x >> 6;
        const int wm = wid / WN, wn = wid % WN;
        i32x8_t a[TM], b[TN];
        uint32_t sa[TM], sb[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            frag(b[j], lb, wn * WTN + j * 32);
            scale(sb[j], slb, wn * WTN + j * 32, kb);
        }
#pragma unroll
        for (int i = 0; i < TM / 2; ++i) {
            if (i >= NA) continue;
            frag(a[i], la, wm * WTM + i * 32);
            scale(sa[i], sla, wm * WTM + i * 32, kb);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(b[j]), "+v"(sb[j]));
#pragma unroll
        for (int i = 0; i < TM / 2; ++i)
            if (i < NA) asm volatile("" : "+v"(a[i]), "+v"(sa[i]));
#pragma unroll
        for (int i = TM / 2; i < TM; ++i) {
            if (i >= NA) continue;
            frag(a[i], la, wm * WTM + i * 32);
            scale(sa[i], sla, wm * WTM + i * 32, kb);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) sb[j] = kb_ok ? sb[j] : 127u;
#pragma unroll
        for (int i = 0; i < TM / 2; ++i) sa[i] = kb_ok ? sa[i] : 127u;
        mfmas<NA>(a, b, sa, sb, 0, TM / 2, hook);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = TM / 2; i < TM; ++i) {
            if (i >= NA) continue;
            asm volatile("" : "+v"(a[i]), "+v"(sa[i]));
            sa[i] = kb_ok ? sa[i] : 127u;
        }
        mfmas<NA>(a, b, sa, sb, TM / 2, TM, hook);
    }

    template <int NA, class Hook>
    MOE_DEVICE void mfmas(const i32x8_t (&a)[TM], const i32x8_t (&b)[TN], const uint32_t (&sa)[TM],
                          const uint32_t (&sb)[TN], int i0, int i1, Hook& hook) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                // operands swapped, as in the bf16 engine: B is the hardware A
                if (i < NA)
                    this->acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        b[j], a[i], this->acc[i][j], 0, 0, 0, (int)sb[j], 0, (int)sa[i]);
                hook(i * TN + j);
            }
    }

    // Gate_up tile with paired rows: A = SiLU(G) * U in fp32, then Q_MX over
    // each row's 32 columns of this wave (one MX group: this lane's 16 values
    // and those of lane l^32).  Writes codes to aq (ld bytes) and the group's
    // scale byte to as[row][blk0 + wn].
    MOE_DEVICE void store_swiglu_mx(uint8_t* __restrict__ aq, int64_t ldq, uint8_t* __restrict__ as,
                                    int64_t ld_as, int blk0, int rows_valid, int cols_valid) const {
        static_assert(TN == 2, "one gate and one up fragment per wave");
        const int lane = threadIdx.x & 63;
        const int wid = threadIdx.x >> 6;
        const int wm = wid / WN, wn = wid % WN;
        if (wn * 32 >= cols_valid) return;  // uniform across the wave
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 32 + (lane & 31);
            float av[16];
            float amax = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float gv = this->acc[i][0][r], uv = this->acc[i][1][r];
                av[r] = gv * silu_sigmoid(gv) * uv;
                amax = fmaxf(amax, fabsf(av[r]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
            const uint32_t sbyte = mx_scale_byte(amax);
            const float inv = mx_inv_scale(sbyte);
            if (row < rows_valid) {
                uint8_t* orow = aq + (int64_t)row * ldq + wn * 32 + (lane >> 5) * 4;
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<uint32_t*>(orow + g * 8) =
                        e4m3_pack4(av[4 * g] * inv, av[4 * g + 1] * inv, av[4 * g + 2] * inv,
                                   av[4 * g + 3] * inv);
                if (lane < 32) as[(int64_t)row * ld_as + blk0 + wn] = (uint8_t)sbyte;
            }
        }
    }
};

// One output tile over the ring, as gemm_tile (gmm_engine.h), plus the scale
// ring: the scale group of step s (s/8) sits in slot (s/8)&1, loaded ahead
// with the operands of its first step.  Every wave issues the same loads in
// the same order, so the vmcnt wait of gemm_tile still covers step s: a
// scale load among the newer loads only makes that wait conservative.
template <int BM, int BN, int WM, int WN, class Store>
MOE_DEVICE void gemm_tile_mx(const uint8_t* a_base, int a_olim, const uint8_t* a_sc, int64_t ld_as,
                             const uint8_t* b_base, int b_olim, int b_pair, const uint8_t* b_sc,
                             int64_t ld_bs, int K, int rows_valid, int cols_valid, bf16_t* smem,
                             uint8_t* ssc, const Store& store,
                             const RowGather& gather = RowGather{nullptr, 1, 0, nullptr}) {
    using DA = Dma<BM, true>;
    using DB = Dma<BN, true>;
    constexpr int kStage = (BM + BN) * BK;
    constexpr int kPer = DA::kInst + DB::kInst;
    const bf16_t* a16 = reinterpret_cast<const bf16_t*>(a_base);
    const bf16_t* b16 = reinterpret_cast<const bf16_t*>(b_base);
    const int64_t ld16 = K / 2;  // row length in 2-byte units
    const int red = K / 2;
    const int nblocks = K / kMxGroup;
    DA da;
    DB db;
    ScaleDma sd;
    if (gather.slot) da.init_gather(ld16, a_olim, gather);
    else da.init(ld16, a_olim);
    db.init(ld16, b_olim, b_pair);
    sd.init(ld_as, a_olim, ld_bs, b_olim, b_pair, gather);
    EngineMx<BM, BN, WM, WN> eng;
    eng.zero();
    const int nk = (red + BK - 1) / BK;
    auto issue = [&](int step) {
        bf16_t* st = smem + (step % kNST) * kStage;
        da.issue(DA::stage(a16, ld16, step), st, red - step * BK);
        db.issue(DB::stage(b16, ld16, step), st + BM * BK, red - step * BK);
    };
    constexpr int kMfmaPerStep = EngineMx<BM, BN, WM, WN>::TM * EngineMx<BM, BN, WM, WN>::TN;
    static_assert(kMfmaPerStep >= kPer, "load spacing");
    sd.issue(a_sc, b_sc, 0, nblocks, ssc);
#pragma unroll
    for (int p = 0; p < kNST - 1; ++p) issue(p);
    const int lane_grp = (threadIdx.x >> 5) & 1;
    const int wrow0 = (wave_id() / WN) * (BM / WM), wcol0 = (wave_id() % WN) * (BN / WN);
    auto run_steps = [&](auto active_tag) {
        for (int s = 0; s < nk; ++s) {
            wait_vmcnt<(kNST - 2) * kPer>();
            __builtin_amdgcn_s_barrier();
            const int nxt = s + kNST - 1;
            if (nxt % kStepsPerScaleLoad == 0) {
                const int g = nxt / kStepsPerScaleLoad;
                sd.issue(a_sc, b_sc, g, nblocks, ssc + (g & 1) * kScaleSlot);
            }
            bf16_t* nst = smem + (nxt % kNST) * kStage;
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(DA::stage(a16, ld16, nxt));
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(DB::stage(b16, ld16, nxt));
            const int left = red - nxt * BK;
            auto hook = [&](int m) {
#pragma unroll
                for (int q = 0; q < kPer; ++q) {
                    if (m == (q + 1) * kMfmaPerStep / kPer - 1) {
                        if (q < DA::kInst) da.issue_one(q, ra, nst, left);
                        else db.issue_one(q - DA::kInst, rb, nst + BM * BK, left);
                    }
                }
            };
            if constexpr (decltype(active_tag)::value > 0) {
                const bf16_t* st = smem + (s % kNST) * kStage;
                const uint8_t* sl = ssc + ((s / kStepsPerScaleLoad) & 1) * kScaleSlot;
                const int kb = 2 * s + lane_grp;
                eng.template compute<decltype(active_tag)::value>(st, st + BM * BK, sl, sl + BM * 16,
                                                                  kb & 15, kb < nblocks, hook);
            } else {
#pragma unroll
                for (int m = 0; m < kMfmaPerStep; ++m) hook(m);
            }
        }
    };
    // 32-row fragments of this wave with valid rows: one copy of the step
    // loop per count, so the full-tile loop carries no branch
    constexpr int TM = EngineMx<BM, BN, WM, WN>::TM;
    static_assert(TM == 4, "fragment-count dispatch below");
    const int na = wcol0 < cols_valid ? (rows_valid - wrow0 + 31) / 32 : 0;
    if (na >= TM) run_steps(std::integral_constant<int, TM>{});
    else if (na <= 0) run_steps(std::integral_constant<int, 0>{});
    else if (na == 1) run_steps(std::integral_constant<int, 1>{});
    else if (na == 2) run_steps(std::integral_constant<int, 2>{});
    else run_steps(std::integral_constant<int, 3>{});
    wait_vmcnt<0>();  // no LDS write may outlive the workgroup
    store(eng);
}

// ---------------------------------------------------------------------------
// Row-grouped MX GEMM: tiles (expert M-tile, N-tile) on persistent
// workgroups, scheduled as in gmm_rows_kernel.
//   SWIGLU false: y [M_cap, N] bf16 = DQ(x) @ DQ(w[e])^T, w[e] [N][K].
//   SWIGLU true:  N = 2I weight rows; a tile covers kBN/2 output columns c,
//                 reading gate rows c and up rows I + c; writes (aq, as).
// ---------------------------------------------------------------------------
//   GATHER:      X / XS hold token rows and grouped row r is token
//                slot[r] / top_k (RowGather), as in gmm_rows_kernel.
template <bool SWIGLU, bool GATHER = false>
__global__ __launch_bounds__(kThreads, 1) void gmm_mx_rows_kernel(
    const uint8_t* __restrict__ X, const uint8_t* __restrict__ XS, int64_t ld_xs,
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ WS, int64_t ld_ws,
    const int64_t* __restrict__ group_list, int E, int64_t M_cap, int K, int N,
    bf16_t* __restrict__ Y, uint8_t* __restrict__ AQ, uint8_t* __restrict__ AS, int64_t ld_as,
    int32_t* dev_err, const int32_t* __restrict__ slot, int top_k, int nslots) {
    constexpr int kCols = SWIGLU ? kBN / 2 : kBN;  // output columns per tile
    __shared__ __attribute__((aligned(1024))) bf16_t smem[kSmemElems];
    __shared__ __attribute__((aligned(16))) uint8_t ssc[2 * kScaleSlot];
    __shared__ int64_t s_scan[kThreads / 64];
    __shared__ int s_off[kMaxExperts], s_cnt[kMaxExperts], s_tst[kMaxExperts];
    const int Ncols = SWIGLU ? N / 2 : N;
    const int NT = (Ncols + kCols - 1) / kCols;
    // gather arguments through LDS, read at each tile's start (see gmm_rows_kernel)
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
    const int ntiles = row_tile_starts<kBM>(s_cnt, E, s_tst, s_scan) * NT;
    const XcdRange xr = xcd_range(blockIdx.x & 7, ntiles);
    for (int j = blockIdx.x >> 3; j < xr.count; j += gridDim.x >> 3) {
        const RowTile rt = row_tile_at<kBM>(s_off, s_cnt, s_tst, E, NT, xr.first + j);
        const int e = rt.e, row0 = rt.row0, rows_valid = rt.rows_valid;
        const int n0 = __builtin_amdgcn_readfirstlane(rt.nt * kCols);
        const int cols_left = Ncols - n0;
        const uint8_t* We = W + ((int64_t)e * N + n0) * K;
        const uint8_t* Se = WS + ((int64_t)e * N + n0) * ld_ws;
        const uint8_t* Xt = GATHER ? X : X + (int64_t)row0 * K;
        const uint8_t* XSt = GATHER ? XS : XS + (int64_t)row0 * ld_xs;
        const RowGather ga{GATHER ? s_slot + row0 : nullptr, GATHER ? s_gather[0] : 1, GATHER ? s_gather[1] : 0,
                           GATHER ? s_err : nullptr};
        if constexpr (SWIGLU) {
            const int tile_cols = 2 * cols_left < kBN ? 2 * cols_left : kBN;
            gemm_tile_mx<kBM, kBN, kWM, kWN>(
                Xt, rows_valid, XSt, ld_xs, We, cols_left, Ncols, Se, ld_ws, K, rows_valid, tile_cols,
                smem, ssc, [&](const auto& eng) {
                    eng.store_swiglu_mx(AQ + (int64_t)row0 * Ncols + n0, Ncols,
                                        AS + (int64_t)row0 * ld_as, ld_as, n0 / kMxGroup, rows_valid,
                                        cols_left);
                }, ga);
        } else {
            bf16_t* y = Y + (int64_t)row0 * N + n0;
            gemm_tile_mx<kBM, kBN, kWM, kWN>(
                Xt, rows_valid, XSt, ld_xs, We, cols_left, 0, Se, ld_ws, K, rows_valid, cols_left, smem,
                ssc, [&](const auto& eng) { eng.store(y, N, rows_valid, cols_left, smem); });
        }
        __syncthreads();  // every wave is done with its epilogue image before the next tile's copies
    }
}

// ---------------------------------------------------------------------------
// Decode-shaped MX GEMM: weight streaming.  When experts own a few rows
// each, the work is reading every active expert's MX weights once; a 256-row
// tile would idle.  A wave owns a column group of 64 weight rows (two 32-row
// MFMA operands: 64 output columns, or for SWIGLU the 32 gate and the
// matching 32 up rows of 32 output columns) and streams its whole reduction
// in batches of four 64-element steps.  Each batch lands in a private LDS
// stage by coalesced LDS DMA (4 rows x 256 bytes per instruction), is read
// back in the MFMA operand layout (lane l: row l%32, bytes 16*(l/32).. and
// 32+16*(l/32).. of each 64-byte step), and the stage is refilled with the
// next batch while the MFMAs run.  The expert's rows are the other operand,
// 32 at a time (zeros past the last row), read from L2; scale bytes come 8
// per batch and row.
//
// Direct register loads in the MFMA layout touch 32 rows x 32 bytes per
// instruction; on 442 MB of weights that pattern reads at 4.6 TB/s against
// 5.4 TB/s for the coalesced one.  Splitting the reduction across the waves
// of a block (partial sums meeting in LDS) measured 10-20 % slower on the
// decode shapes than whole-reduction waves, so there is no split.
// ---------------------------------------------------------------------------
constexpr int kStreamThreads = 256;
constexpr int kStreamSteps = 4;          // 64-element steps per batch
constexpr int kSeg = kStreamSteps * 64;  // bytes of a row per batch
constexpr int kDmaInst = 64 * kSeg / 1024;

// The 8 scale bytes of a batch (one row); batches start at multiples of 8
// bytes and scale rows at multiples of 16, so the load is aligned.
struct ScaleBatch {
    u32x2_t w;
    MOE_DEVICE void load(const uint8_t* p) { w = *reinterpret_cast<const u32x2_t*>(p); }
    MOE_DEVICE void unit() { w = u32x2_t{0x7F7F7F7Fu, 0x7F7F7F7Fu}; }
    // scale of group 2s + c of the batch
    MOE_DEVICE uint32_t pick(int s, int c) const {
        const int b = 2 * s + c;
        return (w[b >> 2] >> (8 * (b & 3))) & 0xFFu;
    }
};

// GATHER: X / XS hold token rows; grouped row r is token slot[r] / top_k
// (a bad entry loads a zero row and sets MOE_DEVERR_SLOT).
// ROUTE (GMM1 of moe_decode_fwd_mx, X / XS the token rows): the group ranges
// and each row's slot come from ra.ids (route.h) instead of group_list and
// slot, kRouteRows rows of the expert at a time; the blocks of the first
// column group write sorted_slot and row_id_map for their expert's rows, and
// the grid's last block the call outputs.
constexpr int kRouteRows = 256;
template <bool SWIGLU, bool GATHER = false, bool ROUTE = false>
__global__ __launch_bounds__(kStreamThreads) void gmm_mx_stream_kernel(
    const uint8_t* __restrict__ X, const uint8_t* __restrict__ XS, int64_t ld_xs,
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ WS, int64_t ld_ws,
    const int64_t* __restrict__ group_list, int E, int64_t M_cap, int K, int N,
    bf16_t* __restrict__ Y, uint8_t* __restrict__ AQ, uint8_t* __restrict__ AS, int64_t ld_as,
    int32_t* dev_err, const int32_t* __restrict__ slot, int top_k, int nslots, const RouteArgs ra) {
    static_assert(!(GATHER && ROUTE), "one way to find the rows");
    static_assert(kStreamThreads == kRouteThreads, "the routing helpers assume this block size");
    constexpr int kWaves = kStreamThreads / 64;
    constexpr int kColsPerWave = SWIGLU ? 32 : 64;
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int64_t s_scan[kStreamThreads / 64];
    __shared__ int s_rows[ROUTE ? kRouteRows : 1];
    __shared__ __attribute__((aligned(1024))) uint8_t stage[kWaves][64 * kSeg];  // one batch per wave
    if constexpr (ROUTE) {
        const bool last = blockIdx.x == gridDim.x - 1;
        route_group_ranges(ra.ids, nslots, E, s_off, s_cnt, s_scan, dev_err, last);
        if (last) route_call_outputs(ra, E, nslots, s_cnt);
    } else {
        load_group_ranges(group_list, E, M_cap, s_off, s_cnt, s_scan, dev_err);
    }
    const int Nout = SWIGLU ? N / 2 : N;
    const int NB = (Nout + kColsPerWave * kWaves - 1) / (kColsPerWave * kWaves);
    const int e = blockIdx.x / NB, nb = blockIdx.x % NB;
    const int off = s_off[e], cnt = s_cnt[e];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int c0 = (nb * kWaves + wid) * kColsPerWave;  // first output column of the wave
    const bool active = cnt > 0 && c0 < Nout;            // uniform per wave
    if (!ROUTE && !active) return;                       // no barrier follows without ROUTE
    const int c = lane >> 5, r32 = lane & 31;
    // this lane's weight row in each of the two operands (for its scales)
    int wrow[2];
    bool wok[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        wrow[t] = SWIGLU ? (t == 0 ? c0 : Nout + c0) + r32 : c0 + 32 * t + r32;
        wok[t] = SWIGLU ? c0 + r32 < Nout : wrow[t] < N;
    }
    const uint8_t* We = W + (int64_t)e * N * K;
    const uint8_t* WSe = WS + (int64_t)e * N * ld_ws;
    const int nsteps = (K + 63) / 64;
    const int nblocks = K / kMxGroup;

    // LDS DMA of a batch: instruction i moves rows 4i .. 4i+3 of the wave's
    // 64 (operand t = i / 8), lane l 16 bytes of row 4i + l/16.  Lane l
    // fetches chunk (l%16) ^ (row%16) of the row's batch segment, so chunk q
    // of row r lands at position q ^ (r%16): the MFMA-layout reads below
    // (16 rows, one chunk) then hit 16 distinct bank groups.
    const int dq = lane & 15;
    uint8_t* wst = &stage[wid][0];
    auto dma_batch = [&](int s0) {
#pragma unroll
        for (int i = 0; i < kDmaInst; ++i) {
            const int t = i / 8;                       // operand
            const int r = 4 * (i % 8) + (lane >> 4);   // row within the operand
            const int row = SWIGLU ? (t == 0 ? c0 : Nout + c0) + r : c0 + 32 * t + r;
            const bool rok = SWIGLU ? c0 + r < Nout : row < N;
            const int q = dq ^ (r & 15);
            const int k = 64 * s0 + 16 * q;
            const uint32_t v = rok && k < K ? (uint32_t)((int64_t)row * K + k) : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(We), (LDS_AS void*)(wst + i * 1024), 16, v,
                                                     0, 0, 0);
        }
    };
    // the 16-byte piece (step s, half h) of this lane's row in operand t
    auto lds_piece = [&](int t, int s, int h) {
        const int r = r32;
        const int q = 4 * s + 2 * h + c;
        return wst + (t * 8 + (r >> 2)) * 1024 + (r & 3) * 256 + ((q ^ (r & 15)) << 4);
    };

    // rows [ch, ch + nrows) of the expert per chunk (one chunk unless ROUTE)
    for (int ch = 0; ch < cnt; ch += ROUTE ? kRouteRows : cnt) {  // uniform across the block
    const int nrows = ROUTE && cnt - ch > kRouteRows ? kRouteRows : cnt - ch;
    if constexpr (ROUTE) {
        route_rows(ra.ids, nslots, e, ch, nrows, s_rows, s_scan);
        if (nb == 0)
            for (int i = threadIdx.x; i < nrows; i += kStreamThreads) {
                ra.sorted_slot[off + ch + i] = s_rows[i];
                ra.row_id_map[s_rows[i]] = off + ch + i;
            }
    }
    for (int rg = ch; active && rg < ch + nrows; rg += 32) {  // uniform across the wave
        const int xr = rg + r32;           // this lane's expert row
        const bool xok = xr < cnt;         // the row exists (and is written)
        bool xld = xok;                    // its operand row is loaded (else zeros)
        int src = off + xr;                // its source row: grouped row, or token (slot)
        if constexpr (ROUTE) src = xok ? s_rows[xr - ch] / top_k : 0;
        if (GATHER && xok) {
            const int sl = slot[off + xr];
            xld = sl >= 0 && sl < nslots;
            if (!xld && dev_err) atomicOr(dev_err, MOE_DEVERR_SLOT);
            src = xld ? sl / top_k : 0;
        }
        const uint8_t* xrow = X + (int64_t)src * K;
        const uint8_t* xsrow = XS + (int64_t)src * ld_xs;
        f32x16_t acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[t][q] = 0.f;
        dma_batch(0);
        for (int s0 = 0; s0 < nsteps; s0 += kStreamSteps) {
            u32x4_t wa[2][kStreamSteps][2], xa[kStreamSteps][2];
            ScaleBatch wsc[2], xsc;
            const int sb = 2 * s0;  // first scale byte of the batch
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (wok[t] && sb < nblocks) wsc[t].load(WSe + (int64_t)wrow[t] * ld_ws + sb);
                else wsc[t].unit();
            }
#pragma unroll
            for (int s = 0; s < kStreamSteps; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = 64 * (s0 + s) + 32 * h + 16 * c;
                    xa[s][h] = xld && k < K ? ld16(xrow + k) : u32x4_t{0u, 0u, 0u, 0u};
                }
            if (xld && sb < nblocks) xsc.load(xsrow + sb);
            else xsc.unit();
            // this batch's DMA (and every load above) has landed; read the
            // weights in the MFMA layout, then refill the stage with the
            // next batch while the MFMAs run
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s = 0; s < kStreamSteps; ++s)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        asm volatile("ds_read_b128 %0, %1"
                                     : "=v"(wa[t][s][h])
                                     : "v"(lds_addr(lds_piece(t, s, h))));
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s = 0; s < kStreamSteps; ++s)
#pragma unroll
                    for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(wa[t][s][h]));
            if (s0 + kStreamSteps < nsteps) dma_batch(s0 + kStreamSteps);
#pragma unroll
            for (int s = 0; s < kStreamSteps; ++s) {
                const bool kb_ok = 2 * (s0 + s) + c < nblocks;  // padding bytes are no scales
                const int sx = kb_ok ? (int)xsc.pick(s, c) : 127;
                const i32x8_t xv = __builtin_bit_cast(i32x8_t, u32x8_t_of(xa[s][0], xa[s][1]));
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int sw = kb_ok ? (int)wsc[t].pick(s, c) : 127;
                    const i32x8_t wv = __builtin_bit_cast(i32x8_t, u32x8_t_of(wa[t][s][0], wa[t][s][1]));
                    acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, xv, acc[t], 0, 0, 0, sw,
                                                                             0, sx);
                }
            }
        }
        // lane: expert row xr, output columns 8g + 4c + q of each operand
        if constexpr (SWIGLU) {
            float av[16];
            float amax = 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float gv = acc[0][q], uv = acc[1][q];
                av[q] = gv * silu_sigmoid(gv) * uv;
                amax = fmaxf(amax, fabsf(av[q]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
            const uint32_t sbyte = mx_scale_byte(amax);
            const float inv = mx_inv_scale(sbyte);
            if (xok) {
                uint8_t* orow = AQ + (int64_t)(off + xr) * Nout + c0 + 4 * c;
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<uint32_t*>(orow + 8 * g) =
                        e4m3_pack4(av[4 * g] * inv, av[4 * g + 1] * inv, av[4 * g + 2] * inv,
                                   av[4 * g + 3] * inv);
                if (c == 0) AS[(int64_t)(off + xr) * ld_as + c0 / kMxGroup] = (uint8_t)sbyte;
            }
        } else if (xok) {
            bf16_t* orow = Y + (int64_t)(off + xr) * N;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = c0 + 32 * t + 8 * g + 4 * c;
                    if (col < N) {
                        u32x2_t pk;
                        pk[0] = pack_bf16x2(acc[t][4 * g], acc[t][4 * g + 1]);
                        pk[1] = pack_bf16x2(acc[t][4 * g + 2], acc[t][4 * g + 3]);
                        *reinterpret_cast<u32x2_t*>(orow + col) = pk;
                    }
                }
        }
    }
    if constexpr (ROUTE) __syncthreads();  // s_rows is refilled for the next chunk
    }
}

}  // namespace

// Decode-shaped calls (a few rows per expert on average) stream the weights.
static bool gmm_mx_stream_applies(int64_t E, int64_t M_cap) {
    switch (forced_gmm_variant()) {
        case kVariantTile: return false;
        case kVariantStream: return true;
        default: return M_cap <= 8 * E;
    }
}

hipError_t launch_gmm_mx_fwd(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs, const uint8_t* wq,
                             const uint8_t* ws, int64_t ld_ws, const int64_t* group_list, int64_t E,
                             int64_t M_cap, int64_t K, int64_t N, uint16_t* y, int32_t* dev_err,
                             hipStream_t stream) {
    if (M_cap == 0) return hipSuccess;
    if (gmm_mx_stream_applies(E, M_cap)) {
        const int64_t NB = (N + 64 * 4 - 1) / (64 * 4);
        hipLaunchKernelGGL(gmm_mx_stream_kernel<false>, dim3((unsigned)(E * NB)),
                           dim3(kStreamThreads), 0, stream, xq, xs, ld_xs, wq, ws, ld_ws, group_list,
                           (int)E, M_cap, (int)K, (int)N, y, nullptr, nullptr, (int64_t)0, dev_err, nullptr,
                           1, 0, RouteArgs{});
        return hipGetLastError();
    }
    const int64_t grid = num_cus() / 8 * 8;  // persistent, see gmm_mx_rows_kernel
    hipLaunchKernelGGL(gmm_mx_rows_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       xq, xs, ld_xs, wq, ws, ld_ws, group_list, (int)E, M_cap, (int)K, (int)N, y,
                       nullptr, nullptr, (int64_t)0, dev_err, nullptr, 1, 0);
    return hipGetLastError();
}

hipError_t launch_gmm_mx_fwd_swiglu(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs,
                                    const uint8_t* w1q, const uint8_t* w1s, int64_t ld_w1s,
                                    const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K,
                                    int64_t I, uint8_t* aq, uint8_t* as, int64_t ld_as,
                                    int32_t* dev_err, hipStream_t stream, const GatherRows& g) {
    if (M_cap == 0) return hipSuccess;
    if (gmm_mx_stream_applies(E, M_cap)) {
        const int64_t NB = (I + 32 * 4 - 1) / (32 * 4);
        if (g.slot)
            hipLaunchKernelGGL((gmm_mx_stream_kernel<true, true>), dim3((unsigned)(E * NB)),
                               dim3(kStreamThreads), 0, stream, xq, xs, ld_xs, w1q, w1s, ld_w1s,
                               group_list, (int)E, M_cap, (int)K, (int)(2 * I), nullptr, aq, as, ld_as,
                               dev_err, g.slot, (int)g.top_k, (int)g.nslots, RouteArgs{});
        else
            hipLaunchKernelGGL(gmm_mx_stream_kernel<true>, dim3((unsigned)(E * NB)),
                               dim3(kStreamThreads), 0, stream, xq, xs, ld_xs, w1q, w1s, ld_w1s,
                               group_list, (int)E, M_cap, (int)K, (int)(2 * I), nullptr, aq, as, ld_as,
                               dev_err, nullptr, 1, 0, RouteArgs{});
        return hipGetLastError();
    }
    const int64_t grid = num_cus() / 8 * 8;  // persistent, see gmm_mx_rows_kernel
    if (g.slot)
        hipLaunchKernelGGL((gmm_mx_rows_kernel<true, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, xq, xs, ld_xs, w1q, w1s, ld_w1s, group_list, (int)E, M_cap, (int)K,
                           (int)(2 * I), nullptr, aq, as, ld_as, dev_err, g.slot, (int)g.top_k,
                           (int)g.nslots);
    else
        hipLaunchKernelGGL(gmm_mx_rows_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           xq, xs, ld_xs, w1q, w1s, ld_w1s, group_list, (int)E, M_cap, (int)K,
                           (int)(2 * I), nullptr, aq, as, ld_as, dev_err, nullptr, 1, 0);
    return hipGetLastError();
}

hipError_t launch_gmm_mx_stream_route(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs, const int32_t* ids,
                                      int64_t T, int64_t top_k, const uint8_t* w1q, const uint8_t* w1s,
                                      int64_t ld_w1s, int64_t E, int64_t K, int64_t I, uint8_t* aq, uint8_t* as,
                                      int64_t ld_as, int32_t* row_id_map, int32_t* sorted_slot,
                                      int64_t* tokens_per_expert, int32_t* dev_err, hipStream_t stream) {
    RouteArgs ra;
    ra.ids = ids;
    ra.row_id_map = row_id_map;
    ra.sorted_slot = sorted_slot;
    ra.tokens_per_expert = tokens_per_expert;
    const int64_t S = T * top_k;
    const int64_t NB = (I + 32 * 4 - 1) / (32 * 4);
    hipLaunchKernelGGL((gmm_mx_stream_kernel<true, false, true>), dim3((unsigned)(E * NB)), dim3(kStreamThreads), 0,
                       stream, xq, xs, ld_xs, w1q, w1s, ld_w1s, nullptr, (int)E, S, (int)K, (int)(2 * I), nullptr,
                       aq, as, ld_as, dev_err, nullptr, (int)top_k, (int)S, ra);
    return hipGetLastError();
}

}  // namespace moegmm
