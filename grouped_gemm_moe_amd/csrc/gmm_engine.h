// The MFMA tile engine of the grouped matmul kernels (gfx950): HBM -> LDS
// operand staging, the LDS ring, MFMA fragments and the tile epilogues,
// shared by the bf16 kernels (gmm.hip) and the MXFP8 kernels (gmm_mx.hip).
//
// Design (MI355X-first):
//  * group_list never leaves the device.  Every workgroup reads it, scans it
//    in LDS and finds its own tile: a row-grouped tile list for fwd / dX (sum
//    over experts of ceil(n_e/BM) M-tiles times the N-tiles, walked in an
//    XCD-aware order so neighbouring tiles share an L2) and an (expert,
//    k-tile, n-tile) list for dW, largest experts first.  The kernels run
//    persistent workgroups, one per CU.
//  * One MFMA engine: 256x256 output tile per workgroup, 8 waves (two per
//    SIMD, so one hides the other's waits) of 128x64 each,
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  A wave whose
//    sub-tile lies wholly past the tile's valid rows or columns (the last
//    row tile of an expert) skips its LDS reads and MFMAs and only issues
//    its share of the loads.
//  * Operands go HBM -> LDS with buffer_load ... lds (16 bytes per lane, no
//    VGPR staging).  Lanes whose element lies outside the problem (ragged
//    rows, reduction tails, rows past an expert) get an out-of-range buffer
//    offset, which loads zeros -- so partial tiles need no special path.
//  * Each operand keeps its HBM orientation in LDS.  A reduction-contiguous
//    tile ([outer][BK]) is read with ds_read_b128; an outer-contiguous tile
//    ([BK][outer]) is read with ds_read_b64_tr_b16,
//    the gfx950 transposing LDS read, which hands each lane 4 consecutive
//    reduction elements of one column.  16-byte chunks are XOR-swizzled per
//    row so both reads hit every LDS bank pair at most twice per pass.
//  * A ring of NST LDS stages (4 x 32 KiB, BK = 32): the loads of the next
//    NST-1 steps fly while a step runs its MFMAs.  One barrier per step;
//    each wave waits only for its own loads of the step about to be read.
//  * The MFMA is issued with operands swapped (B fragment as the hardware A
//    operand) so each lane holds 4 consecutive output columns.  The epilogue
//    rounds to bf16 (RNE) into an LDS image of the tile and writes it out as
//    whole 128-byte lines with non-temporal stores.
#pragma once

#include <type_traits>

#include "common.h"

#define LDS_AS __attribute__((address_space(3)))

namespace moegmm {

namespace {

constexpr int kThreads = 512;  // 8 waves
constexpr int kWaves = kThreads / 64;

// The ring: (BK, NST) = (32, 4), or (64, 2) as a build option.  Both hold
// 128 KiB, which the epilogue images need.
#ifndef MOEGMM_BK
#define MOEGMM_BK 32
#endif
#ifndef MOEGMM_NST
#define MOEGMM_NST 4
#endif
constexpr int BK = MOEGMM_BK;     // reduction depth of one LDS stage
constexpr int kNST = MOEGMM_NST;  // LDS stages in the ring
// The LDS array of a GMM workgroup: kNST stages of a 256 x 256 tile.  Other
// tile shapes run rings of their own stage count in the same array, and the
// epilogues use it for their images.
constexpr int kRingElems = kNST * (256 + 256) * BK;
static_assert((BK == 32 && kNST == 4) || (BK == 64 && kNST == 2), "ring of 128 KiB");

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// Buffer resource covering the whole 31-bit offset range from `base`; every
// lane's offset is computed in bounds or set to kOOB, which the hardware
// range check turns into a zero load.
constexpr int kNumRecords = 0x7FFFFFF0;
constexpr uint32_t kOOB = 0x7FFFFFF0u;

MOE_DEVICE __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kNumRecords,
                                             0x00020000);
}

// Non-temporal 16-byte store of lane data to base + byte offset `off`
// (base wave-uniform); an offset of kOOB drops the lane's store.
#ifndef MOEGMM_STORE_AUX
#define MOEGMM_STORE_AUX 2  // cache policy bits of the epilogue stores: nt
#endif
MOE_DEVICE void store_nt16(u32x4_t v, const void* base, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, make_rsrc(base), off, 0, MOEGMM_STORE_AUX);
}

// Wave index as a scalar (the LDS-DMA destination must be wave-uniform).
MOE_DEVICE int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// LDS swizzles (16-byte chunk index XOR) for the two tile orientations.
// [outer][BK] tiles: 16 consecutive rows read at one logical chunk must land
// on distinct bank groups (64 banks x 4 bytes).
MOE_DEVICE int swz_k(int o) { return BK == 64 ? ((o ^ (o >> 3)) & 7) : ((o >> 2) & 3); }
MOE_DEVICE int swz_mn(int k) { return (k & 3) << 2; }         // [64][outer] tiles

// Rows of a reduction-contiguous operand taken from a token matrix instead of
// a permuted copy of it: tile row o is token slot[o] / top_k, where slot (the
// permute's sorted_slot, advanced to the tile's first row) holds a slot index
// in [0, nslots).  A row whose entry is outside that range loads zeros and
// sets MOE_DEVERR_SLOT.  slot == nullptr: no gather.
struct RowGather {
    const int32_t* slot;
    int top_k, nslots;
    int32_t* dev_err;
};

// ---------------------------------------------------------------------------
// HBM -> LDS copies of one operand tile per reduction step.  A wave
// instruction moves 1 KiB: lane l's 16 bytes land at LDS byte 16*l of it, so
// the lane -> global-address map decides the LDS layout (and the swizzle).
// ---------------------------------------------------------------------------
template <int BO, bool KMAJOR>
struct Dma;

// Reduction-contiguous operand: element (o, q) at base[o*ld + q].
// LDS tile [BO][BK]; one instruction fills 1024 / (2*BK) rows.
template <int BO>
struct Dma<BO, true> {
    static constexpr int kCPR = BK / 8;                  // 16-byte chunks per row
    static constexpr int kRowsPerInst = 64 / kCPR;
    static constexpr int kInst = BO / kRowsPerInst / kWaves;  // per wave
    static_assert(kInst >= 1 && BO % (kRowsPerInst * kWaves) == 0, "tile/threads mismatch");
    uint32_t off[kInst];
    int red[kInst];
    uint32_t ok_mask;

    // pair > 0: tile rows are 32-row groups taken alternately from operand
    // row r and row pair + r (gate and up halves of a gate_up weight), as in
    // the outer-contiguous case below; outer_lim then bounds r.
    MOE_DEVICE void init(int64_t ld, int outer_lim, int pair = 0) {
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        ok_mask = 0;
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int o = (wid * kInst + i) * kRowsPerInst + lane / kCPR;
            const int c = (lane % kCPR) ^ swz_k(o);
            int vo = o, go = o;
            if (pair > 0) {
                vo = (o >> 6) * 32 + (o & 31);
                go = ((o >> 5) & 1) * pair + vo;
            }
            off[i] = (uint32_t)(((int64_t)go * ld + c * 8) * 2);
            red[i] = c * 8;
            if (vo < outer_lim) ok_mask |= 1u << i;
        }
    }
    // Gathered rows (no pair): row o of the tile is token g.slot[o] / g.top_k
    // of a token matrix with row stride ld, whose T * ld elements span less
    // than 2^30, so every offset fits the 31-bit buffer range.
    MOE_DEVICE void init_gather(int64_t ld, int outer_lim, const RowGather& g) {
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        ok_mask = 0;
        bool bad = false;
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int o = (wid * kInst + i) * kRowsPerInst + lane / kCPR;
            const int c = (lane % kCPR) ^ swz_k(o);
            int tok = 0;
            if (o < outer_lim) {
                const int s = g.slot[o];
                if (s >= 0 && s < g.nslots) {
                    tok = s / g.top_k;
                    ok_mask |= 1u << i;
                } else {
                    bad = true;
                }
            }
            off[i] = (uint32_t)(((int64_t)tok * ld + c * 8) * 2);
            red[i] = c * 8;
        }
        if (bad && g.dev_err) atomicOr(g.dev_err, MOE_DEVERR_SLOT);
    }
    // stage_base: element (0, s*BK); red_left: valid reduction length from there
    MOE_DEVICE void issue(const bf16_t* stage_base, bf16_t* lds, int red_left) const {
        const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(stage_base);
        const int wid = wave_id();
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const uint32_t v = ((ok_mask >> i) & 1u) && red[i] < red_left ? off[i] : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (LDS_AS void*)(lds + (wid * kInst + i) * 512), 16, v, 0, 0, 0);
        }
    }
    static MOE_DEVICE const bf16_t* stage(const bf16_t* base, int64_t, int s) { return base + s * BK; }
    // instruction i of this wave's share of one stage
    MOE_DEVICE void issue_one(int i, __amdgpu_buffer_rsrc_t rsrc, bf16_t* lds, int red_left) const {
        const uint32_t v = ((ok_mask >> i) & 1u) && red[i] < red_left ? off[i] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (LDS_AS void*)(lds + (wave_id() * kInst + i) * 512), 16, v, 0, 0, 0);
    }
};

// Outer-contiguous operand: element (o, q) at base[q*ld + o].
// LDS tile [BK][BO]; one instruction fills 1024 / (2*BO) rows.
template <int BO>
struct Dma<BO, false> {
    static constexpr int kChunks = BO / 8;
    static constexpr int kRowsPerInst = 64 / kChunks;
    static constexpr int kInst = BK / kRowsPerInst / kWaves;  // per wave
    static_assert(kChunks >= 16 && 64 % kChunks == 0 && kInst >= 1 &&
                      BK % (kRowsPerInst * kWaves) == 0, "outer tile must be 128 or 256");
    uint32_t off[kInst];
    int red[kInst];
    uint32_t ok_mask;

    // pair > 0: the tile's columns are 32-wide groups taken alternately from
    // column c and column pair + c of the operand (gate and up halves of a
    // gate_up weight), so that tile groups 2g and 2g+1 hold the same
    // output columns 32g..32g+31; outer_lim then bounds c.
    MOE_DEVICE void init(int64_t ld, int outer_lim, int pair = 0) {
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        ok_mask = 0;
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int k = (wid * kInst + i) * kRowsPerInst + lane / kChunks;
            const int col = ((lane % kChunks) ^ swz_mn(k)) * 8;
            int vc = col, gc = col;
            if (pair > 0) {
                vc = (col >> 6) * 32 + (col & 31);
                gc = ((col >> 5) & 1) * pair + vc;
            }
            off[i] = (uint32_t)(((int64_t)k * ld + gc) * 2);
            red[i] = k;
            if (vc < outer_lim) ok_mask |= 1u << i;
        }
    }
    MOE_DEVICE void issue(const bf16_t* stage_base, bf16_t* lds, int red_left) const {
        const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(stage_base);
        const int wid = wave_id();
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const uint32_t v = ((ok_mask >> i) & 1u) && red[i] < red_left ? off[i] : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (LDS_AS void*)(lds + (wid * kInst + i) * 512), 16, v, 0, 0, 0);
        }
    }
    static MOE_DEVICE const bf16_t* stage(const bf16_t* base, int64_t ld, int s) {
        return base + (int64_t)s * BK * ld;
    }
    // instruction i of this wave's share of one stage
    MOE_DEVICE void issue_one(int i, __amdgpu_buffer_rsrc_t rsrc, bf16_t* lds, int red_left) const {
        const uint32_t v = ((ok_mask >> i) & 1u) && red[i] < red_left ? off[i] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (LDS_AS void*)(lds + (wave_id() * kInst + i) * 512), 16, v, 0, 0, 0);
    }
};

// Reduction-contiguous operand whose rows do not split evenly over the waves
// (BO = 320: 20 copies of 16 rows per stage for 8 waves).  Copy g = w +
// kWaves * i of wave w fills rows 16g .. 16g+15 at LDS slot g, the same
// layout as Dma<BO, true>; a wave's copies past the last one go, with every
// lane out of range, to a spare 1 KiB slot (`spare`), so that every wave
// issues the same number of copies and the in-order wait counts hold.
template <int BO>
struct DmaTallA {
    static constexpr int kCPR = BK / 8;
    static constexpr int kRowsPerInst = 64 / kCPR;
    static constexpr int kInstTotal = BO / kRowsPerInst;
    static constexpr int kInst = (kInstTotal + kWaves - 1) / kWaves;  // per wave
    static_assert(BO % kRowsPerInst == 0, "whole copies");
    uint32_t off[kInst];
    int red[kInst];
    uint32_t ok_mask;
    bf16_t* spare;

    MOE_DEVICE int slot(int i) const { return wave_id() + kWaves * i; }
    MOE_DEVICE void init(int64_t ld, int outer_lim, int pair = 0) {
        (void)pair;
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        ok_mask = 0;
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int g = wid + kWaves * i;
            const int o = g * kRowsPerInst + lane / kCPR;
            const int c = (lane % kCPR) ^ swz_k(o);
            off[i] = (uint32_t)(((int64_t)o * ld + c * 8) * 2);
            red[i] = c * 8;
            if (g < kInstTotal && o < outer_lim) ok_mask |= 1u << i;
        }
    }
    MOE_DEVICE void init_gather(int64_t ld, int outer_lim, const RowGather& gt) {
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        ok_mask = 0;
        bool bad = false;
#pragma unroll
        for (int i = 0; i < kInst; ++i) {
            const int g = wid + kWaves * i;
            const int o = g * kRowsPerInst + lane / kCPR;
            const int c = (lane % kCPR) ^ swz_k(o);
            int tok = 0;
            if (g < kInstTotal && o < outer_lim) {
                const int sl = gt.slot[o];
                if (sl >= 0 && sl < gt.nslots) {
                    tok = sl / gt.top_k;
                    ok_mask |= 1u << i;
                } else {
                    bad = true;
                }
            }
            off[i] = (uint32_t)(((int64_t)tok * ld + c * 8) * 2);
            red[i] = c * 8;
        }
        if (bad && gt.dev_err) atomicOr(gt.dev_err, MOE_DEVERR_SLOT);
    }
    MOE_DEVICE void issue_one(int i, __amdgpu_buffer_rsrc_t rsrc, bf16_t* lds, int red_left) const {
        const uint32_t v = ((ok_mask >> i) & 1u) && red[i] < red_left ? off[i] : kOOB;
        const int g = slot(i);
        bf16_t* dst = g < kInstTotal ? lds + g * 512 : spare;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)dst, 16, v, 0, 0, 0);
    }
    MOE_DEVICE void issue(const bf16_t* stage_base, bf16_t* lds, int red_left) const {
        const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(stage_base);
#pragma unroll
        for (int i = 0; i < kInst; ++i) issue_one(i, rsrc, lds, red_left);
    }
    static MOE_DEVICE const bf16_t* stage(const bf16_t* base, int64_t, int s) { return base + s * BK; }
};

// ---------------------------------------------------------------------------
// MFMA operand fragments: lane l gets T[o0 + l%32][k0 + 8*(l/32) + 0..7].
//
// The reads are issued as inline asm on purpose: the loads of the next
// reduction step are in flight into the other LDS stage while these run, and
// the compiler, unable to prove the two stages apart through computed
// addresses, would otherwise wait for those loads first.  The caller waits
// for the reads itself (lds_wait) before feeding the fragments to MFMAs.
// ---------------------------------------------------------------------------
MOE_DEVICE uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

template <int BO, bool KMAJOR>
struct Frag;

template <int BO>
struct Frag<BO, true> {
    static MOE_DEVICE void load(bf16x8_t& v, const bf16_t* lds, int o0, int k0) {
        const int lane = threadIdx.x & 63;
        const int o = o0 + (lane & 31);
        const int c = (k0 >> 3) + (lane >> 5);
        asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(lds_addr(lds + o * BK + ((c ^ swz_k(o)) << 3))));
    }
};

// ds_read_b64_tr_b16 over a 16-lane group: lane s supplies the address of 4
// consecutive columns (o .. o+3) of reduction row kb + s/4; lane L receives
// column ob + L of rows kb .. kb+3.  Two such reads (rows +0..3 and +4..7)
// give the 8 reduction elements of one MFMA operand lane.
template <int BO>
struct Frag<BO, false> {
    static MOE_DEVICE void load(bf16x8_t& v, const bf16_t* lds, int o0, int k0) {
        const int lane = threadIdx.x & 63;
        const int g = lane >> 4, s = lane & 15;
        const int o = o0 + ((g & 1) << 4) + ((s & 3) << 2);
        const int k = k0 + ((g >> 1) << 3) + (s >> 2);
        const int cc = ((o >> 3) ^ swz_mn(k)) << 3;   // swz_mn(k) == swz_mn(k + 4)
        const uint32_t a = lds_addr(lds + k * BO + cc + (o & 7));
        u32x2_t lo, hi;
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(a));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(a), "i"(4 * BO * 2));
        const u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
        v = __builtin_bit_cast(bf16x8_t, w);
    }
};

// Wait for every outstanding LDS read; the fragments pass through the asm so
// that no use of them can be scheduled above the wait.
template <int TM, int TN>
MOE_DEVICE void lds_wait(bf16x8_t (&a)[TM], bf16x8_t (&b)[TN]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(a[t]));
#pragma unroll
    for (int t = 0; t < TN; ++t) asm volatile("" : "+v"(b[t]));
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
MOE_DEVICE void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// f(integral_constant<int, i>) for i = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
MOE_DEVICE void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------------------
// The tile engine: C[BM][BN] = A[BM][red] * B[red][BN], fp32 accumulation.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool A_KMAJOR, bool B_KMAJOR>
struct Engine {
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(WM * WN == kThreads / 64 && TM >= 1 && TN >= 1, "wave grid");
    f32x16_t acc[TM][TN];

    MOE_DEVICE void zero() {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    // NA: the wave's 32-row fragments that hold valid rows (the others are
    // past an expert's last row: their LDS reads and MFMAs are skipped).
    template <int NA = TM>
    MOE_DEVICE void load_frags(bf16x8_t (&a)[TM], bf16x8_t (&b)[TN], const bf16_t* la, const bf16_t* lb,
                               int ks) const {
        const int wid = threadIdx.x >> 6;
        const int wm = wid / WN, wn = wid % WN;
#pragma unroll
        for (int t = 0; t < NA; ++t) Frag<BM, A_KMAJOR>::load(a[t], la, wm * WTM + t * 32, ks * 16);
#pragma unroll
        for (int t = 0; t < TN; ++t) Frag<BN, B_KMAJOR>::load(b[t], lb, wn * WTN + t * 32, ks * 16);
    }

    // MFMAs of one sub-step; hook(m) runs after the m-th MFMA slot of the
    // step (m counts across sub-steps, skipped fragments included), so loads
    // can be spread between MFMAs and every hook runs whatever NA is.
    template <int NA = TM, class Hook>
    MOE_DEVICE void mfmas(const bf16x8_t (&a)[TM], const bf16x8_t (&b)[TN], int ks, Hook& hook) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (i < NA) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
                hook(ks * TM * TN + i * TN + j);
            }
    }

    // One reduction step from LDS: fragments of sub-step ks+1 are read while
    // the MFMAs of sub-step ks run.
    template <int NA = TM, class Hook>
    MOE_DEVICE void compute(const bf16_t* la, const bf16_t* lb, Hook& hook) {
        static_assert(BK / 16 == 2 || BK / 16 == 4, "sub-steps");
        static_assert(NA >= 1 && NA <= TM, "active fragments");
        bf16x8_t a0[TM], b0[TN], a1[TM], b1[TN];
        load_frags<NA>(a0, b0, la, lb, 0);
        lds_wait(a0, b0);
        load_frags<NA>(a1, b1, la, lb, 1);
        mfmas<NA>(a0, b0, 0, hook);
        lds_wait(a1, b1);
        if constexpr (BK / 16 == 4) {
            load_frags<NA>(a0, b0, la, lb, 2);
            mfmas<NA>(a1, b1, 1, hook);
            lds_wait(a0, b0);
            load_frags<NA>(a1, b1, la, lb, 3);
            mfmas<NA>(a0, b0, 2, hook);
            lds_wait(a1, b1);
            mfmas<NA>(a1, b1, 3, hook);
        } else {
            mfmas<NA>(a1, b1, 1, hook);
        }
    }

    // Epilogues.  A lane holds rows (l%32) and 4 consecutive columns per
    // (i, j, g) of its wave's sub-tile, so writing straight from the
    // accumulators would scatter 8-byte pieces over 32 rows per instruction.
    // Instead the tile is rounded to bf16 into LDS (the ring is free once
    // every wave has left the main loop), read back as whole rows and written
    // 16 bytes per lane, a full 128-byte line per 8 lanes, with non-temporal
    // stores: the output is not read again by this kernel and should not
    // displace operand lines in L2.
    //
    // Wave image: [WTM rows][64 columns] bf16, 16-byte chunk c of row r at
    // chunk c ^ ((r >> 1) & 7), so the 32 rows written by one instruction
    // spread over the banks.
    MOE_DEVICE void store(bf16_t* __restrict__ out, int64_t ld, int rows_valid, int cols_valid,
                          bf16_t* smem) const {
        static_assert(WTN == 64, "one 128-byte row segment per wave row");
        // at most 4 fragments (128 rows) per pass through the wave's image:
        // taller wave tiles (160 rows) take a second pass through the same
        // image (each wave reads back its own writes first)
        constexpr int kPassFr = TM < 4 ? TM : 4;
        static_assert(kWaves * kPassFr * 32 * WTN <= kRingElems, "images fit the LDS array");
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));  // keeps this address math out of an enclosing tile loop
        const int lane = tid & 63;
        const int wid = wave_id();
        const int wm = wid / WN, wn = wid % WN;
        __syncthreads();  // every wave is done reading the ring
        bf16_t* img = smem + wid * (kPassFr * 32 * WTN);
        const int c = lane & 7;
        const uint32_t lane_off = (uint32_t)(((int64_t)(lane >> 3) * ld + c * 8) * 2);
        static_for<0, (TM + kPassFr - 1) / kPassFr>([&](auto pc_) {
            constexpr int p0 = decltype(pc_)::value * kPassFr;
            constexpr int np = TM - p0 < kPassFr ? TM - p0 : kPassFr;
#pragma unroll
            for (int i = 0; i < np; ++i) {
                const int r = i * 32 + (lane & 31);
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int pc = (j * 4 + g) ^ ((r >> 1) & 7);
                        u32x2_t pk;
                        pk[0] = pack_bf16x2(acc[p0 + i][j][4 * g + 0], acc[p0 + i][j][4 * g + 1]);
                        pk[1] = pack_bf16x2(acc[p0 + i][j][4 * g + 2], acc[p0 + i][j][4 * g + 3]);
                        *reinterpret_cast<u32x2_t*>(img + r * 64 + pc * 8 + (lane >> 5) * 4) = pk;
                    }
            }
            // Each wave reads back only its own image (no barrier): all reads
            // first, then one unconditional store per 8 rows, masked lanes
            // getting an out-of-range offset, so the reads overlap each other.
            constexpr int kIt = np * 4;
            u32x4_t v[kIt];
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int r = it * 8 + (lane >> 3);
                v[it] = *reinterpret_cast<const u32x4_t*>(img + r * 64 + ((c ^ ((r >> 1) & 7)) << 3));
            }
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int r0 = wm * WTM + p0 * 32 + it * 8;
                const bool ok = r0 + (lane >> 3) < rows_valid && wn * WTN + c * 8 < cols_valid;
                store_nt16(v[it], out + (int64_t)r0 * ld + wn * WTN, ok ? lane_off : kOOB);
            }
        });
    }

    // Input-gradient tile of the down GMM fused with the SwiGLU backward.
    // The accumulators hold dA (fp32, not rounded).  With G = h[:, c] and
    // U = h[:, pair + c] at the same rows and columns and s = sigmoid(G),
    // writes dG = dA*U*s*(1 + G*(1 - s)) to dh[:, c] and dU = dA*G*s to
    // dh[:, pair + c], each rounded once (RNE).
    // A wave takes its rows 32 at a time (one accumulator fragment row),
    // through two 8 KiB LDS regions used in turn: G and U of the next 32 rows
    // arrive by LDS DMA as whole 128-byte lines while the current ones are
    // read back in the accumulator layout, turned into dG and dU in place,
    // and sent out as whole lines (16-byte chunk c of region row r at chunk
    // c ^ ((r >> 1) & 7), as in store()).  Every wave issues the same loads
    // and stores (lanes outside the tile get an out-of-range offset), so the
    // in-order vector-memory counter tells when a region has landed.  dh may
    // be h: a wave reads G and U of exactly the outputs it writes, before it
    // writes them.
    MOE_DEVICE void store_swiglu_bwd(bf16_t* dh, const bf16_t* h, int64_t ld, int pair, int rows_valid,
                                     int cols_valid, bf16_t* smem) const {
        static_assert(WTN == 64 && TM >= 2, "128-byte row segments, at least two passes");
        constexpr int kRows = 32;       // rows per pass
        constexpr int kIt = kRows / 8;  // 8 rows of 128 bytes per instruction
        constexpr int kRegion = 2 * kRows * WTN;  // G and U of one pass, bf16 elements
        static_assert(kWaves * 2 * kRegion <= kRingElems, "regions fit the LDS array");
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));  // keeps this address math out of an enclosing tile loop
        const int lane = tid & 63;
        const int wid = wave_id();
        const int wm = wid / WN, wn = wid % WN;
        const int lr = lane >> 3, pch = lane & 7;  // row, physical chunk of one 1 KiB transfer
        const int wcol = wn * WTN;
        const uint32_t row_off = (uint32_t)(((int64_t)lr * ld) * 2);
        bf16_t* regions = smem + wid * (2 * kRegion);
        __syncthreads();  // every wave is done reading the ring
        auto fetch = [&](int i) {  // G and U of pass i into region i & 1 (zeros outside the tile)
            bf16_t* img_g = regions + (i & 1) * kRegion;
            const int row_base = wm * WTM + i * kRows;
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int r = it * 8 + lr;
                const int lc = pch ^ ((r >> 1) & 7);  // logical chunk that lands at pch
                const bool ok = row_base + r < rows_valid && wcol + lc * 8 < cols_valid;
                const uint32_t off = ok ? row_off + (uint32_t)(lc * 16) : kOOB;
                const bf16_t* src = h + (int64_t)(row_base + it * 8) * ld + wcol;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src), (LDS_AS void*)(img_g + it * 512),
                                                         16, off, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src + pair),
                                                         (LDS_AS void*)(img_g + kRows * WTN + it * 512), 16,
                                                         off, 0, 0, 0);
            }
        };
        const uint32_t out_off = (uint32_t)(((int64_t)lr * ld + pch * 8) * 2);
        fetch(0);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i + 1 < TM) fetch(i + 1);
            // pass i's transfers have landed once at most the later ones are
            // outstanding: pass i+1's (2 kIt) and pass i-1's stores (2 kIt)
            if (i == 0) wait_vmcnt<2 * kIt>();
            else if (i + 1 < TM) wait_vmcnt<4 * kIt>();
            else wait_vmcnt<2 * kIt>();
            bf16_t* img_g = regions + (i & 1) * kRegion;
            bf16_t* img_u = img_g + kRows * WTN;
            const int r = lane & 31;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int o = r * 64 + (((j * 4 + g) ^ ((r >> 1) & 7)) << 3) + (lane >> 5) * 4;
                    const u32x2_t gq = *reinterpret_cast<const u32x2_t*>(img_g + o);
                    const u32x2_t uq = *reinterpret_cast<const u32x2_t*>(img_u + o);
                    float dgv[4], duv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float gv = (q & 1) ? bf16_hi(gq[q >> 1]) : bf16_lo(gq[q >> 1]);
                        const float uv = (q & 1) ? bf16_hi(uq[q >> 1]) : bf16_lo(uq[q >> 1]);
                        const float dv = acc[i][j][4 * g + q];
                        const float sg = silu_sigmoid(gv);
                        dgv[q] = dv * uv * sg * (1.0f + gv * (1.0f - sg));
                        duv[q] = dv * gv * sg;
                    }
                    u32x2_t pg, pu;
                    pg[0] = pack_bf16x2(dgv[0], dgv[1]);
                    pg[1] = pack_bf16x2(dgv[2], dgv[3]);
                    pu[0] = pack_bf16x2(duv[0], duv[1]);
                    pu[1] = pack_bf16x2(duv[2], duv[3]);
                    // the same 8 bytes this lane read: no other lane touches them
                    *reinterpret_cast<u32x2_t*>(img_g + o) = pg;
                    *reinterpret_cast<u32x2_t*>(img_u + o) = pu;
                }
            u32x4_t vg[kIt], vu[kIt];
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int rr = it * 8 + lr;
                const int o = rr * 64 + ((pch ^ ((rr >> 1) & 7)) << 3);
                vg[it] = *reinterpret_cast<const u32x4_t*>(img_g + o);
                vu[it] = *reinterpret_cast<const u32x4_t*>(img_u + o);
            }
            const int row_base = wm * WTM + i * kRows;
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int r0 = row_base + it * 8;
                const bool ok = r0 + lr < rows_valid && wcol + pch * 8 < cols_valid;
                bf16_t* dst = dh + (int64_t)r0 * ld + wcol;
                store_nt16(vg[it], dst, ok ? out_off : kOOB);
                store_nt16(vu[it], dst + pair, ok ? out_off : kOOB);
            }
        }
    }

    // Gate_up tile with paired columns (see Dma::init): fragment 0 of a wave
    // holds the gate values G and fragment 1 the up values U of the same 32
    // output columns.  Writes A = SiLU(G) * U (rounded once, from the fp32
    // accumulators) and, when h is given, G and U themselves to h[:, c] and
    // h[:, pair + c].  An output row of the tile (BN/2 columns) spans the
    // WN waves of a wave row, so the images here cover the whole tile:
    // [BM][BN/2] bf16 each (A and G together fill the ring; U follows in a
    // second pass), 16-byte chunk c of row r at chunk c ^ (r % 16).
    MOE_DEVICE void store_swiglu(bf16_t* __restrict__ a, int64_t lda, bf16_t* __restrict__ h,
                                 int64_t ldh, int pair, int rows_valid, int cols_valid,
                                 bf16_t* smem) const {
        static_assert(TN == 2, "one gate and one up fragment per wave");
        constexpr int kCols = BN / 2, kChunks = kCols / 8;  // one output row: kChunks 16-byte chunks
        // A and G side by side when both images fit the LDS array, else one
        // image at a time (A, then G, then U)
        constexpr bool kTwo = 2 * BM * kCols <= kRingElems;
        static_assert(kChunks == 16 && BM * kCols <= kRingElems, "images fit the LDS array");
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));  // keeps this address math out of an enclosing tile loop
        const int lane = tid & 63;
        const int wid = wave_id();
        const int wm = wid / WN, wn = wid % WN;
        bf16_t* img_a = smem;
        bf16_t* img_g = kTwo ? smem + BM * kCols : smem;
        auto put = [&](bf16_t* img, int r, int c, uint32_t lo, uint32_t hi) {
            u32x2_t pk;
            pk[0] = lo;
            pk[1] = hi;
            *reinterpret_cast<u32x2_t*>(img + r * kCols + ((c ^ (r & 15)) << 3) + (lane >> 5) * 4) = pk;
        };
        // whole rows out: 16 lanes per row, 16 bytes each; a wave covers 4
        // rows per pass.  All reads first, then unconditional stores (masked
        // lanes get an out-of-range offset).
        auto copy_out = [&](const bf16_t* img, bf16_t* dst, int64_t ld) {
            constexpr int kRowsPerPass = kThreads / kChunks;
            constexpr int kIt = BM / kRowsPerPass;
            const int c = lane % kChunks;
            u32x4_t v[kIt];
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int r = it * kRowsPerPass + wid * 4 + lane / kChunks;
                v[it] = *reinterpret_cast<const u32x4_t*>(img + r * kCols + ((c ^ (r & 15)) << 3));
            }
            const uint32_t lane_off = (uint32_t)(((int64_t)(lane / kChunks) * ld + c * 8) * 2);
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int r0 = it * kRowsPerPass + wid * 4;
                const bool ok = r0 + lane / kChunks < rows_valid && c * 8 < cols_valid;
                store_nt16(v[it], dst + (int64_t)r0 * ld, ok ? lane_off : kOOB);
            }
        };
        __syncthreads();  // every wave is done reading the ring
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = wn * 4 + g;
                float av[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float gv = acc[i][0][4 * g + q], uv = acc[i][1][4 * g + q];
                    av[q] = gv * silu_sigmoid(gv) * uv;
                }
                put(img_a, r, c, pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
                if (kTwo && h)
                    put(img_g, r, c, pack_bf16x2(acc[i][0][4 * g], acc[i][0][4 * g + 1]),
                        pack_bf16x2(acc[i][0][4 * g + 2], acc[i][0][4 * g + 3]));
            }
        }
        __syncthreads();
        copy_out(img_a, a, lda);
        if (!h) return;
        if constexpr (!kTwo) {
            __syncthreads();  // image A is read out; G takes its place
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    put(img_g, r, wn * 4 + g, pack_bf16x2(acc[i][0][4 * g], acc[i][0][4 * g + 1]),
                        pack_bf16x2(acc[i][0][4 * g + 2], acc[i][0][4 * g + 3]));
            }
            __syncthreads();
        }
        copy_out(img_g, h, ldh);
        __syncthreads();  // the image is read out; U takes its place
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
            for (int g = 0; g < 4; ++g)
                put(img_a, r, wn * 4 + g, pack_bf16x2(acc[i][1][4 * g], acc[i][1][4 * g + 1]),
                    pack_bf16x2(acc[i][1][4 * g + 2], acc[i][1][4 * g + 3]));
        }
        __syncthreads();
        copy_out(img_a, h + pair, ldh);
    }
};

// One output tile over a ring of NST LDS stages.  Per step s: wait for this
// wave's copies of step s (the NST-2 later steps stay in flight), barrier
// (all copies of step s landed; step s-1 fully read), then run step s while
// refilling the stage read at step s-1 with step s+NST-1, one load after
// every few MFMAs so the memory pipe and the MFMA pipe work side by side.
// Steps past the end still "load", with every lane out of range: that only
// writes zeros into a stage nobody reads again, and keeps the number of
// loads in flight constant (no data-dependent wait counts, no branches).
// `smem` holds NST stages of [A tile | B tile].
// `store(eng)` writes the result; rows_valid / cols_valid (in tile columns)
// decide which waves have any work.
// LDS_ELEMS: size of `smem`.  An A tile whose rows do not split evenly over
// the waves (DmaTallA) also uses 512 elements after the ring.
template <int BM, int BN, int WM, int WN, bool A_KMAJOR, bool B_KMAJOR, int NST = kNST,
          int LDS_ELEMS = kRingElems, class Store>
MOE_DEVICE void gemm_tile(const bf16_t* a_base, int64_t lda, int a_olim, const bf16_t* b_base,
                          int64_t ldb, int b_olim, int b_pair, int red_len, int rows_valid,
                          int cols_valid, bf16_t* smem, const Store& store,
                          const RowGather& gather = RowGather{nullptr, 1, 0, nullptr}) {
    constexpr bool kTallA = A_KMAJOR && BM % (Dma<256, true>::kRowsPerInst * kWaves) != 0;
    using DA = std::conditional_t<kTallA, DmaTallA<BM>, Dma<BM, A_KMAJOR>>;
    using DB = Dma<BN, B_KMAJOR>;
    constexpr int kStage = (BM + BN) * BK;       // elements per stage
    constexpr int kPer = DA::kInst + DB::kInst;  // loads per wave per stage
    static_assert(NST >= 2 && NST * kStage + (kTallA ? 512 : 0) <= LDS_ELEMS, "ring within the LDS array");
    DA da;
    DB db;
    if constexpr (kTallA) da.spare = smem + NST * kStage;
    if constexpr (A_KMAJOR) {
        if (gather.slot) da.init_gather(lda, a_olim, gather);
        else da.init(lda, a_olim);
    } else {
        da.init(lda, a_olim);
    }
    db.init(ldb, b_olim, b_pair);
    Engine<BM, BN, WM, WN, A_KMAJOR, B_KMAJOR> eng;
    eng.zero();
    const int nk = (red_len + BK - 1) / BK;
    auto issue = [&](int step) {
        bf16_t* st = smem + (step % NST) * kStage;
        da.issue(DA::stage(a_base, lda, step), st, red_len - step * BK);
        db.issue(DB::stage(b_base, ldb, step), st + BM * BK, red_len - step * BK);
    };
    // the MFMAs of one step; load q goes after MFMA (q+1)*kMfmaPerStep/kPer - 1
    constexpr int kMfmaPerStep = (BK / 16) * (BM / WM / 32) * (BN / WN / 32);
    static_assert(kMfmaPerStep >= kPer, "load spacing");
#pragma unroll
    for (int p = 0; p < NST - 1; ++p) issue(p);
    // this wave's corner of the output tile; two copies of the step loop
    // (active and idle wave), so the common one carries no branch
    const int wrow0 = (wave_id() / WN) * (BM / WM), wcol0 = (wave_id() % WN) * (BN / WN);
    auto run_steps = [&](auto active_tag) {
    for (int s = 0; s < nk; ++s) {
        wait_vmcnt<(NST - 2) * kPer>();
        __builtin_amdgcn_s_barrier();
        const int nxt = s + NST - 1;
        bf16_t* nst = smem + (nxt % NST) * kStage;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(DA::stage(a_base, lda, nxt));
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(DB::stage(b_base, ldb, nxt));
        const int left = red_len - nxt * BK;
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
            const bf16_t* st = smem + (s % NST) * kStage;
            eng.template compute<decltype(active_tag)::value>(st, st + BM * BK, hook);
        } else {
#pragma unroll
            for (int m = 0; m < kMfmaPerStep; ++m) hook(m);
        }
    }
    };
    // 32-row fragments of this wave with valid rows: a copy of the step loop
    // per count, so the full-tile loop carries no branch
    constexpr int TM = BM / WM / 32;
    const int na = wcol0 < cols_valid ? (rows_valid - wrow0 + 31) / 32 : 0;
    if (na >= TM) run_steps(std::integral_constant<int, TM>{});
    else if (na <= 0) run_steps(std::integral_constant<int, 0>{});
    else if (na == 1) run_steps(std::integral_constant<int, 1>{});
    else if constexpr (TM > 2) {
        if (na == 2) run_steps(std::integral_constant<int, 2>{});
        else run_steps(std::integral_constant<int, TM - 1>{});
    } else {
        run_steps(std::integral_constant<int, TM>{});
    }
    wait_vmcnt<0>();  // no LDS write may outlive the workgroup
    store(eng);
}

// Workgroups are dealt round-robin to the 8 XCDs (workgroup b runs on XCD
// b % 8).  XCD x owns the contiguous range [first, first + count) of n
// logical tiles, so tiles that share operands share its L2.
struct XcdRange {
    int first, count;
};
MOE_DEVICE XcdRange xcd_range(int xcd, int n) {
    const int q = n >> 3, r = n & 7;
    return XcdRange{xcd * q + (xcd < r ? xcd : r), q + (xcd < r ? 1 : 0)};
}

// 256x256 output tiles, 8 waves of 128x64: the copy split, the epilogue
// images and the SwiGLU passes assume this shape (see their static_asserts).
constexpr int kBM = 256, kBN = 256, kWM = 2, kWN = 4;
// Half-height tiles for an expert's last rows when they number at most 128
// (MixedTile): 128 x 512, 8 waves of 128 x 64 in one row, a 3-stage ring of
// 40 KiB stages.
constexpr int kHM = 128, kHN = 512, kHWM = 1, kHWN = 8, kHNST = 3;
constexpr int kSmemElems = kRingElems;
static_assert(kSmemElems == kNST * (kBM + kBN) * BK, "the ring of full tiles fills the LDS array");
// two workgroups per CU when the LDS ring and the accumulators allow it: one
// workgroup's epilogue and first loads then overlap the other's MFMAs
constexpr int kAccRegs = (kBM / kWM) * (kBN / kWN) / 64;
constexpr int kOccupancy = (kSmemElems * 2 <= 80 * 1024 && kAccRegs <= 128) ? 2 : 1;

// ---------------------------------------------------------------------------
// Tiles of a row-grouped GEMM: (expert M-tile, N-tile) pairs, sum over
// experts of ceil(n_e/BM) M-tiles times NT N-tiles, in logical order
// expert-major, then M-tile, then N-tile.
// ---------------------------------------------------------------------------
struct RowTile {
    int e, row0, rows_valid, nt;
};

// s_tst[e] = number of BM-row tiles of the experts before e; returns the
// total.  All threads of the block; ends with a barrier.
template <int BM>
MOE_DEVICE int row_tile_starts(const int* s_cnt, int E, int* s_tst, int64_t* s_scan) {
    const int per = (E + kThreads - 1) / kThreads;
    const int e0 = threadIdx.x * per;
    int64_t my_tiles = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) my_tiles += (s_cnt[e0 + i] + BM - 1) / BM;
    int64_t total_mt;
    int64_t run = block_exclusive_scan<int64_t>(my_tiles, s_scan, &total_mt);
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) {
            s_tst[e0 + i] = (int)run;
            run += (s_cnt[e0 + i] + BM - 1) / BM;
        }
    __syncthreads();
    return (int)total_mt;
}

// Logical tile lt (M-tile lt / NT, N-tile lt % NT) of a row-grouped GEMM.
template <int BM>
MOE_DEVICE RowTile row_tile_at(const int* s_off, const int* s_cnt, const int* s_tst, int E, int NT,
                               int lt) {
    const int mt = lt / NT;
    int lo = 0, hi = E - 1;  // last expert whose first tile is <= mt
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tst[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    // block-uniform values read from LDS: keep them in scalar registers
    RowTile rt;
    rt.e = __builtin_amdgcn_readfirstlane(lo);
    rt.row0 = __builtin_amdgcn_readfirstlane(s_off[rt.e] + (mt - s_tst[rt.e]) * BM);
    const int row_end = __builtin_amdgcn_readfirstlane(s_off[rt.e] + s_cnt[rt.e]);
    rt.rows_valid = row_end - rt.row0 < BM ? row_end - rt.row0 : BM;
    rt.nt = lt % NT;
    return rt;
}

// ---------------------------------------------------------------------------
// Row tiles with tall last tiles (the SwiGLU forward).  When an expert's rows
// past its last full kBM-row tile number at most kTallM - kBM, that tile
// takes them too (a kTallM x kBN tile: 8 waves of 160 x 64) instead of a
// tile of their own, which would stream the whole weight panel again for a
// few rows.  Every output still takes the same MFMAs in the same order.
// ---------------------------------------------------------------------------
constexpr int kTallM = 320;
// LDS of a workgroup that runs tall tiles: a 4-stage ring of 320 x 256
// tiles and the spare slot of DmaTallA.
constexpr int kSmemTallElems = kNST * (kTallM + kBN) * BK + 512;

MOE_DEVICE int tall_mtiles(int n) {
    const int full = n / kBM, rem = n - full * kBM;
    return (full >= 1 && rem > 0 && rem <= kTallM - kBM) ? full : (n + kBM - 1) / kBM;
}

// s_tst[e] = first row tile of expert e (tall_mtiles of each); returns the
// total.  All threads of the block; ends with a barrier.
MOE_DEVICE int tall_tile_starts(const int* s_cnt, int E, int* s_tst, int64_t* s_scan) {
    const int per = (E + kThreads - 1) / kThreads;
    const int e0 = threadIdx.x * per;
    int64_t mine = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) mine += tall_mtiles(s_cnt[e0 + i]);
    int64_t total;
    int64_t run = block_exclusive_scan<int64_t>(mine, s_scan, &total);
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) {
            s_tst[e0 + i] = (int)run;
            run += tall_mtiles(s_cnt[e0 + i]);
        }
    __syncthreads();
    return (int)total;
}

// The total of tall_tile_starts without the per-expert starts.  All
// threads of the block; ends with a barrier.
MOE_DEVICE int tall_tile_count(const int* s_cnt, int E, int64_t* s_scan) {
    const int per = (E + kThreads - 1) / kThreads;
    const int e0 = threadIdx.x * per;
    int64_t mine = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) mine += tall_mtiles(s_cnt[e0 + i]);
    int64_t total;
    block_exclusive_scan<int64_t>(mine, s_scan, &total);
    __syncthreads();
    return (int)total;
}

// Logical tile lt (row tile lt / NT, column tile lt % NT); an expert's last
// row tile holds all of its remaining rows (up to kTallM).
MOE_DEVICE RowTile tall_tile_at(const int* s_off, const int* s_cnt, const int* s_tst, int E, int NT, int lt) {
    const int mt = lt / NT;
    int lo = 0, hi = E - 1;  // last expert whose first tile is <= mt
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tst[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    RowTile rt;
    rt.e = __builtin_amdgcn_readfirstlane(lo);
    const int local = __builtin_amdgcn_readfirstlane(mt - s_tst[rt.e]);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[rt.e]);
    rt.row0 = __builtin_amdgcn_readfirstlane(s_off[rt.e] + local * kBM);
    const int left = cnt - local * kBM;
    rt.rows_valid = local == tall_mtiles(cnt) - 1 ? left : (left < kBM ? left : kBM);
    rt.nt = lt % NT;
    return rt;
}

// ---------------------------------------------------------------------------
// Row tiles with half-height remainders.  An expert's rows go in kBM-row
// tiles of NT column tiles each, and when its last r rows number at most
// kBM/2, in one row of NTH half-height tiles of kBM/2 rows and 2*kBN columns
// instead.  Those tiles use the same 128 x 64 wave tiles (one row of 8
// waves), so every output takes the same MFMAs in the same order; but a tile
// of few rows costs nearly as much as a full one (it streams the whole
// weight panel), and there are half as many of them.
// ---------------------------------------------------------------------------
struct MixedTile {
    int e, row0, rows_valid, nt;
    bool half;
};

MOE_DEVICE int expert_tiles(int cnt, int NT, int NTH) {
    const int full = cnt / kBM, rem = cnt - full * kBM;
    return full * NT + (rem == 0 ? 0 : (2 * rem <= kBM ? NTH : NT));
}

// The total of mixed_tile_starts without the per-expert starts.  All
// threads of the block; ends with a barrier.
MOE_DEVICE int mixed_tile_count(const int* s_cnt, int E, int NT, int NTH, int64_t* s_scan) {
    const int per = (E + kThreads - 1) / kThreads;
    const int e0 = threadIdx.x * per;
    int64_t mine = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) mine += expert_tiles(s_cnt[e0 + i], NT, NTH);
    int64_t total;
    block_exclusive_scan<int64_t>(mine, s_scan, &total);
    __syncthreads();
    return (int)total;
}

// s_tst[e] = first tile of expert e; returns the total.  All threads of the
// block; ends with a barrier.
MOE_DEVICE int mixed_tile_starts(const int* s_cnt, int E, int NT, int NTH, int* s_tst, int64_t* s_scan) {
    const int per = (E + kThreads - 1) / kThreads;
    const int e0 = threadIdx.x * per;
    int64_t mine = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) mine += expert_tiles(s_cnt[e0 + i], NT, NTH);
    int64_t total;
    int64_t run = block_exclusive_scan<int64_t>(mine, s_scan, &total);
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) {
            s_tst[e0 + i] = (int)run;
            run += expert_tiles(s_cnt[e0 + i], NT, NTH);
        }
    __syncthreads();
    return (int)total;
}

// Logical tile lt: expert-major, then row tile, then column tile.
MOE_DEVICE MixedTile mixed_tile_at(const int* s_off, const int* s_cnt, const int* s_tst, int E, int NT,
                                   int lt) {
    int lo = 0, hi = E - 1;  // last expert whose first tile is <= lt
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tst[mid] <= lt) lo = mid; else hi = mid - 1;
    }
    MixedTile mt;
    mt.e = __builtin_amdgcn_readfirstlane(lo);
    const int local = __builtin_amdgcn_readfirstlane(lt - s_tst[mt.e]);
    const int off = __builtin_amdgcn_readfirstlane(s_off[mt.e]);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[mt.e]);
    const int full = cnt / kBM;
    if (local < full * NT) {
        mt.row0 = off + (local / NT) * kBM;
        mt.rows_valid = kBM;
        mt.nt = local % NT;
        mt.half = false;
    } else {
        mt.row0 = off + full * kBM;
        mt.rows_valid = cnt - full * kBM;
        mt.nt = local - full * NT;
        mt.half = 2 * mt.rows_valid <= kBM;
    }
    return mt;
}

}  // namespace

}  // namespace moegmm
