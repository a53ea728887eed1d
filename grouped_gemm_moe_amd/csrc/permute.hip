// moe_permute on gfx950: histogram of expert ids, stable grouping of slots by
// expert, and the gather of token rows into expert-contiguous order.
//
// What is computed follows "NPU Training Operators - GMM" (section
// "Qwen3.5 MoE 路径": permute by the selected experts, tokens_per_expert as a
// histogram of the ids; section 算子语义: the worked example, whose permuted
// order lists each expert's tokens in token order) and "MegaMoE" (A16W16
// Dispatch: X_e stacks the tokens routed to e in a fixed order, row(i,k) finds
// token i in it).  The fixed order chosen here is ascending slot index, which
// makes every output unique and bit-reproducible; no float is involved.
//
// Kernels (all deterministic; the only atomics are integer counts in LDS):
//   1. hist    -- one block per chunk of slots: per-block expert histogram.
//   2. scan    -- per expert, an exclusive prefix over blocks, then the
//                 expert offsets (exclusive scan over experts); writes
//                 tokens_per_expert and the per-block starting rows.
//   3. scatter -- one block per chunk: each wave ranks its slots within the
//                 expert in slot order (wave ballots emulate a match-any on
//                 the expert id) and writes row_id_map and sorted_slot.
//   4. gather  -- copies token rows to their permuted rows with 16-byte loads
//                 and stores (coalesced inside each row): each piece of a
//                 token row is loaded once and stored to all of the token's
//                 slot rows; four loads in flight per thread.  The MXFP8
//                 variant quantises the row as it goes (E4M3 codes + E8M0
//                 scales).
// For at most 4096 slots (decode-sized calls) steps 1-3 run as one
// single-workgroup kernel, so the whole permute is two launches.  Where the
// per-block histograms fit LDS (blocks x experts <= 12288) every scatter
// block repeats the scan itself, so steps 2 and 3 are one launch; larger
// tables are scanned by segments of block rows over many workgroups.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "mx.h"

namespace moegmm {

// The per-block histograms of moe_permute_noalloc live here instead of in a
// caller workspace: 1 MiB, held by each device the library runs on until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol); it uses the device address that
// static_scratch() looks up once per device.
constexpr size_t kStaticScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kPermThreads = 256;          // 4 waves
constexpr int kWaves = kPermThreads / 64;
constexpr int64_t kSmallSlots = 4096;      // single-workgroup path up to this many slots

// Slots per block: a multiple of 4*64 so that each wave gets whole groups of
// 64; grown with S so the number of blocks stays <= 4096.
int64_t permute_chunk(int64_t S) {
    const int64_t base = 1024;
    int64_t mult = (S + base * 4096 - 1) / (base * 4096);
    if (mult < 1) mult = 1;
    return base * mult;
}

MOE_DEVICE bool valid_id(int32_t id, int E) { return id >= 0 && id < E; }

__global__ __launch_bounds__(kPermThreads) void permute_hist_kernel(
    const int32_t* __restrict__ ids, int64_t S, int E, int64_t chunk, int32_t* __restrict__ blk_hist,
    int32_t* dev_err) {
    __shared__ int32_t hist[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int64_t s0 = (int64_t)blockIdx.x * chunk;
    const int64_t s1 = s0 + chunk < S ? s0 + chunk : S;
    int bad = 0;
    // kHistLoads ids in flight per thread, then their counts (one load per
    // iteration would wait out an L2 round trip each time)
    constexpr int kHistLoads = 4;
    for (int64_t s = s0 + threadIdx.x; s < s1; s += (int64_t)blockDim.x * kHistLoads) {
        int32_t id[kHistLoads];
#pragma unroll
        for (int u = 0; u < kHistLoads; ++u) {
            const int64_t su = s + (int64_t)u * blockDim.x;
            id[u] = su < s1 ? ids[su] : -1;
        }
#pragma unroll
        for (int u = 0; u < kHistLoads; ++u) {
            if (valid_id(id[u], E)) atomicAdd(&hist[id[u]], 1);
            else if (id[u] != -1) bad = 1;
        }
    }
    if (bad && dev_err) atomicOr(dev_err, MOE_DEVERR_EXPERT_ID);
    __syncthreads();
    int32_t* out = blk_hist + (int64_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
}

// Tables too large for the fused scan (blocks x experts > kScanLdsInts) are
// scanned in two launches.  1: segments of kSegBlocks block rows, one thread
// per (expert, segment): the entries become exclusive prefixes within the
// segment, the segment's total goes to seg[segment][expert].  2: one block
// turns the segment totals into each segment's first row (the expert's
// offset over all experts plus the segments before) and writes
// tokens_per_expert.  The scatter then starts block b of expert e at
// table[b][e] + seg[b / kSegBlocks][e].
constexpr int64_t kScanLdsInts = 12288;  // 48 KiB
constexpr int64_t kSegBlocks = 64;

int64_t scan_segments(int64_t nblk) { return (nblk + kSegBlocks - 1) / kSegBlocks; }

__global__ __launch_bounds__(kPermThreads) void permute_segscan_kernel(int32_t* __restrict__ blk_hist,
                                                                     int64_t nblk, int E,
                                                                     int32_t* __restrict__ seg) {
    const int e = blockIdx.x * kPermThreads + threadIdx.x;
    if (e >= E) return;
    const int64_t b0 = (int64_t)blockIdx.y * kSegBlocks;
    const int64_t b1 = b0 + kSegBlocks < nblk ? b0 + kSegBlocks : nblk;
    int32_t run = 0;
    for (int64_t b = b0; b < b1; ++b) {
        const int32_t v = blk_hist[b * E + e];
        blk_hist[b * E + e] = run;
        run += v;
    }
    seg[(int64_t)blockIdx.y * E + e] = run;
}

// One block.  Thread i owns experts [i*per, i*per + per) so that the scan
// over threads runs in ascending expert order.
__global__ __launch_bounds__(kPermThreads) void permute_segbase_kernel(int32_t* __restrict__ seg,
                                                                     int64_t nseg, int E,
                                                                     int64_t* __restrict__ tokens_per_expert) {
    __shared__ int64_t scan_tmp[kPermThreads / 64];
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per;
    int64_t cnt[4] = {0, 0, 0, 0};
    int64_t mine = 0;
    for (int i = 0; i < per && i < 4; ++i) {
        const int e = e0 + i;
        if (e >= E) break;
        int64_t c = 0;
        for (int64_t q = 0; q < nseg; ++q) c += seg[q * E + e];
        cnt[i] = c;
        mine += c;
    }
    int64_t total;
    int64_t off = block_exclusive_scan<int64_t>(mine, scan_tmp, &total);
    for (int i = 0; i < per && i < 4; ++i) {
        const int e = e0 + i;
        if (e >= E) break;
        tokens_per_expert[e] = cnt[i];
        int64_t run = off;
        for (int64_t q = 0; q < nseg; ++q) {
            const int32_t v = seg[q * E + e];
            seg[q * E + e] = (int32_t)run;
            run += v;
        }
        off += cnt[i];
    }
}

// Per-wave pieces shared by the multi-block and the single-block paths.  Each
// wave owns the slot range [w0, w1) (consecutive ranges in wave order).

// counts per expert of the wave's slots into cnt (LDS, zeroed by the caller)
MOE_DEVICE void wave_counts(const int32_t* __restrict__ ids, int64_t w0, int64_t w1, int E,
                            int32_t* cnt) {
    const int lane = threadIdx.x & 63;
    for (int64_t s = w0 + lane; s < w1; s += 64) {
        const int32_t id = ids[s];
        if (valid_id(id, E)) atomicAdd(&cnt[id], 1);
    }
}

// Stable rank of one group of 64 consecutive slots (g .. g+63, lane l holds
// slot g+l with expert `id`, -1 if masked or past w1) within its expert.
// next_row[e] holds the wave's next row for expert e and is advanced.
MOE_DEVICE void rank_group(int64_t g, int64_t w1, int32_t id, int E, int nbits, int32_t* next_row,
                           int32_t* __restrict__ row_id_map, int32_t* __restrict__ sorted_slot) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t s = g + lane;
    const bool ok = valid_id(id, E);
    const int key = ok ? id : 0;
    // peers = lanes with the same expert (match-any built from ballots)
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    int32_t row = -1;
    if (ok) row = next_row[key] + __popcll(peers & lt_mask);
    // all lanes have read next_row before the leaders update it
    __builtin_amdgcn_wave_barrier();
    if (ok && (peers & lt_mask) == 0) next_row[key] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (s < w1) {
        row_id_map[s] = row;
        if (ok) sorted_slot[row] = (int32_t)s;
    }
}

MOE_DEVICE int id_bits(int E) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    return nbits;
}

// Stable rank of every slot within its expert, groups of 64 slots in order.
MOE_DEVICE void wave_rank_scatter(const int32_t* __restrict__ ids, int64_t w0, int64_t w1, int E,
                                  int32_t* next_row, int32_t* __restrict__ row_id_map,
                                  int32_t* __restrict__ sorted_slot) {
    const int lane = threadIdx.x & 63;
    const int nbits = id_bits(E);
    for (int64_t g = w0; g < w1; g += 64) {
        const int64_t s = g + lane;
        rank_group(g, w1, (s < w1) ? ids[s] : -1, E, nbits, next_row, row_id_map, sorted_slot);
    }
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t S, int E, int64_t chunk,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ seg_base,
    int32_t* __restrict__ row_id_map, int32_t* __restrict__ sorted_slot) {
    __shared__ int32_t next_row[kWaves][kMaxExperts];
    const int wid = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kWaves * E; i += blockDim.x) next_row[i / E][i % E] = 0;
    __syncthreads();

    const int64_t s0 = (int64_t)blockIdx.x * chunk;
    const int64_t sub = chunk / kWaves;  // slots per wave, multiple of 64
    const int64_t w0 = s0 + wid * sub;
    const int64_t w1 = w0 + sub < S ? w0 + sub : S;

    wave_counts(ids, w0, w1, E, next_row[wid]);
    __syncthreads();
    // starting row of every wave for every expert
    const int32_t* base = blk_base + (int64_t)blockIdx.x * E;
    const int32_t* sbase = seg_base + (int64_t)blockIdx.x / kSegBlocks * E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int32_t run = base[e] + sbase[e];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int32_t c = next_row[w][e];
            next_row[w][e] = run;
            run += c;
        }
    }
    __syncthreads();
    wave_rank_scatter(ids, w0, w1, E, next_row[wid], row_id_map, sorted_slot);
}

// Scan and scatter in one launch, for chunks of kFusedChunk slots whose
// per-block table fits LDS: every block stages the whole table, finds each
// expert's total and its own blocks-before prefix, scans the totals over
// experts (block 0 writes tokens_per_expert) and ranks its slots as
// permute_scatter_kernel does.  The blocks repeat the scan instead of
// waiting for one block to do it; each wave loads its 4 x 64 expert ids once,
// together with the table, and keeps them in registers.
constexpr int64_t kFusedChunk = 1024;
constexpr int kFusedGroups = kFusedChunk / kWaves / 64;  // 64-slot groups per wave

__global__ __launch_bounds__(kPermThreads) void permute_scan_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t S, int E, int64_t nblk, const int32_t* __restrict__ blk_hist,
    int64_t* __restrict__ tokens_per_expert, int32_t* __restrict__ row_id_map,
    int32_t* __restrict__ sorted_slot) {
    __shared__ int32_t s_hist[kScanLdsInts];
    __shared__ int32_t next_row[kWaves][kMaxExperts];
    __shared__ int64_t scan_tmp[kPermThreads / 64];
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w0 = (int64_t)blockIdx.x * kFusedChunk + wid * (kFusedChunk / kWaves);
    const int64_t w1 = w0 + kFusedChunk / kWaves < S ? w0 + kFusedChunk / kWaves : S;
    int32_t id[kFusedGroups];
#pragma unroll
    for (int q = 0; q < kFusedGroups; ++q) {
        const int64_t s = w0 + q * 64 + lane;
        id[q] = s < w1 ? ids[s] : -1;
    }
    const int64_t n = nblk * E;
    // the table with kStageLoads loads in flight per thread (a plain copy loop
    // waits out one L2 round trip per entry it stages)
    constexpr int kStageLoads = 16;
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += (int64_t)blockDim.x * kStageLoads) {
        int32_t v[kStageLoads];
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int64_t i = i0 + (int64_t)u * blockDim.x;
            v[u] = i < n ? blk_hist[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int64_t i = i0 + (int64_t)u * blockDim.x;
            if (i < n) s_hist[i] = v[u];
        }
    }
    for (int i = threadIdx.x; i < kWaves * E; i += blockDim.x) next_row[i / E][i % E] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kFusedGroups; ++q)
        if (valid_id(id[q], E)) atomicAdd(&next_row[wid][id[q]], 1);
    // per expert (thread owns <= 4, in expert order): the total over blocks
    // and the part in blocks before this one
    const int per = (E + kPermThreads - 1) / kPermThreads;
    const int e0 = threadIdx.x * per;
    int64_t tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
    int64_t mine = 0;
    for (int i = 0; i < per && i < 4; ++i) {
        const int e = e0 + i;
        if (e >= E) break;
        for (int64_t b = 0; b < nblk; ++b) {
            const int32_t c = s_hist[b * E + e];
            tot[i] += c;
            pre[i] += b < (int64_t)blockIdx.x ? c : 0;
        }
        mine += tot[i];
    }
    int64_t total;
    int64_t off = block_exclusive_scan<int64_t>(mine, scan_tmp, &total);  // its barriers also order the counts
    for (int i = 0; i < per && i < 4; ++i) {
        const int e = e0 + i;
        if (e >= E) break;
        if (blockIdx.x == 0) tokens_per_expert[e] = tot[i];
        int32_t run = (int32_t)(off + pre[i]);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int32_t c = next_row[w][e];
            next_row[w][e] = run;
            run += c;
        }
        off += tot[i];
    }
    __syncthreads();
    const int nbits = id_bits(E);
#pragma unroll
    for (int q = 0; q < kFusedGroups; ++q)
        rank_group(w0 + q * 64, w1, id[q], E, nbits, next_row[wid], row_id_map, sorted_slot);
}

// All of histogram, expert offsets and ranking in one workgroup, for inputs
// of at most one chunk (decode-sized calls: one launch instead of three).
__global__ __launch_bounds__(kPermThreads) void permute_small_kernel(
    const int32_t* __restrict__ ids, int64_t S, int E, int64_t* __restrict__ tokens_per_expert,
    int32_t* __restrict__ row_id_map, int32_t* __restrict__ sorted_slot, int32_t* dev_err) {
    __shared__ int32_t next_row[kWaves][kMaxExperts];
    __shared__ int64_t scan_tmp[kPermThreads / 64];
    const int wid = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < kWaves * E; i += blockDim.x) next_row[i / E][i % E] = 0;
    __syncthreads();
    const int64_t sub = (S + kWaves * 64 - 1) / (kWaves * 64) * 64;  // multiple of 64
    const int64_t w0 = wid * sub < S ? wid * sub : S;
    const int64_t w1 = w0 + sub < S ? w0 + sub : S;
    // the wave's ids, loaded once (at most kSmallSlots / kWaves per wave)
    constexpr int kPerLane = (int)(kSmallSlots / (kWaves * 64));
    int32_t id[kPerLane];
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const int64_t s = w0 + q * 64 + lane;
        id[q] = s < w1 ? ids[s] : -1;
    }
    int bad = 0;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        if (valid_id(id[q], E)) atomicAdd(&next_row[wid][id[q]], 1);
        else if (id[q] != -1) bad = 1;
    }
    if (bad && dev_err) atomicOr(dev_err, MOE_DEVERR_EXPERT_ID);
    __syncthreads();
    // per-expert totals, scanned in expert order (thread owns <= 4 experts)
    const int per = (E + kPermThreads - 1) / kPermThreads;
    const int e0 = threadIdx.x * per;
    int64_t tot[4] = {0, 0, 0, 0};
    int64_t mine = 0;
    for (int i = 0; i < per && i < 4; ++i) {
        const int e = e0 + i;
        if (e >= E) break;
        for (int w = 0; w < kWaves; ++w) tot[i] += next_row[w][e];
        mine += tot[i];
    }
    int64_t total;
    int64_t off = block_exclusive_scan<int64_t>(mine, scan_tmp, &total);
    for (int i = 0; i < per && i < 4; ++i) {
        const int e = e0 + i;
        if (e >= E) break;
        tokens_per_expert[e] = tot[i];
        int32_t run = (int32_t)off;
        for (int w = 0; w < kWaves; ++w) {
            const int32_t c = next_row[w][e];
            next_row[w][e] = run;
            run += c;
        }
        off += tot[i];
    }
    __syncthreads();
    const int nbits = id_bits(E);
#pragma unroll
    for (int q = 0; q < kPerLane; ++q)
        if (w0 + q * 64 < w1) rank_group(w0 + q * 64, w1, id[q], E, nbits, next_row[wid], row_id_map, sorted_slot);
}

// Gather, token by token: a block owns tpb consecutive tokens, loads each
// 16-byte piece of a token row once and stores it to every row its valid
// slots map to (top_k stores per load), so a top-8 permute reads x once.
#ifndef MOEGMM_GATHER_SLOTS
#define MOEGMM_GATHER_SLOTS 16
#endif
constexpr int kGatherMaxSlots = MOEGMM_GATHER_SLOTS;  // tpb * top_k <= max(this, top_k)
static_assert(kGatherMaxSlots <= 64, "32-bit piece indices: tokens per block x 2^18 pieces < 2^31");
constexpr int kGatherUnroll = 4;     // 16-byte loads in flight per thread

__global__ __launch_bounds__(kPermThreads) void permute_gather_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ row_id_map, int64_t T, int top_k,
    int64_t H, int tpb, uint16_t* __restrict__ x_perm) {
    __shared__ int32_t rows[kGatherMaxSlots > 32 ? kGatherMaxSlots : 32];  // top_k <= 32
    const int64_t S = T * top_k;
    const int64_t t0 = (int64_t)blockIdx.x * tpb;
    const int nslots = tpb * top_k;
    if ((int)threadIdx.x < nslots) {
        const int64_t s = t0 * top_k + threadIdx.x;
        const int32_t r = (s < S) ? row_id_map[s] : -1;
        rows[threadIdx.x] = (r >= 0 && r < S) ? r : -1;
    }
    __syncthreads();
    // 32-bit piece indices: at most 16 tokens of 2^18 pieces per block
    const int cpr = (int)(H / 8);  // 16-byte chunks per row
    const int tok = (int)(T - t0 < tpb ? T - t0 : tpb);
    const int total = tok * cpr;
    const uint16_t* xb = x + t0 * H;
    for (int i0 = (int)threadIdx.x; i0 < total; i0 += kPermThreads * kGatherUnroll) {
        u32x4_t v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int i = i0 + u * kPermThreads;
            if (i < total) {
                const int tt = i / cpr, c = i - tt * cpr;
                v[u] = ld16(xb + (int64_t)tt * H + c * 8);
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int i = i0 + u * kPermThreads;
            if (i < total) {
                const int tt = i / cpr, c = i - tt * cpr;
                for (int k = 0; k < top_k; ++k) {
                    const int32_t r = rows[tt * top_k + k];
                    if (r >= 0) st16(x_perm + (int64_t)r * H + c * 8, v[u]);
                }
            }
        }
    }
}

// The same gather with MX quantisation of each token row on the way (row-wise
// Q_MX commutes with the gather, so a top-k token is quantised once): a lane
// owns 32 bytes of a row (16 bf16, two loads), a lane pair one group of 32,
// and the pair meets on the group's maximum with one DPP permute
// (pair_max); each lane stores its 16 codes as one 16-byte store, and the
// pair's first lane the scale byte, to every slot row of the token.
__global__ __launch_bounds__(kPermThreads) void permute_gather_mx_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ row_id_map, int64_t T, int top_k,
    int64_t H, int tpb, int64_t ld_s, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
    __shared__ int32_t rows[kGatherMaxSlots > 32 ? kGatherMaxSlots : 32];  // top_k <= 32
    const int64_t S = T * top_k;
    const int64_t t0 = (int64_t)blockIdx.x * tpb;
    const int nslots = tpb * top_k;
    if ((int)threadIdx.x < nslots) {
        const int64_t s = t0 * top_k + threadIdx.x;
        const int32_t r = (s < S) ? row_id_map[s] : -1;
        rows[threadIdx.x] = (r >= 0 && r < S) ? r : -1;
    }
    __syncthreads();
    const int cpr = (int)(H / 16);  // 32-byte pieces per row, even (H is a multiple of 32)
    const int tok = (int)(T - t0 < tpb ? T - t0 : tpb);
    const int total = tok * cpr;    // even; at most 16 tokens x 2^17 pieces
    const uint16_t* xb = x + t0 * H;
    // every lane runs the same number of iterations (the pair maximum needs both lanes)
    constexpr int kU = kGatherUnroll / 2;  // pieces per lane per iteration (two loads each)
    constexpr int kStep = kPermThreads * kU;
    const int iters = (total + kStep - 1) / kStep;
    for (int it = 0; it < iters; ++it) {
        const int i0 = it * kStep + (int)threadIdx.x;
        u32x4_t v[kU][2];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int i = i0 + u * kPermThreads;
            v[u][0] = v[u][1] = u32x4_t{0u, 0u, 0u, 0u};
            if (i < total) {
                const int tt = i / cpr, c = i - tt * cpr;
                const uint16_t* p = xb + (int64_t)tt * H + c * 16;
                v[u][0] = ld16(p);
                v[u][1] = ld16(p + 8);
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int i = i0 + u * kPermThreads;
            float f[16];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    f[8 * h + 2 * c] = bf16_lo(v[u][h][c]);
                    f[8 * h + 2 * c + 1] = bf16_hi(v[u][h][c]);
                }
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(f[c]));
            amax = pair_max(amax);
            if (i < total) {  // whole pairs agree: total and i0 - threadIdx.x are even
                const uint32_t sb = mx_scale_byte(amax);
                const float inv = mx_inv_scale(sb);
                u32x4_t o;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[q] = e4m3_pack4(f[4 * q] * inv, f[4 * q + 1] * inv, f[4 * q + 2] * inv, f[4 * q + 3] * inv);
                const int tt = i / cpr, c = i - tt * cpr;
                for (int k = 0; k < top_k; ++k) {
                    const int32_t r = rows[tt * top_k + k];
                    if (r >= 0) {
                        st16(xq + (int64_t)r * H + c * 16, o);
                        if ((c & 1) == 0) xs[(int64_t)r * ld_s + (c >> 1)] = (uint8_t)sb;
                    }
                }
            }
        }
    }
}

// Tokens per gather block: up to kGatherMaxSlots slots, but at most T/256
// tokens so that the launch still has some 256 blocks to spread.  (16 slots
// measured best on the decode, prefill and top-1 EP shapes; 32 and 64 lose
// up to 50 % on the EP shape.)
int gather_tokens_per_block(int64_t T, int64_t top_k) {
    int64_t tpb = kGatherMaxSlots / top_k;
    const int64_t cap = T / 256;
    if (tpb > cap) tpb = cap;
    return tpb < 1 ? 1 : (int)tpb;
}

}  // namespace

size_t permute_static_scratch_bytes() { return kStaticScratchBytes; }

// Device address of `scratch` on the current device, looked up on the first
// call per device (hipGetSymbolAddress; each device holds its own copy of the
// array at its own address) and kept.  nullptr, with the error, on failure.
static void* static_scratch(hipError_t* err) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

// The per-block table, then (for the two-launch scan) the segment table.
static size_t table_bytes(int64_t nblk, int64_t E) {
    return ((size_t)(nblk * E) * sizeof(int32_t) + 255) / 256 * 256;
}
size_t permute_workspace_bytes(int64_t S, int64_t E) {
    const int64_t chunk = permute_chunk(S);
    const int64_t nblk = (S + chunk - 1) / chunk;
    size_t bytes = table_bytes(nblk, E);
    if (!(chunk == kFusedChunk && nblk * E <= kScanLdsInts))
        bytes += ((size_t)(scan_segments(nblk) * E) * sizeof(int32_t) + 255) / 256 * 256;
    return bytes < 256 ? 256 : bytes;
}

hipError_t launch_permute(const uint16_t* x, const int32_t* ids, int64_t T, int64_t top_k,
                          int64_t H, int64_t E, uint16_t* x_perm, uint8_t* xq, uint8_t* xs,
                          int64_t ld_xs, int32_t* row_id_map, int32_t* sorted_slot,
                          int64_t* tokens_per_expert, void* ws, int32_t* dev_err,
                          hipStream_t stream) {
    const int64_t S = T * top_k;
    const int64_t chunk = permute_chunk(S);
    const int64_t nblk = (S + chunk - 1) / chunk;
    int32_t* blk = static_cast<int32_t*>(ws);
    if (S > 0 && S <= kSmallSlots) {
        hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kPermThreads), 0, stream, ids, S,
                           (int)E, tokens_per_expert, row_id_map, sorted_slot, dev_err);
    } else {
        if (nblk > 0)
            hipLaunchKernelGGL(permute_hist_kernel, dim3((unsigned)nblk), dim3(kPermThreads), 0,
                               stream, ids, S, (int)E, chunk, blk, dev_err);
        if (nblk > 0 && chunk == kFusedChunk && nblk * E <= kScanLdsInts) {
            hipLaunchKernelGGL(permute_scan_scatter_kernel, dim3((unsigned)nblk), dim3(kPermThreads), 0,
                               stream, ids, S, (int)E, nblk, blk, tokens_per_expert, row_id_map,
                               sorted_slot);
        } else {
            // also for no slots at all: then only tokens_per_expert (zeros) is written
            int32_t* seg = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + table_bytes(nblk, E));
            const int64_t nseg = scan_segments(nblk);
            if (nblk > 0)
                hipLaunchKernelGGL(permute_segscan_kernel,
                                   dim3((unsigned)((E + kPermThreads - 1) / kPermThreads), (unsigned)nseg),
                                   dim3(kPermThreads), 0, stream, blk, nblk, (int)E, seg);
            hipLaunchKernelGGL(permute_segbase_kernel, dim3(1), dim3(kPermThreads), 0, stream, seg, nseg,
                               (int)E, tokens_per_expert);
            if (nblk > 0)
                hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)nblk), dim3(kPermThreads), 0, stream,
                                   ids, S, (int)E, chunk, blk, seg, row_id_map, sorted_slot);
        }
    }
    if (nblk > 0 && (xq || x_perm)) {  // neither: the index kernels only
        const int tpb = gather_tokens_per_block(T, top_k);
        const int64_t gblk = (T + tpb - 1) / tpb;
        if (xq)
            hipLaunchKernelGGL(permute_gather_mx_kernel, dim3((unsigned)gblk), dim3(kPermThreads),
                               0, stream, x, row_id_map, T, (int)top_k, H, tpb, ld_xs, xq, xs);
        else
            hipLaunchKernelGGL(permute_gather_kernel, dim3((unsigned)gblk), dim3(kPermThreads), 0,
                               stream, x, row_id_map, T, (int)top_k, H, tpb, x_perm);
    }
    return hipGetLastError();
}

hipError_t launch_permute_noalloc(const uint16_t* x, const int32_t* ids, int64_t T, int64_t top_k,
                                  int64_t H, int64_t E, uint16_t* x_perm, int32_t* row_id_map,
                                  int32_t* sorted_slot, int64_t* tokens_per_expert, int32_t* dev_err,
                                  hipStream_t stream) {
    hipError_t err = hipSuccess;
    void* ws = static_scratch(&err);
    if (ws == nullptr) return err;
    // the histograms are written whole by every call before they are read:
    // nothing in the scratch needs clearing
    return launch_permute(x, ids, T, top_k, H, E, x_perm, nullptr, nullptr, 0, row_id_map, sorted_slot,
                          tokens_per_expert, ws, dev_err, stream);
}

}  // namespace moegmm
