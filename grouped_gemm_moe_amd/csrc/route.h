// Routing inside a decode-shaped forward GMM (moe_decode_fwd,
// moe_decode_fwd_mx): every workgroup counts the expert histogram of the
// slots' ids itself and ranks its own expert's slots, so no permute launch
// runs before the GMM.  The results are those of moe_permute_index ("NPU
// Training Operators - GMM", 算子语义: tokens_per_expert as the histogram of
// the selected ids; rows grouped by expert, in slot order inside an expert).
// For workgroups of kRouteThreads threads.
#pragma once

#include "common.h"

namespace moegmm {

constexpr int kRouteThreads = 256;

// Routing inputs of a routed forward GMM and the maps it writes.
struct RouteArgs {
    const int32_t* ids = nullptr;          // [T * top_k] expert of each slot, or -1
    int32_t* row_id_map = nullptr;         // [T * top_k] slot -> row (OUT)
    int32_t* sorted_slot = nullptr;        // [T * top_k] row -> slot (OUT)
    int64_t* tokens_per_expert = nullptr;  // [E] (OUT)
};

// Slots [s0, s1) of this thread: S slots in contiguous chunks, so that
// ranks in slot order follow from one block scan of per-thread counts.
MOE_DEVICE void slot_chunk(int S, int& s0, int& s1) {
    const int C = (S + kRouteThreads - 1) / kRouteThreads;
    s0 = threadIdx.x * C < S ? threadIdx.x * C : S;
    s1 = s0 + C < S ? s0 + C : S;
}

// The routed gate_up's group ranges: every block counts the histogram of the
// slots' expert ids itself (ids outside [-1, E) count nowhere and, from the
// block with `report`, set MOE_DEVERR_EXPERT_ID), then takes the exclusive
// offsets -- the tokens_per_expert and row offsets that moe_permute_index
// produces.  All threads; ends with a barrier.
MOE_DEVICE void route_group_ranges(const int32_t* __restrict__ ids, int S, int E, int* s_off, int* s_cnt,
                                   int64_t* s_scan, int32_t* dev_err, bool report) {
    for (int e = threadIdx.x; e < E; e += kRouteThreads) s_cnt[e] = 0;
    __syncthreads();
    int s0, s1;
    slot_chunk(S, s0, s1);
    bool bad = false;
    for (int s = s0; s < s1; ++s) {
        const int id = ids[s];
        if (id >= 0 && id < E) atomicAdd(&s_cnt[id], 1);
        else bad |= id != -1;
    }
    if (bad && report && dev_err) atomicOr(dev_err, MOE_DEVERR_EXPERT_ID);
    __syncthreads();
    const int per = (E + kRouteThreads - 1) / kRouteThreads;
    const int e0 = threadIdx.x * per;
    int64_t mine = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) mine += s_cnt[e0 + i];
    int64_t total;
    int64_t run = block_exclusive_scan<int64_t>(mine, s_scan, &total);
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) {
            s_off[e0 + i] = (int)run;
            run += s_cnt[e0 + i];
        }
    __syncthreads();
}

// The slots of expert e ranked rank0 .. rank0 + rows - 1 in slot order, into
// s_rows.  All threads; ends with a barrier.
MOE_DEVICE void route_rows(const int32_t* __restrict__ ids, int S, int e, int rank0, int rows, int* s_rows,
                           int64_t* s_scan) {
    int s0, s1;
    slot_chunk(S, s0, s1);
    int64_t mine = 0;
    for (int s = s0; s < s1; ++s) mine += ids[s] == e;
    int64_t total;
    int64_t rank = block_exclusive_scan<int64_t>(mine, s_scan, &total);
    for (int s = s0; s < s1 && rank < rank0 + rows; ++s)
        if (ids[s] == e) {
            if (rank >= rank0) s_rows[rank - rank0] = s;
            ++rank;
        }
    __syncthreads();
}

// The routed gate_up's whole-call outputs, by one block: tokens_per_expert,
// and row_id_map = -1 for the slots that take no part.
MOE_DEVICE void route_call_outputs(const RouteArgs& ra, int E, int S, const int* s_cnt) {
    for (int e = threadIdx.x; e < E; e += kRouteThreads) ra.tokens_per_expert[e] = s_cnt[e];
    for (int s = threadIdx.x; s < S; s += kRouteThreads) {
        const int id = ra.ids[s];
        if (!(id >= 0 && id < E)) ra.row_id_map[s] = -1;
    }
}

}  // namespace moegmm
