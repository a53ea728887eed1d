// C ABI of libmoegmm: argument validation, workspace sizing and dispatch to
// the gfx950 kernels.  Host-checkable problems return a status before
// anything is enqueued, in the spirit of the two-phase interface of the
// MoeTokenPermuteWithRoutingMapGrad article (sections 3 and 4.2-4.3: check
// null and invalid arguments, report a workspace size, then execute), and of
// "MegaMoE" (constraints: mismatched arguments are rejected, never silently
// handled another way).
#include <hip/hip_runtime.h>

#include "launch.h"
#include "moegmm.h"

namespace {

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxTopK = 32;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool dim_ok(int64_t d) { return d > 0 && d % 8 == 0 && d <= (int64_t(1) << 24); }
// GMM operand tiles address up to 256 rows of a matrix with 32-bit byte
// offsets, which bounds the row length (K or N) at 2^21 elements.
constexpr int64_t kMaxGmmDim = int64_t(1) << 21;

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// The MX kernels address one expert's weight codes ([N][K] bytes) with 31-bit
// byte offsets from the expert's base (the weight-streaming kernel walks all
// N rows from it, the SwiGLU tile pairs gate row c with up row N/2 + c), so
// an expert's codes must stay below that range.
constexpr int64_t kMaxMxExpertBytes = 0x7FFF0000;

// An MX tensor's scale rows: at least ceil(K/32) bytes, padded to 16.
bool mx_ld_ok(int64_t ld_s, int64_t K) { return ld_s >= (K + 31) / 32 && ld_s % 16 == 0; }

moe_status check_gmm_mx(const void* xq, const void* xs, int64_t ld_xs, const void* wq,
                        const void* ws, int64_t ld_ws, const void* gl, int64_t E, int64_t M_cap,
                        int64_t K, int64_t N) {
    if (!gl || !wq || !ws || (M_cap > 0 && (!xq || !xs))) return MOE_ERR_NULL;
    if (E < 1 || E > kMaxE || M_cap < 0 || M_cap > kMaxRows || !dim_ok(K) || !dim_ok(N) ||
        K % 32 != 0 || K > kMaxGmmDim || N > kMaxGmmDim || N * K > kMaxMxExpertBytes)
        return MOE_ERR_INVALID;
    if (!mx_ld_ok(ld_xs, K) || !mx_ld_ok(ld_ws, K)) return MOE_ERR_INVALID;
    if (!aligned(xq, 16) || !aligned(xs, 16) || !aligned(wq, 16) || !aligned(ws, 16) ||
        !aligned(gl, 8))
        return MOE_ERR_INVALID;
    if (M_cap * K > (int64_t(1) << 40) || M_cap * N > (int64_t(1) << 40) ||
        E * K * N > (int64_t(1) << 40) || M_cap * ld_xs > (int64_t(1) << 40) ||
        E * N * ld_ws > (int64_t(1) << 40))
        return MOE_ERR_INVALID;
    return MOE_OK;
}

// Byte ranges [a, a + na) and [b, b + nb) share an address (empty ranges never do).
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

moe_status check_gmm_common(const void* a, const void* b, const void* gl, const void* out,
                            int64_t E, int64_t M_cap, int64_t K, int64_t N, size_t ws_need,
                            size_t ws_bytes, const void* ws) {
    if (!gl || (M_cap > 0 && (!a || !out)) || !b) return MOE_ERR_NULL;
    if (E < 1 || E > kMaxE || M_cap < 0 || M_cap > kMaxRows || !dim_ok(K) || !dim_ok(N) ||
        K > kMaxGmmDim || N > kMaxGmmDim)
        return MOE_ERR_INVALID;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16) || !aligned(gl, 8))
        return MOE_ERR_INVALID;
    if (M_cap * K > (int64_t(1) << 40) || M_cap * N > (int64_t(1) << 40) ||
        E * K * N > (int64_t(1) << 40))
        return MOE_ERR_INVALID;
    if (ws_need > 0 && (ws == nullptr || ws_bytes < ws_need)) return MOE_ERR_WORKSPACE;
    if (ws_need > 0 && !aligned(ws, 16)) return MOE_ERR_INVALID;
    return MOE_OK;
}

// The token-row arguments of the gathered forward calls: x [T, K] holds the
// tokens, sorted_slot [M_cap] (M_cap <= T * top_k) the slot of each grouped
// row.  Every byte offset into x must fit 31 bits: T * K < 2^30 elements.
moe_status check_gather(const void* x, const int32_t* sorted_slot, int64_t T, int64_t top_k,
                        int64_t M_cap, int64_t K) {
    if (M_cap > 0 && (!x || !sorted_slot)) return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || T * top_k > kMaxRows || M_cap > T * top_k)
        return MOE_ERR_INVALID;
    if (K > 0 && T * K >= (int64_t(1) << 30)) return MOE_ERR_INVALID;
    if (!aligned(sorted_slot, 4)) return MOE_ERR_INVALID;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_INVALID: return "MOE_ERR_INVALID: a size, limit or alignment is out of range";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than the queried size";
        case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: the HIP runtime rejected a launch";
    }
    return "unknown moe_status";
}

int moegmm_abi_version(void) { return 11; }

size_t moe_permute_workspace_size(int64_t T, int64_t top_k, int64_t E) {
    if (T < 0 || top_k < 1 || E < 1) return 0;
    return moegmm::permute_workspace_bytes(T * top_k, E);
}

}  // extern "C"

namespace {

// Arguments of moe_permute other than the workspace.
moe_status check_permute(const uint16_t* x, const int32_t* topk_ids, int64_t T, int64_t top_k,
                         int64_t H, int64_t E, const uint16_t* x_perm, const int32_t* row_id_map,
                         const int32_t* sorted_slot, const int64_t* tokens_per_expert) {
    if (!tokens_per_expert) return MOE_ERR_NULL;
    if (T > 0 && (!x || !topk_ids || !x_perm || !row_id_map || !sorted_slot)) return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || E < 1 || E > kMaxE || !dim_ok(H))
        return MOE_ERR_INVALID;
    if (T * top_k > kMaxRows) return MOE_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(x_perm, 16) || !aligned(topk_ids, 4) ||
        !aligned(row_id_map, 4) || !aligned(sorted_slot, 4) || !aligned(tokens_per_expert, 8))
        return MOE_ERR_INVALID;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_permute(const uint16_t* x, const int32_t* topk_ids, int64_t T, int64_t top_k,
                       int64_t H, int64_t E, uint16_t* x_perm, int32_t* row_id_map,
                       int32_t* sorted_slot, int64_t* tokens_per_expert, void* ws,
                       size_t ws_bytes, int32_t* dev_err, void* stream) {
    if (!ws) return MOE_ERR_NULL;
    moe_status st = check_permute(x, topk_ids, T, top_k, H, E, x_perm, row_id_map, sorted_slot,
                                  tokens_per_expert);
    if (st != MOE_OK) return st;
    if (!aligned(ws, 4)) return MOE_ERR_INVALID;
    if (ws_bytes < moegmm::permute_workspace_bytes(T * top_k, E)) return MOE_ERR_WORKSPACE;
    return from_hip(moegmm::launch_permute(x, topk_ids, T, top_k, H, E, x_perm, nullptr, nullptr,
                                           0, row_id_map, sorted_slot, tokens_per_expert, ws,
                                           dev_err, static_cast<hipStream_t>(stream)));
}

moe_status moe_permute_noalloc(const uint16_t* x, const int32_t* topk_ids, int64_t T, int64_t top_k,
                               int64_t H, int64_t E, uint16_t* x_perm, int32_t* row_id_map,
                               int32_t* sorted_slot, int64_t* tokens_per_expert, int32_t* dev_err,
                               void* stream) {
    moe_status st = check_permute(x, topk_ids, T, top_k, H, E, x_perm, row_id_map, sorted_slot,
                                  tokens_per_expert);
    if (st != MOE_OK) return st;
    if (moegmm::permute_workspace_bytes(T * top_k, E) > moegmm::permute_static_scratch_bytes())
        return MOE_ERR_WORKSPACE;
    return from_hip(moegmm::launch_permute_noalloc(x, topk_ids, T, top_k, H, E, x_perm, row_id_map,
                                                   sorted_slot, tokens_per_expert, dev_err,
                                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_permute_index(const int32_t* topk_ids, int64_t T, int64_t top_k, int64_t E,
                             int32_t* row_id_map, int32_t* sorted_slot, int64_t* tokens_per_expert,
                             void* ws, size_t ws_bytes, int32_t* dev_err, void* stream) {
    if (!ws || !tokens_per_expert) return MOE_ERR_NULL;
    if (T > 0 && (!topk_ids || !row_id_map || !sorted_slot)) return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || E < 1 || E > kMaxE || T * top_k > kMaxRows)
        return MOE_ERR_INVALID;
    if (!aligned(topk_ids, 4) || !aligned(row_id_map, 4) || !aligned(sorted_slot, 4) ||
        !aligned(tokens_per_expert, 8) || !aligned(ws, 4))
        return MOE_ERR_INVALID;
    if (ws_bytes < moegmm::permute_workspace_bytes(T * top_k, E)) return MOE_ERR_WORKSPACE;
    // no x and no x_perm: the launcher runs the index kernels only
    return from_hip(moegmm::launch_permute(nullptr, topk_ids, T, top_k, 8, E, nullptr, nullptr, nullptr,
                                           0, row_id_map, sorted_slot, tokens_per_expert, ws, dev_err,
                                           static_cast<hipStream_t>(stream)));
}

size_t gmm_workspace_size(int64_t E, int64_t M_cap, int64_t K, int64_t N, int op) {
    return moegmm::gmm_workspace_bytes(E, M_cap, K, N, op);
}

moe_status gmm_fwd(const uint16_t* x, const uint16_t* w, const int64_t* group_list, int64_t E,
                   int64_t M_cap, int64_t K, int64_t N, uint16_t* y, void* ws, size_t ws_bytes,
                   int32_t* dev_err, void* stream) {
    moe_status st = check_gmm_common(x, w, group_list, y, E, M_cap, K, N,
                                     moegmm::gmm_workspace_bytes(E, M_cap, K, N, MOE_GMM_OP_FWD),
                                     ws_bytes, ws);
    if (st != MOE_OK) return st;
    return from_hip(moegmm::launch_gmm_fwd(x, w, group_list, E, M_cap, K, N, y, ws, dev_err,
                                           static_cast<hipStream_t>(stream)));
}

moe_status gmm_fwd_swiglu(const uint16_t* x, const uint16_t* w1, const int64_t* group_list,
                          int64_t E, int64_t M_cap, int64_t K, int64_t I, uint16_t* a,
                          uint16_t* h, void* ws, size_t ws_bytes, int32_t* dev_err,
                          void* stream) {
    if (!dim_ok(I)) return MOE_ERR_INVALID;
    moe_status st = check_gmm_common(x, w1, group_list, a, E, M_cap, K, 2 * I,
                                     moegmm::gmm_workspace_bytes(E, M_cap, K, 2 * I, MOE_GMM_OP_FWD),
                                     ws_bytes, ws);
    if (st != MOE_OK) return st;
    if (!aligned(h, 16)) return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_gmm_fwd_swiglu(x, w1, group_list, E, M_cap, K, I, a, h, ws,
                                                  dev_err, static_cast<hipStream_t>(stream)));
}

moe_status gmm_fwd_gather(const uint16_t* x, const int32_t* sorted_slot, int64_t T, int64_t top_k,
                          const uint16_t* w, const int64_t* group_list, int64_t E, int64_t M_cap,
                          int64_t K, int64_t N, uint16_t* y, void* ws, size_t ws_bytes,
                          int32_t* dev_err, void* stream) {
    moe_status st = check_gather(x, sorted_slot, T, top_k, M_cap, K);
    if (st != MOE_OK) return st;
    st = check_gmm_common(x, w, group_list, y, E, M_cap, K, N,
                          moegmm::gmm_workspace_bytes(E, M_cap, K, N, MOE_GMM_OP_FWD), ws_bytes, ws);
    if (st != MOE_OK) return st;
    moegmm::GatherRows g;
    g.slot = sorted_slot;
    g.top_k = top_k;
    g.nslots = T * top_k;
    return from_hip(moegmm::launch_gmm_fwd(x, w, group_list, E, M_cap, K, N, y, ws, dev_err,
                                           static_cast<hipStream_t>(stream), g));
}

moe_status gmm_fwd_swiglu_gather(const uint16_t* x, const int32_t* sorted_slot, int64_t T,
                                 int64_t top_k, const uint16_t* w1, const int64_t* group_list,
                                 int64_t E, int64_t M_cap, int64_t K, int64_t I, uint16_t* a,
                                 uint16_t* h, void* ws, size_t ws_bytes, int32_t* dev_err,
                                 void* stream) {
    if (!dim_ok(I)) return MOE_ERR_INVALID;
    moe_status st = check_gather(x, sorted_slot, T, top_k, M_cap, K);
    if (st != MOE_OK) return st;
    st = check_gmm_common(x, w1, group_list, a, E, M_cap, K, 2 * I,
                          moegmm::gmm_workspace_bytes(E, M_cap, K, 2 * I, MOE_GMM_OP_FWD), ws_bytes, ws);
    if (st != MOE_OK) return st;
    if (!aligned(h, 16)) return MOE_ERR_INVALID;
    moegmm::GatherRows g;
    g.slot = sorted_slot;
    g.top_k = top_k;
    g.nslots = T * top_k;
    return from_hip(moegmm::launch_gmm_fwd_swiglu(x, w1, group_list, E, M_cap, K, I, a, h, ws, dev_err,
                                                  static_cast<hipStream_t>(stream), g));
}

moe_status swiglu_gmm_fwd(const uint16_t* h, const uint16_t* w2, const int64_t* group_list, int64_t E,
                          int64_t M_cap, int64_t I, int64_t N, uint16_t* a, uint16_t* y, int32_t* dev_err,
                          void* stream) {
    if (!dim_ok(I)) return MOE_ERR_INVALID;
    moe_status st = check_gmm_common(h, w2, group_list, y, E, M_cap, I, N, 0, 0, nullptr);
    if (st != MOE_OK) return st;
    if (M_cap > 0 && !a) return MOE_ERR_NULL;
    if (!aligned(a, 16) || M_cap * 2 * I > (int64_t(1) << 40)) return MOE_ERR_INVALID;
    const size_t bh = (size_t)(M_cap * 2 * I) * 2, ba = (size_t)(M_cap * I) * 2, by = (size_t)(M_cap * N) * 2;
    if (overlaps(a, ba, h, bh) || overlaps(a, ba, y, by) || overlaps(y, by, h, bh)) return MOE_ERR_INVALID;
    if (M_cap == 0) return MOE_OK;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (moegmm::gmm_stream_applies(E, M_cap, I))
        return from_hip(moegmm::launch_stream_swiglu_in(h, w2, group_list, E, M_cap, I, N, a, y, dev_err, hs));
    hipError_t e = moegmm::launch_swiglu(h, group_list, E, M_cap, I, a, hs);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(moegmm::launch_gmm_fwd(a, w2, group_list, E, M_cap, I, N, y, nullptr, dev_err, hs));
}

moe_status gmm_bwd_input(const uint16_t* dy, const uint16_t* w, const int64_t* group_list,
                         int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dx, void* ws,
                         size_t ws_bytes, int32_t* dev_err, void* stream) {
    moe_status st = check_gmm_common(
        dy, w, group_list, dx, E, M_cap, K, N,
        moegmm::gmm_workspace_bytes(E, M_cap, K, N, MOE_GMM_OP_BWD_INPUT), ws_bytes, ws);
    if (st != MOE_OK) return st;
    return from_hip(moegmm::launch_gmm_bwd_input(dy, w, group_list, E, M_cap, K, N, dx, ws, dev_err,
                                                 static_cast<hipStream_t>(stream)));
}

moe_status gmm_bwd_weight(const uint16_t* x, const uint16_t* dy, const int64_t* group_list,
                          int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dw, void* ws,
                          size_t ws_bytes, int32_t* dev_err, void* stream) {
    if (!dw) return MOE_ERR_NULL;
    if (M_cap > 0 && !dy) return MOE_ERR_NULL;
    moe_status st = check_gmm_common(
        x, dy ? dy : x, group_list, dw, E, M_cap, K, N,
        moegmm::gmm_workspace_bytes(E, M_cap, K, N, MOE_GMM_OP_BWD_WEIGHT), ws_bytes, ws);
    if (st != MOE_OK) return st;
    if (!aligned(dw, 16)) return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_gmm_bwd_weight(x, dy, group_list, E, M_cap, K, N, dw, ws,
                                                  dev_err, static_cast<hipStream_t>(stream)));
}

moe_status gmm_bwd(const uint16_t* x, const uint16_t* dy, const uint16_t* w, const int64_t* group_list,
                   int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dx, uint16_t* dw,
                   void* ws, size_t ws_bytes, int32_t* dev_err, void* stream) {
    if (!dw || !dx) return MOE_ERR_NULL;
    if (M_cap > 0 && (!x || !dy)) return MOE_ERR_NULL;
    moe_status st = check_gmm_common(dy ? dy : w, w, group_list, dx, E, M_cap, K, N,
                                     moegmm::gmm_workspace_bytes(E, M_cap, K, N, MOE_GMM_OP_BWD),
                                     ws_bytes, ws);
    if (st != MOE_OK) return st;
    if (!aligned(x, 16) || !aligned(dw, 16)) return MOE_ERR_INVALID;
    const size_t bx = (size_t)(M_cap * K) * 2, bdy = (size_t)(M_cap * N) * 2, bw = (size_t)(E * K * N) * 2;
    if (overlaps(dx, bx, x, bx) || overlaps(dx, bx, dy, bdy) || overlaps(dx, bx, w, bw) ||
        overlaps(dx, bx, dw, bw) || overlaps(dw, bw, x, bx) || overlaps(dw, bw, dy, bdy) ||
        overlaps(dw, bw, w, bw))
        return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_gmm_bwd(x, dy, w, group_list, E, M_cap, K, N, dx, dw, ws, dev_err,
                                           static_cast<hipStream_t>(stream)));
}

moe_status gmm_bwd_swiglu(const uint16_t* x, const uint16_t* dy, const uint16_t* w, const uint16_t* h,
                          const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K, int64_t N,
                          uint16_t* dh, uint16_t* dw, void* ws, size_t ws_bytes, int32_t* dev_err,
                          void* stream) {
    if (!dw || !dh) return MOE_ERR_NULL;
    if (M_cap > 0 && (!x || !dy || !h)) return MOE_ERR_NULL;
    moe_status st = check_gmm_common(dy ? dy : w, w, group_list, dh, E, M_cap, K, N,
                                     moegmm::gmm_workspace_bytes(E, M_cap, K, N, MOE_GMM_OP_BWD),
                                     ws_bytes, ws);
    if (st != MOE_OK) return st;
    if (!aligned(x, 16) || !aligned(h, 16) || !aligned(dw, 16)) return MOE_ERR_INVALID;
    if (M_cap * 2 * K > (int64_t(1) << 40)) return MOE_ERR_INVALID;
    const size_t bx = (size_t)(M_cap * K) * 2, bdy = (size_t)(M_cap * N) * 2, bw = (size_t)(E * K * N) * 2;
    const size_t bh = 2 * bx;
    if ((dh != h && overlaps(dh, bh, h, bh)) || overlaps(dh, bh, x, bx) || overlaps(dh, bh, dy, bdy) ||
        overlaps(dh, bh, w, bw) || overlaps(dh, bh, dw, bw) || overlaps(dw, bw, x, bx) ||
        overlaps(dw, bw, dy, bdy) || overlaps(dw, bw, w, bw) || overlaps(dw, bw, h, bh))
        return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_gmm_bwd_swiglu(x, dy, w, h, group_list, E, M_cap, K, N, dh, dw, ws,
                                                  dev_err, static_cast<hipStream_t>(stream)));
}

moe_status swiglu(const uint16_t* h, const int64_t* group_list, int64_t E, int64_t M_cap,
                  int64_t I, uint16_t* a, void* stream) {
    if (!group_list || (M_cap > 0 && (!h || !a))) return MOE_ERR_NULL;
    if (E < 1 || E > kMaxE || M_cap < 0 || M_cap > kMaxRows || !dim_ok(I)) return MOE_ERR_INVALID;
    if (!aligned(h, 16) || !aligned(a, 16) || !aligned(group_list, 8)) return MOE_ERR_INVALID;
    return from_hip(
        moegmm::launch_swiglu(h, group_list, E, M_cap, I, a, static_cast<hipStream_t>(stream)));
}

moe_status swiglu_bwd(const uint16_t* da, const uint16_t* h, const int64_t* group_list, int64_t E,
                      int64_t M_cap, int64_t I, uint16_t* dh, void* stream) {
    if (!group_list || (M_cap > 0 && (!h || !da || !dh))) return MOE_ERR_NULL;
    if (E < 1 || E > kMaxE || M_cap < 0 || M_cap > kMaxRows || !dim_ok(I)) return MOE_ERR_INVALID;
    if (!aligned(h, 16) || !aligned(da, 16) || !aligned(dh, 16) || !aligned(group_list, 8))
        return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_swiglu_bwd(da, h, group_list, E, M_cap, I, dh,
                                              static_cast<hipStream_t>(stream)));
}

moe_status moe_unpermute(const uint16_t* y_perm, const int32_t* row_id_map, const float* probs,
                         int64_t T, int64_t top_k, int64_t H, uint16_t* out, int32_t* dev_err,
                         void* stream) {
    if (T > 0 && (!y_perm || !row_id_map || !probs || !out)) return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || !dim_ok(H) || T * top_k > kMaxRows)
        return MOE_ERR_INVALID;
    if (!aligned(y_perm, 16) || !aligned(out, 16) || !aligned(row_id_map, 4) || !aligned(probs, 4))
        return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_unpermute(y_perm, row_id_map, probs, T, top_k, H, out, dev_err,
                                             static_cast<hipStream_t>(stream)));
}

moe_status moe_decode_fwd(const uint16_t* x, const int32_t* topk_ids, const float* probs,
                          const uint16_t* w1, const uint16_t* w2, int64_t T, int64_t top_k, int64_t H,
                          int64_t I, int64_t E, uint16_t* out, int32_t* row_id_map, int32_t* sorted_slot,
                          int64_t* tokens_per_expert, uint16_t* h, uint16_t* a, uint16_t* y_perm,
                          int32_t* dev_err, void* stream) {
    if (!w1 || !w2 || !tokens_per_expert) return MOE_ERR_NULL;
    if (T > 0 && (!x || !topk_ids || !probs || !out || !row_id_map || !sorted_slot || !h || !a || !y_perm))
        return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || E < 1 || E > kMaxE || !dim_ok(H) || !dim_ok(I) ||
        T * top_k > kMaxRows || !moegmm::decode_fwd_applies(T, top_k, H, I, E))
        return MOE_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16) || !aligned(h, 16) ||
        !aligned(a, 16) || !aligned(y_perm, 16) || !aligned(topk_ids, 4) || !aligned(probs, 4) ||
        !aligned(row_id_map, 4) || !aligned(sorted_slot, 4) || !aligned(tokens_per_expert, 8))
        return MOE_ERR_INVALID;
    const size_t S = (size_t)(T * top_k);
    const void* buf[] = {x, topk_ids, probs, out, row_id_map, sorted_slot, tokens_per_expert, h, a, y_perm};
    const size_t len[] = {(size_t)(T * H) * 2, S * 4, S * 4, (size_t)(T * H) * 2, S * 4, S * 4,
                          (size_t)E * 8, S * 2 * (size_t)I * 2, S * (size_t)I * 2, S * (size_t)H * 2};
    // every output (index 3 on) apart from every other buffer
    for (int i = 3; i < 10; ++i)
        for (int j = 0; j < 10; ++j)
            if (i != j && overlaps(buf[i], len[i], buf[j], len[j])) return MOE_ERR_INVALID;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = moegmm::launch_gmm_stream_route(x, topk_ids, T, top_k, w1, E, H, 2 * I, h, row_id_map,
                                                   sorted_slot, tokens_per_expert, dev_err, hs);
    if (e != hipSuccess || T == 0) return from_hip(e);
    e = moegmm::launch_stream_swiglu_in(h, w2, tokens_per_expert, E, (int64_t)S, I, H, a, y_perm, dev_err, hs);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(moegmm::launch_unpermute(y_perm, row_id_map, probs, T, top_k, H, out, dev_err, hs));
}

moe_status moe_decode_fwd_mx(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs, const int32_t* topk_ids,
                             const float* probs, const uint8_t* w1q, const uint8_t* w1s, int64_t ld_w1s,
                             const uint8_t* w2q, const uint8_t* w2s, int64_t ld_w2s, int64_t T, int64_t top_k,
                             int64_t H, int64_t I, int64_t E, uint16_t* out, int32_t* row_id_map,
                             int32_t* sorted_slot, int64_t* tokens_per_expert, uint8_t* aq, uint8_t* as,
                             int64_t ld_as, uint16_t* y_perm, int32_t* dev_err, void* stream) {
    if (!tokens_per_expert) return MOE_ERR_NULL;
    if (T > 0 && (!topk_ids || !probs || !out || !row_id_map || !sorted_slot || !aq || !as || !y_perm))
        return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || E < 1 || E > kMaxE || !dim_ok(H) || !dim_ok(I) ||
        T * top_k > kMaxRows || !moegmm::decode_fwd_applies(T, top_k, H, I, E) || I % 32 != 0)
        return MOE_ERR_INVALID;
    const int64_t S = T * top_k;
    // GMM1 on T token rows ([T, H] codes), GMM2 on S rows of A ([S, I] codes)
    moe_status st = check_gmm_mx(xq, xs, ld_xs, w1q, w1s, ld_w1s, tokens_per_expert, E, T, H, 2 * I);
    if (st != MOE_OK) return st;
    st = check_gmm_mx(aq, as, ld_as, w2q, w2s, ld_w2s, tokens_per_expert, E, S, I, H);
    if (st != MOE_OK) return st;
    if (!aligned(out, 16) || !aligned(y_perm, 16) || !aligned(topk_ids, 4) || !aligned(probs, 4) ||
        !aligned(row_id_map, 4) || !aligned(sorted_slot, 4))
        return MOE_ERR_INVALID;
    const size_t bS = (size_t)S;
    const void* buf[] = {xq, xs, topk_ids, probs, out, row_id_map, sorted_slot, tokens_per_expert, aq, as, y_perm};
    const size_t len[] = {(size_t)(T * H), (size_t)(T * ld_xs), bS * 4, bS * 4, (size_t)(T * H) * 2, bS * 4,
                          bS * 4, (size_t)E * 8, bS * (size_t)I, bS * (size_t)ld_as, bS * (size_t)H * 2};
    // every output (index 4 on) apart from every other buffer
    for (int i = 4; i < 11; ++i)
        for (int j = 0; j < 11; ++j)
            if (i != j && overlaps(buf[i], len[i], buf[j], len[j])) return MOE_ERR_INVALID;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = moegmm::launch_gmm_mx_stream_route(xq, xs, ld_xs, topk_ids, T, top_k, w1q, w1s, ld_w1s, E, H, I,
                                                      aq, as, ld_as, row_id_map, sorted_slot, tokens_per_expert,
                                                      dev_err, hs);
    if (e != hipSuccess || T == 0) return from_hip(e);
    e = moegmm::launch_gmm_mx_fwd(aq, as, ld_as, w2q, w2s, ld_w2s, tokens_per_expert, E, S, I, H, y_perm, dev_err, hs);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(moegmm::launch_unpermute(y_perm, row_id_map, probs, T, top_k, H, out, dev_err, hs));
}

moe_status moe_unpermute_bwd(const uint16_t* dout, const uint16_t* y_perm,
                             const int32_t* row_id_map, const float* probs, int64_t T,
                             int64_t top_k, int64_t H, uint16_t* dy_perm, float* dprobs,
                             int32_t* dev_err, void* stream) {
    if (T > 0 && (!dout || !y_perm || !row_id_map || !probs || !dy_perm || !dprobs))
        return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || !dim_ok(H) || T * top_k > kMaxRows)
        return MOE_ERR_INVALID;
    if (!aligned(dout, 16) || !aligned(y_perm, 16) || !aligned(dy_perm, 16) ||
        !aligned(row_id_map, 4) || !aligned(probs, 4) || !aligned(dprobs, 4))
        return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_unpermute_bwd(dout, y_perm, row_id_map, probs, T, top_k, H,
                                                 dy_perm, dprobs, dev_err,
                                                 static_cast<hipStream_t>(stream)));
}

moe_status moe_permute_bwd(const uint16_t* dx_perm, const int32_t* row_id_map, int64_t T,
                           int64_t top_k, int64_t H, uint16_t* dx, int32_t* dev_err,
                           void* stream) {
    if (T > 0 && (!dx_perm || !row_id_map || !dx)) return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || !dim_ok(H) || T * top_k > kMaxRows)
        return MOE_ERR_INVALID;
    if (!aligned(dx_perm, 16) || !aligned(dx, 16) || !aligned(row_id_map, 4))
        return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_permute_bwd(dx_perm, row_id_map, T, top_k, H, dx, dev_err,
                                               static_cast<hipStream_t>(stream)));
}

moe_status mx_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ld_s, uint8_t* q,
                       uint8_t* s, void* stream) {
    if (rows > 0 && (!x || !q || !s)) return MOE_ERR_NULL;
    if (rows < 0 || rows > kMaxRows || K <= 0 || K % 32 != 0 || K > (int64_t(1) << 24) ||
        !mx_ld_ok(ld_s, K) || rows * K > (int64_t(1) << 40))
        return MOE_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(q, 16)) return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_mx_quantize(x, rows, K, ld_s, q, s,
                                               static_cast<hipStream_t>(stream)));
}

moe_status moe_permute_mx(const uint16_t* x, const int32_t* topk_ids, int64_t T, int64_t top_k,
                          int64_t H, int64_t E, uint8_t* xq, uint8_t* xs, int64_t ld_xs,
                          int32_t* row_id_map, int32_t* sorted_slot, int64_t* tokens_per_expert,
                          void* ws, size_t ws_bytes, int32_t* dev_err, void* stream) {
    if (!tokens_per_expert || !ws) return MOE_ERR_NULL;
    if (T > 0 && (!x || !topk_ids || !xq || !xs || !row_id_map || !sorted_slot))
        return MOE_ERR_NULL;
    if (T < 0 || top_k < 1 || top_k > kMaxTopK || E < 1 || E > kMaxE || !dim_ok(H) ||
        H % 32 != 0 || !mx_ld_ok(ld_xs, H))
        return MOE_ERR_INVALID;
    if (T * top_k > kMaxRows) return MOE_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(topk_ids, 4) ||
        !aligned(row_id_map, 4) || !aligned(sorted_slot, 4) || !aligned(tokens_per_expert, 8) ||
        !aligned(ws, 4))
        return MOE_ERR_INVALID;
    if (ws_bytes < moegmm::permute_workspace_bytes(T * top_k, E)) return MOE_ERR_WORKSPACE;
    return from_hip(moegmm::launch_permute(x, topk_ids, T, top_k, H, E, nullptr, xq, xs, ld_xs,
                                           row_id_map, sorted_slot, tokens_per_expert, ws,
                                           dev_err, static_cast<hipStream_t>(stream)));
}

moe_status gmm_mx_fwd(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs, const uint8_t* wq,
                      const uint8_t* ws, int64_t ld_ws, const int64_t* group_list, int64_t E,
                      int64_t M_cap, int64_t K, int64_t N, uint16_t* y, int32_t* dev_err,
                      void* stream) {
    moe_status st = check_gmm_mx(xq, xs, ld_xs, wq, ws, ld_ws, group_list, E, M_cap, K, N);
    if (st != MOE_OK) return st;
    if (M_cap > 0 && !y) return MOE_ERR_NULL;
    if (!aligned(y, 16)) return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_gmm_mx_fwd(xq, xs, ld_xs, wq, ws, ld_ws, group_list, E, M_cap,
                                              K, N, y, dev_err,
                                              static_cast<hipStream_t>(stream)));
}

moe_status gmm_mx_fwd_swiglu(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs,
                             const uint8_t* w1q, const uint8_t* w1s, int64_t ld_w1s,
                             const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K,
                             int64_t I, uint8_t* aq, uint8_t* as, int64_t ld_as,
                             int32_t* dev_err, void* stream) {
    if (!dim_ok(I) || I % 32 != 0 || !mx_ld_ok(ld_as, I)) return MOE_ERR_INVALID;
    moe_status st = check_gmm_mx(xq, xs, ld_xs, w1q, w1s, ld_w1s, group_list, E, M_cap, K, 2 * I);
    if (st != MOE_OK) return st;
    if (M_cap > 0 && (!aq || !as)) return MOE_ERR_NULL;
    if (!aligned(aq, 16) || !aligned(as, 16) || M_cap * ld_as > (int64_t(1) << 40))
        return MOE_ERR_INVALID;
    return from_hip(moegmm::launch_gmm_mx_fwd_swiglu(xq, xs, ld_xs, w1q, w1s, ld_w1s, group_list,
                                                     E, M_cap, K, I, aq, as, ld_as, dev_err,
                                                     static_cast<hipStream_t>(stream)));
}

moe_status gmm_mx_fwd_swiglu_gather(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs,
                                    const int32_t* sorted_slot, int64_t T, int64_t top_k,
                                    const uint8_t* w1q, const uint8_t* w1s, int64_t ld_w1s,
                                    const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K,
                                    int64_t I, uint8_t* aq, uint8_t* as, int64_t ld_as,
                                    int32_t* dev_err, void* stream) {
    if (!dim_ok(I) || I % 32 != 0 || !mx_ld_ok(ld_as, I)) return MOE_ERR_INVALID;
    moe_status st = check_gather(xq, sorted_slot, T, top_k, M_cap, K);
    if (st != MOE_OK) return st;
    // the token rows' sizes (T rows) are bounded by the gather's T * K < 2^30
    st = check_gmm_mx(xq, xs, ld_xs, w1q, w1s, ld_w1s, group_list, E, M_cap, K, 2 * I);
    if (st != MOE_OK) return st;
    if (M_cap > 0 && (!aq || !as)) return MOE_ERR_NULL;
    if (!aligned(aq, 16) || !aligned(as, 16) || M_cap * ld_as > (int64_t(1) << 40))
        return MOE_ERR_INVALID;
    moegmm::GatherRows g;
    g.slot = sorted_slot;
    g.top_k = top_k;
    g.nslots = T * top_k;
    return from_hip(moegmm::launch_gmm_mx_fwd_swiglu(xq, xs, ld_xs, w1q, w1s, ld_w1s, group_list,
                                                     E, M_cap, K, I, aq, as, ld_as, dev_err,
                                                     static_cast<hipStream_t>(stream), g));
}

}  // extern "C"
