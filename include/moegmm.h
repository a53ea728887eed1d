/*
 * moegmm.h -- C ABI of the routed-expert MoE hot path for AMD MI355X (gfx950).
 *
 * What the calls compute (sources are web pages, cited by title and section):
 *
 *   [GMM]       "NPU Training Operators - GMM": section 算子语义 (operator
 *               semantics) -- the per-expert loop over row ranges taken from
 *               the cumulative sum of group_list, the input table
 *               (x[sum(group_list), hidden], weight[num_experts, hidden, out]),
 *               the worked example with an empty expert, and the two backward
 *               products right after it; section "Qwen3.5 MoE 路径" -- the
 *               chain permute -> histc -> gate_up GMM -> SwiGLU -> down GMM ->
 *               probs-weighted unpermute, and its GMM shape table.
 *   [MegaMoE]   "MegaMoE" (ops-transformer mc2/mega_moe): section 功能说明,
 *               activation formulas (SwiGLU), the A16W16 scenario (Dispatch,
 *               Expert Compute, Token Combine), and the parameter table
 *               (topkIds int32 in [0, experts), topK in [1, 32]).
 *   [PermGrad]  "CANN ops-transformer 算子详解：MoeTokenPermuteWithRoutingMapGrad":
 *               section 3 (size query, then execute with a caller workspace),
 *               section 4.1 (-1 marks an invalid slot), section 4.3 (null and
 *               invalid arguments are reported before any work), section 6.2
 *               (FP32 accumulation over a token's top-k slots, one cast back).
 *   [MX]        "MegaMoE": the A8W8-FP scenario -- tokens gathered per expert
 *               are MX-quantised (groups of 32, FP8 elements, FLOAT8_E8M0
 *               scales), GMM1 dequantises inside the matmul, the activation
 *               output is MX-quantised again for GMM2; its parameter table
 *               (activation scales of shape (rows, CeilDiv(H, 32)), weights
 *               with the hidden size as the last dimension).  The group
 *               quantiser itself follows the OCP Microscaling (MX) v1.0
 *               definition: shared exponent floor(log2(max|v|)) - 8 (clamped
 *               to >= -127; an all-zero group takes -127), E4M3 elements
 *               rounded to nearest even and saturated at +-448.
 *   [MegaBlocks] "03 · grouped GEMM 路径": section 4.2 -- the grouped GEMM
 *               there needs the group sizes on the host, a device-to-host
 *               synchronisation this library avoids: group_list stays on the
 *               device and every kernel builds its own tile schedule from it.
 *
 * Conventions for every call below
 *   - All tensor pointers are DEVICE pointers to row-major, contiguous memory.
 *     bf16 tensors are arrays of uint16_t bit patterns; bf16 pointers must be
 *     16-byte aligned.  Other pointers must be aligned to their element size.
 *   - The caller owns all memory.  The library never allocates device memory
 *     and never synchronises: each call only enqueues kernels on `stream`
 *     (a hipStream_t; NULL means the default stream) and returns.
 *   - Outputs must not alias inputs.
 *   - Host-checkable problems (NULL required pointer, sizes out of range,
 *     misalignment, a workspace smaller than the queried size) return an error
 *     status BEFORE anything is enqueued.
 *   - Data-dependent problems are reported through `dev_err` (nullable): a
 *     device int32 the caller zeroes; kernels OR bits into it
 *     (MOE_DEVERR_*).  Kernels clamp offending values so that they never read
 *     or write out of bounds; outputs are unspecified when a bit is set.  Read
 *     it after synchronising the stream.
 *   - Row counts: `group_list` (a.k.a. tokens_per_expert) is a DEVICE int64
 *     array of per-expert COUNTS n_e; expert e owns rows off_e .. off_e+n_e-1
 *     where off_e = n_0 + ... + n_{e-1}.  An empty expert owns no row and does
 *     not shift later offsets.  R = sum(n_e) must not exceed M_cap; rows at or
 *     beyond R are neither read for results nor written (except as stated).
 *   - Limits: 1 <= E <= 1024; 1 <= top_k <= 32; T*top_k < 2^31;
 *     hidden / intermediate / K / N are positive multiples of 8, at most
 *     2^24 (hidden, intermediate) and 2^21 (the GMM's K and N);
 *     E*K*N, M_cap*K and M_cap*N are at most 2^40.
 */
#ifndef MOEGMM_H
#define MOEGMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,      /* a required pointer is NULL                        */
    MOE_ERR_INVALID = 2,   /* a size, limit or alignment is out of range        */
    MOE_ERR_WORKSPACE = 3, /* ws_bytes is below the size the query returned     */
    MOE_ERR_LAUNCH = 4     /* the HIP runtime rejected a launch                 */
} moe_status;

/* bits OR-ed into *dev_err by the kernels */
#define MOE_DEVERR_EXPERT_ID 1  /* an expert id outside [-1, E)               */
#define MOE_DEVERR_GROUP_LIST 2 /* a negative count, or sum(group_list) > M_cap */
#define MOE_DEVERR_ROW_MAP 4    /* a row_id_map entry outside [-1, T*top_k)   */
#define MOE_DEVERR_SLOT 8       /* a sorted_slot entry outside [0, T*top_k) for
                                   a row below sum(group_list) (gathered GMMs) */

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status s);

/* ABI version of this header; bumped on any signature change. */
int moegmm_abi_version(void);

/* ------------------------------------------------------------------------
 * moe_permute -- histogram + stable permute of token rows by expert.
 * [GMM] "Qwen3.5 MoE 路径": token permute by selected experts, and
 * tokens_per_expert as a histogram of the selected ids; worked example in
 * 算子语义.  [MegaMoE] A16W16 Dispatch: X_e stacks the tokens routed to e in a
 * fixed order and row(i,k) locates token i in it.  [PermGrad] 4.1: id -1
 * marks a slot that takes no part.
 *
 *   x          [T, H] bf16             token rows
 *   topk_ids   [T, top_k] int32        expert of each slot s = t*top_k + k, or -1
 *   x_perm     [T*top_k, H] bf16  OUT  row r = x[sorted_slot[r] / top_k], r < R;
 *                                      rows >= R untouched
 *   row_id_map [T*top_k] int32    OUT  slot -> row, -1 for a masked slot
 *   sorted_slot[T*top_k] int32    OUT  row -> slot for r < R; entries >= R untouched
 *   tokens_per_expert [E] int64   OUT  n_e (this is the group_list of the GMMs)
 *   ws / ws_bytes                      caller workspace, >= moe_permute_workspace_size
 * Rows are grouped by expert in ascending expert order and, inside an expert,
 * in ascending slot order -- so the result is unique and bit-reproducible.
 * Ids outside [-1, E) set MOE_DEVERR_EXPERT_ID and are treated as masked.
 * T == 0 is allowed (tokens_per_expert is zeroed).
 * ---------------------------------------------------------------------- */
size_t moe_permute_workspace_size(int64_t T, int64_t top_k, int64_t E);
moe_status moe_permute(const uint16_t* x, const int32_t* topk_ids, int64_t T, int64_t top_k,
                       int64_t H, int64_t E, uint16_t* x_perm, int32_t* row_id_map,
                       int32_t* sorted_slot, int64_t* tokens_per_expert, void* ws,
                       size_t ws_bytes, int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute_noalloc -- moe_permute with no workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments,
 * outputs, ordering and errors as moe_permute; its scratch (the per-block
 * expert histograms) is a static 1 MiB device array of the library, which
 * each device it runs on holds until the process ends.
 *
 * Limit: moe_permute_workspace_size(T, top_k, E) <= 1 MiB (1048576 bytes),
 * e.g. E = 1024 experts with up to 262144 slots, E = 128 with up to 2M;
 * larger calls return MOE_ERR_WORKSPACE before anything is enqueued.
 * Allocates nothing: no hipMalloc/hipFree; the first call on a device looks
 * up the array's device address (hipGetSymbolAddress) and keeps it.
 * Every call on one device shares that array and leaves its contents behind
 * (each call writes the histograms whole before reading them): calls that
 * may overlap in time on one device -- different streams, or different host
 * threads -- race on it and must not be issued.
 * ---------------------------------------------------------------------- */
moe_status moe_permute_noalloc(const uint16_t* x, const int32_t* topk_ids, int64_t T, int64_t top_k,
                               int64_t H, int64_t E, uint16_t* x_perm, int32_t* row_id_map,
                               int32_t* sorted_slot, int64_t* tokens_per_expert, int32_t* dev_err,
                               void* stream);

/* ------------------------------------------------------------------------
 * moe_permute_index -- moe_permute without the row gather: the histogram,
 * the stable ranks and the maps only, for a forward that reads the token rows
 * through gmm_fwd_gather / gmm_fwd_swiglu_gather instead of a permuted copy.
 * Same citations, ordering, workspace (moe_permute_workspace_size) and
 * errors as moe_permute; row_id_map, sorted_slot and tokens_per_expert come
 * out bit-identical to moe_permute's.  x and x_perm do not exist here.
 * ---------------------------------------------------------------------- */
moe_status moe_permute_index(const int32_t* topk_ids, int64_t T, int64_t top_k, int64_t E,
                             int32_t* row_id_map, int32_t* sorted_slot, int64_t* tokens_per_expert,
                             void* ws, size_t ws_bytes, int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * gmm_fwd -- grouped matmul  y[off_e + i, :] = x[off_e + i, :] @ w[e]  for
 * every expert e and 0 <= i < n_e.   [GMM] 算子语义: the per-expert loop and
 * its input table; [MegaMoE] Expert Compute: H_e = X_e W1[e], Y_e = A_e W2[e].
 *
 *   x [M_cap, K] bf16, w [E, K, N] bf16, group_list [E] int64 (device),
 *   y [M_cap, N] bf16 OUT (rows < R written; rows >= R untouched).
 * bf16 products accumulate in fp32; each output is rounded once (RNE).
 * w[e] of an empty expert is never read.
 * The kernel is chosen by shape: weight streaming when experts own a few
 * rows each (M_cap <= 8E), row tiles otherwise.  For tests only, the
 * environment variable MOEGMM_FORCE_VARIANT = "tile" or "stream", read at
 * every call, forces one of them (streaming where its staging fits,
 * K <= 4096, and M_cap <= 2^16) for gmm_fwd, gmm_fwd_swiglu and the MX
 * forward calls.
 * ---------------------------------------------------------------------- */
/* Workspace bytes of GMM op `op` (MOE_GMM_OP_*).  gmm_bwd needs
 * MOE_GMM_QUEUE_BYTES (1152): its tile queue, counters the kernel increments with atomics.  gmm_bwd_weight
 * needs the same 1152, or, on a tile grid too small to fill the GPU (E * KT *
 * NT tiles of 256 x 256 at most half the CUs) where it splits each expert's
 * row reduction into S chunks, 2048 + tiles * S * 256 KiB: the queue, then
 * the chunks' fp32 partial tiles from byte 2048 on (up to 64 MiB).  The other
 * ops need none (0) and take NULL.  A workspace that is needed must be 16-byte
 * aligned (else MOE_ERR_INVALID), and its first 1152 bytes (the queue)
 * zero-filled before
 * its first use; every call leaves them zero-filled again (the partial tiles
 * are scratch), so one workspace serves any number of calls issued one after
 * another.  Calls that may run at the same time (on different streams) need
 * distinct workspaces.  Too small or NULL: MOE_ERR_WORKSPACE. */
size_t gmm_workspace_size(int64_t E, int64_t M_cap, int64_t K, int64_t N, int op);
#define MOE_GMM_OP_FWD 0
#define MOE_GMM_OP_BWD_INPUT 1
#define MOE_GMM_OP_BWD_WEIGHT 2
#define MOE_GMM_OP_BWD 3 /* gmm_bwd: both gradients in one launch */
#define MOE_GMM_QUEUE_BYTES 1152 /* the zero-filled prefix of a GMM workspace */
moe_status gmm_fwd(const uint16_t* x, const uint16_t* w, const int64_t* group_list, int64_t E,
                   int64_t M_cap, int64_t K, int64_t N, uint16_t* y, void* ws, size_t ws_bytes,
                   int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * gmm_fwd_swiglu -- the gate_up grouped matmul fused with SwiGLU:
 *   [G | U] = x[off_e + i, :] @ w1[e]   (G = first I columns, U = last I)
 *   a[off_e + i, j] = SiLU(G[j]) * U[j],  SiLU(z) = z / (1 + e^-z)
 * computed from the fp32 accumulators and rounded once (RNE); G and U are not
 * rounded in between.  [MegaMoE] Expert Compute (H_e = X_e W1[e], split along
 * its columns into G and U, then the activation) with the clamp unset;
 * [GMM] "Qwen3.5 MoE 路径" (gate_up GMM, then SwiGLU).
 *
 *   x [M_cap, K] bf16, w1 [E, K, 2I] bf16, group_list [E] int64,
 *   a [M_cap, I] bf16 OUT (rows < R written; rows >= R untouched),
 *   h [M_cap, 2I] bf16 OUT or NULL: when given, also gets [G | U] rounded
 *   once, exactly as gmm_fwd would write them (for the SwiGLU backward).
 * Workspace: gmm_workspace_size(E, M_cap, K, 2I, MOE_GMM_OP_FWD).
 * ---------------------------------------------------------------------- */
moe_status gmm_fwd_swiglu(const uint16_t* x, const uint16_t* w1, const int64_t* group_list,
                          int64_t E, int64_t M_cap, int64_t K, int64_t I, uint16_t* a,
                          uint16_t* h, void* ws, size_t ws_bytes, int32_t* dev_err,
                          void* stream);

/* ------------------------------------------------------------------------
 * swiglu_gmm_fwd -- the activation and the down grouped matmul in one call:
 *   a[r, :] = SiLU(G) * U  with G = h[r, :I], U = h[r, I:]   (as swiglu)
 *   y[off_e + i, :] = a[off_e + i, :] @ w2[e]                (as gmm_fwd)
 * [MegaMoE] activation formulas and Expert Compute (A_e W2[e]); [GMM]
 * "Qwen3.5 MoE 路径" (SwiGLU, then the down GMM).  Where experts own a few
 * rows each (the weight-streaming shapes of gmm_fwd) one kernel applies
 * SwiGLU while it stages the rows and also writes a; otherwise swiglu then
 * gmm_fwd.  a and y are bit-identical to those two calls.
 *
 *   h [M_cap, 2I] bf16, w2 [E, I, N] bf16, group_list [E] int64,
 *   a [M_cap, I] bf16 OUT, y [M_cap, N] bf16 OUT (rows >= R untouched).
 * a, y and h must not overlap.  Limits as gmm_fwd with K = I.
 * ---------------------------------------------------------------------- */
moe_status swiglu_gmm_fwd(const uint16_t* h, const uint16_t* w2, const int64_t* group_list, int64_t E,
                          int64_t M_cap, int64_t I, int64_t N, uint16_t* a, uint16_t* y, int32_t* dev_err,
                          void* stream);

/* ------------------------------------------------------------------------
 * gmm_fwd_gather / gmm_fwd_swiglu_gather -- gmm_fwd / gmm_fwd_swiglu whose
 * grouped operand is read straight from the token rows instead of from a
 * permuted copy: grouped row r is x[sorted_slot[r] / top_k].  The dispatch
 * (token rows stacked per expert) is fused into the first matmul's operand
 * loads.  [MegaMoE] 功能说明 (dispatch, the first linear layer, activation,
 * second linear layer and combine as one operator) and A16W16 Dispatch (X_e
 * stacks the rows x_i of the tokens routed to expert e); the product itself
 * is gmm_fwd's ([GMM] 算子语义).
 *
 *   x           [T, K] bf16       token rows (moe_permute's x)
 *   sorted_slot [M_cap] int32     row -> slot, from moe_permute or
 *                                 moe_permute_index over the same ids
 *   T, top_k                      as given to the permute; M_cap <= T*top_k
 *   w, group_list, E, K, N, y / w1, I, a, h, ws: as gmm_fwd / gmm_fwd_swiglu.
 * Outputs are bit-identical to gmm_fwd(_swiglu) on moe_permute's x_perm.
 * Entries of sorted_slot for rows r < sum(group_list) must lie in
 * [0, T*top_k); others read a zero row and set MOE_DEVERR_SLOT.  Rows at or
 * past sum(group_list) are not read.  Limit: T*K < 2^30 (x spans less than
 * 2 GiB), else MOE_ERR_INVALID.
 * ---------------------------------------------------------------------- */
moe_status gmm_fwd_gather(const uint16_t* x, const int32_t* sorted_slot, int64_t T, int64_t top_k,
                          const uint16_t* w, const int64_t* group_list, int64_t E, int64_t M_cap,
                          int64_t K, int64_t N, uint16_t* y, void* ws, size_t ws_bytes,
                          int32_t* dev_err, void* stream);
moe_status gmm_fwd_swiglu_gather(const uint16_t* x, const int32_t* sorted_slot, int64_t T,
                                 int64_t top_k, const uint16_t* w1, const int64_t* group_list,
                                 int64_t E, int64_t M_cap, int64_t K, int64_t I, uint16_t* a,
                                 uint16_t* h, void* ws, size_t ws_bytes, int32_t* dev_err,
                                 void* stream);

/* ------------------------------------------------------------------------
 * gmm_bwd_input -- dx[off_e + i, :] = dy[off_e + i, :] @ w[e]^T.
 * [GMM] 算子语义, backward: the input gradient is the output gradient times
 * the transposed weight, over the same group boundaries.
 *
 *   dy [M_cap, N] bf16, w [E, K, N] bf16, group_list [E] int64,
 *   dx [M_cap, K] bf16 OUT (rows < R written; rows >= R untouched).
 * ---------------------------------------------------------------------- */
moe_status gmm_bwd_input(const uint16_t* dy, const uint16_t* w, const int64_t* group_list,
                         int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dx, void* ws,
                         size_t ws_bytes, int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * gmm_bwd_weight -- dw[e] = x[rows_e]^T @ dy[rows_e]   (sum over the n_e rows).
 * [GMM] 算子语义, backward: the weight gradient of each expert is its input
 * rows transposed times its output-gradient rows.
 *
 *   x [M_cap, K] bf16, dy [M_cap, N] bf16, group_list [E] int64,
 *   dw [E, K, N] bf16 OUT -- every expert written; exact zeros for n_e == 0.
 * The reduction order of every output is fixed by the shape, so the result
 * is bit-reproducible whatever order the tiles run in.  Where the tile grid
 * cannot fill the GPU the rows of each expert are reduced in S chunks (S from
 * the shape and the device's CU count, chunks of at least 256 rows) whose
 * fp32 partials are then
 * added in chunk order; elsewhere each output is one fp32 sum over the rows.
 * Workspace: gmm_workspace_size(E, M_cap, K, N, MOE_GMM_OP_BWD_WEIGHT) bytes,
 * its first 1152 bytes zero-filled before the first call (left so by every
 * call).
 * ---------------------------------------------------------------------- */
moe_status gmm_bwd_weight(const uint16_t* x, const uint16_t* dy, const int64_t* group_list,
                          int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dw, void* ws,
                          size_t ws_bytes, int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * gmm_bwd -- gmm_bwd_input and gmm_bwd_weight of one grouped matmul in one
 * launch:  dx[off_e + i, :] = dy[off_e + i, :] @ w[e]^T  and
 *          dw[e] = x[rows_e]^T @ dy[rows_e].
 * [GMM] 算子语义, backward (both gradients over the same group boundaries).
 * Every output is bit-identical to what the two separate calls write
 * (gmm_bwd_weight where it does not split the row reduction: this call
 * never splits it); one launch lets the short weight-gradient tiles fill the CUs the input
 * gradient's last round of tiles leaves idle.
 *
 *   x [M_cap, K] bf16, dy [M_cap, N] bf16, w [E, K, N] bf16, group_list [E],
 *   dx [M_cap, K] bf16 OUT (rows < R written; rows >= R untouched),
 *   dw [E, K, N] bf16 OUT (every expert; exact zeros for n_e == 0).
 * dx and dw must not overlap each other or any input (MOE_ERR_INVALID):
 * both are written while the inputs are still being read.
 * Workspace: gmm_workspace_size(E, M_cap, K, N, MOE_GMM_OP_BWD) bytes,
 * zero-filled before the first call (left zero-filled by every call).
 * ---------------------------------------------------------------------- */
moe_status gmm_bwd(const uint16_t* x, const uint16_t* dy, const uint16_t* w, const int64_t* group_list,
                   int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dx, uint16_t* dw,
                   void* ws, size_t ws_bytes, int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * gmm_bwd_swiglu -- gmm_bwd of the down GMM with the SwiGLU backward applied
 * to its input gradient in the same launch:
 *   dA = dy[rows_e] @ w[e]^T (fp32, never rounded),
 *   dh[:, j] = dA * U * s * (1 + G * (1 - s)),  dh[:, K + j] = dA * G * s,
 *   with G = h[:, j], U = h[:, K + j], s = 1 / (1 + e^-G),
 *   dw[e] = x[rows_e]^T @ dy[rows_e].
 * [GMM] 算子语义, backward of the down GMM; the SwiGLU derivative is derived
 * (not on the pages): d SiLU(z)/dz = s + z s (1 - s).  dh is what
 * swiglu_bwd(gmm_bwd_input(dy, w), h) writes, except that dA is not rounded
 * to bf16 in between; dw is bit-identical to gmm_bwd_weight.
 *
 *   x [M_cap, K] bf16 (the activation A), dy [M_cap, N] bf16, w [E, K, N]
 *   bf16 (W2), h [M_cap, 2K] bf16 (H = [G | U]), group_list [E] int64,
 *   dh [M_cap, 2K] bf16 OUT (rows < R written; rows >= R untouched), may be
 *   h itself (in place: each output is written after its G and U are read),
 *   dw [E, K, N] bf16 OUT.
 * Otherwise dh and dw must not overlap each other or any input
 * (MOE_ERR_INVALID).  Workspace as gmm_bwd (MOE_GMM_OP_BWD).
 * ---------------------------------------------------------------------- */
moe_status gmm_bwd_swiglu(const uint16_t* x, const uint16_t* dy, const uint16_t* w, const uint16_t* h,
                          const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K, int64_t N,
                          uint16_t* dh, uint16_t* dw, void* ws, size_t ws_bytes, int32_t* dev_err,
                          void* stream);

/* ------------------------------------------------------------------------
 * swiglu -- a[r, j] = SiLU(h[r, j]) * h[r, I + j],  SiLU(z) = z / (1 + e^-z),
 * for rows r < R = sum(group_list) (clamped to M_cap).  gate = first I
 * columns, up = last I columns; no clamp.  [MegaMoE] activation formulas,
 * swiglu with the clamp unset; [GMM] "Qwen3.5 MoE 路径": one gate_up GMM then
 * a SwiGLU split.
 *
 *   h [M_cap, 2I] bf16, a [M_cap, I] bf16 OUT (rows >= R untouched).
 * fp32 arithmetic, one RNE rounding per output.
 * ---------------------------------------------------------------------- */
moe_status swiglu(const uint16_t* h, const int64_t* group_list, int64_t E, int64_t M_cap,
                  int64_t I, uint16_t* a, void* stream);

/* ------------------------------------------------------------------------
 * swiglu_bwd -- derivative of swiglu (derived by calculus; not on the pages):
 *   s = sigma(G);  dG = dA * U * s * (1 + G (1 - s));  dU = dA * G * s;
 *   dh = [dG | dU]  for rows r < R.
 *
 *   da [M_cap, I] bf16, h [M_cap, 2I] bf16, dh [M_cap, 2I] bf16 OUT.
 * dh may be h (in place, the exception to "outputs must not alias inputs"):
 * the memory-optimised backward writes dH over the dead H ([MegaBlocks]
 * section 4, memory-optimised backward: reuse buffers that are dead).
 * ---------------------------------------------------------------------- */
moe_status swiglu_bwd(const uint16_t* da, const uint16_t* h, const int64_t* group_list, int64_t E,
                      int64_t M_cap, int64_t I, uint16_t* dh, void* stream);

/* ------------------------------------------------------------------------
 * moe_unpermute -- probs-weighted combine back to token order:
 *   out[t, :] = sum over k = 0..top_k-1 with row_id_map[t*top_k+k] >= 0 of
 *               probs[t, k] * y_perm[row_id_map[t*top_k + k], :]
 * accumulated in fp32 in ascending k, rounded once (RNE); a token with no
 * valid slot gets zeros.  [MegaMoE] Token Combine; [PermGrad] 6.2.
 *
 *   y_perm [T*top_k, H] bf16, row_id_map [T*top_k] int32, probs [T, top_k] fp32,
 *   out [T, H] bf16 OUT.
 * Entries of row_id_map outside [-1, T*top_k) set MOE_DEVERR_ROW_MAP and are
 * skipped.  Deterministic: no atomics.
 * ---------------------------------------------------------------------- */
moe_status moe_unpermute(const uint16_t* y_perm, const int32_t* row_id_map, const float* probs,
                         int64_t T, int64_t top_k, int64_t H, uint16_t* out, int32_t* dev_err,
                         void* stream);

/* ------------------------------------------------------------------------
 * moe_decode_fwd -- the whole routed-expert layer forward for decode-shaped
 * calls (a few rows per expert), in three launches: the gate_up GMM routes
 * its own rows (every workgroup of the weight-streaming kernel counts the
 * expert histogram of topk_ids and ranks its own expert's slots, so no
 * permute launch runs first: moe_permute_index and gmm_fwd_gather in one),
 * then swiglu_gmm_fwd (the down GMM on SwiGLU(h)) and moe_unpermute.
 * [MegaMoE] 功能说明 (dispatch fused into the first linear layer) and Token
 * Combine; [GMM] "Qwen3.5 MoE 路径" (permute, gate_up GMM, SwiGLU, down GMM,
 * unpermute).
 *
 *   x [T, H] bf16, topk_ids [T, top_k] int32 (or -1), probs [T, top_k] fp32,
 *   w1 [E, H, 2I] bf16, w2 [E, I, H] bf16,
 *   out [T, H] bf16 OUT             the layer output, as moe_unpermute
 *   row_id_map, sorted_slot [T*top_k] int32, tokens_per_expert [E] int64 OUT
 *                                   as moe_permute_index
 *   h [T*top_k, 2I], a [T*top_k, I], y_perm [T*top_k, H] bf16 OUT
 *                                   as gmm_fwd_gather / swiglu_gmm_fwd
 *                                   (rows >= R untouched)
 * Every output is bit-identical to the chain moe_permute_index ->
 * gmm_fwd_gather -> swiglu_gmm_fwd -> moe_unpermute on the same inputs.
 * Shapes: T*top_k <= 8*E and <= 16384, H <= 4096, I <= 4096 (else
 * MOE_ERR_INVALID: use that chain).  Outputs must not overlap each other or
 * the inputs.  Ids outside [-1, E) set MOE_DEVERR_EXPERT_ID and are masked.
 * No workspace.
 * ---------------------------------------------------------------------- */
/* ------------------------------------------------------------------------
 * moe_decode_fwd_mx -- the A8W8-FP (MXFP8) decode layer forward with the
 * routing fused into GMM1, as moe_decode_fwd does for bf16: GMM1 + SwiGLU +
 * requantisation reads the quantised token rows (mx_quantize of x) and
 * routes its own rows, then gmm_mx_fwd (GMM2) and moe_unpermute.  [MegaMoE]
 * A8W8-FP (GMM1 -> activation -> requantisation -> GMM2) and 功能说明
 * (dispatch fused into the first linear layer).
 *
 *   xq [T, H] fp8 codes, xs [T, ld_xs] E8M0 scales: mx_quantize(x)
 *   topk_ids, probs [T, top_k]; w1q/w1s, w2q/w2s as gmm_mx_fwd_swiglu / gmm_mx_fwd
 *   out [T, H] bf16, row_id_map, sorted_slot [T*top_k], tokens_per_expert [E],
 *   aq [T*top_k, I] + as [T*top_k, ld_as], y_perm [T*top_k, H] bf16 OUT
 * Every output is bit-identical to moe_permute_index ->
 * gmm_mx_fwd_swiglu_gather -> gmm_mx_fwd -> moe_unpermute on the same
 * inputs.  Shapes as moe_decode_fwd (else MOE_ERR_INVALID), limits as the MX
 * calls; I % 32 == 0.  No workspace.
 * ---------------------------------------------------------------------- */
moe_status moe_decode_fwd_mx(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs, const int32_t* topk_ids,
                             const float* probs, const uint8_t* w1q, const uint8_t* w1s, int64_t ld_w1s,
                             const uint8_t* w2q, const uint8_t* w2s, int64_t ld_w2s, int64_t T, int64_t top_k,
                             int64_t H, int64_t I, int64_t E, uint16_t* out, int32_t* row_id_map,
                             int32_t* sorted_slot, int64_t* tokens_per_expert, uint8_t* aq, uint8_t* as,
                             int64_t ld_as, uint16_t* y_perm, int32_t* dev_err, void* stream);

moe_status moe_decode_fwd(const uint16_t* x, const int32_t* topk_ids, const float* probs,
                          const uint16_t* w1, const uint16_t* w2, int64_t T, int64_t top_k, int64_t H,
                          int64_t I, int64_t E, uint16_t* out, int32_t* row_id_map, int32_t* sorted_slot,
                          int64_t* tokens_per_expert, uint16_t* h, uint16_t* a, uint16_t* y_perm,
                          int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * moe_unpermute_bwd -- gradients of moe_unpermute with respect to y_perm and
 * probs, given dout = d(loss)/d(out):
 *   dy_perm[row(t,k), :] = probs[t, k] * dout[t, :]        (rounded once, RNE)
 *   dprobs[t, k]         = sum_h dout[t, h] * y_perm[row(t,k), h]   (fp32)
 * with row(t,k) = row_id_map[t*top_k + k]; a masked slot (-1) gets
 * dprobs = 0 and writes no row.  [MegaMoE] Token Combine, differentiated:
 * the combine is linear in each of y_perm and probs.
 *
 *   dout [T, H] bf16, y_perm [T*top_k, H] bf16, row_id_map [T*top_k] int32,
 *   probs [T, top_k] fp32; dy_perm [T*top_k, H] bf16 OUT (the rows that some
 *   valid slot points at are written, the others untouched), dprobs
 *   [T, top_k] fp32 OUT.
 * Entries of row_id_map outside [-1, T*top_k) set MOE_DEVERR_ROW_MAP and are
 * skipped.  Deterministic: every sum runs in a fixed order, no atomics.
 * ---------------------------------------------------------------------- */
moe_status moe_unpermute_bwd(const uint16_t* dout, const uint16_t* y_perm,
                             const int32_t* row_id_map, const float* probs, int64_t T,
                             int64_t top_k, int64_t H, uint16_t* dy_perm, float* dprobs,
                             int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute_bwd -- the token gradient of moe_permute:
 *   dx[t, :] = sum over k = 0..top_k-1 with row_id_map[t*top_k+k] >= 0 of
 *              dx_perm[row_id_map[t*top_k + k], :]
 * accumulated in fp32 in ascending k, rounded once (RNE); a token with no
 * valid slot gets zeros.  [PermGrad] section 2.3 (each permuted row's
 * gradient is added back onto the token it was copied from) and section 6.2
 * (a token walks its top-k slots, skips -1, accumulates in FP32, casts back
 * once).
 *
 *   dx_perm [T*top_k, H] bf16, row_id_map [T*top_k] int32 (as written by
 *   moe_permute), dx [T, H] bf16 OUT.
 * Entries of row_id_map outside [-1, T*top_k) set MOE_DEVERR_ROW_MAP and are
 * skipped.  Deterministic: no atomics.
 * ---------------------------------------------------------------------- */
moe_status moe_permute_bwd(const uint16_t* dx_perm, const int32_t* row_id_map, int64_t T,
                           int64_t top_k, int64_t H, uint16_t* dx, int32_t* dev_err,
                           void* stream);

/* ------------------------------------------------------------------------
 * MXFP8 (A8W8-FP) calls.  [MX]
 *
 * An MX tensor is a pair: codes [rows, K] uint8 (E4M3FN bit patterns,
 * row-major) and scales [rows, ld_s] uint8 (E8M0: byte b means 2^(b-127)),
 * one scale per group of 32 consecutive codes of a row.  The scale row
 * stride ld_s is at least ceil(K/32) and a multiple of 16; scale bytes past
 * ceil(K/32) are padding, never read as scales and never written.  K must be
 * a multiple of 32.  Codes and scale pointers must be 16-byte aligned.
 * Weights are stored reduction-contiguous: w[e] is [N, K] (N output
 * columns), so an expert's weight is an MX tensor of N rows.  One expert's
 * codes must hold fewer than 2^31 - 2^16 bytes (N * K <= 0x7FFF0000; N = 2I
 * for gmm_mx_fwd_swiglu): the kernels address them with 31-bit offsets from
 * the expert's base.  Larger experts return MOE_ERR_INVALID.
 * ---------------------------------------------------------------------- */

/* ------------------------------------------------------------------------
 * mx_quantize -- Q_MX of each row of a bf16 matrix:
 *   x [rows, K] bf16; q [rows, K] codes OUT, s [rows, ld_s] scales OUT.
 * Exact: the decisions depend only on the bf16 inputs.  Used for
 * activations and to prepare MXFP8 weights ([E*N, K] rows).
 * ---------------------------------------------------------------------- */
moe_status mx_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ld_s, uint8_t* q,
                       uint8_t* s, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute_mx -- moe_permute whose gather writes Q_MX of each token row:
 * the same row_id_map / sorted_slot / tokens_per_expert, and
 *   xq [T*top_k, H] codes OUT, xs [T*top_k, ld_xs] scales OUT
 * (row r of (xq, xs) = Q_MX(x[sorted_slot[r] / top_k, :])).  [MX] the
 * tokens gathered per expert are quantised; quantising a row before or after
 * the gather gives the same bytes, so each token is quantised once.
 * H must be a multiple of 32.  Workspace as for moe_permute.
 * ---------------------------------------------------------------------- */
moe_status moe_permute_mx(const uint16_t* x, const int32_t* topk_ids, int64_t T, int64_t top_k,
                          int64_t H, int64_t E, uint8_t* xq, uint8_t* xs, int64_t ld_xs,
                          int32_t* row_id_map, int32_t* sorted_slot, int64_t* tokens_per_expert,
                          void* ws, size_t ws_bytes, int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * gmm_mx_fwd -- MX grouped matmul:
 *   y[rows_e, :] = DQ(xq, xs)[rows_e, :] @ DQ(wq[e], ws[e])^T
 * over the row ranges of group_list ([GMM] 算子语义 loop; [MX] GMM2, with
 * dequantisation inside the matmul).  fp32 accumulation of the exactly
 * scaled fp8 products; y rounded once to bf16 (RNE).
 *
 *   xq [M_cap, K] codes, xs [M_cap, ld_xs] scales;
 *   wq [E, N, K] codes, ws [E, N, ld_ws] scales;
 *   y [M_cap, N] bf16 OUT (rows >= R untouched).
 * Limits as for gmm_fwd, plus K % 32 == 0 and N * K <= 0x7FFF0000.
 * ---------------------------------------------------------------------- */
moe_status gmm_mx_fwd(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs, const uint8_t* wq,
                      const uint8_t* ws, int64_t ld_ws, const int64_t* group_list, int64_t E,
                      int64_t M_cap, int64_t K, int64_t N, uint16_t* y, int32_t* dev_err,
                      void* stream);

/* ------------------------------------------------------------------------
 * gmm_mx_fwd_swiglu -- GMM1 of the A8W8-FP block with the activation and the
 * requantisation fused:
 *   [G | U] = DQ(xq, xs)[rows_e, :] @ DQ(w1q[e], w1s[e])^T   (fp32)
 *   A = SiLU(G) * U                                          (fp32)
 *   (aq, as) = Q_MX(A)  over groups of 32 columns of A
 * w1[e] holds the I gate rows first, then the I up rows.  The scale decision
 * is taken on the fp32 A.  [MX]; [MegaMoE] activation formulas (swiglu).
 *
 *   xq [M_cap, K], xs [M_cap, ld_xs]; w1q [E, 2I, K], w1s [E, 2I, ld_w1s];
 *   aq [M_cap, I] codes OUT, as [M_cap, ld_as] scales OUT (rows >= R and
 *   scale padding untouched).
 * Limits as for gmm_fwd_swiglu, plus K % 32 == 0, I % 32 == 0 and
 * 2I * K <= 0x7FFF0000.
 * ---------------------------------------------------------------------- */
moe_status gmm_mx_fwd_swiglu(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs,
                             const uint8_t* w1q, const uint8_t* w1s, int64_t ld_w1s,
                             const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K,
                             int64_t I, uint8_t* aq, uint8_t* as, int64_t ld_as,
                             int32_t* dev_err, void* stream);

/* ------------------------------------------------------------------------
 * gmm_mx_fwd_swiglu_gather -- gmm_mx_fwd_swiglu whose grouped operand rows
 * are read from token rows instead of a permuted copy: grouped row r is row
 * sorted_slot[r] / top_k of (xq, xs), the MX quantisation of the T token rows
 * (mx_quantize of x).  Q_MX works row by row, so these are the bytes that
 * moe_permute_mx would have written for row r, and the outputs are
 * bit-identical to gmm_mx_fwd_swiglu on them.  [MX] (tokens gathered per
 * expert are MX-quantised); [MegaMoE] 功能说明 (dispatch fused with the
 * expert computation), as gmm_fwd_gather.
 *
 *   xq [T, K] codes, xs [T, ld_xs] scales; sorted_slot [M_cap] int32 from
 *   moe_permute_index (or moe_permute) over the same ids; M_cap <= T*top_k;
 *   everything else as gmm_mx_fwd_swiglu.
 * Bad sorted_slot entries and limits as gmm_fwd_gather (T*K < 2^30).
 * ---------------------------------------------------------------------- */
moe_status gmm_mx_fwd_swiglu_gather(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs,
                                    const int32_t* sorted_slot, int64_t T, int64_t top_k,
                                    const uint8_t* w1q, const uint8_t* w1s, int64_t ld_w1s,
                                    const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K,
                                    int64_t I, uint8_t* aq, uint8_t* as, int64_t ld_as,
                                    int32_t* dev_err, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEGMM_H */
