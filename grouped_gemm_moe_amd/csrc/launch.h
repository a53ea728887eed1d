// Internal launchers (host side).  Each enqueues kernels on `stream` and
// returns hipGetLastError(); argument validation happens in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moegmm {

// permute.hip
size_t permute_workspace_bytes(int64_t S, int64_t E);
// The gather writes bf16 rows to x_perm, or, when xq is given, their MX
// quantisation to xq (codes) and xs (scales, row stride ld_xs).
hipError_t launch_permute(const uint16_t* x, const int32_t* ids, int64_t T, int64_t top_k,
                          int64_t H, int64_t E, uint16_t* x_perm, uint8_t* xq, uint8_t* xs,
                          int64_t ld_xs, int32_t* row_id_map, int32_t* sorted_slot,
                          int64_t* tokens_per_expert, void* ws, int32_t* dev_err,
                          hipStream_t stream);

// moe_permute with its histograms in a static device array (no workspace);
// the caller checks permute_workspace_bytes(S, E) <= permute_static_scratch_bytes().
size_t permute_static_scratch_bytes();
hipError_t launch_permute_noalloc(const uint16_t* x, const int32_t* ids, int64_t T, int64_t top_k,
                                  int64_t H, int64_t E, uint16_t* x_perm, int32_t* row_id_map,
                                  int32_t* sorted_slot, int64_t* tokens_per_expert, int32_t* dev_err,
                                  hipStream_t stream);

// gmm.hip
// Compute units of the current device (cached per device; 256 if the query fails).
int num_cus();

// Forward GMM operand rows gathered from token rows: with slot given, x is the
// token matrix [nslots / top_k, K] and row r of the grouped operand is token
// slot[r] / top_k (slot entries in [0, nslots), else zeros and
// MOE_DEVERR_SLOT).  slot == nullptr: x is the grouped operand itself.
struct GatherRows {
    const int32_t* slot = nullptr;
    int64_t top_k = 1;
    int64_t nslots = 0;
};

size_t gmm_workspace_bytes(int64_t E, int64_t M_cap, int64_t K, int64_t N, int op);
hipError_t launch_gmm_fwd(const uint16_t* x, const uint16_t* w, const int64_t* group_list,
                          int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* y, void* ws,
                          int32_t* dev_err, hipStream_t stream, const GatherRows& g = GatherRows{});
hipError_t launch_gmm_bwd_input(const uint16_t* dy, const uint16_t* w, const int64_t* group_list,
                                int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dx,
                                void* ws, int32_t* dev_err, hipStream_t stream);
hipError_t launch_gmm_bwd_weight(const uint16_t* x, const uint16_t* dy, const int64_t* group_list,
                                 int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* dw,
                                 void* ws, int32_t* dev_err, hipStream_t stream);

// dx and dw of one grouped matmul in one persistent launch (queue in ws)
hipError_t launch_gmm_bwd(const uint16_t* x, const uint16_t* dy, const uint16_t* w,
                          const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K, int64_t N,
                          uint16_t* dx, uint16_t* dw, void* ws, int32_t* dev_err, hipStream_t stream);

// the same for the down GMM, its dA tiles turned into dH = swiglu_bwd(dA, h)
hipError_t launch_gmm_bwd_swiglu(const uint16_t* x, const uint16_t* dy, const uint16_t* w,
                                 const uint16_t* h, const int64_t* group_list, int64_t E, int64_t M_cap,
                                 int64_t K, int64_t N, uint16_t* dh, uint16_t* dw, void* ws,
                                 int32_t* dev_err, hipStream_t stream);

hipError_t launch_gmm_fwd_swiglu(const uint16_t* x, const uint16_t* w1, const int64_t* group_list,
                                 int64_t E, int64_t M_cap, int64_t K, int64_t I, uint16_t* a,
                                 uint16_t* h, void* ws, int32_t* dev_err, hipStream_t stream,
                                 const GatherRows& g = GatherRows{});

// Test-only kernel choice for the forward GMMs, from the environment
// variable MOEGMM_FORCE_VARIANT, read at every call: "tile" runs the
// row-tile kernels and "stream" the weight-streaming kernels (where their
// staging fits) whatever the shape; unset or anything else, the library
// chooses by shape.  Lets tests run both kernels on one input.
enum GmmVariant { kVariantAuto = 0, kVariantTile = 1, kVariantStream = 2 };
GmmVariant forced_gmm_variant();

// gmm_stream.hip (decode-shaped forward)
bool gmm_stream_applies(int64_t E, int64_t M_cap, int64_t K);
// y = SwiGLU(h) @ w2[e] in one weight-streaming launch (a = SwiGLU(h) too)
hipError_t launch_stream_swiglu_in(const uint16_t* h, const uint16_t* w2, const int64_t* group_list,
                                   int64_t E, int64_t M_cap, int64_t I, int64_t N, uint16_t* a, uint16_t* y,
                                   int32_t* dev_err, hipStream_t stream);
hipError_t launch_gmm_stream(const uint16_t* x, const uint16_t* w, const int64_t* group_list,
                             int64_t E, int64_t M_cap, int64_t K, int64_t N, uint16_t* y,
                             int32_t* dev_err, hipStream_t stream, const GatherRows& g);
hipError_t launch_gmm_stream_swiglu(const uint16_t* x, const uint16_t* w1,
                                    const int64_t* group_list, int64_t E, int64_t M_cap,
                                    int64_t K, int64_t I, uint16_t* a, uint16_t* h,
                                    int32_t* dev_err, hipStream_t stream, const GatherRows& g);
// The decode layer forward (moe_decode_fwd): the shapes it takes, and its
// gate_up launch, which routes its own rows from ids (moe_permute_index and
// gmm_fwd_gather in one weight-streaming launch: h, the maps and
// tokens_per_expert as those two calls write them).
bool decode_fwd_applies(int64_t T, int64_t top_k, int64_t H, int64_t I, int64_t E);
hipError_t launch_gmm_stream_route(const uint16_t* x, const int32_t* ids, int64_t T, int64_t top_k,
                                   const uint16_t* w1, int64_t E, int64_t K, int64_t N, uint16_t* h,
                                   int32_t* row_id_map, int32_t* sorted_slot, int64_t* tokens_per_expert,
                                   int32_t* dev_err, hipStream_t stream);

// gmm_mx.hip (MXFP8)
hipError_t launch_gmm_mx_fwd(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs, const uint8_t* wq,
                             const uint8_t* ws, int64_t ld_ws, const int64_t* group_list, int64_t E,
                             int64_t M_cap, int64_t K, int64_t N, uint16_t* y, int32_t* dev_err,
                             hipStream_t stream);
hipError_t launch_gmm_mx_fwd_swiglu(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs,
                                    const uint8_t* w1q, const uint8_t* w1s, int64_t ld_w1s,
                                    const int64_t* group_list, int64_t E, int64_t M_cap, int64_t K,
                                    int64_t I, uint8_t* aq, uint8_t* as, int64_t ld_as,
                                    int32_t* dev_err, hipStream_t stream,
                                    const GatherRows& g = GatherRows{});

// GMM1 of moe_decode_fwd_mx: the MX streaming gate_up + SwiGLU + requant
// reading quantised token rows, routing its own rows from ids (h, the maps
// and tokens_per_expert as moe_permute_index + gmm_mx_fwd_swiglu_gather).
hipError_t launch_gmm_mx_stream_route(const uint8_t* xq, const uint8_t* xs, int64_t ld_xs, const int32_t* ids,
                                      int64_t T, int64_t top_k, const uint8_t* w1q, const uint8_t* w1s,
                                      int64_t ld_w1s, int64_t E, int64_t K, int64_t I, uint8_t* aq, uint8_t* as,
                                      int64_t ld_as, int32_t* row_id_map, int32_t* sorted_slot,
                                      int64_t* tokens_per_expert, int32_t* dev_err, hipStream_t stream);

// mx_quant.hip
hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ld_s, uint8_t* q,
                              uint8_t* s, hipStream_t stream);

// elementwise.hip
hipError_t launch_swiglu(const uint16_t* h, const int64_t* group_list, int64_t E, int64_t M_cap,
                         int64_t I, uint16_t* a, hipStream_t stream);
hipError_t launch_swiglu_bwd(const uint16_t* da, const uint16_t* h, const int64_t* group_list,
                             int64_t E, int64_t M_cap, int64_t I, uint16_t* dh,
                             hipStream_t stream);
hipError_t launch_unpermute(const uint16_t* y_perm, const int32_t* row_id_map, const float* probs,
                            int64_t T, int64_t top_k, int64_t H, uint16_t* out, int32_t* dev_err,
                            hipStream_t stream);
hipError_t launch_permute_bwd(const uint16_t* dx_perm, const int32_t* row_id_map, int64_t T,
                              int64_t top_k, int64_t H, uint16_t* dx, int32_t* dev_err,
                              hipStream_t stream);
hipError_t launch_unpermute_bwd(const uint16_t* dout, const uint16_t* y_perm,
                                const int32_t* row_id_map, const float* probs, int64_t T,
                                int64_t top_k, int64_t H, uint16_t* dy_perm, float* dprobs,
                                int32_t* dev_err, hipStream_t stream);

}  // namespace moegmm
