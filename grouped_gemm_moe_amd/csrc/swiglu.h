// SiLU(G) * U of 8 bf16 pairs, rounded once to bf16 (RNE) -- the activation
// between the two GMMs ("MegaMoE", activation formulas: swiglu).  Shared by
// the swiglu kernel and the weight-streaming down GMM that applies it while
// staging its rows, so that both give the same bits.
#pragma once

#include "common.h"

namespace moegmm {

MOE_DEVICE u32x4_t swiglu8(u32x4_t g, u32x4_t u) {
    u32x4_t o;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float g0 = bf16_lo(g[d]), g1 = bf16_hi(g[d]);
        const float u0 = bf16_lo(u[d]), u1 = bf16_hi(u[d]);
        o[d] = pack_bf16x2(g0 * silu_sigmoid(g0) * u0, g1 * silu_sigmoid(g1) * u1);
    }
    return o;
}

}  // namespace moegmm
