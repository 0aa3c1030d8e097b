// The gated RMSNorm of a Gated DeltaNet layer's output, per lane: y = o / sqrt(mean(o^2) + eps)
// * w * silu(z) over one value head ("Architecture Thread I: Gated Attention, DeltaNet, and Hybrid
// Models", section "Modern Architecture Improvements", output normalisation; the SiLU output gate
// of the Gated DeltaNet block in "Gated Attention Architectures").  One head's row is spread over
// an aligned group of lanes, N consecutive channels per lane.  The standalone kernel
// (layer_ops.hip) and the fused epilogue of the chunk kernel (chunk_mfma.hip) both call this, so
// the two give bit-identical results for the same o.
#pragma once

#include "device_common.hpp"

namespace gdn {

// SiLU(x) = x sigmoid(x), with the hardware reciprocal (1 ulp) in place of a full division
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// a lane's value moved across the wave by a DPP pattern (no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the `group` lanes of this lane's head (group a power of two <= 64, aligned).  Within a
// row of 16 lanes the partners come by DPP: lanes 1 and 2 apart inside a quad, then the mirror
// images inside a half row and a row (after the quad steps every lane of a quad holds the quad's
// sum, so pairing mirror images pairs whole quads, then whole half rows); beyond a row by lane
// exchange.  Each step adds two equal-rank partial sums, so every lane of the group ends with
// the same bits.
__device__ __forceinline__ float group_sum(float x, int group)
{
    if (group >= 2) x += dpp_move<0xB1>(x);    // quad_perm [1,0,3,2]
    if (group >= 4) x += dpp_move<0x4E>(x);    // quad_perm [2,3,0,1]
    if (group >= 8) x += dpp_move<0x141>(x);   // row_half_mirror
    if (group >= 16) x += dpp_move<0x140>(x);  // row_mirror
    if (group >= 32) x += __shfl_xor(x, 16, 64);
    if (group >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// every lane of the wave must call this (the sum is a cross-lane butterfly)
template <int N>
__device__ __forceinline__ void gated_norm_lane(const float (&o)[N], const float (&z)[N], const float (&w)[N],
                                                int group, float inv_d, float eps, float (&y)[N])
{
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) ss = fmaf(o[e], o[e], ss);
    const float r = rsqrtf(group_sum(ss, group) * inv_d + eps);
#pragma unroll
    for (int e = 0; e < N; ++e) y[e] = o[e] * r * w[e] * silu(z[e]);
}

}  // namespace gdn
