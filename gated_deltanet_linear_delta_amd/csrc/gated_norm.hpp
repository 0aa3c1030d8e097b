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

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }

// sum over the `group` lanes of this lane's head (group a power of two <= 64, aligned)
__device__ __forceinline__ float group_sum(float x, int group)
{
    for (int s = 1; s < group; s <<= 1) x += __shfl_xor(x, s, 64);
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
