// Chunkwise gated delta rule on the float32 vector units of gfx950 (any supported dtype, head
// dims 32/64/128, chunk 16/32/64).  This is the float32 path (float32 inputs need float32
// products) and the path for shapes the matrix-core kernel does not take.
//
// The chunk algebra is the WY/UT form named in "Gated Attention Architectures", section 3 (the
// DeltaNet WY representation of section 2 extended with per-chunk cumulative decay products).
// Per chunk of C positions with entry state h0 (= S^T, [dk, dv]) and the per-chunk log-decay
// cumsum gc_r = g_1 + ... + g_r:
//     A      = strictly-lower( beta_r exp(gc_r - gc_i) (k_r . k_i) )            [C, C]
//     R      = diag(beta) V - diag(beta exp(gc)) K h0                              [C, dv]
//     Delta  = (I + A)^{-1} R         (forward substitution)
//     O      = diag(exp(gc)) Q h0 + lower-incl( exp(gc_r - gc_i) (q_r . k_i) ) Delta
//     h1     = exp(gc_C) h0 + sum_i exp(gc_C - gc_i) k_i Delta_i^T
// Positions past T in the last chunk enter with k = q = v = 0, g = 0, beta = 0, which leaves
// every result unchanged.  Only differences gc_r - gc_i with r >= i are exponentiated.
//
// Work layout: one 512-thread workgroup per (batch, value head, 32-column tile of dv).  Value
// columns of the state evolve independently, so column tiles are independent chains.  Everything
// for one chunk lives in LDS in float32.
#include "device_common.hpp"
#include "launch.hpp"
#include "simt_chunk.hpp"

namespace gdn {

namespace {

constexpr int SIMT_NT = 512;

// One 512-thread workgroup per (batch, value head, column tile): grid (B * Hv, DV / BV).
template <typename T, int DK, int DV, int BV>
__global__ __launch_bounds__(SIMT_NT) void chunk_simt_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* s0, float* sf, T* __restrict__ o,
    int T_max, int Hqk, int Hv, int grp, int C, float scale, const int* cu, int total)
{
    extern __shared__ float lds[];
    simt_chunk_body<T, DK, DV, BV, true, SIMT_NT>(lds, blockIdx.x, blockIdx.y, q, k, v, g, beta, s0, sf, o, nullptr,
                                                   T_max, Hqk, Hv, grp, C, scale, cu, total);
}

}  // namespace

template <typename T, int DK, int DV>
static hipError_t launch_simt_t(const ChunkArgs& a, hipStream_t st)
{
    constexpr int BV = DV < 32 ? DV : 32;
    using L = SimtLds<DK, BV>;
    auto kern = chunk_simt_kernel<T, DK, DV, BV>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)L::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.B * a.Hv, DV / BV), dim3(SIMT_NT), L::bytes, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.g, a.beta, a.s0, a.sf,
                       (T*)a.o, a.T, a.Hqk, a.Hv, a.Hv / a.Hqk, a.chunk, a.scale, a.cu, a.total);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_simt_dt(const ChunkArgs& a, hipStream_t st)
{
#define GDN_SIMT_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_simt_t<T, DK_, DV_>(a, st);
    GDN_SIMT_CASE(32, 32) GDN_SIMT_CASE(32, 64) GDN_SIMT_CASE(32, 128)
    GDN_SIMT_CASE(64, 32) GDN_SIMT_CASE(64, 64) GDN_SIMT_CASE(64, 128)
    GDN_SIMT_CASE(128, 32) GDN_SIMT_CASE(128, 64) GDN_SIMT_CASE(128, 128)
#undef GDN_SIMT_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_simt(const ChunkArgs& a, hipStream_t st)
{
    if (a.chunk > SIMT_CMAX) return hipErrorInvalidValue;
    return a.dtype_bf16 ? launch_simt_dt<bf16>(a, st) : launch_simt_dt<float>(a, st);
}

// T == 0: the final state is the initial state.
__global__ void state_copy_kernel(const float* __restrict__ s0, float* __restrict__ sf, size_t n)
{
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        sf[e] = s0 ? s0[e] : 0.f;
}

hipError_t launch_state_copy(const float* s0, float* sf, size_t n, hipStream_t st)
{
    if (n == 0 || s0 == sf) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, s0, sf, n);
    return hipGetLastError();
}

// The affine state map of an empty sequence: M = I [chains, dk, dk], N = 0 [chains, dk, dv].
__global__ void identity_map_kernel(float* __restrict__ m, float* __restrict__ n, size_t chains, int dk, int dv)
{
    const size_t nm = chains * dk * dk, nn = chains * dk * dv;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < nm + nn; e += (size_t)gridDim.x * blockDim.x) {
        if (e < nm) {
            const size_t r = e % ((size_t)dk * dk);
            m[e] = r / dk == r % dk ? 1.f : 0.f;
        } else {
            n[e - nm] = 0.f;
        }
    }
}

hipError_t launch_identity_map(float* m, float* n, size_t chains, int dk, int dv, hipStream_t st)
{
    const size_t total = chains * dk * (dk + dv);
    if (total == 0) return hipSuccess;
    size_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(identity_map_kernel, dim3((unsigned)blocks), dim3(256), 0, st, m, n, chains, dk, dv);
    return hipGetLastError();
}

}  // namespace gdn
