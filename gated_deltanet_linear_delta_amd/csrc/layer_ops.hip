// The steps on either side of the gated delta rule in a Gated DeltaNet layer, as two
// memory-bound gfx950 kernels ("Architecture Thread I: Gated Attention, DeltaNet, and Hybrid
// Models", section "Modern Architecture Improvements": query/key go through a short causal
// convolution, SiLU and L2 normalisation, values through the convolution and SiLU, and the output
// is normalised with RMSNorm before the output projection; the output gate multiplies by SiLU of
// a gate projection as in the Gated DeltaNet block of "Gated Attention Architectures" and the
// gated RMSNorm named in "The Transformer Isn't Alone Anymore").
//
// Both stream the token rows: a lane owns 16 bytes of channels (8 bf16 or 4 float32), a wave
// 64 such runs (512 bf16 channels: four 128-wide heads) of one tensor, and neighbouring waves take
// neighbouring channel blocks of the same tokens, so each load instruction reads 1 KB of one row
// and a workgroup reads whole rows.  The per-head reductions (L2 norm, RMS) are butterfly sums
// over the head's group of d / 8 (or d / 4) lanes.  Each element is read and written once; the
// roofline is HBM.
//
// * qkv_prologue_kernel: per (batch row, channel block, run of PTT tokens): loads the run and the
//   W - 1 tokens before it up front (before token 0: the caller's conv state), then per token
//   forms the depthwise causal convolution, SiLU and, for q and k, the L2 norm; the run holding
//   the last token also writes the conv state the next call continues from (the last W - 1
//   inputs).
// * gated_rmsnorm_kernel: per (batch row, channel block, run of RTT tokens):
//   y = o / sqrt(mean(o^2) + eps) * w * silu(z) over each head's dv channels.
#include <stdint.h>

#include "device_common.hpp"
#include "gated_norm.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int PTT = 16;   // tokens per wave, prologue
constexpr int RTT = 8;    // tokens per wave, gated RMSNorm

// 16 bytes of a row as N floats (N = 8 for bf16, 4 for float32)
template <typename T>
struct Vec;
template <>
struct Vec<bf16> {
    static constexpr int N = 8;
    typedef bf16x8 raw;
    static __device__ __forceinline__ void get(raw r, float (&x)[N])
    {
#pragma unroll
        for (int e = 0; e < N; ++e) x[e] = (float)r[e];
    }
    static __device__ __forceinline__ raw put(const float (&x)[N])
    {
        raw r;
#pragma unroll
        for (int e = 0; e < N; ++e) r[e] = (bf16)x[e];
        return r;
    }
};
template <>
struct Vec<float> {
    static constexpr int N = 4;
    typedef floatx4 raw;
    static __device__ __forceinline__ void get(raw r, float (&x)[N])
    {
#pragma unroll
        for (int e = 0; e < N; ++e) x[e] = r[e];
    }
    static __device__ __forceinline__ raw put(const float (&x)[N]) { return raw{x[0], x[1], x[2], x[3]}; }
};

template <typename T, int W>
__global__ __launch_bounds__(256) void qkv_prologue_kernel(const T* __restrict__ q_in, const T* __restrict__ k_in,
                                                           const T* __restrict__ v_in, const float* __restrict__ wq,
                                                           const float* __restrict__ wk, const float* __restrict__ wv,
                                                           const float* st_in, float* st_out, T* __restrict__ q,
                                                           T* __restrict__ k, T* __restrict__ v, int T_len, int Hqk,
                                                           int Hv, int dk, int dv, float eps, int nwaves)
{
    using V = Vec<T>;
    constexpr int N = V::N;
    constexpr int CB = 64 * N;             // channels per wave
    constexpr int NW = PTT + W - 1;        // tokens of the window
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= nwaves) return;
    const int lane = threadIdx.x & 63;
    const int cq = Hqk * dk, cv = Hv * dv;
    const int nbq = (cq + CB - 1) / CB, nbv = (cv + CB - 1) / CB, nb = 2 * nbq + nbv;
    const int nrun = (T_len + PTT - 1) / PTT;
    const int blk = gw % nb;
    const int run = (gw / nb) % nrun;
    const int b = gw / nb / nrun;
    // which tensor, its channel count and head dim, and this lane's first channel in it
    const int which = blk < nbq ? 0 : blk < 2 * nbq ? 1 : 2;
    const int cn = which == 2 ? cv : cq;
    const int d = which == 2 ? dv : dk;
    const int c = (blk - (which == 2 ? 2 * nbq : which * nbq)) * CB + lane * N;
    const bool act = c < cn;
    const int cc = act ? c : 0;
    const T* x_in = (which == 0 ? q_in : which == 1 ? k_in : v_in) + (size_t)b * T_len * cn + cc;
    T* y = (which == 0 ? q : which == 1 ? k : v) + (size_t)b * T_len * cn + cc;
    const float* wt = (which == 0 ? wq : which == 1 ? wk : wv) + (size_t)cc * W;
    const int Ctot = 2 * cq + cv;
    const int cs = (which == 0 ? 0 : which == 1 ? cq : 2 * cq) + cc;   // channel in the conv state
    const int t0 = run * PTT;

    float wts[N][W];
#pragma unroll
    for (int e = 0; e < N; ++e)
#pragma unroll
        for (int j = 0; j < W; ++j) wts[e][j] = wt[e * W + j];
    // the run's inputs, raw: tokens t0 - (W - 1) .. t0 + PTT - 1 (those inside the sequence)
    // (token indexes clamped into the sequence: the clamped copies are never used or stored)
    typename V::raw raw[NW];
#pragma unroll
    for (int s = 0; s < NW; ++s) {
        const int t = min(max(t0 - (W - 1) + s, 0), T_len - 1);
        raw[s] = *reinterpret_cast<const typename V::raw*>(x_in + (size_t)t * cn);
    }
    // sliding window win[j] = x[t - (W - 1) + j] in float32; before token 0 from the conv state
    float win[W][N];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int t = t0 - (W - 1) + j;
        if (t >= 0) {
            V::get(raw[j], win[j]);
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e)
                win[j][e] = st_in ? st_in[((size_t)b * Ctot + cs + e) * (W - 1) + (W - 1) + t] : 0.f;
        }
    }
    const bool l2 = which < 2;
    const int group = d / N;   // lanes per head
#pragma unroll
    for (int s = 0; s < PTT; ++s) {
        const int t = t0 + s;
        if (s > 0) {
#pragma unroll
            for (int j = 0; j < W - 1; ++j)
#pragma unroll
                for (int e = 0; e < N; ++e) win[j][e] = win[j + 1][e];
        }
        V::get(raw[s + W - 1], win[W - 1]);
        float yv[N];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < W; ++j) a = fmaf(wts[e][j], win[j][e], a);
            yv[e] = silu(a);
            ss = fmaf(yv[e], yv[e], ss);
        }
        if (l2) {
            const float r = rsqrtf(group_sum(ss, group) + eps);
#pragma unroll
            for (int e = 0; e < N; ++e) yv[e] *= r;
        }
        if (act && t < T_len) *reinterpret_cast<typename V::raw*>(y + (size_t)t * cn) = V::put(yv);
        // after the last token the window holds x[T - W .. T - 1]: the conv state to continue from
        if (t == T_len - 1 && st_out && act) {
#pragma unroll
            for (int e = 0; e < N; ++e)
#pragma unroll
                for (int j = 0; j < W - 1; ++j) st_out[((size_t)b * Ctot + cs + e) * (W - 1) + j] = win[j + 1][e];
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const T* o, const T* z, const float* __restrict__ w,
                                                            int w_head_stride, T* y, int T_len, int Hv, int dv,
                                                            float eps, int nwaves)
{
    using V = Vec<T>;
    constexpr int N = V::N;
    constexpr int CB = 64 * N;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= nwaves) return;
    const int lane = threadIdx.x & 63;
    const int cn = Hv * dv;
    const int nb = (cn + CB - 1) / CB;
    const int nrun = (T_len + RTT - 1) / RTT;
    const int blk = gw % nb;
    const int run = (gw / nb) % nrun;
    const int b = gw / nb / nrun;
    const int c = blk * CB + lane * N;
    const bool act = c < cn;
    const int cc = act ? c : 0;
    const int h = cc / dv, ch = cc % dv;   // head and its first channel
    const int t0 = run * RTT;
    const int nt = min(RTT, T_len - t0);
    const size_t base = ((size_t)b * T_len + t0) * cn + cc;
    float wc[N];
    {
        const float* wp = w + (size_t)h * w_head_stride + ch;
#pragma unroll
        for (int e = 0; e < N; ++e) wc[e] = wp[e];
    }
    // o and z of the whole run up front, then one token after another
    // (past the end of the sequence the last token is read again and not stored)
    typename V::raw ro[RTT], rz[RTT];
#pragma unroll
    for (int s = 0; s < RTT; ++s) {
        const size_t off = base + (size_t)min(s, nt - 1) * cn;
        ro[s] = *reinterpret_cast<const typename V::raw*>(o + off);
        rz[s] = *reinterpret_cast<const typename V::raw*>(z + off);
    }
    const int group = dv / N;
    const float inv_d = 1.f / (float)dv;
#pragma unroll
    for (int s = 0; s < RTT; ++s) {
        float ov[N], zv[N], yv[N];
        V::get(ro[s], ov);
        V::get(rz[s], zv);
        gated_norm_lane<N>(ov, zv, wc, group, inv_d, eps, yv);
        if (act && s < nt) *reinterpret_cast<typename V::raw*>(y + base + (size_t)s * cn) = V::put(yv);
    }
}

template <typename T>
hipError_t launch_prologue_t(const PrologueArgs& a, hipStream_t st)
{
    constexpr int CB = 64 * Vec<T>::N;
    const long cq = (long)a.Hqk * a.dk, cv = (long)a.Hv * a.dv;
    const long nb = 2 * ((cq + CB - 1) / CB) + (cv + CB - 1) / CB;
    const long nwaves = (long)a.B * nb * (((long)a.T + PTT - 1) / PTT);
    if (nwaves == 0) return hipSuccess;
    if (nwaves > INT32_MAX - 3) return hipErrorInvalidValue;
    const unsigned nblk = (unsigned)((nwaves + 3) / 4);
#define GDN_PRO_W(W_)                                                                                          \
    if (a.W == W_) {                                                                                           \
        hipLaunchKernelGGL((qkv_prologue_kernel<T, W_>), dim3(nblk), dim3(256), 0, st, (const T*)a.q_in,       \
                           (const T*)a.k_in, (const T*)a.v_in, a.wq, a.wk, a.wv, a.st_in, a.st_out, (T*)a.q,     \
                           (T*)a.k, (T*)a.v, a.T, a.Hqk, a.Hv, a.dk, a.dv, a.eps, (int)nwaves);                  \
        return hipGetLastError();                                                                              \
    }
    GDN_PRO_W(1) GDN_PRO_W(2) GDN_PRO_W(3) GDN_PRO_W(4)
#undef GDN_PRO_W
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_rmsnorm_t(const RmsNormArgs& a, hipStream_t st)
{
    constexpr int CB = 64 * Vec<T>::N;
    const long cn = (long)a.Hv * a.dv;
    const long nwaves = (long)a.B * (((long)cn + CB - 1) / CB) * (((long)a.T + RTT - 1) / RTT);
    if (nwaves == 0) return hipSuccess;
    if (nwaves > INT32_MAX - 3) return hipErrorInvalidValue;
    const unsigned nblk = (unsigned)((nwaves + 3) / 4);
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T>), dim3(nblk), dim3(256), 0, st, (const T*)a.o, (const T*)a.z, a.w,
                       a.w_head_stride, (T*)a.y, a.T, a.Hv, a.dv, a.eps, (int)nwaves);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_prologue(const PrologueArgs& a, hipStream_t st)
{
    return a.dtype_bf16 ? launch_prologue_t<bf16>(a, st) : launch_prologue_t<float>(a, st);
}

hipError_t launch_gated_rmsnorm(const RmsNormArgs& a, hipStream_t st)
{
    return a.dtype_bf16 ? launch_rmsnorm_t<bf16>(a, st) : launch_rmsnorm_t<float>(a, st);
}

}  // namespace gdn
