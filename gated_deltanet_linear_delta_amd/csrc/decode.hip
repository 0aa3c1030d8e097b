// Fused decode step of the gated delta rule on gfx950: one pass over each head's float32 state.
//
// Decoding reads and rewrites the whole [dk, dv] state per head for a handful of flops per
// element, so it is bound by HBM ("The Transformer Isn't Alone Anymore", section "The hidden
// consequence: long context"; O(d^2) per step in the summary comparison table of "Gated
// Attention Architectures").  With the state stored as h = S^T ([dk, dv], dv contiguous) and the
// erase/write form of the update ("Architecture Thread I", DeltaNet section, gated as in its
// "Gated DeltaNet" equation):
//     u = h^T k,  w = h^T q,  delta = beta (v - alpha u),
//     h <- alpha h + k delta^T,   o = h_new^T q = alpha w + delta (k . q)
// so one read of h feeds both reductions and the readout needs no second pass.
//
// Layout of the work: one 256-thread workgroup per (batch, value head).  Thread t owns the four
// consecutive columns 4*(t % (dv/4)) .. +3 and the rows r = t / (dv/4) + s * (256 / (dv/4)), so
// one wave instruction moves whole 512-byte rows with 16-byte loads and stores.  Row-partials are
// summed with lane butterflies inside a wave, then across the four waves through LDS.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {

// The new state is written with nontemporal stores: it is not read again in this step, and
// streaming it past the caches rather than allocating it in L2 and the Infinity Cache lets the
// reads of later heads keep those caches (measured on the 512 MiB decode state: 164 us per step
// against 211 us with ordinary stores).
__device__ __forceinline__ void st_state(float* p, floatx4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(p));
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    T* __restrict__ o, int Hqk, int Hv, int grp, float scale)
{
    constexpr int NT = 256;
    constexpr int CG = DV / 4;      // threads per state row (4 columns each)
    constexpr int RPP = NT / CG;    // rows covered by one pass of the workgroup
    constexpr int RPT = DK / RPP;   // rows per thread
    static_assert(CG <= 64 && RPT >= 1 && DK % RPP == 0, "unsupported head dims");

    const int head = blockIdx.x;    // b * Hv + j
    const int b = head / Hv;
    const int j = head - b * Hv;
    const int i = j / grp;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int wave = tid >> 6;

    __shared__ float ks[DK];
    __shared__ float qs[DK];
    constexpr int NWV = NT / 64;    // waves
    __shared__ float red[NWV][CG][9];

    float* hp = state + (size_t)head * DK * DV + 4 * cg;
    floatx4 h[RPT];
#pragma unroll
    for (int s = 0; s < RPT; ++s) h[s] = ld4(hp + (size_t)(rg + s * RPP) * DV);

    const T* kp = k + ((size_t)b * Hqk + i) * DK;
    const T* qp = q + ((size_t)b * Hqk + i) * DK;
    for (int r = tid; r < DK; r += NT) {
        ks[r] = to_f32(kp[r]);
        qs[r] = to_f32(qp[r]) * scale;
    }
    const size_t vo = ((size_t)b * Hv + j) * DV + 4 * cg;
    const floatx4 vv = load4f(v + vo);
    const float alpha = expf(g[head]);
    const float bt = beta[head];
    __syncthreads();

    float u[4] = {0.f, 0.f, 0.f, 0.f}, w[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int s = 0; s < RPT; ++s) {
        const float kr = ks[rg + s * RPP];
        const float qr = qs[rg + s * RPP];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u[c] = fmaf(h[s][c], kr, u[c]);
            w[c] = fmaf(h[s][c], qr, w[c]);
        }
        kq = fmaf(kr, qr, kq);
    }
    if (CG < 64) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u[c] = xor_sum(u[c], CG);
            w[c] = xor_sum(w[c], CG);
        }
        kq = xor_sum(kq, CG);
    }
    if ((tid & 63) < CG) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            red[wave][cg][c] = u[c];
            red[wave][cg][4 + c] = w[c];
        }
        red[wave][cg][8] = kq;
    }
    __syncthreads();
    float ut[4], wt[4], kqt = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) { ut[c] = 0.f; wt[c] = 0.f; }
#pragma unroll
    for (int x = 0; x < NWV; ++x) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ut[c] += red[x][cg][c];
            wt[c] += red[x][cg][4 + c];
        }
        kqt += red[x][cg][8];
    }
    float d[4];
    floatx4 ov;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        d[c] = bt * (vv[c] - alpha * ut[c]);
        ov[c] = alpha * wt[c] + d[c] * kqt;
    }
    if (rg == 0) store4f(o + vo, ov);
#pragma unroll
    for (int s = 0; s < RPT; ++s) {
        const float kr = ks[rg + s * RPP];
        floatx4 hn;
#pragma unroll
        for (int c = 0; c < 4; ++c) hn[c] = fmaf(alpha, h[s][c], kr * d[c]);
        st_state(hp + (size_t)(rg + s * RPP) * DV, hn);
    }
}

template <typename T, int DK, int DV>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t st)
{
    hipLaunchKernelGGL((recurrent_step_kernel<T, DK, DV>), dim3(a.B * a.Hv), dim3(256), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.g, a.beta, a.state, (T*)a.o,
                       a.Hqk, a.Hv, a.Hv / a.Hqk, a.scale);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_step_dt(const StepArgs& a, hipStream_t st)
{
#define GDN_STEP_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_step_t<T, DK_, DV_>(a, st);
    GDN_STEP_CASE(32, 32) GDN_STEP_CASE(32, 64) GDN_STEP_CASE(32, 128)
    GDN_STEP_CASE(64, 32) GDN_STEP_CASE(64, 64) GDN_STEP_CASE(64, 128)
    GDN_STEP_CASE(128, 32) GDN_STEP_CASE(128, 64) GDN_STEP_CASE(128, 128)
#undef GDN_STEP_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_recurrent_step(const StepArgs& a, hipStream_t st)
{
    return a.dtype_bf16 ? launch_step_dt<bf16>(a, st) : launch_step_dt<float>(a, st);
}

}  // namespace gdn
