// Kimi Delta Attention (KDA) prefill on the float32 vector units of gfx950: the delta rule with
// one decay per key channel ("Gated Attention Architectures", section 8, Mathematical
// Formulation):
//     S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t v_t k_t^T,  o_t = S_t^T q_t,
//     D_t = diag(alpha_t) over the dk key channels, g = log alpha given per (token, head, channel)
// with S in R^{dk x dv} stored [B, Hv, dk, dv] as the Gated DeltaNet state is.
//
// Chunkwise (the same WY/UT algebra as the Gated DeltaNet chunk kernels, with the scalar decay
// products replaced by per-channel ones).  Per chunk of C positions with entry state h0,
// gc[r][m] = g[1][m] + ... + g[r][m] and E_rim = exp(gc[r][m] - gc[i][m]) for i <= r:
//     A     = strictly-lower( beta_r sum_m k_rm k_im E_rim )
//     R     = diag(beta) V - diag(beta) (e^gc * K) h0,     Delta = (I + A)^{-1} R
//     O     = (e^gc * Q) h0 + lower-incl( sum_m q_rm k_im E_rim ) Delta
//     h1    = diag(e^gL) h0 + (e^(gL - gc) * K)^T Delta,    gL = gc of the chunk's last row
// The pairwise decays are exponentials of differences (never above 1), so no factor overflows
// however strong a channel's decay is within a chunk.
//
// Work layout: one 1024-thread workgroup per (batch, value head, 32-column tile of dv); chunks
// of 16 or 32 positions; everything for one chunk in LDS in float32.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int KDA_NT = 1024;
constexpr int KDA_CMAX = 32;
constexpr int KDA_BV = 32;

template <int DK>
struct KdaLds {
    static constexpr int KP = DK + 1;
    static constexpr int CP = KDA_CMAX + 1;
    static constexpr size_t k = 0;
    static constexpr size_t q = k + (size_t)KDA_CMAX * KP;
    static constexpr size_t gc = q + (size_t)KDA_CMAX * KP;
    static constexpr size_t v = gc + (size_t)KDA_CMAX * KP;
    static constexpr size_t h = v + (size_t)KDA_CMAX * KDA_BV;
    static constexpr size_t a = h + (size_t)DK * KDA_BV;
    static constexpr size_t aq = a + (size_t)KDA_CMAX * CP;
    static constexpr size_t r = aq + (size_t)KDA_CMAX * CP;
    static constexpr size_t bt = r + (size_t)KDA_CMAX * KDA_BV;
    static constexpr size_t floats = bt + KDA_CMAX;
    static constexpr size_t bytes = floats * sizeof(float);
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(KDA_NT) void kda_chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const float* s0, float* sf,   // s0 and sf may be the same buffer
    T* __restrict__ o, int T_len, int Hqk, int Hv, int grp, int C, float scale)
{
    using L = KdaLds<DK>;
    constexpr int KP = L::KP, CP = L::CP, BV = KDA_BV;
    extern __shared__ float lds[];
    float* Ks = lds + L::k;
    float* Qs = lds + L::q;
    float* Gs = lds + L::gc;
    float* Vs = lds + L::v;
    float* hs = lds + L::h;
    float* As = lds + L::a;
    float* Aq = lds + L::aq;
    float* Rs = lds + L::r;
    float* bs = lds + L::bt;

    const int head = blockIdx.x;   // b * Hv + j
    const int b = head / Hv, j = head - b * Hv, i = j / grp;
    const int c0 = blockIdx.y * BV;
    const int tid = threadIdx.x;
    const size_t sbase = (size_t)head * DK * DV + c0;
    for (int e = tid; e < DK * BV; e += KDA_NT) hs[e] = s0 ? s0[sbase + (size_t)(e / BV) * DV + e % BV] : 0.f;

    constexpr int PER = (KDA_CMAX * BV + KDA_NT - 1) / KDA_NT;
    for (int t0 = 0; t0 < T_len; t0 += C) {
        const int n = min(C, T_len - t0);
        __syncthreads();   // the previous chunk is done with every buffer
        for (int e = tid; e < C * DK; e += KDA_NT) {
            const int r = e / DK, m = e % DK;
            float kv = 0.f, qv = 0.f, gv = 0.f;
            if (r < n) {
                const size_t tok = (size_t)b * T_len + t0 + r;
                kv = to_f32(k[(tok * Hqk + i) * DK + m]);
                qv = to_f32(q[(tok * Hqk + i) * DK + m]) * scale;
                gv = log_decay(g[(tok * Hv + j) * DK + m]);
            }
            Ks[r * KP + m] = kv;
            Qs[r * KP + m] = qv;
            Gs[r * KP + m] = gv;
        }
        for (int e = tid; e < C * BV; e += KDA_NT) {
            const int r = e / BV, c = e % BV;
            Vs[e] = r < n ? to_f32(v[(((size_t)b * T_len + t0 + r) * Hv + j) * DV + c0 + c]) : 0.f;
        }
        if (tid < C) bs[tid] = tid < n ? beta[((size_t)b * T_len + t0 + tid) * Hv + j] : 0.f;
        __syncthreads();
        // per-channel cumulative log decay down the chunk (rows past T add 0)
        for (int m = tid; m < DK; m += KDA_NT) {
            float acc = 0.f;
            for (int r = 0; r < C; ++r) {
                acc += Gs[r * KP + m];
                Gs[r * KP + m] = acc;
            }
        }
        __syncthreads();
        // A (strictly lower, beta-scaled) and the output matrix (lower including the diagonal)
        for (int e = tid; e < C * C; e += KDA_NT) {
            const int r = e / C, s = e % C;
            float a = 0.f, aq = 0.f;
            if (s <= r) {
                float kk = 0.f, qk = 0.f;
#pragma unroll 4
                for (int m = 0; m < DK; ++m) {
                    const float w = __expf(Gs[r * KP + m] - Gs[s * KP + m]) * Ks[s * KP + m];
                    kk = fmaf(Ks[r * KP + m], w, kk);
                    qk = fmaf(Qs[r * KP + m], w, qk);
                }
                aq = qk;
                if (s < r) a = bs[r] * kk;
            }
            As[r * CP + s] = a;
            Aq[r * CP + s] = aq;
        }
        __syncthreads();
        // R = beta (V - (e^gc * K) h0);  keep (e^gc * Q) h0 for the output
        float qh[PER];
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * KDA_NT;
            qh[p] = 0.f;
            if (e < C * BV) {
                const int r = e / BV, c = e % BV;
                float x = 0.f, y = 0.f;
#pragma unroll 4
                for (int m = 0; m < DK; ++m) {
                    const float hm = hs[m * BV + c];
                    const float eg = __expf(Gs[r * KP + m]);
                    x = fmaf(eg * Ks[r * KP + m], hm, x);
                    y = fmaf(eg * Qs[r * KP + m], hm, y);
                }
                Rs[e] = bs[r] * (Vs[e] - x);
                qh[p] = y;
            }
        }
        __syncthreads();
        // Delta = (I + A)^{-1} R: forward substitution down the rows, one thread per column
        if (tid < BV) {
            for (int r = 1; r < C; ++r) {
                float acc = Rs[r * BV + tid];
#pragma unroll 8
                for (int s = 0; s < r; ++s) acc = fmaf(-As[r * CP + s], Rs[s * BV + tid], acc);
                Rs[r * BV + tid] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * KDA_NT;
            if (e < C * BV) {
                const int r = e / BV, c = e % BV;
                float acc = qh[p];
                for (int s = 0; s <= r; ++s) acc = fmaf(Aq[r * CP + s], Rs[s * BV + c], acc);
                if (r < n) o[(((size_t)b * T_len + t0 + r) * Hv + j) * DV + c0 + c] = from_f32<T>(acc);
            }
        }
        // h1 = diag(e^gL) h0 + (e^(gL - gc) * K)^T Delta
        for (int e = tid; e < DK * BV; e += KDA_NT) {
            const int m = e / BV, c = e % BV;
            const float gL = Gs[(C - 1) * KP + m];
            float acc = __expf(gL) * hs[e];
            for (int r = 0; r < C; ++r) acc = fmaf(__expf(gL - Gs[r * KP + m]) * Ks[r * KP + m], Rs[r * BV + c], acc);
            hs[e] = acc;
        }
    }
    __syncthreads();
    if (sf) {
        for (int e = tid; e < DK * BV; e += KDA_NT) sf[sbase + (size_t)(e / BV) * DV + e % BV] = hs[e];
    }
}

template <typename T, int DK, int DV>
hipError_t launch_kda_t(const KdaArgs& a, hipStream_t st)
{
    using L = KdaLds<DK>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    auto kern = kda_chunk_kernel<T, DK, DV>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.B * a.Hv, DV / KDA_BV), dim3(KDA_NT), L::bytes, st, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, a.g, a.beta, a.s0, a.sf, (T*)a.o, a.T, a.Hqk, a.Hv,
                       a.Hv / a.Hqk, a.chunk, a.scale);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_kda_dt(const KdaArgs& a, hipStream_t st)
{
#define GDN_KDA_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_kda_t<T, DK_, DV_>(a, st);
    GDN_KDA_CASE(32, 32) GDN_KDA_CASE(32, 64) GDN_KDA_CASE(32, 128)
    GDN_KDA_CASE(64, 32) GDN_KDA_CASE(64, 64) GDN_KDA_CASE(64, 128)
    GDN_KDA_CASE(128, 32) GDN_KDA_CASE(128, 64) GDN_KDA_CASE(128, 128)
#undef GDN_KDA_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kda_chunk(const KdaArgs& a, hipStream_t st)
{
    if (a.chunk > KDA_CMAX || a.chunk <= 0) return hipErrorInvalidValue;
    return a.dtype_bf16 ? launch_kda_dt<bf16>(a, st) : launch_kda_dt<float>(a, st);
}

}  // namespace gdn
