// The chunkwise gated delta rule on the float32 vector units of gfx950, as a device function
// shared by the float32 prefill kernel (chunk_simt.hip) and the backward pass's state recompute
// (chunk_bwd.hip).  The algebra and the work layout are described in chunk_simt.hip.
#pragma once

#include "device_common.hpp"

namespace gdn {

constexpr int SIMT_CMAX = 64;   // longest chunk

template <int DK, int BV>
struct SimtLds {
    static constexpr int KP = DK + 1;  // padded row pitch for K and Q
    static constexpr int CP = SIMT_CMAX + 1;
    static constexpr size_t k_off = 0;
    static constexpr size_t q_off = k_off + (size_t)SIMT_CMAX * KP;
    static constexpr size_t v_off = q_off + (size_t)SIMT_CMAX * KP;
    static constexpr size_t h_off = v_off + (size_t)SIMT_CMAX * BV;
    static constexpr size_t a_off = h_off + (size_t)DK * BV;
    static constexpr size_t aq_off = a_off + (size_t)SIMT_CMAX * CP;
    static constexpr size_t r_off = aq_off + (size_t)SIMT_CMAX * CP;
    static constexpr size_t gc_off = r_off + (size_t)SIMT_CMAX * BV;
    static constexpr size_t b_off = gc_off + SIMT_CMAX;
    static constexpr size_t eg_off = b_off + SIMT_CMAX;
    static constexpr size_t ed_off = eg_off + SIMT_CMAX;
    static constexpr size_t floats = ed_off + SIMT_CMAX;
    static constexpr size_t bytes = floats * sizeof(float);
};

// OUT false: the states only (o is null): the output-only products Q K^T and Q h0 are skipped.
template <typename T, int DK, int DV, int BV, bool OUT, int NTH>
__device__ __forceinline__ void simt_chunk_body(
    float* lds, int head, int tile,   // head = b * Hv + j; tile = column tile of BV
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* s0, float* sf,  // may be the same buffer (in-place state update)
    T* __restrict__ o,           // may be null (states only)
    float* __restrict__ hst,     // null, or [B, Hv, NT, DK, DV]: the state entering every chunk
    int T_max, int Hqk, int Hv, int grp, int C, float scale,
    const int* cu, int total)    // packed sequences (cu[0..B] offsets), or null for rows of T_max
{
    using L = SimtLds<DK, BV>;
    float* Ks = lds + L::k_off;
    float* Qs = lds + L::q_off;
    float* Vs = lds + L::v_off;
    float* hs = lds + L::h_off;
    float* As = lds + L::a_off;
    float* Aq = lds + L::aq_off;
    float* Rs = lds + L::r_off;
    float* gcs = lds + L::gc_off;
    float* bs = lds + L::b_off;
    float* egs = lds + L::eg_off;   // exp(gc_r)
    float* eds = lds + L::ed_off;   // exp(gc_C - gc_r)

    const int b = head / Hv;
    const int j = head - b * Hv;
    const int i = j / grp;
    const int c0 = tile * BV;       // first value column of this tile
    const int tid = threadIdx.x;
    // first token and length of this batch row (offsets clamped into [0, total], lengths into
    // [0, T_max], so no access leaves the tensors whatever cu holds)
    size_t tok0 = (size_t)b * T_max;
    int T_len = T_max;
    if (cu) {
        const int s = min(max(cu[b], 0), total), e = min(max(cu[b + 1], s), total);
        tok0 = (size_t)s;
        T_len = min(e - s, T_max);
    }

    // Entry state tile h[m][c] = state[b, j, m, c0 + c].
    const size_t sbase = (size_t)head * DK * DV + c0;
    for (int e = tid; e < DK * BV; e += NTH) {
        const int m = e / BV, c = e % BV;
        hs[e] = s0 ? s0[sbase + (size_t)m * DV + c] : 0.f;
    }

    for (int t0 = 0; t0 < T_len; t0 += C) {
        const int n = min(C, T_len - t0);
        __syncthreads();  // previous chunk finished with every LDS buffer
        if (hst) {
            const int NT = (T_max + C - 1) / C;
            float* hp = hst + ((size_t)head * NT + t0 / C) * DK * DV + c0;
            for (int e = tid; e < DK * BV; e += NTH) hp[(size_t)(e / BV) * DV + e % BV] = hs[e];
        }
        for (int e = tid; e < C * DK; e += NTH) {
            const int r = e / DK, m = e % DK;
            float kv = 0.f, qv = 0.f;
            if (r < n) {
                const size_t off = ((tok0 + t0 + r) * Hqk + i) * DK + m;
                kv = to_f32(k[off]);
                if (OUT) qv = to_f32(q[off]) * scale;
            }
            Ks[r * L::KP + m] = kv;
            if (OUT) Qs[r * L::KP + m] = qv;
        }
        for (int e = tid; e < C * BV; e += NTH) {
            const int r = e / BV, c = e % BV;
            Vs[e] = r < n ? to_f32(v[((tok0 + t0 + r) * Hv + j) * DV + c0 + c]) : 0.f;
        }
        if (tid < C) {
            const size_t off = (tok0 + t0 + tid) * Hv + j;
            gcs[tid] = tid < n ? g[off] : 0.f;
            bs[tid] = tid < n ? beta[off] : 0.f;
        }
        __syncthreads();
        if (tid < 64) {  // per-chunk log-decay cumsum (C <= 64 terms): a scan across wave 0
            float x = tid < C ? gcs[tid] : 0.f;
#pragma unroll
            for (int sh = 1; sh < 64; sh <<= 1) {
                const float y = __shfl_up(x, sh, 64);
                if (tid >= sh) x += y;
            }
            const float last = __shfl(x, C - 1, 64);
            if (tid < C) {
                gcs[tid] = x;
                egs[tid] = expf(x);
                eds[tid] = expf(last - x);
            }
        }
        __syncthreads();
        // A (strictly lower, beta-scaled) and the output mask matrix (lower incl. diagonal).
        for (int e = tid; e < C * C; e += NTH) {
            const int r = e / C, c = e % C;
            float a = 0.f, aq = 0.f;
            if (c <= r) {
                float kk = 0.f, qk = 0.f;
                for (int m = 0; m < DK; ++m) {
                    const float kc = Ks[c * L::KP + m];
                    kk = fmaf(Ks[r * L::KP + m], kc, kk);
                    if (OUT) qk = fmaf(Qs[r * L::KP + m], kc, qk);
                }
                const float gam = expf(gcs[r] - gcs[c]);
                aq = gam * qk;
                if (c < r) a = bs[r] * gam * kk;
            }
            As[r * L::CP + c] = a;
            Aq[r * L::CP + c] = aq;
        }
        __syncthreads();
        // R = beta V - beta exp(gc) (K h0); keep exp(gc) (Q h0) for the output.
        constexpr int PER = (SIMT_CMAX * BV + NTH - 1) / NTH;
        float qh[PER];
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = tid + p * NTH;
            qh[p] = 0.f;
            if (e < C * BV) {
                const int r = e / BV, c = e % BV;
                float x = 0.f, y = 0.f;
                for (int m = 0; m < DK; ++m) {
                    const float hm = hs[m * BV + c];
                    x = fmaf(Ks[r * L::KP + m], hm, x);
                    if (OUT) y = fmaf(Qs[r * L::KP + m], hm, y);
                }
                Rs[e] = bs[r] * (Vs[e] - egs[r] * x);
                qh[p] = egs[r] * y;
            }
        }
        __syncthreads();
        // Delta = (I + A)^{-1} R, forward substitution down the rows, one thread per column.
        if (tid < BV) {
            for (int r = 1; r < C; ++r) {
                float acc = Rs[r * BV + tid];
#pragma unroll 8
                for (int c = 0; c < r; ++c) acc = fmaf(-As[r * L::CP + c], Rs[c * BV + tid], acc);
                Rs[r * BV + tid] = acc;
            }
        }
        __syncthreads();
        // O = exp(gc) Q h0 + Aq Delta
        if (OUT) {
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int e = tid + p * NTH;
                if (e < C * BV) {
                    const int r = e / BV, c = e % BV;
                    float acc = qh[p];
                    for (int x = 0; x <= r; ++x) acc = fmaf(Aq[r * L::CP + x], Rs[x * BV + c], acc);
                    if (r < n) o[((tok0 + t0 + r) * Hv + j) * DV + c0 + c] = from_f32<T>(acc);
                }
            }
        }
        // K~ = exp(gc_C - gc_r) k_r in place (K is not read again in this chunk)
        for (int e = tid; e < C * DK; e += NTH) {
            const int r = e / DK, m = e % DK;
            Ks[r * L::KP + m] *= eds[r];
        }
        __syncthreads();
        // h1 = exp(gc_C) h0 + sum_r K~_r Delta_r^T
        const float ec = egs[C - 1];
        for (int e = tid; e < DK * BV; e += NTH) {
            const int m = e / BV, c = e % BV;
            float acc = ec * hs[e];
#pragma unroll 8
            for (int r = 0; r < C; ++r) acc = fmaf(Ks[r * L::KP + m], Rs[r * BV + c], acc);
            hs[e] = acc;
        }
    }
    __syncthreads();
    if (sf) {
        for (int e = tid; e < DK * BV; e += NTH) {
            const int m = e / BV, c = e % BV;
            sf[sbase + (size_t)m * DV + c] = hs[e];
        }
    }
}

}  // namespace gdn
