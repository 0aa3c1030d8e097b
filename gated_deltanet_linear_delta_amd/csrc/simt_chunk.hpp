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

// D += A B for one 16 x 16 tile on the float32 matrix cores (v_mfma_f32_16x16x4_f32): lane l
// supplies A[l % 16][k + l / 16] = a(l % 16, k + l / 16) and B[k + l / 16][l % 16] =
// b(k + l / 16, l % 16) for k = k0, k0 + 4, ... < k1 (k1 - k0 a multiple of 4) and holds
// D[4 (l / 16) + x][l % 16] in element x.  Unrolled by 4: at 8 the backward's gradient kernel
// kept enough hoisted LDS addresses live to spill 104 registers per lane (23 at 4) and ran 8%
// slower.
template <typename FA, typename FB>
__device__ __forceinline__ floatx4 mfma_f32_tile(floatx4 acc, int k0, int k1, FA&& a, FB&& b)
{
    const int l = threadIdx.x & 63, i = l & 15, kq = l >> 4;
#pragma unroll 4
    for (int k = k0; k < k1; k += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(i, k + kq), b(k + kq, i), acc, 0, 0, 0);
    return acc;
}

// Two tiles in one pass over k: D0 += A0 B0 and D1 += A1 B1, with the operands in the layout of
// mfma_f32_tile.  Where the two tiles share an operand (the same expression in both), each step
// reads it from LDS once for both products.
template <typename FA0, typename FB0, typename FA1, typename FB1>
__device__ __forceinline__ void mfma_f32_pair(floatx4& d0, floatx4& d1, int k0, int k1, FA0&& a0, FB0&& b0,
                                              FA1&& a1, FB1&& b1)
{
    const int l = threadIdx.x & 63, i = l & 15, kq = l >> 4;
#pragma unroll 4
    for (int k = k0; k < k1; k += 4) {
        d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0(i, k + kq), b0(k + kq, i), d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1(i, k + kq), b1(k + kq, i), d1, 0, 0, 0);
    }
}

// OUT false: the states only (o is null): the output-only products Q K^T and Q h0 are skipped.
// CMAX: the longest chunk the caller passes (C <= CMAX <= SIMT_CMAX).
// PF: load each chunk's inputs into registers a chunk ahead (see below), else at the chunk's turn.
// AIN: A and the decay exponentials come formed from Ain (per (batch, value head, chunk): A, three
// more [C][C] matrices, e^gc, e^(gL - gc); with PF and without the output) instead of from the
// chunk's K K^T tiles and log-decay cumsum.
template <typename T, int DK, int DV, int BV, bool OUT, int NTH, int CMAX = SIMT_CMAX, bool PF = false,
          bool AIN = false>
__device__ __forceinline__ void simt_chunk_body(
    float* lds, int head, int tile,   // head = b * Hv + j; tile = column tile of BV
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* s0, float* sf,  // may be the same buffer (in-place state update)
    T* __restrict__ o,           // may be null (states only)
    float* __restrict__ hst,     // null, or [B, Hv, NT, DK, DV]: the state entering every chunk
    int T_max, int Hqk, int Hv, int grp, int C, float scale,
    const int* cu, int total,    // packed sequences (cu[0..B] offsets), or null for rows of T_max
    const float* __restrict__ Ain = nullptr)
{
    static_assert(!AIN || (PF && !OUT), "A from memory rides the prefetch of the states-only pass");
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

    // With PF, each chunk's inputs are loaded into registers a chunk ahead: the loads of the next
    // chunk are in flight while this one computes, and land in LDS at the top of its turn.  The
    // loads are unconditional, with the row clamped into the sequence (rows past its end are
    // zeroed when they are written to LDS).  The states-only pass of the backward (32-token
    // chunks) gains from it; the output kernel at 64-token chunks (16 K and 16 Q registers per
    // thread at 512 threads) measured slower with it than with the loads at each chunk's turn.
    constexpr int KPT = PF ? (CMAX * DK + NTH - 1) / NTH : 1;   // K (and Q) elements per thread
    constexpr int VPT = PF ? (CMAX * BV + NTH - 1) / NTH : 1;   // V elements per thread
    constexpr int APT = AIN ? (CMAX * CMAX + NTH - 1) / NTH : 1;   // A elements per thread
    T kr[KPT], qr[OUT ? KPT : 1], vr[VPT];
    float ar[APT];
    float gr = 0.f, br = 0.f, er = 0.f;
    auto fetch = [&](int t0) {   // t0 < T_len; rows at or past T_len read row T_len - 1
        if constexpr (AIN) {
            const float* ap = Ain + ((size_t)head * ((T_max + C - 1) / C) + t0 / C) * (4 * C * C + 2 * C);
#pragma unroll
            for (int p = 0; p < APT; ++p) {
                const int e = tid + p * NTH;
                if (e < C * C) ar[p] = ap[e];
            }
            if (tid < 2 * C) er = ap[4 * C * C + tid];   // e^gc, then e^(gL - gc)
        }
#pragma unroll
        for (int p = 0; p < KPT; ++p) {
            const int e = tid + p * NTH, r = e / DK, m = e % DK;
            const size_t off = ((tok0 + min(t0 + r, T_len - 1)) * Hqk + i) * DK + m;
            kr[p] = k[off];
            if (OUT) qr[p] = q[off];
        }
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int e = tid + p * NTH, r = e / BV, c = e % BV;
            vr[p] = v[((tok0 + min(t0 + r, T_len - 1)) * Hv + j) * DV + c0 + c];
        }
        if (tid < C) {
            const size_t off = (tok0 + min(t0 + tid, T_len - 1)) * Hv + j;
            gr = log_decay(g[off]);
            br = beta[off];
        }
    };
    if (PF && T_len > 0) fetch(0);

    for (int t0 = 0; t0 < T_len; t0 += C) {
        const int n = min(C, T_len - t0);
        __syncthreads();  // previous chunk finished with every LDS buffer
        if (hst) {
            const int NT = (T_max + C - 1) / C;
            float* hp = hst + ((size_t)head * NT + t0 / C) * DK * DV + c0;
            for (int e = tid; e < DK * BV; e += NTH) hp[(size_t)(e / BV) * DV + e % BV] = hs[e];
        }
        if constexpr (PF) {
#pragma unroll
            for (int p = 0; p < KPT; ++p) {
                const int e = tid + p * NTH, r = e / DK, m = e % DK;
                if (e < C * DK) {
                    Ks[r * L::KP + m] = r < n ? to_f32(kr[p]) : 0.f;
                    if (OUT) Qs[r * L::KP + m] = r < n ? to_f32(qr[p]) * scale : 0.f;
                }
            }
#pragma unroll
            for (int p = 0; p < VPT; ++p) {
                const int e = tid + p * NTH;
                if (e < C * BV) Vs[e] = e / BV < n ? to_f32(vr[p]) : 0.f;
            }
            if (tid < C) {
                gcs[tid] = tid < n ? gr : 0.f;
                bs[tid] = tid < n ? br : 0.f;
            }
            if constexpr (AIN) {
#pragma unroll
                for (int p = 0; p < APT; ++p) {
                    const int e = tid + p * NTH;
                    if (e < C * C) As[(e / C) * L::CP + e % C] = ar[p];
                }
                if (tid < 2 * C) (tid < C ? egs : eds)[tid % C] = er;
            }
            if (t0 + C < T_len) fetch(t0 + C);
        } else {
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
                gcs[tid] = tid < n ? log_decay(g[off]) : 0.f;
                bs[tid] = tid < n ? beta[off] : 0.f;
            }
        }
        __syncthreads();
        if constexpr (!AIN) {
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
        }
        // The dense products run on the float32 matrix cores (mfma_f32_tile: float32 products,
        // so float32 inputs keep float32 accuracy), one 16 x 16 output tile per wave at a time.
        const int nw = NTH / 64, w = tid >> 6, lane = tid & 63, li = lane & 15, lq = lane >> 4;
        const int CT = C / 16;          // row tiles of the chunk
        constexpr int BT = BV / 16;     // column tiles of the value tile
        // A (strictly lower, beta-scaled) and the output mask matrix (lower incl. diagonal):
        // tiles (R, S) with S <= R of K K^T and Q K^T, then the decays exp(gc_r - gc_s)
        if (!AIN) for (int tt = w; tt < CT * (CT + 1) / 2; tt += nw) {
            int R = 0;
            while ((R + 1) * (R + 2) / 2 <= tt) ++R;
            const int S = tt - R * (R + 1) / 2;
            const float* Kr = Ks + 16 * R * L::KP;
            const float* Qr = Qs + 16 * R * L::KP;
            const float* Kc = Ks + 16 * S * L::KP;
            auto bk = [&](int k, int jj) { return Kc[jj * L::KP + k]; };
            const floatx4 ga = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, DK,
                                             [&](int ii, int k) { return Kr[ii * L::KP + k]; }, bk);
            floatx4 gq = {0.f, 0.f, 0.f, 0.f};
            if (OUT) gq = mfma_f32_tile(gq, 0, DK, [&](int ii, int k) { return Qr[ii * L::KP + k]; }, bk);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * R + 4 * lq + x, c = 16 * S + li;
                const float gam = c <= r ? expf(gcs[r] - gcs[c]) : 0.f;
                As[r * L::CP + c] = c < r ? bs[r] * gam * ga[x] : 0.f;
                if (OUT) Aq[r * L::CP + c] = gam * gq[x];
            }
        }
        // R = beta V - beta exp(gc) (K h0); keep exp(gc) (Q h0) for the output: tiles (R, T) of
        // the chunk's rows and the value columns (at most one per wave)
        floatx4 qh = {0.f, 0.f, 0.f, 0.f};
        const int tr = w / BT, tc = w % BT;   // this wave's (R, T) tile, when w < CT * BT
        if (w < CT * BT) {
            auto bh = [&](int k, int jj) { return hs[k * BV + 16 * tc + jj]; };
            const floatx4 xk = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, DK,
                                             [&](int ii, int k) { return Ks[(16 * tr + ii) * L::KP + k]; }, bh);
            if (OUT) qh = mfma_f32_tile(qh, 0, DK, [&](int ii, int k) { return Qs[(16 * tr + ii) * L::KP + k]; }, bh);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * tr + 4 * lq + x, c = 16 * tc + li;
                Rs[r * BV + c] = bs[r] * (Vs[r * BV + c] - egs[r] * xk[x]);
                qh[x] *= egs[r];
            }
        }
        __syncthreads();
        // Delta = (I + A)^{-1} R blockwise over 16-row blocks D = 0, 16, ...: forward substitution
        // inside the block (one thread per column, the column in registers, fully unrolled; A read
        // by broadcast, four partial sums per row), then the rows below it take R -= A[rows, D..]
        // Delta[D..] on the matrix cores.
        for (int D = 0; D < C; D += 16) {
            if (tid < BV) {
                float y[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) y[r] = Rs[(D + r) * BV + tid];
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    float acc[4] = {y[r], 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < r; ++c) acc[c & 3] = fmaf(-As[(D + r) * L::CP + D + c], y[c], acc[c & 3]);
                    y[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) Rs[(D + r) * BV + tid] = y[r];
            }
            __syncthreads();
            if (D + 16 < C) {
                const int RT0 = D / 16 + 1;   // first row tile below the block
                for (int tt = w; tt < (CT - RT0) * BT; tt += nw) {
                    const int R = RT0 + tt / BT, T2 = tt % BT;
                    const floatx4 u4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, 16,
                                                     [&](int ii, int k) { return As[(16 * R + ii) * L::CP + D + k]; },
                                                     [&](int k, int jj) { return Rs[(D + k) * BV + 16 * T2 + jj]; });
#pragma unroll
                    for (int x = 0; x < 4; ++x) Rs[(16 * R + 4 * lq + x) * BV + 16 * T2 + li] -= u4[x];
                }
                __syncthreads();
            }
        }
        // O = exp(gc) Q h0 + Aq Delta (Aq is zero right of the diagonal: k up to the tile's end)
        if (OUT && w < CT * BT) {
            const floatx4 ot = mfma_f32_tile(qh, 0, 16 * (tr + 1),
                                             [&](int ii, int k) { return Aq[(16 * tr + ii) * L::CP + k]; },
                                             [&](int k, int jj) { return Rs[k * BV + 16 * tc + jj]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * tr + 4 * lq + x, c = 16 * tc + li;
                if (r < n) o[((tok0 + t0 + r) * Hv + j) * DV + c0 + c] = from_f32<T>(ot[x]);
            }
        }
        // h1 = exp(gc_C) h0 + sum_r exp(gc_C - gc_r) k_r Delta_r^T: tiles (M, T) of the state; with
        // as many 16-row blocks M as waves, each wave takes both column tiles of its M (BT = 2),
        // reading the K operand once for the two
        const float ec = egs[C - 1];
        if constexpr (BT == 2 && DK / 16 >= NTH / 64) {
            for (int M = w; M < DK / 16; M += nw) {
                floatx4 d0, d1;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    d0[x] = ec * hs[(16 * M + 4 * lq + x) * BV + li];
                    d1[x] = ec * hs[(16 * M + 4 * lq + x) * BV + 16 + li];
                }
                auto ak = [&](int ii, int k) { return eds[k] * Ks[k * L::KP + 16 * M + ii]; };
                mfma_f32_pair(d0, d1, 0, C, ak, [&](int k, int jj) { return Rs[k * BV + jj]; },
                              ak, [&](int k, int jj) { return Rs[k * BV + 16 + jj]; });
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    hs[(16 * M + 4 * lq + x) * BV + li] = d0[x];
                    hs[(16 * M + 4 * lq + x) * BV + 16 + li] = d1[x];
                }
            }
        } else for (int tt = w; tt < (DK / 16) * BT; tt += nw) {
            const int M = tt / BT, T2 = tt % BT;
            floatx4 acc;
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[x] = ec * hs[(16 * M + 4 * lq + x) * BV + 16 * T2 + li];
            acc = mfma_f32_tile(acc, 0, C, [&](int ii, int k) { return eds[k] * Ks[k * L::KP + 16 * M + ii]; },
                                [&](int k, int jj) { return Rs[k * BV + 16 * T2 + jj]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) hs[(16 * M + 4 * lq + x) * BV + 16 * T2 + li] = acc[x];
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
