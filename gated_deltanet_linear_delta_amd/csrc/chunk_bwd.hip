// Backward pass of the chunkwise gated delta rule on the float32 vector units of gfx950: the
// gradients of a loss through O and the final state with respect to q, k, v, g, beta and the
// initial state ("Gated Attention Architectures", section 3, names hardware-efficient chunkwise
// training for Gated DeltaNet; the algebra below is the reverse of the forward chunk steps,
// derived from them).
//
// Forward chunk (positions r of one chunk, entry state h = S^T [dk, dv], gc the in-chunk
// log-decay cumsum, gL its last value, Gamma_rs = exp(gc_r - gc_s)):
//   A = strictly-lower(diag(beta)(K K^T * Gamma)),  T = (I + A)^{-1}
//   W = T diag(beta e^gc) K,  U = T diag(beta) V,  Delta = U - W h
//   M = lower-incl((scale Q) K^T * Gamma),  O = diag(e^gc)(scale Q) h + M Delta
//   h' = e^gL h + (diag(e^(gL - gc)) K)^T Delta
// Backward, given dO and the gradient dh' of the chunk's exit state:
//   dDelta = diag(e^(gL-gc)) K dh' + M^T dO
//   dh     = e^gL dh' + (scale Q)^T diag(e^gc) dO - W^T dDelta      (the entry state's gradient)
//   dW = -dDelta h^T,  dV = diag(beta) T^T dDelta,  dT = dDelta (diag(beta) V)^T + dW (diag(beta e^gc) K)^T,
//   dA = strictly-lower(-T^T dT T^T),  and the gates' and keys' terms of every product;
//   dg = reverse cumulative sum of dgc inside the chunk.
//
// Three launches (chunks of 32 positions, value columns in tiles of 32):
// 0. bwd_gram_kernel, one workgroup per (batch, value head, chunk): A and M of the chunk into the
//    workspace (they depend on the chunk's inputs only);
// 1. bwd_pass_kernel, two independent sequential passes side by side, one workgroup per (batch,
//    value head, column tile) each: the float32 forward chunk step run again, storing the state
//    entering every chunk (workspace H), and the reverse state pass, storing each chunk's
//    exit-state gradient (workspace dH) and the initial state's gradient;
// 2. bwd_chunk_kernel: one workgroup per (batch, query/key head, chunk), over the value heads of
//    the group and the column tiles in turn, with dq and dk accumulated in registers, so every
//    gradient is written once (no atomics, deterministic).
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "simt_chunk.hpp"

namespace gdn {

namespace {

constexpr int BW_NT = 512;    // threads per workgroup of the per-chunk kernel
constexpr int DH_NT = 512;   // threads per workgroup of the two sequential passes
constexpr int BW_C = 32;     // chunk length of the backward pass
constexpr int BW_BV = 32;    // value columns per tile
constexpr int BW_CP = BW_C + 1;
constexpr int BW_VP = BW_BV + 1;
// per (batch, value head, chunk) in the workspace: A, M, G, T [4][C][C], then e^gc and e^(gL - gc)
constexpr int BW_AWS = 4 * BW_C * BW_C + 2 * BW_C;

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 halfx8;
// D += A B on the float16 matrix cores, 16 x 16 x 32 (lane l supplies A[l % 16][8 (l / 16) + e]
// and B[8 (l / 16) + e][l % 16], e = 0..7, and holds D[4 (l / 16) + x][l % 16])
__device__ __forceinline__ floatx4 mfma_h(halfx8 a, halfx8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------- reverse state pass

template <int DK>
struct DhLds {
    static constexpr int KP = DK + 1;
    static constexpr size_t k = 0;
    static constexpr size_t q = k + (size_t)BW_C * KP;
    static constexpr size_t dO = q + (size_t)BW_C * KP;
    static constexpr size_t dh = dO + (size_t)BW_C * BW_VP;
    static constexpr size_t a = dh + (size_t)DK * BW_BV;
    static constexpr size_t m = a + (size_t)BW_C * BW_CP;
    static constexpr size_t y = m + (size_t)BW_C * BW_CP;
    static constexpr size_t gc = y + (size_t)BW_C * BW_VP;
    static constexpr size_t eg = gc + BW_C;
    static constexpr size_t ed = eg + BW_C;
    static constexpr size_t bt = ed + BW_C;
    static constexpr size_t floats = bt + BW_C;
    static constexpr size_t bytes = floats * sizeof(float);
};

template <typename T, int DK, int DV>
__device__ __forceinline__ void bwd_dh_body(float* lds, int head, int tile, const T* __restrict__ q,
                                            const T* __restrict__ k, const float* __restrict__ g,
                                            const float* __restrict__ beta, const T* __restrict__ dout,
                                            const float* __restrict__ dsf, float* __restrict__ dH,
                                            float* __restrict__ ds0, int T_len, int Hqk, int Hv, int grp,
                                            float scale, const float* __restrict__ Ain)
{
    using L = DhLds<DK>;
    constexpr int KP = L::KP;
    float* Ks = lds + L::k;
    float* Qs = lds + L::q;
    float* dOs = lds + L::dO;
    float* dhs = lds + L::dh;
    float* As = lds + L::a;
    float* Ms = lds + L::m;
    float* Ys = lds + L::y;
    float* egs = lds + L::eg;
    float* eds = lds + L::ed;
    float* bs = lds + L::bt;

    const int b = head / Hv, j = head - b * Hv, i = j / grp;   // head = b * Hv + j
    const int c0 = tile * BW_BV;
    const int tid = threadIdx.x;
    const int NT = (T_len + BW_C - 1) / BW_C;
    const size_t sbase = (size_t)head * DK * DV + c0;

    for (int e = tid; e < DK * BW_BV; e += DH_NT)
        dhs[e] = dsf ? dsf[sbase + (size_t)(e / BW_BV) * DV + e % BW_BV] : 0.f;
    // Each chunk's inputs are loaded into registers a chunk ahead (the chunk before it, as the
    // pass runs backwards), with unconditional loads of rows clamped into the sequence; rows past
    // its end are zeroed when they are written to LDS.
    constexpr int KPT = (BW_C * DK + DH_NT - 1) / DH_NT;
    constexpr int VPT = (BW_C * BW_BV + DH_NT - 1) / DH_NT;
    constexpr int APT = 2 * BW_C * BW_C / DH_NT;   // A and M elements per thread
    static_assert(APT * DH_NT == 2 * BW_C * BW_C, "A and M spread evenly");
    T kr[KPT], qr[KPT], dr[VPT];
    float ar[APT];
    float er = 0.f, br = 0.f;
    auto fetch = [&](int t0) {   // 0 <= t0 < T_len
        const float* ap = Ain + ((size_t)head * NT + t0 / BW_C) * BW_AWS;
#pragma unroll
        for (int p = 0; p < APT; ++p) ar[p] = ap[tid + p * DH_NT];
#pragma unroll
        for (int p = 0; p < KPT; ++p) {
            const int e = tid + p * DH_NT, r = e / DK, m = e % DK;
            const size_t off = (((size_t)b * T_len + min(t0 + r, T_len - 1)) * Hqk + i) * DK + m;
            kr[p] = k[off];
            qr[p] = q[off];
        }
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int e = tid + p * DH_NT, r = e / BW_BV, c = e % BW_BV;
            dr[p] = dout[(((size_t)b * T_len + min(t0 + r, T_len - 1)) * Hv + j) * DV + c0 + c];
        }
        if (tid < BW_C) br = beta[((size_t)b * T_len + min(t0 + tid, T_len - 1)) * Hv + j];
        if (tid < 2 * BW_C) er = ap[4 * BW_C * BW_C + tid];   // e^gc, then e^(gL - gc)
    };
    if (NT > 0) fetch((NT - 1) * BW_C);
    for (int ci = NT - 1; ci >= 0; --ci) {
        const int t0 = ci * BW_C, n = min(BW_C, T_len - t0);
        __syncthreads();
        // the exit-state gradient of this chunk, for the per-chunk kernel
        float* dp = dH + ((size_t)head * NT + ci) * DK * DV + c0;
        for (int e = tid; e < DK * BW_BV; e += DH_NT) dp[(size_t)(e / BW_BV) * DV + e % BW_BV] = dhs[e];
#pragma unroll
        for (int p = 0; p < KPT; ++p) {
            const int e = tid + p * DH_NT, r = e / DK, m = e % DK;
            if (e < BW_C * DK) {
                Ks[r * KP + m] = r < n ? to_f32(kr[p]) : 0.f;
                Qs[r * KP + m] = r < n ? to_f32(qr[p]) * scale : 0.f;
            }
        }
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int e = tid + p * DH_NT, r = e / BW_BV, c = e % BW_BV;
            if (e < BW_C * BW_BV) dOs[r * BW_VP + c] = r < n ? to_f32(dr[p]) : 0.f;
        }
        if (tid < BW_C) bs[tid] = tid < n ? br : 0.f;
        if (tid < 2 * BW_C) (tid < BW_C ? egs : eds)[tid % BW_C] = er;
#pragma unroll
        for (int p = 0; p < APT; ++p) {   // A, then M: [2][C][C]
            const int e = tid + p * DH_NT, mat = e / (BW_C * BW_C), rc = e % (BW_C * BW_C);
            (mat ? Ms : As)[(rc / BW_C) * BW_CP + rc % BW_C] = ar[p];
        }
        if (ci > 0) fetch(t0 - BW_C);
        __syncthreads();
        // The dense products on the float32 matrix cores (mfma_f32_tile), one 16 x 16 output tile
        // per wave at a time.
        constexpr int CT = BW_C / 16, BT = BW_BV / 16;
        const int w = tid >> 6, lane = tid & 63, li = lane & 15, lq = lane >> 4;
        // dDelta = diag(ed) K dh' + M^T dO: tiles (R, T) of the chunk's rows and the columns; M^T's
        // column r is nonzero from row r on, so its sum starts at the tile's first row
        if (w < CT * BT) {
            const int tr = w / BT, tc = w % BT;
            const floatx4 xk = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, DK,
                                             [&](int ii, int kk) { return Ks[(16 * tr + ii) * KP + kk]; },
                                             [&](int kk, int jj) { return dhs[kk * BW_BV + 16 * tc + jj]; });
            const floatx4 xm = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 16 * tr, BW_C,
                                             [&](int ii, int kk) { return Ms[kk * BW_CP + 16 * tr + ii]; },
                                             [&](int kk, int jj) { return dOs[kk * BW_VP + 16 * tc + jj]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * tr + 4 * lq + x;
                Ys[r * BW_VP + 16 * tc + li] = fmaf(eds[r], xk[x], xm[x]);
            }
        }
        __syncthreads();
        // y = (I + A)^{-T} dDelta = T^T dDelta, back substitution over the two 16-row blocks:
        // y_1 = (I + A_11^T)^{-1} dDelta_1, then dDelta_0 -= A_10^T y_1 on the matrix cores, then
        // y_0 = (I + A_00^T)^{-1} dDelta_0.  Within a block one thread per column, the column in
        // registers (fully unrolled; A read by broadcast, four partial sums per row).
        static_assert(BW_C == 32, "two row blocks");
        auto back_block = [&](int D) {
            float y[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] = Ys[(D + r) * BW_VP + tid];
#pragma unroll
            for (int r = 14; r >= 0; --r) {
                float acc[4] = {y[r], 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = r + 1; s2 < 16; ++s2)
                    acc[(s2 - r - 1) & 3] = fmaf(-As[(D + s2) * BW_CP + D + r], y[s2], acc[(s2 - r - 1) & 3]);
                y[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Ys[(D + r) * BW_VP + tid] = y[r];
        };
        if (tid < BW_BV) back_block(16);
        __syncthreads();
        if (w < BW_BV / 16) {
            const floatx4 t4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, 16,
                                             [&](int ii, int kk) { return As[(16 + kk) * BW_CP + ii]; },
                                             [&](int kk, int jj) { return Ys[(16 + kk) * BW_VP + 16 * w + jj]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) Ys[(4 * lq + x) * BW_VP + 16 * w + li] -= t4[x];
        }
        __syncthreads();
        if (tid < BW_BV) back_block(0);
        __syncthreads();
        // entry-state gradient: e^gL dh' + (scale Q)^T diag(e^gc) dO - (diag(beta e^gc) K)^T y:
        // tiles (M, T) of the state
        const float eL = egs[BW_C - 1];
        if constexpr (BT == 2 && DK / 16 >= DH_NT / 64) {
            // both column tiles of one 16-row block M per wave: the Q and K operands read once
            for (int M = w; M < DK / 16; M += DH_NT / 64) {
                floatx4 d0, d1;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    d0[x] = eL * dhs[(16 * M + 4 * lq + x) * BW_BV + li];
                    d1[x] = eL * dhs[(16 * M + 4 * lq + x) * BW_BV + 16 + li];
                }
                auto aq = [&](int ii, int kk) { return egs[kk] * Qs[kk * KP + 16 * M + ii]; };
                auto ak = [&](int ii, int kk) { return -bs[kk] * egs[kk] * Ks[kk * KP + 16 * M + ii]; };
                mfma_f32_pair(d0, d1, 0, BW_C, aq, [&](int kk, int jj) { return dOs[kk * BW_VP + jj]; },
                              aq, [&](int kk, int jj) { return dOs[kk * BW_VP + 16 + jj]; });
                mfma_f32_pair(d0, d1, 0, BW_C, ak, [&](int kk, int jj) { return Ys[kk * BW_VP + jj]; },
                              ak, [&](int kk, int jj) { return Ys[kk * BW_VP + 16 + jj]; });
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    dhs[(16 * M + 4 * lq + x) * BW_BV + li] = d0[x];
                    dhs[(16 * M + 4 * lq + x) * BW_BV + 16 + li] = d1[x];
                }
            }
        } else for (int tt = w; tt < (DK / 16) * BT; tt += DH_NT / 64) {
            const int M = tt / BT, T2 = tt % BT;
            floatx4 acc;
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[x] = eL * dhs[(16 * M + 4 * lq + x) * BW_BV + 16 * T2 + li];
            acc = mfma_f32_tile(acc, 0, BW_C, [&](int ii, int kk) { return egs[kk] * Qs[kk * KP + 16 * M + ii]; },
                                [&](int kk, int jj) { return dOs[kk * BW_VP + 16 * T2 + jj]; });
            acc = mfma_f32_tile(acc, 0, BW_C,
                                [&](int ii, int kk) { return -bs[kk] * egs[kk] * Ks[kk * KP + 16 * M + ii]; },
                                [&](int kk, int jj) { return Ys[kk * BW_VP + 16 * T2 + jj]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) dhs[(16 * M + 4 * lq + x) * BW_BV + 16 * T2 + li] = acc[x];
        }
    }
    __syncthreads();
    if (ds0) {
        for (int e = tid; e < DK * BW_BV; e += DH_NT) ds0[sbase + (size_t)(e / BW_BV) * DV + e % BW_BV] = dhs[e];
    }
}

// The chunk matrices that depend on the chunk's q, k, g and beta only, for every (batch, value
// head, chunk), formed here in parallel so that the sequential passes and the gradient kernel
// load them instead of forming them inside their serial chains.  Aw[(b Hv + j) NT + ci] holds
// [4][C][C]: A = strictly-lower(diag(beta) G), M = lower-incl((scale Q) K^T * Gamma),
// G = strictly-lower(K K^T * Gamma), T = (I + A)^{-1}.  One 256-thread workgroup per (batch,
// value head, chunk); the 16 x 16 tiles on the float32 matrix cores in the same order as the
// consumers took them before.
constexpr int GR_NT = 256;

template <typename T, int DK>
__global__ __launch_bounds__(GR_NT) void bwd_gram_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const float* __restrict__ g, const float* __restrict__ beta,
                                                         float* __restrict__ Aw, int T_len, int Hqk, int Hv, int grp,
                                                         float scale)
{
    constexpr int KP = DK + 1, CT = BW_C / 16;
    __shared__ float Ks[BW_C * KP], Qs[BW_C * KP], gcs[BW_C], bs[BW_C];
    __shared__ float Gs[BW_C * BW_CP], Tm[BW_C * BW_CP], Xs[16 * BW_VP];
    const int NT = (T_len + BW_C - 1) / BW_C;
    const int ci = blockIdx.x % NT, head = blockIdx.x / NT;
    const int b = head / Hv, j = head - b * Hv, i = j / grp;
    const int t0 = ci * BW_C, n = min(BW_C, T_len - t0);
    const int tid = threadIdx.x;
    for (int e = tid; e < BW_C * DK; e += GR_NT) {
        const int r = e / DK, m = e % DK;
        float kv = 0.f, qv = 0.f;
        if (r < n) {
            const size_t off = (((size_t)b * T_len + t0 + r) * Hqk + i) * DK + m;
            kv = to_f32(k[off]);
            qv = to_f32(q[off]) * scale;
        }
        Ks[r * KP + m] = kv;
        Qs[r * KP + m] = qv;
    }
    if (tid < BW_C) {
        const size_t off = ((size_t)b * T_len + t0 + tid) * Hv + j;
        gcs[tid] = tid < n ? log_decay(g[off]) : 0.f;
        bs[tid] = tid < n ? beta[off] : 0.f;
    }
    __syncthreads();
    if (tid < 64) {   // per-chunk log-decay cumsum: a scan across wave 0
        float x = tid < BW_C ? gcs[tid] : 0.f;
#pragma unroll
        for (int sh = 1; sh < 64; sh <<= 1) {
            const float y = __shfl_up(x, sh, 64);
            if (tid >= sh) x += y;
        }
        const float last = __shfl(x, BW_C - 1, 64);
        if (tid < BW_C) {
            gcs[tid] = x;
            float* Eo = Aw + ((size_t)head * NT + ci) * BW_AWS + 4 * BW_C * BW_C;
            Eo[tid] = expf(x);
            Eo[BW_C + tid] = expf(last - x);
        }
    }
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63, li = lane & 15, lq = lane >> 4;
    float* Ao = Aw + ((size_t)head * NT + ci) * BW_AWS;
    float* Mo = Ao + BW_C * BW_C;
    float* Go = Mo + BW_C * BW_C;
    float* To = Go + BW_C * BW_C;
    for (int tt = w; tt < CT * CT; tt += GR_NT / 64) {   // tiles (R, S); those above the diagonal are zero
        const int R = tt / CT, S = tt % CT;
        floatx4 ga = {0.f, 0.f, 0.f, 0.f}, gq = {0.f, 0.f, 0.f, 0.f};
        if (S <= R) {
            auto bk = [&](int kk, int jj) { return Ks[(16 * S + jj) * KP + kk]; };
            mfma_f32_pair(ga, gq, 0, DK, [&](int ii, int kk) { return Ks[(16 * R + ii) * KP + kk]; }, bk,
                          [&](int ii, int kk) { return Qs[(16 * R + ii) * KP + kk]; }, bk);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * R + 4 * lq + x, sc = 16 * S + li;
            const float gam = sc <= r ? expf(gcs[r] - gcs[sc]) : 0.f;
            Ao[r * BW_C + sc] = sc < r ? bs[r] * gam * ga[x] : 0.f;
            Mo[r * BW_C + sc] = gam * gq[x];
            const float gv = sc < r ? gam * ga[x] : 0.f;
            Go[r * BW_C + sc] = gv;
            Gs[r * BW_CP + sc] = gv;
        }
    }
    __syncthreads();
    // T = (I + diag(beta) G)^{-1} blockwise over the two 16 x 16 diagonal blocks: each diagonal
    // block T_DD = (I + A_DD)^{-1} by forward substitution (one thread per column, the column in
    // registers, G read by broadcast), then T_10 = -T_11 A_10 T_00 on the matrix cores
    static_assert(BW_C == 32, "two diagonal blocks");
    if (tid < BW_C) {
        const int s = tid, D = 16 * (s / 16), sl = s % 16;
        float y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < r; ++u) acc[u & 3] = fmaf(Gs[(D + r) * BW_CP + D + u], y[u], acc[u & 3]);
            const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            y[r] = r == sl ? 1.f : (r > sl ? -bs[D + r] * sum : 0.f);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            Tm[(D + r) * BW_CP + s] = y[r];
            if (D) Tm[r * BW_CP + s] = 0.f;   // above the diagonal blocks
        }
    }
    __syncthreads();
    // X = A_10 T_00 (A = diag(beta) G), then T_10 = -T_11 X: wave 0
    if (w == 0) {
        const floatx4 x4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, 16,
                                         [&](int ii, int kk) { return bs[16 + ii] * Gs[(16 + ii) * BW_CP + kk]; },
                                         [&](int kk, int jj) { return Tm[kk * BW_CP + jj]; });
#pragma unroll
        for (int x = 0; x < 4; ++x) Xs[(4 * lq + x) * BW_VP + li] = x4[x];
    }
    __syncthreads();
    if (w == 0) {
        const floatx4 t4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, 16,
                                         [&](int ii, int kk) { return Tm[(16 + ii) * BW_CP + 16 + kk]; },
                                         [&](int kk, int jj) { return Xs[kk * BW_VP + jj]; });
#pragma unroll
        for (int x = 0; x < 4; ++x) Tm[(16 + 4 * lq + x) * BW_CP + li] = -t4[x];
    }
    __syncthreads();
    for (int e = tid; e < BW_C * BW_C; e += GR_NT) To[e] = Tm[(e / BW_C) * BW_CP + e % BW_C];
}

// The two sequential passes of the backward in one launch, side by side: workgroups
// 0 .. n_chains * NTILE - 1 recompute the states entering every chunk (the float32 forward chunk
// step, no output), the others run the reverse state pass.  The passes do not depend on each
// other, and each has only one workgroup per (batch, value head, column tile), so together they
// fill twice as many compute units as either alone.  512 threads per workgroup for both
// (at 1,024 the 128-register cap spilled the register-column substitutions).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(DH_NT) void bwd_pass_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const float* s0, const T* __restrict__ dout, const float* __restrict__ dsf,
    float* __restrict__ H, float* __restrict__ dH, float* __restrict__ ds0, int T_len, int Hqk, int Hv, int grp,
    float scale, int n_state_blocks, const float* __restrict__ Aw)
{
    constexpr int BV = DV < BW_BV ? DV : BW_BV;
    static_assert(BV == BW_BV || DV < BW_BV, "one column tiling for both passes");
    constexpr int NTILE = DV / BV;
    extern __shared__ float lds[];
    const int bid = blockIdx.x;
    if (bid < n_state_blocks) {
        simt_chunk_body<T, DK, DV, BV, false, DH_NT, BW_C, true, true>(lds, bid / NTILE, bid % NTILE, q, k, v, g, beta,
                                                                    s0, nullptr, nullptr, H, T_len, Hqk, Hv, grp, BW_C,
                                                                    scale, nullptr, 0, Aw);
    } else {
        const int x = bid - n_state_blocks;
        bwd_dh_body<T, DK, DV>(lds, x / NTILE, x % NTILE, q, k, g, beta, dout, dsf, dH, ds0, T_len, Hqk, Hv, grp,
                               scale, Aw);
    }
}

// ------------------------------------------------------------------- per-chunk gradients

template <int DK, bool H16 = false>
struct BwLds {
    static constexpr int KP = DK + 1;
    static constexpr int HP = BW_BV + 1;
    static constexpr size_t k = 0;                                   // K [C][KP]
    static constexpr size_t q = k + (size_t)BW_C * KP;               // scale Q
    static constexpr size_t w = q + (size_t)BW_C * KP;               // W
    static constexpr size_t tm = w + (size_t)BW_C * KP;              // T [C][CP]
    static constexpr size_t gm = tm + (size_t)BW_C * BW_CP;          // K K^T * Gamma, strictly lower
    static constexpr size_t mm = gm + (size_t)BW_C * BW_CP;          // M
    static constexpr size_t dt = mm + (size_t)BW_C * BW_CP;          // dT, later dA
    static constexpr size_t dm = dt + (size_t)BW_C * BW_CP;          // dM, later E, Z, Dk
    static constexpr size_t h = dm + (size_t)BW_C * BW_CP;           // h tile [DK][HP], later dW [C][KP]
    static constexpr size_t dh = h + (size_t)DK * HP;                // dh' tile, later X / K dKB
    static constexpr size_t v = dh + (size_t)DK * HP;                // V tile [C][VP]
    static constexpr size_t dO = v + (size_t)BW_C * BW_VP;
    static constexpr size_t dl = dO + (size_t)BW_C * BW_VP;          // Delta
    static constexpr size_t dd = dl + (size_t)BW_C * BW_VP;          // dDelta
    static constexpr size_t p1 = dd + (size_t)BW_C * BW_VP;          // row-sum scratch
    static constexpr size_t p2 = p1 + (size_t)BW_C * BW_VP;
    static constexpr size_t gc = p2 + (size_t)BW_C * BW_VP;
    static constexpr size_t eg = gc + BW_C;
    static constexpr size_t ed = eg + BW_C;
    static constexpr size_t bt = ed + BW_C;
    static constexpr size_t dgc = bt + BW_C;
    static constexpr size_t dbt = dgc + BW_C;
    static constexpr size_t red = dbt + BW_C;                         // [NT + 1]
    static constexpr size_t floats = red + BW_NT + 1;
    // H16: float16 copies of the column tile's operands of the accumulator products (h, dh'
    // [DK][HP16]; Delta, dDelta, dO [C][HP16]), after the float32 part (bytes)
    static constexpr int HP16 = BW_BV + 8;
    static constexpr size_t h16 = (floats * sizeof(float) + 15) / 16 * 16;
    static constexpr size_t dh16 = h16 + (size_t)DK * HP16 * 2;
    static constexpr size_t d16 = dh16 + (size_t)DK * HP16 * 2;
    static constexpr size_t dd16 = d16 + (size_t)BW_C * HP16 * 2;
    static constexpr size_t do16 = dd16 + (size_t)BW_C * HP16 * 2;
    static constexpr size_t bytes = H16 ? do16 + (size_t)BW_C * HP16 * 2 : floats * sizeof(float);
    static_assert((size_t)BW_C * KP <= (size_t)DK * HP, "dW / X fit the tile buffers");
};

// H16: H and dH hold each chunk's matrices as float16, transposed, [dv][dk] (the layout of the
// float16 sequential passes), instead of float32 [dk][dv].
template <typename T, int DK, int DV, bool H16>
__global__ __launch_bounds__(BW_NT) void bwd_chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const T* __restrict__ dout, const float* __restrict__ H,
    const float* __restrict__ dH, T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta, int T_len, int Hqk, int Hv, int grp, float scale,
    const float* __restrict__ Aw)
{
    using L = BwLds<DK, H16>;
    constexpr int KP = L::KP, HP = L::HP, HP16 = L::HP16;
    // accumulators of the [C, DK] gradients in the layout of 16 x 16 float32 matrix-core tiles
    // (mfma_f32_tile): tile u of the [C, DK] matrix is rows 16 (u / MTL) .., columns 16 (u % MTL) ..;
    // wave w owns tiles w, w + NWV, ... (TPW per wave), and element 4 t + x of lane l for the
    // wave's t-th tile (R0, M0) is row R0 + 4 (l / 16) + x, column M0 + l % 16
    constexpr int MTL = DK / 16, NTL = (BW_C / 16) * MTL, NWV = BW_NT / 64;
    constexpr int TPW = (NTL + NWV - 1) / NWV, PE = 4 * TPW;
    extern __shared__ float lds[];
    float* Ks = lds + L::k;
    float* Qs = lds + L::q;
    float* Ws = lds + L::w;
    float* Tm = lds + L::tm;
    float* Gs = lds + L::gm;
    float* Ms = lds + L::mm;
    float* dTs = lds + L::dt;
    float* dMs = lds + L::dm;
    float* hs = lds + L::h;
    float* dhs = lds + L::dh;
    float* Vs = lds + L::v;
    float* dOs = lds + L::dO;
    float* Ds = lds + L::dl;
    float* dDs = lds + L::dd;
    float* P1 = lds + L::p1;
    float* P2 = lds + L::p2;
    float* gcs = lds + L::gc;
    float* egs = lds + L::eg;
    float* eds = lds + L::ed;
    float* bs = lds + L::bt;
    float* dgcs = lds + L::dgc;
    float* dbts = lds + L::dbt;
    float* red = lds + L::red;
    _Float16* h16s = reinterpret_cast<_Float16*>(reinterpret_cast<unsigned char*>(lds) + L::h16);
    _Float16* dh16s = reinterpret_cast<_Float16*>(reinterpret_cast<unsigned char*>(lds) + L::dh16);
    _Float16* D16s = reinterpret_cast<_Float16*>(reinterpret_cast<unsigned char*>(lds) + L::d16);
    _Float16* dD16s = reinterpret_cast<_Float16*>(reinterpret_cast<unsigned char*>(lds) + L::dd16);
    _Float16* dO16s = reinterpret_cast<_Float16*>(reinterpret_cast<unsigned char*>(lds) + L::do16);

    const int NT = (T_len + BW_C - 1) / BW_C;
    const int ci = blockIdx.x % NT;
    const int bi = blockIdx.x / NT;
    const int i = bi % Hqk, b = bi / Hqk;
    const int t0 = ci * BW_C, n = min(BW_C, T_len - t0);
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, li = lane & 15, lq = lane >> 4;
    auto tile_ok = [&](int t) { return w + t * NWV < NTL; };
    auto tile_r0 = [&](int t) { return 16 * ((w + t * NWV) / MTL); };
    auto tile_m0 = [&](int t) { return 16 * ((w + t * NWV) % MTL); };

    for (int e = tid; e < BW_C * DK; e += BW_NT) {
        const int r = e / DK, m = e % DK;
        float kv = 0.f, qv = 0.f;
        if (r < n) {
            const size_t off = (((size_t)b * T_len + t0 + r) * Hqk + i) * DK + m;
            kv = to_f32(k[off]);
            qv = to_f32(q[off]) * scale;
        }
        Ks[r * KP + m] = kv;
        Qs[r * KP + m] = qv;
    }
    float aQ[PE], aK[PE];
#pragma unroll
    for (int p = 0; p < PE; ++p) aQ[p] = aK[p] = 0.f;

#pragma unroll 1
    for (int jj = 0; jj < grp; ++jj) {
        const int j = i * grp + jj;
        const size_t head = (size_t)b * Hv + j;
        __syncthreads();   // the previous head is done with every buffer
        if (tid < BW_C) {
            const size_t off = ((size_t)b * T_len + t0 + tid) * Hv + j;
            gcs[tid] = tid < n ? log_decay(g[off]) : 0.f;
            bs[tid] = tid < n ? beta[off] : 0.f;
            dgcs[tid] = 0.f;
            dbts[tid] = 0.f;
        }
        for (int e = tid; e < BW_C * BW_CP; e += BW_NT) {
            dTs[e] = 0.f;
            dMs[e] = 0.f;
        }
        // per-wave row partials of three row sums (P2: sum_m Q (dO h^T), K . X, K . dKB)
        static_assert(3 * NWV * BW_C <= BW_C * BW_VP, "per-wave row partials fit the scratch");
        for (int e = tid; e < 3 * NWV * BW_C; e += BW_NT) P2[e] = 0.f;
        {   // G, M and T of this chunk, formed by bwd_gram_kernel ([4][C][C]: A, M, G, T)
            const float* gp = Aw + (head * NT + ci) * BW_AWS;
            for (int e = tid; e < BW_C * BW_C; e += BW_NT) {
                const int r = e / BW_C, c = e % BW_C;
                Ms[r * BW_CP + c] = gp[BW_C * BW_C + e];
                Gs[r * BW_CP + c] = gp[2 * BW_C * BW_C + e];
                Tm[r * BW_CP + c] = gp[3 * BW_C * BW_C + e];
            }
        }
        __syncthreads();
        if (tid < 64) {   // per-chunk log-decay cumsum: a scan across wave 0
            float x = tid < BW_C ? gcs[tid] : 0.f;
#pragma unroll
            for (int sh = 1; sh < 64; sh <<= 1) {
                const float y = __shfl_up(x, sh, 64);
                if (tid >= sh) x += y;
            }
            const float last = __shfl(x, BW_C - 1, 64);
            if (tid < BW_C) {
                gcs[tid] = x;
                egs[tid] = expf(x);
                eds[tid] = expf(last - x);
            }
        }
        __syncthreads();
        constexpr int CT = BW_C / 16;
        constexpr int VT = BW_BV / 16, DT = CT * VT;   // value-column tiles; Delta (dDelta) tiles
        // W = T diag(beta e^gc) K: tiles (R, M) (T lower triangular: the sum stops at the tile's rows)
        for (int tt = w; tt < CT * MTL; tt += BW_NT / 64) {
            const int R = tt / MTL, M = tt % MTL;
            const floatx4 acc = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, 16 * (R + 1),
                                              [&](int ii, int kk) { return Tm[(16 * R + ii) * BW_CP + kk] * bs[kk] * egs[kk]; },
                                              [&](int kk, int jj) { return Ks[kk * KP + 16 * M + jj]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) Ws[(16 * R + 4 * lq + x) * KP + 16 * M + li] = acc[x];
        }
        float aW[PE], aX[PE], aS[PE];   // aS: dO h^T of this head over the tiles (for dgc)
#pragma unroll
        for (int p = 0; p < PE; ++p) aW[p] = aX[p] = aS[p] = 0.f;
        float dbr[4] = {0.f, 0.f, 0.f, 0.f};   // dV waves: row sums of V . (T^T dDelta), over the tiles
        float dgl = 0.f;

        // Each column tile's h, dh', V and dO are loaded into registers while the tile before it
        // computes (h and dh' as 16-byte loads; rows of V and dO past the sequence's end read its
        // last row and are zeroed when written to LDS).
        constexpr int HE = H16 ? 8 : 4;                       // elements per load
        constexpr int H4 = DK * BW_BV / HE;                   // loads of h (and of dh') per tile
        constexpr int HPT = (H4 + BW_NT - 1) / BW_NT;
        constexpr int VPT = BW_C * BW_BV / BW_NT;             // elements of V (and of dO) per thread
        static_assert(VPT * BW_NT == BW_C * BW_BV, "V tile spread evenly");
        using HR = typename std::conditional<H16, halfx8, floatx4>::type;
        HR hr[HPT], dhr[HPT];
        T vr[VPT], dor[VPT];
        auto fetch = [&](int c0) {
#pragma unroll
            for (int p = 0; p < HPT; ++p) {
                const int e4 = tid + p * BW_NT;
                if (e4 < H4) {
                    if constexpr (H16) {
                        // rows 8 (e4 / BV) .. +7 of column e4 % BV (consecutive threads take
                        // consecutive columns, so the LDS writes below are conflict-free)
                        const size_t off = (head * NT + ci) * DK * DV + (size_t)(c0 + e4 % BW_BV) * DK + 8 * (e4 / BW_BV);
                        hr[p] = *reinterpret_cast<const halfx8*>(reinterpret_cast<const _Float16*>(H) + off);
                        dhr[p] = *reinterpret_cast<const halfx8*>(reinterpret_cast<const _Float16*>(dH) + off);
                    } else {
                        // columns 4 (e4 % (BV / 4)) .. +3 of row e4 / (BV / 4)
                        const size_t off = (head * NT + ci) * DK * DV + (size_t)(e4 / (BW_BV / 4)) * DV + c0 +
                                           4 * (e4 % (BW_BV / 4));
                        hr[p] = ld4(H + off);
                        dhr[p] = ld4(dH + off);
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < VPT; ++p) {
                const int e = tid + p * BW_NT, r = e / BW_BV, c = e % BW_BV;
                const size_t off = (((size_t)b * T_len + t0 + min(r, n - 1)) * Hv + j) * DV + c0 + c;
                vr[p] = v[off];
                dor[p] = dout[off];
            }
        };
        fetch(0);

#pragma unroll 1
        for (int c0 = 0; c0 < DV; c0 += BW_BV) {
            __syncthreads();   // W written; the previous tile's row sums done
#pragma unroll
            for (int p = 0; p < HPT; ++p) {
                const int e4 = tid + p * BW_NT;
                if (e4 < H4) {
                    // element x of the load at (m + x, c) (H16) or (m, c + x)
                    const int m = H16 ? 8 * (e4 / BW_BV) : e4 / (BW_BV / 4);
                    const int c = H16 ? e4 % BW_BV : 4 * (e4 % (BW_BV / 4));
                    constexpr int XS = H16 ? HP : 1;
#pragma unroll
                    for (int x = 0; x < HE; ++x) {
                        hs[m * HP + c + x * XS] = (float)hr[p][x];
                        dhs[m * HP + c + x * XS] = (float)dhr[p][x];
                        if constexpr (H16) {
                            h16s[(m + x) * HP16 + c] = hr[p][x];
                            dh16s[(m + x) * HP16 + c] = dhr[p][x];
                        }
                    }
                }
            }
#pragma unroll
            for (int p = 0; p < VPT; ++p) {
                const int e = tid + p * BW_NT, r = e / BW_BV, c = e % BW_BV;
                Vs[r * BW_VP + c] = r < n ? to_f32(vr[p]) : 0.f;
                const float dov = r < n ? to_f32(dor[p]) : 0.f;
                dOs[r * BW_VP + c] = dov;
                if constexpr (H16) dO16s[r * HP16 + c] = (_Float16)dov;
            }
            if (c0 + BW_BV < DV) fetch(c0 + BW_BV);
            __syncthreads();
            // Delta = T (beta V) - W h and dDelta = diag(ed) K dh' + M^T dO over the (C / 16) x (BV / 16)
            // tiles on the float32 matrix cores: one wave per tile for Delta and another for dDelta
            // (T is lower triangular and M^T upper, so their sums stop at, or start at, the tile's
            // own rows)
            static_assert(2 * DT <= BW_NT / 64, "a wave per tile of each");
            if (w < 2 * DT) {
                const int tr = (w % DT) / VT, tc = w % VT;
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                if (w < DT) {
                    const floatx4 u = mfma_f32_tile(z, 0, 16 * (tr + 1),
                                                    [&](int ii, int kk) { return Tm[(16 * tr + ii) * BW_CP + kk] * bs[kk]; },
                                                    [&](int kk, int jj) { return Vs[kk * BW_VP + 16 * tc + jj]; });
                    const floatx4 wh = mfma_f32_tile(z, 0, DK, [&](int ii, int kk) { return Ws[(16 * tr + ii) * KP + kk]; },
                                                     [&](int kk, int jj) { return hs[kk * HP + 16 * tc + jj]; });
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const float dl = u[x] - wh[x];
                        Ds[(16 * tr + 4 * lq + x) * BW_VP + 16 * tc + li] = dl;
                        if constexpr (H16) D16s[(16 * tr + 4 * lq + x) * HP16 + 16 * tc + li] = (_Float16)dl;
                    }
                } else {
                    const floatx4 kd = mfma_f32_tile(z, 0, DK, [&](int ii, int kk) { return Ks[(16 * tr + ii) * KP + kk]; },
                                                     [&](int kk, int jj) { return dhs[kk * HP + 16 * tc + jj]; });
                    const floatx4 md = mfma_f32_tile(z, 16 * tr, BW_C,
                                                     [&](int ii, int kk) { return Ms[kk * BW_CP + 16 * tr + ii]; },
                                                     [&](int kk, int jj) { return dOs[kk * BW_VP + 16 * tc + jj]; });
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int r = 16 * tr + 4 * lq + x;
                        const float dd = fmaf(eds[r], kd[x], md[x]);
                        dDs[r * BW_VP + 16 * tc + li] = dd;
                        if constexpr (H16) dD16s[r * HP16 + 16 * tc + li] = (_Float16)dd;
                    }
                }
            }
            for (int e = tid; e < DK * BW_BV; e += BW_NT) {
                const int m = e / BW_BV, c = e % BW_BV;
                dgl = fmaf(dhs[m * HP + c], hs[m * HP + c], dgl);
            }
            __syncthreads();
            // dV = diag(beta) T^T dDelta (complete for this tile); the row-sum term of dbeta
            const int tr = w / VT, tc = w % VT;
            if (w < DT) {
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                const floatx4 tdu = mfma_f32_tile(z, 16 * tr, BW_C,
                                                  [&](int ii, int kk) { return Tm[kk * BW_CP + 16 * tr + ii]; },
                                                  [&](int kk, int jj) { return dDs[kk * BW_VP + 16 * tc + jj]; });
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int r = 16 * tr + 4 * lq + x, c = 16 * tc + li;
                    if (r < n) dv[(((size_t)b * T_len + t0 + r) * Hv + j) * DV + c0 + c] = from_f32<T>(bs[r] * tdu[x]);
                    float u = Vs[r * BW_VP + c] * tdu[x];
#pragma unroll
                    for (int sh = 1; sh < 16; sh <<= 1) u += __shfl_xor(u, sh, 64);
                    dbr[x] += u;
                }
            }
            // dT += dDelta (diag(beta) V)^T over all (R, S) tiles, dM += dO Delta^T over the tiles
            // with S <= R (lower incl), summed over the tile's value columns on the matrix cores:
            // waves 0 .. CT^2 - 1 take the dT tiles, the next CT (CT + 1) / 2 the dM tiles
            static_assert(CT * CT + CT * (CT + 1) / 2 <= BW_NT / 64, "one [C, C] tile per wave");
            if (w < CT * CT) {
                const int R = w / CT, S = w % CT;
                const floatx4 x4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, BW_BV,
                                                 [&](int ii, int kk) { return dDs[(16 * R + ii) * BW_VP + kk]; },
                                                 [&](int kk, int jj) { return Vs[(16 * S + jj) * BW_VP + kk]; });
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int r = 16 * R + 4 * lq + x, sc = 16 * S + li;
                    dTs[r * BW_CP + sc] += bs[sc] * x4[x];
                }
            } else if (w < CT * CT + CT * (CT + 1) / 2) {
                const int tt = w - CT * CT;
                int R = 0;
                while ((R + 1) * (R + 2) / 2 <= tt) ++R;
                const int S = tt - R * (R + 1) / 2;
                const floatx4 y4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, BW_BV,
                                                 [&](int ii, int kk) { return dOs[(16 * R + ii) * BW_VP + kk]; },
                                                 [&](int kk, int jj) { return Ds[(16 * S + jj) * BW_VP + kk]; });
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int r = 16 * R + 4 * lq + x, sc = 16 * S + li;
                    if (sc <= r) dMs[r * BW_CP + sc] += y4[x];
                }
            }
            // dW -= dDelta h^T;  X += Delta dh'^T;  dQ += diag(e^gc) dO h^T: this wave's
            // accumulator tile, summed over the tile's value columns on the matrix cores
#pragma unroll
            for (int t = 0; t < TPW; ++t) if (tile_ok(t)) {
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                const int r0 = tile_r0(t), m0 = tile_m0(t);
                floatx4 sw, sx, sq;
                if constexpr (H16) {
                    // one float16 16 x 16 x 32 product each (k = the tile's 32 value columns): lane l
                    // supplies row l % 16 of A and column l % 16 of B, k = 8 (l / 16) .. + 7
                    const halfx8 bh = *reinterpret_cast<const halfx8*>(h16s + (m0 + li) * HP16 + 8 * lq);
                    const halfx8 bdh = *reinterpret_cast<const halfx8*>(dh16s + (m0 + li) * HP16 + 8 * lq);
                    sw = mfma_h(*reinterpret_cast<const halfx8*>(dD16s + (r0 + li) * HP16 + 8 * lq), bh, z);
                    sx = mfma_h(*reinterpret_cast<const halfx8*>(D16s + (r0 + li) * HP16 + 8 * lq), bdh, z);
                    sq = mfma_h(*reinterpret_cast<const halfx8*>(dO16s + (r0 + li) * HP16 + 8 * lq), bh, z);
                } else {
                    auto bh = [&](int kk, int jj) { return hs[(m0 + jj) * HP + kk]; };
                    sw = mfma_f32_tile(z, 0, BW_BV, [&](int ii, int kk) { return dDs[(r0 + ii) * BW_VP + kk]; }, bh);
                    sx = mfma_f32_tile(z, 0, BW_BV, [&](int ii, int kk) { return Ds[(r0 + ii) * BW_VP + kk]; },
                                       [&](int kk, int jj) { return dhs[(m0 + jj) * HP + kk]; });
                    sq = mfma_f32_tile(z, 0, BW_BV, [&](int ii, int kk) { return dOs[(r0 + ii) * BW_VP + kk]; }, bh);
                }
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int p = 4 * t + x;
                    aW[p] -= sw[x];
                    aX[p] += sx[x];
                    aQ[p] = fmaf(egs[r0 + 4 * lq + x], sq[x], aQ[p]);
                    aS[p] += sq[x];
                }
            }
            __syncthreads();
        }

        // ---- the terms that need every column: dW, X, dM, dT are complete now
        dgl = xor_sum(dgl, 1);
        if ((tid & 63) == 0) red[tid >> 6] = dgl;
        // the row sums sum_m (scale Q)_rm (dO h^T)_rm (a dgc term) and sum_m K_rm X_rm of this
        // head: each lane over its accumulator entries, summed across the 16 lanes of a row, one
        // partial per (wave, row) (a wave's tiles cover distinct rows)
#pragma unroll
        for (int p = 0; p < PE; ++p) {
            const int r = tile_r0(p / 4) + 4 * lq + p % 4, m = tile_m0(p / 4) + li;
            float v = tile_ok(p / 4) ? Qs[r * KP + m] * aS[p] : 0.f;
            float u = tile_ok(p / 4) ? Ks[r * KP + m] * aX[p] : 0.f;
#pragma unroll
            for (int sh = 1; sh < 16; sh <<= 1) {
                v += __shfl_xor(v, sh, 64);
                u += __shfl_xor(u, sh, 64);
            }
            if (li == 0 && tile_ok(p / 4)) {
                P2[w * BW_C + r] = v;
                P2[(NWV + w) * BW_C + r] = u;
            }
        }
        // P1 rows: [VT][C] the dV waves' dbeta partials, then [C] the M terms of dgc,
        // sum_{s < r} dM_rs M_rs - sum_{u > r} dM_ur M_ur (16 lanes per row; the diagonal terms
        // cancel), then [2][C] the same of A below
        static_assert(BW_NT == 16 * BW_C && (VT + 3) * BW_C <= BW_C * BW_VP, "row-term layout");
        float* dbP = P1;
        float* mP = P1 + VT * BW_C;
        float* aP = mP + BW_C;
        if (w < DT && li == 0) {
#pragma unroll
            for (int x = 0; x < 4; ++x) dbP[(w % VT) * BW_C + 16 * (w / VT) + 4 * lq + x] = dbr[x];
        }
        {
            const int r = tid >> 4, sub = tid & 15;
            float d = 0.f;
#pragma unroll
            for (int s2 = sub; s2 < BW_C; s2 += 16) {
                if (s2 < r) d = fmaf(dMs[r * BW_CP + s2], Ms[r * BW_CP + s2], d);
                if (s2 > r) d = fmaf(-dMs[s2 * BW_CP + r], Ms[s2 * BW_CP + r], d);
            }
#pragma unroll
            for (int sh = 1; sh < 16; sh <<= 1) d += __shfl_xor(d, sh, 64);
            if (sub == 0) mP[r] = d;
        }
        __syncthreads();
        float* dWs = hs;    // [C][KP]
#pragma unroll
        for (int p = 0; p < PE; ++p) if (tile_ok(p / 4)) {
            const int r = tile_r0(p / 4) + 4 * lq + p % 4, m = tile_m0(p / 4) + li;
            dWs[r * KP + m] = aW[p];
        }
        if (tid == 0) {
            float s = 0.f;
#pragma unroll 4
            for (int x = 0; x < BW_NT / 64; ++x) s += red[x];
            red[BW_NT] = egs[BW_C - 1] * s;   // e^gL <dh', h>
        }
        __syncthreads();
        // h' = e^gL h + (diag(ed) K)^T Delta:  dK += diag(ed) X, dgc -= ed (K . X), dgL += sum of those
#pragma unroll
        for (int p = 0; p < PE; ++p) if (tile_ok(p / 4)) {
            const int r = tile_r0(p / 4) + 4 * lq + p % 4;
            aK[p] = fmaf(eds[r], aX[p], aK[p]);
        }
        if (tid < BW_C) {
            const int r = tid;
            float kx = 0.f, s2 = 0.f;
#pragma unroll
            for (int x = 0; x < NWV; ++x) {
                s2 += P2[x * BW_C + r];
                kx += P2[(NWV + x) * BW_C + r];
            }
            const float ted = eds[r] * kx;
            dgcs[r] = fmaf(egs[r], s2, dgcs[r]) - ted + mP[r];
#pragma unroll
            for (int x = 0; x < VT; ++x) dbts[r] += dbP[x * BW_C + r];
            // dgL += sum_r ted_r, across the 32 lanes
            float tsum = ted;
#pragma unroll
            for (int sh = 1; sh < BW_C; sh <<= 1) tsum += __shfl_xor(tsum, sh, 64);
            if (r == 0) red[BW_NT] += tsum;   // written by this thread above
        }
        __syncthreads();
        // E = dM * Gamma (lower incl)
        for (int e = tid; e < BW_C * BW_C; e += BW_NT) {
            const int r = e / BW_C, s = e % BW_C;
            dMs[r * BW_CP + s] = s <= r ? dMs[r * BW_CP + s] * expf(gcs[r] - gcs[s]) : 0.f;
        }
        __syncthreads();
        // dQ += E K;  dK += E^T (scale Q);  dKB = T^T dW -> dK += diag(beta e^gc) dKB, on this
        // wave's accumulator tile (E lower incl and T lower: the sums stop at, or start at, the
        // tile's rows)
#pragma unroll
        for (int t = 0; t < TPW; ++t) if (tile_ok(t)) {
            const floatx4 z = {0.f, 0.f, 0.f, 0.f};
            const int R0 = tile_r0(t), M0 = tile_m0(t);
            const floatx4 eq = mfma_f32_tile(z, 0, R0 + 16, [&](int ii, int kk) { return dMs[(R0 + ii) * BW_CP + kk]; },
                                             [&](int kk, int jj) { return Ks[kk * KP + M0 + jj]; });
            const floatx4 ek = mfma_f32_tile(z, R0, BW_C, [&](int ii, int kk) { return dMs[kk * BW_CP + R0 + ii]; },
                                             [&](int kk, int jj) { return Qs[kk * KP + M0 + jj]; });
            const floatx4 kb = mfma_f32_tile(z, R0, BW_C, [&](int ii, int kk) { return Tm[kk * BW_CP + R0 + ii]; },
                                             [&](int kk, int jj) { return dWs[kk * KP + M0 + jj]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int p = 4 * t + x, r = R0 + 4 * lq + x, m = M0 + li;
                aQ[p] += eq[x];
                aK[p] += ek[x] + bs[r] * egs[r] * kb[x];
                // the row sums of K . dKB, per (wave, row) as above
                float u = Ks[r * KP + m] * kb[x];
#pragma unroll
                for (int sh = 1; sh < 16; sh <<= 1) u += __shfl_xor(u, sh, 64);
                if (li == 0) P2[(2 * NWV + w) * BW_C + r] = u;
            }
        }
        // dT += dW (diag(beta e^gc) K)^T: tiles (R, S) of the full [C, C], each over the two halves
        // of dk on two waves; the second half goes to the Delta buffer and Z below adds it
        static_assert(2 * CT * CT == NWV && DK % 8 == 0, "two waves per dT tile");
        float* dT2 = Ds;
        {
            const int R = (w % (CT * CT)) / CT, S = w % CT, kh = w / (CT * CT);
            const floatx4 x4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, kh * (DK / 2), (kh + 1) * (DK / 2),
                                             [&](int ii, int kk) { return dWs[(16 * R + ii) * KP + kk]; },
                                             [&](int kk, int jj) { return Ks[(16 * S + jj) * KP + kk]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * R + 4 * lq + x, sc = 16 * S + li;
                if (kh == 0)
                    dTs[r * BW_CP + sc] += bs[sc] * egs[sc] * x4[x];
                else
                    dT2[r * BW_VP + sc] = bs[sc] * egs[sc] * x4[x];
            }
        }
        __syncthreads();
        if (tid < BW_C) {
            const int r = tid;
            float kb = 0.f;
#pragma unroll
            for (int x = 0; x < NWV; ++x) kb += P2[(2 * NWV + x) * BW_C + r];
            dbts[r] = fmaf(egs[r], kb, dbts[r]);
            dgcs[r] = fmaf(bs[r] * egs[r], kb, dgcs[r]);
        }
        // Z = dT T^T (into the dM buffer), one 16 x 16 tile (R, S) per wave on the matrix cores
        // (T lower triangular: the sum over u stops at the tile's last column)
        static_assert(CT * CT <= NWV, "a wave per tile of Z and of dA");
        if (w < CT * CT) {
            const int R = w / CT, S = w % CT;
            const floatx4 z4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, 16 * (S + 1),
                                             [&](int ii, int kk) {
                                                 return dTs[(16 * R + ii) * BW_CP + kk] + dT2[(16 * R + ii) * BW_VP + kk];
                                             },
                                             [&](int kk, int jj) { return Tm[(16 * S + jj) * BW_CP + kk]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) dMs[(16 * R + 4 * lq + x) * BW_CP + 16 * S + li] = z4[x];
        }
        __syncthreads();
        // dA = strictly-lower(-T^T Z) (into the dT buffer), the same way (T^T upper: the sum over
        // u starts at the tile's first row; the tile above the diagonal is zero)
        if (w < CT * CT) {
            const int R = w / CT, S = w % CT;
            floatx4 a4 = {0.f, 0.f, 0.f, 0.f};
            if (S <= R)
                a4 = mfma_f32_tile(a4, 16 * R, BW_C, [&](int ii, int kk) { return Tm[kk * BW_CP + 16 * R + ii]; },
                                   [&](int kk, int jj) { return dMs[kk * BW_CP + 16 * S + jj]; });
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * R + 4 * lq + x, sc = 16 * S + li;
                dTs[r * BW_CP + sc] = sc < r ? -a4[x] : 0.f;
            }
        }
        __syncthreads();
        // A = diag(beta) G:  dbeta_r += sum_{s < r} dA_rs G_rs and dgc_r += beta_r (that sum)
        // - sum_{u > r} dA_ur beta_u G_ur (16 lanes per row; added by the scan below);
        // Dk = dA beta_r Gamma
        {
            const int r = tid >> 4, sub = tid & 15;
            float rs = 0.f, cs = 0.f;
#pragma unroll
            for (int s2 = sub; s2 < BW_C; s2 += 16) {
                if (s2 < r) rs = fmaf(dTs[r * BW_CP + s2], Gs[r * BW_CP + s2], rs);
                if (s2 > r) cs = fmaf(dTs[s2 * BW_CP + r] * bs[s2], Gs[s2 * BW_CP + r], cs);
            }
#pragma unroll
            for (int sh = 1; sh < 16; sh <<= 1) {
                rs += __shfl_xor(rs, sh, 64);
                cs += __shfl_xor(cs, sh, 64);
            }
            if (sub == 0) {
                aP[r] = rs;
                aP[BW_C + r] = cs;
            }
        }
        for (int e = tid; e < BW_C * BW_C; e += BW_NT) {
            const int r = e / BW_C, s = e % BW_C;
            dMs[r * BW_CP + s] = s < r ? dTs[r * BW_CP + s] * bs[r] * expf(gcs[r] - gcs[s]) : 0.f;
        }
        __syncthreads();
        // dK += Dk K + Dk^T K on this wave's accumulator tile (Dk strictly lower)
#pragma unroll
        for (int t = 0; t < TPW; ++t) if (tile_ok(t)) {
            const floatx4 z = {0.f, 0.f, 0.f, 0.f};
            const int R0 = tile_r0(t), M0 = tile_m0(t);
            auto bk = [&](int kk, int jj) { return Ks[kk * KP + M0 + jj]; };
            const floatx4 x1 = mfma_f32_tile(z, 0, R0 + 16, [&](int ii, int kk) { return dMs[(R0 + ii) * BW_CP + kk]; }, bk);
            const floatx4 x2 = mfma_f32_tile(z, R0, BW_C, [&](int ii, int kk) { return dMs[kk * BW_CP + R0 + ii]; }, bk);
#pragma unroll
            for (int x = 0; x < 4; ++x) aK[4 * t + x] += x1[x] + x2[x];
        }
        // dg = reverse cumulative sum of dgc (the chunk's last gc also carries dgL): a suffix
        // scan across wave 0, which wrote dgc, dbeta and dgL
        if (tid < 64) {
            float x = tid < BW_C ? dgcs[tid] + bs[tid] * aP[tid] - aP[BW_C + tid] : 0.f;
#pragma unroll
            for (int sh = 1; sh < BW_C; sh <<= 1) {
                const float y = __shfl_down(x, sh, 64);
                if (tid + sh < BW_C) x += y;
            }
            if (tid < n) {
                const size_t off = ((size_t)b * T_len + t0 + tid) * Hv + j;
                dg[off] = red[BW_NT] + x;
                dbeta[off] = dbts[tid] + aP[tid];
            }
        }
    }
#pragma unroll
    for (int p = 0; p < PE; ++p) if (tile_ok(p / 4)) {
        const int r = tile_r0(p / 4) + 4 * lq + p % 4, m = tile_m0(p / 4) + li;
        if (r < n) {
            const size_t off = (((size_t)b * T_len + t0 + r) * Hqk + i) * DK + m;
            dq[off] = from_f32<T>(scale * aQ[p]);
            dk[off] = from_f32<T>(aK[p]);
        }
    }
}

template <typename T, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st)
{
    const int NT = (int)(((long)a.T + BW_C - 1) / BW_C);
    float* Hs = a.ws;
    float* dHs = a.ws + (size_t)a.B * a.Hv * NT * DK * DV;
    float* Aw = dHs + (size_t)a.B * a.Hv * NT * DK * DV;
    const int grp = a.Hv / a.Hqk;
    hipError_t e;
    // 0. A and M of every chunk
    auto gram = bwd_gram_kernel<T, DK>;
    hipLaunchKernelGGL(gram, dim3((unsigned)((long)a.B * a.Hv * NT)), dim3(GR_NT), 0, st,
                       (const T*)a.q, (const T*)a.k, a.g, a.beta, Aw, a.T, a.Hqk, a.Hv, grp, a.scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 1 + 2. the states entering every chunk and the reverse state pass, in one launch: on the
    // float16 matrix cores for bf16 inputs where that kernel takes the shape
    const bool p16 = bwd_pass16_supported(a);
    if (p16) {
        e = launch_bwd_pass16(a, Hs, dHs, Aw, st);
        if (e != hipSuccess) return e;
    } else {
        constexpr int BV = DV < BW_BV ? DV : BW_BV;
        constexpr size_t lb = SimtLds<DK, BV>::bytes > DhLds<DK>::bytes ? SimtLds<DK, BV>::bytes : DhLds<DK>::bytes;
        static_assert(lb <= 160 * 1024, "LDS budget");
        auto kern = bwd_pass_kernel<T, DK, DV>;
        e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lb);
        if (e != hipSuccess) return e;
        const int nblk = a.B * a.Hv * (DV / BV);
        hipLaunchKernelGGL(kern, dim3((unsigned)(2 * nblk)), dim3(DH_NT), lb, st, (const T*)a.q, (const T*)a.k,
                           (const T*)a.v, a.g, a.beta, a.s0, (const T*)a.dout, a.dsf, Hs, dHs, a.ds0, a.T, a.Hqk,
                           a.Hv, grp, a.scale, nblk, Aw);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // 3. per-chunk gradients
    {
        static_assert(BwLds<DK, true>::bytes <= 160 * 1024 && BwLds<DK, false>::bytes <= 160 * 1024, "LDS budget");
        const size_t lb = p16 ? BwLds<DK, true>::bytes : BwLds<DK, false>::bytes;
        auto kern = p16 ? bwd_chunk_kernel<T, DK, DV, true> : bwd_chunk_kernel<T, DK, DV, false>;
        e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lb);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)((long)a.B * a.Hqk * NT)), dim3(BW_NT), lb, st,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, a.g, a.beta, (const T*)a.dout, Hs, dHs,
                           (T*)a.dq, (T*)a.dk, (T*)a.dv, a.dg, a.dbeta, a.T, a.Hqk, a.Hv, grp, a.scale, Aw);
        e = hipGetLastError();
    }
    return e;
}

template <typename T>
hipError_t launch_bwd_dt(const BwdArgs& a, hipStream_t st)
{
#define GDN_BWD_CASE(DK_, DV_) \
    if (a.dk_ == DK_ && a.dv_ == DV_) return launch_bwd_t<T, DK_, DV_>(a, st);
    GDN_BWD_CASE(32, 32) GDN_BWD_CASE(32, 64) GDN_BWD_CASE(32, 128)
    GDN_BWD_CASE(64, 32) GDN_BWD_CASE(64, 64) GDN_BWD_CASE(64, 128)
    GDN_BWD_CASE(128, 32) GDN_BWD_CASE(128, 64) GDN_BWD_CASE(128, 128)
#undef GDN_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace

size_t chunk_bwd_workspace_bytes(int B, int T, int Hv, int dk, int dv)
{
    const size_t NT = ((size_t)T + BW_C - 1) / BW_C;
    return (2 * (size_t)B * Hv * NT * dk * dv + (size_t)B * Hv * NT * BW_AWS) * sizeof(float);
}

hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t st)
{
    return a.dtype_bf16 ? launch_bwd_dt<bf16>(a, st) : launch_bwd_dt<float>(a, st);
}

}  // namespace gdn
