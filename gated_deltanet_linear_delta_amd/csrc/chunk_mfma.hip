// Fused chunkwise gated delta rule on the gfx950 matrix cores (bf16 inputs, float16 matrix
// operands, float32 state and accumulation).  One workgroup of four waves carries one (batch,
// value head, column tile) chain through every chunk of the sequence; nothing but the inputs, O
// and the states touches HBM.
//
// Chunk algebra (the WY/UT form named in "Gated Attention Architectures", section 3: the DeltaNet
// WY representation of section 2 extended with per-chunk cumulative decay products).  Rows are
// chunk positions r = 0..63, gc_r is the per-chunk inclusive cumsum of g = log alpha, h0 = S^T is
// the entry state [dk, BV]:
//   A     = strictly-lower( beta_r exp(gc_r - gc_i) (k_r . k_i) )       T = (I + A)^{-1}
//   R     = diag(beta) V - diag(beta exp(gc)) (K h0)
//   Delta = T R
//   O     = scale ( diag(exp(gc)) (Q h0) + lower-incl( exp(gc_r - gc_i) (q_r . k_i) ) Delta )
//   h1    = exp(gc_63) h0 + K^T diag(exp(gc_63 - gc)) Delta
// The output step has the shape of GLA's chunkwise parallel form ("Gated Attention
// Architectures", section 1) with V replaced by the state-corrected Delta.  Positions past T in
// the last chunk enter as zeros with g = beta = 0, which changes no result.
//
// gfx950 mapping
// * Matrix products use v_mfma_f32_16x16x32_f16 (A 16x32, B 32x16, D 16x16 float32).  A lane
//   holds D rows 4*(lane/16)+i of column lane%16.  Two D tiles stacked along rows therefore give
//   a lane the rows {4g..4g+3, 16+4g..16+4g+3}: used as the B operand of a product over those
//   rows, they need only that the A operand is read with the same permutation of k ("perm-K").
//   The state h (MFMA accumulators) feeds K h and Q h, and Delta feeds (Aqk Delta) and
//   (K^T Delta) straight from registers; only A operands come from LDS.
// * Each wave owns BV/4 state columns (value columns are independent chains), so the state never
//   leaves the wave's registers between chunks.
// * T = (I + A)^{-1}: the four 16x16 diagonal blocks are inverted by forward substitution in
//   float32 (one wave per block), then merged 16 -> 32 -> 64 with matrix products:
//   T_21 = -T_22 A_21 T_11 (16x16x16), then T_hi,lo = -T_hi (A_hi,lo T_lo) (16x16x32).
// * The next chunk's q, k, v, g, beta are loaded into registers while the current chunk computes.
// * Workgroups of one query/key head (its value heads and column tiles read the same q, k) are
//   placed on the same XCD so that the second read of q and k hits that XCD's L2.
#include <stdlib.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

// Matrix-core operands are float16: the same MFMA rate as bf16 on gfx950 with a 3-bit longer
// significand.  q and k arrive as bf16 and convert to float16 exactly (up to float16 subnormals,
// far below what matters next to unit-norm rows); everything else is rounded once from float32.
typedef _Float16 op_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 opx8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 opx4;

constexpr int CH = 64;          // chunk length
constexpr int NW = 4;           // waves per workgroup
constexpr int NTHR = NW * 64;
constexpr int CP = CH + 8;      // element pitch of [*, 64] matrices (T, Aqk, K^T)
constexpr int AFP = CH + 4;     // float pitch of the float32 A matrix

template <int DK, int BV>
struct MLds {
    static constexpr int KP = DK + 8;    // element pitch of K and Q rows
    static constexpr int VP = BV + 8;    // bf16 pitch of V and O rows
    static constexpr size_t ks = 0;                                     // K   [64][KP] f16
    static constexpr size_t qs = ks + (size_t)CH * KP * 2;              // Q   [64][KP] f16
    static constexpr size_t kt = qs + (size_t)CH * KP * 2;              // K^T [DK][CP] f16
    static constexpr size_t vs = kt + (size_t)DK * CP * 2;              // V   [64][VP] bf16
    static constexpr size_t os = vs + (size_t)CH * VP * 2;              // O   [64][VP] bf16
    static constexpr size_t tm = os + (size_t)CH * VP * 2;              // T   [64][CP] f16
    static constexpr size_t aq = tm + (size_t)CH * CP * 2;              // Aqk [64][CP] f16
    static constexpr size_t af = aq + (size_t)CH * CP * 2;              // A   [64][AFP] f32
    static constexpr size_t vec = af + (size_t)CH * AFP * 4;            // 8 x [64] f32
    static constexpr size_t bytes = vec + (size_t)8 * CH * 4;
};

// vec slots
constexpr int V_G = 0;     // raw g, then gc (inclusive cumsum)
constexpr int V_B = 1;     // beta
constexpr int V_EG = 2;    // exp(gc)
constexpr int V_BEG = 3;   // beta exp(gc)
constexpr int V_ED = 4;    // exp(gc_63 - gc)

__device__ __forceinline__ floatx4 mfma32(opx8 a, opx8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(opx4 a, opx4 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// A-operand fragment of a 32-wide k block, perm-K order: row `row`, elements
// [kb + 4g .. kb + 4g + 3] then [kb + 16 + 4g .. kb + 16 + 4g + 3] of a row-major matrix.
__device__ __forceinline__ opx8 frag_perm(const op_t* m, int pitch, int row, int kb, int g)
{
    const op_t* p = m + row * pitch + kb + 4 * g;
    const opx4 lo = *reinterpret_cast<const opx4*>(p);
    const opx4 hi = *reinterpret_cast<const opx4*>(p + 16);
    return opx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Standard-order fragment: elements [kb + 8g .. kb + 8g + 7] of row `row`.
__device__ __forceinline__ opx8 frag_std(const op_t* m, int pitch, int row, int kb, int g)
{
    return *reinterpret_cast<const opx8*>(m + row * pitch + kb + 8 * g);
}

// Two stacked D tiles (rows 0-15 in `a`, 16-31 in `b`) as a perm-K B operand.
__device__ __forceinline__ opx8 pack_perm(floatx4 a, floatx4 b)
{
    return opx8{(op_t)a[0], (op_t)a[1], (op_t)a[2], (op_t)a[3],
                (op_t)b[0], (op_t)b[1], (op_t)b[2], (op_t)b[3]};
}

__device__ __forceinline__ opx8 to_op(bf16x8 x)
{
    return opx8{(op_t)(float)x[0], (op_t)(float)x[1], (op_t)(float)x[2], (op_t)(float)x[3],
                (op_t)(float)x[4], (op_t)(float)x[5], (op_t)(float)x[6], (op_t)(float)x[7]};
}

__device__ __forceinline__ floatx4 ld4s(const float* p) { return *reinterpret_cast<const floatx4*>(p); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// global loads and stores (__syncthreads would also drain those, exposing a full HBM round trip
// of the next chunk's prefetch at every barrier).  Waves exchange data only through LDS here.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace

template <int DK, int DV, int BV>
__global__ __launch_bounds__(NTHR, 1) void chunk_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* s0, float* sf,  // may be the same buffer (in-place state update)
    bf16* __restrict__ o, int T_len, int Hqk, int Hv, int grp, float scale, int xcd_remap)
{
    using L = MLds<DK, BV>;
    constexpr int NTILE = DV / BV;
    constexpr int NCOL = BV / NW;       // state columns per wave
    constexpr int NTN = NCOL / 16;      // 16-column tiles per wave
    constexpr int MT = DK / 16;         // 16-row tiles of the state
    constexpr int KB = DK / 32;         // 32-wide k blocks over dk
    constexpr int SEGK = CH * DK / 8;   // 16-byte segments of a K (or Q) chunk
    constexpr int SEGV = CH * BV / 8;   // 16-byte segments of a V chunk tile
    constexpr int PK = SEGK / NTHR;
    constexpr int PV = SEGV / NTHR;
    static_assert(NTN >= 1 && SEGK % NTHR == 0 && SEGV % NTHR == 0, "tile shape");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    op_t* Ks = reinterpret_cast<op_t*>(smem + L::ks);
    op_t* Qs = reinterpret_cast<op_t*>(smem + L::qs);
    op_t* KT = reinterpret_cast<op_t*>(smem + L::kt);
    bf16* Vs = reinterpret_cast<bf16*>(smem + L::vs);
    bf16* Os = reinterpret_cast<bf16*>(smem + L::os);
    op_t* Tm = reinterpret_cast<op_t*>(smem + L::tm);
    op_t* Aq = reinterpret_cast<op_t*>(smem + L::aq);
    float* Af = reinterpret_cast<float*>(smem + L::af);
    float* vec = reinterpret_cast<float*>(smem + L::vec);

    // ---- which chain this workgroup carries
    int lid = blockIdx.x;
    if (xcd_remap) lid = (lid & 7) * (gridDim.x >> 3) + (lid >> 3);
    const int tile = lid % NTILE;
    lid /= NTILE;
    const int jj = lid % grp;
    lid /= grp;
    const int i = lid % Hqk;
    const int b = lid / Hqk;
    const int j = i * grp + jj;
    const int c0 = tile * BV;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15;      // MFMA column / row-in-tile index
    const int lg = lane >> 4;      // MFMA lane group

    const size_t qk_row = (size_t)Hqk * DK;   // elements between consecutive tokens of q, k
    const size_t v_row = (size_t)Hv * DV;
    const bf16* qb = q + ((size_t)b * T_len * Hqk + i) * DK;
    const bf16* kb_ = k + ((size_t)b * T_len * Hqk + i) * DK;
    const bf16* vb = v + ((size_t)b * T_len * Hv + j) * DV + c0;
    bf16* ob = o + ((size_t)b * T_len * Hv + j) * DV + c0;
    const float* gb = g + (size_t)b * T_len * Hv + j;
    const float* bb = beta + (size_t)b * T_len * Hv + j;

    // ---- zero the parts of T and Aqk that no chunk writes (upper blocks)
    for (int e = tid; e < CH * CP; e += NTHR) {
        Tm[e] = (op_t)0.f;
        Aq[e] = (op_t)0.f;
    }

    // ---- entry state in MFMA accumulator layout: hacc[nt][mt][x] = h[16mt + 4lg + x][col]
    floatx4 hacc[NTN][MT];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) hacc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (s0) {
        const float* sp = s0 + ((size_t)b * Hv + j) * DK * DV + c0 + w * NCOL + ln;
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) hacc[nt][mt][x] = sp[(size_t)(16 * mt + 4 * lg + x) * DV + nt * 16];
    }

    // ---- global -> register staging of one chunk.  Loads are unconditional (rows past T are
    // clamped to the last valid row) and rows past T are zeroed only when written to LDS, so no
    // load destination is written early and the prefetch never waits on earlier memory traffic.
    bf16x8 rk[PK], rq[PK], rv[PV];
    float rg = 0.f, rb = 0.f;
    int n_pref = 0;
    auto load_chunk = [&](int t0) {
        const int n = min(CH, T_len - t0);
        n_pref = n;
#pragma unroll
        for (int p = 0; p < PK; ++p) {
            const int s = tid + p * NTHR;
            const int r = min(s / (DK / 8), n - 1), c8 = (s % (DK / 8)) * 8;
            const size_t off = (size_t)(t0 + r) * qk_row + c8;
            rk[p] = *reinterpret_cast<const bf16x8*>(kb_ + off);
            rq[p] = *reinterpret_cast<const bf16x8*>(qb + off);
        }
#pragma unroll
        for (int p = 0; p < PV; ++p) {
            const int s = tid + p * NTHR;
            const int r = min(s / (BV / 8), n - 1), c8 = (s % (BV / 8)) * 8;
            rv[p] = *reinterpret_cast<const bf16x8*>(vb + (size_t)(t0 + r) * v_row + c8);
        }
        if (w == 0) {
            const size_t off = (size_t)(t0 + min(lane, n - 1)) * Hv;
            rg = gb[off];
            rb = bb[off];
        }
    };
    auto store_chunk = [&]() {
        const int n = n_pref;
#pragma unroll
        for (int p = 0; p < PK; ++p) {
            const int s = tid + p * NTHR;
            const int r = s / (DK / 8), c8 = (s % (DK / 8)) * 8;
            const bool live = r < n;
            *reinterpret_cast<opx8*>(Ks + r * L::KP + c8) = live ? to_op(rk[p]) : opx8{};
            *reinterpret_cast<opx8*>(Qs + r * L::KP + c8) = live ? to_op(rq[p]) : opx8{};
        }
#pragma unroll
        for (int p = 0; p < PV; ++p) {
            const int s = tid + p * NTHR;
            const int r = s / (BV / 8), c8 = (s % (BV / 8)) * 8;
            *reinterpret_cast<bf16x8*>(Vs + r * L::VP + c8) = r < n ? rv[p] : bf16x8{};
        }
        if (w == 0) {
            vec[V_G * CH + lane] = lane < n ? rg : 0.f;
            vec[V_B * CH + lane] = lane < n ? rb : 0.f;
        }
    };

    load_chunk(0);
    store_chunk();

    for (int t0 = 0; t0 < T_len; t0 += CH) {
        const int n = min(CH, T_len - t0);
        const bool has_next = t0 + CH < T_len;
        lds_barrier();                                   // chunk t0 staged in LDS
        if (has_next) load_chunk(t0 + CH);                 // in flight during this chunk

        // ---- (1) per-chunk log-decay cumsum and per-row factors (wave 0); K^T (all waves)
        if (w == 0) {
            float x = vec[V_G * CH + lane];
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                const float y = __shfl_up(x, s, 64);
                if (lane >= s) x += y;
            }
            const float last = __shfl(x, 63, 64);
            const float bt = vec[V_B * CH + lane];
            const float eg = __expf(x);
            vec[V_G * CH + lane] = x;
            vec[V_EG * CH + lane] = eg;
            vec[V_BEG * CH + lane] = bt * eg;
            vec[V_ED * CH + lane] = __expf(last - x);
        }
        // K^T[m][c] = K[c][m]: each thread assembles 8 consecutive c of one row m
        for (int s = tid; s < DK * (CH / 8); s += NTHR) {
            const int m = s % DK, c8 = (s / DK) * 8;
            opx8 t;
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = Ks[(c8 + e) * L::KP + m];
            *reinterpret_cast<opx8*>(KT + m * CP + c8) = t;
        }
        lds_barrier();

        // ---- (2) K K^T and Q K^T on the 10 lower 16x16 tiles each; masks and decays applied
        {
            // tile lists per wave: (is_qk, ti, tj)
            const int gcl = ln;                      // column within tile
            auto do_tile = [&](bool qk, int ti, int tj) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb2 = 0; kb2 < DK; kb2 += 32) {
                    const opx8 a = frag_std(qk ? Qs : Ks, L::KP, 16 * ti + ln, kb2, lg);
                    const opx8 bm = frag_std(Ks, L::KP, 16 * tj + ln, kb2, lg);
                    acc = mfma32(a, bm, acc);
                }
                const int c = 16 * tj + gcl;
                const float gcc = vec[V_G * CH + c];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int r = 16 * ti + 4 * lg + x;
                    const float gam = c <= r ? __expf(vec[V_G * CH + r] - gcc) : 0.f;
                    if (qk) {
                        Aq[r * CP + c] = (op_t)(gam * acc[x]);
                    } else {
                        Af[r * AFP + c] = c < r ? vec[V_B * CH + r] * gam * acc[x] : 0.f;
                    }
                }
            };
            if (w == 0) {
                for (int tj = 0; tj < 4; ++tj) do_tile(false, 3, tj);
                do_tile(true, 0, 0);
            } else if (w == 1) {
                for (int tj = 0; tj < 3; ++tj) do_tile(false, 2, tj);
                for (int tj = 0; tj < 2; ++tj) do_tile(true, 1, tj);
            } else if (w == 2) {
                do_tile(false, 0, 0);
                for (int tj = 0; tj < 2; ++tj) do_tile(false, 1, tj);
                for (int tj = 0; tj < 3; ++tj) do_tile(true, 2, tj);
            } else {
                for (int tj = 0; tj < 4; ++tj) do_tile(true, 3, tj);
            }
        }
        lds_barrier();

        // ---- (3) T = (I + A)^{-1}
        // (3a) diagonal block w: column ln of (I + A_ww)^{-1} by forward substitution (float32)
        float tcol[16];
        {
            const float* Ab = Af + (16 * w) * AFP + 16 * w;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == ln) ? 1.f : 0.f;
#pragma unroll
                for (int x = 0; x < r; ++x) s = fmaf(-Ab[r * AFP + x], tcol[x], s);
                tcol[r] = s;
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                float val = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) val = (r == 4 * lg + x) ? tcol[r] : val;
                Tm[(16 * w + 4 * lg + x) * CP + 16 * w + ln] = (op_t)val;
            }
        }
        // this lane's B-operand view of its block: rows 4lg..4lg+3 of column ln
        opx4 tb;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            float val = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) val = (r == 4 * lg + x) ? tcol[r] : val;
            tb[x] = (op_t)val;
        }
        lds_barrier();
        // (3b) T_{w+1,w} = -T_{w+1,w+1} A_{w+1,w} T_ww for w in {0, 2}
        floatx4 t10 = {0.f, 0.f, 0.f, 0.f};
        if (w == 0 || w == 2) {
            const floatx4 af = ld4s(Af + (16 * (w + 1) + ln) * AFP + 16 * w + 4 * lg);
            const opx4 aa = {(op_t)af[0], (op_t)af[1], (op_t)af[2], (op_t)af[3]};
            const floatx4 p = mfma16(aa, tb, floatx4{0.f, 0.f, 0.f, 0.f});
            const opx4 pb = {(op_t)p[0], (op_t)p[1], (op_t)p[2], (op_t)p[3]};
            const opx4 td = *reinterpret_cast<const opx4*>(Tm + (16 * (w + 1) + ln) * CP + 16 * (w + 1) + 4 * lg);
            t10 = mfma16(td, pb, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                t10[x] = -t10[x];
                Tm[(16 * (w + 1) + 4 * lg + x) * CP + 16 * w + ln] = (op_t)t10[x];
            }
        }
        lds_barrier();
        // (3c) T[32:64, 0:32] = -T_hi (A[32:64, 0:32] T_lo); wave w in {0,1} takes column tile w
        if (w < 2) {
            // T_lo[:, 16w + ln] as a perm-K B operand: rows {4lg..+3} then {16 + 4lg..+3}
            opx8 tlo;
            if (w == 0) {
                tlo = opx8{tb[0], tb[1], tb[2], tb[3], (op_t)t10[0], (op_t)t10[1], (op_t)t10[2], (op_t)t10[3]};
            } else {
                tlo = opx8{(op_t)0.f, (op_t)0.f, (op_t)0.f, (op_t)0.f, tb[0], tb[1], tb[2], tb[3]};
            }
            floatx4 q1[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const float* ar = Af + (32 + 16 * a + ln) * AFP;
                const floatx4 lo = ld4s(ar + 4 * lg);
                const floatx4 hi = ld4s(ar + 16 + 4 * lg);
                const opx8 aa = {(op_t)lo[0], (op_t)lo[1], (op_t)lo[2], (op_t)lo[3],
                                 (op_t)hi[0], (op_t)hi[1], (op_t)hi[2], (op_t)hi[3]};
                q1[a] = mfma32(aa, tlo, floatx4{0.f, 0.f, 0.f, 0.f});
            }
            const opx8 q1b = pack_perm(q1[0], q1[1]);
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const opx8 th = frag_perm(Tm, CP, 32 + 16 * a + ln, 32, lg);
                floatx4 r = mfma32(th, q1b, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int x = 0; x < 4; ++x) Tm[(32 + 16 * a + 4 * lg + x) * CP + 16 * w + ln] = (op_t)(-r[x]);
            }
        }
        lds_barrier();

        // ---- (4) the chain: X = K h, Y = Q h, R, Delta = T R, O, h update
        const float ec = __expf(vec[V_G * CH + 63]);
        {
            opx8 hb[NTN][KB];
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) hb[nt][kk] = pack_perm(hacc[nt][2 * kk], hacc[nt][2 * kk + 1]);

            floatx4 X[NTN][4], Y[NTN][4];
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    X[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
                    Y[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    const opx8 ak = frag_perm(Ks, L::KP, 16 * mt + ln, 32 * kk, lg);
                    const opx8 aqf = frag_perm(Qs, L::KP, 16 * mt + ln, 32 * kk, lg);
#pragma unroll
                    for (int nt = 0; nt < NTN; ++nt) {
                        X[nt][mt] = mfma32(ak, hb[nt][kk], X[nt][mt]);
                        Y[nt][mt] = mfma32(aqf, hb[nt][kk], Y[nt][mt]);
                    }
                }
            // R = beta V - beta exp(gc) X  (rows 16mt + 4lg + x)
            opx8 rbf[NTN][2];
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) {
                const int col = w * NCOL + nt * 16 + ln;
                floatx4 rr[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int r0 = 16 * mt + 4 * lg;
                    const floatx4 bt = ld4s(vec + V_B * CH + r0);
                    const floatx4 beg = ld4s(vec + V_BEG * CH + r0);
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        rr[mt][x] = bt[x] * (float)Vs[(r0 + x) * L::VP + col] - beg[x] * X[nt][mt][x];
                }
                rbf[nt][0] = pack_perm(rr[0], rr[1]);
                rbf[nt][1] = pack_perm(rr[2], rr[3]);
            }
            // Delta = T R (T lower triangular: row tile mt needs k blocks <= mt/2)
            floatx4 D[NTN][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) D[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int cb = 0; cb <= mt / 2; ++cb) {
                    const opx8 at = frag_perm(Tm, CP, 16 * mt + ln, 32 * cb, lg);
#pragma unroll
                    for (int nt = 0; nt < NTN; ++nt) D[nt][mt] = mfma32(at, rbf[nt][cb], D[nt][mt]);
                }
            }
            opx8 db[NTN][2], dtb[NTN][2];
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    db[nt][cb] = pack_perm(D[nt][2 * cb], D[nt][2 * cb + 1]);
                    const floatx4 e0 = ld4s(vec + V_ED * CH + 32 * cb + 4 * lg);
                    const floatx4 e1 = ld4s(vec + V_ED * CH + 32 * cb + 16 + 4 * lg);
                    floatx4 d0 = D[nt][2 * cb], d1 = D[nt][2 * cb + 1];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        d0[x] *= e0[x];
                        d1[x] *= e1[x];
                    }
                    dtb[nt][cb] = pack_perm(d0, d1);
                }
            // O = scale (exp(gc) Y + Aqk Delta), staged in LDS as bf16 rows
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const floatx4 eg = ld4s(vec + V_EG * CH + 16 * mt + 4 * lg);
                floatx4 oacc[NTN];
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
                    for (int x = 0; x < 4; ++x) oacc[nt][x] = eg[x] * Y[nt][mt][x];
#pragma unroll
                for (int cb = 0; cb <= mt / 2; ++cb) {
                    const opx8 aa = frag_perm(Aq, CP, 16 * mt + ln, 32 * cb, lg);
#pragma unroll
                    for (int nt = 0; nt < NTN; ++nt) oacc[nt] = mfma32(aa, db[nt][cb], oacc[nt]);
                }
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) {
                    const int col = w * NCOL + nt * 16 + ln;
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        Os[(16 * mt + 4 * lg + x) * L::VP + col] = (bf16)(scale * oacc[nt][x]);
                }
            }
            // h <- exp(gc_63) h + K^T (exp(gc_63 - gc) Delta)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
                    for (int x = 0; x < 4; ++x) hacc[nt][mt][x] *= ec;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const opx8 akt = frag_perm(KT, CP, 16 * mt + ln, 32 * cb, lg);
#pragma unroll
                    for (int nt = 0; nt < NTN; ++nt) hacc[nt][mt] = mfma32(akt, dtb[nt][cb], hacc[nt][mt]);
                }
            }
        }
        lds_barrier();                                   // O staged; chunk buffers free
        // ---- (5) next chunk -> LDS, O rows -> global (16-byte stores).  The store loop has a
        // fixed trip count so the compiler can count outstanding memory operations exactly and
        // the next chunk's prefetch never waits for these stores to land.
        if (has_next) store_chunk();
#pragma unroll
        for (int p = 0; p < PV; ++p) {
            const int s = tid + p * NTHR;
            const int r = s / (BV / 8), c8 = (s % (BV / 8)) * 8;
            const bf16x8 val = *reinterpret_cast<const bf16x8*>(Os + r * L::VP + c8);
            if (r < n) *reinterpret_cast<bf16x8*>(ob + (size_t)(t0 + r) * v_row + c8) = val;
        }
    }

    // ---- final state
    if (sf) {
        const size_t sb = ((size_t)b * Hv + j) * DK * DV + c0;
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) {
            const int col = w * NCOL + nt * 16 + ln;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) sf[sb + (size_t)(16 * mt + 4 * lg + x) * DV + col] = hacc[nt][mt][x];
        }
    }
}

namespace {

int choose_bv(const ChunkArgs& a)
{
    if (const char* e = getenv("GDN_MFMA_BV")) {
        const int bv = atoi(e);
        if ((bv == 64 || bv == 128) && a.dv % bv == 0) return bv;
    }
    // Enough workgroups to cover the 256 compute units with whole-dv chains?  Otherwise split
    // the value columns (independent chains) into 64-wide tiles.
    const long chains = (long)a.B * a.Hv;
    if (a.dv == 64) return 64;
    return chains >= 192 ? 128 : 64;
}

template <int DK, int DV, int BV>
hipError_t launch_mfma_t(const ChunkArgs& a, hipStream_t st)
{
    using L = MLds<DK, BV>;
    auto kern = chunk_mfma_kernel<DK, DV, BV>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    const int grp = a.Hv / a.Hqk;
    const long nblk = (long)a.B * a.Hv * (DV / BV);
    // XCD-major placement when every XCD gets whole query/key-head groups
    const long per_xcd = nblk / 8;
    const int remap = (nblk % 8 == 0) && (per_xcd % ((long)grp * (DV / BV)) == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(NTHR), L::bytes, st, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, a.g, a.beta, a.s0, a.sf, (bf16*)a.o, a.T,
                       a.Hqk, a.Hv, grp, a.scale, remap);
    return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a)
{
    if (getenv("GDN_DISABLE_MFMA")) return false;
    return a.dtype_bf16 && a.chunk == CH && (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t st)
{
    const int bv = choose_bv(a);
#define GDN_MFMA_CASE(DK_, DV_, BV_) \
    if (a.dk == DK_ && a.dv == DV_ && bv == BV_) return launch_mfma_t<DK_, DV_, BV_>(a, st);
    GDN_MFMA_CASE(128, 128, 128) GDN_MFMA_CASE(128, 128, 64) GDN_MFMA_CASE(128, 64, 64)
    GDN_MFMA_CASE(64, 128, 128) GDN_MFMA_CASE(64, 128, 64) GDN_MFMA_CASE(64, 64, 64)
#undef GDN_MFMA_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
