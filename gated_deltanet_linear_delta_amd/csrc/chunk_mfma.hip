// Chunkwise gated delta rule on the gfx950 matrix cores (bf16 inputs, float16 matrix operands,
// float32 state and accumulation).
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
// the last chunk enter as zeros with g = beta = 0, which changes no result.  The scale is folded
// into exp(gc) of the output step and into the Q K^T matrix ("Aqk") when they are built.
//
// Two ways to run it, both built from the same per-chunk state step (chain_chunk):
//
// * Fused (chunk_mfma_kernel): one workgroup carries one (batch, value head, column tile) chain
//   through every chunk; nothing but the inputs, O and the states touches HBM.  Four "prep" waves
//   build everything of chunk n+1 that does not depend on the state (the cumsum, K K^T, Q K^T,
//   the decay masks and T) and stage the inputs in LDS, while four "chain" waves carry the state
//   through chunk n.  Four workgroup barriers per chunk.  Suits many chains: the prep work runs
//   beside the chain on the same compute unit.
// * Split (chunk_prep_kernel + chunk_state_kernel): the state-independent part of every chunk is
//   built first, all chunks at once (one wave per chunk and value head), into a workspace: T,
//   scaled Aqk and the gate vectors, 13.5 KB per chunk.  The state pass then only stages inputs
//   and runs the chain, with one barrier per chunk.  Suits few, long chains, where the
//   sequential per-chunk latency of the state pass is the whole cost.
//
// gfx950 mapping
// * Each chain wave owns 16 or 32 state columns (value columns evolve independently), so the
//   state never leaves its registers.
// * Matrix products use v_mfma_f32_16x16x32_f16 (A 16x32, B 32x16, D 16x16 float32).  A lane
//   holds D rows 4*(lane/16)+i of column lane%16.  Two D tiles stacked along rows therefore give
//   a lane the rows {4g..4g+3, 16+4g..16+4g+3}: used as the B operand of a product over those
//   rows, they need only that the A operand is read with the same permutation of k ("perm-K").
//   The state h feeds K h and Q h, and Delta feeds (Aqk Delta) and (K^T Delta) from registers.
// * K^T operands and V in accumulator layout are read straight from the row-major K and V tiles
//   with the gfx950 transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group the
//   sixteen 8-byte reads form a 16x4 matrix D and lane i receives D[i/4 + 4j][i%4], j = 0..3.
// * T: the four 16x16 diagonal blocks are inverted by forward substitution in float32, then
//   merged 16 -> 32 -> 64 with matrix products:
//   T_21 = -T_22 A_21 T_11 (16x16x16), then T_hi,lo = -T_hi (A_hi,lo T_lo) (16x16x32).
// * Operands are float16: the same MFMA rate as bf16 on gfx950 with a 3-bit longer significand.
//   q and k arrive as bf16 and convert exactly (up to float16 subnormals, far below what matters
//   next to unit-norm rows); every other operand is rounded once from float32.  The Gram
//   products of the split path take q and k as bf16 directly (exact products either way).
// * Row pitches are padded so that the 8- and 16-byte fragment reads of 8 consecutive rows
//   cover all 64 LDS banks once.
// * Workgroups of one query/key head (its value heads and column tiles read the same q, k) are
//   placed on the same XCD so that repeated reads of q and k hit that XCD's L2.
#include <stdlib.h>
#include <string.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

typedef _Float16 op_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 opx8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 opx4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short shortx4;

constexpr int CH = 64;            // chunk length
constexpr int NPW = 4;            // prep waves of the fused kernel
constexpr int NCW = 4;            // chain waves of the fused kernel
constexpr int NTHR = (NPW + NCW) * 64;
constexpr int NLW = 4;            // loader waves of the state-pass kernel
constexpr int CP = CH + 8;        // element pitch of [64][64] fp16 matrices (T, Aqk)
constexpr int AFP = CH + 4;       // float pitch of the float32 A matrix

template <int DK, int BV>
struct MLds {
    static constexpr int KP = DK + 8;            // element pitch of K and Q rows
    static constexpr int VP = BV + 16;           // element pitch of V rows
    static constexpr size_t kq_bytes = (size_t)CH * KP * 2;
    static constexpr size_t ks = 0;                                 // K   [2][64][KP] f16
    static constexpr size_t qs = ks + 2 * kq_bytes;                 // Q   [2][64][KP] f16
    static constexpr size_t vs = qs + 2 * kq_bytes;                 // V   [64][VP] bf16
    static constexpr size_t tm = vs + (size_t)CH * VP * 2;          // T   [64][CP] f16
    static constexpr size_t aq = tm + (size_t)CH * CP * 2;          // Aqk [64][CP] f16
    static constexpr size_t af = aq + (size_t)CH * CP * 2;          // A^T [64][AFP] f32
    static constexpr size_t vec = af + (size_t)CH * AFP * 4;        // [2][8][64] f32
    static constexpr size_t bytes = vec + (size_t)2 * 8 * CH * 4;
};

// per-chunk vectors (rows of 64 floats)
constexpr int V_G = 0;     // gc (inclusive cumsum of g within the chunk)
constexpr int V_B = 1;     // beta
constexpr int V_EG = 2;    // scale exp(gc)
constexpr int V_BEG = 3;   // beta exp(gc)
constexpr int V_ED = 4;    // exp(gc_63 - gc)
constexpr int V_EC = 5;    // exp(gc_63) (every element)
constexpr int NVEC = 6;

// Workspace of the split path, per (batch, value head, chunk): T and Aqk as float16 in the
// column-permuted order (below), only the 16x32 blocks a product reads (rows 0-31: columns
// 0-31; rows 32-63: columns 0-63), then the NVEC gate vectors.
constexpr int WS_T = 0;
constexpr int WS_AQ = 3072 * 2;
constexpr int WS_VEC = 2 * 3072 * 2;
constexpr int WS_CHUNK = WS_VEC + NVEC * CH * 4;   // 13824 bytes
static_assert(WS_CHUNK % 16 == 0, "workspace chunk");

__device__ __forceinline__ int blk_off(int r, int pc) { return r < 32 ? r * 32 + pc : 1024 + (r - 32) * 64 + pc; }

__device__ __forceinline__ floatx4 mfma32(opx8 a, opx8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(opx4 a, opx4 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_bf(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Column order of every float16 matrix in LDS (K, Q, T, Aqk): within each 32-column block the
// 4-column groups are stored in the order 0, 4, 1, 5, 2, 6, 3, 7, so that lane group g's perm-K
// set {4g..4g+3, 16+4g..16+4g+3} is one contiguous 16-byte run.  LDS costs about the same per
// instruction for 8 and 16 bytes, so this halves the fragment reads.
__device__ __forceinline__ int pcol(int c)
{
    const int q = (c >> 2) & 7;
    const int p = q < 4 ? 2 * q : 2 * (q - 4) + 1;
    return (c & ~31) + 4 * p + (c & 3);
}

// Fragment of a column-permuted matrix: physical elements [kb + 8g .. kb + 8g + 7] of row `row`,
// which are the logical perm-K elements of lane group g (also a valid standard-order fragment
// when both operands of a product are read this way, as for K K^T and Q K^T).
__device__ __forceinline__ opx8 frag(const op_t* m, int pitch, int row, int kb, int g)
{
    return *reinterpret_cast<const opx8*>(m + row * pitch + kb + 8 * g);
}

// Transposing LDS read (see the header comment): returns four 16-bit values.
__device__ __forceinline__ shortx4 ld_tr(const void* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) shortx4*)(const_cast<void*>(p)));
}

// K^T A operand (perm-K over chunk positions) for the 16 dk rows of tile mt: lane (row ml,
// group g) gets K[kb + 4g + j][16mt + ml] and K[kb + 16 + 4g + j][16mt + ml], j = 0..3, from the
// column-permuted K (logical columns 16mt + 4q .. +3 sit at physical 32(mt/2) + 4(2q + mt%2)).
// The same read gives the B operand of any column-permuted row-major matrix (B[k][n] = M[k][n]).
__device__ __forceinline__ opx8 frag_kt(const op_t* k, int pitch, int mt, int kb, int lane)
{
    const int m = lane & 15, g = lane >> 4;
    const op_t* p = k + (kb + 4 * g + (m >> 2)) * pitch + 32 * (mt >> 1) + 4 * (2 * (m & 3) + (mt & 1));
    const opx4 lo = __builtin_bit_cast(opx4, ld_tr(p));
    const opx4 hi = __builtin_bit_cast(opx4, ld_tr(p + 16 * pitch));
    return opx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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

__device__ __forceinline__ opx8 to_op(bf16x4 a, bf16x4 b)
{
    return opx8{(op_t)(float)a[0], (op_t)(float)a[1], (op_t)(float)a[2], (op_t)(float)a[3],
                (op_t)(float)b[0], (op_t)(float)b[1], (op_t)(float)b[2], (op_t)(float)b[3]};
}

__device__ __forceinline__ floatx4 ld4s(const float* p) { return *reinterpret_cast<const floatx4*>(p); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// global loads and stores (__syncthreads would also drain those, exposing a full HBM round trip
// of the prefetch at every barrier).  Waves exchange data only through LDS here.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Ordering point for lanes of one wave that exchange data through LDS: the compiler moves no
// memory access across it and the wave's LDS operations have completed.
__device__ __forceinline__ void wave_lds_fence()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_cumsum(float x, int lane)
{
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const float y = __shfl_up(x, s, 64);
        if (lane >= s) x += y;
    }
    return x;
}

// =======================================================================================
// One chunk of the state pass for one chain wave (column group cw): reads the staged chunk from
// LDS (K, Q column-permuted float16 [64][DK+8]; V bf16 [64][BV+16]; T, Aqk column-permuted
// float16 [64][CP]; the gate vectors), stores its O rows (ob points at the chunk's first token,
// column tile start) and advances the state columns it owns.  `sync` runs between the three
// phases: a workgroup barrier in the fused kernel (where other waves write LDS meanwhile), a
// scheduling fence in the split path.
template <int DK, int BV, int NW, typename Sync>
__device__ __forceinline__ void chain_chunk(floatx4 (&hacc)[BV / NW / 16][DK / 16], const op_t* Ks,
                                            const op_t* Qs, const bf16* Vs, const op_t* Tm,
                                            const op_t* Aq, const float* vs, bf16* ob, size_t v_row,
                                            int nv, int cw, int lane, Sync&& sync)
{
    constexpr int KP = DK + 8;
    constexpr int VP = BV + 16;
    constexpr int NCOL = BV / NW;       // state columns of this wave
    constexpr int NTN = NCOL / 16;      // 16-column tiles
    constexpr int MT = DK / 16;         // 16-row tiles of the state
    constexpr int KB = DK / 32;         // 32-wide k blocks over dk
    // With one 16-column tile per wave the Q fragments for phase 2 are loaded in phase 1 and the
    // K^T fragments for phase 3 in phase 2; with two tiles the registers do not allow it and each
    // product loads its fragments when its phase starts.
    constexpr bool PRE = NTN == 1;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    opx8 hb[NTN][KB];
    opx8 db[NTN][2], dtb[NTN][2];
    opx8 aqf[KB][4];
    opx8 akt[2][MT];

    // phase 1: X = K h, R = beta V - beta exp(gc) X, Delta = T R.  Every product's A fragments
    // are loaded before its MFMAs, behind a scheduling barrier, so the LDS latency is paid once
    // per product rather than once per MFMA.
    {
        // K fragments: all up front with one tile per wave; with two tiles (twice the MFMAs per
        // k block) one k block ahead, which keeps the registers within budget
        constexpr int AHEAD = PRE ? KB : 1;
        opx8 ak[KB][4];
#pragma unroll
        for (int kk = 0; kk < AHEAD; ++kk)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) ak[kk][mt] = frag(Ks, KP, 16 * mt + ln, 32 * kk, lg);
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) hb[nt][kk] = pack_perm(hacc[nt][2 * kk], hacc[nt][2 * kk + 1]);
        __builtin_amdgcn_sched_barrier(0);
        floatx4 X[NTN][4];
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) X[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            if (kk + AHEAD < KB) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) ak[kk + AHEAD][mt] = frag(Ks, KP, 16 * mt + ln, 32 * (kk + AHEAD), lg);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) X[nt][mt] = mfma32(ak[kk][mt], hb[nt][kk], X[nt][mt]);
        }
        // V rows 16mt+4lg..+3 of this lane's columns via the transposing read; row vectors
        bf16x4 vv[NTN][4];
        floatx4 bt[4], beg[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt)
                vv[nt][mt] = __builtin_bit_cast(bf16x4, ld_tr(Vs + (16 * mt + 4 * lg + (ln >> 2)) * VP +
                                                               cw * NCOL + 16 * nt + 4 * (ln & 3)));
            bt[mt] = ld4s(vs + V_B * CH + 16 * mt + 4 * lg);
            beg[mt] = ld4s(vs + V_BEG * CH + 16 * mt + 4 * lg);
        }
        opx8 at[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int cb = 0; cb <= mt / 2; ++cb) at[mt][cb] = frag(Tm, CP, 16 * mt + ln, 32 * cb, lg);
        opx8 rbf[NTN][2];
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) {
            floatx4 rr[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) rr[mt][x] = bt[mt][x] * (float)vv[nt][mt][x] - beg[mt][x] * X[nt][mt][x];
            rbf[nt][0] = pack_perm(rr[0], rr[1]);
            rbf[nt][1] = pack_perm(rr[2], rr[3]);
        }
        // Delta = T R (T lower triangular: row tile mt needs k blocks cb <= mt/2)
        floatx4 D[NTN][4];
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) D[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int mt = 2 * cb; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) D[nt][mt] = mfma32(at[mt][cb], rbf[nt][cb], D[nt][mt]);
        floatx4 ed[2][2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            ed[cb][0] = ld4s(vs + V_ED * CH + 32 * cb + 4 * lg);
            ed[cb][1] = ld4s(vs + V_ED * CH + 32 * cb + 16 + 4 * lg);
        }
        if constexpr (PRE) {
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) aqf[kk][mt] = frag(Qs, KP, 16 * mt + ln, 32 * kk, lg);
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) {
                db[nt][cb] = pack_perm(D[nt][2 * cb], D[nt][2 * cb + 1]);
                floatx4 d0 = D[nt][2 * cb], d1 = D[nt][2 * cb + 1];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    d0[x] *= ed[cb][0][x];
                    d1[x] *= ed[cb][1][x];
                }
                dtb[nt][cb] = pack_perm(d0, d1);
            }
    }
    sync();
    // phase 2: Y = Q h, O = exp(gc) Y + Aqk Delta (scale folded into both) -> HBM; then the K^T
    // fragments for phase 3
    {
        if constexpr (!PRE) {
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) aqf[kk][mt] = frag(Qs, KP, 16 * mt + ln, 32 * kk, lg);
            __builtin_amdgcn_sched_barrier(0);
        }
        opx8 aa[4][2];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int cb = 0; cb <= ct / 2; ++cb) aa[ct][cb] = frag(Aq, CP, 16 * ct + ln, 32 * cb, lg);
        float eg[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) eg[ct] = vs[V_EG * CH + 16 * ct + ln];
        // O is formed transposed, O^T = (h^T Q^T) diag(exp(gc)) + Delta^T Aqk^T: the same
        // fragments with the operand roles swapped, and the accumulator layout then gives each
        // lane four consecutive value columns of one token (one 8-byte store).
        floatx4 OT[NTN][4];
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) OT[nt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) OT[nt][ct] = mfma32(hb[nt][kk], aqf[kk][ct], OT[nt][ct]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
                for (int x = 0; x < 4; ++x) OT[nt][ct][x] *= eg[ct];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int ct = 2 * cb; ct < 4; ++ct)
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) OT[nt][ct] = mfma32(db[nt][cb], aa[ct][cb], OT[nt][ct]);
        if constexpr (PRE) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) akt[cb][mt] = frag_kt(Ks, KP, mt, 32 * cb, lane);
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int tok = 16 * ct + ln;
            if (tok < nv) {
                bf16* op = ob + (size_t)tok * v_row + cw * NCOL + 4 * lg;
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) {
                    const bf16x4 ov = {(bf16)OT[nt][ct][0], (bf16)OT[nt][ct][1], (bf16)OT[nt][ct][2],
                                       (bf16)OT[nt][ct][3]};
                    *reinterpret_cast<bf16x4*>(op + 16 * nt) = ov;
                }
            }
        }
    }
    sync();
    // phase 3: h <- exp(gc_63) h + K^T (exp(gc_63 - gc) Delta)
    {
        if constexpr (!PRE) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) akt[cb][mt] = frag_kt(Ks, KP, mt, 32 * cb, lane);
        }
        const float ec = vs[V_EC * CH];
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) hacc[nt][mt][x] *= ec;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) hacc[nt][mt] = mfma32(akt[cb][mt], dtb[nt][cb], hacc[nt][mt]);
    }
}

// Entry state of one chain wave's columns (zeros when s0 is null), and its final state.
template <int DK, int DV, int NTN>
__device__ __forceinline__ void load_state(floatx4 (&hacc)[NTN][DK / 16], const float* s0, size_t head,
                                           int col, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int mt = 0; mt < DK / 16; ++mt) hacc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (s0) {
        const float* sp = s0 + head * DK * DV + col + ln;
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int mt = 0; mt < DK / 16; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) hacc[nt][mt][x] = sp[(size_t)(16 * mt + 4 * lg + x) * DV + nt * 16];
    }
}

template <int DK, int DV, int NTN>
__device__ __forceinline__ void store_state(const floatx4 (&hacc)[NTN][DK / 16], float* sf, size_t head,
                                            int col, int lane)
{
    if (!sf) return;
    const int ln = lane & 15, lg = lane >> 4;
    float* sp = sf + head * DK * DV + col + ln;
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int mt = 0; mt < DK / 16; ++mt)
#pragma unroll
            for (int x = 0; x < 4; ++x) sp[(size_t)(16 * mt + 4 * lg + x) * DV + nt * 16] = hacc[nt][mt][x];
}

// (batch, query/key head, value head, column tile) of a workgroup; XCD-major placement when
// asked (workgroup ids are dealt to the 8 XCDs round-robin).
struct ChainId {
    int b, i, j, tile;
};

__device__ __forceinline__ ChainId chain_id(int ntile, int Hqk, int grp, int xcd_remap)
{
    int lid = blockIdx.x;
    if (xcd_remap) lid = (lid & 7) * (gridDim.x >> 3) + (lid >> 3);
    ChainId c;
    c.tile = lid % ntile;
    lid /= ntile;
    const int jj = lid % grp;
    lid /= grp;
    c.i = lid % Hqk;
    c.b = lid / Hqk;
    c.j = c.i * grp + jj;
    return c;
}

}  // namespace

// =======================================================================================
// Fused kernel
template <int DK, int DV, int BV>
__global__ __launch_bounds__(NTHR, 1) void chunk_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* s0, float* sf,  // may be the same buffer (in-place state update)
    bf16* __restrict__ o, int T_len, int Hqk, int Hv, int grp, float scale, int xcd_remap)
{
    using L = MLds<DK, BV>;
    constexpr int NTILE = DV / BV;
    constexpr int NCOL = BV / NCW;      // state columns per chain wave
    constexpr int NTN = NCOL / 16;      // 16-column tiles per chain wave
    constexpr int MT = DK / 16;         // 16-row tiles of the state
    constexpr int KB = DK / 32;         // 32-wide k blocks over dk
    constexpr int PK = CH * DK / 8 / (NPW * 64);   // 16-byte K (or Q) segments per prep lane
    constexpr int PV = CH * BV / 8 / (NPW * 64);   // 16-byte V segments per prep lane
    static_assert(NTN >= 1 && PK >= 1 && PV >= 1, "tile shape");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16* Vs = reinterpret_cast<bf16*>(smem + L::vs);
    op_t* Tm = reinterpret_cast<op_t*>(smem + L::tm);
    op_t* Aq = reinterpret_cast<op_t*>(smem + L::aq);
    float* Af = reinterpret_cast<float*>(smem + L::af);
    auto Kslot = [&](int s) { return reinterpret_cast<op_t*>(smem + L::ks + (size_t)s * L::kq_bytes); };
    auto Qslot = [&](int s) { return reinterpret_cast<op_t*>(smem + L::qs + (size_t)s * L::kq_bytes); };
    auto vslot = [&](int s) { return reinterpret_cast<float*>(smem + L::vec) + s * 8 * CH; };

    const ChainId id = chain_id(NTILE, Hqk, grp, xcd_remap);
    const int b = id.b, i = id.i, j = id.j;
    const int c0 = id.tile * BV;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15;      // MFMA column / row-in-tile index
    const int lg = lane >> 4;      // MFMA lane group
    const bool is_prep = w < NPW;
    const int pw = w;              // prep wave index (prep waves)
    const int cw = w - NPW;        // chain wave index (chain waves)
    const int ptid = tid;          // prep thread index 0..255 (prep waves)

    const int NT = (T_len + CH - 1) / CH;
    const size_t qk_row = (size_t)Hqk * DK;   // elements between consecutive tokens of q, k
    const size_t v_row = (size_t)Hv * DV;
    const bf16* qb = q + ((size_t)b * T_len * Hqk + i) * DK;
    const bf16* kb_ = k + ((size_t)b * T_len * Hqk + i) * DK;
    const bf16* vb = v + ((size_t)b * T_len * Hv + j) * DV + c0;
    bf16* ob = o + ((size_t)b * T_len * Hv + j) * DV + c0;
    const float* gb = g + (size_t)b * T_len * Hv + j;
    const float* bb = beta + (size_t)b * T_len * Hv + j;

    // =====================================================================================
    // prep-wave state: prefetch registers and the parts of T it keeps between phases
    bf16x8 rk[PK], rq[PK], rv[PV];
    float rg = 0.f, rb = 0.f;
    float tcol[16];
    opx4 tb = {};
    floatx4 t10 = {0.f, 0.f, 0.f, 0.f};

    // loads of chunk c's q, k, g, beta (rows past T clamped; zeroed when staged)
    auto load_kq = [&](int c) {
        const int t0 = c * CH, n = min(CH, T_len - t0);
#pragma unroll
        for (int p = 0; p < PK; ++p) {
            const int s = ptid + p * NPW * 64;
            const int r = min(s / (DK / 8), n - 1), c8 = (s % (DK / 8)) * 8;
            const size_t off = (size_t)(t0 + r) * qk_row + c8;
            rk[p] = *reinterpret_cast<const bf16x8*>(kb_ + off);
            rq[p] = *reinterpret_cast<const bf16x8*>(qb + off);
        }
        if (pw == 0) {
            const size_t off = (size_t)(t0 + min(lane, n - 1)) * Hv;
            rg = gb[off];
            rb = bb[off];
        }
    };
    auto load_v = [&](int c) {
        const int t0 = c * CH, n = min(CH, T_len - t0);
#pragma unroll
        for (int p = 0; p < PV; ++p) {
            const int s = ptid + p * NPW * 64;
            const int r = min(s / (BV / 8), n - 1), c8 = (s % (BV / 8)) * 8;
            rv[p] = *reinterpret_cast<const bf16x8*>(vb + (size_t)(t0 + r) * v_row + c8);
        }
    };
    // stage chunk c's q, k (float16) into slot c&1, and its per-row vectors (wave 0 scans g)
    auto stage_kq = [&](int c) {
        const int n = min(CH, T_len - c * CH);
        op_t* Ks = Kslot(c & 1);
        op_t* Qs = Qslot(c & 1);
#pragma unroll
        for (int p = 0; p < PK; ++p) {
            const int s = ptid + p * NPW * 64;
            const int r = s / (DK / 8), c8 = (s % (DK / 8)) * 8;
            const bool live = r < n;
            const opx8 kv = live ? to_op(rk[p]) : opx8{};
            const opx8 qv = live ? to_op(rq[p]) : opx8{};
            op_t* kr = Ks + r * L::KP;
            op_t* qr = Qs + r * L::KP;
            *reinterpret_cast<opx4*>(kr + pcol(c8)) = opx4{kv[0], kv[1], kv[2], kv[3]};
            *reinterpret_cast<opx4*>(kr + pcol(c8 + 4)) = opx4{kv[4], kv[5], kv[6], kv[7]};
            *reinterpret_cast<opx4*>(qr + pcol(c8)) = opx4{qv[0], qv[1], qv[2], qv[3]};
            *reinterpret_cast<opx4*>(qr + pcol(c8 + 4)) = opx4{qv[4], qv[5], qv[6], qv[7]};
        }
        if (pw == 0) {
            const float x = wave_cumsum(lane < n ? rg : 0.f, lane);
            const float bt = lane < n ? rb : 0.f;
            const float last = __shfl(x, 63, 64);
            const float eg = __expf(x);
            float* vs = vslot(c & 1);
            vs[V_G * CH + lane] = x;
            vs[V_B * CH + lane] = bt;
            vs[V_EG * CH + lane] = scale * eg;
            vs[V_BEG * CH + lane] = bt * eg;
            vs[V_ED * CH + lane] = __expf(last - x);
            vs[V_EC * CH + lane] = __expf(last);
        }
    };
    auto stage_v = [&](int c) {
        const int n = min(CH, T_len - c * CH);
#pragma unroll
        for (int p = 0; p < PV; ++p) {
            const int s = ptid + p * NPW * 64;
            const int r = s / (BV / 8), c8 = (s % (BV / 8)) * 8;
            *reinterpret_cast<bf16x8*>(Vs + r * L::VP + c8) = r < n ? rv[p] : bf16x8{};
        }
    };
    // NTL 16x16 tiles (ti[t], tj[t]) of K K^T (qk = false, into A^T) or Q K^T (qk = true, into
    // Aqk) of chunk c, with the decay mask and beta (or the scale) applied.  The k-block loop is
    // outermost so the tiles' MFMAs interleave instead of waiting on each other.
    auto gram_tiles = [&](int c, bool qk, const auto& ti, const auto& tj) {
        constexpr int NTL = sizeof(ti) / sizeof(ti[0]);
        const op_t* Ks = Kslot(c & 1);
        const op_t* Xs = qk ? Qslot(c & 1) : Ks;
        const float* vs = vslot(c & 1);
        opx8 af[NTL][KB], bf[NTL][KB];
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                af[t][kk] = frag(Xs, L::KP, 16 * ti[t] + ln, 32 * kk, lg);
                bf[t][kk] = frag(Ks, L::KP, 16 * tj[t] + ln, 32 * kk, lg);
            }
        floatx4 acc[NTL];
#pragma unroll
        for (int t = 0; t < NTL; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
            for (int t = 0; t < NTL; ++t) acc[t] = mfma32(af[t][kk], bf[t][kk], acc[t]);
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int cc = 16 * tj[t] + ln;
            const int r0 = 16 * ti[t] + 4 * lg;
            const float gcc = vs[V_G * CH + cc];
            const floatx4 gr = ld4s(vs + V_G * CH + r0);
            const floatx4 br = ld4s(vs + V_B * CH + r0);
            floatx4 out;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float gam = cc <= r0 + x ? __expf(gr[x] - gcc) : 0.f;
                out[x] = qk ? scale * gam * acc[t][x] : (cc < r0 + x ? br[x] * gam * acc[t][x] : 0.f);
            }
            if (qk) {
#pragma unroll
                for (int x = 0; x < 4; ++x) Aq[(r0 + x) * CP + pcol(cc)] = (op_t)out[x];
            } else {
                *reinterpret_cast<floatx4*>(Af + cc * AFP + r0) = out;   // A^T[cc][r0..r0+3]
            }
        }
    };
    if (is_prep) {
        // ================================================================= prep waves
        // zero the parts of T and Aqk that no chunk writes (upper blocks)
        for (int e = ptid; e < CH * CP; e += NPW * 64) {
            Tm[e] = (op_t)0.f;
            Aq[e] = (op_t)0.f;
        }
        load_kq(0);
        load_v(0);
        stage_kq(0);
        if (NT > 1) load_kq(1);
        lds_barrier();
        // iteration n: build chunk n + 1 while the chain waves carry chunk n
        for (int n = -1; n < NT; ++n) {
            const bool on = n + 1 < NT;
            const int c = n + 1;
            // interval 1: K K^T tiles of chunk c -> A (10 lower tiles: 3, 3, 2, 2 per wave)
            if (on) {
                if (pw == 0) gram_tiles(c, false, (const int[3]){3, 3, 3}, (const int[3]){0, 1, 2});
                else if (pw == 1) gram_tiles(c, false, (const int[3]){3, 2, 2}, (const int[3]){3, 0, 1});
                else if (pw == 2) gram_tiles(c, false, (const int[2]){2, 1}, (const int[2]){2, 0});
                else gram_tiles(c, false, (const int[2]){1, 0}, (const int[2]){1, 0});
            }
            lds_barrier();
            // interval 2: diagonal block pw of T, (I + A_ww)^{-1} column ln by right-looking
            // forward substitution in float32 (after row x is final, every later row takes its
            // update at once, so the dependent chain is 15 steps long); stage V of chunk c,
            // prefetch V of chunk c + 1
            if (on) {
                const float* At = Af + (16 * pw) * AFP + 16 * pw;   // At[x * AFP + r] = A_ww[r][x]
#pragma unroll
                for (int r = 0; r < 16; ++r) tcol[r] = (r == ln) ? 1.f : 0.f;
#pragma unroll
                for (int x = 0; x < 15; ++x) {
                    floatx4 col[4];
#pragma unroll
                    for (int q4 = (x + 1) / 4; q4 < 4; ++q4) col[q4] = ld4s(At + x * AFP + 4 * q4);
#pragma unroll
                    for (int r = x + 1; r < 16; ++r) tcol[r] = fmaf(-col[r / 4][r % 4], tcol[x], tcol[r]);
                }
                // lanes of group 0 write the column; each lane reads back its rows 4lg..4lg+3
                // (same wave, so the LDS writes are seen in order)
                op_t* tc = Tm + (16 * pw) * CP + pcol(16 * pw + ln);
                if (lg == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) tc[r * CP] = (op_t)tcol[r];
                }
#pragma unroll
                for (int x = 0; x < 4; ++x) tb[x] = tc[(4 * lg + x) * CP];
                stage_v(c);
                if (c + 1 < NT) load_v(c + 1);
            }
            lds_barrier();
            // interval 3: T_{w+1,w} = -T_{w+1,w+1} A_{w+1,w} T_ww for w in {0, 2};
            // Q K^T tiles of chunk c -> Aqk (10 lower tiles including the diagonal)
            if (on) {
                if (pw == 0 || pw == 2) {
                    const float* at = Af + (16 * pw + 4 * lg) * AFP + 16 * (pw + 1) + ln;
                    const opx4 aa = {(op_t)at[0], (op_t)at[AFP], (op_t)at[2 * AFP], (op_t)at[3 * AFP]};
                    const floatx4 p = mfma16(aa, tb, floatx4{0.f, 0.f, 0.f, 0.f});
                    const opx4 pb = {(op_t)p[0], (op_t)p[1], (op_t)p[2], (op_t)p[3]};
                    const opx4 td = *reinterpret_cast<const opx4*>(Tm + (16 * (pw + 1) + ln) * CP + pcol(16 * (pw + 1) + 4 * lg));
                    t10 = mfma16(td, pb, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        t10[x] = -t10[x];
                        Tm[(16 * (pw + 1) + 4 * lg + x) * CP + pcol(16 * pw + ln)] = (op_t)t10[x];
                    }
                }
                if (pw == 0) gram_tiles(c, true, (const int[3]){3, 3, 3}, (const int[3]){0, 1, 2});
                else if (pw == 1) gram_tiles(c, true, (const int[3]){3, 2, 2}, (const int[3]){3, 0, 1});
                else if (pw == 2) gram_tiles(c, true, (const int[2]){2, 1}, (const int[2]){2, 0});
                else gram_tiles(c, true, (const int[2]){1, 0}, (const int[2]){1, 0});
            }
            lds_barrier();
            // interval 4: T[32:64, 0:32] = -T_hi (A[32:64, 0:32] T_lo), waves 0, 1 (column tile pw);
            // stage q, k of chunk n + 2 into slot n&1 (the chain waves finished with it in
            // interval 3) and prefetch chunk n + 3
            if (on && pw < 2) {
                opx8 tlo;
                if (pw == 0) {
                    tlo = opx8{tb[0], tb[1], tb[2], tb[3], (op_t)t10[0], (op_t)t10[1], (op_t)t10[2], (op_t)t10[3]};
                } else {
                    tlo = opx8{(op_t)0.f, (op_t)0.f, (op_t)0.f, (op_t)0.f, tb[0], tb[1], tb[2], tb[3]};
                }
                floatx4 q1[2];
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const float* ac = Af + (4 * lg) * AFP + 32 + 16 * a + ln;
                    const opx8 aa = {(op_t)ac[0], (op_t)ac[AFP], (op_t)ac[2 * AFP], (op_t)ac[3 * AFP],
                                     (op_t)ac[16 * AFP], (op_t)ac[17 * AFP], (op_t)ac[18 * AFP], (op_t)ac[19 * AFP]};
                    q1[a] = mfma32(aa, tlo, floatx4{0.f, 0.f, 0.f, 0.f});
                }
                const opx8 q1b = pack_perm(q1[0], q1[1]);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const opx8 th = frag(Tm, CP, 32 + 16 * a + ln, 32, lg);
                    const floatx4 r = mfma32(th, q1b, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int x = 0; x < 4; ++x) Tm[(32 + 16 * a + 4 * lg + x) * CP + pcol(16 * pw + ln)] = (op_t)(-r[x]);
                }
            }
            if (n + 2 < NT) {
                stage_kq(n + 2);
                if (n + 3 < NT) load_kq(n + 3);
            }
            lds_barrier();
        }
    } else {
        // ================================================================= chain waves
        // the state columns in MFMA accumulator layout,
        // hacc[nt][mt][x] = h[16mt + 4lg + x][cw*NCOL + 16nt + ln]
        floatx4 hacc[NTN][MT];
        const size_t head = (size_t)b * Hv + j;
        load_state<DK, DV, NTN>(hacc, s0, head, c0 + cw * NCOL, lane);
        lds_barrier();
        // iteration n: carry chunk n (the prep waves build chunk n + 1 meanwhile); the same
        // four barriers per iteration as the prep waves
        for (int n = -1; n < NT; ++n) {
            if (n >= 0) {
                const int t0 = n * CH;
                chain_chunk<DK, BV, NCW>(hacc, Kslot(n & 1), Qslot(n & 1), Vs, Tm, Aq, vslot(n & 1),
                                         ob + (size_t)t0 * v_row, v_row, min(CH, T_len - t0), cw, lane,
                                         [] { lds_barrier(); });
            } else {
                lds_barrier();
                lds_barrier();
            }
            lds_barrier();
            // interval 4: nothing for the chain waves (the prep waves finish T and restage q, k)
            lds_barrier();
        }
        store_state<DK, DV, NTN>(hacc, sf, head, c0 + cw * NCOL, lane);
    }
}

// =======================================================================================
// Split path, kernel 1: everything of one chunk that does not depend on the state, for one
// value head, by one wave: the gate cumsum and vectors, A (K K^T with beta and the decay mask),
// T = (I + A)^{-1}, and Aqk (Q K^T with the decay mask and the scale).  Workgroups are ordered
// (batch, query/key head, chunk, value head of the group), so the group's value heads read the
// same q, k rows back to back.
template <int DK>
__global__ __launch_bounds__(64) void chunk_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, unsigned char* __restrict__ ws, int T_len, int Hqk, int Hv,
    int grp, int NT, float scale)
{
    constexpr int KB = DK / 32;
    __shared__ __attribute__((aligned(16))) float Af[CH * AFP];   // A^T, float32
    __shared__ __attribute__((aligned(16))) op_t Tm[CH * CP];     // T, column-permuted float16
    __shared__ __attribute__((aligned(16))) float pg[CH];         // gc
    __shared__ __attribute__((aligned(16))) float pb[CH];         // beta

    int lid = blockIdx.x;
    const int jj = lid % grp;
    lid /= grp;
    const int c = lid % NT;
    lid /= NT;
    const int i = lid % Hqk;
    const int b = lid / Hqk;
    const int j = i * grp + jj;
    const int lane = threadIdx.x, ln = lane & 15, lg = lane >> 4;
    const int t0 = c * CH, n = min(CH, T_len - t0);
    const size_t qk_row = (size_t)Hqk * DK;
    const bf16* kp = k + ((size_t)b * T_len + t0) * qk_row + (size_t)i * DK;
    const bf16* qp = q + ((size_t)b * T_len + t0) * qk_row + (size_t)i * DK;
    unsigned char* wc = ws + (((size_t)b * Hv + j) * NT + c) * WS_CHUNK;

    // Gram fragments straight from HBM (standard k order on both sides); rows past T are clamped
    // and masked below
    bf16x8 kf[4][KB], qf[4][KB];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const size_t off = (size_t)min(16 * mt + ln, n - 1) * qk_row + 32 * kk + 8 * lg;
            kf[mt][kk] = *reinterpret_cast<const bf16x8*>(kp + off);
            qf[mt][kk] = *reinterpret_cast<const bf16x8*>(qp + off);
        }
    // gates: cumsum and the per-row vectors
    {
        const size_t go = ((size_t)b * T_len + t0 + min(lane, n - 1)) * Hv + j;
        const float gl = g[go], bl = beta[go];
        const float x = wave_cumsum(lane < n ? gl : 0.f, lane);
        const float bt = lane < n ? bl : 0.f;
        const float last = __shfl(x, 63, 64);
        const float eg = __expf(x);
        pg[lane] = x;
        pb[lane] = bt;
        float* wv = reinterpret_cast<float*>(wc + WS_VEC);
        wv[V_G * CH + lane] = x;
        wv[V_B * CH + lane] = bt;
        wv[V_EG * CH + lane] = scale * eg;
        wv[V_BEG * CH + lane] = bt * eg;
        wv[V_ED * CH + lane] = __expf(last - x);
        wv[V_EC * CH + lane] = __expf(last);
    }
    // zero T's two stored strictly-upper 16x16 blocks (rows 0-15 x physical columns 0-31 and
    // rows 32-47 x 32-63; the diagonal blocks written next overwrite their half)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = 32 * p + (lane >> 2), c8 = 32 * p + 8 * (lane & 3);
        *reinterpret_cast<opx8*>(Tm + r * CP + c8) = opx8{};
    }
    wave_lds_fence();

    constexpr int TI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int TJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    // A = strictly-lower( beta_r exp(gc_r - gc_i) (k_r . k_i) ), stored transposed in float32
    {
        floatx4 acc[10];
#pragma unroll
        for (int t = 0; t < 10; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
            for (int t = 0; t < 10; ++t) acc[t] = mfma_bf(kf[TI[t]][kk], kf[TJ[t]][kk], acc[t]);
#pragma unroll
        for (int t = 0; t < 10; ++t) {
            const int cc = 16 * TJ[t] + ln;
            const int r0 = 16 * TI[t] + 4 * lg;
            const float gcc = pg[cc];
            const floatx4 gr = ld4s(pg + r0);
            const floatx4 br = ld4s(pb + r0);
            floatx4 out;
#pragma unroll
            for (int x = 0; x < 4; ++x) out[x] = cc < r0 + x ? br[x] * __expf(gr[x] - gcc) * acc[t][x] : 0.f;
            *reinterpret_cast<floatx4*>(Af + cc * AFP + r0) = out;   // A^T[cc][r0..r0+3]
        }
    }
    // Aqk = lower-incl( scale exp(gc_r - gc_i) (q_r . k_i) ), formed as K Q^T so that a lane
    // holds four consecutive columns of one row (one 8-byte store); rows past T are zero
    {
        op_t* wa = reinterpret_cast<op_t*>(wc + WS_AQ);
#pragma unroll
        for (int t = 0; t < 10; ++t) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) acc = mfma_bf(kf[TJ[t]][kk], qf[TI[t]][kk], acc);
            const int r = 16 * TI[t] + ln;
            const int i0 = 16 * TJ[t] + 4 * lg;
            const float gr = pg[r];
            const floatx4 gi = ld4s(pg + i0);
            opx4 out;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                out[x] = (op_t)((i0 + x <= r && r < n) ? scale * __expf(gr - gi[x]) * acc[x] : 0.f);
            *reinterpret_cast<opx4*>(wa + blk_off(r, pcol(i0))) = out;
        }
        // the stored strictly-upper blocks (0, 1) and (2, 3)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r = 32 * p + ln, i0 = 32 * p + 16 + 4 * lg;
            *reinterpret_cast<opx4*>(wa + blk_off(r, pcol(i0))) = opx4{};
        }
    }
    wave_lds_fence();
    // diagonal blocks of T: lane group lg inverts block lg, lane ln forms its column ln by
    // right-looking forward substitution in float32
    {
        const float* At = Af + (16 * lg) * AFP + 16 * lg;   // At[x * AFP + r] = A_ww[r][x]
        float tcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) tcol[r] = (r == ln) ? 1.f : 0.f;
#pragma unroll
        for (int x = 0; x < 15; ++x) {
            floatx4 col[4];
#pragma unroll
            for (int q4 = (x + 1) / 4; q4 < 4; ++q4) col[q4] = ld4s(At + x * AFP + 4 * q4);
#pragma unroll
            for (int r = x + 1; r < 16; ++r) tcol[r] = fmaf(-col[r / 4][r % 4], tcol[x], tcol[r]);
        }
        op_t* tc = Tm + (16 * lg) * CP + pcol(16 * lg + ln);
#pragma unroll
        for (int r = 0; r < 16; ++r) tc[r * CP] = (op_t)tcol[r];
    }
    wave_lds_fence();
    // T_{w+1,w} = -T_{w+1,w+1} A_{w+1,w} T_ww, w = 0 and 2
    {
        floatx4 t10[2];
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
            const int w = 2 * wi;
            const float* at = Af + (16 * w + 4 * lg) * AFP + 16 * (w + 1) + ln;
            const opx4 aa = {(op_t)at[0], (op_t)at[AFP], (op_t)at[2 * AFP], (op_t)at[3 * AFP]};
            const op_t* tw = Tm + (16 * w + 4 * lg) * CP + pcol(16 * w + ln);
            const opx4 tb = {tw[0], tw[CP], tw[2 * CP], tw[3 * CP]};
            const floatx4 p = mfma16(aa, tb, floatx4{0.f, 0.f, 0.f, 0.f});
            const opx4 pb = {(op_t)p[0], (op_t)p[1], (op_t)p[2], (op_t)p[3]};
            const opx4 td = *reinterpret_cast<const opx4*>(Tm + (16 * (w + 1) + ln) * CP + pcol(16 * (w + 1) + 4 * lg));
            t10[wi] = mfma16(td, pb, floatx4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
            const int w = 2 * wi;
#pragma unroll
            for (int x = 0; x < 4; ++x) Tm[(16 * (w + 1) + 4 * lg + x) * CP + pcol(16 * w + ln)] = (op_t)(-t10[wi][x]);
        }
    }
    wave_lds_fence();
    // T[32:64, 0:32] = -T_hi (A[32:64, 0:32] T_lo)
    {
        opx8 tlo[2], aa[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) tlo[p] = frag_kt(Tm, CP, p, 0, lane);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const float* ac = Af + (4 * lg) * AFP + 32 + 16 * a + ln;
            aa[a] = opx8{(op_t)ac[0], (op_t)ac[AFP], (op_t)ac[2 * AFP], (op_t)ac[3 * AFP],
                         (op_t)ac[16 * AFP], (op_t)ac[17 * AFP], (op_t)ac[18 * AFP], (op_t)ac[19 * AFP]};
        }
        floatx4 q1[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int p = 0; p < 2; ++p) q1[a][p] = mfma32(aa[a], tlo[p], floatx4{0.f, 0.f, 0.f, 0.f});
        floatx4 r[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const opx8 qb = pack_perm(q1[0][p], q1[1][p]);
#pragma unroll
            for (int a = 0; a < 2; ++a) r[a][p] = mfma32(frag(Tm, CP, 32 + 16 * a + ln, 32, lg), qb, floatx4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int x = 0; x < 4; ++x) Tm[(32 + 16 * a + 4 * lg + x) * CP + pcol(16 * p + ln)] = (op_t)(-r[a][p][x]);
    }
    wave_lds_fence();
    // T -> workspace (the stored blocks, 16 bytes per lane per step, consecutive)
    {
        op_t* wt = reinterpret_cast<op_t*>(wc + WS_T);
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            const int s = lane + 64 * p;
            const int r = s < 128 ? s >> 2 : 32 + ((s - 128) >> 3);
            const int c8 = s < 128 ? 8 * (s & 3) : 8 * ((s - 128) & 7);
            *reinterpret_cast<opx8*>(wt + 8 * s) = *reinterpret_cast<const opx8*>(Tm + r * CP + c8);
        }
    }
}

// Split path, kernel 2: the state pass.  One workgroup per (batch, value head, column tile of
// BV = 16 NW NTN columns): NW chain waves run chain_chunk on chunk n while NLW loader waves stage
// chunk n + 1 (q, k converted to column-permuted float16; V; T, Aqk and the gate vectors copied
// from the workspace) into the other half of a double-buffered LDS, and prefetch chunk n + 2 into
// registers.  One workgroup barrier per chunk.
template <int DK, int BV>
struct SLds {
    static constexpr int KP = DK + 8;
    static constexpr int VP = BV + 16;
    static constexpr size_t k = 0;                                   // K   [64][KP] f16
    static constexpr size_t q = k + (size_t)CH * KP * 2;             // Q   [64][KP] f16
    static constexpr size_t v = q + (size_t)CH * KP * 2;             // V   [64][VP] bf16
    static constexpr size_t t = v + (size_t)CH * VP * 2;             // T   [64][CP] f16
    static constexpr size_t a = t + (size_t)CH * CP * 2;             // Aqk [64][CP] f16
    static constexpr size_t e = a + (size_t)CH * CP * 2;             // [NVEC][64] f32
    static constexpr size_t slot = e + (size_t)NVEC * CH * 4;
    static constexpr size_t bytes = 2 * slot;
};

template <int DK, int DV, int NW, int NTN>
__global__ __launch_bounds__((NLW + NW) * 64, 1) void chunk_state_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const unsigned char* __restrict__ ws, const float* s0, float* sf, bf16* __restrict__ o,
    int T_len, int Hqk, int Hv, int grp, int xcd_remap)
{
    constexpr int BV = 16 * NW * NTN;
    using L = SLds<DK, BV>;
    constexpr int NTILE = DV / BV;
    constexpr int MT = DK / 16;
    constexpr int NLT = NLW * 64;                       // loader threads
    constexpr int RK = DK / 8;                          // 16-byte runs per K row
    constexpr int PK = CH * RK / NLT;                   // K (and Q) runs per loader lane
    constexpr int RV = BV / 8;                          // 16-byte runs per V row
    constexpr int PV = (CH * RV + NLT - 1) / NLT;       // V runs per loader lane
    constexpr int NWS = WS_CHUNK / 16;                  // 16-byte runs of a workspace chunk
    constexpr int PW = (NWS + NLT - 1) / NLT;
    static_assert(PK >= 1 && CH * RK % NLT == 0, "tile shape");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const ChainId id = chain_id(NTILE, Hqk, grp, xcd_remap);
    const int b = id.b, i = id.i, j = id.j;
    const int c0 = id.tile * BV;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int NT = (T_len + CH - 1) / CH;
    const size_t qk_row = (size_t)Hqk * DK;
    const size_t v_row = (size_t)Hv * DV;
    const size_t head = (size_t)b * Hv + j;

    if (w < NLW) {
        // ================================================================= loader waves
        const bf16* qb = q + ((size_t)b * T_len * Hqk + i) * DK;
        const bf16* kb_ = k + ((size_t)b * T_len * Hqk + i) * DK;
        const bf16* vb = v + ((size_t)b * T_len * Hv + j) * DV + c0;
        const unsigned char* wh = ws + head * NT * WS_CHUNK;
        bf16x4 rk[PK][2], rq[PK][2];
        bf16x8 rv[PV];
        floatx4 rw[PW];
        // K, Q run s of a chunk: row s / RK, physical 16-byte run m = s % RK of the column-
        // permuted row, i.e. logical columns 32(m/4) + 4(m%4) .. +3 and the same + 16
        auto load = [&](int c) {
            const int t0 = c * CH, n = min(CH, T_len - t0);
#pragma unroll
            for (int p = 0; p < PK; ++p) {
                const int s = tid + p * NLT;
                const int r = min(s / RK, n - 1), m = s % RK;
                const size_t off = (size_t)(t0 + r) * qk_row + 32 * (m >> 2) + 4 * (m & 3);
                rk[p][0] = *reinterpret_cast<const bf16x4*>(kb_ + off);
                rk[p][1] = *reinterpret_cast<const bf16x4*>(kb_ + off + 16);
                rq[p][0] = *reinterpret_cast<const bf16x4*>(qb + off);
                rq[p][1] = *reinterpret_cast<const bf16x4*>(qb + off + 16);
            }
#pragma unroll
            for (int p = 0; p < PV; ++p) {
                const int s = min(tid + p * NLT, CH * RV - 1);
                const int r = min(s / RV, n - 1), c8 = (s % RV) * 8;
                rv[p] = *reinterpret_cast<const bf16x8*>(vb + (size_t)(t0 + r) * v_row + c8);
            }
            const unsigned char* wcn = wh + (size_t)c * WS_CHUNK;
#pragma unroll
            for (int p = 0; p < PW; ++p) {
                const int s = min(tid + p * NLT, NWS - 1);
                rw[p] = *reinterpret_cast<const floatx4*>(wcn + 16 * s);
            }
        };
        auto stage = [&](int c) {
            const int n = min(CH, T_len - c * CH);
            unsigned char* sb = smem + (size_t)(c & 1) * L::slot;
            op_t* Ks = reinterpret_cast<op_t*>(sb + L::k);
            op_t* Qs = reinterpret_cast<op_t*>(sb + L::q);
            bf16* Vs = reinterpret_cast<bf16*>(sb + L::v);
#pragma unroll
            for (int p = 0; p < PK; ++p) {
                const int s = tid + p * NLT;
                const int r = s / RK, m = s % RK;
                const bool live = r < n;
                *reinterpret_cast<opx8*>(Ks + r * L::KP + 8 * m) = live ? to_op(rk[p][0], rk[p][1]) : opx8{};
                *reinterpret_cast<opx8*>(Qs + r * L::KP + 8 * m) = live ? to_op(rq[p][0], rq[p][1]) : opx8{};
            }
#pragma unroll
            for (int p = 0; p < PV; ++p) {
                const int s = tid + p * NLT;
                if (s < CH * RV) {
                    const int r = s / RV, c8 = (s % RV) * 8;
                    *reinterpret_cast<bf16x8*>(Vs + r * L::VP + c8) = r < n ? rv[p] : bf16x8{};
                }
            }
#pragma unroll
            for (int p = 0; p < PW; ++p) {
                const int s = tid + p * NLT;
                if (s < NWS) {
                    // workspace run s -> T (s < 384), Aqk (< 768) or the vectors
                    unsigned char* dst;
                    if (s < 768) {
                        const int u = s < 384 ? s : s - 384;
                        const int r = u < 128 ? u >> 2 : 32 + ((u - 128) >> 3);
                        const int c8 = u < 128 ? 8 * (u & 3) : 8 * ((u - 128) & 7);
                        dst = sb + (s < 384 ? L::t : L::a) + (size_t)(r * CP + c8) * 2;
                    } else {
                        dst = sb + L::e + (size_t)(s - 768) * 16;
                    }
                    *reinterpret_cast<floatx4*>(dst) = rw[p];
                }
            }
        };
        load(0);
        stage(0);
        if (NT > 1) load(1);
        lds_barrier();
        for (int n = 0; n < NT; ++n) {
            if (n + 1 < NT) {
                stage(n + 1);
                if (n + 2 < NT) load(n + 2);
            }
            lds_barrier();
        }
    } else {
        // ================================================================= chain waves
        const int cw = w - NLW;
        floatx4 hacc[NTN][MT];
        load_state<DK, DV, NTN>(hacc, s0, head, c0 + cw * 16 * NTN, lane);
        bf16* ob = o + ((size_t)b * T_len * Hv + j) * DV + c0;
        lds_barrier();
        for (int n = 0; n < NT; ++n) {
            const unsigned char* sb = smem + (size_t)(n & 1) * L::slot;
            const int t0 = n * CH;
            chain_chunk<DK, BV, NW>(hacc, reinterpret_cast<const op_t*>(sb + L::k),
                                    reinterpret_cast<const op_t*>(sb + L::q),
                                    reinterpret_cast<const bf16*>(sb + L::v),
                                    reinterpret_cast<const op_t*>(sb + L::t),
                                    reinterpret_cast<const op_t*>(sb + L::a),
                                    reinterpret_cast<const float*>(sb + L::e), ob + (size_t)t0 * v_row,
                                    v_row, min(CH, T_len - t0), cw, lane,
                                    [] { __builtin_amdgcn_sched_barrier(0); });
            lds_barrier();
        }
        store_state<DK, DV, NTN>(hacc, sf, head, c0 + cw * 16 * NTN, lane);
    }
}

namespace {

int env_int(const char* name, int dflt)
{
    const char* e = getenv(name);
    return e ? atoi(e) : dflt;
}

int choose_bv(const ChunkArgs& a)
{
    const int bv = env_int("GDN_MFMA_BV", 0);
    if ((bv == 64 || bv == 128) && a.dv % bv == 0) return bv;
    // Enough workgroups to cover the 256 compute units with whole-dv chains?  Otherwise split
    // the value columns (independent chains) into 64-wide tiles.
    const long chains = (long)a.B * a.Hv;
    if (a.dv == 64) return 64;
    return chains >= 192 ? 128 : 64;
}

// Column-tile width of the state pass: the narrowest tile that keeps the workgroup count within
// one per compute unit (each workgroup holds about 120-150 KB of LDS), so short-chain workloads
// spread over the chip; wide tiles when the chains alone fill it.
int choose_split_bv(const ChunkArgs& a)
{
    const int bv = env_int("GDN_SPLIT_BV", 0);
    if ((bv == 16 || bv == 32 || bv == 64 || bv == 128) && a.dv % bv == 0) return bv;
    const long chains = (long)a.B * a.Hv;
    for (int w = 16; w < a.dv; w *= 2)
        if (chains * (a.dv / w) <= 256) return w;
    return a.dv;
}

bool use_split(const ChunkArgs& a)
{
    if (const char* e = getenv("GDN_MFMA_PATH")) {
        if (!strcmp(e, "split")) return true;
        if (!strcmp(e, "fused")) return false;
    }
    return (long)a.B * a.Hv < 192;
}

template <int DK, int DV, int BV>
hipError_t launch_fused_t(const ChunkArgs& a, hipStream_t st)
{
    using L = MLds<DK, BV>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
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

template <int DK, int DV, int NW, int NTN>
hipError_t launch_state_t(const ChunkArgs& a, void* ws, hipStream_t st)
{
    constexpr int BV = 16 * NW * NTN;
    using L = SLds<DK, BV>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    auto kern = chunk_state_kernel<DK, DV, NW, NTN>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    const int grp = a.Hv / a.Hqk;
    const long nblk = (long)a.B * a.Hv * (DV / BV);
    const long per_xcd = nblk / 8;
    const int remap = (nblk % 8 == 0) && (per_xcd % ((long)grp * (DV / BV)) == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3((NLW + NW) * 64), L::bytes, st, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, (const unsigned char*)ws, a.s0, a.sf,
                       (bf16*)a.o, a.T, a.Hqk, a.Hv, grp, remap);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_split_t(const ChunkArgs& a, void* ws, hipStream_t st)
{
    const int grp = a.Hv / a.Hqk;
    const int NT = (a.T + CH - 1) / CH;
    const long nprep = (long)a.B * a.Hv * NT;
    hipLaunchKernelGGL(chunk_prep_kernel<DK>, dim3((unsigned)nprep), dim3(64), 0, st, (const bf16*)a.q,
                       (const bf16*)a.k, a.g, a.beta, (unsigned char*)ws, a.T, a.Hqk, a.Hv, grp, NT, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (choose_split_bv(a)) {
    case 16: return launch_state_t<DK, DV, 1, 1>(a, ws, st);
    case 32: return launch_state_t<DK, DV, 2, 1>(a, ws, st);
    case 64: return launch_state_t<DK, DV, 4, 1>(a, ws, st);
    default:
        if constexpr (DV >= 128) return launch_state_t<DK, DV, 4, 2>(a, ws, st);
        return hipErrorInvalidValue;
    }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a)
{
    if (getenv("GDN_DISABLE_MFMA")) return false;
    return a.dtype_bf16 && a.chunk == CH && (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128);
}

bool chunk_mfma_split(const ChunkArgs& a) { return chunk_mfma_supported(a) && use_split(a); }

size_t chunk_mfma_workspace_bytes(const ChunkArgs& a)
{
    if (!chunk_mfma_split(a)) return 0;
    const size_t NT = ((size_t)a.T + CH - 1) / CH;
    return (size_t)a.B * a.Hv * NT * WS_CHUNK;
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, void* ws, hipStream_t st)
{
    if (use_split(a)) {
        if (a.dk == 128 && a.dv == 128) return launch_split_t<128, 128>(a, ws, st);
        if (a.dk == 128 && a.dv == 64) return launch_split_t<128, 64>(a, ws, st);
        if (a.dk == 64 && a.dv == 128) return launch_split_t<64, 128>(a, ws, st);
        if (a.dk == 64 && a.dv == 64) return launch_split_t<64, 64>(a, ws, st);
        return hipErrorInvalidValue;
    }
    const int bv = choose_bv(a);
#define GDN_MFMA_CASE(DK_, DV_, BV_) \
    if (a.dk == DK_ && a.dv == DV_ && bv == BV_) return launch_fused_t<DK_, DV_, BV_>(a, st);
    GDN_MFMA_CASE(128, 128, 128) GDN_MFMA_CASE(128, 128, 64) GDN_MFMA_CASE(128, 64, 64)
    GDN_MFMA_CASE(64, 128, 128) GDN_MFMA_CASE(64, 128, 64) GDN_MFMA_CASE(64, 64, 64)
#undef GDN_MFMA_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
