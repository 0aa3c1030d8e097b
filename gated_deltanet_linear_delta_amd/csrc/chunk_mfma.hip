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
// Three ways to run it, all built from the same per-chunk state step (chain_delta, chain_out,
// chain_update) and, for the state-independent part, the same prep steps (prep_store_a,
// prep_solve_t, prep_store_aqk, prep_store_t):
//
// * Pipelined fused (chunk_pipe_kernel): one workgroup carries one (batch, value head, column
//   tile) chain through every chunk; nothing but the inputs, O and the states touches HBM.
//   Three prep waves build chunk n+1 (T, Aqk, the staged K, Q, V and the gate vectors), each a
//   whole part on its own, while the chain waves carry chunk n; one workgroup barrier per
//   chunk.  Suits many chains: the prep work runs beside the chain on the same compute unit.
// * Fused (chunk_mfma_kernel): the same split of work over four prep and four chain waves, with
//   four barriers per chunk; it carries the gated output norm.
// * Split (chunk_prep_kernel + chunk_state_kernel): the state-independent part of every chunk is
//   built first, all chunks at once (one wave per chunk and value head), into a workspace: T,
//   scaled Aqk and the gate vectors, 13.5 KB per chunk.  The state pass then only stages inputs
//   and runs the chain, with one barrier per chunk.  Suits few, long chains, where the
//   sequential per-chunk latency of the state pass is the whole cost.  Long rows whose state
//   pass leaves compute units idle run in pieces: one launch (chunk_overlap_kernel) per piece
//   carries its state pass on some compute units and the next piece's prep on the others.
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
//   q and k arrive as bf16 and convert exactly for unit-norm rows (components below 2^-14 become
//   float16 subnormals, an error of at most 2^-25); every other operand (v, the state, T, R,
//   Delta) is rounded once from float32, which bounds the magnitudes the inputs may reach.  The Gram
//   products of the split path take q and k as bf16 directly (exact products either way).
// * Row pitches are padded so that the 8- and 16-byte fragment reads of 8 consecutive rows
//   cover all 64 LDS banks once.
// * Workgroups of one query/key head (its value heads and column tiles read the same q, k) are
//   placed on the same XCD so that repeated reads of q and k hit that XCD's L2.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "gated_norm.hpp"
#include "launch.hpp"
#include "simt_chunk.hpp"

namespace gdn {

// Per-phase cycle stamps of workgroup 0 (lane 0 of each wave, chunks 2..33), compiled in only
// with -DGDN_PHASE_TRACE for performance analysis; gdn_phase_trace_read copies them out.
#ifdef GDN_PHASE_TRACE
__device__ long long gdn_phase_ts[16][32][8];
#define GDN_TRACE(n, k)                                                                   \
    do {                                                                                  \
        if (blockIdx.x == 0 && (threadIdx.x & 63) == 0 && (n) >= 2 && (n) < 34)            \
            gdn_phase_ts[threadIdx.x >> 6][(n) - 2][k] = __builtin_readcyclecounter();    \
    } while (0)
// the prep kernel's stamps go to the otherwise unused row 15
#define GDN_TRACE_PREP(k)                                                                 \
    do {                                                                                  \
        if (blockIdx.x == 0 && threadIdx.x == 0) gdn_phase_ts[15][0][k] = __builtin_readcyclecounter(); \
    } while (0)
#else
#define GDN_TRACE(n, k) \
    do {                \
    } while (0)
#define GDN_TRACE_PREP(k) \
    do {                  \
    } while (0)
#endif

// Index checks of the debug build (-DGDN_DEBUG, libgdn_debug.so): a failed check sets its bit in
// gdn_debug_flags with a vector atomic OR and the kernel goes on (every checked access is also
// clamped or guarded by the code around it), so a bad index shows up as a flag that
// gdn_debug_take_flags returns to the host, not as a fault.  Bits: 0 prep unit, 1 state-pass
// chain, 2 state-pass segment, 3 state-pass workspace chunk, 4 state-pass output token, 5
// pipelined-kernel chain and tokens, 6 combined launch, 7 fused-kernel chain and tokens.
#ifdef GDN_DEBUG
__device__ unsigned int gdn_debug_flags;
#define GDN_CHECK(cond, bit)                                                     \
    do {                                                                          \
        if (!(cond)) atomicOr(&gdn_debug_flags, 1u << (bit));                     \
    } while (0)
#else
#define GDN_CHECK(cond, bit) \
    do {                     \
    } while (0)
#endif

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

template <int DK, int BV, bool GATED = false>
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
    static constexpr int OP = BV + 8;            // element pitch of the staged output rows
    static constexpr size_t os = vec + (size_t)2 * 8 * CH * 4;      // O   [64][OP] bf16 (gated only)
    static constexpr size_t bytes = os + (GATED ? (size_t)CH * OP * 2 : 0);
    static_assert(os % 16 == 0, "16-byte aligned rows");
};

// per-chunk vectors (rows of 64 floats); the first four feed the state step, the fifth the output
constexpr int V_B = 0;     // beta
constexpr int V_BEG = 1;   // beta exp(gc)
constexpr int V_ED = 2;    // exp(gc_63 - gc)
constexpr int V_EC = 3;    // exp(gc_63) (every element)
constexpr int V_EG = 4;    // scale exp(gc)
constexpr int V_G = 5;     // gc (inclusive cumsum of g within the chunk)
constexpr int V_EN = 6;    // exp(-gc) (pipelined kernel only; used where the chunk's decay allows it)
constexpr int NVEC = 7;
// exp(gc_r - gc_c) = exp(gc_r) exp(-gc_c) with both factors normal floats when the chunk's total
// log-decay gc_63 is above this (exp(-60) and exp(60) are far inside float32's normal range);
// chunks that decay faster take the per-element exponentials
constexpr float GC_FACTOR_MIN = -60.f;

// Workspace of the split path, per (batch, value head, chunk), in two parts: what the state step
// reads (T, then the rows V_B..V_EC) and what the output step reads (Aqk, then the row V_EG).
// T and Aqk are float16 in MFMA fragment order: the six 16x32 operand blocks a product reads
// ((row tile, k block) = (0,0), (1,0), (2,0), (2,1), (3,0), (3,1)), each as 64 lanes x 16 bytes
// holding what frag() would read from the column-permuted matrix, so a wave loads a fragment
// with one coalesced 16-byte load.
constexpr int WS_T = 0;
constexpr int WS_CV = WS_T + 3072 * 2;
constexpr int WS_AQ = WS_CV + 4 * CH * 4;
constexpr int WS_EG = WS_AQ + 3072 * 2;
constexpr int WS_CHUNK = WS_EG + CH * 4;   // 13568 bytes
static_assert(WS_CHUNK % 16 == 0 && WS_AQ % 16 == 0, "workspace chunk");
// After the [B, Hv, NT] chunks: per (batch, query/key head, chunk) the q rows of the chunk as
// float16 B operands of the output product O^T = h^T Q^T, fragment (dk block kk, token tile ct)
// at (kk * 4 + ct) * 1 KB: lane (n, g) holds q[16ct + n][32kk + 4g .. +3] and [32kk + 16 + 4g .. +3].
template <int DK>
constexpr size_t ws_q_bytes() { return (size_t)CH * DK * 2; }

// fragment block of (row tile mt, k block cb), cb <= mt / 2
__device__ __forceinline__ constexpr int tblk(int mt, int cb) { return mt < 2 ? mt : 2 + 2 * (mt - 2) + cb; }
// element offset of (row r, physical column pc) of T or Aqk in the fragment-ordered layout
__device__ __forceinline__ int frag_off(int r, int pc)
{
    const int lane = (r & 15) + 16 * ((pc & 31) >> 3);
    return (tblk(r >> 4, pc >> 5) * 64 + lane) * 8 + (pc & 7);
}

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

// to_op, or zero where `keep` is false, without a branch (a select on the result's bits: the
// compiler had wrapped each conditional conversion in its own branch)
__device__ __forceinline__ opx8 to_op_or_zero(bf16x8 x, bool keep)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const unsigned int m = keep ? 0xffffffffu : 0u;
    return __builtin_bit_cast(opx8, __builtin_bit_cast(u32x4, to_op(x)) & m);
}

// bf16 -> float16 for one pair-run: x = logical columns c .. c+7, y = c+16 .. c+23 of a
// 32-column block (c = 8a) give the physical runs {c..c+3, c+16..c+19} and {c+4..c+7,
// c+20..c+23}.  Each 32-bit pair is widened to two float32 (shift / mask) and narrowed with one
// packed convert, three instructions per pair; exact for the unit-norm q, k rows (up to float16
// subnormals).
__device__ __forceinline__ unsigned int bf16x2_to_h2(unsigned int w)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const float lo = __builtin_bit_cast(float, w << 16);
    const float hi = __builtin_bit_cast(float, w & 0xffff0000u);
    return __builtin_bit_cast(unsigned int, h2{(_Float16)lo, (_Float16)hi});
}

__device__ __forceinline__ void bf16_pair_to_op(bf16x8 x, bf16x8 y, opx8& run0, opx8& run1)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 a = __builtin_bit_cast(u32x4, x), b = __builtin_bit_cast(u32x4, y);
    run0 = __builtin_bit_cast(opx8, u32x4{bf16x2_to_h2(a[0]), bf16x2_to_h2(a[1]), bf16x2_to_h2(b[0]), bf16x2_to_h2(b[1])});
    run1 = __builtin_bit_cast(opx8, u32x4{bf16x2_to_h2(a[2]), bf16x2_to_h2(a[3]), bf16x2_to_h2(b[2]), bf16x2_to_h2(b[3])});
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

// The same prefix sum with cross-lane moves only (no LDS round trip): Hillis-Steele steps of 1,
// 2, 4 and 8 inside each row of 16 lanes, then each row adds the running total of the rows before
// it (lane 15 into rows 1 and 3, then lane 31 into rows 2 and 3).  Lanes a move has no source
// for add zero.  The additions group differently from wave_cumsum's, so the two may differ in the
// last bit.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_take(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_cumsum_dpp(float x)
{
    x += dpp_take<0x111, 0xf>(x);   // row_shr:1
    x += dpp_take<0x112, 0xf>(x);   // row_shr:2
    x += dpp_take<0x114, 0xf>(x);   // row_shr:4
    x += dpp_take<0x118, 0xf>(x);   // row_shr:8
    x += dpp_take<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_take<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// =======================================================================================
// The per-chunk state step of one chain wave, in three phases.  The wave owns NTN 16-column
// tiles of the state; `Vc` and `ob` point at its first column (V tile in LDS, O row of the
// chunk's first token).  Inputs are the staged chunk in LDS: K, Q column-permuted float16
// [64][DK+8]; V bf16 with pitch VP; T, Aqk column-permuted float16 [64][CP]; the gate vectors.
//
// phase 3: h <- h + K^T (exp(gc_63 - gc) Delta) (h already carries its decay from phase 1).
// K^T fragments, 16 dk rows x 32 chunk positions each.
template <int DK>
__device__ __forceinline__ void load_kt(const op_t* Ks, int cb, int lane, opx8 (&akt)[DK / 16])
{
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt) akt[mt] = frag_kt(Ks, DK + 8, mt, 32 * cb, lane);
}

template <int DK, int NTN>
__device__ __forceinline__ void apply_kt(floatx4 (&hacc)[NTN][DK / 16], const opx8 (&akt)[DK / 16],
                                         const opx8 (&dtb)[NTN][2], int cb)
{
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) hacc[nt][mt] = mfma32(akt[mt], dtb[nt][cb], hacc[nt][mt]);
}

// phase 1: hb = h (float16, perm-K), X = K h, R = beta V - beta exp(gc) X, Delta = T R,
//          db = Delta and dtb = exp(gc_63 - gc) Delta (float16, perm-K); then h <- exp(gc_63) h
//          (the decay part of the update; phase 3 adds K^T dtb).
// Every product's A fragments are loaded before its MFMAs, behind a scheduling barrier, so the
// LDS latency is paid once per product rather than once per MFMA; with one tile per wave the V
// tile and the gate vectors are fetched up front too.
// CHDEC: the state decays by a factor per dk row (ech[m], one decay per key channel) instead of
// the scalar exp(gc_63).
// RV32: Vc holds beta V already formed, float32 and transposed (column c, row r at c * VP + r),
// so that R takes one multiply-add per element.
template <int DK, int NTN, int VP, bool KT = false, bool CHDEC = false, bool RV32 = false, typename TF>
__device__ __forceinline__ void chain_delta(floatx4 (&hacc)[NTN][DK / 16], const op_t* Ks,
                                            const void* Vc, TF&& tfrag, const float* vs, int lane,
                                            opx8 (&hb)[NTN][DK / 32], opx8 (&db)[NTN][2],
                                            opx8 (&dtb)[NTN][2], opx8 (*akt)[DK / 16] = nullptr,
                                            const float* ech = nullptr)
{
    constexpr int KP = DK + 8;
    constexpr int KB = DK / 32;
    constexpr int MT = DK / 16;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    // LDS reads complete in issue order and a wave can wait on at most 15 of them at a time, so
    // they are issued in the order of use, behind scheduling fences: K blocks 0 and 1 and T
    // first, then one more K block per k step of X = K h, then V and the row vectors.  With two
    // tiles per wave (twice the MFMAs per k block) K runs one block ahead and V and the vectors
    // follow X, which keeps the registers within budget.
    opx8 ak[KB][4];
    opx8 at[4][2];
    bf16x4 vv[NTN][4];
    floatx4 rv[NTN][4];
    floatx4 bt[4], beg[4], ed[2][2];
    auto load_k = [&](int kk) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) ak[kk][mt] = frag(Ks, KP, 16 * mt + ln, 32 * kk, lg);
    };
    // T fragments (row tile mt, k block cb) from the caller: LDS reads or registers
    auto load_t = [&] {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int cb = 0; cb <= mt / 2; ++cb) at[mt][cb] = tfrag(mt, cb);
    };
    // V rows 16mt+4lg..+3 of this lane's columns via the transposing read (or beta V as four
    // consecutive float32 rows); row vectors
    auto load_rows = [&] {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) {
                if constexpr (RV32)
                    rv[nt][mt] = ld4s(static_cast<const float*>(Vc) + (16 * nt + ln) * VP + 16 * mt + 4 * lg);
                else
                    vv[nt][mt] = __builtin_bit_cast(
                        bf16x4, ld_tr(static_cast<const bf16*>(Vc) + (16 * mt + 4 * lg + (ln >> 2)) * VP + 16 * nt + 4 * (ln & 3)));
            }
            if constexpr (!RV32) bt[mt] = ld4s(vs + V_B * CH + 16 * mt + 4 * lg);
            beg[mt] = ld4s(vs + V_BEG * CH + 16 * mt + 4 * lg);
        }
    };
    auto load_ed = [&] {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            ed[cb][0] = ld4s(vs + V_ED * CH + 32 * cb + 4 * lg);
            ed[cb][1] = ld4s(vs + V_ED * CH + 32 * cb + 16 + 4 * lg);
        }
    };
    constexpr bool EARLY = NTN == 1;
    constexpr int AHEAD = EARLY ? 2 : 1;
#pragma unroll
    for (int kk = 0; kk < AHEAD; ++kk) load_k(kk);
    if constexpr (EARLY) load_t();
    __builtin_amdgcn_sched_barrier(0);
    const float ec = vs[V_EC * CH];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) hb[nt][kk] = pack_perm(hacc[nt][2 * kk], hacc[nt][2 * kk + 1]);
    floatx4 X[NTN][4];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) X[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
        if (kk + AHEAD < KB) load_k(kk + AHEAD);
        if constexpr (EARLY) {
            if (kk + AHEAD == KB) load_rows();
            if (kk + AHEAD == KB + 1) load_ed();
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) X[nt][mt] = mfma32(ak[kk][mt], hb[nt][kk], X[nt][mt]);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!EARLY) {
        load_t();
        load_rows();
        load_ed();
    }
    // KT: the K^T fragments of phase 3, into the registers the K fragments free, their LDS
    // latency hidden behind the rest of this phase
    if constexpr (KT) {
        load_kt<DK>(Ks, 0, lane, akt[0]);
        load_kt<DK>(Ks, 1, lane, akt[1]);
    }
    // the decay of the state (its packed copy hb is already taken), while the MFMAs run
    if constexpr (CHDEC) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const floatx4 e4 = ld4s(ech + 16 * mt + 4 * lg);
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
                for (int x = 0; x < 4; ++x) hacc[nt][mt][x] *= e4[x];
        }
    } else {
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) hacc[nt][mt][x] *= ec;
    }
    opx8 rbf[NTN][2];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt) {
        floatx4 rr[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                if constexpr (RV32)
                    rr[mt][x] = rv[nt][mt][x] - beg[mt][x] * X[nt][mt][x];
                else
                    rr[mt][x] = bt[mt][x] * (float)vv[nt][mt][x] - beg[mt][x] * X[nt][mt][x];
            }
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

// phase 2: O = exp(gc) (Q h) + Aqk Delta (the scale is folded into both) -> HBM.  O is formed
// transposed, O^T = (h^T Q^T) diag(exp(gc)) + Delta^T Aqk^T: the same fragments with the operand
// roles swapped, and the accumulator layout then gives each lane four consecutive value columns
// of one token (one 8-byte store).  afrag(ct, cb) returns the Aqk fragment of row tile ct and
// k block cb (column-permuted row-major in LDS, or fragment order).
template <int DK, int NTN, typename AF>
__device__ __forceinline__ void chain_out(const opx8 (&hb)[NTN][DK / 32], const opx8 (&db)[NTN][2],
                                          const op_t* Qs, AF&& afrag, const float* egv, bf16* ob,
                                          size_t v_row, int nv, int lane)
{
    constexpr int KP = DK + 8;
    constexpr int KB = DK / 32;
    constexpr int AHEAD = NTN == 1 ? KB : 1;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    opx8 aqf[KB][4];
#pragma unroll
    for (int kk = 0; kk < AHEAD; ++kk)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) aqf[kk][ct] = frag(Qs, KP, 16 * ct + ln, 32 * kk, lg);
    opx8 aa[4][2];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int cb = 0; cb <= ct / 2; ++cb) aa[ct][cb] = afrag(ct, cb);
    float eg[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) eg[ct] = egv[16 * ct + ln];
    floatx4 OT[NTN][4];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) OT[nt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
        if (kk + AHEAD < KB) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) aqf[kk + AHEAD][ct] = frag(Qs, KP, 16 * ct + ln, 32 * (kk + AHEAD), lg);
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) OT[nt][ct] = mfma32(hb[nt][kk], aqf[kk][ct], OT[nt][ct]);
    }
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
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int tok = 16 * ct + ln;
        if (tok < nv) {
            bf16* op = ob + (size_t)tok * v_row + 4 * lg;
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) {
                const bf16x4 ov = {(bf16)OT[nt][ct][0], (bf16)OT[nt][ct][1], (bf16)OT[nt][ct][2],
                                   (bf16)OT[nt][ct][3]};
                *reinterpret_cast<bf16x4*>(op + 16 * nt) = ov;
            }
        }
    }
}

// phase 3 with its own fragment loads
template <int DK, int NTN>
__device__ __forceinline__ void chain_update(floatx4 (&hacc)[NTN][DK / 16], const op_t* Ks,
                                             const opx8 (&dtb)[NTN][2], int lane)
{
    // one tile: every K^T fragment up front; two tiles: the second k block during the first's MFMAs
    opx8 akt[2][DK / 16];
    load_kt<DK>(Ks, 0, lane, akt[0]);
    if constexpr (NTN == 1) load_kt<DK>(Ks, 1, lane, akt[1]);
    apply_kt<DK, NTN>(hacc, akt[0], dtb, 0);
    if constexpr (NTN != 1) load_kt<DK>(Ks, 1, lane, akt[1]);
    apply_kt<DK, NTN>(hacc, akt[1], dtb, 1);
}

// The three phases in one wave (column group cw of NW), with `sync` between them: a workgroup
// barrier in the fused kernel (where other waves write LDS meanwhile), a scheduling fence in the
// state pass.
template <int DK, int BV, int NW, typename Sync>
__device__ __forceinline__ void chain_chunk(floatx4 (&hacc)[BV / NW / 16][DK / 16], const op_t* Ks,
                                            const op_t* Qs, const bf16* Vs, const op_t* Tm,
                                            const op_t* Aq, const float* vs, bf16* ob, size_t v_row,
                                            int nv, int cw, int lane, Sync&& sync)
{
    constexpr int NCOL = BV / NW;
    constexpr int NTN = NCOL / 16;
    opx8 hb[NTN][DK / 32], db[NTN][2], dtb[NTN][2];
    const int ln = lane & 15, lg = lane >> 4;
    chain_delta<DK, NTN, BV + 16>(hacc, Ks, Vs + cw * NCOL,
                                  [&](int mt, int cb) { return frag(Tm, CP, 16 * mt + ln, 32 * cb, lg); }, vs,
                                  lane, hb, db, dtb);
    sync();
    chain_out<DK, NTN>(hb, db, Qs, [&](int ct, int cb) { return frag(Aq, CP, 16 * ct + ln, 32 * cb, lg); },
                       vs + V_EG * CH, ob + cw * NCOL, v_row, nv, lane);
    sync();
    chain_update<DK, NTN>(hacc, Ks, dtb, lane);
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

// Final state = initial state (zeros when s0 is null) for `ncols` columns from `col`: an empty
// packed sequence.  Plain element copies, one wave.
template <int DK, int DV>
__device__ __forceinline__ void copy_state_cols(const float* s0, float* sf, size_t head, int col, int ncols, int lane)
{
    if (!sf) return;
    for (int e = lane; e < DK * ncols; e += 64) {
        const size_t off = head * DK * DV + (size_t)(e / ncols) * DV + col + e % ncols;
        sf[off] = s0 ? s0[off] : 0.f;
    }
}

// (batch, query/key head, value head, column tile) of a workgroup; XCD-major placement when
// asked (workgroup ids are dealt to the 8 XCDs round-robin).
struct ChainId {
    int b, i, j, tile;
};

// First token and length of batch row b: uniform rows of T_len tokens, or (cu set) packed
// sequences with offsets cu[0..N] into total tokens, each at most T_len long.  Offsets are
// clamped into [0, total] and lengths into [0, T_len], so no access leaves the tensors whatever
// cu holds.
struct SeqSpan {
    size_t tok0;
    int len;
};
__device__ __forceinline__ SeqSpan seq_span(const int* cu, int b, int T_len, int total)
{
    if (!cu) return SeqSpan{(size_t)b * T_len, T_len};
    const int s = min(max(cu[b], 0), total);
    const int e = min(max(cu[b + 1], s), total);
    return SeqSpan{(size_t)s, min(e - s, T_len)};
}

__device__ __forceinline__ ChainId chain_id_of(int lid, int nblk, int ntile, int Hqk, int grp, int xcd_remap)
{
    if (xcd_remap) lid = (lid & 7) * (nblk >> 3) + (lid >> 3);
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

__device__ __forceinline__ ChainId chain_id(int ntile, int Hqk, int grp, int xcd_remap)
{
    return chain_id_of(blockIdx.x, gridDim.x, ntile, Hqk, grp, xcd_remap);
}

}  // namespace

// =======================================================================================
// Fused kernel.  GATED (whole value heads per workgroup, BV == DV): the output is the layer's
// gated RMSNorm y = O / sqrt(mean(O^2) + eps) * w * silu(z) instead of O.  The chain waves stage
// O of a chunk in LDS in the output phase and, in the interval the prep waves spend finishing T,
// normalise 16 whole token rows each and write y; O itself never reaches HBM.
template <int DK, int DV, int BV, bool GATED, bool VARLEN>
__global__ __launch_bounds__(NTHR, 1) void chunk_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* s0, float* sf,  // may be the same buffer (in-place state update)
    bf16* o,                     // O, or y when gated (y may be z exactly)
    const bf16* z, const float* __restrict__ nw, int nw_stride, float eps,
    int T_max, int Hqk, int Hv, int grp, float scale, int xcd_remap, const int* cu, int total)
{
    using L = MLds<DK, BV, GATED>;
    static_assert(!GATED || BV == DV, "the gated epilogue needs whole value heads");
    static_assert(CH == 16 * NCW, "16 output rows per chain wave in the gated epilogue");
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
    GDN_CHECK((int)gridDim.x % (Hv * NTILE) == 0 && b < (int)gridDim.x / (Hv * NTILE) && i < Hqk && j < Hv &&
                  j / grp == i, 7);

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15;      // MFMA column / row-in-tile index
    const int lg = lane >> 4;      // MFMA lane group
    const bool is_prep = w < NPW;
    const int pw = w;              // prep wave index (prep waves)
    const int cw = w - NPW;        // chain wave index (chain waves)
    const int ptid = tid;          // prep thread index 0..255 (prep waves)

    const SeqSpan sq = VARLEN ? seq_span(cu, b, T_max, total) : SeqSpan{(size_t)b * T_max, T_max};
    const int T_len = sq.len;
    if (VARLEN && T_len == 0) {
        // an empty sequence: the final state is the initial one (every wave leaves here, before
        // any barrier)
        if (!is_prep) copy_state_cols<DK, DV>(s0, sf, (size_t)b * Hv + j, c0 + cw * NCOL, NCOL, lane);
        return;
    }
    const int NT = (T_len + CH - 1) / CH;
    const size_t qk_row = (size_t)Hqk * DK;   // elements between consecutive tokens of q, k
    const size_t v_row = (size_t)Hv * DV;
    const bf16* qb = q + (sq.tok0 * Hqk + i) * DK;
    const bf16* kb_ = k + (sq.tok0 * Hqk + i) * DK;
    const bf16* vb = v + (sq.tok0 * Hv + j) * DV + c0;
    bf16* ob = o + (sq.tok0 * Hv + j) * DV + c0;
    const float* gb = g + sq.tok0 * Hv + j;
    const float* bb = beta + sq.tok0 * Hv + j;

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
            rg = log_decay(gb[off]);
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
        // gated epilogue: a row of O is DV / 8 lanes of 8 consecutive columns; a pass covers
        // 64 / (DV / 8) rows and a chain wave owns rows 16 cw .. 16 cw + 15
        constexpr int ECB = DV / 8;
        constexpr int ERP = 64 / ECB;
        constexpr int EPASS = 16 / ERP;
        const int ecb = lane % ECB, esub = lane / ECB;
        bf16* Os = reinterpret_cast<bf16*>(smem + L::os);
        const bf16* zb = z + (sq.tok0 * Hv + j) * DV + 8 * ecb;
        bf16* yb = o + (sq.tok0 * Hv + j) * DV + 8 * ecb;
        bf16x8 zr[EPASS];
        float wc[8];
        if constexpr (GATED) {
#pragma unroll
            for (int e = 0; e < 8; ++e) wc[e] = nw[(size_t)j * nw_stride + 8 * ecb + e];
        }
        lds_barrier();
        // iteration -1: the prep waves build chunk 0
        for (int x = 0; x < 4; ++x) lds_barrier();
        // iteration n: carry chunk n (the prep waves build chunk n + 1 meanwhile); the same
        // four barriers per iteration as the prep waves
        for (int n = 0; n < NT; ++n) {
            const int t0 = n * CH;
            const int nv = min(CH, T_len - t0);
            if constexpr (GATED) {
                chain_chunk<DK, BV, NCW>(hacc, Kslot(n & 1), Qslot(n & 1), Vs, Tm, Aq, vslot(n & 1),
                                         Os, (size_t)L::OP, CH, cw, lane, [] { lds_barrier(); });
                // this chunk's gate rows, loaded now to arrive during the barrier wait (rows past
                // the sequence clamped to its last row and not stored)
#pragma unroll
                for (int p = 0; p < EPASS; ++p) {
                    const int tok = 16 * cw + ERP * p + esub;
                    zr[p] = *reinterpret_cast<const bf16x8*>(zb + (size_t)(t0 + min(tok, nv - 1)) * v_row);
                }
                lds_barrier();
                // interval 4: y of chunk n from the staged O rows (written by all chain waves
                // before the last two barriers)
#pragma unroll
                for (int p = 0; p < EPASS; ++p) {
                    const int tok = 16 * cw + ERP * p + esub;
                    const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(Os + tok * L::OP + 8 * ecb);
                    float ov[8], zv[8], yv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        ov[e] = (float)o8[e];
                        zv[e] = (float)zr[p][e];
                    }
                    gated_norm_lane<8>(ov, zv, wc, ECB, 1.f / (float)DV, eps, yv);
                    if (tok < nv) {
                        bf16x8 y8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) y8[e] = (bf16)yv[e];
                        *reinterpret_cast<bf16x8*>(yb + (size_t)(t0 + tok) * v_row) = y8;
                    }
                }
                lds_barrier();
            } else {
                chain_chunk<DK, BV, NCW>(hacc, Kslot(n & 1), Qslot(n & 1), Vs, Tm, Aq, vslot(n & 1),
                                         ob + (size_t)t0 * v_row, v_row, nv, cw, lane, [] { lds_barrier(); });
                lds_barrier();
                // interval 4: nothing for the chain waves (the prep waves finish T and restage q, k)
                lds_barrier();
            }
        }
        store_state<DK, DV, NTN>(hacc, sf, head, c0 + cw * NCOL, lane);
    }
}

// =======================================================================================
// Pieces of the per-chunk prep (the state-independent part of a chunk) shared by the prep
// kernel of the split path and the T and Aqk waves of the fused kernel.  Inputs are the raw
// lower Gram tiles (TI, TJ) of K K^T (gk) and K Q^T (gq, Aqk transposed) in accumulator layout and
// the gate values this lane's tiles need: gc and beta of rows 16t + 4lg .. +3 (g4, b4) and gc of
// row 16t + ln (g1), t = 0..3.
constexpr int TI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
constexpr int TJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
// A in two parts: the diagonal 16x16 blocks transposed in float32 for the solve (Ad[w][x][r] =
// A_ww[r][x]), the off-diagonal blocks the merges read transposed in float16 (Ah[i][r - 16] =
// A[r][i], i < 48 <= r + 16); T assembled column-permuted in float16 (Tm)
constexpr int ADP = 20, AHP = 56;
constexpr int PREP_AD = 4 * 16 * ADP;   // floats
constexpr int PREP_AH = 48 * AHP;       // halves
constexpr int PREP_TM = CH * CP;        // halves

// A = strictly-lower( beta_r exp(gc_r - gc_i) (k_r . k_i) )
__device__ __forceinline__ void prep_store_a(const floatx4 (&gk)[10], const floatx4 (&g4)[4], const floatx4 (&b4)[4],
                                             const float (&g1)[4], float* Ad, op_t* Ah, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int t = 0; t < 10; ++t) {
        const int cc = 16 * TJ[t] + ln;
        const int r0 = 16 * TI[t] + 4 * lg;
        const float gcc = g1[TJ[t]];
        const floatx4 gr = g4[TI[t]];
        const floatx4 br = b4[TI[t]];
        floatx4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = cc < r0 + e ? br[e] * __expf(gr[e] - gcc) * gk[t][e] : 0.f;
        if (TI[t] == TJ[t])
            *reinterpret_cast<floatx4*>(Ad + (16 * TI[t] + ln) * ADP + 4 * lg) = out;
        else
            *reinterpret_cast<opx4*>(Ah + cc * AHP + r0 - 16) = opx4{(op_t)out[0], (op_t)out[1], (op_t)out[2], (op_t)out[3]};
    }
}

// Aqk = lower-incl( scale exp(gc_r - gc_i) (q_r . k_i) ), rows at or past n zero, into `wa` in
// fragment order (the six stored blocks, their strictly-upper parts zero)
__device__ __forceinline__ void prep_store_aqk(const floatx4 (&gq)[10], const floatx4 (&g4)[4], const float (&g1)[4],
                                               float scale, int n, op_t* wa, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int t = 0; t < 10; ++t) {
        const int r = 16 * TI[t] + ln;
        const int i0 = 16 * TJ[t] + 4 * lg;
        const float gr = g1[TI[t]];
        const floatx4 gi = g4[TJ[t]];
        opx4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (op_t)((i0 + e <= r && r < n) ? scale * __expf(gr - gi[e]) * gq[t][e] : 0.f);
        *reinterpret_cast<opx4*>(wa + frag_off(r, pcol(i0))) = out;
    }
    // the stored strictly-upper blocks (0, 1) and (2, 3)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = 32 * p + ln, i0 = 32 * p + 16 + 4 * lg;
        *reinterpret_cast<opx4*>(wa + frag_off(r, pcol(i0))) = opx4{};
    }
}

// prep_store_a with the decay factorised: A[r][c] = (beta_r exp(gc_r)) exp(-gc_c) (k_r . k_c);
// br4 = beta exp(gc) of the lane's rows, en1 = exp(-gc) of its columns
__device__ __forceinline__ void prep_store_a_fac(const floatx4 (&gk)[10], const floatx4 (&br4)[4], const float (&en1)[4],
                                                 float* Ad, op_t* Ah, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int t = 0; t < 10; ++t) {
        const int cc = 16 * TJ[t] + ln;
        const int r0 = 16 * TI[t] + 4 * lg;
        const float ec = en1[TJ[t]];
        const floatx4 br = br4[TI[t]];
        floatx4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = cc < r0 + e ? br[e] * ec * gk[t][e] : 0.f;
        if (TI[t] == TJ[t])
            *reinterpret_cast<floatx4*>(Ad + (16 * TI[t] + ln) * ADP + 4 * lg) = out;
        else
            *reinterpret_cast<opx4*>(Ah + cc * AHP + r0 - 16) = opx4{(op_t)out[0], (op_t)out[1], (op_t)out[2], (op_t)out[3]};
    }
}

// prep_store_aqk with the decay factorised: Aqk[r][i] = (scale exp(gc_r)) exp(-gc_i) (q_r . k_i);
// eg1 = scale exp(gc) of the lane's rows r, en4 = exp(-gc) of its columns i
__device__ __forceinline__ void prep_store_aqk_fac(const floatx4 (&gq)[10], const float (&eg1)[4], const floatx4 (&en4)[4],
                                                   int n, op_t* wa, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int t = 0; t < 10; ++t) {
        const int r = 16 * TI[t] + ln;
        const int i0 = 16 * TJ[t] + 4 * lg;
        const float er = eg1[TI[t]];
        const floatx4 ei = en4[TJ[t]];
        opx4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (op_t)((i0 + e <= r && r < n) ? er * ei[e] * gq[t][e] : 0.f);
        *reinterpret_cast<opx4*>(wa + frag_off(r, pcol(i0))) = out;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = 32 * p + ln, i0 = 32 * p + 16 + 4 * lg;
        *reinterpret_cast<opx4*>(wa + frag_off(r, pcol(i0))) = opx4{};
    }
}

// T = (I + A)^{-1} into Tm (column-permuted float16; its strictly-upper blocks (0, 1) and
// (2, 3) must hold zeros): the four diagonal blocks by forward substitution in float32, then
// T_{w+1,w} = -T_{w+1,w+1} A_{w+1,w} T_ww (w = 0, 2) and T[32:64, 0:32] = -T_hi (A[32:64, 0:32] T_lo)
// on the matrix cores.  One wave; A written by the same wave before.
__device__ __forceinline__ void prep_solve_t(const float* Ad, const op_t* Ah, op_t* Tm, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
    wave_lds_fence();
    // the A operands of the merges (independent of T), fetched before the solve
    opx4 a10[2];
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) {
        const op_t* at = Ah + (32 * wi + 4 * lg) * AHP + 32 * wi + ln;   // A[16(w+1)+ln][16w+4lg+j]
        a10[wi] = opx4{at[0], at[AHP], at[2 * AHP], at[3 * AHP]};
    }
    opx8 a2[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const op_t* ac = Ah + (4 * lg) * AHP + 16 + 16 * a + ln;   // A[32+16a+ln][k], perm-K
        a2[a] = opx8{ac[0], ac[AHP], ac[2 * AHP], ac[3 * AHP], ac[16 * AHP], ac[17 * AHP], ac[18 * AHP], ac[19 * AHP]};
    }
    // diagonal blocks of T: lane group lg inverts block lg, lane ln forms its column ln by
    // right-looking forward substitution in float32; each step's column of A is fetched two
    // steps ahead
    {
        const float* At = Ad + (16 * lg) * ADP;   // At[x * ADP + r] = A_ww[r][x]
        float tcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) tcol[r] = (r == ln) ? 1.f : 0.f;
        floatx4 col[3][4];   // rotating: step x uses slot x % 3
        auto fetch = [&](int x) {
#pragma unroll
            for (int q4 = (x + 1) / 4; q4 < 4; ++q4) col[x % 3][q4] = ld4s(At + x * ADP + 4 * q4);
        };
        fetch(0);
        fetch(1);
#pragma unroll
        for (int x = 0; x < 15; ++x) {
            if (x + 2 < 15) fetch(x + 2);
#pragma unroll
            for (int r = x + 1; r < 16; ++r) tcol[r] = fmaf(-col[x % 3][r / 4][r % 4], tcol[x], tcol[r]);
        }
        op_t* tc = Tm + (16 * lg) * CP + pcol(16 * lg + ln);
#pragma unroll
        for (int r = 0; r < 16; ++r) tc[r * CP] = (op_t)tcol[r];
    }
    GDN_TRACE_PREP(3);
    wave_lds_fence();
    // T_{w+1,w} = -T_{w+1,w+1} A_{w+1,w} T_ww, w = 0 and 2
    {
        floatx4 t10[2];
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
            const int w = 2 * wi;
            const op_t* tw = Tm + (16 * w + 4 * lg) * CP + pcol(16 * w + ln);
            const opx4 tb = {tw[0], tw[CP], tw[2 * CP], tw[3 * CP]};
            const opx4 td = *reinterpret_cast<const opx4*>(Tm + (16 * (w + 1) + ln) * CP + pcol(16 * (w + 1) + 4 * lg));
            const floatx4 p = mfma16(a10[wi], tb, floatx4{0.f, 0.f, 0.f, 0.f});
            const opx4 pb2 = {(op_t)p[0], (op_t)p[1], (op_t)p[2], (op_t)p[3]};
            t10[wi] = mfma16(td, pb2, floatx4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
            const int w = 2 * wi;
#pragma unroll
            for (int e = 0; e < 4; ++e) Tm[(16 * (w + 1) + 4 * lg + e) * CP + pcol(16 * w + ln)] = (op_t)(-t10[wi][e]);
        }
    }
    wave_lds_fence();
    // T[32:64, 0:32] = -T_hi (A[32:64, 0:32] T_lo)
    {
        opx8 tlo[2], th[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) tlo[p] = frag_kt(Tm, CP, p, 0, lane);
#pragma unroll
        for (int a = 0; a < 2; ++a) th[a] = frag(Tm, CP, 32 + 16 * a + ln, 32, lg);
        floatx4 q1[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int p = 0; p < 2; ++p) q1[a][p] = mfma32(a2[a], tlo[p], floatx4{0.f, 0.f, 0.f, 0.f});
        floatx4 r[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const opx8 qb = pack_perm(q1[0][p], q1[1][p]);
#pragma unroll
            for (int a = 0; a < 2; ++a) r[a][p] = mfma32(th[a], qb, floatx4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) Tm[(32 + 16 * a + 4 * lg + e) * CP + pcol(16 * p + ln)] = (op_t)(-r[a][p][e]);
    }
}

// T from Tm into `wt` in fragment order: the six 16x32 blocks a product reads, 64 lanes x 16 bytes
__device__ __forceinline__ void prep_store_t(const op_t* Tm, opx8* wt, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
    constexpr int BM[6] = {0, 1, 2, 2, 3, 3}, BC[6] = {0, 0, 0, 1, 0, 1};
#pragma unroll
    for (int bk = 0; bk < 6; ++bk) wt[bk * 64 + lane] = frag(Tm, CP, 16 * BM[bk] + ln, 32 * BC[bk], lg);
}

// Zero the strictly-upper blocks (0, 1) and (2, 3) of T that Tm stores (rows 0-15 x physical
// columns 0-31 and rows 32-47 x 32-63; the diagonal blocks written later overwrite their half).
__device__ __forceinline__ void prep_zero_t_upper(op_t* Tm, int lane)
{
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = 32 * p + (lane >> 2), c8 = 32 * p + 8 * (lane & 3);
        *reinterpret_cast<opx8*>(Tm + r * CP + c8) = opx8{};
    }
}

// =======================================================================================
// Split path, kernel 1: everything of one chunk that does not depend on the state, by one wave
// per (batch, query/key head, chunk).  The raw K K^T and K Q^T products are formed once (q, k
// are shared by the query/key head's group of value heads); then for each value head of the
// group in turn: the gate cumsum and vectors, A (beta and the decay mask), T = (I + A)^{-1}, and
// Aqk (the decay mask and the scale), all into the workspace.
// LDS of one prep wave: A and T (prep_store_a, prep_solve_t), gc and beta; about 20 KB
struct PrepLds {
    static constexpr size_t ad = 0;                                  // f32 [PREP_AD]
    static constexpr size_t ah = ad + (size_t)PREP_AD * 4;           // f16 [PREP_AH]
    static constexpr size_t tm = ah + (size_t)PREP_AH * 2;           // T, column-permuted f16
    static constexpr size_t pg = tm + (size_t)PREP_TM * 2;           // gc [64] f32
    static constexpr size_t pb = pg + (size_t)CH * 4;                // beta [64] f32
    static constexpr size_t bytes = pb + (size_t)CH * 4;
    static_assert(ah % 16 == 0 && tm % 16 == 0 && pg % 16 == 0 && bytes % 16 == 0, "16-byte aligned parts");
};

// One unit of the prep work, run by one wave on its own: (batch row b, chunk c, query/key head i)
// from unit index u over the chunks c_base .. c_base + NTg - 1, with the head fastest.  Its
// results go to chunk c of the workspace (NT chunks per row).
template <int DK, bool VARLEN>
__device__ __forceinline__ void prep_unit(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                          const float* __restrict__ g, const float* __restrict__ beta,
                                          unsigned char* __restrict__ ws, unsigned char* __restrict__ wsq,
                                          int T_max, int Hqk, int Hv, int grp, int NT, float scale,
                                          const int* cu, int total, int u, int c_base, int NTg,
                                          unsigned char* lds)
{
    constexpr int KB = DK / 32;
    float* Ad = reinterpret_cast<float*>(lds + PrepLds::ad);
    op_t* Ah = reinterpret_cast<op_t*>(lds + PrepLds::ah);
    op_t* Tm = reinterpret_cast<op_t*>(lds + PrepLds::tm);
    float* pg = reinterpret_cast<float*>(lds + PrepLds::pg);
    float* pb = reinterpret_cast<float*>(lds + PrepLds::pb);
    const int i = u % Hqk;
    u /= Hqk;
    const int c = c_base + u % NTg;
    const int b = u / NTg;
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    GDN_CHECK(u >= 0 && c >= 0 && c < NT && NTg >= 1 && c_base + NTg <= NT && grp * Hqk == Hv, 0);
    const SeqSpan sq = VARLEN ? seq_span(cu, b, T_max, total) : SeqSpan{(size_t)b * T_max, T_max};
    const int t0 = c * CH;
    if (VARLEN && t0 >= sq.len) return;   // past this sequence's last chunk
    const int n = min(CH, sq.len - t0);
    const size_t qk_row = (size_t)Hqk * DK;
    const bf16* kp = k + (sq.tok0 + t0) * qk_row + (size_t)i * DK;
    const bf16* qp = q + (sq.tok0 + t0) * qk_row + (size_t)i * DK;

    // gates of the group's first value head, then the Gram fragments straight from HBM (standard
    // k order on both sides); rows past T are clamped and masked below
    const size_t grow = (sq.tok0 + t0 + min(lane, n - 1)) * Hv + (size_t)i * grp;
    float gl = log_decay(g[grow]), bl = beta[grow];
    bf16x8 kf[4][KB], qf[4][KB];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const size_t off = (size_t)min(16 * mt + ln, n - 1) * qk_row + 32 * kk + 8 * lg;
            kf[mt][kk] = *reinterpret_cast<const bf16x8*>(kp + off);
            qf[mt][kk] = *reinterpret_cast<const bf16x8*>(qp + off);
        }
    GDN_TRACE_PREP(0);
    prep_zero_t_upper(Tm, lane);
    // raw lower tiles (TI, TJ): K K^T rows TI x columns TJ, and K Q^T rows TJ of K x columns TI
    // of Q (Aqk transposed, so that a lane later holds four consecutive columns of one row)
    floatx4 gk[10], gq[10];
#pragma unroll
    for (int t = 0; t < 10; ++t) gk[t] = gq[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int t = 0; t < 10; ++t) {
            gk[t] = mfma_bf(kf[TI[t]][kk], kf[TJ[t]][kk], gk[t]);
            gq[t] = mfma_bf(kf[TJ[t]][kk], qf[TI[t]][kk], gq[t]);
        }
    GDN_TRACE_PREP(1);
    // q as output-product operands: multiplying by identity columns moves q^T into accumulator
    // layout exactly (D[m][n] = q[16ct + n][32kk + off + m]); two such tiles stacked (off = 0, 16)
    // are the perm-K B operand.  Stored once for the head group.
    {
        opx8* wq = reinterpret_cast<opx8*>(wsq + (((size_t)b * Hqk + i) * NT + c) * ws_q_bytes<DK>());
        bf16x8 eye[2];
#pragma unroll
        for (int off = 0; off < 2; ++off)
#pragma unroll
            for (int e = 0; e < 8; ++e) eye[off][e] = (bf16)((8 * lg + e == ln + 16 * off) ? 1.f : 0.f);
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const floatx4 lo = mfma_bf(eye[0], qf[ct][kk], floatx4{0.f, 0.f, 0.f, 0.f});
                const floatx4 hi = mfma_bf(eye[1], qf[ct][kk], floatx4{0.f, 0.f, 0.f, 0.f});
                wq[(kk * 4 + ct) * 64 + lane] = pack_perm(lo, hi);
            }
    }

    for (int jj = 0; jj < grp; ++jj) {
        const int j = i * grp + jj;
        unsigned char* wc = ws + (((size_t)b * Hv + j) * NT + c) * WS_CHUNK;
        // gates: cumsum and the per-row vectors; the next head's gates load meanwhile
        const float x = wave_cumsum(lane < n ? gl : 0.f, lane);
        const float bt = lane < n ? bl : 0.f;
        if (jj + 1 < grp) {
            gl = log_decay(g[grow + jj + 1]);
            bl = beta[grow + jj + 1];
        }
        const float last = __shfl(x, 63, 64);
        const float eg = __expf(x);
        wave_lds_fence();   // the previous head is done with pg, pb
        pg[lane] = x;
        pb[lane] = bt;
        {
            float* wv = reinterpret_cast<float*>(wc + WS_CV);
            wv[V_B * CH + lane] = bt;
            wv[V_BEG * CH + lane] = bt * eg;
            wv[V_ED * CH + lane] = __expf(last - x);
            wv[V_EC * CH + lane] = __expf(last);
            reinterpret_cast<float*>(wc + WS_EG)[lane] = scale * eg;
        }
        wave_lds_fence();
        // the gate values this lane's tiles need, fetched together: gc and beta of rows
        // 16t + 4lg .. +3 and gc of row 16t + ln, t = 0..3
        floatx4 g4[4], b4[4];
        float g1[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            g4[t] = ld4s(pg + 16 * t + 4 * lg);
            b4[t] = ld4s(pb + 16 * t + 4 * lg);
            g1[t] = pg[16 * t + ln];
        }
        // A = strictly-lower( beta_r exp(gc_r - gc_i) (k_r . k_i) ): diagonal blocks in float32,
        // the rest in float16, both transposed
        prep_store_a(gk, g4, b4, g1, Ad, Ah, lane);
        // Aqk = lower-incl( scale exp(gc_r - gc_i) (q_r . k_i) ); rows past T are zero
        prep_store_aqk(gq, g4, g1, scale, n, reinterpret_cast<op_t*>(wc + WS_AQ), lane);
        GDN_TRACE_PREP(2);
        // T = (I + A)^{-1}, then into the workspace in fragment order (one coalesced 16-byte
        // store per block)
        prep_solve_t(Ad, Ah, Tm, lane);
        GDN_TRACE_PREP(4);
        wave_lds_fence();
        prep_store_t(Tm, reinterpret_cast<opx8*>(wc + WS_T), lane);
        GDN_TRACE_PREP(5);
    }
}

// One workgroup (one wave) per unit of chunks c_base .. c_base + NTg - 1.  The units run with
// the head fastest: the head group of one chunk reads the same g, beta lines and adjacent q, k
// rows, so those workgroups run together, and on one XCD (workgroup ids are dealt to the 8 XCDs
// round-robin) so that they share its L2.
template <int DK, bool VARLEN>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void chunk_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, unsigned char* __restrict__ ws, unsigned char* __restrict__ wsq,
    int T_max, int Hqk, int Hv, int grp, int NT, float scale, int xcd_remap, const int* cu, int total,
    int c_base, int NTg)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[PrepLds::bytes];
    int u = blockIdx.x;
    if (xcd_remap) u = (u & 7) * (gridDim.x >> 3) + (u >> 3);
    prep_unit<DK, VARLEN>(q, k, g, beta, ws, wsq, T_max, Hqk, Hv, grp, NT, scale, cu, total, u, c_base, NTg, lds);
}

// =======================================================================================
// Pipelined fused kernel: one workgroup per (batch, value head, column tile of BV columns) with
// NW chain waves and four prep waves, and one workgroup barrier per chunk.  While the chain
// waves carry chunk n out of LDS slot n & 1, the prep waves build chunk n + 1 in the other slot,
// each prep wave a whole part of it on its own, so that no wave waits on another inside a chunk:
// * T wave: the chunk's k rows from HBM straight into MFMA fragments, K K^T, A and the blocked
//   solve for T = (I + A)^{-1} into a column-permuted matrix of its own, double-buffered like the
//   slots, from which the chain waves read T's fragments (no copy into the slot);
// * Aqk wave: q and k rows into fragments, K Q^T and Aqk into the slot in fragment order;
// * V wave: the chunk's V tile and K (column-permuted float16) into the slot;
// * Q wave: the chunk's Q (column-permuted float16) into the slot, and the gate vectors of the
//   chunk after it (the cumsum of log alpha and the decay factors built from it) into a ring of
//   three sets, which the T and Aqk waves read in the next period and the chain waves in the one
//   after.  Staging Q and forming the vectors had been the T and Aqk waves' own work, and those
//   two set the period; this wave takes them off both.
// Each prep wave loads the next chunk's operands while it works on this one; no prep wave waits
// on a global load it issued in the same period.  The chain waves read every operand from LDS (T
// and Aqk with one 16-byte read per fragment) and run the delta, output and update phases back
// to back.
constexpr int PIPE_PW = 4;   // prep waves of the pipelined kernel
template <int DK, int BV>
struct PLds {
    static constexpr int KP = DK + 8;            // element pitch of K and Q rows
    static constexpr int VP = BV + 16;           // element pitch of V rows
    static constexpr size_t k = 0;                                  // K   [64][KP] f16
    static constexpr size_t q = k + (size_t)CH * KP * 2;            // Q   [64][KP] f16
    static constexpr size_t v = q + (size_t)CH * KP * 2;            // V   [64][VP] bf16
    static constexpr size_t aq = v + (size_t)CH * VP * 2;           // Aqk 6 fragment blocks f16
    static constexpr size_t slot = aq + 6 * 64 * 16;
    static constexpr size_t ad = 2 * slot;                          // T wave: A
    static constexpr size_t ah = ad + (size_t)PREP_AD * 4;
    static constexpr size_t tm = ah + (size_t)PREP_AH * 2;          // T [2][64][CP] f16, column-permuted
    static constexpr size_t vr = tm + (size_t)2 * PREP_TM * 2;      // gate vectors [3][NVEC][64] f32
    static constexpr size_t bytes = vr + (size_t)3 * NVEC * CH * 4;
    static_assert(slot % 16 == 0 && v % 16 == 0 && aq % 16 == 0 && tm % 16 == 0 && vr % 16 == 0,
                  "16-byte aligned parts");
};

// A copy of x the compiler cannot see through: lane-derived values (addresses, masks) computed
// from it inside a loop are recomputed each iteration instead of being hoisted out and kept live
// (or spilled) across the whole loop.
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// Rows 16 mt + ln, columns 32 kk + 8 lg .. +7 of a chunk's q or k (rows clamped to the chunk's
// last token: the callers mask what lies past it) into MFMA fragments.
template <int KB>
__device__ __forceinline__ void load_rows_frag(bf16x8 (&f)[4][KB], const bf16* p, size_t row, int n, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
            f[mt][kk] = *reinterpret_cast<const bf16x8*>(p + (size_t)min(16 * mt + ln, n - 1) * row + 32 * kk + 8 * lg);
}

// The same fragments into an LDS matrix as column-permuted float16 with pitch KP, rows at or
// past n zero.
template <int KB, int KP>
__device__ __forceinline__ void store_rows_frag(const bf16x8 (&f)[4][KB], op_t* m, int n, int lane)
{
    const int ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const int r = 16 * mt + ln, c8 = 32 * kk + 8 * lg;
            const opx8 x = to_op_or_zero(f[mt][kk], r < n);
            op_t* mr = m + r * KP;
            *reinterpret_cast<opx4*>(mr + pcol(c8)) = opx4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<opx4*>(mr + pcol(c8 + 4)) = opx4{x[4], x[5], x[6], x[7]};
        }
}

// A chunk's q or k rows as whole rows: lane + 64 p takes the 16 bytes at segment s % (DK / 8) of
// row s / (DK / 8), so each load instruction covers DK / 16 whole rows (a fragment-ordered load
// covers 64 bytes of each of 16 rows).  Rows are clamped to the chunk's last token; the store
// below zeroes what lies past it.
template <int DK>
__device__ __forceinline__ void load_rows_lin(bf16x8 (&f)[DK / 8], const bf16* p, size_t row, int n, int lane)
{
    constexpr int SEG = DK / 8;
#pragma unroll
    for (int pp = 0; pp < DK / 8; ++pp) {
        const int s = lane + 64 * pp;
        f[pp] = *reinterpret_cast<const bf16x8*>(p + (size_t)min(s / SEG, n - 1) * row + (s % SEG) * 8);
    }
}

// The same rows into an LDS matrix as column-permuted float16 with pitch KP, rows at or past n zero.
template <int DK, int KP>
__device__ __forceinline__ void store_rows_lin(const bf16x8 (&f)[DK / 8], op_t* m, int n, int lane)
{
    constexpr int SEG = DK / 8;
#pragma unroll
    for (int pp = 0; pp < DK / 8; ++pp) {
        const int s = lane + 64 * pp;
        const int r = s / SEG, c8 = (s % SEG) * 8;
        const opx8 x = to_op_or_zero(f[pp], r < n);
        op_t* mr = m + r * KP;
        *reinterpret_cast<opx4*>(mr + pcol(c8)) = opx4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<opx4*>(mr + pcol(c8 + 4)) = opx4{x[4], x[5], x[6], x[7]};
    }
}

template <int DK, int DV, int BV, int NW, bool VARLEN>
__global__ __launch_bounds__((NW + PIPE_PW) * 64, 1) void chunk_pipe_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* s0, float* sf,  // may be the same buffer (in-place state update)
    bf16* __restrict__ o, int T_max, int Hqk, int Hv, int grp, float scale, int xcd_remap, const int* cu,
    int total)
{
    using L = PLds<DK, BV>;
    constexpr int NTILE = DV / BV;
    constexpr int NCOL = BV / NW;      // state columns per chain wave
    constexpr int NTN = NCOL / 16;     // 16-column tiles per chain wave
    constexpr int MT = DK / 16;
    constexpr int KB = DK / 32;
    constexpr int PV = CH * BV / 8 / 64;   // 16-byte V segments per lane of the V wave
    static_assert(NTN >= 1 && NCOL % 16 == 0 && PV >= 1, "tile shape");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const ChainId id = chain_id(NTILE, Hqk, grp, xcd_remap);
    const int b = id.b, i = id.i, j = id.j, c0 = id.tile * BV;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const SeqSpan sq = VARLEN ? seq_span(cu, b, T_max, total) : SeqSpan{(size_t)b * T_max, T_max};
    const int T_len = sq.len;
    GDN_CHECK((int)gridDim.x % (Hv * NTILE) == 0 && b < (int)gridDim.x / (Hv * NTILE) && i < Hqk && j < Hv &&
                  j / grp == i && T_len >= 0 && T_len <= T_max &&
                  sq.tok0 + T_len <= (VARLEN ? (size_t)total : (size_t)(gridDim.x / (Hv * NTILE)) * T_max), 5);
    if (VARLEN && T_len == 0) {
        // an empty sequence: the final state is the initial one (every wave leaves here, before
        // any barrier)
        if (w < NW) copy_state_cols<DK, DV>(s0, sf, (size_t)b * Hv + j, c0 + w * NCOL, NCOL, lane);
        return;
    }
    const int NT = (T_len + CH - 1) / CH;
    const size_t qk_row = (size_t)Hqk * DK;
    const size_t v_row = (size_t)Hv * DV;
    const size_t tok0 = sq.tok0;
    auto slot = [&](int c) { return smem + (size_t)(c & 1) * L::slot; };
    // gate vectors of chunk c: written by the Q wave in the period before chunk c is built, read
    // by the T and Aqk waves while they build it and by the chain waves in the period after
    auto ring = [&](int c) { return reinterpret_cast<float*>(smem + L::vr) + (c % 3) * (NVEC * CH); };

    if (w < NW) {
        // ================================================================= chain waves
        // hacc[nt][mt][x] = h[16mt + 4lg + x][col + 16nt + ln]
        floatx4 hacc[NTN][MT];
        const size_t head = (size_t)b * Hv + j;
        const int col = c0 + w * NCOL;
        load_state<DK, DV, NTN>(hacc, s0, head, col, lane);
        bf16* ob = o + (tok0 * Hv + j) * DV + col;
        lds_barrier();   // gate vectors of chunk 0 in the ring
        lds_barrier();   // chunk 0 built
        for (int n = 0; n < NT; ++n) {
            const unsigned char* sb = slot(n);
            const op_t* Ks = reinterpret_cast<const op_t*>(sb + L::k);
            const op_t* Qs = reinterpret_cast<const op_t*>(sb + L::q);
            const bf16* Vs = reinterpret_cast<const bf16*>(sb + L::v) + w * NCOL;
            const op_t* Tn = reinterpret_cast<const op_t*>(smem + L::tm) + (n & 1) * PREP_TM;
            const opx8* Af = reinterpret_cast<const opx8*>(sb + L::aq);
            const int ln = lane & 15, lg = lane >> 4;
            const float* vs = ring(n);
            const int t0 = n * CH;
            opx8 hb[NTN][KB], db[NTN][2], dtb[NTN][2];
            GDN_TRACE(n, 0);
            chain_delta<DK, NTN, L::VP>(hacc, Ks, Vs,
                                        [&](int mt, int cb) { return frag(Tn, CP, 16 * mt + ln, 32 * cb, lg); },
                                        vs, lane, hb, db, dtb);
            GDN_TRACE(n, 1);
            chain_out<DK, NTN>(hb, db, Qs, [&](int ct, int cb) { return Af[tblk(ct, cb) * 64 + lane]; },
                               vs + V_EG * CH, ob + (size_t)t0 * v_row, v_row, min(CH, T_len - t0), lane);
            GDN_TRACE(n, 2);
            chain_update<DK, NTN>(hacc, Ks, dtb, lane);
            GDN_TRACE(n, 3);
            lds_barrier();   // chunk n + 1 built, slot n & 1 free
        }
        store_state<DK, DV, NTN>(hacc, sf, head, col, lane);
        return;
    }

    // ===================================================================== prep waves
    // a prologue barrier (the Q wave puts chunk 0's gate vectors in the ring), then chunk c is
    // built before the barrier that ends period c - 1; one more barrier matches the chain waves'
    // last
    const int pw = w - NW;
    const bf16* kb_ = k + (tok0 * Hqk + i) * DK;
    const bf16* qb = q + (tok0 * Hqk + i) * DK;
    if (pw == 0) {
        // T wave
        float* Ad = reinterpret_cast<float*>(smem + L::ad);
        op_t* Ah = reinterpret_cast<op_t*>(smem + L::ah);
        op_t* Tm0 = reinterpret_cast<op_t*>(smem + L::tm);
        prep_zero_t_upper(Tm0, lane);
        prep_zero_t_upper(Tm0 + PREP_TM, lane);
        bf16x8 kf[4][KB];
        auto load = [&](int c) {
            const int t0 = c * CH;
            load_rows_frag<KB>(kf, kb_ + (size_t)t0 * qk_row, qk_row, min(CH, T_len - t0), lane);
        };
        if (NT > 0) load(0);
        lds_barrier();
        for (int c = 0; c < NT; ++c) {
            const int lane = opaque(threadIdx.x & 63);
            floatx4 gk[10];
#pragma unroll
            for (int t = 0; t < 10; ++t) gk[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int t = 0; t < 10; ++t) gk[t] = mfma_bf(kf[TI[t]][kk], kf[TJ[t]][kk], gk[t]);
            GDN_TRACE(c, 0);
            if (c + 1 < NT) load(c + 1);
            const float* vs = ring(c);
            const int ln = lane & 15, lg = lane >> 4;
            GDN_TRACE(c, 1);
            if (vs[V_G * CH + CH - 1] > GC_FACTOR_MIN) {
                floatx4 br4[4];
                float en1[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    br4[t] = ld4s(vs + V_BEG * CH + 16 * t + 4 * lg);
                    en1[t] = vs[V_EN * CH + 16 * t + ln];
                }
                prep_store_a_fac(gk, br4, en1, Ad, Ah, lane);
            } else {
                floatx4 g4[4], b4[4];
                float g1[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    g4[t] = ld4s(vs + V_G * CH + 16 * t + 4 * lg);
                    b4[t] = ld4s(vs + V_B * CH + 16 * t + 4 * lg);
                    g1[t] = vs[V_G * CH + 16 * t + ln];
                }
                prep_store_a(gk, g4, b4, g1, Ad, Ah, lane);
            }
            GDN_TRACE(c, 2);
            // T into the chunk's matrix, which the chain waves read in the next period
            prep_solve_t(Ad, Ah, Tm0 + (c & 1) * PREP_TM, lane);
            GDN_TRACE(c, 3);
            lds_barrier();
        }
    } else if (pw == 1) {
        // Aqk wave
        bf16x8 kf[4][KB], qf[4][KB];
        auto load = [&](int c) {
            const int t0 = c * CH, n = min(CH, T_len - t0);
            load_rows_frag<KB>(kf, kb_ + (size_t)t0 * qk_row, qk_row, n, lane);
            load_rows_frag<KB>(qf, qb + (size_t)t0 * qk_row, qk_row, n, lane);
        };
        if (NT > 0) load(0);
        lds_barrier();
        for (int c = 0; c < NT; ++c) {
            unsigned char* sb = slot(c);
            const int n = min(CH, T_len - c * CH);
            const int lane = opaque(threadIdx.x & 63);
            // K Q^T: rows TJ of K x columns TI of Q (Aqk transposed)
            floatx4 gq[10];
#pragma unroll
            for (int t = 0; t < 10; ++t) gq[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int t = 0; t < 10; ++t) gq[t] = mfma_bf(kf[TJ[t]][kk], qf[TI[t]][kk], gq[t]);
            GDN_TRACE(c, 0);
            if (c + 1 < NT) load(c + 1);
            GDN_TRACE(c, 1);
            const float* vs = ring(c);
            const int ln = lane & 15, lg = lane >> 4;
            if (vs[V_G * CH + CH - 1] > GC_FACTOR_MIN) {
                floatx4 en4[4];
                float eg1[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    en4[t] = ld4s(vs + V_EN * CH + 16 * t + 4 * lg);
                    eg1[t] = vs[V_EG * CH + 16 * t + ln];
                }
                prep_store_aqk_fac(gq, eg1, en4, n, reinterpret_cast<op_t*>(sb + L::aq), lane);
            } else {
                floatx4 g4[4];
                float g1[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    g4[t] = ld4s(vs + V_G * CH + 16 * t + 4 * lg);
                    g1[t] = vs[V_G * CH + 16 * t + ln];
                }
                prep_store_aqk(gq, g4, g1, scale, n, reinterpret_cast<op_t*>(sb + L::aq), lane);
            }
            GDN_TRACE(c, 2);
            lds_barrier();
        }
    } else if (pw == 2) {
        // V wave: V and K into the slot
        const bf16* vb = v + (tok0 * Hv + j) * DV + c0;
        bf16x8 rv[PV];
        bf16x8 kf[4][KB];
        auto load_v = [&](int c) {
            const int t0 = c * CH, n = min(CH, T_len - t0);
#pragma unroll
            for (int p = 0; p < PV; ++p) {
                const int s = lane + 64 * p;
                const int r = min(s / (BV / 8), n - 1), c8 = (s % (BV / 8)) * 8;
                rv[p] = *reinterpret_cast<const bf16x8*>(vb + (size_t)(t0 + r) * v_row + c8);
            }
            load_rows_frag<KB>(kf, kb_ + (size_t)t0 * qk_row, qk_row, n, lane);
        };
        if (NT > 0) load_v(0);
        lds_barrier();
        for (int c = 0; c < NT; ++c) {
            bf16* Vs = reinterpret_cast<bf16*>(slot(c) + L::v);
            const int n = min(CH, T_len - c * CH);
#pragma unroll
            for (int p = 0; p < PV; ++p) {
                const int s = lane + 64 * p;
                const int r = s / (BV / 8), c8 = (s % (BV / 8)) * 8;
                *reinterpret_cast<bf16x8*>(Vs + r * L::VP + c8) = r < n ? rv[p] : bf16x8{};
            }
            store_rows_frag<KB, L::KP>(kf, reinterpret_cast<op_t*>(slot(c) + L::k), n, opaque(lane));
            GDN_TRACE(c, 0);
            if (c + 1 < NT) load_v(c + 1);
            GDN_TRACE(c, 1);
            lds_barrier();
        }
    } else {
        // Q wave: Q into the slot; the gate vectors of the chunk after, into the ring
        const float* gb = g + tok0 * Hv + j;
        const float* bb = beta + tok0 * Hv + j;
        bf16x8 qf[DK / 8];
        float rg = 0.f, rb = 0.f;
        auto load_q = [&](int c) {
            const int t0 = c * CH;
            load_rows_lin<DK>(qf, qb + (size_t)t0 * qk_row, qk_row, min(CH, T_len - t0), lane);
        };
        // g, beta of chunk c, rows past the sequence clamped (masked below)
        auto load_g = [&](int c) {
            const int t0 = c * CH, n = min(CH, T_len - t0);
            const size_t off = (size_t)(t0 + min(lane, n - 1)) * Hv;
            rg = gb[off];
            rb = bb[off];
        };
        // the gate vectors of chunk c from its raw g, beta (one token per lane)
        auto put_vec = [&](int c) {
            const int n = min(CH, T_len - c * CH);
            const float x = wave_cumsum_dpp(lane < n ? log_decay(rg) : 0.f);
            const float bt = lane < n ? rb : 0.f;
            const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
            const float eg = __expf(x);
            float* vs = ring(c);
            vs[V_G * CH + lane] = x;
            vs[V_B * CH + lane] = bt;
            vs[V_BEG * CH + lane] = bt * eg;
            vs[V_ED * CH + lane] = __expf(last - x);
            vs[V_EC * CH + lane] = __expf(last);
            vs[V_EG * CH + lane] = scale * eg;
            vs[V_EN * CH + lane] = __expf(fminf(-x, -GC_FACTOR_MIN));
        };
        if (NT > 0) {
            load_g(0);
            put_vec(0);
            if (NT > 1) load_g(1);
            load_q(0);
        }
        lds_barrier();
        for (int c = 0; c < NT; ++c) {
            const int n = min(CH, T_len - c * CH);
            if (c + 1 < NT) put_vec(c + 1);
            GDN_TRACE(c, 0);
            store_rows_lin<DK, L::KP>(qf, reinterpret_cast<op_t*>(slot(c) + L::q), n, opaque(lane));
            GDN_TRACE(c, 1);
            if (c + 2 < NT) load_g(c + 2);
            if (c + 1 < NT) load_q(c + 1);
            GDN_TRACE(c, 2);
            lds_barrier();
        }
    }
    lds_barrier();
}

// Split path, kernel 2: the state pass.  One workgroup per (batch, value head, column tile of
// BV = 16 NW columns) with SLW loader waves, NW chain waves (16 state columns each) and SOW
// output waves, one barrier per chunk.  The chain waves are the critical path; every other role
// is sized to finish inside their period.
// * Loaders stage chunk n + 1's K (q, k converted to column-permuted float16), V and state-step
//   vectors into double-buffered LDS while the chain waves carry chunk n, from registers loaded
//   two chunks ahead (one chunk ahead left the staging waiting on the loads).  That is all that
//   goes through LDS besides the hand-over below: LDS bandwidth is what a chunk's latency is most
//   sensitive to.
// * A chain wave reads T straight from the workspace in fragment order (16-byte coalesced loads,
//   one chunk ahead, double-buffered in registers over a two-chunk loop), runs the Delta and
//   update phases, and hands its packed h and Delta to the output waves through LDS.
// * Each output wave forms two token tiles of O of chunk n - 1, for every column group, in
//   iteration n from those hand-overs and Q, Aqk and scale exp(gc) read from the workspace in
//   fragment order, double-buffered two chunks ahead.
constexpr int SLW = 2;   // loader waves of the state pass
constexpr int SOW = 2;   // output waves of the state pass (two token tiles of every chunk each)

// Segments of a chain (the affine chunk scan).  Over a chunk the state map is affine,
// h_out = M h_in + N with M = e^gL I - K~^T W and N = K~^T U (the WY form of the chunk,
// "Gated Attention Architectures", sections 2 and 3), and such maps compose, so a chain can be
// cut into segments of `len` chunks (grid y = segment):
// * transport (XPORT): each segment is run from h = [0 | I] over the value columns and dk more
//   columns whose V is zero; the value columns end as the segment's N, the extra ones as its M
//   (written to nout [chain][seg][dk][dv] and mout [chain][seg][dk][dk]), with no output;
// * prefill: each segment starts from hin [chain][seg][dk][dv] (the entry states the combine
//   kernel forms from the transports) and writes its O; the last segment writes the final
//   state.  hin null: one segment from s0.
struct SegArgs {
    int len;            // chunks per segment
    const float* hin;   // prefill: entry state of every segment, or null
    float* mout;        // transport outputs
    float* nout;
    int base = 0;       // first chunk of segment 0 (a later piece of the rows)
};

template <int DK, int BV, int NW>
struct SLds {
    static constexpr int KP = DK + 8;
    // With one chain wave (its per-chunk latency is the whole period) the loaders stage beta V,
    // float32 and transposed (pitch RVP: conflict-free 16-byte reads), which takes two vector
    // instructions per element off the chain; with two the loaders' extra work costs more than
    // it saves (measured on the 64K-token workload), and V stays bf16 row-major (pitch VP).
    static constexpr bool RV32 = NW == 1;
    static constexpr int RVP = CH + 4;
    static constexpr int VP = RV32 ? RVP : BV + 16;
    // K, V and the state-step vectors in two slots: the chain waves read chunk n while the
    // loaders stage chunk n + 1
    static constexpr size_t kbytes = (size_t)CH * KP * 2;
    static constexpr size_t vbytes = RV32 ? (size_t)BV * RVP * 4 : (size_t)CH * VP * 2;
    static constexpr size_t cvbytes = (size_t)4 * CH * 4;
    static constexpr size_t k = 0;                                   // K   [2][64][KP] f16
    static constexpr size_t v = k + 2 * kbytes;                      // beta V [2][BV][RVP] f32 or V [2][64][VP] bf16
    static constexpr size_t cv = v + 2 * vbytes;                     // rows V_B..V_EC [2][4][64] f32
    // chain -> output hand-over, [2][NW]: hb (DK/32 fragments) then db (2), each fragment 64
    // lanes x 16 bytes
    static constexpr size_t hx_frags = DK / 32 + 2;
    static constexpr size_t hx = cv + 2 * cvbytes;
    static constexpr size_t bytes = hx + 2 * NW * hx_frags * 1024;
    static_assert(v % 16 == 0 && cv % 16 == 0 && hx % 16 == 0, "16-byte aligned parts");
};

// The state pass of workgroup `blk` of `nblk` (segment `seg` of `nseg`), in the LDS at smem.
template <int DK, int DV, int NW, bool VARLEN, bool XPORT>
__device__ __forceinline__ void state_body(
    const bf16* __restrict__ k, const bf16* __restrict__ v, const unsigned char* __restrict__ ws,
    const unsigned char* __restrict__ wsq, const float* s0, float* sf, bf16* __restrict__ o, int T_max, int Hqk,
    int Hv, int grp, int xcd_remap, const int* cu, int total, SegArgs sg, int blk, int nblk, int seg_y, int nseg,
    unsigned char* smem)
{
    constexpr int BV = 16 * NW;
    using L = SLds<DK, BV, NW>;
    constexpr int NTILE = (XPORT ? DV + DK : DV) / BV;   // transport: dk more columns (M)
    static_assert(DV % BV == 0 && DK % BV == 0, "a tile lies in the value or the M columns");
    constexpr int MT = DK / 16;
    constexpr int KB = DK / 32;
    constexpr int NLT = SLW * 64;                       // loader threads
    constexpr int RP = DK / 16;                         // 32-byte pair-runs per K row
    constexpr int PK = CH * RP / NLT;                   // pair-runs per loader lane
    constexpr int RV = BV / 8;                          // 16-byte runs per V row
    constexpr int PV = (CH * RV + NLT - 1) / NLT;       // V runs per loader lane
    constexpr int CVR = 4 * CH * 4 / 16;                // 16-byte runs of the state-step vectors
    static_assert(PK >= 1 && CH * RP % NLT == 0 && CVR <= NLT, "tile shape");

    const ChainId id = chain_id_of(blk, nblk, NTILE, Hqk, grp, xcd_remap);
    const int b = id.b, i = id.i, j = id.j;
    const int c0 = id.tile * BV;
    const int nrows = nblk / (Hv * NTILE);   // batch rows (sequences) of the launch
    GDN_CHECK(blk < nblk && nblk % (Hv * NTILE) == 0 && b < nrows && i < Hqk && j < Hv && j / grp == i &&
                  id.tile < NTILE && seg_y < nseg, 1);
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    // Roles by wave index.  Wave w runs on SIMD w % 4, and the chain waves (the latency-bound
    // critical path) get SIMDs of their own: waves 0 and 1 form O, waves 2 .. NW + 1 carry the
    // chains, waves NW + 2 and NW + 3 load (the two output waves and the two loaders each on
    // different SIMDs).
    static_assert(SLW == 2 && SOW == 2 && NW <= 2, "wave roles");
    const bool is_chain = w >= 2 && w < 2 + NW;
    const bool is_loader = w >= 2 + NW;
    const int li = w - (2 + NW);     // loader index (loader waves)
    const int cw = w - 2;            // chain wave index (chain waves)
    const size_t head = (size_t)b * Hv + j;
    SeqSpan sq = VARLEN ? seq_span(cu, b, T_max, total) : SeqSpan{(size_t)b * T_max, T_max};
    if (VARLEN && sq.len == 0) {
        // an empty sequence: the final state is the initial one (every wave leaves here, before
        // any barrier)
        if (is_chain) copy_state_cols<DK, DV>(s0, sf, head, c0 + cw * 16, 16, lane);
        return;
    }
    // this workgroup's segment: chunks cb .. cb + NT - 1 of the row, a shorter sequence that
    // starts cb chunks in (the launcher gives every segment at least one chunk)
    const int seg = VARLEN ? 0 : seg_y;
    const int cb = sg.base + seg * sg.len;
    if (!VARLEN) {
        const int rem = sq.len - cb * CH;
        sq.tok0 += (size_t)cb * CH;
        sq.len = (rem + CH - 1) / CH > sg.len ? sg.len * CH : rem;
    }
    const int T_len = sq.len;
    const int NT = (T_len + CH - 1) / CH;       // this segment's chunks
    const int NTS = (T_max + CH - 1) / CH;      // chunks per row of the workspace
    const int qk_row = Hqk * DK;
    const size_t v_row = (size_t)Hv * DV;
    const unsigned char* wh = ws + (head * NTS + cb) * WS_CHUNK;
    const bool mcols = XPORT && c0 >= DV;       // transport columns of M: V is zero
    GDN_CHECK(NT >= 1 && cb >= 0 && cb + NT <= NTS && T_len <= (NTS - cb) * CH &&
                  sq.tok0 + T_len <= (VARLEN ? (size_t)total : (size_t)nrows * T_max), 2);
    auto kslot = [&](int c) { return reinterpret_cast<op_t*>(smem + L::k + (size_t)(c & 1) * L::kbytes); };
    auto vslot = [&](int c) { return smem + L::v + (size_t)(c & 1) * L::vbytes; };
    auto cvslot = [&](int c) { return reinterpret_cast<float*>(smem + L::cv + (size_t)(c & 1) * L::cvbytes); };
    auto hxp = [&](int c, int cw) {
        return reinterpret_cast<opx8*>(smem + L::hx + ((size_t)(c & 1) * NW + cw) * L::hx_frags * 1024);
    };

    if (is_loader) {
        // ================================================================= loader waves
        const int ltid = li * 64 + lane;   // loader thread index
        const bf16* kb_ = k + (sq.tok0 * Hqk + i) * DK;
        const bf16* vb = v + (sq.tok0 * Hv + j) * DV + (mcols ? 0 : c0);
        const int vrow = Hv * DV;
        // one chunk's loads; two in flight, so each has two periods to arrive
        struct LdBuf {
            bf16x8 rk[PK][2];
            bf16x8 rv[PV];
            float rb[PV];   // beta of each V run's row
            floatx4 rc;
        };
        // K pair-run s of a chunk: row s / RP, 32-column block pr / 2 (pr = s % RP), half
        // a = pr % 2.  Two 16-byte loads (logical columns 32 blk + 8a .. +7 and the same + 16)
        // hold exactly the physical runs 4 blk + 2a and + 1 of the column-permuted row, which sit
        // side by side: 32 contiguous bytes in LDS.  Rows past T are loaded clamped to the last
        // row and staged as they are: their beta is 0, so T keeps them out of Delta (identity
        // rows) and they add nothing anywhere.
        int kq_r[PK], kq_c[PK];
#pragma unroll
        for (int p = 0; p < PK; ++p) {
            const int s = ltid + p * NLT, pr = s % RP;
            kq_r[p] = s / RP;
            kq_c[p] = 32 * (pr >> 1) + 8 * (pr & 1);
        }
        auto load_chain = [&](int c, LdBuf& r) {
            const int t0 = c * CH, n = min(CH, T_len - t0);
            GDN_CHECK(c >= 0 && c < NT && n >= 1 && (head * NTS + cb + c) < (size_t)nrows * Hv * NTS, 3);
            const bf16* kc = kb_ + (size_t)t0 * qk_row;
#pragma unroll
            for (int p = 0; p < PK; ++p) {
                const int off = min(kq_r[p], n - 1) * qk_row + kq_c[p];
                r.rk[p][0] = *reinterpret_cast<const bf16x8*>(kc + off);
                r.rk[p][1] = *reinterpret_cast<const bf16x8*>(kc + off + 16);
            }
            const bf16* vc = vb + (size_t)t0 * vrow;
            if (!mcols) {
                const float* bc = reinterpret_cast<const float*>(wh + (size_t)c * WS_CHUNK + WS_CV) + V_B * CH;
#pragma unroll
                for (int p = 0; p < PV; ++p) {
                    const int s = min(ltid + p * NLT, CH * RV - 1);
                    r.rv[p] = *reinterpret_cast<const bf16x8*>(vc + min(s / RV, n - 1) * vrow + (s % RV) * 8);
                    if constexpr (L::RV32) r.rb[p] = bc[s / RV];   // 0 past the last row: clamped rows add nothing
                }
            }
            if (ltid < CVR) r.rc = *reinterpret_cast<const floatx4*>(wh + (size_t)c * WS_CHUNK + WS_CV + 16 * ltid);
        };
        auto stage_chain = [&](int c, const LdBuf& r) {
            op_t* Ks = kslot(c);
            unsigned char* Vs = vslot(c);
#pragma unroll
            for (int p = 0; p < PK; ++p) {
                opx8* dst = reinterpret_cast<opx8*>(Ks + kq_r[p] * L::KP + 16 * ((ltid + p * NLT) % RP));
                bf16_pair_to_op(r.rk[p][0], r.rk[p][1], dst[0], dst[1]);
            }
            if (!mcols) {
#pragma unroll
                for (int p = 0; p < PV; ++p) {
                    const int s = ltid + p * NLT;
                    if (s < CH * RV) {
                        if constexpr (L::RV32) {
                            // beta V, float32, transposed: the 8 columns of this run at row s / RV
                            float* dst = reinterpret_cast<float*>(Vs) + (s % RV) * 8 * L::RVP + s / RV;
#pragma unroll
                            for (int e = 0; e < 8; ++e) dst[e * L::RVP] = r.rb[p] * (float)r.rv[p][e];
                        } else {
                            *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(Vs) + (s / RV) * L::VP + (s % RV) * 8) = r.rv[p];
                        }
                    }
                }
            }
            if (ltid < CVR) reinterpret_cast<floatx4*>(cvslot(c))[ltid] = r.rc;
        };
        if (mcols) {
            // the M columns' V is zero in both slots for the whole segment
            for (int s = ltid; s < (int)(L::vbytes / 16); s += NLT)
#pragma unroll
                for (int slot = 0; slot < 2; ++slot)
                    reinterpret_cast<floatx4*>(vslot(slot))[s] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        // Prefetches are issued unconditionally (chunk index clamped to the last chunk; the
        // extra loads at the end are harmless) so that every path through the loop has the same
        // memory operations in flight and each wait covers exactly the loads it needs.
        // iteration n stages chunk n + 1 from buffer (n + 1) % 2, then loads chunk n + 3 into it
        LdBuf bufA, bufB;
        load_chain(0, bufA);
        stage_chain(0, bufA);
        load_chain(min(1, NT - 1), bufB);
        load_chain(min(2, NT - 1), bufA);
        lds_barrier();
        auto step = [&](int n, LdBuf& r) {
            GDN_TRACE(n, 0);
            if (n + 1 < NT) stage_chain(n + 1, r);
            GDN_TRACE(n, 1);
            load_chain(min(n + 3, NT - 1), r);
            GDN_TRACE(n, 2);
            lds_barrier();
        };
        int n = 0;
        for (; n + 1 < NT; n += 2) {
            step(n, bufB);
            step(n + 1, bufA);
        }
        if (n < NT) step(n, bufB);
    } else if (is_chain) {
        // ================================================================= chain waves
        const int col = c0 + cw * 16;
        floatx4 hacc[1][MT];
        if constexpr (XPORT) {
            // h = [0 | I]: zeros in the value columns, the identity in the M columns
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) hacc[0][mt][x] = 16 * mt + 4 * lg + x == col - DV + ln ? 1.f : 0.f;
        } else if (sg.hin) {
            load_state<DK, DV, 1>(hacc, sg.hin + (head * nseg + seg) * DK * DV, 0, col, lane);
        } else {
            load_state<DK, DV, 1>(hacc, s0, head, col, lane);
        }
        // T fragments of chunk c (fragment order in the workspace)
        auto load_tf = [&](int c, opx8 (&t)[6], int lane) {
            const opx8* src = reinterpret_cast<const opx8*>(wh + (size_t)c * WS_CHUNK + WS_T);
#pragma unroll
            for (int bk = 0; bk < 6; ++bk) t[bk] = src[bk * 64 + lane];
        };
        // Transport M columns: V is zero there, so the chunk step is linear in h and may run on
        // h scaled by a power of two per column (exact in float32).  Scaling each column's largest
        // entry into [0.5, 1) before the step keeps the float16 operands made from h, R and Delta
        // in float16's normal range however far M has decayed.
        auto col_scale = [&]() {
            float mx = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) mx = fmaxf(mx, fabsf(hacc[0][mt][x]));
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));   // the four lanes of one column
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            int e = 0;
            frexpf(mx, &e);
            return mx > 0.f ? ldexpf(1.f, -max(e, -120)) : 1.f;
        };
        auto rescale = [&](float f) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int x = 0; x < 4; ++x) hacc[0][mt][x] *= f;
        };
        auto step = [&](int n, const opx8 (&tc)[6], opx8 (&tn)[6]) {
            GDN_TRACE(n, 0);
            const int lane = opaque(threadIdx.x & 63);
            float sc = 1.f;
            if (mcols) {
                sc = col_scale();
                rescale(sc);
            }
            load_tf(min(n + 1, NT - 1), tn, lane);   // unconditional: see the loaders
            const op_t* Ks = kslot(n);
            opx8 hb[1][KB], db[1][2], dtb[1][2];
            opx8 akt[2][MT];
            const void* Vc = L::RV32 ? (const void*)(reinterpret_cast<const float*>(vslot(n)) + cw * 16 * L::RVP)
                                     : (const void*)(reinterpret_cast<const bf16*>(vslot(n)) + cw * 16);
            chain_delta<DK, 1, L::VP, true, false, L::RV32>(hacc, Ks, Vc, [&](int mt, int cb) { return tc[tblk(mt, cb)]; },
                                            cvslot(n), lane, hb, db, dtb, akt);
            opx8* hx = hxp(n, cw);
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) hx[kk * 64 + lane] = hb[0][kk];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) hx[(KB + cb) * 64 + lane] = db[0][cb];
            GDN_TRACE(n, 1);
            apply_kt<DK, 1>(hacc, akt[0], dtb, 0);
            apply_kt<DK, 1>(hacc, akt[1], dtb, 1);
            if (mcols) rescale(1.f / sc);
            GDN_TRACE(n, 2);
            lds_barrier();
        };
        opx8 tA[6], tB[6];
        load_tf(0, tA, lane);
        lds_barrier();
        int n = 0;
        for (; n + 1 < NT; n += 2) {
            step(n, tA, tB);
            step(n + 1, tB, tA);
        }
        if (n < NT) step(n, tA, tB);
        if constexpr (XPORT) {
            if (col < DV)
                store_state<DK, DV, 1>(hacc, sg.nout + (head * nseg + seg) * DK * DV, 0, col, lane);
            else
                store_state<DK, DK, 1>(hacc, sg.mout + (head * nseg + seg) * DK * DK, 0, col - DV, lane);
        } else if (seg == nseg - 1) {
            store_state<DK, DV, 1>(hacc, sf, head, col, lane);
        }
    } else if (XPORT) {
        // no output: the same barriers as the other roles
        for (int n = 0; n <= NT; ++n) lds_barrier();
    } else {
        // ================================================================= output waves
        // Output wave ow forms token tiles {0, 3} (ow = 0) or {1, 2} (ow = 1) of O of chunk n - 1
        // in iteration n, for every column group: the two sets take the same number of products.
        auto role = [&](auto owc) {
            constexpr int OWC = decltype(owc)::value;
            constexpr int CT0 = OWC == 0 ? 0 : 1, CT1 = OWC == 0 ? 3 : 2;
            auto ctile = [](int t) { return t == 0 ? CT0 : CT1; };
            bf16* ob = o + (sq.tok0 * Hv + j) * DV + c0;
            const unsigned char* wqh = wsq + (((size_t)b * Hqk + i) * NTS + cb) * ws_q_bytes<DK>();
            // inputs of one chunk's output step for these token tiles, all in fragment order from
            // the workspace: Q, the Aqk blocks (ct, cb <= ct / 2) and scale exp(gc);
            // double-buffered, loaded two chunks ahead of their use
            struct OutIn {
                opx8 qf[KB][2];
                opx8 af[2][2];
                float eg[2];
            };
            auto load_in = [&](int c, OutIn& in) {
                const opx8* qs = reinterpret_cast<const opx8*>(wqh + (size_t)c * ws_q_bytes<DK>());
#pragma unroll
                for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                    for (int t = 0; t < 2; ++t) in.qf[kk][t] = qs[(kk * 4 + ctile(t)) * 64 + lane];
                const unsigned char* wc = wh + (size_t)c * WS_CHUNK;
                const opx8* a = reinterpret_cast<const opx8*>(wc + WS_AQ);
                const float* e = reinterpret_cast<const float*>(wc + WS_EG);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int cb = 0; cb <= ctile(t) / 2; ++cb) in.af[t][cb] = a[tblk(ctile(t), cb) * 64 + lane];
                    in.eg[t] = e[16 * ctile(t) + ln];
                }
            };
            // O^T = (h^T Q^T) diag(scale exp(gc)) + Delta^T (scale Aqk)^T for chunk m (see
            // chain_out), column group by column group
            auto out = [&](int m, const OutIn& in) {
                const int lane = opaque(threadIdx.x & 63), ln = lane & 15, lg = lane >> 4;
                const int t0 = m * CH, nv = min(CH, T_len - t0);
#pragma unroll
                for (int cgw = 0; cgw < NW; ++cgw) {
                    const opx8* hx = hxp(m, cgw);
                    opx8 hb[KB];
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk) hb[kk] = hx[kk * 64 + lane];
                    opx8 db[2];
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) db[cb] = hx[(KB + cb) * 64 + lane];
                    floatx4 OT[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) OT[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                        for (int t = 0; t < 2; ++t) OT[t] = mfma32(hb[kk], in.qf[kk][t], OT[t]);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int x = 0; x < 4; ++x) OT[t][x] *= in.eg[t];
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int cb = 0; cb <= ctile(t) / 2; ++cb) OT[t] = mfma32(db[cb], in.af[t][cb], OT[t]);
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int tok = 16 * ctile(t) + ln;
                        if (tok < nv) {
                            GDN_CHECK(sq.tok0 + t0 + tok < (VARLEN ? (size_t)total : (size_t)nrows * T_max), 4);
                            const bf16x4 ov = {(bf16)OT[t][0], (bf16)OT[t][1], (bf16)OT[t][2], (bf16)OT[t][3]};
                            *reinterpret_cast<bf16x4*>(ob + (size_t)(t0 + tok) * v_row + 16 * cgw + 4 * lg) = ov;
                        }
                    }
                }
            };
            // iteration n forms O of chunk n - 1 from buffer (n - 1) % 2, then loads chunk n + 1
            // into it
            auto step = [&](int n, OutIn& cur) {
                GDN_TRACE(n, 0);
                if (n >= 1) {
                    out(n - 1, cur);
                    GDN_TRACE(n, 1);
                    load_in(min(n + 1, NT - 1), cur);   // unconditional: see the loaders
                }
                GDN_TRACE(n, 2);
                lds_barrier();
            };
            OutIn bufA, bufB;
            load_in(0, bufA);
            load_in(min(1, NT - 1), bufB);
            lds_barrier();
            int n = 0;
            for (; n + 1 < NT; n += 2) {
                step(n, bufB);       // n even: O of chunk n - 1 (odd) is in bufB
                step(n + 1, bufA);   // O of chunk n (even) is in bufA
            }
            if (n < NT) step(n, bufB);
            if ((NT - 1) % 2 == 0)
                out(NT - 1, bufA);
            else
                out(NT - 1, bufB);
        };
        if (w == 0)
            role(std::integral_constant<int, 0>{});
        else
            role(std::integral_constant<int, 1>{});
    }
}

template <int DK, int DV, int NW, bool VARLEN, bool XPORT = false>
__global__ __launch_bounds__((SLW + NW + SOW) * 64) __attribute__((amdgpu_waves_per_eu(2))) void chunk_state_kernel(
    const bf16* __restrict__ k, const bf16* __restrict__ v, const unsigned char* __restrict__ ws,
    const unsigned char* __restrict__ wsq, const float* s0, float* sf, bf16* __restrict__ o, int T_max, int Hqk,
    int Hv, int grp, int xcd_remap, const int* cu, int total, SegArgs sg)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    state_body<DK, DV, NW, VARLEN, XPORT>(k, v, ws, wsq, s0, sf, o, T_max, Hqk, Hv, grp, xcd_remap, cu, total, sg,
                                          blockIdx.x, gridDim.x, blockIdx.y, gridDim.y, smem);
}

// The state pass of one piece of the rows (chunks sg.base .. sg.base + sg.len - 1) beside the
// prep of the next piece (chunks c_base .. c_base + NTg - 1), in one launch: workgroups
// 0 .. nstate - 1 run the state pass, the others (on the compute units it leaves free: one
// workgroup per compute unit, as the LDS size allows no more) run prep units, one per wave at a
// time.  The two parts share no data, and the launch boundary orders each piece's prep before
// its state pass.
template <int DK, int DV, int NW>
__global__ __launch_bounds__((SLW + NW + SOW) * 64) __attribute__((amdgpu_waves_per_eu(2))) void chunk_overlap_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, unsigned char* __restrict__ ws, unsigned char* __restrict__ wsq,
    const float* s0, float* sf, bf16* __restrict__ o, int T_max, int Hqk, int Hv, int grp, float scale,
    int xcd_remap, SegArgs sg, int nstate, int c_base, int NTg, int nunits)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    GDN_CHECK(nstate >= 1 && nstate < (int)gridDim.x && nunits == nunits / (Hqk * NTg) * Hqk * NTg && sg.base >= 0, 6);
    if ((int)blockIdx.x < nstate) {
        state_body<DK, DV, NW, false, false>(k, v, ws, wsq, s0, sf, o, T_max, Hqk, Hv, grp, xcd_remap, nullptr, 0,
                                             sg, blockIdx.x, nstate, 0, 1, smem);
        return;
    }
    constexpr int NWAVE = SLW + NW + SOW;
    const int w = threadIdx.x >> 6;
    const int NT = (T_max + CH - 1) / CH;
    const int npw = ((int)gridDim.x - nstate) * NWAVE;   // prep waves; nunits = B Hqk NTg units
    for (int u = ((int)blockIdx.x - nstate) * NWAVE + w; u < nunits; u += npw)
        prep_unit<DK, false>(q, k, g, beta, ws, wsq, T_max, Hqk, Hv, grp, NT, scale, nullptr, 0, u, c_base, NTg,
                             smem + (size_t)w * PrepLds::bytes);
}

namespace {

#ifdef GDN_TEST_HOOKS
// Only in the test-hooks build of the library (libgdn_hooks.so, which the tests load to run every
// kernel family on small shapes): environment overrides of the automatic route choice.  The
// release library reads no environment; its route and workspace size follow from the arguments.
int env_int(const char* name, int dflt)
{
    const char* e = getenv(name);
    return e ? atoi(e) : dflt;
}
const char* env_str(const char* name) { return getenv(name); }
#else
int env_int(const char*, int dflt) { return dflt; }
const char* env_str(const char*) { return nullptr; }
#endif

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

// Column-tile width of the state pass, 16 (one chain wave) or 32 (two): 16 while that still
// gives at most one workgroup per compute unit, so short-chain workloads spread over the chip
// (measured: two 16-column workgroups sharing a CU run slower than one 32-column one).
int choose_split_bv(const ChunkArgs& a)
{
    const int bv = env_int("GDN_SPLIT_BV", 0);
    if (bv == 16 || bv == 32) return bv;
    const long chains = (long)a.B * a.Hv;
    return chains * (a.dv / 16) <= 256 ? 16 : 32;
}

// The pipelined fused kernel (chunk_pipe_kernel) serves calls with enough chains to fill the
// chip, uniform or packed (measured: 0.62 ms against 0.81 ms for chunk_mfma_kernel on 8 x 8192
// tokens x 32 value heads); a gated call on this route takes the fused kernel with the gated
// epilogue.  With fewer chains the split path wins: the pipelined kernel builds T and Aqk once
// per column tile, the split path once per value head.
bool use_pipe(const ChunkArgs& a)
{
    if (const char* e = env_str("GDN_MFMA_PATH")) return !strcmp(e, "pipe");
    return (long)a.B * a.Hv >= 192;
}

// Column-tile width of the pipelined kernel: the widest of 128, 64, 32 that still gives at least
// 192 workgroups, else 16.
int choose_pipe_bv(const ChunkArgs& a)
{
    const int bv = env_int("GDN_PIPE_BV", 0);
    if ((bv == 16 || bv == 32 || bv == 64 || bv == 128) && bv <= a.dv) return bv;
    const long chains = (long)a.B * a.Hv;
    for (int c = 128; c >= 32; c /= 2)
        if (c <= a.dv && chains * (a.dv / c) >= 192) return c;
    return 16;
}

bool use_split(const ChunkArgs& a)
{
    if (use_pipe(a)) return false;
    if (const char* e = env_str("GDN_MFMA_PATH")) {
        if (!strcmp(e, "split")) return true;
        if (!strcmp(e, "fused")) return false;
    }
    return (long)a.B * a.Hv < 192;
}

// Pieces of the split path: the rows cut into pieces of PIECE chunks; the prep of piece p + 1
// runs in the same launch as the state pass of piece p, on the compute units the state pass
// leaves free (chunk_overlap_kernel), and only piece 0's prep runs alone.  Taken when the state
// pass leaves at least 32 compute units idle and the rows hold at least two pieces; uniform
// batches only.  Measured on the 64K-token workload (48 value heads, 192 state workgroups on the
// 256 compute units): the prep alone took 295 us on the whole chip and the state pass 1,297 us;
// run side by side on 64 and 192 compute units they took 866 and 1,422 us.
int piece_len() { return std::max(16, env_int("GDN_SPLIT_PIECE", 128)); }

long split_state_blocks(const ChunkArgs& a) { return (long)a.B * a.Hv * (a.dv / choose_split_bv(a)); }

// The shape takes pieces on a 256-compute-unit device; the workspace then holds the state
// handed from piece to piece (a function of the arguments only).
bool pieces_shape(const ChunkArgs& a)
{
    const long NT = ((long)a.T + CH - 1) / CH;
    return !a.cu && use_split(a) && NT >= 2L * piece_len() && split_state_blocks(a) <= 256 - 32;
}

// Compute units of the current device (cached per device).
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = -1;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int DK, int DV, int BV, bool GATED, bool VARLEN = false>
hipError_t launch_fused_t(const ChunkArgs& a, hipStream_t st)
{
    if (!VARLEN && a.cu) return launch_fused_t<DK, DV, BV, GATED, true>(a, st);
    using L = MLds<DK, BV, GATED>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    auto kern = chunk_mfma_kernel<DK, DV, BV, GATED, VARLEN>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    const int grp = a.Hv / a.Hqk;
    const long nblk = (long)a.B * a.Hv * (DV / BV);
    // XCD-major placement when every XCD gets whole query/key-head groups
    const long per_xcd = nblk / 8;
    const int remap = (nblk % 8 == 0) && (per_xcd % ((long)grp * (DV / BV)) == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(NTHR), L::bytes, st, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, a.g, a.beta, a.s0, a.sf,
                       (bf16*)(GATED ? a.y : a.o), (const bf16*)a.z, a.norm_w, a.norm_w_stride, a.eps, a.T,
                       a.Hqk, a.Hv, grp, a.scale, remap, a.cu, a.total);
    return hipGetLastError();
}

// The state pass over `nseg` segments of sg.len chunks (grid y); nseg = 1, sg.len = NT for a
// whole chain from s0.
template <int DK, int DV, int BV, int NW, bool VARLEN = false>
hipError_t launch_pipe_t(const ChunkArgs& a, hipStream_t st)
{
    if (!VARLEN && a.cu) return launch_pipe_t<DK, DV, BV, NW, true>(a, st);
    using L = PLds<DK, BV>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    auto kern = chunk_pipe_kernel<DK, DV, BV, NW, VARLEN>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    const int grp = a.Hv / a.Hqk;
    const long nblk = (long)a.B * a.Hv * (DV / BV);
    const long per_xcd = nblk / 8;
    const int remap = (nblk % 8 == 0) && (per_xcd % ((long)grp * (DV / BV)) == 0) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3((NW + PIPE_PW) * 64), L::bytes, st, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, a.g, a.beta, a.s0, a.sf, (bf16*)a.o, a.T, a.Hqk, a.Hv,
                       grp, a.scale, remap, a.cu, a.total);
    return hipGetLastError();
}

template <int DK, int DV, int NW, bool VARLEN, bool XPORT = false>
hipError_t launch_state_t(const ChunkArgs& a, void* ws, hipStream_t st, SegArgs sg, int nseg)
{
    constexpr int BV = 16 * NW;
    constexpr int NTILE = (XPORT ? DV + DK : DV) / BV;
    using L = SLds<DK, BV, NW>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    auto kern = chunk_state_kernel<DK, DV, NW, VARLEN, XPORT>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    const int grp = a.Hv / a.Hqk;
    const long nblk = (long)a.B * a.Hv * NTILE;
    const long per_xcd = nblk / 8;
    const int remap = (nblk % 8 == 0) && (per_xcd % ((long)grp * NTILE) == 0) ? 1 : 0;
    const int NT = (int)(((long)a.T + CH - 1) / CH);
    const unsigned char* wsq = (const unsigned char*)ws + (size_t)a.B * a.Hv * NT * WS_CHUNK;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk, (unsigned)nseg), dim3((SLW + NW + SOW) * 64), L::bytes, st,
                       (const bf16*)a.k, (const bf16*)a.v, (const unsigned char*)ws, wsq, a.s0, a.sf, (bf16*)a.o,
                       a.T, a.Hqk, a.Hv, grp, remap, a.cu, a.total, sg);
    return hipGetLastError();
}

// The prep of chunks c_base .. c_base + NTg - 1 of every row (all of them by default).
template <int DK, bool VARLEN>
hipError_t launch_prep_t(const ChunkArgs& a, void* ws, hipStream_t st, int c_base = 0, int NTg = -1)
{
    const int grp = a.Hv / a.Hqk;
    const int NT = (int)(((long)a.T + CH - 1) / CH);
    if (NTg < 0) NTg = NT;
    const long nprep = (long)a.B * a.Hqk * NTg;
    unsigned char* wsq = (unsigned char*)ws + (size_t)a.B * a.Hv * NT * WS_CHUNK;
    hipLaunchKernelGGL((chunk_prep_kernel<DK, VARLEN>), dim3((unsigned)nprep), dim3(64), 0, st, (const bf16*)a.q,
                       (const bf16*)a.k, a.g, a.beta, (unsigned char*)ws, wsq, a.T, a.Hqk, a.Hv, grp, NT,
                       a.scale, nprep % 8 == 0 ? 1 : 0, a.cu, a.total, c_base, NTg);
    return hipGetLastError();
}

// The split path in pieces (see pieces_shape): piece 0's prep alone, then one launch per piece of
// its state pass beside the next piece's prep, the last piece's state pass alone.  The state
// passes hand the state on through the workspace.
template <int DK, int DV, int NW>
hipError_t launch_pieces_t(const ChunkArgs& a, void* ws, hipStream_t st, int ncu)
{
    constexpr int BV = 16 * NW;
    constexpr int NWAVE = SLW + NW + SOW;
    using L = SLds<DK, BV, NW>;
    constexpr size_t lds = L::bytes > NWAVE * PrepLds::bytes ? L::bytes : NWAVE * PrepLds::bytes;
    static_assert(lds <= 160 * 1024, "LDS budget");
    auto kern = chunk_overlap_kernel<DK, DV, NW>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int NT = (int)(((long)a.T + CH - 1) / CH);
    const int len = piece_len();
    const int P = (NT + len - 1) / len;
    const int grp = a.Hv / a.Hqk;
    const long nstate = (long)a.B * a.Hv * (DV / BV);
    const int remap = (nstate % 8 == 0) && ((nstate / 8) % ((long)grp * (DV / BV)) == 0) ? 1 : 0;
    unsigned char* wsq = (unsigned char*)ws + (size_t)a.B * a.Hv * NT * WS_CHUNK;
    float* hand = reinterpret_cast<float*>(wsq + (size_t)a.B * a.Hqk * NT * ws_q_bytes<DK>());
    e = launch_prep_t<DK, false>(a, ws, st, 0, std::min(len, NT));
    for (int p = 0; p < P && e == hipSuccess; ++p) {
        SegArgs sg{len, nullptr, nullptr, nullptr};
        sg.base = p * len;
        const float* s0p = p == 0 ? a.s0 : hand;
        float* sfp = p == P - 1 ? a.sf : hand;
        if (p + 1 < P) {
            const int cn = (p + 1) * len, ntg = std::min(len, NT - cn);
            hipLaunchKernelGGL(kern, dim3((unsigned)ncu), dim3(NWAVE * 64), lds, st, (const bf16*)a.q,
                               (const bf16*)a.k, (const bf16*)a.v, a.g, a.beta, (unsigned char*)ws, wsq, s0p, sfp,
                               (bf16*)a.o, a.T, a.Hqk, a.Hv, grp, a.scale, remap, sg, (int)nstate, cn, ntg,
                               a.B * a.Hqk * ntg);
            e = hipGetLastError();
        } else {
            ChunkArgs ap = a;
            ap.s0 = s0p;
            ap.sf = sfp;
            e = launch_state_t<DK, DV, NW, false>(ap, ws, st, sg, 1);
        }
    }
    return e;
}

template <int DK, int DV, bool VARLEN = false>
hipError_t launch_split_t(const ChunkArgs& a, void* ws, hipStream_t st)
{
    if (!VARLEN && a.cu) return launch_split_t<DK, DV, true>(a, ws, st);
    if (!VARLEN && pieces_shape(a)) {
        const int ncu = device_cus();
        if (ncu - split_state_blocks(a) >= 32)
            return choose_split_bv(a) == 16 ? launch_pieces_t<DK, DV, 1>(a, ws, st, ncu)
                                            : launch_pieces_t<DK, DV, 2>(a, ws, st, ncu);
    }
    hipError_t e = launch_prep_t<DK, VARLEN>(a, ws, st);
    if (e != hipSuccess) return e;
    const int NT = (int)(((long)a.T + CH - 1) / CH);
    const SegArgs whole{NT, nullptr, nullptr, nullptr};
    if (choose_split_bv(a) == 16) return launch_state_t<DK, DV, 1, VARLEN>(a, ws, st, whole, 1);
    return launch_state_t<DK, DV, 2, VARLEN>(a, ws, st, whole, 1);
}

// ---------------------------------------------------------------- affine chunk scan
// Entry states of the segments of every chain from their transports: h_0 = S0 (zeros when
// null), h_{s+1} = M_s h_s + N_s, float32.  One workgroup of 2 DK threads per (chain, 32-column
// tile); each thread keeps a 4 x 4 block of the new state, M_s is staged transposed in LDS.
template <int DK, int DV>
__global__ __launch_bounds__(2 * DK) void seg_combine_kernel(const float* s0, const float* __restrict__ mseg,
                                                             const float* __restrict__ nseg, float* __restrict__ hin,
                                                             int P)
{
    constexpr int MP = DK + 4;   // row pitch of the transposed M (16-byte rows)
    constexpr int NTH = 2 * DK;
    extern __shared__ __attribute__((aligned(16))) float cmb[];
    float* Mt = cmb;             // [DK][MP], Mt[k][m] = M[m][k]
    float* hs = cmb + DK * MP;   // [DK][32], the current entry state's tile
    const size_t head = blockIdx.x;
    const int c0 = blockIdx.y * 32;
    const int tid = threadIdx.x;
    const int m0 = 4 * (tid >> 3), cc = 4 * (tid & 7);
    for (int e = tid; e < DK * 8; e += NTH) {
        const int m = e >> 3, c = 4 * (e & 7);
        const floatx4 x = s0 ? *reinterpret_cast<const floatx4*>(s0 + (head * DK + m) * DV + c0 + c)
                             : floatx4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<floatx4*>(hs + m * 32 + c) = x;
        *reinterpret_cast<floatx4*>(hin + (head * P * DK + m) * DV + c0 + c) = x;
    }
    for (int s = 0; s + 1 < P; ++s) {
        const float* M = mseg + (head * (P - 1) + s) * DK * DK;
        const float* N = nseg + (head * (P - 1) + s) * DK * DV;
        for (int e = tid; e < DK * DK / 4; e += NTH) {
            const int m = e % DK, k4 = 4 * (e / DK);
            const floatx4 x = *reinterpret_cast<const floatx4*>(M + (size_t)m * DK + k4);
#pragma unroll
            for (int y = 0; y < 4; ++y) Mt[(k4 + y) * MP + m] = x[y];
        }
        floatx4 acc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = *reinterpret_cast<const floatx4*>(N + (size_t)(m0 + r) * DV + c0 + cc);
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < DK; ++kk) {
            const floatx4 a = *reinterpret_cast<const floatx4*>(Mt + kk * MP + m0);
            const floatx4 h = *reinterpret_cast<const floatx4*>(hs + kk * 32 + cc);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[r][y] = fmaf(a[r], h[y], acc[r][y]);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            *reinterpret_cast<floatx4*>(hs + (m0 + r) * 32 + cc) = acc[r];
            *reinterpret_cast<floatx4*>(hin + ((head * P + s + 1) * DK + m0 + r) * DV + c0 + cc) = acc[r];
        }
    }
}

struct ScanLayout {
    int L, P;                       // chunks per segment, segments
    size_t prep, mout, nout, hin, bytes;
};

ScanLayout scan_layout(const ChunkArgs& a, int segments)
{
    ScanLayout s{};
    const int NT = (int)(((long)a.T + CH - 1) / CH);
    s.L = (NT + segments - 1) / segments;
    s.P = (NT + s.L - 1) / s.L;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t chains = (size_t)a.B * a.Hv;
    s.prep = 0;
    s.mout = up((size_t)a.B * NT * (a.Hv * (size_t)WS_CHUNK + a.Hqk * (size_t)CH * a.dk * 2));
    s.nout = s.mout + up(chains * (s.P - 1) * a.dk * a.dk * 4);
    s.hin = s.nout + up(chains * (s.P - 1) * a.dk * a.dv * 4);
    s.bytes = s.hin + up(chains * s.P * a.dk * a.dv * 4);
    return s;
}

template <int DK, int DV>
hipError_t launch_scan_t(const ChunkArgs& a, int segments, void* ws, hipStream_t st)
{
    const ScanLayout sl = scan_layout(a, segments);
    unsigned char* w = (unsigned char*)ws;
    hipError_t e = launch_prep_t<DK, false>(a, ws, st);
    if (e != hipSuccess) return e;
    const long chains = (long)a.B * a.Hv;
    float* mout = (float*)(w + sl.mout);
    float* nout = (float*)(w + sl.nout);
    float* hin = (float*)(w + sl.hin);
    if (sl.P > 1) {
        const SegArgs xs{sl.L, nullptr, mout, nout};
        e = chains * (sl.P - 1) * ((DV + DK) / 16) <= 256
                ? launch_state_t<DK, DV, 1, false, true>(a, ws, st, xs, sl.P - 1)
                : launch_state_t<DK, DV, 2, false, true>(a, ws, st, xs, sl.P - 1);
        if (e != hipSuccess) return e;
        constexpr size_t cl = (size_t)DK * (DK + 4) * 4 + (size_t)DK * 32 * 4;
        auto comb = seg_combine_kernel<DK, DV>;
        e = hipFuncSetAttribute((const void*)comb, hipFuncAttributeMaxDynamicSharedMemorySize, (int)cl);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(comb, dim3((unsigned)chains, DV / 32), dim3(2 * DK), cl, st, a.s0, (const float*)mout,
                           (const float*)nout, hin, sl.P);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const SegArgs fs{sl.L, sl.P > 1 ? hin : nullptr, nullptr, nullptr};
    return chains * sl.P * (DV / 16) <= 256 ? launch_state_t<DK, DV, 1, false>(a, ws, st, fs, sl.P)
                                            : launch_state_t<DK, DV, 2, false>(a, ws, st, fs, sl.P);
}

template <int DK, int DV>
hipError_t launch_transport_t(const ChunkArgs& a, float* m_out, float* n_out, void* ws, hipStream_t st)
{
    hipError_t e = launch_prep_t<DK, false>(a, ws, st);
    if (e != hipSuccess) return e;
    const int NT = (int)(((long)a.T + CH - 1) / CH);
    const SegArgs xs{NT, nullptr, m_out, n_out};
    return (long)a.B * a.Hv * ((DV + DK) / 16) <= 256 ? launch_state_t<DK, DV, 1, false, true>(a, ws, st, xs, 1)
                                                      : launch_state_t<DK, DV, 2, false, true>(a, ws, st, xs, 1);
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a)
{
    if (env_str("GDN_DISABLE_MFMA")) return false;
    return a.dtype_bf16 && a.chunk == CH && (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128);
}

bool chunk_mfma_split(const ChunkArgs& a) { return chunk_mfma_supported(a) && use_split(a); }

bool chunk_mfma_pipe(const ChunkArgs& a) { return chunk_mfma_supported(a) && use_pipe(a); }

bool chunk_mfma_gated_fused(const ChunkArgs& a)
{
    return chunk_mfma_supported(a) && !use_split(a) && choose_bv(a) == a.dv;
}

size_t chunk_scan_workspace_bytes(const ChunkArgs& a, int segments) { return scan_layout(a, segments).bytes; }

// Segments for an unsegmented prefill call: enough that the transport pass (32-column tiles over
// the dv + dk columns of every segment but the last) about fills the 256 compute units, used
// only when that gives at least 3 segments of at least 8 chunks each.  With fewer the extra work
// of the maps (about as much again as the state pass over those segments) is not repaid: on one
// GPU's share of a 64K-token prefill under an 8-way head split (6 value heads) 6 segments took
// 0.52 ms against 0.97 ms unsegmented, 2 segments 1.18 ms.
int chunk_auto_segments(const ChunkArgs& a)
{
    if (!chunk_mfma_split(a) || a.cu || a.z) return 1;
    const int env = env_int("GDN_SCAN_SEGMENTS", -1);
    if (env >= 1) return env;
    if (env == 0) return 1;
    const long tiles32 = (long)a.B * a.Hv * ((a.dv + a.dk) / 32);
    const long p = 1 + 256 / tiles32;
    const long NT = ((long)a.T + CH - 1) / CH;
    return p >= 3 && NT >= 8 * p ? (int)p : 1;
}

int chunk_scan_segments(const ChunkArgs& a, int segments) { return scan_layout(a, segments).P; }

size_t chunk_transport_workspace_bytes(const ChunkArgs& a) { return scan_layout(a, 1).mout; }

#define GDN_SCAN_DISPATCH(F, ...)                                                  \
    if (a.dk == 128 && a.dv == 128) return F<128, 128>(a, __VA_ARGS__);           \
    if (a.dk == 128 && a.dv == 64) return F<128, 64>(a, __VA_ARGS__);             \
    if (a.dk == 64 && a.dv == 128) return F<64, 128>(a, __VA_ARGS__);             \
    if (a.dk == 64 && a.dv == 64) return F<64, 64>(a, __VA_ARGS__);               \
    return hipErrorInvalidValue;

hipError_t launch_chunk_scan(const ChunkArgs& a, int segments, void* ws, hipStream_t st)
{
    GDN_SCAN_DISPATCH(launch_scan_t, segments, ws, st)
}

hipError_t launch_chunk_transport(const ChunkArgs& a, float* m_out, float* n_out, void* ws, hipStream_t st)
{
    GDN_SCAN_DISPATCH(launch_transport_t, m_out, n_out, ws, st)
}
#undef GDN_SCAN_DISPATCH

size_t chunk_mfma_workspace_bytes(const ChunkArgs& a)
{
    if (!chunk_mfma_split(a)) return 0;
    const size_t NT = ((size_t)a.T + CH - 1) / CH;
    const size_t hand = pieces_shape(a) ? (size_t)a.B * a.Hv * a.dk * a.dv * 4 : 0;
    return (size_t)a.B * NT * (a.Hv * (size_t)WS_CHUNK + a.Hqk * (size_t)CH * a.dk * 2) + hand;
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
    if (!a.z && use_pipe(a)) {
        const int bv = choose_pipe_bv(a);
#define GDN_PIPE_CASE(DK_, DV_, BV_, NW_) \
    if (a.dk == DK_ && a.dv == DV_ && bv == BV_) return launch_pipe_t<DK_, DV_, BV_, NW_>(a, st);
        GDN_PIPE_CASE(128, 128, 128, 4) GDN_PIPE_CASE(128, 128, 64, 4) GDN_PIPE_CASE(128, 128, 32, 2)
        GDN_PIPE_CASE(128, 128, 16, 1) GDN_PIPE_CASE(128, 64, 64, 4) GDN_PIPE_CASE(128, 64, 32, 2)
        GDN_PIPE_CASE(128, 64, 16, 1) GDN_PIPE_CASE(64, 128, 128, 4) GDN_PIPE_CASE(64, 128, 64, 4)
        GDN_PIPE_CASE(64, 128, 32, 2) GDN_PIPE_CASE(64, 128, 16, 1) GDN_PIPE_CASE(64, 64, 64, 4)
        GDN_PIPE_CASE(64, 64, 32, 2) GDN_PIPE_CASE(64, 64, 16, 1)
#undef GDN_PIPE_CASE
        return hipErrorInvalidValue;
    }
    const int bv = choose_bv(a);
    if (a.z) {
        // the gated epilogue needs whole value heads per workgroup (chunk_mfma_gated_fused)
        if (bv != a.dv) return hipErrorInvalidValue;
        if (a.dk == 128 && a.dv == 128) return launch_fused_t<128, 128, 128, true>(a, st);
        if (a.dk == 128 && a.dv == 64) return launch_fused_t<128, 64, 64, true>(a, st);
        if (a.dk == 64 && a.dv == 128) return launch_fused_t<64, 128, 128, true>(a, st);
        if (a.dk == 64 && a.dv == 64) return launch_fused_t<64, 64, 64, true>(a, st);
        return hipErrorInvalidValue;
    }
#define GDN_MFMA_CASE(DK_, DV_, BV_) \
    if (a.dk == DK_ && a.dv == DV_ && bv == BV_) return launch_fused_t<DK_, DV_, BV_, false>(a, st);
    GDN_MFMA_CASE(128, 128, 128) GDN_MFMA_CASE(128, 128, 64) GDN_MFMA_CASE(128, 64, 64)
    GDN_MFMA_CASE(64, 128, 128) GDN_MFMA_CASE(64, 128, 64) GDN_MFMA_CASE(64, 64, 64)
#undef GDN_MFMA_CASE
    return hipErrorInvalidValue;
}

// =======================================================================================
// Kimi Delta Attention on the matrix cores ("Gated Attention Architectures", section 8): the
// delta rule with one decay per key channel.  With gc[r][m] the in-chunk cumulative log decay
// of key channel m and gL = gc[63], every in-chunk operand is a product with a factor at most 1:
//     Kh = e^gc * K,  Kt = e^(gL - gc) * K,  Qh = scale e^gc * Q,
//     A  = strictly-lower(beta_r sum_m k_rm k_im e^(gc_rm - gc_im)),  T = (I + A)^{-1},
//     Aq = lower-incl(scale sum_m q_rm k_im e^(gc_rm - gc_im))
// and the state step is the Gated DeltaNet one with those operands:
//     Delta = T (beta V - beta Kh h),  O = Qh h + Aq Delta,  h <- diag(e^gL) h + Kt^T Delta.
// kda_prep_kernel forms the chunk's operands in parallel over (batch, value head, chunk) on the
// vector units (the pairwise decays are exponentials of differences, float32) and writes them as
// float16; kda_state_kernel carries the chains on the matrix cores with the chain-wave steps of
// the Gated DeltaNet kernels.
namespace {

constexpr int KQ_NT = 1024;   // threads of the prep kernel

// per (batch, value head, chunk) workspace block: Kh, Kt, Qh [64][DK] f16; T, Aq [64][64] f16;
// beta [64] f32; e^gL [DK] f32
template <int DK>
struct KdaWs {
    static constexpr size_t kh = 0;
    static constexpr size_t kt = kh + (size_t)CH * DK * 2;
    static constexpr size_t qh = kt + (size_t)CH * DK * 2;
    static constexpr size_t tm = qh + (size_t)CH * DK * 2;
    static constexpr size_t aq = tm + (size_t)CH * CH * 2;
    static constexpr size_t bt = aq + (size_t)CH * CH * 2;
    static constexpr size_t el = bt + (size_t)CH * 4;
    static constexpr size_t bytes = el + (size_t)DK * 4;
};

template <typename T, int DK>
__global__ __launch_bounds__(KQ_NT) void kda_prep_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const float* __restrict__ g, const float* __restrict__ beta,
                                                         unsigned char* __restrict__ ws, int T_len, int Hqk, int Hv,
                                                         int grp, int NT, float scale)
{
    using W = KdaWs<DK>;
    constexpr int KP = DK + 1, AP = CH + 4;   // A, Aq rows 16-byte aligned
    extern __shared__ float lds[];
    float* Ks = lds;
    float* Qs = Ks + CH * KP;
    float* Gs = Qs + CH * KP;
    float* As = Gs + CH * KP;
    float* Aqs = As + CH * AP;
    float* bs = Aqs + CH * AP;
    float* Ts = bs + CH;   // T = (I + A)^{-1} in float32 [CH][AP]

    const int c = blockIdx.x % NT;
    const int head = blockIdx.x / NT;   // b * Hv + j
    const int b = head / Hv, j = head - b * Hv, i = j / grp;
    const int tid = threadIdx.x;
    const int t0 = c * CH, n = min(CH, T_len - t0);
#pragma unroll
    for (int e = tid; e < CH * DK; e += KQ_NT) {
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
    if (tid < CH) bs[tid] = tid < n ? beta[((size_t)b * T_len + t0 + tid) * Hv + j] : 0.f;
    __syncthreads();
    // per-channel cumsum down the 64 rows: 8 lanes per channel, 8 rows each, the lanes' totals
    // scanned across the 8-lane group
    static_assert(DK * 8 <= KQ_NT, "eight lanes per channel");
    if (tid < DK * 8) {
        const int m = tid >> 3, rg = tid & 7;
        float x[8];
        float run = 0.f;
#pragma unroll
        for (int y = 0; y < 8; ++y) {
            run += Gs[(8 * rg + y) * KP + m];
            x[y] = run;
        }
        float pre = run;   // inclusive scan of the group totals over rg
#pragma unroll
        for (int sh = 1; sh < 8; sh <<= 1) {
            const float u = __shfl_up(pre, sh, 8);
            if (rg >= sh) pre += u;
        }
        pre -= run;        // exclusive
#pragma unroll
        for (int y = 0; y < 8; ++y) Gs[(8 * rg + y) * KP + m] = x[y] + pre;
    }
    __syncthreads();
    // A (beta-scaled, strictly lower) and Aq (lower including the diagonal); the upper parts are
    // zeros.
    for (int e = tid; e < CH * CH; e += KQ_NT) {
        const int r = e / CH, s = e % CH;
        if (s > r) {
            As[r * AP + s] = 0.f;
            Aqs[r * AP + s] = 0.f;
        }
    }
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    if (w < 6) {
        // The six 16 x 16 blocks below the diagonal blocks, one wave each, on the matrix cores.
        // Block row R, block column S < R: the last row p = 16 S + 15 of block S lies between
        // every pair (r > p >= s), so each term splits into two factors of at most |k|:
        //     k_rm k_sm e^(gc_rm - gc_sm) = (k_rm e^(gc_rm - gc_pm)) (k_sm e^(gc_pm - gc_sm)),
        // float16 operands formed in registers (A: rows of block R, B: rows of block S; both
        // take channel 32 kk + 8 lg + x in element x of lane group lg, so the sum pairs channels).
        const int R = w < 3 ? w + 1 : (w < 5 ? w - 1 : 3);
        const int S = w < 3 ? 0 : (w < 5 ? 1 : 2);
        const int pr = 16 * S + 15;
        const int ra = 16 * R + ln, sb = 16 * S + ln;
        floatx4 ca = {0.f, 0.f, 0.f, 0.f}, cq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            opx8 fa, fq, fb;
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int m = 32 * kk + 8 * lg + x;
                const float gp = Gs[pr * KP + m];
                const float er = __expf(Gs[ra * KP + m] - gp);
                const float es = __expf(gp - Gs[sb * KP + m]);
                fa[x] = (op_t)(Ks[ra * KP + m] * er);
                fq[x] = (op_t)(Qs[ra * KP + m] * er);
                fb[x] = (op_t)(Ks[sb * KP + m] * es);
            }
            ca = mfma32(fa, fb, ca);
            cq = mfma32(fq, fb, cq);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * R + 4 * lg + x;   // accumulator row 4 lg + x, column ln
            As[r * AP + sb] = bs[r] * ca[x];
            Aqs[r * AP + sb] = cq[x];
        }
    } else {
        // The four diagonal blocks (16 * 17 / 2 pairs each) on the vector units: pairwise decays
        // as exponentials of differences, one pair per lane of waves 6 .. 15 (pair t of a block is
        // row r, column s with t = r (r + 1) / 2 + s).
        for (int pq = tid - 6 * 64; pq < 4 * 136; pq += KQ_NT - 6 * 64) {
            const int blk = pq / 136, t = pq - blk * 136;
            int r = (int)((sqrtf(8.f * t + 1.f) - 1.f) * 0.5f);
            r += (r + 1) * (r + 2) / 2 <= t;   // round-off guard: r (r + 1) / 2 <= t < (r + 1) (r + 2) / 2
            r -= r * (r + 1) / 2 > t;
            const int s = 16 * blk + t - r * (r + 1) / 2;
            r += 16 * blk;
            float kk = 0.f, qk = 0.f;
#pragma unroll 4
            for (int m = 0; m < DK; ++m) {
                const float wv = __expf(Gs[r * KP + m] - Gs[s * KP + m]) * Ks[s * KP + m];
                kk = fmaf(Ks[r * KP + m], wv, kk);
                qk = fmaf(Qs[r * KP + m], wv, qk);
            }
            As[r * AP + s] = s < r ? bs[r] * kk : 0.f;
            Aqs[r * AP + s] = qk;
        }
    }
    __syncthreads();
    unsigned char* wb = ws + ((size_t)head * NT + c) * W::bytes;
    // The chunk's operands for the state pass, which do not depend on T: written by waves 1.. while
    // wave 0 runs the first block of the solve below.
    auto write_operands = [&](int t, int nt) {
        op_t* kh = reinterpret_cast<op_t*>(wb + W::kh);
        op_t* kt = reinterpret_cast<op_t*>(wb + W::kt);
        op_t* qh = reinterpret_cast<op_t*>(wb + W::qh);
        for (int e = t; e < CH * DK; e += nt) {
            const int r = e / DK, m = e % DK;
            const float gr = Gs[r * KP + m], gl = Gs[(CH - 1) * KP + m];
            kh[e] = (op_t)(__expf(gr) * Ks[r * KP + m]);
            kt[e] = (op_t)(__expf(gl - gr) * Ks[r * KP + m]);
            qh[e] = (op_t)(__expf(gr) * Qs[r * KP + m]);
        }
        op_t* aw = reinterpret_cast<op_t*>(wb + W::aq);
        for (int e = t; e < CH * CH; e += nt) aw[e] = (op_t)Aqs[(e / CH) * AP + e % CH];
        float* bw = reinterpret_cast<float*>(wb + W::bt);
        float* ew = reinterpret_cast<float*>(wb + W::el);
        if (t < CH) bw[t] = bs[t];
        for (int m = t; m < DK; m += nt) ew[m] = __expf(Gs[(CH - 1) * KP + m]);
    };
    // T = (I + A)^{-1} blockwise over four 16-row blocks D: the identity's columns by forward
    // substitution inside block D (one thread per column, 16 rows in registers, A read by
    // broadcast, four partial sums), then the rows below take R -= A[rows, D..] T[D..] as float32
    // matrix-core tiles.  Each thread's dependent chain is 16 rows instead of 64.
    for (int e = tid; e < CH * CH; e += KQ_NT) Ts[(e / CH) * AP + e % CH] = e / CH == e % CH ? 1.f : 0.f;
    __syncthreads();
    for (int D = 0; D < CH; D += 16) {
        if (tid < CH) {
            float y[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] = Ts[(D + r) * AP + tid];
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                float acc[4] = {y[r], 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < r; ++u) acc[u & 3] = fmaf(-As[(D + r) * AP + D + u], y[u], acc[u & 3]);
                y[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Ts[(D + r) * AP + tid] = y[r];
        } else if (D == 0) {
            write_operands(tid - CH, KQ_NT - CH);
        }
        __syncthreads();
        if (D + 16 < CH) {
            const int RT0 = D / 16 + 1;   // first row tile below the block
            for (int tt = w; tt < (CH / 16 - RT0) * (CH / 16); tt += KQ_NT / 64) {
                const int R = RT0 + tt / (CH / 16), T2 = tt % (CH / 16);
                const floatx4 u4 = mfma_f32_tile(floatx4{0.f, 0.f, 0.f, 0.f}, 0, 16,
                                                 [&](int ii, int kk) { return As[(16 * R + ii) * AP + D + kk]; },
                                                 [&](int kk, int jj) { return Ts[(D + kk) * AP + 16 * T2 + jj]; });
#pragma unroll
                for (int x = 0; x < 4; ++x) Ts[(16 * R + 4 * lg + x) * AP + 16 * T2 + ln] -= u4[x];
            }
            __syncthreads();
        }
    }
    op_t* tw = reinterpret_cast<op_t*>(wb + W::tm);
    for (int e = tid; e < CH * CH; e += KQ_NT) tw[e] = (op_t)Ts[(e / CH) * AP + e % CH];
}

template <int DK>
constexpr size_t kda_prep_lds_bytes()
{
    return ((size_t)3 * CH * (DK + 1) + (size_t)3 * CH * (CH + 4) + CH) * sizeof(float);
}

// LDS of the state kernel: two slots, each Kh, Kt, Qh [64][DK+8] f16 (column-permuted), T, Aq
// [64][CP] f16 (column-permuted), V [64][32] bf16, the row vectors [8][64] f32, e^gL [DK] f32
template <int DK>
struct KsLds {
    static constexpr int KP = DK + 8;
    static constexpr int VP = 32;
    static constexpr size_t kh = 0;
    static constexpr size_t kt = kh + (size_t)CH * KP * 2;
    static constexpr size_t qh = kt + (size_t)CH * KP * 2;
    static constexpr size_t tm = qh + (size_t)CH * KP * 2;
    static constexpr size_t aq = tm + (size_t)CH * CP * 2;
    static constexpr size_t v = aq + (size_t)CH * CP * 2;
    static constexpr size_t vec = v + (size_t)CH * VP * 2;
    static constexpr size_t ech = vec + (size_t)8 * CH * 4;
    static constexpr size_t slot = ech + (size_t)DK * 4;
    static constexpr size_t bytes = 2 * slot;
    static_assert(slot % 16 == 0 && kt % 16 == 0 && tm % 16 == 0 && v % 16 == 0 && vec % 16 == 0, "alignment");
};

// one workgroup of 4 waves per (batch, value head, 16-column tile): wave 0 carries the chain of
// chunk n from slot n & 1 while waves 1..3 stage chunk n + 1 into the other slot; one barrier
// per chunk
template <int DK, int DV>
__global__ __launch_bounds__(256) void kda_state_kernel(const bf16* __restrict__ v,
                                                        const unsigned char* __restrict__ ws, const float* s0,
                                                        float* sf, bf16* __restrict__ o, int T_len, int Hv, int NT)
{
    using L = KsLds<DK>;
    using W = KdaWs<DK>;
    constexpr int NTILE = DV / 16;
    constexpr int KP = L::KP;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tile = blockIdx.x % NTILE;
    const size_t head = blockIdx.x / NTILE;   // b * Hv + j
    const int b = (int)(head / Hv), j = (int)(head - (size_t)b * Hv);
    const int c0 = tile * 16;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t v_row = (size_t)Hv * DV;
    const bf16* vb = v + ((size_t)b * T_len * Hv + j) * DV + c0;

    // loaders (waves 1..3): chunk c's operands are loaded into registers one chunk period before
    // they are stored into LDS slot c & 1, so the global-load latency overlaps a whole chunk of
    // the chain wave's work.
    constexpr int RK = DK / 8;
    constexpr int NK = (3 * CH * RK + 191) / 192, NM = (2 * CH * 8 + 191) / 192, NE = (DK + 191) / 192;
    const int lt = (int)threadIdx.x - 64;   // loader thread 0..191 (negative on the chain wave)
    struct Stage {
        opx8 xk[NK], xm[NM];   // Kh, Kt, Qh runs; T, Aq runs
        bf16x8 xv;             // V run (64 rows x 2 runs of 8)
        float bt, el[NE];      // beta; e^gL per channel
    };
    // Every load is issued unconditionally with its index clamped (the chunk index too), so each
    // path has the same loads in flight.
    auto load = [&](int c, Stage& x) {
        const unsigned char* wb = ws + (head * NT + c) * W::bytes;
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int e = min(lt + p * 192, 3 * CH * RK - 1);
            const int mtx = e / (CH * RK), rr = (e / RK) % CH, c8 = (e % RK) * 8;
            x.xk[p] = *reinterpret_cast<const opx8*>(wb + (mtx == 0 ? W::kh : mtx == 1 ? W::kt : W::qh) +
                                                     ((size_t)rr * DK + c8) * 2);
        }
#pragma unroll
        for (int p = 0; p < NM; ++p) {
            const int e = min(lt + p * 192, 2 * CH * 8 - 1);
            const int mtx = e / (CH * 8), rr = (e / 8) % CH, c8 = (e % 8) * 8;
            x.xm[p] = *reinterpret_cast<const opx8*>(wb + (mtx == 0 ? W::tm : W::aq) + ((size_t)rr * CH + c8) * 2);
        }
        const int t0 = c * CH, n = min(CH, T_len - t0);
        const int rv = min(lt / 2, n - 1), cv = (lt % 2) * 8;
        x.xv = *reinterpret_cast<const bf16x8*>(vb + (size_t)(t0 + rv) * v_row + cv);
        x.bt = reinterpret_cast<const float*>(wb + W::bt)[min(lt, CH - 1)];
#pragma unroll
        for (int p = 0; p < NE; ++p) x.el[p] = reinterpret_cast<const float*>(wb + W::el)[min(lt + p * 192, DK - 1)];
    };
    auto store = [&](int c, const Stage& x) {
        unsigned char* sb = smem + (size_t)(c & 1) * L::slot;
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int e = lt + p * 192;
            if (e < 3 * CH * RK) {
                const int mtx = e / (CH * RK), rr = (e / RK) % CH, c8 = (e % RK) * 8;
                op_t* dst = reinterpret_cast<op_t*>(sb + (mtx == 0 ? L::kh : mtx == 1 ? L::kt : L::qh)) + rr * KP;
                *reinterpret_cast<opx4*>(dst + pcol(c8)) = opx4{x.xk[p][0], x.xk[p][1], x.xk[p][2], x.xk[p][3]};
                *reinterpret_cast<opx4*>(dst + pcol(c8 + 4)) = opx4{x.xk[p][4], x.xk[p][5], x.xk[p][6], x.xk[p][7]};
            }
        }
#pragma unroll
        for (int p = 0; p < NM; ++p) {
            const int e = lt + p * 192;
            if (e < 2 * CH * 8) {
                const int mtx = e / (CH * 8), rr = (e / 8) % CH, c8 = (e % 8) * 8;
                op_t* dst = reinterpret_cast<op_t*>(sb + (mtx == 0 ? L::tm : L::aq)) + rr * CP;
                *reinterpret_cast<opx4*>(dst + pcol(c8)) = opx4{x.xm[p][0], x.xm[p][1], x.xm[p][2], x.xm[p][3]};
                *reinterpret_cast<opx4*>(dst + pcol(c8 + 4)) = opx4{x.xm[p][4], x.xm[p][5], x.xm[p][6], x.xm[p][7]};
            }
        }
        // V rows past T are zero
        const int t0 = c * CH, n = min(CH, T_len - t0);
        if (lt < 2 * CH) {
            const int rr = lt / 2, c8 = (lt % 2) * 8;
            *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(sb + L::v) + rr * L::VP + c8) = rr < n ? x.xv : bf16x8{};
        }
        // row vectors: beta (V_B, V_BEG: e^gc is inside Kh), ones (V_ED, V_EG), e^gL per channel
        float* vs = reinterpret_cast<float*>(sb + L::vec);
        if (lt < CH) {
            vs[V_B * CH + lt] = x.bt;
            vs[V_BEG * CH + lt] = x.bt;
            vs[V_ED * CH + lt] = 1.f;
            vs[V_EC * CH + lt] = 1.f;
            vs[V_EG * CH + lt] = 1.f;
        }
        float* ech = reinterpret_cast<float*>(sb + L::ech);
#pragma unroll
        for (int p = 0; p < NE; ++p)
            if (lt + p * 192 < DK) ech[lt + p * 192] = x.el[p];
    };

    floatx4 hacc[1][DK / 16];
    Stage pre;
    if (w == 0) {
        load_state<DK, DV, 1>(hacc, s0, head, c0, lane);
    } else {
        load(0, pre);
        store(0, pre);
        load(min(1, NT - 1), pre);
    }
    __syncthreads();
    for (int n = 0; n < NT; ++n) {
        if (w == 0) {
            const unsigned char* sb = smem + (size_t)(n & 1) * L::slot;
            const op_t* Kh = reinterpret_cast<const op_t*>(sb + L::kh);
            const op_t* Kt = reinterpret_cast<const op_t*>(sb + L::kt);
            const op_t* Qh = reinterpret_cast<const op_t*>(sb + L::qh);
            const op_t* Tm = reinterpret_cast<const op_t*>(sb + L::tm);
            const op_t* Aq = reinterpret_cast<const op_t*>(sb + L::aq);
            const bf16* Vs = reinterpret_cast<const bf16*>(sb + L::v);
            const float* vs = reinterpret_cast<const float*>(sb + L::vec);
            const float* ech = reinterpret_cast<const float*>(sb + L::ech);
            const int ln = lane & 15, lg = lane >> 4;
            const int t0 = n * CH;
            opx8 hb[1][DK / 32], db[1][2], dtb[1][2];
            chain_delta<DK, 1, L::VP, false, true>(hacc, Kh, Vs,
                                                   [&](int mt, int cb) { return frag(Tm, CP, 16 * mt + ln, 32 * cb, lg); },
                                                   vs, lane, hb, db, dtb, nullptr, ech);
            chain_out<DK, 1>(hb, db, Qh, [&](int ct, int cb) { return frag(Aq, CP, 16 * ct + ln, 32 * cb, lg); }, vs + V_EG * CH, o + ((size_t)b * T_len * Hv + j) * DV + c0 + (size_t)t0 * v_row,
                             v_row, min(CH, T_len - t0), lane);
            chain_update<DK, 1>(hacc, Kt, dtb, lane);
        } else {
            if (n + 1 < NT) store(n + 1, pre);
            load(min(n + 2, NT - 1), pre);
        }
        __syncthreads();
    }
    if (w == 0) store_state<DK, DV, 1>(hacc, sf, head, c0, lane);
}

template <typename T, int DK, int DV>
hipError_t launch_kda_mfma_t(const KdaArgs& a, void* ws, hipStream_t st)
{
    const int NT = (int)(((long)a.T + CH - 1) / CH);
    const int grp = a.Hv / a.Hqk;
    auto prep = kda_prep_kernel<T, DK>;
    constexpr size_t pl = kda_prep_lds_bytes<DK>();
    static_assert(pl <= 160 * 1024, "LDS budget");
    hipError_t e = hipFuncSetAttribute((const void*)prep, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep, dim3((unsigned)((long)a.B * a.Hv * NT)), dim3(KQ_NT), pl, st, (const T*)a.q,
                       (const T*)a.k, a.g, a.beta, (unsigned char*)ws, a.T, a.Hqk, a.Hv, grp, NT, a.scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    using L = KsLds<DK>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    auto kern = kda_state_kernel<DK, DV>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)((long)a.B * a.Hv * (DV / 16))), dim3(256), L::bytes, st,
                       (const bf16*)a.v, (const unsigned char*)ws, a.s0, a.sf, (bf16*)a.o, a.T, a.Hv, NT);
    return hipGetLastError();
}

}  // namespace

bool kda_mfma_supported(const KdaArgs& a)
{
    return a.dtype_bf16 && a.chunk == CH && (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128);
}

size_t kda_mfma_workspace_bytes(int B, int T, int Hv, int dk)
{
    const size_t NT = ((size_t)T + CH - 1) / CH;
    const size_t per = dk == 128 ? KdaWs<128>::bytes : KdaWs<64>::bytes;
    return (size_t)B * Hv * NT * per;
}

hipError_t launch_kda_mfma(const KdaArgs& a, void* ws, hipStream_t st)
{
    if (a.dk == 128 && a.dv == 128) return launch_kda_mfma_t<bf16, 128, 128>(a, ws, st);
    if (a.dk == 128 && a.dv == 64) return launch_kda_mfma_t<bf16, 128, 64>(a, ws, st);
    if (a.dk == 64 && a.dv == 128) return launch_kda_mfma_t<bf16, 64, 128>(a, ws, st);
    if (a.dk == 64 && a.dv == 64) return launch_kda_mfma_t<bf16, 64, 64>(a, ws, st);
    return hipErrorInvalidValue;
}

// =======================================================================================
// The backward pass's two sequential passes on the float16 matrix cores (bf16 inputs, chunks of
// 32 tokens, the backward's own chunking): the states entering every chunk (the forward chunk
// step again, without its output) and the reverse state pass, which stores each chunk's
// exit-state gradient and finally dS0 (the algebra is in chunk_bwd.hip's header).  The chunk
// matrices come formed from the backward's gram kernel (float32 A, M, G, T and the decay
// exponentials per (batch, value head, chunk)); T itself is applied, not a substitution with A.
// Per chunk of the reverse pass (rows r of the chunk, dh' the exit-state gradient, 16 columns
// per chain wave):
//   dDelta = diag(e^(gL - gc)) K dh' + M^T dO,   dR = T^T dDelta,
//   dh = e^gL dh' + (scale Q)^T diag(e^gc) dO - K^T diag(beta e^gc) dR.
// One workgroup per (batch, value head, 32-column tile) and pass: two chain waves of 16 columns
// and four loader waves that stage the next chunk (K; Q and dO, or V; T or its transpose; M^T; the
// row vectors) into double-buffered LDS, one barrier per chunk.  The operands are float16 in
// the layouts of the forward kernels (column-permuted rows; perm-K fragments), rows past the
// sequence zero.
constexpr int BC = 32;                        // chunk length of the backward
constexpr int B16_NTH = 384;                  // two chain waves, four loader waves
constexpr int BC_AWS = 4 * BC * BC + 2 * BC;  // floats per chunk of the gram kernel's output

template <int DK>
struct B16Lds {
    static constexpr int KP = DK + 8;    // K and Q rows, column-permuted f16
    static constexpr int MP = BC + 8;    // [32][MP] f16: T (or T^T) and M^T, column-permuted
    static constexpr int VP = 32 + 16;   // the tile's V or dO rows, bf16
    static constexpr size_t kq = (size_t)BC * KP * 2;
    static constexpr size_t mm = (size_t)BC * MP * 2;
    static constexpr size_t k = 0, q = k + kq, t = q + kq, m = t + mm, v = m + mm;
    static constexpr size_t vec = v + (size_t)BC * VP * 2;   // beta, e^gc, e^(gL - gc): [3][32] f32
    static constexpr int HSP = DK + 8;                        // the chain waves' state, [32 columns][HSP] f16
    static constexpr size_t hst = vec + 3 * BC * 4;
    static constexpr size_t slot = hst + (size_t)32 * HSP * 2;
    static constexpr size_t bytes = 2 * slot;
    static_assert(q % 16 == 0 && t % 16 == 0 && m % 16 == 0 && v % 16 == 0 && vec % 16 == 0 && hst % 16 == 0 &&
                      slot % 16 == 0,
                  "16-byte aligned parts");
};

template <int DK, int DV>
__global__ __launch_bounds__(B16_NTH) void bwd_pass16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                         const bf16* __restrict__ v, const float* __restrict__ beta,
                                                         const float* s0, const bf16* __restrict__ dout,
                                                         const float* dsf, float* __restrict__ H,
                                                         float* __restrict__ dH, float* ds0,
                                                         const float* __restrict__ Aw, int T_len, int Hqk, int Hv,
                                                         int grp, float scale, int nblk)
{
    using L = B16Lds<DK>;
    constexpr int NTILE = DV / 32;
    constexpr int MT = DK / 16, KB = DK / 32;
    constexpr int NLT = B16_NTH - 128;       // loader threads
    constexpr int RP = DK / 16;              // 32-byte pair-runs per K row
    constexpr int PK = (BC * RP + NLT - 1) / NLT;   // pair-runs per loader thread
    static_assert(BC * BC == 4 * NLT, "one float4 of T and of M per loader thread");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const bool rev = (int)blockIdx.x >= nblk;
    const int x = rev ? (int)blockIdx.x - nblk : (int)blockIdx.x;
    const size_t head = (size_t)(x / NTILE);   // b * Hv + j
    const int c0 = (x % NTILE) * 32;
    const int b = (int)(head / Hv), j = (int)(head % Hv), i = j / grp;
    const int NT = (T_len + BC - 1) / BC;
    const int w = threadIdx.x >> 6;
    const size_t qk_row = (size_t)Hqk * DK, v_row = (size_t)Hv * DV;
    const size_t tok0 = (size_t)b * T_len;
    auto slot = [&](int n) { return smem + (size_t)(n & 1) * L::slot; };
    auto chunk_of = [&](int n) { return rev ? NT - 1 - n : n; };

    // the loader role, compiled once per pass (REV: the reverse pass)
    auto loaders = [&](auto rev_c) {
        constexpr bool REV = decltype(rev_c)::value;
        const int lt = (int)threadIdx.x - 128;
        struct Buf {
            bf16x8 rk[PK][2], rq[PK][2];
            bf16x8 rv;
            floatx4 rt, rm;
            float rvec;
        };
        // Every loader thread of a pass issues the same loads in every step, whatever its role
        // (the V and vector loads it does not stage read a valid address and are dropped), so
        // that each wait before staging covers exactly the loads of the chunk being staged and
        // none of those in flight behind it.  With loads under branches the compiler is left a
        // smaller count of loads in flight to wait for, down to all of them.
        auto load = [&](int c, Buf& r) {
            const int t0 = c * BC, n = min(BC, T_len - t0);
#pragma unroll
            for (int p = 0; p < PK; ++p) {
                const int s = min(lt + p * NLT, BC * RP - 1), row = min(s / RP, n - 1), pr = s % RP;
                const size_t off = (tok0 + t0 + row) * qk_row + (size_t)i * DK + 32 * (pr >> 1) + 8 * (pr & 1);
                r.rk[p][0] = *reinterpret_cast<const bf16x8*>(k + off);
                r.rk[p][1] = *reinterpret_cast<const bf16x8*>(k + off + 16);
                if constexpr (REV) {
                    r.rq[p][0] = *reinterpret_cast<const bf16x8*>(q + off);
                    r.rq[p][1] = *reinterpret_cast<const bf16x8*>(q + off + 16);
                }
            }
            {   // the tile's V or dO rows (staged by the first two loader waves)
                const int row = min((lt & 127) / 4, n - 1), c8 = (lt % 4) * 8;
                r.rv = *reinterpret_cast<const bf16x8*>((REV ? dout : v) + (tok0 + t0 + row) * v_row + (size_t)j * DV + c0 + c8);
            }
            // T and M, four consecutive elements of a row per thread (coalesced); the reverse
            // pass transposes them as it writes them to LDS
            const float* aw = Aw + (head * NT + c) * BC_AWS;
            r.rt = ld4s(aw + 3 * BC * BC + 4 * lt);
            if constexpr (REV) r.rm = ld4s(aw + BC * BC + 4 * lt);
            // row vectors: beta (from the input; rows past the sequence clamped here and zeroed
            // when staged), e^gc, e^(gL - gc)
            r.rvec = *(lt < BC ? beta + (tok0 + t0 + min(lt, n - 1)) * Hv + j : aw + 4 * BC * BC + min(lt - BC, 2 * BC - 1));
        };
        auto stage = [&](int c, int n_slot, const Buf& r) {
            unsigned char* sb = slot(n_slot);
            const int n = min(BC, T_len - c * BC);
            op_t* Ks = reinterpret_cast<op_t*>(sb + L::k);
            op_t* Qs = reinterpret_cast<op_t*>(sb + L::q);
#pragma unroll
            for (int p = 0; p < PK; ++p) {
                const int s = lt + p * NLT, row = s / RP, pr = s % RP;
                if (s >= BC * RP) break;
                opx8 r0, r1;
                bf16_pair_to_op(r.rk[p][0], r.rk[p][1], r0, r1);
                if (row >= n) r0 = r1 = opx8{};
                opx8* dk_ = reinterpret_cast<opx8*>(Ks + row * L::KP + 16 * pr);
                dk_[0] = r0;
                dk_[1] = r1;
                if constexpr (REV) {
                    bf16_pair_to_op(r.rq[p][0], r.rq[p][1], r0, r1);
                    if (row >= n) r0 = r1 = opx8{};
                    opx8* dq_ = reinterpret_cast<opx8*>(Qs + row * L::KP + 16 * pr);
                    dq_[0] = r0;
                    dq_[1] = r1;
                }
            }
            if (lt < 128) {
                const int row = lt / 4, c8 = (lt % 4) * 8;
                *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(sb + L::v) + row * L::VP + c8) =
                    row < n ? r.rv : bf16x8{};
            }
            op_t* Ts = reinterpret_cast<op_t*>(sb + L::t);
            op_t* Ms = reinterpret_cast<op_t*>(sb + L::m);
            {
                // elements (rr, cc .. cc + 3) of T: at (rr, cc) in the forward pass, at (cc, rr)
                // (T^T, and M^T) in the reverse one
                const int rr = (4 * lt) / BC, cc = (4 * lt) % BC;
                if constexpr (REV) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Ts[(cc + e) * L::MP + pcol(rr)] = (op_t)r.rt[e];
                        Ms[(cc + e) * L::MP + pcol(rr)] = (op_t)r.rm[e];
                    }
                } else {
                    // four consecutive logical columns stay adjacent under the permutation
                    *reinterpret_cast<opx4*>(Ts + rr * L::MP + pcol(cc)) =
                        opx4{(op_t)r.rt[0], (op_t)r.rt[1], (op_t)r.rt[2], (op_t)r.rt[3]};
                }
            }
            if (lt < 3 * BC) reinterpret_cast<float*>(sb + L::vec)[lt] = lt < BC && lt >= n ? 0.f : r.rvec;
        };
        // the state (or state gradient) the chain waves put in slot n during step n, float16,
        // transposed, to H (dH): the tile's 32 columns of the chunk's [dv][dk] block are one
        // contiguous run, copied in 16-byte pieces
        auto copy_out = [&](int n) {
            const op_t* src = reinterpret_cast<const op_t*>(slot(n) + L::hst);
            op_t* dst = reinterpret_cast<op_t*>(REV ? dH : H) + ((head * NT + chunk_of(n)) * DV + c0) * DK;
            constexpr int R8 = DK / 8;   // 16-byte pieces per column
            static_assert(32 * R8 % NLT == 0, "whole copies per loader thread");
#pragma unroll
            for (int p = 0; p < 32 * R8 / NLT; ++p) {
                const int e = lt + p * NLT, col = e / R8, k8 = e % R8;
                *reinterpret_cast<opx8*>(dst + (size_t)col * DK + 8 * k8) =
                    *reinterpret_cast<const opx8*>(src + col * L::HSP + 8 * k8);
            }
        };
        // step n stages step n + 1 from buffer (n + 1) % 2, loads step n + 3 into it (two chunks
        // of loads in flight, clamped to the last step, as in the forward state pass), then copies
        // out the state of step n - 1 (in the first step, that of step 0 before it is written; the
        // second step writes it again, from the same threads)
        Buf bA, bB;
        if (NT > 0) {
            load(chunk_of(0), bA);
            stage(chunk_of(0), 0, bA);
            load(chunk_of(min(1, NT - 1)), bB);
            load(chunk_of(min(2, NT - 1)), bA);
        }
        lds_barrier();
        auto step = [&](int n, Buf& r) {
            if (n + 1 < NT) stage(chunk_of(n + 1), n + 1, r);
            load(chunk_of(min(n + 3, NT - 1)), r);
            copy_out(max(n - 1, 0));
            lds_barrier();
        };
        int n = 0;
        for (; n + 1 < NT; n += 2) {
            step(n, bB);
            step(n + 1, bA);
        }
        if (n < NT) step(n, bB);
        if (NT > 0) copy_out(NT - 1);
    };

    if (w >= 2) {
        // ================================================================= loader waves
        if (rev)
            loaders(std::true_type{});
        else
            loaders(std::false_type{});
    } else {
        // ================================================================= chain waves
        const int col = c0 + 16 * w;
        floatx4 hacc[1][MT];
        load_state<DK, DV, 1>(hacc, rev ? dsf : s0, head, col, threadIdx.x & 63);
        lds_barrier();
        for (int n = 0; n < NT; ++n) {
            const int lane = opaque(threadIdx.x & 63), ln = lane & 15, lg = lane >> 4;
            const unsigned char* sb = slot(n);
            const op_t* Ks = reinterpret_cast<const op_t*>(sb + L::k);
            const op_t* Qs = reinterpret_cast<const op_t*>(sb + L::q);
            const op_t* Ts = reinterpret_cast<const op_t*>(sb + L::t);
            const op_t* Ms = reinterpret_cast<const op_t*>(sb + L::m);
            const bf16* Vs = reinterpret_cast<const bf16*>(sb + L::v) + 16 * w;
            const float* vs = reinterpret_cast<const float*>(sb + L::vec);
            // this chunk's state (forward) or exit-state gradient (reverse) for the gradient kernel:
            // float16, transposed, [B, Hv, NT, dv, dk], into the slot, from where the loader waves
            // copy it out in the next step with coalesced 16-byte stores.  These stores are the
            // pass's largest traffic; float16 halves them, and the values are the float16 operands
            // the pass itself multiplies with.
            {
                op_t* sp = reinterpret_cast<op_t*>(slot(n) + L::hst) + (16 * w + ln) * L::HSP + 4 * lg;
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    *reinterpret_cast<opx4*>(sp + 16 * m) =
                        opx4{(op_t)hacc[0][m][0], (op_t)hacc[0][m][1], (op_t)hacc[0][m][2], (op_t)hacc[0][m][3]};
            }
            opx8 hb[KB];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) hb[kk] = pack_perm(hacc[0][2 * kk], hacc[0][2 * kk + 1]);
            // K h (or K dh'): the chunk's two 16-row tiles
            floatx4 X[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) X[mt] = mfma32(frag(Ks, L::KP, 16 * mt + ln, 32 * kk, lg), hb[kk], X[mt]);
            // V (or dO) rows 16mt + 4lg .. +3 of this lane's column; the row vectors
            bf16x4 vr[2];
            floatx4 bt[2], eg[2], ed[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                vr[mt] = __builtin_bit_cast(bf16x4, ld_tr(Vs + (16 * mt + 4 * lg + (ln >> 2)) * L::VP + 4 * (ln & 3)));
                bt[mt] = ld4s(vs + 16 * mt + 4 * lg);
                eg[mt] = ld4s(vs + BC + 16 * mt + 4 * lg);
                ed[mt] = ld4s(vs + 2 * BC + 16 * mt + 4 * lg);
            }
            const float eL = vs[BC + BC - 1];
            floatx4 Y[2];
            if (!rev) {
                // R = beta V - beta e^gc K h, Delta = T R, h <- e^gL h + K^T diag(e^(gL - gc)) Delta
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Y[mt][e] = bt[mt][e] * ((float)vr[mt][e] - eg[mt][e] * X[mt][e]);
                const opx8 rb = pack_perm(Y[0], Y[1]);
                floatx4 D[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    D[mt] = mfma32(frag(Ts, L::MP, 16 * mt + ln, 0, lg), rb, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) D[mt][e] *= ed[mt][e];
                const opx8 db = pack_perm(D[0], D[1]);
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) hacc[0][m][e] *= eL;
#pragma unroll
                for (int m = 0; m < MT; ++m) hacc[0][m] = mfma32(frag_kt(Ks, L::KP, m, 0, lane), db, hacc[0][m]);
            } else {
                // dDelta = diag(e^(gL - gc)) K dh' + M^T dO, dR = T^T dDelta,
                // dh = e^gL dh' + (scale Q)^T diag(e^gc) dO - K^T diag(beta e^gc) dR
                const opx8 dob = to_op(vr[0], vr[1]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const floatx4 P = mfma32(frag(Ms, L::MP, 16 * mt + ln, 0, lg), dob, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) Y[mt][e] = ed[mt][e] * X[mt][e] + P[e];
                }
                const opx8 ddb = pack_perm(Y[0], Y[1]);
                floatx4 R[2], G[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    R[mt] = mfma32(frag(Ts, L::MP, 16 * mt + ln, 0, lg), ddb, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        R[mt][e] *= -bt[mt][e] * eg[mt][e];
                        G[mt][e] = scale * eg[mt][e] * (float)vr[mt][e];
                    }
                }
                const opx8 gb = pack_perm(G[0], G[1]), rb = pack_perm(R[0], R[1]);
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) hacc[0][m][e] *= eL;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    hacc[0][m] = mfma32(frag_kt(Qs, L::KP, m, 0, lane), gb, hacc[0][m]);
                    hacc[0][m] = mfma32(frag_kt(Ks, L::KP, m, 0, lane), rb, hacc[0][m]);
                }
            }
            lds_barrier();
        }
        if (rev) store_state<DK, DV, 1>(hacc, ds0, head, col, threadIdx.x & 63);
    }
}

template <int DK, int DV>
hipError_t launch_bwd_pass16_t(const BwdArgs& a, float* H, float* dH, const float* Aw, hipStream_t st)
{
    using L = B16Lds<DK>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    auto kern = bwd_pass16_kernel<DK, DV>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    const int nblk = a.B * a.Hv * (DV / 32);
    hipLaunchKernelGGL(kern, dim3((unsigned)(2 * nblk)), dim3(B16_NTH), L::bytes, st, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, a.beta, a.s0, (const bf16*)a.dout, a.dsf, H, dH, a.ds0, Aw, a.T, a.Hqk,
                       a.Hv, a.Hv / a.Hqk, a.scale, nblk);
    return hipGetLastError();
}

bool bwd_pass16_supported(const BwdArgs& a)
{
    return a.dtype_bf16 && (a.dk_ == 64 || a.dk_ == 128) && (a.dv_ == 32 || a.dv_ == 64 || a.dv_ == 128);
}

hipError_t launch_bwd_pass16(const BwdArgs& a, float* H, float* dH, const float* Aw, hipStream_t st)
{
#define GDN_B16_CASE(DK_, DV_) \
    if (a.dk_ == DK_ && a.dv_ == DV_) return launch_bwd_pass16_t<DK_, DV_>(a, H, dH, Aw, st);
    GDN_B16_CASE(64, 32) GDN_B16_CASE(64, 64) GDN_B16_CASE(64, 128)
    GDN_B16_CASE(128, 32) GDN_B16_CASE(128, 64) GDN_B16_CASE(128, 128)
#undef GDN_B16_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn

#ifdef GDN_PHASE_TRACE
extern "C" int gdn_phase_trace_read(long long* host)
{
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn::gdn_phase_ts), sizeof(gdn::gdn_phase_ts), 0,
                                    hipMemcpyDeviceToHost);
}
#endif

#ifdef GDN_DEBUG
namespace gdn {
namespace {
// one failed check at the given bit, and nothing else: the flags' path end to end
__global__ void debug_fail_kernel(int bit) { GDN_CHECK(threadIdx.x != 0, bit); }
}  // namespace
}  // namespace gdn

extern "C" int gdn_debug_self_test(int bit)
{
    if (bit < 0 || bit > 31) return -1;
    hipLaunchKernelGGL(gdn::debug_fail_kernel, dim3(1), dim3(64), 0, nullptr, bit);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The index checks that failed since the last call (bits as in GDN_CHECK), then cleared; the
// current device's copy.  Exported only by the debug build.
extern "C" unsigned int gdn_debug_take_flags(void)
{
    unsigned int h = 0;
    const unsigned int z = 0;
    if (hipDeviceSynchronize() != hipSuccess) return 0xffffffffu;
    if (hipMemcpyFromSymbol(&h, HIP_SYMBOL(gdn::gdn_debug_flags), sizeof(h)) != hipSuccess) return 0xffffffffu;
    if (hipMemcpyToSymbol(HIP_SYMBOL(gdn::gdn_debug_flags), &z, sizeof(z)) != hipSuccess) return 0xffffffffu;
    return h;
}
#endif
