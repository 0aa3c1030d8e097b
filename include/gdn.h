/*
 * gdn.h -- C ABI of libgdn.so: the gated delta rule (Gated DeltaNet core) on AMD MI355X (gfx950).
 *
 * The operation ("Architecture Thread I: Gated Attention, DeltaNet, and Hybrid Models", section
 * "Gated DeltaNet", state-update equation; restated in "Gated Attention Architectures",
 * section 3 "Gated DeltaNet", Mathematical Formulation), per batch row b and value head j:
 *
 *     S_t = S_{t-1} ( alpha_t (I - beta_t k_t k_t^T) ) + beta_t v_t k_t^T,      o_t = S_t q_t
 *
 * with S_t in R^{dv x dk}, alpha_t = exp(g_t) the decay gate and beta_t the write strength.  The
 * readout o_t = S_t q_t is the linear-attention readout of "Gated Attention Architectures",
 * section 1.  This library stores the state transposed, h = S^T, as [dk, dv] per head (the
 * [d_k, d_v] memory of "Decoding Next-Generation LLM Architectures", section 3.2).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library never allocates,
 *    frees, or keeps a pointer after the call returns.  Tensors are dense, contiguous, row-major
 *    in the layouts given.  q, k, v, o and the states must be 16-byte aligned; g and beta
 *    4-byte aligned.
 *  - q, k, v and o share one dtype (gdn_dtype_t).  g = log alpha, beta and the state are float32.
 *  - Gate range.  g <= 0 (alpha in [0, 1], the decay gate); g = -inf (alpha = 0: the state is
 *    cleared, "Gated Attention Architectures", section 3) is accepted.  The prefill kernels raise
 *    g to at least -100 before use: exp(-100) lies below float32's normal range, so this changes
 *    no result beyond float32 rounding, and it keeps differences of in-chunk sums of g finite.
 *    beta in [0, 1] (the write strength).  g > 0 (alpha > 1, a growing state) is outside the
 *    supported range of the bf16 matrix-core routes below; the float32 routes and decode accept it
 *    while every value stays finite in float32.
 *  - Operand range of the bf16 matrix-core routes (gdn_chunk_fwd_kernel_name "mfma_pipe",
 *    "mfma", "mfma_split", "mfma_scan"; gdn_chunk_fwd_gated, _varlen, _scan, gdn_chunk_transport and
 *    gdn_kda_chunk_fwd at chunk 64).  Their products take float16 operands (the same matrix-core
 *    rate as bf16 with a 3-bit longer significand) and accumulate in float32.  The operands are
 *    q, k, v, the state, (I + A)^{-1}, and per chunk R = beta (v - e^gc k^T h) and
 *    Delta = (I + A)^{-1} R, so every one of them must stay below 65504 in magnitude.  With
 *    L2-normalised q and k, g <= 0 and beta in [0, 1] (the intended use: "Architecture Thread I",
 *    section "Modern Architecture Improvements", normalises q and k before the recurrence) that
 *    holds while |v| and the entries of the state stay below about 2^11 (the tests run |v| and
 *    |initial_state| up to 2^10).  Outside that range the float16 operands may overflow and the
 *    results are unspecified (inf or NaN may appear); the float32 route has no such limit.  bf16
 *    components of q and k below 2^-14 in magnitude become float16 subnormals (absolute error at
 *    most 2^-25, negligible next to a unit-norm row).
 *  - Grouped heads: Hv must be a multiple of Hqk; value head j reads query/key head
 *    floor(j / (Hv / Hqk)) (contiguous groups).
 *  - q is multiplied by `scale` before the readout (1.0 gives o_t = S_t q_t exactly).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call returns
 *    without synchronising.  Results are valid once the stream has completed the work.
 *  - Errors: every argument is validated before any device work is enqueued.  On an error
 *    status nothing is enqueued and no output is touched.  GDN_ERR_LAUNCH means a kernel launch
 *    failed; outputs are then undefined.
 *  - The library is deterministic (no atomics: identical inputs give bit-identical outputs),
 *    thread-safe and reentrant.  Calls that share output buffers must not overlap.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,       /* a size is negative / zero where not allowed, or Hv % Hqk != 0 */
    GDN_ERR_UNSUPPORTED = 3, /* head dim, chunk size or dtype outside the compiled variants */
    GDN_ERR_ALIGN = 4,       /* a tensor is not 16-byte aligned (g, beta: 4-byte) */
    GDN_ERR_WORKSPACE = 5,   /* workspace smaller than gdn_chunk_fwd_workspace_bytes() */
    GDN_ERR_ALIAS = 6,       /* an output overlaps an input it may not overlap */
    GDN_ERR_NO_DEVICE = 7,   /* no HIP device is visible */
    GDN_ERR_LAUNCH = 8       /* a kernel launch failed (hipGetLastError) */
} gdn_status_t;

typedef enum {
    GDN_F32 = 0,   /* q, k, v, o are float32 */
    GDN_BF16 = 1   /* q, k, v, o are bfloat16; products accumulate in float32 (operand range above) */
} gdn_dtype_t;

/*
 * gdn_chunk_fwd_workspace_bytes -- device scratch (bytes) that gdn_chunk_fwd needs for these
 * sizes; 0 when the path chosen for them needs none.  The split matrix-core path (few, long
 * sequences: see gdn_chunk_fwd_kernel_name) needs, per 64-token chunk of each batch row,
 * 13,568 bytes per value head (T = (I + A)^{-1}, the masked Q K^T and the gate vectors) plus
 * 128 * dk bytes per query/key head (q as matrix-core operands), all built before the state
 * pass reads them; rows of at least 256 chunks whose state pass leaves at least 32 of 256
 * compute units free are run in pieces of 128 chunks (each piece's operands built beside the
 * previous piece's state pass), and then B * Hv * dk * dv * 4 bytes more hold the state handed
 * from piece to piece.  When the chains are too few to fill the GPU and long (gdn_chunk_fwd_kernel_name says
 * "mfma_scan") it is gdn_chunk_fwd_scan_workspace_bytes for the segment count chosen.  The result
 * depends only on the arguments.  Pure host function; needs no device; 0 for invalid sizes.
 */
size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                     gdn_dtype_t dtype);

/*
 * gdn_chunk_fwd -- prefill: run the gated delta rule over T tokens for B sequences.
 *
 * Computed chunkwise ("Gated Attention Architectures", section 3: the DeltaNet WY representation
 * extended with per-chunk cumulative decay products gamma_j = prod of alpha_i from the chunk
 * start to position j).  Per chunk of `chunk` positions the kernels take the per-chunk
 * log-decay cumsum, form the strictly lower matrix A = tril(diag(beta)(K K^T * Gamma), -1) with
 * Gamma_ri = exp(gc_r - gc_i), apply (I + A)^{-1} (the UT/WY transform), carry the state across
 * chunks in float32, and form O = (Q * exp(gc)) h + (Q K^T * Gamma) Delta.  The result equals the
 * token-by-token recurrence up to rounding.
 *
 *   q, k           [B, T, Hqk, dk]   dtype
 *   v              [B, T, Hv,  dv]   dtype
 *   g, beta        [B, T, Hv]        float32   (g = log alpha_t)
 *   initial_state  [B, Hv, dk, dv]   float32, or NULL for a zero initial state
 *   final_state    [B, Hv, dk, dv]   float32 output, or NULL to skip; may equal initial_state
 *                                    (updated in place) but may not partially overlap it
 *   o              [B, T, Hv, dv]    dtype output; must not overlap any other argument
 *   chunk          16, 32 or 64.  T need not be a multiple of chunk (the last chunk is partial).
 *   dk, dv         32, 64 or 128 each.
 *   workspace      device scratch of at least gdn_chunk_fwd_workspace_bytes(...) bytes (16-byte
 *                  aligned, owned by the caller, contents need not be initialised and are
 *                  undefined afterwards; must not overlap any other argument), or NULL when
 *                  that is 0.  Calls sharing a workspace must not overlap in time.
 *   stream         hipStream_t (as void*), NULL for the default stream.
 * B == 0 is a no-op.  T == 0 writes final_state (a copy of initial_state, or zeros) and no o.
 */
gdn_status_t gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* initial_state, float* final_state,
                           void* o, int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                           gdn_dtype_t dtype, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Size of the fixed device array gdn_chunk_fwd_noalloc uses as its workspace (64 MiB per device). */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd for callers that cannot allocate device memory (code
 * under HIP stream or graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and results, with no workspace argument.  Where gdn_chunk_fwd needs
 * a workspace, this call uses a fixed array of GDN_NOALLOC_SCRATCH_BYTES that the library holds
 * on each device it runs on (from the time its code is loaded there until the process ends); it
 * calls no allocating routine.  The array's device address is looked up once per device, on the
 * first call that needs it.
 *   every argument       as gdn_chunk_fwd (caller-owned inputs and outputs; `stream`'s device,
 *                        or the current device for the null stream, runs the work)
 * Limit: sizes for which gdn_chunk_fwd_workspace_bytes exceeds GDN_NOALLOC_SCRATCH_BYTES return
 * GDN_ERR_WORKSPACE before anything is enqueued (the fused and float32 routes need none, so
 * only the split and scan routes of long sequences with few chains can hit it).  All calls on one
 * device share that device's array and each leaves its contents behind (nothing in it needs to
 * start at zero): calls on one device that overlap in time (other streams, other threads) race
 * on it and must be serialised by the caller.  Other errors as gdn_chunk_fwd.
 */
gdn_status_t gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* initial_state, float* final_state,
                                   void* o, int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                   gdn_dtype_t dtype, float scale, void* stream);

/*
 * gdn_recurrent_step -- decode: one token per sequence, state updated in place.
 *
 * One pass over the state per head (decoding is memory-bound: "The Transformer Isn't Alone
 * Anymore", section "The hidden consequence: long context"; per-step cost O(d^2):
 * "Gated Attention Architectures", summary comparison table).  Using the erase/write form of
 * the update ("Architecture Thread I", DeltaNet section) with h = S^T:
 *     u = h^T k,  delta = beta (v - alpha u),  h <- alpha h + k delta^T,  o = h^T (scale q)
 *
 *   q, k    [B, Hqk, dk]    dtype
 *   v       [B, Hv, dv]     dtype
 *   g, beta [B, Hv]         float32
 *   state   [B, Hv, dk, dv] float32, read and overwritten in place
 *   o       [B, Hv, dv]     dtype output; must not overlap any other argument
 *   dk, dv  32, 64 or 128 each.
 * B == 0 is a no-op.
 */
gdn_status_t gdn_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, float* state, void* o, int B, int Hqk, int Hv,
                                int dk, int dv, gdn_dtype_t dtype, float scale, void* stream);

/*
 * gdn_chunk_fwd_kernel_name -- which kernel family gdn_chunk_fwd would run for these sizes:
 * "mfma_pipe" (one fused matrix-core kernel in which prep waves build chunk n + 1 while chain
 * waves carry chunk n; chosen when B * Hv >= 192), "mfma" (the fused matrix-core kernel of the
 * gated epilogue and of packed sequences with as many chains; gdn_chunk_fwd itself does not
 * choose it), "mfma_split" (a parallel per-chunk prep kernel, then the matrix-core state pass;
 * fewer chains), "mfma_scan" (the
 * affine chunk scan of gdn_chunk_fwd_scan: so few chains that 32-column tiles over dv + dk
 * columns give at most 128 workgroups, cut into p = 1 + 256 / (B * Hv * (dv + dk) / 32)
 * segments when T holds at least 8 p chunks), "mfma_f32" (the float32 kernel: the chunk algebra
 * in float32 with its dense products on the float32 matrix cores; float32 inputs, chunk != 64 or
 * head dim 32), or NULL when the sizes are unsupported.  The choice depends only on the
 * arguments.  Pure host function.
 */
const char* gdn_chunk_fwd_kernel_name(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                      gdn_dtype_t dtype);

/* gdn_status_string -- static, human-readable text for a status code (never NULL). */
const char* gdn_status_string(gdn_status_t status);

/*
 * gdn_qkv_prologue -- the steps between the q, k, v projections and the recurrence, in one
 * launch: a short causal depthwise convolution over time, SiLU, and for q and k an L2
 * normalisation over each head's channels ("Architecture Thread I: Gated Attention, DeltaNet,
 * and Hybrid Models", section "Modern Architecture Improvements": query/key take Linear ->
 * Short Conv -> SiLU -> L2 Norm, value Linear -> Short Conv -> SiLU).  Per channel c of token t:
 *     a = sum_{j=0}^{W-1} w[c][j] x[t - (W-1) + j]        (x before token 0: the conv state)
 *     y = silu(a) = a / (1 + exp(-a));   q, k:  y <- y / sqrt(sum over the head's channels y^2 + eps)
 *
 *   q_in, k_in [B, T, Hqk, dk] dtype     v_in [B, T, Hv, dv] dtype   (the projections' outputs)
 *   conv_q, conv_k [Hqk*dk, W] float32   conv_v [Hv*dv, W] float32   (channel-major taps, tap
 *                                         W-1 multiplies the current token; no bias)
 *   conv_state_in  [B, 2*Hqk*dk + Hv*dv, W-1] float32 or NULL (zeros): per channel (q's, then
 *                  k's, then v's) the W-1 inputs before token 0, oldest first
 *   conv_state_out same shape or NULL: the last W-1 inputs (of this call, after the state), for
 *                  a continuation; may not overlap conv_state_in (use two buffers in turn)
 *   q, k, v        outputs, shapes and dtype of the inputs; may not overlap any input or each
 *                  other
 *   W = width, 1..4.  dk, dv 32, 64 or 128.  eps >= 0.
 * All pointers are caller-owned device memory; tensors 16-byte aligned, float arrays 4-byte.
 * B == 0 is a no-op; T == 0 only writes conv_state_out (= conv_state_in, or zeros).
 * Errors as gdn_chunk_fwd (nothing is enqueued on an error).
 */
gdn_status_t gdn_qkv_prologue(const void* q_in, const void* k_in, const void* v_in, const float* conv_q,
                              const float* conv_k, const float* conv_v, const float* conv_state_in,
                              float* conv_state_out, void* q, void* k, void* v, int B, int T, int Hqk,
                              int Hv, int dk, int dv, int width, gdn_dtype_t dtype, float eps,
                              void* stream);

/*
 * gdn_gated_rmsnorm -- the step after the recurrence: RMSNorm over each value head's channels
 * ("Architecture Thread I", section "Modern Architecture Improvements", output normalisation),
 * times SiLU of the gate projection z (the gated RMSNorm of "The Transformer Isn't Alone
 * Anymore", Qwen3-Next reconstruction; the output gate of the Gated DeltaNet block in "Gated
 * Attention Architectures"):
 *     y = o / sqrt(mean over the head's dv channels of o^2 + eps) * w * silu(z)
 *
 *   o, z   [B, T, Hv, dv] dtype        y  [B, T, Hv, dv] dtype, may be o or z itself (in place)
 *          but may not overlap them otherwise, nor the weight
 *   weight [dv] float32 shared by the heads (weight_per_head 0) or [Hv, dv] (1).  A
 *          zero-centred weight (stored as 1 + delta) is passed as its value 1 + delta.
 *   dv 32, 64 or 128.  eps >= 0.
 * B == 0 or T == 0 is a no-op.  Errors as gdn_chunk_fwd.
 */
gdn_status_t gdn_gated_rmsnorm(const void* o, const void* z, const float* weight, int weight_per_head,
                               void* y, int B, int T, int Hv, int dv, gdn_dtype_t dtype, float eps,
                               void* stream);

/*
 * gdn_chunk_fwd_gated_workspace_bytes -- device scratch (bytes) that gdn_chunk_fwd_gated needs:
 * gdn_chunk_fwd's own, plus, where the gated RMSNorm cannot run inside the recurrence's kernel,
 * room for O (B*T*Hv*dv elements of dtype, after the first part rounded up to 256 bytes).  Pure
 * host function; 0 for invalid sizes.
 */
size_t gdn_chunk_fwd_gated_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                           gdn_dtype_t dtype);

/*
 * gdn_chunk_fwd_gated -- prefill followed by the layer's output normalisation: gdn_chunk_fwd's
 * O, then the gated RMSNorm of gdn_gated_rmsnorm,
 *     y = O / sqrt(mean over the head's dv channels of O^2 + eps) * w * silu(z),
 * with O rounded to dtype before the norm, as when the two calls run one after the other (same
 * sources as those two).  Where the fused matrix-core kernel holds whole value heads (bf16,
 * chunk 64, dk and dv 64 or 128, enough chains that gdn_chunk_fwd_kernel_name says "mfma_pipe")
 * the norm runs inside that kernel ("mfma") and O never reaches device memory; its O matches
 * gdn_chunk_fwd's (the pipelined kernel there) to the bf16 tolerance, not bit for bit, since the
 * two kernels round T and Aqk in different orders.  Otherwise O goes through the workspace and a
 * second kernel, and the result is bit for bit gdn_chunk_fwd followed by gdn_gated_rmsnorm.
 *
 *   q, k, v, g, beta, initial_state, final_state, sizes, chunk, dtype, scale: as gdn_chunk_fwd
 *   z              [B, T, Hv, dv] dtype, the gate projection
 *   norm_weight    [dv] float32 shared by the heads (weight_per_head 0) or [Hv, dv] (1)
 *   eps            >= 0
 *   y              [B, T, Hv, dv] dtype output; may be z itself (in place) but may not overlap
 *                  z otherwise, nor any other argument
 *   workspace      at least gdn_chunk_fwd_gated_workspace_bytes(...) bytes, as gdn_chunk_fwd
 * B == 0 is a no-op.  T == 0 writes final_state only.  Errors as gdn_chunk_fwd; a
 * weight_per_head other than 0 or 1 is GDN_ERR_SHAPE, a negative or NaN eps
 * GDN_ERR_UNSUPPORTED.
 */
gdn_status_t gdn_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* initial_state, float* final_state,
                                 const void* z, const float* norm_weight, int weight_per_head, float eps,
                                 void* y, int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                 gdn_dtype_t dtype, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * gdn_chunk_bwd_workspace_bytes -- device scratch (bytes) that gdn_chunk_bwd needs: the state
 * entering every 32-token chunk and the gradient of the state leaving it (2 * dk * dv floats per
 * chunk and value head), and per chunk and value head four 32 x 32 matrices (K K^T and Q K^T with
 * the decays and gates, and the inverse of the unit triangular system) and the chunk's 2 * 32
 * decay exponentials, float32: B * Hv * ceil(T / 32) * (2 * dk * dv + 4 * 32 * 32 + 2 * 32) * 4
 * bytes.  Pure host function; 0 for invalid sizes.
 */
size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, gdn_dtype_t dtype);

/*
 * gdn_chunk_bwd -- backward pass of gdn_chunk_fwd: the gradients of a loss L through O and the
 * final state, with respect to q, k, v, g, beta and the initial state.  Computed chunkwise by
 * reversing the forward chunk steps ("Gated Attention Architectures", section 3, names chunkwise
 * hardware-efficient training for Gated DeltaNet): the states entering every chunk are
 * recomputed, a reverse pass carries dL/dh from the last chunk to the first, and every chunk's
 * gradients then follow in parallel.  The result equals the gradient of the token-by-token
 * recurrence up to rounding; it does not depend on the forward call's chunk size.  For bf16
 * inputs with dk in {64, 128} and dv in {32, 64, 128} the two sequential passes (the state
 * recompute and the reverse pass) and the per-chunk products dDelta h^T, Delta dh^T and dO h^T
 * take float16 operands: besides the forward's operand range (above), grad_o, grad_final_state,
 * every state gradient dL/dh and the per-chunk Delta and dL/dDelta must stay below 65504 in
 * magnitude; the other per-chunk products are float32.
 *
 *   q, k, v, g, beta, initial_state, sizes, dtype, scale: as gdn_chunk_fwd (inputs)
 *   grad_o            [B, T, Hv, dv] dtype: dL/dO
 *   grad_final_state  [B, Hv, dk, dv] float32 dL/d(final state), or NULL for zero
 *   grad_q, grad_k    [B, T, Hqk, dk] dtype outputs (a query/key head's gradient sums over the
 *                     value heads of its group)
 *   grad_v            [B, T, Hv, dv] dtype output
 *   grad_g, grad_beta [B, T, Hv] float32 outputs (g = log alpha)
 *   grad_initial_state [B, Hv, dk, dv] float32 output, or NULL to skip
 *   workspace         at least gdn_chunk_bwd_workspace_bytes(...) bytes, 16-byte aligned
 * Outputs may not overlap any input, each other or the workspace.  Every output element is
 * written exactly once (no atomics): the result is deterministic.  B == 0 is a no-op; T == 0
 * writes grad_initial_state only (= grad_final_state, or zeros).  Errors as gdn_chunk_fwd.
 */
gdn_status_t gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           const float* initial_state, const void* grad_o, const float* grad_final_state,
                           void* grad_q, void* grad_k, void* grad_v, float* grad_g, float* grad_beta,
                           float* grad_initial_state, int B, int T, int Hqk, int Hv, int dk, int dv,
                           gdn_dtype_t dtype, float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_kda_chunk_fwd_workspace_bytes -- device scratch (bytes) gdn_kda_chunk_fwd needs: 0 for
 * chunks of 16 or 32; for chunk 64 (the matrix-core kernels) one block per (batch, value head,
 * chunk) of the chunk's decay-weighted operands in float16 (e^gc K, e^(gL-gc) K, e^gc q, T, the
 * masked Q K^T) and its beta and e^gL vectors: 3*64*dk*2 + 2*64*64*2 + 64*4 + dk*4 bytes.  Pure
 * host function; 0 for invalid sizes.
 */
size_t gdn_kda_chunk_fwd_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype);

/*
 * gdn_kda_chunk_fwd -- Kimi Delta Attention prefill: the delta rule with one decay per key
 * channel ("Gated Attention Architectures", section 8, Mathematical Formulation),
 *     S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t v_t k_t^T,   o_t = S_t^T (scale q_t),
 *     D_t = diag(exp(g_t)) over the dk key channels,
 * with S in R^{dk x dv} stored [B, Hv, dk, dv] (the layout of gdn_chunk_fwd's state).  With the
 * same decay on every channel of a head this is gdn_chunk_fwd's recurrence.  Computed
 * chunkwise: per chunk the pairwise decays exp(gc_r - gc_i) (per channel, from differences of
 * the in-chunk cumulative log decay) weight the K K^T and Q K^T products, (I + A)^{-1} is applied
 * by forward substitution, and the state is carried across chunks in float32.
 *
 *   q, k           [B, T, Hqk, dk]  dtype
 *   v              [B, T, Hv, dv]   dtype
 *   g              [B, T, Hv, dk]   float32, log alpha per key channel (<= 0 for a decay)
 *   beta           [B, T, Hv]       float32
 *   initial_state, final_state, o, scale, stream: as gdn_chunk_fwd
 *   chunk          16 or 32 (float32 vector kernel, any supported dtype and head dims 32, 64,
 *                  128), or 64 (matrix-core kernels: bf16, dk and dv 64 or 128; every in-chunk
 *                  operand carries a decay factor at most 1, so float16 operands hold them)
 *   workspace      at least gdn_kda_chunk_fwd_workspace_bytes(...) bytes (16-byte aligned,
 *                  caller-owned, not overlapping any other argument), or NULL when that is 0
 * B == 0 is a no-op; T == 0 writes final_state only.  Errors as gdn_chunk_fwd.
 */
gdn_status_t gdn_kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const float* initial_state, float* final_state, void* o, int B, int T, int Hqk,
                               int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype, float scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd_varlen_workspace_bytes -- device scratch (bytes) gdn_chunk_fwd_varlen needs: that
 * of gdn_chunk_fwd for N rows of max_seqlen tokens (0 when the path chosen needs none).  Pure
 * host function; 0 for invalid sizes.
 */
size_t gdn_chunk_fwd_varlen_workspace_bytes(int N, int max_seqlen, int Hqk, int Hv, int dk, int dv, int chunk,
                                            gdn_dtype_t dtype);

/*
 * gdn_chunk_fwd_varlen -- prefill of N packed sequences of different lengths in one call: the
 * recurrence of gdn_chunk_fwd run independently over each sequence (its own initial and final
 * state; no state flows from one sequence into the next), with the tokens of all sequences
 * concatenated along one axis.  Chunks start at each sequence's first token.
 *
 *   q, k           [total_T, Hqk, dk] dtype      v, o [total_T, Hv, dv] dtype
 *   g, beta        [total_T, Hv] float32
 *   cu_seqlens     [N + 1] int32, DEVICE memory: sequence n is tokens cu[n] .. cu[n+1]-1.  It must
 *                  hold 0 = cu[0] <= cu[1] <= ... <= cu[N] = total_T with every length at most
 *                  max_seqlen; the kernels clamp offsets into [0, total_T] and lengths into
 *                  [0, max_seqlen], so no access leaves the tensors, but other values give
 *                  unspecified results.  Empty sequences are allowed (final state = initial).
 *   initial_state, final_state [N, Hv, dk, dv] float32, as gdn_chunk_fwd (NULL allowed; in place
 *                  allowed)
 *   N              number of sequences; max_seqlen the longest (the work grid is sized by it)
 *   chunk, dtype, scale, sizes, workspace (gdn_chunk_fwd_varlen_workspace_bytes), stream: as
 *                  gdn_chunk_fwd; the kernel family is chosen as gdn_chunk_fwd_kernel_name(N,
 *                  max_seqlen, ...) names it
 * N == 0 is a no-op; total_T == 0 or max_seqlen == 0 writes final_state only.  Errors as
 * gdn_chunk_fwd (cu_seqlens NULL: GDN_ERR_NULL; not 4-byte aligned: GDN_ERR_ALIGN; outputs
 * overlapping it: GDN_ERR_ALIAS).
 */
gdn_status_t gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                  const float* initial_state, float* final_state, void* o, const int* cu_seqlens,
                                  int N, int max_seqlen, int total_T, int Hqk, int Hv, int dk, int dv, int chunk,
                                  gdn_dtype_t dtype, float scale, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Affine chunk scan.  Over a chunk the state map of the gated delta rule is affine in the entry
 * state: in the WY form of the chunk ("Gated Attention Architectures", sections 2 and 3: the
 * DeltaNet WY representation, with the per-chunk decay products of Gated DeltaNet),
 *     h_out = M h_in + N,   M = e^{gL} I - K~^T W  [dk, dk],   N = K~^T U  [dk, dv],
 * with h = S^T the stored state, and such maps compose: (M2, N2) o (M1, N1) = (M2 M1, M2 N1 + N2).
 * So a long chain can be cut into segments whose maps are formed independently (in parallel on
 * one GPU, or one segment per GPU for context parallelism), composed into the segments' entry
 * states, and the segments then run from those states.  Both entry points below use the
 * matrix-core kernels: bf16 inputs, chunk 64, dk and dv 64 or 128 (else GDN_ERR_UNSUPPORTED).
 */

/*
 * gdn_chunk_fwd_scan_workspace_bytes -- device scratch (bytes) gdn_chunk_fwd_scan needs for
 * `segments` requested segments: the per-chunk operands of the matrix-core path (as
 * gdn_chunk_fwd's split path), then float32 M and N of every segment but the last and the entry
 * state of every segment, each region 256-byte aligned.  Pure host function; 0 for invalid or
 * unsupported sizes, for B == 0 and for T == 0.
 */
size_t gdn_chunk_fwd_scan_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                          gdn_dtype_t dtype, int segments);

/*
 * gdn_chunk_fwd_scan_segments -- the number of segments gdn_chunk_fwd_scan uses when asked for
 * `segments`: with NT = ceil(T / 64) chunks, segments of L = ceil(NT / segments) chunks, so
 * ceil(NT / L) of them, each at least one chunk (1 for T == 0).  Pure host function; 0 for invalid
 * or unsupported sizes.
 */
int gdn_chunk_fwd_scan_segments(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype,
                                int segments);

/*
 * gdn_chunk_fwd_scan -- prefill with each (batch, value head) chain cut into segments: the same
 * result as gdn_chunk_fwd up to float rounding (o, final_state and every argument as there), for
 * workloads with too few chains to fill the GPU.  Four launches on `stream`:
 *   1. the per-chunk operands of every chunk (all chunks in parallel);
 *   2. the map (M, N) of every segment but the last, by running its chunks from h = [0 | I] over
 *      the dv value columns and dk more columns whose V is zero (the value columns end as N, the
 *      others as M);
 *   3. the entry states, h_0 = initial_state (zeros when NULL), h_{s+1} = M_s h_s + N_s, float32;
 *   4. every segment from its entry state, writing its O; the last writes final_state.
 *   segments       requested count >= 1 (1: no scan, gdn_chunk_fwd's split path); see
 *                  gdn_chunk_fwd_scan_segments for the count used
 *   workspace      at least gdn_chunk_fwd_scan_workspace_bytes(...) bytes, 16-byte aligned,
 *                  caller-owned, not overlapping any other argument
 * B == 0 is a no-op; T == 0 writes final_state only.  Errors as gdn_chunk_fwd; segments < 1:
 * GDN_ERR_SHAPE.  final_state may be initial_state exactly.
 */
gdn_status_t gdn_chunk_fwd_scan(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                const float* initial_state, float* final_state, void* o, int B, int T, int Hqk,
                                int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype, float scale, int segments,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_transport_workspace_bytes -- device scratch (bytes) gdn_chunk_transport needs: the
 * per-chunk operands of the matrix-core path.  Pure host function; 0 for invalid or unsupported
 * sizes, for B == 0 and for T == 0.
 */
size_t gdn_chunk_transport_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                           gdn_dtype_t dtype);

/*
 * gdn_chunk_transport -- the affine state map of the given T tokens for every (batch, value
 * head) chain: after these tokens the state is M h_in + N for any entry state h_in.  This is the
 * summary one rank computes for its slice of a sequence when a sequence is split across GPUs;
 * the ranks' maps are then composed in order (an exclusive scan) into each rank's entry state.
 *   q              may be NULL (the map does not depend on q); otherwise as gdn_chunk_fwd
 *   k, v, g, beta  as gdn_chunk_fwd
 *   m_out          [B, Hv, dk, dk] float32, device, caller-owned
 *   n_out          [B, Hv, dk, dv] float32, device, caller-owned
 *   workspace      at least gdn_chunk_transport_workspace_bytes(...) bytes, 16-byte aligned
 * M and N are in the stored orientation (h = S^T, [dk, dv]).  B == 0 is a no-op; T == 0 writes
 * M = I and N = 0.  Errors as gdn_chunk_fwd; m_out or n_out overlapping each other, an input or
 * the workspace: GDN_ERR_ALIAS.
 */
gdn_status_t gdn_chunk_transport(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 float* m_out, float* n_out, int B, int T, int Hqk, int Hv, int dk, int dv,
                                 int chunk, gdn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
