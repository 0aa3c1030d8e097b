// Host-side launch interface between the C ABI (api.cpp) and the kernels.  Arguments arrive here
// already validated.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* o;
    int B, Hqk, Hv, dk, dv;
    bool dtype_bf16;
    float scale;
};

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* s0;   // may be null (zero initial state)
    float* sf;         // may be null (final state not wanted); may equal s0
    void* o;
    int B, T, Hqk, Hv, dk, dv, chunk;
    bool dtype_bf16;
    float scale;
    // gated output (fused epilogue of the matrix-core kernel, chunk_mfma_gated_fused): z set
    // means y = RMSNorm(O) * norm_w * silu(z) is written to y and O is not written
    const void* z = nullptr;
    const float* norm_w = nullptr;   // [dv] (stride 0) or [Hv, dv] (stride dv)
    int norm_w_stride = 0;
    float eps = 0.f;
    void* y = nullptr;
    // packed sequences: when cu is set, B is the number of sequences, cu[0..B] (device) their
    // token offsets into `total` tokens (tensors [total, H, d]), and T the longest length
    const int* cu = nullptr;
    int total = 0;
};

hipError_t launch_recurrent_step(const StepArgs& a, hipStream_t st);

// Float32-vector chunkwise kernel: any supported dtype, head dims and chunk size.
hipError_t launch_chunk_simt(const ChunkArgs& a, hipStream_t st);

// Matrix-core chunkwise path: bf16 inputs and the shapes chunk_mfma_supported accepts.  One
// fused kernel (with the state-independent part of each chunk built inside it by prep waves:
// chunk_mfma_pipe for the pipelined one), or (chunk_mfma_split) a parallel per-chunk prep kernel
// that fills a workspace of chunk_mfma_workspace_bytes followed by the state-pass kernel.
bool chunk_mfma_supported(const ChunkArgs& a);
bool chunk_mfma_split(const ChunkArgs& a);
bool chunk_mfma_pipe(const ChunkArgs& a);
// The gated RMSNorm can run inside the fused kernel (whole value heads per workgroup).
bool chunk_mfma_gated_fused(const ChunkArgs& a);
size_t chunk_mfma_workspace_bytes(const ChunkArgs& a);
hipError_t launch_chunk_mfma(const ChunkArgs& a, void* workspace, hipStream_t st);

// Affine chunk scan on the matrix-core split path (shapes chunk_mfma_supported accepts, uniform
// batches): each chain cut into segments whose affine state maps are formed in parallel,
// composed, and then the segments run from their entry states.  chunk_scan_segments gives the
// number of segments actually used for a requested count (every segment holds at least one
// chunk).
size_t chunk_scan_workspace_bytes(const ChunkArgs& a, int segments);
// Segments gdn_chunk_fwd uses on its own (1: no scan), from the number of chains and chunks.
int chunk_auto_segments(const ChunkArgs& a);
int chunk_scan_segments(const ChunkArgs& a, int segments);
hipError_t launch_chunk_scan(const ChunkArgs& a, int segments, void* workspace, hipStream_t st);
// The affine map of the whole given sequence per chain: h_out = M h_in + N, M [B, Hv, dk, dk] and
// N [B, Hv, dk, dv] float32.
size_t chunk_transport_workspace_bytes(const ChunkArgs& a);
hipError_t launch_chunk_transport(const ChunkArgs& a, float* m_out, float* n_out, void* workspace,
                                  hipStream_t st);
// M = I, N = 0 for `chains` chains (the map of an empty sequence).
hipError_t launch_identity_map(float* m, float* n, size_t chains, int dk, int dv, hipStream_t st);

// final_state <- initial_state (or zeros when it is null), for T == 0.
hipError_t launch_state_copy(const float* s0, float* sf, size_t n, hipStream_t st);

// Backward pass (chunk_bwd.hip): gradients through O and the final state.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* s0;     // may be null (zero initial state)
    const void* dout;    // dL/dO, dtype of q
    const float* dsf;    // dL/d(final state) or null (zero)
    void* dq;
    void* dk;
    void* dv;
    float* dg;
    float* dbeta;
    float* ds0;          // may be null (not wanted)
    float* ws;           // chunk_bwd_workspace_bytes
    int B, T, Hqk, Hv, dk_, dv_;
    bool dtype_bf16;
    float scale;
};

size_t chunk_bwd_workspace_bytes(int B, int T, int Hv, int dk, int dv);
hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t st);
// The backward's two sequential passes on the float16 matrix cores (chunk_mfma.hip): bf16
// inputs, dk 64 or 128, dv 32, 64 or 128.  Fill H (the state entering every 32-token chunk) and
// dH (each chunk's exit-state gradient) as float16, transposed, [B, Hv, NT, dv, dk] (in the first
// half of each float32 region), and ds0, from the gram kernel's per-chunk matrices Aw.
bool bwd_pass16_supported(const BwdArgs& a);
hipError_t launch_bwd_pass16(const BwdArgs& a, float* H, float* dH, const float* Aw, hipStream_t st);

// Kimi Delta Attention prefill (kda.hip): g is [B, T, Hv, dk] (one log decay per key channel).
struct KdaArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* s0;   // may be null
    float* sf;         // may be null; may equal s0
    void* o;
    int B, T, Hqk, Hv, dk, dv, chunk;
    bool dtype_bf16;
    float scale;
};

hipError_t launch_kda_chunk(const KdaArgs& a, hipStream_t st);
// Matrix-core KDA (chunk_mfma.hip): bf16, chunk 64, dk and dv 64 or 128; a per-chunk prep kernel
// fills a workspace of kda_mfma_workspace_bytes, then the state pass.
bool kda_mfma_supported(const KdaArgs& a);
size_t kda_mfma_workspace_bytes(int B, int T, int Hv, int dk);
hipError_t launch_kda_mfma(const KdaArgs& a, void* ws, hipStream_t st);

// Layer steps around the recurrence (layer_ops.hip).
struct PrologueArgs {
    const void* q_in;
    const void* k_in;
    const void* v_in;
    const float* wq;       // [Hqk*dk, W]
    const float* wk;       // [Hqk*dk, W]
    const float* wv;       // [Hv*dv, W]
    const float* st_in;    // [B, 2*Hqk*dk + Hv*dv, W-1] or null (zeros)
    float* st_out;         // same shape or null
    void* q;
    void* k;
    void* v;
    int B, T, Hqk, Hv, dk, dv, W;
    bool dtype_bf16;
    float eps;
};

struct RmsNormArgs {
    const void* o;
    const void* z;
    const float* w;        // [dv] shared by the heads (w_head_stride 0) or [Hv, dv] (stride dv)
    int w_head_stride;
    void* y;
    int B, T, Hv, dv;
    bool dtype_bf16;
    float eps;
};

hipError_t launch_qkv_prologue(const PrologueArgs& a, hipStream_t st);
hipError_t launch_gated_rmsnorm(const RmsNormArgs& a, hipStream_t st);

}  // namespace gdn
