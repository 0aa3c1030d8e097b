// Host-only stand-ins for the kernel launchers and route queries of libgdn.so, so that api.cpp's
// argument validation can be built with AddressSanitizer and UndefinedBehaviorSanitizer by the
// host compiler alone (tests/test_sanitizers.py).  No kernel runs: every launcher succeeds
// without doing anything.  The route queries follow the shape of the real ones (bf16 at chunk 64
// takes the matrix-core route; its split path needs a workspace) so the workspace checks run.
#include "launch.hpp"

namespace gdn {

bool chunk_mfma_supported(const ChunkArgs& a)
{
    return a.dtype_bf16 && a.chunk == 64 && (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128);
}
bool chunk_mfma_split(const ChunkArgs& a) { return chunk_mfma_supported(a) && (long)a.B * a.Hv < 192; }
bool chunk_mfma_pipe(const ChunkArgs& a) { return chunk_mfma_supported(a) && (long)a.B * a.Hv >= 192; }
bool chunk_mfma_gated_fused(const ChunkArgs& a) { return chunk_mfma_supported(a) && !chunk_mfma_split(a); }
size_t chunk_mfma_workspace_bytes(const ChunkArgs& a)
{
    return chunk_mfma_split(a) ? (size_t)a.B * (((size_t)a.T + 63) / 64) * (size_t)a.Hv * 13568 : 0;
}
int chunk_auto_segments(const ChunkArgs&) { return 1; }
int chunk_scan_segments(const ChunkArgs& a, int segments)
{
    const long nt = ((long)a.T + 63) / 64;
    if (nt == 0) return 1;
    const long len = (nt + segments - 1) / segments;
    return (int)((nt + len - 1) / len);
}
size_t chunk_scan_workspace_bytes(const ChunkArgs& a, int segments)
{
    return chunk_mfma_workspace_bytes(a) + (size_t)segments * a.B * a.Hv * a.dk * ((size_t)a.dk + a.dv) * 4;
}
size_t chunk_transport_workspace_bytes(const ChunkArgs& a) { return (size_t)a.B * (((size_t)a.T + 63) / 64) * a.Hv * 13568; }
size_t chunk_bwd_workspace_bytes(int B, int T, int Hv, int dk, int dv)
{
    return (size_t)B * Hv * (((size_t)T + 31) / 32) * (2 * (size_t)dk * dv + 4 * 32 * 32 + 64) * 4;
}
bool kda_mfma_supported(const KdaArgs& a) { return a.dtype_bf16 && a.chunk == 64; }
size_t kda_mfma_workspace_bytes(int B, int T, int Hv, int dk)
{
    return (size_t)B * Hv * (((size_t)T + 63) / 64) * (3 * 64 * (size_t)dk * 2 + 2 * 64 * 64 * 2 + 256 + (size_t)dk * 4);
}

hipError_t launch_recurrent_step(const StepArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_chunk_simt(const ChunkArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_chunk_mfma(const ChunkArgs&, void*, hipStream_t) { return hipSuccess; }
hipError_t launch_chunk_scan(const ChunkArgs&, int, void*, hipStream_t) { return hipSuccess; }
hipError_t launch_chunk_transport(const ChunkArgs&, float*, float*, void*, hipStream_t) { return hipSuccess; }
hipError_t launch_identity_map(float*, float*, size_t, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_state_copy(const float*, float*, size_t, hipStream_t) { return hipSuccess; }
hipError_t launch_chunk_bwd(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_kda_chunk(const KdaArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_kda_mfma(const KdaArgs&, void*, hipStream_t) { return hipSuccess; }
hipError_t launch_qkv_prologue(const PrologueArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_gated_rmsnorm(const RmsNormArgs&, hipStream_t) { return hipSuccess; }

}  // namespace gdn
