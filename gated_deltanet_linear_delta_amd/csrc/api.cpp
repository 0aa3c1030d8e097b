// C ABI of libgdn.so: argument validation and dispatch to the gfx950 kernels.
// Every check runs before any work is enqueued; see include/gdn.h for the contract.
#include "gdn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace {

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }
bool dtype_ok(gdn_dtype_t t) { return t == GDN_F32 || t == GDN_BF16; }
size_t dtype_bytes(gdn_dtype_t t) { return t == GDN_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

gdn_status_t device_ok()
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return GDN_ERR_NO_DEVICE;
    return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status_t s)
{
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "invalid sizes (negative or zero size, or Hv not a multiple of Hqk)";
    case GDN_ERR_UNSUPPORTED: return "unsupported head dim, chunk size or dtype";
    case GDN_ERR_ALIGN: return "a pointer is misaligned (tensors need 16 bytes, g and beta 4)";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    case GDN_ERR_ALIAS: return "an output overlaps an input it may not overlap";
    case GDN_ERR_NO_DEVICE: return "no HIP device visible";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

static gdn_status_t check_chunk_sizes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                      gdn_dtype_t dtype)
{
    if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return GDN_ERR_SHAPE;
    if (Hv % Hqk != 0) return GDN_ERR_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || !chunk_ok(chunk) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

static gdn::ChunkArgs make_chunk_args(const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, const float* s0, float* sf, void* o, int B,
                                      int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                      gdn_dtype_t dtype, float scale)
{
    gdn::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.s0 = s0; a.sf = sf; a.o = o;
    a.B = B; a.T = T; a.Hqk = Hqk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.chunk = chunk;
    a.dtype_bf16 = dtype == GDN_BF16;
    a.scale = scale;
    return a;
}

size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                     gdn_dtype_t dtype)
{
    if (check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype) != GDN_OK) return 0;
    gdn::ChunkArgs a = make_chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, B, T, Hqk, Hv, dk, dv, chunk, dtype, 1.f);
    const int seg = gdn::chunk_auto_segments(a);
    if (seg > 1) return gdn::chunk_scan_workspace_bytes(a, seg);
    return gdn::chunk_mfma_workspace_bytes(a);
}

const char* gdn_chunk_fwd_kernel_name(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                      gdn_dtype_t dtype)
{
    if (check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype) != GDN_OK) return nullptr;
    gdn::ChunkArgs a = make_chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, B, T, Hqk, Hv, dk, dv, chunk, dtype, 1.f);
    if (!gdn::chunk_mfma_supported(a)) return "mfma_f32";
    if (gdn::chunk_auto_segments(a) > 1) return "mfma_scan";
    return gdn::chunk_mfma_split(a) ? "mfma_split" : gdn::chunk_mfma_pipe(a) ? "mfma_pipe" : "mfma";
}

gdn_status_t gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* initial_state, float* final_state,
                           void* o, int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                           gdn_dtype_t dtype, float scale, void* workspace, size_t workspace_bytes,
                           void* stream)
{
    gdn_status_t s = check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (s != GDN_OK) return s;
    const size_t need = gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (B == 0) return GDN_OK;
    const bool work = T > 0;
    if (work && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (need && !workspace) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, initial_state, final_state, o, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    if (!aligned4(g) || !aligned4(beta)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const size_t ntok = (size_t)B * T;
    const size_t sbytes = (size_t)B * Hv * dk * dv * sizeof(float);
    const Range rq = range(q, ntok * Hqk * dk * es), rk = range(k, ntok * Hqk * dk * es);
    const Range rv = range(v, ntok * Hv * dv * es), rg = range(g, ntok * Hv * sizeof(float));
    const Range rb = range(beta, ntok * Hv * sizeof(float));
    const Range rs0 = range(initial_state, initial_state ? sbytes : 0);
    const Range rsf = range(final_state, final_state ? sbytes : 0);
    const Range ro = range(o, work ? ntok * Hv * dv * es : 0);
    const Range inputs[] = {rq, rk, rv, rg, rb, rs0};
    for (const Range& r : inputs)
        if (overlap(ro, r) || overlap(rsf, r)) {
            // the final state may be the initial state exactly (in-place update)
            if (&r == &inputs[5] && final_state == initial_state && !overlap(ro, r)) continue;
            return GDN_ERR_ALIAS;
        }
    if (overlap(ro, rsf)) return GDN_ERR_ALIAS;
    const Range rw = range(workspace, need);
    const Range all[] = {rq, rk, rv, rg, rb, rs0, rsf, ro};
    for (const Range& r : all)
        if (overlap(rw, r)) return GDN_ERR_ALIAS;
    s = device_ok();
    if (s != GDN_OK) return s;

    hipStream_t st = (hipStream_t)stream;
    if (!work) {
        if (!final_state) return GDN_OK;
        return gdn::launch_state_copy(initial_state, final_state, sbytes / sizeof(float), st) == hipSuccess
                   ? GDN_OK : GDN_ERR_LAUNCH;
    }
    gdn::ChunkArgs a = make_chunk_args(q, k, v, g, beta, initial_state, final_state, o, B, T, Hqk,
                                       Hv, dk, dv, chunk, dtype, scale);
    const int seg = gdn::chunk_auto_segments(a);
    hipError_t e = seg > 1 ? gdn::launch_chunk_scan(a, seg, workspace, st)
                 : gdn::chunk_mfma_supported(a) ? gdn::launch_chunk_mfma(a, workspace, st)
                                                : gdn::launch_chunk_simt(a, st);
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t gdn_chunk_fwd_gated_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                           gdn_dtype_t dtype)
{
    if (check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype) != GDN_OK) return 0;
    gdn::ChunkArgs a = make_chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, B, T, Hqk, Hv, dk, dv, chunk, dtype, 1.f);
    const size_t base = gdn::chunk_mfma_workspace_bytes(a);
    if (gdn::chunk_mfma_gated_fused(a)) return base;
    // otherwise O goes through the workspace, after the recurrence's own part
    const size_t obytes = (size_t)B * T * Hv * dv * dtype_bytes(dtype);
    return obytes ? align256(base) + obytes : base;
}

gdn_status_t gdn_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* initial_state, float* final_state,
                                 const void* z, const float* norm_weight, int weight_per_head, float eps,
                                 void* y, int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                 gdn_dtype_t dtype, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream)
{
    gdn_status_t s = check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (s != GDN_OK) return s;
    if (weight_per_head != 0 && weight_per_head != 1) return GDN_ERR_SHAPE;
    if (!(eps >= 0.f)) return GDN_ERR_UNSUPPORTED;
    const size_t need = gdn_chunk_fwd_gated_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (B == 0) return GDN_OK;
    const bool work = T > 0;
    if (work && (!q || !k || !v || !g || !beta || !z || !norm_weight || !y)) return GDN_ERR_NULL;
    if (need && !workspace) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, initial_state, final_state, z, y, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    if (!aligned4(g) || !aligned4(beta) || !aligned4(norm_weight)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const size_t ntok = work ? (size_t)B * T : 0;
    const size_t sbytes = (size_t)B * Hv * dk * dv * sizeof(float);
    const Range rq = range(q, ntok * Hqk * dk * es), rk = range(k, ntok * Hqk * dk * es);
    const Range rv = range(v, ntok * Hv * dv * es), rg = range(g, ntok * Hv * sizeof(float));
    const Range rb = range(beta, ntok * Hv * sizeof(float));
    const Range rz = range(z, ntok * Hv * dv * es);
    const Range rw = range(norm_weight, work ? (weight_per_head ? (size_t)Hv : 1) * dv * sizeof(float) : 0);
    const Range rs0 = range(initial_state, initial_state ? sbytes : 0);
    const Range rsf = range(final_state, final_state ? sbytes : 0);
    const Range ry = range(y, ntok * Hv * dv * es);
    // y may be z exactly (each element of z is read before the same lane writes it); the final
    // state may be the initial state exactly
    const Range fixed[] = {rq, rk, rv, rg, rb, rw};
    for (const Range& r : fixed)
        if (overlap(ry, r) || overlap(rsf, r)) return GDN_ERR_ALIAS;
    if ((overlap(ry, rz) && y != z) || overlap(ry, rs0) || overlap(ry, rsf)) return GDN_ERR_ALIAS;
    if (overlap(rsf, rz) || (overlap(rsf, rs0) && final_state != initial_state)) return GDN_ERR_ALIAS;
    const Range rws = range(workspace, need);
    const Range all[] = {rq, rk, rv, rg, rb, rz, rw, rs0, rsf, ry};
    for (const Range& r : all)
        if (overlap(rws, r)) return GDN_ERR_ALIAS;
    s = device_ok();
    if (s != GDN_OK) return s;

    hipStream_t st = (hipStream_t)stream;
    if (!work) {
        if (!final_state) return GDN_OK;
        return gdn::launch_state_copy(initial_state, final_state, sbytes / sizeof(float), st) == hipSuccess
                   ? GDN_OK : GDN_ERR_LAUNCH;
    }
    gdn::ChunkArgs a = make_chunk_args(q, k, v, g, beta, initial_state, final_state, nullptr, B, T, Hqk,
                                       Hv, dk, dv, chunk, dtype, scale);
    const int wstride = weight_per_head ? dv : 0;
    hipError_t e;
    if (gdn::chunk_mfma_gated_fused(a)) {
        a.z = z; a.norm_w = norm_weight; a.norm_w_stride = wstride; a.eps = eps; a.y = y;
        e = gdn::launch_chunk_mfma(a, workspace, st);
    } else {
        void* o = (unsigned char*)workspace + align256(gdn::chunk_mfma_workspace_bytes(a));
        a.o = o;
        e = gdn::chunk_mfma_supported(a) ? gdn::launch_chunk_mfma(a, workspace, st) : gdn::launch_chunk_simt(a, st);
        if (e == hipSuccess) {
            gdn::RmsNormArgs r;
            r.o = o; r.z = z; r.w = norm_weight; r.w_head_stride = wstride; r.y = y;
            r.B = B; r.T = T; r.Hv = Hv; r.dv = dv; r.dtype_bf16 = dtype == GDN_BF16; r.eps = eps;
            e = gdn::launch_gated_rmsnorm(r, st);
        }
    }
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, gdn_dtype_t dtype)
{
    if (check_chunk_sizes(B, T, Hqk, Hv, dk, dv, 32, dtype) != GDN_OK) return 0;
    return gdn::chunk_bwd_workspace_bytes(B, T, Hv, dk, dv);
}

gdn_status_t gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           const float* initial_state, const void* grad_o, const float* grad_final_state,
                           void* grad_q, void* grad_k, void* grad_v, float* grad_g, float* grad_beta,
                           float* grad_initial_state, int B, int T, int Hqk, int Hv, int dk, int dv,
                           gdn_dtype_t dtype, float scale, void* workspace, size_t workspace_bytes, void* stream)
{
    gdn_status_t s = check_chunk_sizes(B, T, Hqk, Hv, dk, dv, 32, dtype);
    if (s != GDN_OK) return s;
    const size_t need = gdn_chunk_bwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, dtype);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (B == 0) return GDN_OK;
    const bool work = T > 0;
    if (work && (!q || !k || !v || !g || !beta || !grad_o || !grad_q || !grad_k || !grad_v || !grad_g || !grad_beta))
        return GDN_ERR_NULL;
    if (need && !workspace) return GDN_ERR_NULL;
    const void* p16[] = {q, k, v, initial_state, grad_o, grad_final_state, grad_q, grad_k, grad_v,
                         grad_initial_state, workspace};
    for (const void* p : p16)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const void* p4[] = {g, beta, grad_g, grad_beta};
    for (const void* p : p4)
        if (p && !aligned4(p)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const size_t ntok = work ? (size_t)B * T : 0;
    const size_t sbytes = (size_t)B * Hv * dk * dv * sizeof(float);
    const Range ins[] = {range(q, ntok * Hqk * dk * es), range(k, ntok * Hqk * dk * es),
                         range(v, ntok * Hv * dv * es), range(g, ntok * Hv * 4), range(beta, ntok * Hv * 4),
                         range(initial_state, initial_state ? sbytes : 0), range(grad_o, ntok * Hv * dv * es),
                         range(grad_final_state, grad_final_state ? sbytes : 0)};
    const Range outs[] = {range(grad_q, ntok * Hqk * dk * es), range(grad_k, ntok * Hqk * dk * es),
                          range(grad_v, ntok * Hv * dv * es), range(grad_g, ntok * Hv * 4),
                          range(grad_beta, ntok * Hv * 4),
                          range(grad_initial_state, grad_initial_state ? sbytes : 0), range(workspace, need)};
    for (const Range& o : outs) {
        for (const Range& r : ins)
            if (overlap(o, r)) return GDN_ERR_ALIAS;
        for (const Range& o2 : outs)
            if (&o2 != &o && overlap(o, o2)) return GDN_ERR_ALIAS;
    }
    s = device_ok();
    if (s != GDN_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    if (!work) {
        if (!grad_initial_state) return GDN_OK;
        return gdn::launch_state_copy(grad_final_state, grad_initial_state, sbytes / sizeof(float), st) == hipSuccess
                   ? GDN_OK : GDN_ERR_LAUNCH;
    }
    gdn::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.s0 = initial_state; a.dout = grad_o;
    a.dsf = grad_final_state; a.dq = grad_q; a.dk = grad_k; a.dv = grad_v; a.dg = grad_g; a.dbeta = grad_beta;
    a.ds0 = grad_initial_state; a.ws = (float*)workspace;
    a.B = B; a.T = T; a.Hqk = Hqk; a.Hv = Hv; a.dk_ = dk; a.dv_ = dv;
    a.dtype_bf16 = dtype == GDN_BF16;
    a.scale = scale;
    return gdn::launch_chunk_bwd(a, st) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

static gdn_status_t check_kda_sizes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype)
{
    if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return GDN_ERR_SHAPE;
    if (Hv % Hqk != 0) return GDN_ERR_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERR_UNSUPPORTED;
    // chunk 64: the matrix-core kernels (bf16, head dims 64 or 128)
    if (chunk == 64 && (dtype != GDN_BF16 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128)))
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

size_t gdn_kda_chunk_fwd_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype)
{
    if (check_kda_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype) != GDN_OK || chunk != 64) return 0;
    return gdn::kda_mfma_workspace_bytes(B, T, Hv, dk);
}

gdn_status_t gdn_kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const float* initial_state, float* final_state, void* o, int B, int T, int Hqk,
                               int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype, float scale, void* workspace,
                               size_t workspace_bytes, void* stream)
{
    gdn_status_t s0s = check_kda_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (s0s != GDN_OK) return s0s;
    const size_t need = gdn_kda_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (B == 0) return GDN_OK;
    const bool work = T > 0;
    if (work && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (need && !workspace) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, initial_state, final_state, o, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    if (!aligned4(g) || !aligned4(beta)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const size_t ntok = work ? (size_t)B * T : 0;
    const size_t sbytes = (size_t)B * Hv * dk * dv * sizeof(float);
    const Range rq = range(q, ntok * Hqk * dk * es), rk = range(k, ntok * Hqk * dk * es);
    const Range rv = range(v, ntok * Hv * dv * es), rg = range(g, ntok * Hv * dk * sizeof(float));
    const Range rb = range(beta, ntok * Hv * sizeof(float));
    const Range rs0 = range(initial_state, initial_state ? sbytes : 0);
    const Range rsf = range(final_state, final_state ? sbytes : 0);
    const Range ro = range(o, ntok * Hv * dv * es);
    const Range inputs[] = {rq, rk, rv, rg, rb, rs0};
    for (const Range& r : inputs)
        if (overlap(ro, r) || overlap(rsf, r)) {
            if (&r == &inputs[5] && final_state == initial_state && !overlap(ro, r)) continue;
            return GDN_ERR_ALIAS;
        }
    if (overlap(ro, rsf)) return GDN_ERR_ALIAS;
    const Range rw = range(workspace, need);
    const Range allk[] = {rq, rk, rv, rg, rb, rs0, rsf, ro};
    for (const Range& r : allk)
        if (overlap(rw, r)) return GDN_ERR_ALIAS;
    gdn_status_t s = device_ok();
    if (s != GDN_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    if (!work) {
        if (!final_state) return GDN_OK;
        return gdn::launch_state_copy(initial_state, final_state, sbytes / sizeof(float), st) == hipSuccess
                   ? GDN_OK : GDN_ERR_LAUNCH;
    }
    gdn::KdaArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.s0 = initial_state; a.sf = final_state; a.o = o;
    a.B = B; a.T = T; a.Hqk = Hqk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.chunk = chunk;
    a.dtype_bf16 = dtype == GDN_BF16;
    a.scale = scale;
    const hipError_t e = chunk == 64 ? gdn::launch_kda_mfma(a, workspace, st) : gdn::launch_kda_chunk(a, st);
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

size_t gdn_chunk_fwd_varlen_workspace_bytes(int N, int max_seqlen, int Hqk, int Hv, int dk, int dv, int chunk,
                                            gdn_dtype_t dtype)
{
    return gdn_chunk_fwd_workspace_bytes(N, max_seqlen, Hqk, Hv, dk, dv, chunk, dtype);
}

gdn_status_t gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                  const float* initial_state, float* final_state, void* o, const int* cu_seqlens,
                                  int N, int max_seqlen, int total_T, int Hqk, int Hv, int dk, int dv, int chunk,
                                  gdn_dtype_t dtype, float scale, void* workspace, size_t workspace_bytes,
                                  void* stream)
{
    if (total_T < 0) return GDN_ERR_SHAPE;
    gdn_status_t s = check_chunk_sizes(N, max_seqlen, Hqk, Hv, dk, dv, chunk, dtype);
    if (s != GDN_OK) return s;
    const size_t need = gdn_chunk_fwd_varlen_workspace_bytes(N, max_seqlen, Hqk, Hv, dk, dv, chunk, dtype);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (N == 0) return GDN_OK;
    const bool work = total_T > 0 && max_seqlen > 0;
    if (!cu_seqlens) return GDN_ERR_NULL;
    if (work && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (need && !workspace) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, initial_state, final_state, o, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    if (!aligned4(g) || !aligned4(beta) || !aligned4(cu_seqlens)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const size_t ntok = work ? (size_t)total_T : 0;
    const size_t sbytes = (size_t)N * Hv * dk * dv * sizeof(float);
    const Range rq = range(q, ntok * Hqk * dk * es), rk = range(k, ntok * Hqk * dk * es);
    const Range rv = range(v, ntok * Hv * dv * es), rg = range(g, ntok * Hv * sizeof(float));
    const Range rb = range(beta, ntok * Hv * sizeof(float));
    const Range rcu = range(cu_seqlens, (size_t)(N + 1) * sizeof(int));
    const Range rs0 = range(initial_state, initial_state ? sbytes : 0);
    const Range rsf = range(final_state, final_state ? sbytes : 0);
    const Range ro = range(o, ntok * Hv * dv * es);
    const Range inputs[] = {rq, rk, rv, rg, rb, rcu, rs0};
    for (const Range& r : inputs)
        if (overlap(ro, r) || overlap(rsf, r)) {
            if (&r == &inputs[6] && final_state == initial_state && !overlap(ro, r)) continue;
            return GDN_ERR_ALIAS;
        }
    if (overlap(ro, rsf)) return GDN_ERR_ALIAS;
    const Range rw = range(workspace, need);
    const Range all[] = {rq, rk, rv, rg, rb, rcu, rs0, rsf, ro};
    for (const Range& r : all)
        if (overlap(rw, r)) return GDN_ERR_ALIAS;
    s = device_ok();
    if (s != GDN_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    if (!work) {
        // every sequence is empty: final states are the initial ones
        if (!final_state) return GDN_OK;
        return gdn::launch_state_copy(initial_state, final_state, sbytes / sizeof(float), st) == hipSuccess
                   ? GDN_OK : GDN_ERR_LAUNCH;
    }
    gdn::ChunkArgs a = make_chunk_args(q, k, v, g, beta, initial_state, final_state, o, N, max_seqlen, Hqk, Hv,
                                       dk, dv, chunk, dtype, scale);
    a.cu = cu_seqlens;
    a.total = total_T;
    hipError_t e = gdn::chunk_mfma_supported(a) ? gdn::launch_chunk_mfma(a, workspace, st)
                                                : gdn::launch_chunk_simt(a, st);
    return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// ------------------------------------------------------------------ affine chunk scan
static bool scan_supported(const gdn::ChunkArgs& a)
{
    return gdn::chunk_mfma_supported(a);
}

size_t gdn_chunk_fwd_scan_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                          gdn_dtype_t dtype, int segments)
{
    if (check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype) != GDN_OK || segments < 1) return 0;
    gdn::ChunkArgs a = make_chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, B, T, Hqk, Hv, dk, dv, chunk, dtype, 1.f);
    if (!scan_supported(a) || B == 0 || T == 0) return 0;
    return gdn::chunk_scan_workspace_bytes(a, segments);
}

int gdn_chunk_fwd_scan_segments(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype,
                                int segments)
{
    if (check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype) != GDN_OK || segments < 1) return 0;
    gdn::ChunkArgs a = make_chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, B, T, Hqk, Hv, dk, dv, chunk, dtype, 1.f);
    if (!scan_supported(a)) return 0;
    if (T == 0) return 1;
    return gdn::chunk_scan_segments(a, segments);
}

gdn_status_t gdn_chunk_fwd_scan(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                const float* initial_state, float* final_state, void* o, int B, int T, int Hqk,
                                int Hv, int dk, int dv, int chunk, gdn_dtype_t dtype, float scale, int segments,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    gdn_status_t s = check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (s != GDN_OK) return s;
    if (segments < 1) return GDN_ERR_SHAPE;
    gdn::ChunkArgs a = make_chunk_args(q, k, v, g, beta, initial_state, final_state, o, B, T, Hqk, Hv, dk, dv,
                                       chunk, dtype, scale);
    if (!scan_supported(a)) return GDN_ERR_UNSUPPORTED;
    const size_t need = gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype, segments);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (B == 0) return GDN_OK;
    const bool work = T > 0;
    if (work && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (need && !workspace) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, initial_state, final_state, o, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    if (!aligned4(g) || !aligned4(beta)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const size_t ntok = (size_t)B * T;
    const size_t sbytes = (size_t)B * Hv * dk * dv * sizeof(float);
    const Range rq = range(q, ntok * Hqk * dk * es), rk = range(k, ntok * Hqk * dk * es);
    const Range rv = range(v, ntok * Hv * dv * es), rg = range(g, ntok * Hv * sizeof(float));
    const Range rb = range(beta, ntok * Hv * sizeof(float));
    const Range rs0 = range(initial_state, initial_state ? sbytes : 0);
    const Range rsf = range(final_state, final_state ? sbytes : 0);
    const Range ro = range(o, work ? ntok * Hv * dv * es : 0);
    const Range inputs[] = {rq, rk, rv, rg, rb, rs0};
    for (const Range& r : inputs)
        if (overlap(ro, r) || overlap(rsf, r)) {
            // in place: the segments read the initial state (combine kernel, first segment)
            // before the last segment writes the final state, on one stream
            if (&r == &inputs[5] && final_state == initial_state && !overlap(ro, r)) continue;
            return GDN_ERR_ALIAS;
        }
    if (overlap(ro, rsf)) return GDN_ERR_ALIAS;
    const Range rw = range(workspace, need);
    const Range all[] = {rq, rk, rv, rg, rb, rs0, rsf, ro};
    for (const Range& r : all)
        if (overlap(rw, r)) return GDN_ERR_ALIAS;
    s = device_ok();
    if (s != GDN_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    if (!work) {
        if (!final_state) return GDN_OK;
        return gdn::launch_state_copy(initial_state, final_state, sbytes / sizeof(float), st) == hipSuccess
                   ? GDN_OK : GDN_ERR_LAUNCH;
    }
    return gdn::launch_chunk_scan(a, segments, workspace, st) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

size_t gdn_chunk_transport_workspace_bytes(int B, int T, int Hqk, int Hv, int dk, int dv, int chunk,
                                           gdn_dtype_t dtype)
{
    if (check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype) != GDN_OK) return 0;
    gdn::ChunkArgs a = make_chunk_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, B, T, Hqk, Hv, dk, dv, chunk, dtype, 1.f);
    if (!scan_supported(a) || B == 0 || T == 0) return 0;
    return gdn::chunk_transport_workspace_bytes(a);
}

gdn_status_t gdn_chunk_transport(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 float* m_out, float* n_out, int B, int T, int Hqk, int Hv, int dk, int dv,
                                 int chunk, gdn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 void* stream)
{
    gdn_status_t s = check_chunk_sizes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (s != GDN_OK) return s;
    gdn::ChunkArgs a = make_chunk_args(q ? q : k, k, v, g, beta, nullptr, nullptr, nullptr, B, T, Hqk, Hv, dk,
                                       dv, chunk, dtype, 1.f);
    if (!scan_supported(a)) return GDN_ERR_UNSUPPORTED;
    const size_t need = gdn_chunk_transport_workspace_bytes(B, T, Hqk, Hv, dk, dv, chunk, dtype);
    if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (B == 0) return GDN_OK;
    const bool work = T > 0;
    if (!m_out || !n_out) return GDN_ERR_NULL;
    if (work && (!k || !v || !g || !beta)) return GDN_ERR_NULL;
    if (need && !workspace) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, m_out, n_out, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    if (!aligned4(g) || !aligned4(beta)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const size_t ntok = work ? (size_t)B * T : 0;
    const Range rq = range(q, ntok * Hqk * dk * es), rk = range(k, ntok * Hqk * dk * es);
    const Range rv = range(v, ntok * Hv * dv * es), rg = range(g, ntok * Hv * sizeof(float));
    const Range rb = range(beta, ntok * Hv * sizeof(float));
    const Range rm = range(m_out, (size_t)B * Hv * dk * dk * sizeof(float));
    const Range rn = range(n_out, (size_t)B * Hv * dk * dv * sizeof(float));
    const Range rw = range(workspace, need);
    const Range others[] = {rq, rk, rv, rg, rb, rw};
    for (const Range& r : others)
        if (overlap(rm, r) || overlap(rn, r)) return GDN_ERR_ALIAS;
    if (overlap(rm, rn)) return GDN_ERR_ALIAS;
    const Range ins[] = {rq, rk, rv, rg, rb};
    for (const Range& r : ins)
        if (overlap(rw, r)) return GDN_ERR_ALIAS;
    s = device_ok();
    if (s != GDN_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    if (!work)
        return gdn::launch_identity_map(m_out, n_out, (size_t)B * Hv, dk, dv, st) == hipSuccess ? GDN_OK
                                                                                              : GDN_ERR_LAUNCH;
    return gdn::launch_chunk_transport(a, m_out, n_out, workspace, st) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status_t gdn_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, float* state, void* o, int B, int Hqk, int Hv,
                                int dk, int dv, gdn_dtype_t dtype, float scale, void* stream)
{
    if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
    if (Hv % Hqk != 0) return GDN_ERR_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || !dtype_ok(dtype)) return GDN_ERR_UNSUPPORTED;
    if (B == 0) return GDN_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, state, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGN;
    if (!aligned4(g) || !aligned4(beta)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const Range rq = range(q, (size_t)B * Hqk * dk * es), rk = range(k, (size_t)B * Hqk * dk * es);
    const Range rv = range(v, (size_t)B * Hv * dv * es), rg = range(g, (size_t)B * Hv * sizeof(float));
    const Range rb = range(beta, (size_t)B * Hv * sizeof(float));
    const Range rs = range(state, (size_t)B * Hv * dk * dv * sizeof(float));
    const Range ro = range(o, (size_t)B * Hv * dv * es);
    const Range inputs[] = {rq, rk, rv, rg, rb};
    for (const Range& r : inputs)
        if (overlap(ro, r) || overlap(rs, r)) return GDN_ERR_ALIAS;
    if (overlap(ro, rs)) return GDN_ERR_ALIAS;
    gdn_status_t s = device_ok();
    if (s != GDN_OK) return s;
    gdn::StepArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
    a.B = B; a.Hqk = Hqk; a.Hv = Hv; a.dk = dk; a.dv = dv;
    a.dtype_bf16 = dtype == GDN_BF16;
    a.scale = scale;
    return gdn::launch_recurrent_step(a, (hipStream_t)stream) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status_t gdn_qkv_prologue(const void* q_in, const void* k_in, const void* v_in, const float* conv_q,
                              const float* conv_k, const float* conv_v, const float* conv_state_in,
                              float* conv_state_out, void* q, void* k, void* v, int B, int T, int Hqk, int Hv,
                              int dk, int dv, int width, gdn_dtype_t dtype, float eps, void* stream)
{
    if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || width <= 0) return GDN_ERR_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || width > 4 || !dtype_ok(dtype) || !(eps >= 0.f))
        return GDN_ERR_UNSUPPORTED;
    const bool work = T > 0;
    const bool state_out = conv_state_out && width > 1;
    if (B == 0 || (!work && !state_out)) return GDN_OK;
    if (work && (!q_in || !k_in || !v_in || !conv_q || !conv_k || !conv_v || !q || !k || !v)) return GDN_ERR_NULL;
    const void* tens[] = {q_in, k_in, v_in, q, k, v};
    for (const void* p : tens)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const void* f4[] = {conv_q, conv_k, conv_v, conv_state_in, conv_state_out};
    for (const void* p : f4)
        if (p && !aligned4(p)) return GDN_ERR_ALIGN;
    const size_t es = dtype_bytes(dtype);
    const size_t ntok = (size_t)B * T;
    const size_t cq = (size_t)Hqk * dk, cv = (size_t)Hv * dv;
    const size_t sbytes = (size_t)B * (2 * cq + cv) * (width - 1) * sizeof(float);
    const Range ins[] = {range(q_in, work ? ntok * cq * es : 0), range(k_in, work ? ntok * cq * es : 0),
                         range(v_in, work ? ntok * cv * es : 0), range(conv_q, work ? cq * width * 4 : 0),
                         range(conv_k, work ? cq * width * 4 : 0), range(conv_v, work ? cv * width * 4 : 0),
                         range(conv_state_in, conv_state_in ? sbytes : 0)};
    const Range outs[] = {range(q, work ? ntok * cq * es : 0), range(k, work ? ntok * cq * es : 0),
                          range(v, work ? ntok * cv * es : 0), range(conv_state_out, state_out ? sbytes : 0)};
    for (const Range& o : outs) {
        for (const Range& r : ins)
            if (overlap(o, r)) return GDN_ERR_ALIAS;
        for (const Range& o2 : outs)
            if (&o2 != &o && overlap(o, o2)) return GDN_ERR_ALIAS;
    }
    gdn_status_t s = device_ok();
    if (s != GDN_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    if (!work)
        return gdn::launch_state_copy(conv_state_in, conv_state_out, sbytes / sizeof(float), st) == hipSuccess
                   ? GDN_OK : GDN_ERR_LAUNCH;
    gdn::PrologueArgs a;
    a.q_in = q_in; a.k_in = k_in; a.v_in = v_in; a.wq = conv_q; a.wk = conv_k; a.wv = conv_v;
    a.st_in = width > 1 ? conv_state_in : nullptr;
    a.st_out = state_out ? conv_state_out : nullptr;
    a.q = q; a.k = k; a.v = v;
    a.B = B; a.T = T; a.Hqk = Hqk; a.Hv = Hv; a.dk = dk; a.dv = dv; a.W = width;
    a.dtype_bf16 = dtype == GDN_BF16;
    a.eps = eps;
    return gdn::launch_qkv_prologue(a, st) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status_t gdn_gated_rmsnorm(const void* o, const void* z, const float* weight, int weight_per_head, void* y,
                               int B, int T, int Hv, int dv, gdn_dtype_t dtype, float eps, void* stream)
{
    if (B < 0 || T < 0 || Hv <= 0 || dv <= 0 || (weight_per_head != 0 && weight_per_head != 1)) return GDN_ERR_SHAPE;
    if (!head_dim_ok(dv) || !dtype_ok(dtype) || !(eps >= 0.f)) return GDN_ERR_UNSUPPORTED;
    if (B == 0 || T == 0) return GDN_OK;
    if (!o || !z || !weight || !y) return GDN_ERR_NULL;
    if (!aligned16(o) || !aligned16(z) || !aligned16(y) || !aligned4(weight)) return GDN_ERR_ALIGN;
    const size_t bytes = (size_t)B * T * Hv * dv * dtype_bytes(dtype);
    const Range ro = range(o, bytes), rz = range(z, bytes), ry = range(y, bytes);
    const Range rw = range(weight, (weight_per_head ? (size_t)Hv : 1) * dv * sizeof(float));
    // y may be o or z exactly (each element is read before it is written, by the same lane)
    if ((overlap(ry, ro) && y != o) || (overlap(ry, rz) && y != z) || overlap(ry, rw)) return GDN_ERR_ALIAS;
    gdn_status_t s = device_ok();
    if (s != GDN_OK) return s;
    gdn::RmsNormArgs a;
    a.o = o; a.z = z; a.w = weight; a.w_head_stride = weight_per_head ? dv : 0; a.y = y;
    a.B = B; a.T = T; a.Hv = Hv; a.dv = dv;
    a.dtype_bf16 = dtype == GDN_BF16;
    a.eps = eps;
    return gdn::launch_gated_rmsnorm(a, (hipStream_t)stream) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // extern "C"
