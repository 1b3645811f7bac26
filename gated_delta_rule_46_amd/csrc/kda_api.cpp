// C ABI: argument validation (before any HIP call) and dispatch.
#include "../../include/kda.h"

#include <hip/hip_runtime_api.h>

#include "kda_launch.h"

namespace {

thread_local int g_last_hip = 0;

bool size_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }
bool aligned(const void* p, uintptr_t a = 16) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return KDA_OK;
    g_last_hip = (int)e;
    return KDA_EHIP;
}

}  // namespace

namespace kda {

int validate_chunk_fwd(int stage, const void* q, const void* k, const void* v, const void* gate, const void* beta,
                       const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv, int chunk,
                       const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* stream, ChunkArgs* args,
                       size_t* need) {
    if (stage != KDA_STAGE_ALL && stage != KDA_STAGE_PREP && stage != KDA_STAGE_STATE) return KDA_EINVAL;
    if (B <= 0 || H <= 0 || T < 0) return KDA_EINVAL;
    if (!size_ok(dk) || !size_ok(dv) || !chunk_ok(chunk)) return KDA_ENOTSUP;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ENOTSUP;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return KDA_ENOTSUP;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen) {
        if (B != 1 || N <= 0) return KDA_EINVAL;
    } else {
        if (N != 0 && N != B) return KDA_EINVAL;
        N = B;
    }
    const bool need_data = T > 0;
    if (need_data && (!q || !k || !v || !gate || !beta || !o)) return KDA_EINVAL;
    const uintptr_t es = dtype == KDA_BF16 ? 2 : 4;
    if (need_data && (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(gate) || !aligned(beta, es) ||
                      !aligned(o, 4)))
        return KDA_EALIGN;
    if ((S0 && !aligned(S0, 4)) || (S_T && !aligned(S_T, 4))) return KDA_EALIGN;
    if (varlen && !aligned(cu_seqlens, 4)) return KDA_EALIGN;
    *need = chunk_workspace_bytes(B, H, T, dk, dv, chunk, varlen, N, dtype == KDA_BF16);
    *args = ChunkArgs{q, k, v, gate, beta, S0, o, S_T, B, H, T, dk, dv, chunk, cu_seqlens, N, dtype == KDA_BF16,
                      gate_kind == KDA_GATE_SCALAR, nullptr, reinterpret_cast<hipStream_t>(stream), stage};
    return KDA_OK;
}

int hip_to_status(hipError_t e) { return hip_status(e); }

}  // namespace kda

extern "C" {

int kda_version(void) { return 100; }

const char* kda_strerror(int status) {
    switch (status) {
        case KDA_OK: return "success";
        case KDA_EINVAL: return "invalid argument";
        case KDA_ENOTSUP: return "unsupported size, chunk, dtype or gate kind";
        case KDA_EALIGN: return "pointer misaligned for its element type, or a 16-byte-aligned buffer is not";
        case KDA_EHIP: return "HIP runtime error";
        case KDA_EWAIT: return "a bounded wait in the forward's state pass expired; o and S_T were not written";
        case KDA_ESCRATCH: return "the call needs more scratch than the library's fixed array (KDA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int kda_last_hip_error(void) { return g_last_hip; }

int kda_chunk_fwd_status(uint32_t status_word) { return status_word == 0u ? KDA_OK : KDA_EWAIT; }

size_t kda_chunk_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int N, int has_cu,
                                     int dtype) {
    if (B <= 0 || H <= 0 || T < 0 || !size_ok(dk) || !size_ok(dv) || !chunk_ok(chunk)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    if (has_cu && (B != 1 || N <= 0)) return 0;
    return kda::chunk_workspace_bytes(B, H, T, dk, dv, chunk, has_cu != 0, has_cu ? N : B, dtype == KDA_BF16);
}

int kda_chunk_fwd_stage(int stage, const void* q, const void* k, const void* v, const void* gate,
                        const void* beta, const float* S0, float* o, float* S_T, int B, int H, int T, int dk,
                        int dv, int chunk, const int32_t* cu_seqlens, int N, int dtype, int gate_kind,
                        void* workspace, size_t workspace_bytes, void* stream) {
    kda::ChunkArgs a;
    size_t need = 0;
    const int st = kda::validate_chunk_fwd(stage, q, k, v, gate, beta, S0, o, S_T, B, H, T, dk, dv, chunk, cu_seqlens,
                                           N, dtype, gate_kind, stream, &a, &need);
    if (st != KDA_OK) return st;
    if (workspace && !aligned(workspace)) return KDA_EALIGN;
    if (!workspace || workspace_bytes < need) return KDA_EINVAL;
    if (T == 0 && !S_T) return KDA_OK;
    if (stage == KDA_STAGE_PREP && T == 0) return KDA_OK;
    a.workspace = workspace;
    return hip_status(kda::launch_chunk_fwd(a));
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                  const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv, int chunk,
                  const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* workspace,
                  size_t workspace_bytes, void* stream) {
    return kda_chunk_fwd_stage(KDA_STAGE_ALL, q, k, v, gate, beta, S0, o, S_T, B, H, T, dk, dv, chunk, cu_seqlens,
                               N, dtype, gate_kind, workspace, workspace_bytes, stream);
}

int kda_chunk_fwd_ew(const void* q, const void* k, const void* v, const void* gate, const void* erase,
                     const void* write, const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv,
                     int chunk, const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* workspace,
                     size_t workspace_bytes, void* stream) {
    kda::ChunkArgs a;
    size_t need = 0;
    // erase stands in for beta in the shared checks (beta is not an input of this form)
    const int st = kda::validate_chunk_fwd(KDA_STAGE_ALL, q, k, v, gate, erase, S0, o, S_T, B, H, T, dk, dv, chunk,
                                           cu_seqlens, N, dtype, gate_kind, stream, &a, &need);
    if (st != KDA_OK) return st;
    if (T > 0 && (!erase || !write)) return KDA_EINVAL;
    if (T > 0 && (!aligned(erase) || !aligned(write))) return KDA_EALIGN;
    if (workspace && !aligned(workspace)) return KDA_EALIGN;
    if (!workspace || workspace_bytes < need) return KDA_EINVAL;
    if (T == 0 && !S_T) return KDA_OK;
    a.beta = nullptr;
    a.erase = erase;
    a.write = write;
    a.workspace = workspace;
    return hip_status(kda::launch_chunk_fwd(a));
}

int kda_decode_step_ew(const void* q, const void* k, const void* v, const void* gate, const void* erase,
                       const void* write, float* S, float* o, int N, int H, int dk, int dv, int dtype, int gate_kind,
                       void* stream) {
    if (N <= 0 || H <= 0) return KDA_EINVAL;
    if (!size_ok(dk) || !size_ok(dv)) return KDA_ENOTSUP;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ENOTSUP;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return KDA_ENOTSUP;
    if (!q || !k || !v || !gate || !erase || !write || !S || !o) return KDA_EINVAL;
    const uintptr_t es = dtype == KDA_BF16 ? 2 : 4;
    if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(gate, es) || !aligned(erase, es) ||
        !aligned(write, es) || !aligned(S) || !aligned(o))
        return KDA_EALIGN;
    kda::DecodeArgs a{q, k, v, gate, nullptr, S, o, N, H, dk, dv, dtype == KDA_BF16,
                      gate_kind == KDA_GATE_SCALAR, reinterpret_cast<hipStream_t>(stream), erase, write};
    return hip_status(kda::launch_decode(a));
}

size_t kda_chunk_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int N, int has_cu) {
    if (B <= 0 || H <= 0 || T < 0 || !size_ok(dk) || !size_ok(dv)) return 0;
    if (has_cu && (B != 1 || N <= 0)) return 0;
    return kda::bwd_workspace_bytes(B, H, T, dk, dv, has_cu != 0, has_cu ? N : B);
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                  const float* S0, const float* dO, const float* dS_T, float* grad_q, float* grad_k,
                  float* grad_v, float* grad_gate, float* grad_beta, float* grad_S0, int B, int H, int T,
                  int dk, int dv, const int32_t* cu_seqlens, int N, int dtype, int gate_kind,
                  void* workspace, size_t workspace_bytes, void* stream) {
    if (B <= 0 || H <= 0 || T < 0) return KDA_EINVAL;
    if (!size_ok(dk) || !size_ok(dv)) return KDA_ENOTSUP;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ENOTSUP;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return KDA_ENOTSUP;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen) {
        if (B != 1 || N <= 0) return KDA_EINVAL;
    } else {
        if (N != 0 && N != B) return KDA_EINVAL;
        N = B;
    }
    const bool need_data = T > 0;
    if (need_data && (!q || !k || !v || !gate || !beta || !dO || !grad_q || !grad_k || !grad_v || !grad_gate ||
                      !grad_beta))
        return KDA_EINVAL;
    const uintptr_t es = dtype == KDA_BF16 ? 2 : 4;
    if (need_data && (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(gate, es) ||
                      !aligned(beta, es) || !aligned(dO) || !aligned(grad_q, 4) || !aligned(grad_k, 4) ||
                      !aligned(grad_v) || !aligned(grad_gate, 4) || !aligned(grad_beta, 4)))
        return KDA_EALIGN;
    if ((S0 && !aligned(S0)) || (dS_T && !aligned(dS_T)) || (grad_S0 && !aligned(grad_S0)) ||
        (workspace && !aligned(workspace)))
        return KDA_EALIGN;
    if (varlen && !aligned(cu_seqlens, 4)) return KDA_EALIGN;
    const size_t need = kda::bwd_workspace_bytes(B, H, T, dk, dv, varlen, N);
    if (!workspace || workspace_bytes < need) return KDA_EINVAL;
    if (!need_data && !grad_S0) return KDA_OK;

    kda::BwdArgs a{q, k, v, gate, beta, S0, dO, dS_T, grad_q, grad_k, grad_v, grad_gate, grad_beta, grad_S0,
                   B, H, T, dk, dv, cu_seqlens, N, dtype == KDA_BF16, gate_kind == KDA_GATE_SCALAR, workspace,
                   reinterpret_cast<hipStream_t>(stream)};
    return hip_status(kda::launch_chunk_bwd(a));
}

size_t kda_chunk_bwd_ew_workspace_bytes(int B, int H, int T, int dk, int dv, int N, int has_cu) {
    if (B <= 0 || H <= 0 || T < 0 || !size_ok(dk) || !size_ok(dv)) return 0;
    if (has_cu && (B != 1 || N <= 0)) return 0;
    return kda::bwd_workspace_bytes(B, H, T, dk, dv, has_cu != 0, has_cu ? N : B, true);
}

int kda_chunk_bwd_ew(const void* q, const void* k, const void* v, const void* gate, const void* erase,
                     const void* write, const float* S0, const float* dO, const float* dS_T, float* grad_q,
                     float* grad_k, float* grad_v, float* grad_gate, float* grad_erase, float* grad_write,
                     float* grad_S0, int B, int H, int T, int dk, int dv, const int32_t* cu_seqlens, int N, int dtype,
                     int gate_kind, void* workspace, size_t workspace_bytes, void* stream) {
    if (B <= 0 || H <= 0 || T < 0) return KDA_EINVAL;
    if (!size_ok(dk) || !size_ok(dv)) return KDA_ENOTSUP;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ENOTSUP;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return KDA_ENOTSUP;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen) {
        if (B != 1 || N <= 0) return KDA_EINVAL;
    } else {
        if (N != 0 && N != B) return KDA_EINVAL;
        N = B;
    }
    const bool need_data = T > 0;
    if (need_data && (!q || !k || !v || !gate || !erase || !write || !dO || !grad_q || !grad_k || !grad_v ||
                      !grad_gate || !grad_erase || !grad_write))
        return KDA_EINVAL;
    const uintptr_t es = dtype == KDA_BF16 ? 2 : 4;
    if (need_data && (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(gate, es) ||
                      !aligned(erase, es) || !aligned(write, es) || !aligned(dO) || !aligned(grad_q, 4) ||
                      !aligned(grad_k, 4) || !aligned(grad_v) || !aligned(grad_gate, 4) || !aligned(grad_erase, 4) ||
                      !aligned(grad_write)))
        return KDA_EALIGN;
    if ((S0 && !aligned(S0)) || (dS_T && !aligned(dS_T)) || (grad_S0 && !aligned(grad_S0)) ||
        (workspace && !aligned(workspace)))
        return KDA_EALIGN;
    if (varlen && !aligned(cu_seqlens, 4)) return KDA_EALIGN;
    const size_t need = kda::bwd_workspace_bytes(B, H, T, dk, dv, varlen, N, true);
    if (!workspace || workspace_bytes < need) return KDA_EINVAL;
    if (!need_data && !grad_S0) return KDA_OK;

    kda::BwdArgs a{q, k, v, gate, nullptr, S0, dO, dS_T, grad_q, grad_k, grad_v, grad_gate, nullptr, grad_S0,
                   B, H, T, dk, dv, cu_seqlens, N, dtype == KDA_BF16, gate_kind == KDA_GATE_SCALAR, workspace,
                   reinterpret_cast<hipStream_t>(stream), erase, write, grad_erase, grad_write};
    return hip_status(kda::launch_chunk_bwd(a));
}

size_t kda_chunk_bwd_cw_workspace_bytes(int B, int H, int T, int dk, int dv, int N, int has_cu) {
    if (B <= 0 || H <= 0 || T < 0 || (dk != 64 && dk != 128) || !size_ok(dv)) return 0;
    if (has_cu && (B != 1 || N <= 0)) return 0;
    return kda::cbwd_workspace_bytes(B, H, T, dk, dv, has_cu != 0, has_cu ? N : B);
}

int kda_chunk_bwd_cw(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                     const float* S0, const float* dO, const float* dS_T, float* grad_q, float* grad_k,
                     float* grad_v, float* grad_gate, float* grad_beta, float* grad_S0, int B, int H, int T,
                     int dk, int dv, const int32_t* cu_seqlens, int N, int dtype, int gate_kind,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (B <= 0 || H <= 0 || T < 0) return KDA_EINVAL;
    if ((dk != 64 && dk != 128) || !size_ok(dv)) return KDA_ENOTSUP;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ENOTSUP;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return KDA_ENOTSUP;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen) {
        if (B != 1 || N <= 0) return KDA_EINVAL;
    } else {
        if (N != 0 && N != B) return KDA_EINVAL;
        N = B;
    }
    const bool need_data = T > 0;
    if (need_data && (!q || !k || !v || !gate || !beta || !dO || !grad_q || !grad_k || !grad_v || !grad_gate ||
                      !grad_beta))
        return KDA_EINVAL;
    const uintptr_t es = dtype == KDA_BF16 ? 2 : 4;
    if (need_data && (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(gate, es) ||
                      !aligned(beta, es) || !aligned(dO) || !aligned(grad_q, 4) || !aligned(grad_k, 4) ||
                      !aligned(grad_v, 4) || !aligned(grad_gate, 4) || !aligned(grad_beta, 4)))
        return KDA_EALIGN;
    if ((S0 && !aligned(S0, 4)) || (dS_T && !aligned(dS_T, 4)) || (grad_S0 && !aligned(grad_S0, 4)) ||
        (workspace && !aligned(workspace)))
        return KDA_EALIGN;
    if (varlen && !aligned(cu_seqlens, 4)) return KDA_EALIGN;
    const size_t need = kda::cbwd_workspace_bytes(B, H, T, dk, dv, varlen, N);
    if (!workspace || workspace_bytes < need) return KDA_EINVAL;
    if (!need_data && !grad_S0) return KDA_OK;
    kda::BwdArgs a{q, k, v, gate, beta, S0, dO, dS_T, grad_q, grad_k, grad_v, grad_gate, grad_beta, grad_S0,
                   B, H, T, dk, dv, cu_seqlens, N, dtype == KDA_BF16, gate_kind == KDA_GATE_SCALAR, workspace,
                   reinterpret_cast<hipStream_t>(stream)};
    return hip_status(kda::launch_cbwd(a));
}

size_t kda_gauge_fold_workspace_bytes(int B, int H, int T, int dk, int N, int has_cu, int gate_kind) {
    if (B <= 0 || H <= 0 || T < 0 || !size_ok(dk)) return 0;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return 0;
    if (has_cu && (B != 1 || N <= 0)) return 0;
    return kda::gauge_fold_workspace_bytes(H, T, has_cu ? N : B, gate_kind == KDA_GATE_SCALAR ? 1 : dk);
}

int kda_gauge_fold(const void* q, const void* k, const void* gate, void* q_out, void* k_out, void* gate_out,
                   int8_t* sign_T, int B, int H, int T, int dk, const int32_t* cu_seqlens, int N, int dtype,
                   int gate_kind, void* workspace, size_t workspace_bytes, void* stream) {
    if (B <= 0 || H <= 0 || T < 0) return KDA_EINVAL;
    if (!size_ok(dk)) return KDA_ENOTSUP;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ENOTSUP;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return KDA_ENOTSUP;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen) {
        if (B != 1 || N <= 0) return KDA_EINVAL;
    } else {
        if (N != 0 && N != B) return KDA_EINVAL;
        N = B;
    }
    const bool need_data = T > 0;
    if (need_data && (!q || !k || !gate || !q_out || !k_out || !gate_out)) return KDA_EINVAL;
    const uintptr_t es = dtype == KDA_BF16 ? 2 : 4;
    const uintptr_t ga = gate_kind == KDA_GATE_SCALAR ? es : 16;   // channel gates are read 8 channels at a time
    if (need_data && (!aligned(q) || !aligned(k) || !aligned(gate, ga) || !aligned(q_out) || !aligned(k_out) ||
                      !aligned(gate_out, ga)))
        return KDA_EALIGN;
    if ((workspace && !aligned(workspace)) || (varlen && !aligned(cu_seqlens, 4))) return KDA_EALIGN;
    const size_t need = kda::gauge_fold_workspace_bytes(H, T, N, gate_kind == KDA_GATE_SCALAR ? 1 : dk);
    if (!workspace || workspace_bytes < need) return KDA_EINVAL;
    if (!need_data && !sign_T) return KDA_OK;
    kda::GaugeArgs a{q, k, gate, q_out, k_out, gate_out, B, H, T, dk, cu_seqlens, N, dtype == KDA_BF16,
                     gate_kind == KDA_GATE_SCALAR, workspace, reinterpret_cast<hipStream_t>(stream)};
    return hip_status(kda::launch_gauge_fold(a, sign_T));
}

namespace {
// Offsets in the gauge route's workspace: the forward's own workspace first
// (so that its status word sits at offset 0, as for kda_chunk_fwd), then the
// folded q, k and gate, c_T and the fold's scratch; off[6] is the total.
void gauge_route_parts(int B, int H, int T, int dk, int dv, int chunk, bool varlen, int N, bool bf16, bool sg,
                       size_t* off) {
    const size_t es = bf16 ? 2 : 4, gdim = sg ? 1 : (size_t)dk;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t qb = al((size_t)B * T * H * dk * es), gb = al((size_t)B * T * H * gdim * es);
    off[5] = 0;                                                                      // forward workspace
    off[0] = al(kda::chunk_workspace_bytes(B, H, T, dk, dv, chunk, varlen, N, bf16));   // q~
    off[1] = off[0] + qb;                                                            // k~
    off[2] = off[1] + qb;                                                            // alpha~
    off[3] = off[2] + gb;                                                            // c_T [N][H][gdim]
    off[4] = off[3] + al((size_t)N * H * gdim);                                      // fold scratch
    off[6] = off[4] + al(kda::gauge_fold_workspace_bytes(H, T, N, (int)gdim));
}
}  // namespace

size_t kda_chunk_fwd_gauge_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int N, int has_cu,
                                           int dtype, int gate_kind) {
    if (B <= 0 || H <= 0 || T < 0 || !size_ok(dk) || !size_ok(dv) || !chunk_ok(chunk)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return 0;
    if (has_cu && (B != 1 || N <= 0)) return 0;
    const bool varlen = has_cu != 0;
    size_t off[7];
    gauge_route_parts(B, H, T, dk, dv, chunk, varlen, varlen ? N : B, dtype == KDA_BF16,
                      gate_kind == KDA_GATE_SCALAR, off);
    return off[6];
}

int kda_chunk_fwd_gauge(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                        const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv, int chunk,
                        const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* workspace,
                        size_t workspace_bytes, void* stream) {
    if (B <= 0 || H <= 0 || T < 0) return KDA_EINVAL;
    if (!size_ok(dk) || !size_ok(dv) || !chunk_ok(chunk)) return KDA_ENOTSUP;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ENOTSUP;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return KDA_ENOTSUP;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen) {
        if (B != 1 || N <= 0) return KDA_EINVAL;
    } else {
        if (N != 0 && N != B) return KDA_EINVAL;
        N = B;
    }
    const bool need_data = T > 0;
    if (need_data && (!q || !k || !v || !gate || !beta || !o)) return KDA_EINVAL;
    const uintptr_t es = dtype == KDA_BF16 ? 2 : 4;
    if (need_data && (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(gate) || !aligned(beta, es) ||
                      !aligned(o, 4)))
        return KDA_EALIGN;
    if ((S0 && !aligned(S0, 4)) || (S_T && !aligned(S_T, 4)) || (workspace && !aligned(workspace))) return KDA_EALIGN;
    if (varlen && !aligned(cu_seqlens, 4)) return KDA_EALIGN;
    const bool sg = gate_kind == KDA_GATE_SCALAR;
    size_t off[7];
    gauge_route_parts(B, H, T, dk, dv, chunk, varlen, N, dtype == KDA_BF16, sg, off);
    const size_t need = off[6];
    if (!workspace || workspace_bytes < need) return KDA_EINVAL;
    if (!need_data && !S_T) return KDA_OK;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* w = static_cast<unsigned char*>(workspace);
    int8_t* sign = reinterpret_cast<int8_t*>(w + off[3]);
    kda::GaugeArgs g{q, k, gate, w + off[0], w + off[1], w + off[2], B, H, T, dk, cu_seqlens, N, dtype == KDA_BF16,
                     sg, w + off[4], st};
    hipError_t e = kda::launch_gauge_fold(g, sign);
    if (e == hipSuccess) {
        kda::ChunkArgs a{w + off[0], w + off[1], v, w + off[2], beta, S0, o, S_T, B, H, T, dk, dv, chunk, cu_seqlens,
                         N, dtype == KDA_BF16, sg, w + off[5], st, KDA_STAGE_ALL};
        e = kda::launch_chunk_fwd(a);
    }
    if (e == hipSuccess && S_T) e = kda::launch_gauge_state_flip(S_T, sign, N, H, dk, dv, sg, st);
    return hip_status(e);
}

int kda_decode_step(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                    float* S, float* o, int N, int H, int dk, int dv, int dtype, int gate_kind, void* stream) {
    if (N <= 0 || H <= 0) return KDA_EINVAL;
    if (!size_ok(dk) || !size_ok(dv)) return KDA_ENOTSUP;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ENOTSUP;
    if (gate_kind != KDA_GATE_CHANNEL && gate_kind != KDA_GATE_SCALAR) return KDA_ENOTSUP;
    if (!q || !k || !v || !gate || !beta || !S || !o) return KDA_EINVAL;
    const uintptr_t es = dtype == KDA_BF16 ? 2 : 4;
    if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(gate, es) || !aligned(beta, es) ||
        !aligned(S) || !aligned(o))
        return KDA_EALIGN;
    kda::DecodeArgs a{q, k, v, gate, beta, S, o, N, H, dk, dv, dtype == KDA_BF16,
                      gate_kind == KDA_GATE_SCALAR, reinterpret_cast<hipStream_t>(stream)};
    return hip_status(kda::launch_decode(a));
}

}  // extern "C"
