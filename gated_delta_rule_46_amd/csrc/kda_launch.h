// Host-side launch descriptors shared by the C-ABI and the kernel files.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    const void *q, *k, *v, *gate, *beta;
    float* S;
    float* o;
    int N, H, dk, dv;
    bool bf16, scalar_gate;
    hipStream_t stream;
    const void* erase = nullptr;   // erase [N, H, dk] and write [N, H, dv] gates, or none
    const void* write = nullptr;
};

struct ChunkArgs {
    const void *q, *k, *v, *gate, *beta;
    const float* S0;
    float* o;
    float* S_T;
    int B, H, T, dk, dv, chunk;
    const int32_t* cu_seqlens;  // device, N+1 entries, or null
    int N;                      // number of sequences (B when cu_seqlens is null)
    bool bf16, scalar_gate;
    void* workspace;
    hipStream_t stream;
    int stages;                 // bit 0: index + prep kernels, bit 1: state kernel
    // decoupled erase [.., dk] and write [.., dv] gates in the input dtype
    // (both set, beta unused) or none (both null)
    const void* erase = nullptr;
    const void* write = nullptr;
};

struct BwdArgs {
    const void *q, *k, *v, *gate, *beta;
    const float *S0, *dO, *dST;                            // dST may be null (zero)
    float *g_q, *g_k, *g_v, *g_gate, *g_beta, *g_S0;       // gradients; g_S0 may be null
    int B, H, T, dk, dv;
    const int32_t* cu_seqlens;                             // device, N+1 entries, or null
    int N;
    bool bf16, scalar_gate;
    void* workspace;
    hipStream_t stream;
    // decoupled erase [.., dk] and write [.., dv] gates in the input dtype
    // (both set, beta and g_beta unused) with their gradients, or none
    const void* erase = nullptr;
    const void* write = nullptr;
    float* g_erase = nullptr;
    float* g_write = nullptr;
};

struct GaugeArgs {
    const void *q, *k, *gate;
    void *q_out, *k_out, *gate_out;
    int B, H, T, dk;
    const int32_t* cu_seqlens;
    int N;
    bool bf16, scalar_gate;
    void* workspace;   // gauge_fold_workspace_bytes(...) bytes: segment parities
    hipStream_t stream;
};

// Bytes of intermediates one (chunk, head) pair occupies in the workspace.
size_t chunk_block_bytes(int dk, int dv, int chunk, bool bf16);
// Upper bound on the number of chunks over all sequences.
long chunk_count_bound(int B, int T, int chunk, bool varlen, int N);
// Total workspace bytes for one forward call.
size_t chunk_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, bool varlen, int N, bool bf16);

// Workspace bytes of one backward call (checkpoints and partial sums).
size_t bwd_workspace_bytes(int B, int H, int T, int dk, int dv, bool varlen, int N, bool ew = false);

// Gauge fold: workspace bytes (segment parities), the fold (c_T into sign_dev
// when it is not null), and the row flip of a final state by c_T.
size_t gauge_fold_workspace_bytes(int H, int T, int N, int gdim);
hipError_t launch_gauge_fold(const GaugeArgs& a, int8_t* sign_dev);
hipError_t launch_gauge_state_flip(float* S, const int8_t* sign, int N, int H, int dk, int dv, bool scalar_gate,
                                   hipStream_t stream);

// Argument checks of kda_chunk_fwd_stage, everything but the workspace (no HIP
// call): KDA_OK with the launch descriptor (workspace left null) and the
// workspace bytes the call needs, or a negative status.
int validate_chunk_fwd(int stage, const void* q, const void* k, const void* v, const void* gate, const void* beta,
                       const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv, int chunk,
                       const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* stream, ChunkArgs* args,
                       size_t* need);
// hipError_t -> KDA status (KDA_EHIP records the code for kda_last_hip_error).
int hip_to_status(hipError_t e);

// Per-sequence first chunk index (cstart, N+1 entries) of packed sequences.
hipError_t launch_chunk_index(const int32_t* cu, int32_t* cstart, int N, int C, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_chunk_bwd(const BwdArgs& a);
// Chunkwise backward (dk 64 or 128): workspace bytes and launch.
size_t cbwd_workspace_bytes(int B, int H, int T, int dk, int dv, bool varlen, int N);
hipError_t launch_cbwd(const BwdArgs& a);
hipError_t launch_chunk_fwd(const ChunkArgs& a);

}  // namespace kda
