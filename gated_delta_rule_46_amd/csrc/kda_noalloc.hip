// kda_chunk_fwd without a caller-supplied workspace, for callers that cannot
// allocate device memory (work recorded under graph capture, allocation-free
// serving loops, harnesses that forbid hipMalloc). The forward's scratch --
// the status header, the chunk index of packed sequences and one block of
// intermediates per (chunk, head) -- lives in a fixed device array instead.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_launch.h"

// One copy per GPU the library runs on, held until the process ends. Host
// code never uses this name as an address: the device address comes from
// hipGetSymbolAddress, once per device, below.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch[MAX_DEVICES] = {};   // device address of `scratch`, per device

// Device address of the scratch array on the current device (looked up on
// the first call made with that device current).
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* gate,
                                     const void* beta, const float* S0, float* o, float* S_T, int B, int H, int T,
                                     int dk, int dv, int chunk, const int32_t* cu_seqlens, int N, int dtype,
                                     int gate_kind, void* stream) {
    kda::ChunkArgs a;
    size_t need = 0;
    const int st = kda::validate_chunk_fwd(KDA_STAGE_ALL, q, k, v, gate, beta, S0, o, S_T, B, H, T, dk, dv, chunk,
                                           cu_seqlens, N, dtype, gate_kind, stream, &a, &need);
    if (st != KDA_OK) return st;
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ESCRATCH;
    if (T == 0 && !S_T) return KDA_OK;
    void* p = nullptr;
    const hipError_t e = scratch_address(&p);
    if (e != hipSuccess) return kda::hip_to_status(e);
    a.workspace = p;   // the kernels take the device address, as they take a caller's workspace
    return kda::hip_to_status(kda::launch_chunk_fwd(a));
}
