// Chunk addressing shared by the forward and the chunkwise backward: which
// tokens a global chunk index covers, for fixed-length batches and for packed
// sequences (cu_seqlens, with a per-sequence chunk index built on the device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct ChunkMap {
    const int32_t* cu;      // null when every sequence has length T
    const int32_t* cstart;  // first chunk of each sequence (N+1), varlen only
    int T, N, NC;           // NC: chunks per sequence when not varlen
    int c0, c1;             // not varlen: this launch covers chunks [c0, c1) of every sequence
};

// Workgroup-local chunk number -> global chunk index.
__device__ __forceinline__ int launch_chunk(const ChunkMap& m, int li) {
    if (m.cu != nullptr) return li;
    const int ns = m.c1 - m.c0;
    return (li / ns) * m.NC + m.c0 + li % ns;
}

// Chunk g -> first token (flattened over batch and time) and token count.
__device__ __forceinline__ bool resolve_chunk(const ChunkMap& m, int g, int C, long& t0, int& n) {
    if (m.cu == nullptr) {
        const int s = g / m.NC, c = g % m.NC;
        t0 = (long)s * m.T + (long)c * C;
        n = min(C, m.T - c * C);
        return true;
    }
    if (g >= m.cstart[m.N]) return false;
    int lo = 0, hi = m.N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (m.cstart[mid] <= g) lo = mid; else hi = mid - 1;
    }
    const int c = g - m.cstart[lo];
    const int len = m.cu[lo + 1] - m.cu[lo];
    t0 = (long)m.cu[lo] + (long)c * C;
    n = min(C, len - c * C);
    return true;
}

}  // namespace kda
