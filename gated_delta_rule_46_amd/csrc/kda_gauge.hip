// Gauge transform of Complex KDA onto positive gates (Complex KDA summary,
// method step 5: the cumulative gate signs are absorbed into keys and
// queries, and the kernels of the positive-gate case run unchanged).
//
// Per sequence, head and key channel (one sign per token and head for the
// scalar gate), with s_t = -1 where alpha_t < 0 and +1 otherwise (zero and
// -0.0 included: a zero gate erases the history, so its sign is immaterial):
//   c_t = s_1 ... s_t,  q~_t = c_t q_t,  k~_t = c_t k_t,  alpha~_t = |alpha_t|
// and the final state of the positive-gate run is mapped back by
// S_T = Diag(c_T) S~_T. Every output value is an input value with its sign
// bit flipped or cleared, so the fold is exact in any precision.
//
// The sign products are a prefix XOR of sign bits along the sequence, done
// in three launches over (sequence, head, 32-token segment): the parity of
// each segment; an exclusive scan over the segments; the fold itself, each
// segment starting from its prefix.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int G_SEG = 32;    // tokens per segment
constexpr int G_UN = 8;      // tokens whose loads are issued together
constexpr int G_NT = 64;     // threads per block (one wave)

struct GaugeParams {
    const void *q, *k, *gate;
    void *qo, *ko, *go;
    uint8_t* par;       // [N][H][nseg][gdim] segment parities, then their exclusive scan
    int8_t* sign;       // [N][H][gdim] c_T, or null
    const int32_t* cu;
    int H, T, dk, gdim, nseg;
};

template <class TIn> struct Bits;
template <> struct Bits<uint16_t> { using U = uint16_t; static constexpr U SIGN = 0x8000u; };
template <> struct Bits<float> { using U = uint32_t; static constexpr U SIGN = 0x80000000u; };

// negative: sign bit set and some other bit set (-0.0 counts as +)
template <class TIn>
__device__ __forceinline__ bool is_neg(typename Bits<TIn>::U x) {
    using U = typename Bits<TIn>::U;
    return (x & Bits<TIn>::SIGN) && (U)(x & (U)~Bits<TIn>::SIGN);
}

__device__ __forceinline__ void seq_bounds(const GaugeParams& p, int s, int& b0, int& t0, int& len) {
    if (p.cu) {
        b0 = 0;
        t0 = p.cu[s];
        len = p.cu[s + 1] - t0;
    } else {
        b0 = s;
        t0 = 0;
        len = p.T;
    }
}

// Thread layout of the parity and fold kernels: each thread owns 8
// consecutive key channels of one (sequence, head) -- 16-byte accesses for
// bf16 -- and the dk / 8 threads of a head are adjacent lanes, so a wave
// reads several heads' contiguous channel rows of one token at once.
constexpr int G_CPT = 8;

template <class TIn>
struct Lane8 {
    using U = typename Bits<TIn>::U;
    static constexpr int NV = (int)(G_CPT * sizeof(U)) / 16;   // 16-byte pieces
    uint4 v[NV];
    __device__ __forceinline__ void load(const U* p) {
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = reinterpret_cast<const uint4*>(p)[i];
    }
    __device__ __forceinline__ void store(U* p) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) reinterpret_cast<uint4*>(p)[i] = v[i];
    }
    __device__ __forceinline__ U get(int c) const { return reinterpret_cast<const U*>(v)[c]; }
    __device__ __forceinline__ void set(int c, U x) { reinterpret_cast<U*>(v)[c] = x; }
};

// (sequence, head) and first channel of this thread; false past the last head
__device__ __forceinline__ bool gauge_lane(const GaugeParams& p, int nsh, int& sh, int& c0) {
    const int tph = p.dk / G_CPT;                      // threads per head
    const int hpb = G_NT / tph;                        // heads per block
    sh = blockIdx.y * hpb + threadIdx.x / tph;
    c0 = (threadIdx.x % tph) * G_CPT;
    return sh < nsh;
}

template <class TIn>
__global__ void __launch_bounds__(G_NT) gauge_parity_kernel(GaugeParams p, int nsh) {
    lds_poison(0);
    using U = typename Bits<TIn>::U;
    int sh, c0;
    if (!gauge_lane(p, nsh, sh, c0)) return;
    const bool sg = p.gdim == 1;
    if (sg && c0 != 0) return;
    const int g = blockIdx.x, s = sh / p.H, h = sh % p.H;
    int b0, t0, len;
    seq_bounds(p, s, b0, t0, len);
    const int ta = g * G_SEG, tb = min(len, ta + G_SEG);
    const U* __restrict__ A = (const U*)p.gate;
    uint32_t x = 0;   // bit c: parity of channel c0 + c (bit 0 only for the scalar gate)
    for (int t = ta; t < tb; t += G_UN) {
        Lane8<TIn> a[G_UN];
#pragma unroll
        for (int u = 0; u < G_UN; ++u) {
            const size_t row = ((size_t)b0 * p.T + t0 + t + u) * p.H + h;
            if (t + u < tb) {
                if (sg) a[u].set(0, A[row]);
                else a[u].load(A + row * p.dk + c0);
            } else {
#pragma unroll
                for (int i = 0; i < Lane8<TIn>::NV; ++i) a[u].v[i] = uint4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < G_UN; ++u)
#pragma unroll
            for (int c = 0; c < (sg ? 1 : G_CPT); ++c) x ^= (uint32_t)is_neg<TIn>(a[u].get(c)) << c;
    }
    uint8_t* dst = p.par + ((size_t)sh * p.nseg + g) * p.gdim + c0;
#pragma unroll
    for (int c = 0; c < (sg ? 1 : G_CPT); ++c) dst[c] = (uint8_t)((x >> c) & 1u);
}

// Exclusive prefix over the segments of each (sequence, head, channel), in
// place; c_T from the total.
__global__ void __launch_bounds__(256) gauge_scan_kernel(GaugeParams p, int rows) {
    lds_poison(0);
    const int r = blockIdx.x * 256 + threadIdx.x;   // (sequence, head) * gdim + channel
    if (r >= rows) return;
    const int sh = r / p.gdim, ch = r % p.gdim;
    uint8_t* __restrict__ base = p.par + (size_t)sh * p.nseg * p.gdim + ch;
    uint32_t acc = 0;
    for (int g0 = 0; g0 < p.nseg; g0 += 32) {   // 32 loads in flight, then the scan
        uint32_t v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) v[u] = g0 + u < p.nseg ? base[(size_t)(g0 + u) * p.gdim] : 0u;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
            if (g0 + u < p.nseg) base[(size_t)(g0 + u) * p.gdim] = (uint8_t)acc;
            acc ^= v[u];
        }
    }
    if (p.sign) p.sign[r] = acc ? (int8_t)-1 : (int8_t)1;
}

template <class TIn>
__global__ void __launch_bounds__(G_NT) gauge_apply_kernel(GaugeParams p, int nsh) {
    lds_poison(0);
    using U = typename Bits<TIn>::U;
    int sh, c0;
    if (!gauge_lane(p, nsh, sh, c0)) return;
    const int g = blockIdx.x, s = sh / p.H, h = sh % p.H;
    int b0, t0, len;
    seq_bounds(p, s, b0, t0, len);
    const int ta = g * G_SEG, tb = min(len, ta + G_SEG);
    if (ta >= tb) return;
    const bool sg = p.gdim == 1;
    const uint8_t* pre = p.par + ((size_t)sh * p.nseg + g) * p.gdim;
    uint32_t par = 0;   // bit c: running parity of channel c0 + c (all bits equal for the scalar gate)
#pragma unroll
    for (int c = 0; c < G_CPT; ++c) par |= (uint32_t)(pre[sg ? 0 : c0 + c] & 1u) << c;
    const U* __restrict__ A = (const U*)p.gate;
    const U* __restrict__ Q = (const U*)p.q;
    const U* __restrict__ K = (const U*)p.k;
    U* __restrict__ Ao = (U*)p.go;
    U* __restrict__ Qo = (U*)p.qo;
    U* __restrict__ Ko = (U*)p.ko;
    for (int t = ta; t < tb; t += G_UN) {
        Lane8<TIn> a[G_UN], qv[G_UN], kv[G_UN];
        U as[G_UN];
#pragma unroll
        for (int u = 0; u < G_UN; ++u) {
            if (t + u >= tb) continue;
            const size_t row = ((size_t)b0 * p.T + t0 + t + u) * p.H + h;
            if (sg) as[u] = A[row];
            else a[u].load(A + row * p.dk + c0);
            qv[u].load(Q + row * p.dk + c0);
            kv[u].load(K + row * p.dk + c0);
        }
#pragma unroll
        for (int u = 0; u < G_UN; ++u) {
            if (t + u >= tb) break;
            const size_t row = ((size_t)b0 * p.T + t0 + t + u) * p.H + h;
            if (sg) {
                par ^= is_neg<TIn>(as[u]) ? 0xFFu : 0u;
                if (c0 == 0) Ao[row] = (U)(as[u] & (U)~Bits<TIn>::SIGN);
            } else {
#pragma unroll
                for (int c = 0; c < G_CPT; ++c) {
                    const U x = a[u].get(c);
                    par ^= (uint32_t)is_neg<TIn>(x) << c;
                    a[u].set(c, (U)(x & (U)~Bits<TIn>::SIGN));
                }
                a[u].store(Ao + row * p.dk + c0);
            }
#pragma unroll
            for (int c = 0; c < G_CPT; ++c) {
                const U flip = ((par >> c) & 1u) ? Bits<TIn>::SIGN : (U)0;
                qv[u].set(c, (U)(qv[u].get(c) ^ flip));
                kv[u].set(c, (U)(kv[u].get(c) ^ flip));
            }
            qv[u].store(Qo + row * p.dk + c0);
            kv[u].store(Ko + row * p.dk + c0);
        }
    }
}

// S [N][H][dk][dv] rows times c_T (+1 / -1 per (sequence, head, channel), or
// one per (sequence, head) for the scalar gate).
__global__ void __launch_bounds__(256) gauge_state_flip_kernel(float* __restrict__ S, const int8_t* __restrict__ sign,
                                                               long rows, int dk, int dv, int gdim) {
    lds_poison(0);
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= rows * dv) return;
    const long r = e / dv;   // (sequence, head) * dk + channel
    const int8_t c = sign[gdim == 1 ? r / dk : r];
    if (c < 0) S[e] = -S[e];
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int gauge_segments(int T) { return (T + G_SEG - 1) / G_SEG; }

size_t gauge_fold_workspace_bytes(int H, int T, int N, int gdim) {
    return al256((size_t)N * H * gauge_segments(T) * gdim + 1);
}

hipError_t launch_gauge_fold(const GaugeArgs& a, int8_t* sign_dev) {
    GaugeParams p;
    p.q = a.q;
    p.k = a.k;
    p.gate = a.gate;
    p.qo = a.q_out;
    p.ko = a.k_out;
    p.go = a.gate_out;
    p.par = static_cast<uint8_t*>(a.workspace);
    p.sign = sign_dev;
    p.cu = a.cu_seqlens;
    p.H = a.H;
    p.T = a.T;
    p.dk = a.dk;
    p.gdim = a.scalar_gate ? 1 : a.dk;
    p.nseg = gauge_segments(a.T);
    const int nsh = a.N * a.H, hpb = G_NT / (a.dk / G_CPT);
    // segments along x (long sequences), groups of heads along y
    const dim3 grid((unsigned)p.nseg, (unsigned)((nsh + hpb - 1) / hpb));
    if (p.nseg > 0) {
        if (a.bf16) hipLaunchKernelGGL(gauge_parity_kernel<uint16_t>, grid, dim3(G_NT), 0, a.stream, p, nsh);
        else hipLaunchKernelGGL(gauge_parity_kernel<float>, grid, dim3(G_NT), 0, a.stream, p, nsh);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // the scan also writes c_T = +1 for sequences without tokens
    const int rows = a.N * a.H * p.gdim;
    hipLaunchKernelGGL(gauge_scan_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, a.stream, p, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nseg == 0) return e;
    if (a.bf16) hipLaunchKernelGGL(gauge_apply_kernel<uint16_t>, grid, dim3(G_NT), 0, a.stream, p, nsh);
    else hipLaunchKernelGGL(gauge_apply_kernel<float>, grid, dim3(G_NT), 0, a.stream, p, nsh);
    return hipGetLastError();
}

hipError_t launch_gauge_state_flip(float* S, const int8_t* sign, int N, int H, int dk, int dv, bool scalar_gate,
                                   hipStream_t stream) {
    const long rows = (long)N * H * dk;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(gauge_state_flip_kernel, dim3((unsigned)((rows * dv + 255) / 256)), dim3(256), 0, stream, S,
                       sign, rows, dk, dv, scalar_gate ? 1 : dk);
    return hipGetLastError();
}

}  // namespace kda
