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
// in three launches over (sequence, head, 256-token segment): the parity of
// each segment; an exclusive scan over the segments; the fold itself, each
// segment starting from its prefix.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int G_SEG = 256;   // tokens per segment
constexpr int G_NT = 128;    // threads per block: one key channel each

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

template <class TIn>
__global__ void __launch_bounds__(G_NT) gauge_parity_kernel(GaugeParams p) {
    using U = typename Bits<TIn>::U;
    const int sh = blockIdx.x, g = blockIdx.y, ch = threadIdx.x;
    const int s = sh / p.H, h = sh % p.H;
    int b0, t0, len;
    seq_bounds(p, s, b0, t0, len);
    if (ch >= p.gdim) return;
    const int ta = g * G_SEG, tb = min(len, ta + G_SEG);
    const U* A = (const U*)p.gate;
    uint32_t x = 0;
    for (int t = ta; t < tb; ++t) x ^= is_neg<TIn>(A[(((size_t)b0 * p.T + t0 + t) * p.H + h) * p.gdim + ch]);
    p.par[((size_t)sh * p.nseg + g) * p.gdim + ch] = (uint8_t)x;
}

// Exclusive prefix over the segments of each (sequence, head, channel), in
// place; c_T from the total.
__global__ void __launch_bounds__(256) gauge_scan_kernel(GaugeParams p, int rows) {
    const int r = blockIdx.x * 256 + threadIdx.x;   // (sequence, head) * gdim + channel
    if (r >= rows) return;
    const int sh = r / p.gdim, ch = r % p.gdim;
    uint32_t acc = 0;
    for (int g = 0; g < p.nseg; ++g) {
        uint8_t* x = p.par + ((size_t)sh * p.nseg + g) * p.gdim + ch;
        const uint32_t v = *x;
        *x = (uint8_t)acc;
        acc ^= v;
    }
    if (p.sign) p.sign[r] = acc ? (int8_t)-1 : (int8_t)1;
}

template <class TIn>
__global__ void __launch_bounds__(G_NT) gauge_apply_kernel(GaugeParams p) {
    using U = typename Bits<TIn>::U;
    const int sh = blockIdx.x, g = blockIdx.y, ch = threadIdx.x;
    const int s = sh / p.H, h = sh % p.H;
    int b0, t0, len;
    seq_bounds(p, s, b0, t0, len);
    if (ch >= p.dk) return;
    const int ta = g * G_SEG, tb = min(len, ta + G_SEG);
    if (ta >= tb) return;
    const bool sg = p.gdim == 1;
    const int gc = sg ? 0 : ch;   // this thread's gate channel
    uint32_t par = p.par[((size_t)sh * p.nseg + g) * p.gdim + gc];
    const U* A = (const U*)p.gate;
    const U* Q = (const U*)p.q;
    const U* K = (const U*)p.k;
    U* Ao = (U*)p.go;
    U* Qo = (U*)p.qo;
    U* Ko = (U*)p.ko;
#pragma unroll 4
    for (int t = ta; t < tb; ++t) {
        const size_t row = ((size_t)b0 * p.T + t0 + t) * p.H + h;
        const U a = A[row * p.gdim + gc];
        par ^= is_neg<TIn>(a);
        const U flip = par ? Bits<TIn>::SIGN : (U)0;
        Qo[row * p.dk + ch] = (U)(Q[row * p.dk + ch] ^ flip);
        Ko[row * p.dk + ch] = (U)(K[row * p.dk + ch] ^ flip);
        if (!sg || ch == 0) Ao[row * p.gdim + gc] = (U)(a & (U)~Bits<TIn>::SIGN);
    }
}

// S [N][H][dk][dv] rows times c_T (+1 / -1 per (sequence, head, channel), or
// one per (sequence, head) for the scalar gate).
__global__ void __launch_bounds__(256) gauge_state_flip_kernel(float* __restrict__ S, const int8_t* __restrict__ sign,
                                                               long rows, int dk, int dv, int gdim) {
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
    const dim3 grid((unsigned)(a.N * a.H), (unsigned)p.nseg);
    if (p.nseg > 0) {
        if (a.bf16) hipLaunchKernelGGL(gauge_parity_kernel<uint16_t>, grid, dim3(G_NT), 0, a.stream, p);
        else hipLaunchKernelGGL(gauge_parity_kernel<float>, grid, dim3(G_NT), 0, a.stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // the scan also writes c_T = +1 for sequences without tokens
    const int rows = a.N * a.H * p.gdim;
    hipLaunchKernelGGL(gauge_scan_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, a.stream, p, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nseg == 0) return e;
    if (a.bf16) hipLaunchKernelGGL(gauge_apply_kernel<uint16_t>, grid, dim3(G_NT), 0, a.stream, p);
    else hipLaunchKernelGGL(gauge_apply_kernel<float>, grid, dim3(G_NT), 0, a.stream, p);
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
