// Chunkwise-parallel forward of the gated delta rule (KDA / Complex KDA / GDN).
//
// Recurrence (Complex KDA summary, background "diagonal-plus-rank-one"):
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.
// The pages name a chunkwise WY-parallel training form for this family; the
// chunk identities below are derived from the recurrence itself.
//
// For a chunk of C tokens entering with state S, with per-channel relative
// gate products rel(r, j) = prod_{j < tau <= r} alpha_tau (rel(r, r) = 1),
// Gamma_r = rel(r, -1) and u_r = beta_r (v_r - (Diag(alpha_r) S_{r-1})^T k_r):
//   A_rj   = beta_r sum_i k_ri rel_i(r, j) k_ji      (j < r)
//   P_rj   = sum_i q_ri rel_i(r, j) k_ji             (j <= r)
//   T      = (I + A)^{-1} Diag(beta)                 (UT form of the WY product)
//   U      = T V - T (Gamma o K) S                   = U~ - W S
//   O      = (Gamma o Q) S + P U
//   S_next = Diag(Gamma_last) S + K_end^T U,         K_end[j] = rel(last, j) o k_j
//
// Two kernels:
//  * prep  -- one workgroup per (chunk, head), all chunks in parallel. Gate
//    products, gated Gram matrices, the triangular inverse, U~ = T V, and the
//    operands W, Gamma o Q, K_end^T, P written to a workspace as MFMA fragments.
//  * state -- walks the chunks of each sequence in order, per 16 value
//    columns ("slice") of one (sequence, head), with that slice of S in fp32
//    registers. bf16, dk = 128, chunk 64: four waves per slice, each holding a
//    quarter of the state rows and loading its quarter of the chunk operands
//    into registers one chunk ahead (one slice per workgroup while the slices
//    fit one per CU; otherwise two slices per workgroup, with copy waves that
//    stage the chunk operands in LDS). dk = 64: two waves per slice. Other
//    cases: one wave per slice with copy waves.
//
// Gated Gram without overflow, with exact signs and zeros: every pair
// (r > j) inside a chunk is separated at exactly one level of the binary
// split of the chunk (halves, quarters, ... single tokens). At that level a
// midpoint m with j <= m < r gives rel(r, j) = rel(r, m) * rel(m, j), a prefix
// product on the right and a suffix product on the left, both plain products
// of gates of magnitude <= 1. Signs and exact zeros carry through the
// multiplications, and nothing is ever divided. One scaled operand per level
// turns the level into an ordinary matrix product; an entry is kept from the
// level that separates its pair.
//
// Precision. Inputs are exact in the operand formats. Matrix operands are
// fp16 with a power-of-two scale per matrix (the scale is a property of the
// data, chosen so the largest entry lies in [0.5, 1)), value-side operands
// with one such scale per column, products accumulate in fp32, and the state
// stays fp32. The triangular inverse runs in fp32. The one term that dominates
// an output -- the current token's own update, P_rr u_r -- is applied in fp32.
// With fp32 inputs every contraction runs on fp32 MFMA instead.
#include <type_traits>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

// vmcnt(0) with lgkmcnt and expcnt left alone (gfx9 s_waitcnt encoding).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// vmcnt(N): wait until at most N vector memory operations of this wave are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm_upto() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// LDS writes of this wave are complete and visible to its own later reads.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// ------------------------------------------------------------------ one (chunk, head) block of the workspace

enum { SC_W = 0, SC_Q = 1, SC_K = 2, SC_P = 3, SC_T = 4, SC_INV = 8 };   // W Q K P inverses: one 16-byte read

template <int DK, int C, bool F32M>
struct Lay {
    using TM = typename std::conditional<F32M, float, _Float16>::type;
    static constexpr int RB = C / 16, CB = DK / 16;
    static constexpr int KSD = (DK + 31) / 32, KSC = (C + 31) / 32;
    static constexpr int FRAG = 64 * 8 * (int)sizeof(TM);   // one 16x32 fragment tile
    static constexpr size_t W_OFF = 0;                                      // W       [RB][KSD] A frags
    static constexpr size_t QG_OFF = W_OFF + (size_t)RB * KSD * FRAG;       // Gamma o Q [RB][KSD]
    static constexpr size_t KE_OFF = QG_OFF + (size_t)RB * KSD * FRAG;      // K_end^T [CB][KSC]
    static constexpr size_t PS_OFF = KE_OFF + (size_t)CB * KSC * FRAG;      // strictly lower P [RB][KSC]
    static constexpr size_t PD_OFF = PS_OFF + (size_t)RB * KSC * FRAG;      // diagonal of P, fp32 [C]
    static constexpr size_t GN_OFF = PD_OFF + (size_t)C * 4;                // gamma_last, fp32 [DK]
    static constexpr size_t SU_OFF = GN_OFF + (size_t)DK * 4;               // inverse scales of U~ columns [128]
    static constexpr size_t SC_OFF = SU_OFF + 128 * 4;                      // matrix scales [8] + inverses [8]
    static constexpr size_t BYTES = (SC_OFF + 64 + 1023) / 1024 * 1024;     // shared part
    // U~ = T V of one 16-column value slice in accumulator layout: lane l holds
    // rows 16 rb + 4 (l / 16) + e of column l % 16. Stored [RB / UPR][64][UPR * 4]
    // so that one lane reads UPR row blocks with one 8- or 16-byte load.
    static constexpr int UPR = (!F32M && RB >= 2) ? 2 : 1;
    static constexpr size_t USL = (size_t)C * 16 * sizeof(TM);
    __host__ __device__ static constexpr size_t u_off(int rb, int lane) {
        return (((size_t)(rb / UPR) * 64 + lane) * UPR + rb % UPR) * 4 * sizeof(TM);
    }
};

// ------------------------------------------------------------------ fragments

template <class TM> struct FragOf;
template <> struct FragOf<_Float16> { using type = f16x8; };
template <> struct FragOf<float> { using type = f32x8; };

template <class TM>
__device__ __forceinline__ typename FragOf<TM>::type to_frag(const f32x8& x, float s) {
    if constexpr (std::is_same<TM, float>::value) {
        return x;   // fp32 operands carry no scale
    } else {
        return to_f16x8(x, s);
    }
}

template <class TM>
__device__ __forceinline__ void st_frag(unsigned char* base, int tile, int lane, const typename FragOf<TM>::type& f) {
    *reinterpret_cast<typename FragOf<TM>::type*>(base + ((size_t)tile * 64 + lane) * sizeof(f)) = f;
}

// 16-deep fp32 product on 16x16 tiles: step m takes K index 4g + m from lane group g.
__device__ __forceinline__ f32x4 mma16_f32(const f32x4& a, const f32x4& b, f32x4 c) {
#pragma unroll
    for (int m = 0; m < 4; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], c, 0, 0, 0);
    return c;
}

// Sum over the four lanes that hold one column of a 16x16 D tile (lanes i,
// i+16, i+32, i+48). Every lane receives the same bits: each step adds the
// same two operands in both lanes of a pair.
__device__ __forceinline__ float colsum4(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t u2 = __float_as_uint(s);
    const auto b = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace kda

#include "kda_chunkmap.h"

namespace kda {

// cstart[s] = sum over earlier sequences of ceil(len / C); one workgroup.
__global__ void __launch_bounds__(256) chunk_index_kernel(const int32_t* __restrict__ cu, int32_t* __restrict__ cstart,
                                                          int N, int C) {
    lds_poison(0);
    __shared__ int32_t part[256];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int s = base + threadIdx.x;
        int v = 0;
        if (s < N) {
            const int len = cu[s + 1] - cu[s];
            v = len > 0 ? (len + C - 1) / C : 0;
        }
        part[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int add = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
            __syncthreads();
            part[threadIdx.x] += add;
            __syncthreads();
        }
        if (s < N) cstart[s + 1] = carry + part[threadIdx.x];
        __syncthreads();
        if (threadIdx.x == 255) carry += part[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) cstart[0] = 0;
}

hipError_t launch_chunk_index(const int32_t* cu, int32_t* cstart, int N, int C, hipStream_t stream) {
    hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(256), 0, stream, cu, cstart, N, C);
    return hipGetLastError();
}

// ------------------------------------------------------------------ prep kernel

// An operand staged in LDS as fragment tiles: tile (row / 16, k / 32); inside
// a tile, lane group g owns a run of 16 slots (one per row i) holding the 8
// values lane (i, g) reads for its fragment (row i, K positions kpos(g, p)).
// Groups and tiles are padded (group stride = 16 slots + 16 or 32 bytes, tile
// stride = 4 groups) so that a wave writing one row, two adjacent K
// positions per lane, hits 4-byte banks that differ in both the group and
// the K step, while each lane's row offset stays a constant: a lane computes
// one base address and reaches every row with the instruction offset.
template <class TM>
struct Stg {
    static constexpr int SLOT = 8 * (int)sizeof(TM);
    static constexpr int GS = 17 * SLOT;   // 272 (fp16) or 544 (fp32) bytes
    static constexpr int TS = 4 * GS;                                 // 1088 or 2176 bytes
};
template <class TM, int KS>
__device__ __forceinline__ uint32_t stage_off(int row, int k) {
    const int R = row >> 4, i = row & 15, s = k >> 5, q = k & 31;
    const int g = (q & 15) >> 2, p = (q & 3) + ((q >> 4) << 2);
    return (uint32_t)((R * KS + s) * Stg<TM>::TS + g * Stg<TM>::GS + i * Stg<TM>::SLOT + p * (int)sizeof(TM));
}
template <class TM, int KS>
__device__ __forceinline__ uint32_t stage_frag_off(int R, int s, int lane) {
    const int i = lane & 15, g = lane >> 4;
    return (uint32_t)((R * KS + s) * Stg<TM>::TS + g * Stg<TM>::GS + i * Stg<TM>::SLOT);
}

template <class F>
__device__ __forceinline__ F lds_ld(uint32_t off) {
    extern __shared__ __align__(16) unsigned char smem[];
    return *reinterpret_cast<const F*>(smem + off);
}
template <class F>
__device__ __forceinline__ void lds_st(uint32_t off, const F& v) {
    extern __shared__ __align__(16) unsigned char smem[];
    *reinterpret_cast<F*>(smem + off) = v;
}

// n consecutive operand values (n = 1, 2 or 4) into LDS.
template <class TM, int NV>
__device__ __forceinline__ void st_vals(uint32_t off, const float* x) {
    typedef TM v2 __attribute__((ext_vector_type(2)));
    typedef TM v4 __attribute__((ext_vector_type(4)));
    if constexpr (NV == 1) {
        lds_st<TM>(off, (TM)x[0]);
    } else if constexpr (NV == 2) {
        lds_st<v2>(off, v2{(TM)x[0], (TM)x[1]});
    } else {
        lds_st<v4>(off, v4{(TM)x[0], (TM)x[1], (TM)x[2], (TM)x[3]});
    }
}

// One lane's values of one input tensor over the 16 tokens of its block, for
// its CPL channels; bf16 inputs stay packed (two channels per register).
template <class TIn, int CPL>
struct Gx {
    float v[16][CPL];
    __device__ __forceinline__ float get(int t, int j) const { return v[t][j]; }
    __device__ __forceinline__ void load(const float* p, int t) {
        if constexpr (CPL == 2) {
            typedef float f2 __attribute__((ext_vector_type(2)));
            const f2 u = *reinterpret_cast<const f2*>(p);
            v[t][0] = u[0];
            v[t][1] = u[1];
        } else {
            v[t][0] = *p;
        }
    }
    __device__ __forceinline__ void fill(int t, float x) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) v[t][j] = x;
    }
    // one value for every channel: fill_from only loads, widen (after all the
    // loads are issued) copies it to the other channels
    __device__ __forceinline__ void fill_from(const float* p, int t) { v[t][0] = *p; }
    __device__ __forceinline__ void widen(int t) {
#pragma unroll
        for (int j = 1; j < CPL; ++j) v[t][j] = v[t][0];
    }
};
template <int CPL>
struct Gx<uint16_t, CPL> {
    uint32_t w[16];   // CPL == 2: channel 0 in the low half; CPL == 1: the low half
    __device__ __forceinline__ float get(int t, int j) const {
        return __uint_as_float(j ? (w[t] & 0xffff0000u) : (w[t] << 16));
    }
    __device__ __forceinline__ void load(const uint16_t* p, int t) {
        if constexpr (CPL == 2) w[t] = *reinterpret_cast<const uint32_t*>(p);
        else w[t] = *p;
    }
    __device__ __forceinline__ void fill(int t, float x) {
        const uint32_t b = __float_as_uint(x) >> 16;
        w[t] = CPL == 2 ? (b | (b << 16)) : b;
    }
    __device__ __forceinline__ void fill_from(const uint16_t* p, int t) { w[t] = *p; }
    __device__ __forceinline__ void widen(int t) {
        if constexpr (CPL == 2) w[t] = w[t] | (w[t] << 16);
    }
};

// The same values once the operand scales are known: k * sK and q * sQ (and
// alpha unscaled). bf16 inputs go to fp16 pairs -- exact, a bf16 value times a
// power of two lands in fp16's normal range -- which mixed-precision FMAs
// read directly; fp32 inputs stay fp32.
template <class TIn, int CPL>
struct Hx {
    float v[16][CPL];
    __device__ __forceinline__ float get(int t, int j) const { return v[t][j]; }
    __device__ __forceinline__ float mul(int t, int j, float f) const { return v[t][j] * f; }
    __device__ __forceinline__ void set(int t, int j, float x) { v[t][j] = x; }
    __device__ __forceinline__ void opaque() {}
};
template <int CPL>
struct Hx<uint16_t, CPL> {
    typedef _Float16 hv __attribute__((ext_vector_type(2)));
    hv v[16];   // CPL == 1 uses the first half
    __device__ __forceinline__ float get(int t, int j) const { return (float)v[t][j]; }
    // value * f in one mixed-precision FMA (the fp16 operand read in place);
    // the +0 addend only changes the sign of a zero product, which no later
    // sum or product here can see
    __device__ __forceinline__ float mul(int t, int j, float f) const { return __builtin_fmaf((float)v[t][j], f, 0.f); }
    __device__ __forceinline__ void set(int t, int j, float x) { v[t][j] = (_Float16)x; }
    // Mark the pairs as rewritten (no instruction): conversions to fp32 are
    // then redone inside each phase, folded into mixed FMAs, rather than
    // kept live across phases.
    __device__ __forceinline__ void opaque() {
#pragma unroll
        for (int t = 0; t < 16; ++t) asm volatile("" : "+v"(v[t]));
    }
};

template <int C, int KSC>
__host__ __device__ constexpr int tf_count() {
    int n = 0;
    for (int rb = 0; rb < C / 16; ++rb) n += (rb / 2 < KSC - 1 ? rb / 2 : KSC - 1) + 1;
    return n;
}
// Index of T fragment (rb, s), s <= rb / 2, in row-block order.
template <int KSC>
__host__ __device__ constexpr int tf_index(int rb, int s) {
    int n = 0;
    for (int r = 0; r < rb; ++r) n += (r / 2 < KSC - 1 ? r / 2 : KSC - 1) + 1;
    return n + s;
}

template <class TIn, int DK, int C, bool F32M, bool EW = false>
struct PrepLds {
    using TM = typename Lay<DK, C, F32M>::TM;
    static constexpr int NBK = C / 16, KSD = (DK + 31) / 32, KSC = (C + 31) / 32, CB = DK / 16;
    static constexpr int TILE = Stg<TM>::TS;                // staged operand tile
    static constexpr int TFT = 64 * 8 * (int)sizeof(TM);    // T fragment tile (lane-ordered)
    static constexpr int LDX = C + 4;   // row stride (floats) of the fp32 inverse arrays
    static constexpr int NTF = tf_count<C, KSC>();
    static constexpr size_t al(size_t x) { return (x + 15) / 16 * 16; }
    static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t BETA = 0;                                   // fp32 [C]
    static constexpr size_t TOT = al(BETA + (size_t)C * 4);             // gate totals per token block [NBK][DK]
    static constexpr size_t RED = al(TOT + (size_t)NBK * DK * 4);       // cross-wave maxima [32]
    static constexpr size_t RGN = al(RED + 32 * 4);                     // reused region
    // staged value rows (value width up to 128)
    static constexpr size_t VST = RGN;
    static constexpr size_t WST = VST + ((size_t)C * 128 * sizeof(TIn) + 1023) / 1024 * 1024;   // write gates
    static constexpr size_t END_V = WST + (EW ? ((size_t)C * 128 * sizeof(TIn) + 1023) / 1024 * 1024 : 0);
    // Gamma o Q and K_end^T tiles
    static constexpr size_t QGT = RGN;
    static constexpr size_t KET = QGT + (size_t)NBK * KSD * TILE;
    static constexpr size_t END_A = KET + (size_t)CB * KSC * TILE;
    // one split level: K-side and Q-side tiles
    static constexpr size_t XT = RGN;
    static constexpr size_t YT = XT + (size_t)NBK * KSD * TILE;
    static constexpr size_t END_L = YT + (size_t)NBK * KSD * TILE;
    // inverse: A and X = (I + A)^{-1}, fp32 row-major
    static constexpr size_t AM = RGN;
    static constexpr size_t XM = al(AM + (size_t)C * LDX * 4);
    static constexpr size_t END_I = al(XM + (size_t)C * LDX * 4);
    // T fragments (over A), then (Gamma o K)^T tiles (over X)
    static constexpr size_t TF = RGN;
    static constexpr size_t GKT = TF + (size_t)NTF * TFT;
    static constexpr size_t END_G = GKT + (size_t)CB * KSC * TILE;
    static constexpr size_t BYTES = mx(mx(mx(END_A, END_L), mx(END_I, END_G)), END_V);
    static_assert(TF + (size_t)NTF * TFT <= END_I, "T fragments fit the inverse area");
};

struct PrepParams {
    const void *q, *k, *v, *gate, *beta;
    const void *erase, *write;   // erase [.., dk] and write [.., dv] gates (erase/write form only)
    unsigned* status;   // cleared by the first workgroup
    unsigned char* ws;
    size_t blk_bytes;
    ChunkMap map;
    int H, DV;
};

// Is local entry (r, j) of a 16x16 diagonal block separated at within-block
// level hh (hh == 0: the diagonal itself)?
__device__ __forceinline__ bool sep_at(int r, int j, int hh) {
    if (hh == 0) return r == j;
    const int w = 2 * hh;
    return (r / w == j / w) && (r % w >= hh) && (j % w < hh);
}

// One (chunk, head) item of the prep work on the four waves of a workgroup.
// EW: decoupled erase and write gates, S_t = (I - k (e o k)^T) Diag(alpha) S
// + k (w o v)^T. The chunk identities keep their form with beta = 1, the
// read key e o k in place of k wherever a row of A or of W = T (Gamma o K) is
// formed (the rows r that read the state), k itself wherever a column of A
// or P or a row of K_end is (the direction the state is written along), and
// w o v in place of v.
template <class TIn, int DK, int C, bool SG, bool F32M, bool EW>
__device__ __forceinline__ void prep_item(const PrepParams& p, int item) {
    using L = Lay<DK, C, F32M>;
    using SM = PrepLds<TIn, DK, C, F32M, EW>;
    using TM = typename L::TM;
    using F = typename FragOf<TM>::type;
    constexpr int RB = L::RB, CB = L::CB, KSD = L::KSD, KSC = L::KSC;
    constexpr int NBK = C / 16;
    constexpr int CPL = DK >= 64 ? DK / 64 : 1;   // channels per lane in the gate phases
    constexpr int ACT = DK >= 64 ? 64 : DK;       // active lanes per wave in the gate phases
    constexpr int LDX = SM::LDX;
    constexpr int NBL = C == 64 ? 2 : (C == 32 ? 1 : 0);   // split levels between 16-token blocks

    extern __shared__ __align__(16) unsigned char smem[];
    float* s_beta = reinterpret_cast<float*>(smem + SM::BETA);
    float* s_tot = reinterpret_cast<float*>(smem + SM::TOT);
    float* s_red = reinterpret_cast<float*>(smem + SM::RED);
    float* s_am = reinterpret_cast<float*>(smem + SM::AM);
    float* s_xm = reinterpret_cast<float*>(smem + SM::XM);

    const int H = p.H, DV = p.DV;
    const int h = item % H, gidx = launch_chunk(p.map, item / H);
    long t0;
    int n;
    if (!resolve_chunk(p.map, gidx, C, t0, n)) return;   // uniform over the workgroup

    const int tid = threadIdx.x, lane = tid % WAVE;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);   // wave index, uniform
    const int li = lane % 16, lg = lane / 16;
    unsigned char* blk = p.ws + ((size_t)gidx * H + h) * p.blk_bytes;
    const TIn* gq = (const TIn*)p.q;
    const TIn* gk = (const TIn*)p.k;
    const TIn* gv = (const TIn*)p.v;
    const TIn* gg = (const TIn*)p.gate;
    const TIn* gb = (const TIn*)p.beta;

    // value rows of the chunk (and write-gate rows) -> LDS, asynchronously
    // and first, so that their latency overlaps that of the gate loads; rows
    // past the chunk end fall outside the descriptor and arrive as zeros
    {
        const int rby = DV * (int)sizeof(TIn);            // bytes of one value row
        const int lpr = rby / 16, rpi = 64 / lpr;          // lanes per row, rows per instruction
        const uint32_t rowb = (uint32_t)H * (uint32_t)rby;
        const int ni = (C * rby + 1023) / 1024;
#pragma unroll
        for (int src = 0; src < (EW ? 2 : 1); ++src) {
            const TIn* base = src == 0 ? gv : (const TIn*)p.write;
            const size_t dst = src == 0 ? SM::VST : SM::WST;
            const __amdgpu_buffer_rsrc_t rv =
                make_rsrc(base + ((size_t)t0 * H + h) * DV, (uint32_t)(n - 1) * rowb + (uint32_t)rby);
            for (int u = w; u < ni; u += 4) {
                const uint32_t voff = (uint32_t)(u * rpi + lane / lpr) * rowb + (uint32_t)(lane % lpr) * 16;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rv, (__attribute__((address_space(3))) void*)(smem + dst + (size_t)u * 1024), 16, voff, 0, 0, 0);
            }
        }
    }

    // ---- gate phases: wave b owns tokens 16b..16b+15, lane owns CPL channels
    const bool gate_lane = (w < NBK) && (lane < ACT);
    const int b = w;
    const int c0 = lane * CPL;
    Gx<TIn, CPL> kk, qq, aa, ee;
    float mk = 0.f, mq = 0.f, me = 0.f;
    // Rows past the chunk end read row n - 1 (n >= 1) and are replaced after
    // the loads: no branch or use of a loaded value between two loads, so all
    // 16 rows are in flight together.
    if (gate_lane) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const size_t row = (size_t)(t0 + min(16 * b + t, n - 1)) * H + h;
            kk.load(gk + row * DK + c0, t);
            qq.load(gq + row * DK + c0, t);
            if constexpr (SG) aa.fill_from(gg + row, t);
            else aa.load(gg + row * DK + c0, t);
            if constexpr (EW) ee.load((const TIn*)p.erase + row * DK + c0, t);
        }
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        if (!gate_lane || 16 * b + t >= n) {
            kk.fill(t, 0.f);
            qq.fill(t, 0.f);
            aa.fill(t, 1.f);
            if constexpr (EW) ee.fill(t, 0.f);
        } else if constexpr (SG) {
            aa.widen(t);
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            mk = fmaxf(mk, fabsf(kk.get(t, j)));
            mq = fmaxf(mq, fabsf(qq.get(t, j)));
            if constexpr (EW) me = fmaxf(me, fabsf(kk.get(t, j) * ee.get(t, j)));
        }
    }
    if constexpr (EW) {
        if (tid < C) s_beta[tid] = tid < n ? 1.f : 0.f;
    } else {
        if (tid < C) s_beta[tid] = tid < n ? ld_in(gb + (size_t)(t0 + tid) * H + h) : 0.f;
    }

    if (gate_lane) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            float tot = 1.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) tot *= aa.get(t, j);
            s_tot[b * DK + c0 + j] = tot;
        }
    }
    mk = wave_max(mk);
    mq = wave_max(mq);
    if constexpr (EW) me = wave_max(me);
    if (lane == 0) { s_red[w] = mk; s_red[4 + w] = mq; }
    if (EW && lane == 0) s_red[24 + w] = me;
    wait_vm_all();
    __syncthreads();
    float sK = 1.f, sQ = 1.f, iK = 1.f, iQ = 1.f, sE = 1.f, iE = 1.f;
    if constexpr (!F32M) {
        const float m1 = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        const float m2 = fmaxf(fmaxf(s_red[4], s_red[5]), fmaxf(s_red[6], s_red[7]));
        sK = pow2_scale_for(m1);
        iK = pow2_inv_scale_for(m1);
        sQ = pow2_scale_for(m2);
        iQ = pow2_inv_scale_for(m2);
        if constexpr (EW) {
            const float m3 = fmaxf(fmaxf(s_red[24], s_red[25]), fmaxf(s_red[26], s_red[27]));
            sE = pow2_scale_for(m3);
            iE = pow2_inv_scale_for(m3);
        }
    }
    // scaled operand values for every later phase: k * sK, q * sQ, alpha
    // (and the read key (e o k) * sE, rounded once to the operand format)
    Hx<TIn, CPL> hk, hq, ha, hke;
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            hk.set(t, j, kk.get(t, j) * sK);
            hq.set(t, j, qq.get(t, j) * sQ);
            ha.set(t, j, aa.get(t, j));
            if constexpr (EW) hke.set(t, j, kk.get(t, j) * ee.get(t, j) * sE);
        }
    // row side of A and of W: the read key (e o k) in the erase/write form
    auto hr_mul = [&](int t, int j, float f) { return EW ? hke.mul(t, j, f) : hk.mul(t, j, f); };

    // ---- value fragments (B operand over tokens), kept in registers until
    // U~ = T V: wave w owns value slices w and w + 4, one scale per column
    F vf[2][KSC];
    float ivs[2];
    {
        const TIn* vst = reinterpret_cast<const TIn*>(smem + SM::VST);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int sl = w + 4 * jj;
            ivs[jj] = 1.f;
            f32x8 x[KSC];
            float mv = 0.f;
            const int col = 16 * sl + li;
            if constexpr (!F32M && C >= 32) {
                // transposing LDS reads: within each group of 16 lanes, lane
                // i receives element i % 4 of the 4-element pieces that lanes
                // i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4 address. Lane s of
                // group g addresses row 32 ks + 16 hf + 4 g + s / 4, columns
                // 16 sl + 4 (s % 4) ..+3, so lane (li, g) gets the column li
                // values of rows kpos(g, 4 hf + 0..3): one B fragment half.
                typedef short v4s __attribute__((ext_vector_type(4)));
                const bool ok = sl < DV / 16;
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int row = 32 * ks + 16 * hf + 4 * lg + li / 4;
                        const int cc = ok ? 16 * sl + 4 * (li % 4) : 0;
                        const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) v4s*)(smem + SM::VST + (size_t)(row * DV + cc) * sizeof(TIn)));
                        v4s rw = r;
                        if constexpr (EW)
                            rw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) v4s*)(smem + SM::WST + (size_t)(row * DV + cc) * sizeof(TIn)));
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            float v = ok ? bf16_bits_to_f32((uint16_t)r[j]) : 0.f;
                            if constexpr (EW) v *= ok ? bf16_bits_to_f32((uint16_t)rw[j]) : 0.f;
                            x[ks][4 * hf + j] = v;
                            mv = fmaxf(mv, fabsf(v));
                        }
                    }
            } else {
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                    for (int pp = 0; pp < 8; ++pp) {
                        const int t = 32 * ks + kpos(lg, pp);
                        float v = (sl < DV / 16 && t < C) ? ld_in(vst + t * DV + col) : 0.f;
                        if constexpr (EW) {
                            const TIn* wst = reinterpret_cast<const TIn*>(smem + SM::WST);
                            v *= (sl < DV / 16 && t < C) ? ld_in(wst + t * DV + col) : 0.f;
                        }
                        x[ks][pp] = v;
                        mv = fmaxf(mv, fabsf(v));
                    }
            }
            float sv = 1.f;
            if constexpr (!F32M) {
                mv = colmax4(mv);
                sv = pow2_scale_for(mv);
                ivs[jj] = pow2_inv_scale_for(mv);
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) vf[jj][ks] = to_frag<TM>(x[ks], sv);
        }
    }
    __syncthreads();

    // ---- Gamma o Q (rows tokens), K_end^T (rows channels), gamma_last
    hk.opaque();
    hq.opaque();
    ha.opaque();
    if constexpr (EW) hke.opaque();
    if (gate_lane) {
        float pre[CPL], suf[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            pre[j] = 1.f;
            suf[j] = 1.f;
            float all = 1.f;
#pragma unroll
            for (int bb = 0; bb < NBK; ++bb) {
                const float tb = s_tot[bb * DK + c0 + j];
                if (bb < b) pre[j] *= tb;
                if (bb > b) suf[j] *= tb;
                all *= tb;
            }
            if (b == 0) reinterpret_cast<float*>(blk + L::GN_OFF)[c0 + j] = all;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float qg[2];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                pre[j] = ha.mul(t, j, pre[j]);
                qg[j] = hq.mul(t, j, pre[j]);
            }
            st_vals<TM, CPL>(SM::QGT + stage_off<TM, KSD>(16 * b + t, c0), qg);
            if constexpr (DK == 16) {
                const float z = 0.f;
                st_vals<TM, 1>(SM::QGT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
            }
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            float ke[16];
            float r = suf[j];
#pragma unroll
            for (int t = 15; t >= 0; --t) {
                ke[t] = hk.mul(t, j, r);
                r = ha.mul(t, j, r);
            }
#pragma unroll
            for (int u = 0; u < 16; u += 4) {
                st_vals<TM, 4>(SM::KET + stage_off<TM, KSC>(c0 + j, 16 * b + u), ke + u);
                if constexpr (C == 16) {
                    const float z[4] = {0.f, 0.f, 0.f, 0.f};
                    st_vals<TM, 4>(SM::KET + stage_off<TM, KSC>(c0 + j, 16 + u), z);
                }
            }
        }
    }
    __syncthreads();
    for (int tt = w; tt < RB * KSD; tt += 4)
        st_frag<TM>(blk + L::QG_OFF, tt, lane, lds_ld<F>(SM::QGT + stage_frag_off<TM, KSD>(tt / KSD, tt % KSD, lane)));
    for (int tt = w; tt < CB * KSC; tt += 4)
        st_frag<TM>(blk + L::KE_OFF, tt, lane, lds_ld<F>(SM::KET + stage_frag_off<TM, KSC>(tt / KSC, tt % KSC, lane)));
    __syncthreads();

    // ---- split levels between 16-token blocks. Each block pair (R > J) is
    // separated at exactly one of them; the wave that takes the pair holds its
    // A^T and P^T tiles (row j, column r) until they are written out.
    f32x4 pa[NBL > 0 ? NBL : 1], pq[NBL > 0 ? NBL : 1];
    int pR[NBL > 0 ? NBL : 1], pJ[NBL > 0 ? NBL : 1];
#pragma unroll
    for (int lev = 0; lev < NBL; ++lev) {
        const int hb = (C >> (lev + 1)) / 16;   // half width in blocks
        hk.opaque();
        hq.opaque();
        ha.opaque();
        if constexpr (EW) hke.opaque();
        if (gate_lane) {
            const int gs = (b / (2 * hb)) * 2 * hb, midb = gs + hb;
            const bool right = b >= midb;
            float f[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                f[j] = 1.f;
                if (right) {
                    for (int bb = midb; bb < b; ++bb) f[j] *= s_tot[bb * DK + c0 + j];
                } else {
                    for (int bb = b + 1; bb < midb; ++bb) f[j] *= s_tot[bb * DK + c0 + j];
                }
            }
            if (right) {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    float x[2], y[2];
#pragma unroll
                    for (int j = 0; j < CPL; ++j) {
                        f[j] = ha.mul(t, j, f[j]);
                        x[j] = hr_mul(t, j, f[j]);
                        y[j] = hq.mul(t, j, f[j]);
                    }
                    st_vals<TM, CPL>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0), x);
                    st_vals<TM, CPL>(SM::YT + stage_off<TM, KSD>(16 * b + t, c0), y);
                    if constexpr (DK == 16) {
                        const float z = 0.f;
                        st_vals<TM, 1>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
                        st_vals<TM, 1>(SM::YT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
                    }
                }
            } else {
#pragma unroll
                for (int t = 15; t >= 0; --t) {
                    float x[2];
#pragma unroll
                    for (int j = 0; j < CPL; ++j) {
                        x[j] = hk.mul(t, j, f[j]);
                        f[j] = ha.mul(t, j, f[j]);
                    }
                    st_vals<TM, CPL>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0), x);
                    if constexpr (DK == 16) {
                        const float z = 0.f;
                        st_vals<TM, 1>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
                    }
                }
            }
        }
        __syncthreads();
        const int npairs = (NBK / (2 * hb)) * hb * hb;
        pR[lev] = -1;
        pJ[lev] = 0;
        pa[lev] = zero4();
        pq[lev] = zero4();
        if (w < npairs) {
            const int gi = w / (hb * hb), rem = w % (hb * hb);
            const int R = gi * 2 * hb + hb + rem / hb, J = gi * 2 * hb + rem % hb;
            f32x4 ta = zero4(), tp = zero4();
#pragma unroll
            for (int s = 0; s < KSD; ++s) {
                const F xj = lds_ld<F>(SM::XT + stage_frag_off<TM, KSD>(J, s, lane));
                const F xr = lds_ld<F>(SM::XT + stage_frag_off<TM, KSD>(R, s, lane));
                const F yr = lds_ld<F>(SM::YT + stage_frag_off<TM, KSD>(R, s, lane));
                ta = mma(xj, xr, ta);
                tp = mma(xj, yr, tp);
            }
            pa[lev] = ta;
            pq[lev] = tp;
            pR[lev] = R;
            pJ[lev] = J;
        }
        __syncthreads();
    }

    // ---- split levels inside each 16-token block (8, 4, 2, 1, then the
    // diagonal): wave b stages and reads only its own block, no barriers.
    f32x4 dA = zero4(), dP = zero4();   // A^T and P^T of diagonal block (b, b)
    if (w < NBK) {
#pragma unroll
        for (int lev = 0; lev < 5; ++lev) {
            const int hh = lev < 4 ? (8 >> lev) : 0;
            hk.opaque();
            hq.opaque();
            ha.opaque();
            if constexpr (EW) hke.opaque();
            if (lane < ACT) {
                if (hh > 0) {
#pragma unroll
                    for (int g0 = 0; g0 < 16; g0 += 2 * hh) {
                        float f[CPL];
#pragma unroll
                        for (int j = 0; j < CPL; ++j) f[j] = 1.f;
#pragma unroll
                        for (int t = g0 + hh; t < g0 + 2 * hh; ++t) {
                            float x[2], y[2];
#pragma unroll
                            for (int j = 0; j < CPL; ++j) {
                                f[j] = ha.mul(t, j, f[j]);
                                x[j] = hr_mul(t, j, f[j]);
                                y[j] = hq.mul(t, j, f[j]);
                            }
                            st_vals<TM, CPL>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0), x);
                            st_vals<TM, CPL>(SM::YT + stage_off<TM, KSD>(16 * b + t, c0), y);
                            if constexpr (DK == 16) {
                                const float z = 0.f;
                                st_vals<TM, 1>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
                                st_vals<TM, 1>(SM::YT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
                            }
                        }
#pragma unroll
                        for (int j = 0; j < CPL; ++j) f[j] = 1.f;
#pragma unroll
                        for (int t = g0 + hh - 1; t >= g0; --t) {
                            float x[2];
#pragma unroll
                            for (int j = 0; j < CPL; ++j) {
                                x[j] = hk.mul(t, j, f[j]);
                                f[j] = ha.mul(t, j, f[j]);
                            }
                            st_vals<TM, CPL>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0), x);
                            if constexpr (DK == 16) {
                                const float z = 0.f;
                                st_vals<TM, 1>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        float x[2], y[2];
#pragma unroll
                        for (int j = 0; j < CPL; ++j) {
                            x[j] = hk.get(t, j);
                            y[j] = hq.get(t, j);
                        }
                        st_vals<TM, CPL>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0), x);
                        st_vals<TM, CPL>(SM::YT + stage_off<TM, KSD>(16 * b + t, c0), y);
                        if constexpr (DK == 16) {
                            const float z = 0.f;
                            st_vals<TM, 1>(SM::XT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
                            st_vals<TM, 1>(SM::YT + stage_off<TM, KSD>(16 * b + t, c0 + 16), &z);
                        }
                    }
                }
            }
            wave_lds_fence();
            f32x4 ta = zero4(), tp = zero4();
#pragma unroll
            for (int s = 0; s < KSD; ++s) {
                const F xb = lds_ld<F>(SM::XT + stage_frag_off<TM, KSD>(b, s, lane));
                const F yb = lds_ld<F>(SM::YT + stage_frag_off<TM, KSD>(b, s, lane));
                if (hh > 0) ta = mma(xb, xb, ta);
                tp = mma(xb, yb, tp);
            }
            // lane (li, lg) holds entries (row j = 4 lg + e, column r = li)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool keep = sep_at(li, 4 * lg + e, hh);
                if (hh > 0) dA[e] = keep ? dA[e] + ta[e] : dA[e];
                dP[e] = keep ? dP[e] + tp[e] : dP[e];
            }
            wave_lds_fence();
        }
    }
    __syncthreads();   // the inverse arrays overlay the level tiles

    // ---- A = Diag(beta) A' into LDS (fp32, row-major); largest |P| below the diagonal
    const float invKK = iK * (EW ? iE : iK), invQK = iQ * iK;
    float mp = 0.f;
    {
        auto put_a = [&](int R, int J, const f32x4& t) {
            const int r = 16 * R + li;
            const float sb = invKK * s_beta[r];
            lds_st<f32x4>(SM::AM + (uint32_t)((r * LDX + 16 * J + 4 * lg) * 4), t * sb);
        };
        if (w < NBK) {
            put_a(b, b, dA);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * lg + e < li) mp = fmaxf(mp, fabsf(dP[e]));
        }
#pragma unroll
        for (int lev = 0; lev < NBL; ++lev) {
            if (pR[lev] >= 0) {
                put_a(pR[lev], pJ[lev], pa[lev]);
#pragma unroll
                for (int e = 0; e < 4; ++e) mp = fmaxf(mp, fabsf(pq[lev][e]));
            }
        }
    }
    mp = wave_max(mp);
    if (lane == 0) s_red[8 + w] = mp;
    __syncthreads();

    // ---- P: strictly lower part as scaled A fragments, diagonal in fp32
    float sP = 1.f, iP = 1.f;
    if constexpr (!F32M) {
        const float m = fmaxf(fmaxf(s_red[8], s_red[9]), fmaxf(s_red[10], s_red[11])) * invQK;
        sP = pow2_scale_for(m);
        iP = pow2_inv_scale_for(m);
    }
    {
        typedef TM v4 __attribute__((ext_vector_type(4)));
        const float cP = invQK * sP;
        // lane (li, lg) holds P[16R + li][16J + 4lg + e]: half J % 2 of fragment (R, J / 2)
        auto put_p = [&](int R, int J, const f32x4& t, bool diag) {
            v4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (TM)((!diag || 4 * lg + e < li) ? t[e] * cP : 0.f);
            *reinterpret_cast<v4*>(blk + L::PS_OFF + ((size_t)(R * KSC + J / 2) * 64 + lane) * 8 * sizeof(TM) +
                                   (J % 2) * 4 * sizeof(TM)) = x;
        };
        if (w < NBK) {
            put_p(b, b, dP, true);
            if (b % 2 == 0) put_p(b, b + 1, zero4(), false);   // upper half of the fragment
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * lg + e == li) reinterpret_cast<float*>(blk + L::PD_OFF)[16 * b + li] = dP[e] * invQK;
        }
#pragma unroll
        for (int lev = 0; lev < NBL; ++lev)
            if (pR[lev] >= 0) put_p(pR[lev], pJ[lev], pq[lev], false);
    }

    // ---- inverses of the 16x16 unit-lower diagonal blocks of I + A, one wave
    // per block: lane (li, lg) keeps rows 4lg..4lg+3 of column li
    if (w < NBK) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (4 * lg + e == li) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            const f32x4 a = lds_ld<f32x4>(SM::AM + (uint32_t)(((16 * b + r) * LDX + 16 * b + 4 * lg) * 4));
            const float part = colsum4(a[0] * x[0] + a[1] * x[1] + a[2] * x[2] + a[3] * x[3]);
            const float xr = r > li ? -part : (r == li ? 1.f : 0.f);
            if (lg == r / 4) x[r % 4] = xr;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) s_xm[(16 * b + 4 * lg + e) * LDX + 16 * b + li] = x[e];
    }
    __syncthreads();
    // ---- off-diagonal blocks by distance, X_RJ = -X_RR sum_{J<=M<R} A_RM X_MJ
#pragma unroll
    for (int d = 1; d < NBK; ++d) {
        if (w < NBK - d) {
            const int J = w, R = w + d;
            f32x4 y = zero4();
            for (int M = J; M < R; ++M) {
                const f32x4 a = lds_ld<f32x4>(SM::AM + (uint32_t)(((16 * R + li) * LDX + 16 * M + 4 * lg) * 4));
                f32x4 bx;
#pragma unroll
                for (int m = 0; m < 4; ++m) bx[m] = s_xm[(16 * M + 4 * lg + m) * LDX + 16 * J + li];
                y = mma16_f32(a, bx, y);
            }
            const f32x4 xr = lds_ld<f32x4>(SM::XM + (uint32_t)(((16 * R + li) * LDX + 16 * R + 4 * lg) * 4));
            const f32x4 res = mma16_f32(xr, y, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) s_xm[(16 * R + 4 * lg + e) * LDX + 16 * J + li] = -res[e];
        }
        __syncthreads();
    }

    // ---- T = X Diag(beta) as A fragments (rows r, K over tokens j <= r), one scale
    constexpr int NTF = SM::NTF;
    f32x8 tv[2];
    float mt = 0.f;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int f = w + 4 * jj;
        tv[jj] = f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (f < NTF) {
            int rb = 0, s = 0;
            for (int r = 0, acc = 0; r < RB; ++r) {
                const int ns = (r / 2 < KSC - 1 ? r / 2 : KSC - 1) + 1;
                if (f < acc + ns) { rb = r; s = f - acc; break; }
                acc += ns;
            }
            const int row = 16 * rb + li;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int c = 32 * s + 16 * half + 4 * lg;
                if (c < C) {
                    const f32x4 xv = lds_ld<f32x4>(SM::XM + (uint32_t)((row * LDX + c) * 4));
                    const f32x4 bv = lds_ld<f32x4>(SM::BETA + (uint32_t)(c * 4));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = (c + e <= row) ? xv[e] * bv[e] : 0.f;
                        tv[jj][4 * half + e] = v;
                        mt = fmaxf(mt, fabsf(v));
                    }
                }
            }
        }
    }
    mt = wave_max(mt);
    if (lane == 0) s_red[12 + w] = mt;
    __syncthreads();
    float sT = 1.f, iT = 1.f;
    if constexpr (!F32M) {
        const float m = fmaxf(fmaxf(s_red[12], s_red[13]), fmaxf(s_red[14], s_red[15]));
        sT = pow2_scale_for(m);
        iT = pow2_inv_scale_for(m);
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int f = w + 4 * jj;
        if (f < NTF) lds_st<F>(SM::TF + (uint32_t)((f * 64 + lane) * sizeof(F)), to_frag<TM>(tv[jj], sT));
    }
    __syncthreads();
    auto tfrag = [&](int rb, int s) { return lds_ld<F>(SM::TF + (uint32_t)((tf_index<KSC>(rb, s) * 64 + lane) * sizeof(F))); };

    // ---- (Gamma o K)^T tiles (rows channels, K over tokens) for W
    hk.opaque();
    ha.opaque();
    if constexpr (EW) hke.opaque();
    if (gate_lane) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            float r = 1.f;
            for (int bb = 0; bb < b; ++bb) r *= s_tot[bb * DK + c0 + j];
            float gk[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                r = ha.mul(t, j, r);
                gk[t] = hr_mul(t, j, r);
            }
#pragma unroll
            for (int u = 0; u < 16; u += 4) {
                st_vals<TM, 4>(SM::GKT + stage_off<TM, KSC>(c0 + j, 16 * b + u), gk + u);
                if constexpr (C == 16) {
                    const float z[4] = {0.f, 0.f, 0.f, 0.f};
                    st_vals<TM, 4>(SM::GKT + stage_off<TM, KSC>(c0 + j, 16 + u), z);
                }
            }
        }
    }

    // ---- U~ = T V for this wave's value slices, one scale per column
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int sl = w + 4 * jj;
        if (sl < DV / 16) {
            f32x4 acc[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                acc[rb] = zero4();
#pragma unroll
                for (int s = 0; s < KSC; ++s)
                    if (s <= rb / 2) acc[rb] = mma(tfrag(rb, s), vf[jj][s], acc[rb]);
            }
            const float cu = iT * ivs[jj];
            float m = 0.f;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[rb][e] *= cu;
                    m = fmaxf(m, fabsf(acc[rb][e]));
                }
            float sU = 1.f, iU = 1.f;
            if constexpr (!F32M) {
                m = colmax4(m);
                sU = pow2_scale_for(m);
                iU = pow2_inv_scale_for(m);
            }
            typedef TM v4 __attribute__((ext_vector_type(4)));
            unsigned char* ub = blk + L::BYTES + (size_t)sl * L::USL;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                v4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (TM)(acc[rb][e] * sU);
                *reinterpret_cast<v4*>(ub + L::u_off(rb, lane)) = x;
            }
            if (lg == 0) reinterpret_cast<float*>(blk + L::SU_OFF)[16 * sl + li] = iU;
        }
    }
    __syncthreads();

    // ---- W = T (Gamma o K), computed as W^T = (Gamma o K)^T T^T: two stacked
    // 16x16 tiles of W^T (channel blocks 2s, 2s+1) are the A fragment of W for
    // token block rb and channel step s.
    constexpr int NWI = (RB * KSD + 3) / 4;
    f32x4 wt[NWI][2];
    float mw = 0.f;
    const float invKT = (EW ? iE : iK) * iT;
#pragma unroll
    for (int j = 0; j < NWI; ++j) {
        wt[j][0] = zero4();
        wt[j][1] = zero4();
        const int it = w + 4 * j;
        if (it >= RB * KSD) continue;
        const int rb = it / KSD, s2 = it % KSD;
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
            if (s > rb / 2) continue;
            const F bf = tfrag(rb, s);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int cb = 2 * s2 + half;
                if (cb >= CB) continue;
                const F af = lds_ld<F>(SM::GKT + stage_frag_off<TM, KSC>(cb, s, lane));
                wt[j][half] = mma(af, bf, wt[j][half]);
            }
        }
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wt[j][half][e] *= invKT;
                mw = fmaxf(mw, fabsf(wt[j][half][e]));
            }
    }
    float sW = 1.f, iW = 1.f;
    if constexpr (!F32M) {
        mw = wave_max(mw);
        if (lane == 0) s_red[16 + w] = mw;
        __syncthreads();
        const float m1 = fmaxf(fmaxf(s_red[16], s_red[17]), fmaxf(s_red[18], s_red[19]));
        sW = pow2_scale_for(m1);
        iW = pow2_inv_scale_for(m1);
    }
#pragma unroll
    for (int j = 0; j < NWI; ++j) {
        const int it = w + 4 * j;
        if (it >= RB * KSD) continue;
        st_frag<TM>(blk + L::W_OFF, it, lane, to_frag<TM>(dtiles_to_frag(wt[j][0], wt[j][1]), sW));
    }
    if (tid == 0) {
        float* sc = reinterpret_cast<float*>(blk + L::SC_OFF);
        sc[SC_W] = sW;
        sc[SC_Q] = sQ;
        sc[SC_K] = sK;
        sc[SC_T] = sT;
        sc[SC_P] = sP;
        sc[SC_INV + SC_W] = iW;
        sc[SC_INV + SC_Q] = iQ;
        sc[SC_INV + SC_K] = iK;
        sc[SC_INV + SC_T] = iT;
        sc[SC_INV + SC_P] = iP;
    }
}

template <class TIn, int DK, int C, bool SG, bool F32M, bool EW>
__global__ void __launch_bounds__(256, F32M ? 1 : (EW ? 2 : 3)) chunk_prep_kernel(PrepParams p) {
    lds_poison((uint32_t)PrepLds<TIn, DK, C, F32M, EW>::BYTES);
    if (blockIdx.x == 0 && threadIdx.x == 0) *p.status = 0u;
    prep_item<TIn, DK, C, SG, F32M, EW>(p, xcd_remap(blockIdx.x, gridDim.x));
}

// ------------------------------------------------------------------ state kernel

// Workgroup -> walker item (hs * nsg + sg: (sequence, head) hs, its part sg).
// The nsg workgroups of one (sequence, head) read the same blocks, so they go
// to one XCD (shared L2); consecutive (sequence, head) pairs go to different
// XCDs, so that sequences of different lengths spread over the XCDs instead
// of one XCD taking all the heads of the longest sequence. Workgroups are
// dispatched round-robin over the XCDs (L % NXCD); when the pair count is not
// a multiple of NXCD the items are spread as xcd_remap does.
__device__ __forceinline__ int walker_item(int L, int total, int nsg) {
    const int nhs = total / nsg;
    if (nhs % NXCD != 0) return xcd_remap(L, total);
    const int x = L % NXCD, r = L / NXCD;
    return (NXCD * (r / nsg) + x) * nsg + r % nsg;
}

struct StateParams {
    const float* S0;
    float* o;
    float* S_T;
    const unsigned char* ws;
    size_t blk_bytes;
    ChunkMap map;
    int H, DV, NSG;   // NSG: workgroups per (sequence, head)
    unsigned* status; // the call's status word: a wave whose bounded wait expired sets STATUS_WAIT_EXPIRED
};

// Bounded LDS flag waits inside one workgroup. Every wave of the workgroup is
// resident and posts its flag once per chunk, so a wait ends long before the
// bound; should it ever expire, the wave stops storing outputs (o through a
// zero-size descriptor, S_T skipped) and raises the status word instead of
// writing values computed from stale operands.
constexpr int WAIT_POLLS = 1 << 24;
constexpr unsigned STATUS_WAIT_EXPIRED = 1u;

__device__ __forceinline__ void raise_status(unsigned* status, int expired) {
    if (expired && (threadIdx.x % 64) == 0) __hip_atomic_fetch_or(status, STATUS_WAIT_EXPIRED, __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_AGENT);
}

// NW compute waves per workgroup, each owning SPW 16-column slices of the
// state; NW copy waves alongside.
template <int DK, int C, bool F32M, int NW, int SPW>
struct StateSmem {
    using L = Lay<DK, C, F32M>;
    static constexpr int NSL = NW * SPW;   // slices per workgroup
    static constexpr size_t UBYTES = ((size_t)NSL * L::USL + 1023) / 1024 * 1024;   // whole 1 KiB copies
    static constexpr size_t BUF = L::BYTES + UBYTES;
    static constexpr int NBUF = (2 * BUF <= 160 * 1024) ? 2 : 1;
    static constexpr size_t BYTES = NBUF * BUF;
};

// Copy one chunk's block -- the shared part and this workgroup's value
// slices -- into LDS with asynchronous buffer-to-LDS loads, 1 KiB per wave
// instruction; the block address lives in scalar registers. The NW copy
// waves split the work.
template <int DK, int C, bool F32M, int NW, int NSL>
__device__ __forceinline__ void stage_chunk(uint32_t lds_off, const unsigned char* gblk, size_t blk_bytes, int sg, int w,
                                            int lane, int rot = 0) {
    using L = Lay<DK, C, F32M>;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int U0 = (int)(L::BYTES / 1024);
    constexpr int UV = (int)((NSL * L::USL + 1023) / 1024);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(gblk, (uint32_t)blk_bytes);
    const int vbase = (int)(L::BYTES + (size_t)sg * NSL * L::USL) - U0 * 1024;
    // rot: start the shared part at piece (rot * 16) mod U0 (issue order only)
    const int r0 = (rot * 16) % U0;
#pragma unroll
    for (int i = w; i < U0 + UV; i += NW) {
        const int u = i < U0 ? (i + r0) % U0 : i;
        const int soff = u < U0 ? u * 1024 : vbase + u * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(smem + lds_off + u * 1024),
                                                 16, lane * 16, soff, 0, 0);
    }
}

// Touch every 128-byte line of a chunk's block (the part this workgroup
// copies) with one 4-byte load, so that its later copy into LDS is served by
// L2. The caller folds the loaded words into a value it keeps.
template <int DK, int C, bool F32M, int NW, int NSL, int NPF>
__device__ __forceinline__ void touch_chunk(uint32_t (&pf)[NPF], const unsigned char* gblk, size_t blk_bytes, int sg,
                                            int w, int lane) {
    using L = Lay<DK, C, F32M>;
    constexpr int L0 = (int)(L::BYTES / 128);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(gblk, (uint32_t)blk_bytes);
    const int vbase = (int)(L::BYTES + (size_t)sg * NSL * L::USL) - L0 * 128;
#pragma unroll
    for (int k = 0; k < NPF; ++k) {
        const int line = (k * NW + w) * 64 + lane;
        const int off = line < L0 ? line * 128 : vbase + line * 128;
        pf[k] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
}

template <int DK, int C, bool F32M, int NW, int SPW>
__global__ void __launch_bounds__(128 * NW) chunk_state_kernel(StateParams p) {
    lds_poison((uint32_t)StateSmem<DK, C, F32M, NW, SPW>::BYTES);
    using L = Lay<DK, C, F32M>;
    using SM = StateSmem<DK, C, F32M, NW, SPW>;
    using TM = typename L::TM;
    using F = typename FragOf<TM>::type;
    constexpr int RB = L::RB, CB = L::CB, KSD = L::KSD, KSC = L::KSC, UPR = L::UPR;
    constexpr int NSL = SM::NSL;
    constexpr uint32_t FB = sizeof(F);   // bytes of one lane's fragment

    const int item = walker_item(blockIdx.x, gridDim.x, p.NSG);
    const int sg = item % p.NSG;
    const int hs = item / p.NSG;
    const int H = p.H, DV = p.DV;
    const int h = hs % H, s = hs / H;
    constexpr int expired = 0;   // this walker has no flag waits
    // waves 0..NW-1 compute SPW 16-column slices each; waves NW..2NW-1 stream
    // the next chunk's block into the other LDS buffer meanwhile
    const int lane = threadIdx.x % 64;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);   // wave index, uniform
    const bool copier = wv >= NW;
    const int w = copier ? wv - NW : wv;
    const int li = lane % 16, lg = lane / 16;
    int col[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) col[j] = 16 * (sg * NSL + w * SPW + j) + li;

    long bos, eos;
    int cs, ce;
    if (p.map.cu == nullptr) {
        bos = (long)s * p.map.T + (long)p.map.c0 * C;
        eos = (long)(s + 1) * p.map.T;
        cs = s * p.map.NC + p.map.c0;
        ce = s * p.map.NC + p.map.c1;
    } else {
        bos = p.map.cu[s];
        eos = p.map.cu[s + 1];
        cs = p.map.cstart[s];
        ce = p.map.cstart[s + 1];
    }

    // state slices: rows 16*cb + 4*lg + e, columns col[j]
    f32x4 S[SPW][CB];
    const size_t sbase = ((size_t)s * H + h) * DK * DV;
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[j][cb][e] = (p.S0 && !copier) ? p.S0[sbase + (size_t)(16 * cb + 4 * lg + e) * DV + col[j]] : 0.f;

    auto gblock = [&](int cg) { return p.ws + ((size_t)cg * H + h) * p.blk_bytes; };
    const uint32_t orow = (uint32_t)H * DV * 4;                 // bytes between token rows of o
    const uint32_t lfr = (uint32_t)lane * FB;                   // this lane's slot in a fragment tile

    constexpr int NPF = (int)((SM::BUF / 128 + 64 * NW - 1) / (64 * NW));   // lines per copy lane
    uint32_t pf[NPF];
    uint32_t sink = 0;
#pragma unroll
    for (int k = 0; k < NPF; ++k) pf[k] = 0;
    if (copier && cs < ce) {
        stage_chunk<DK, C, F32M, NW, NSL>(0, gblock(cs), p.blk_bytes, sg, w, lane);
        wait_vm_all();
    }
    __syncthreads();

    for (int cg = cs; cg < ce; ++cg) {
        if (copier) {
            // double buffer: fetch chunk cg+1 while the compute waves read chunk
            // cg, and pull chunk cg+2 into L2; single buffer: the fetch waits
            // for the compute waves (second barrier below)
            if constexpr (SM::NBUF == 2) {
#pragma unroll
                for (int k = 0; k < NPF; ++k) sink ^= pf[k];
                if (cg + 1 < ce) {
                    stage_chunk<DK, C, F32M, NW, NSL>((uint32_t)(((cg + 1 - cs) % 2) * SM::BUF), gblock(cg + 1),
                                                      p.blk_bytes, sg, w, lane);
                    if (cg + 2 < ce) {
                        touch_chunk<DK, C, F32M, NW, NSL, NPF>(pf, gblock(cg + 2), p.blk_bytes, sg, w, lane);
                        wait_vm_upto<NPF>();
                    } else {
                        wait_vm_all();
                    }
                }
            }
            __syncthreads();
            if constexpr (SM::NBUF == 1) {
                if (cg + 1 < ce) {
                    stage_chunk<DK, C, F32M, NW, NSL>(0, gblock(cg + 1), p.blk_bytes, sg, w, lane);
                    wait_vm_all();
                }
                __syncthreads();
            }
            continue;
        }
        const long t0 = bos + (long)(cg - cs) * C;
        const int n = (int)min((long)C, eos - t0);
        const uint32_t bo = (uint32_t)(((cg - cs) % SM::NBUF) * SM::BUF);
        auto frag = [&](size_t off, int tile) { return lds_ld<F>(bo + (uint32_t)off + (uint32_t)tile * 64 * FB + lfr); };
        auto scl = [&](int i) { return lds_ld<float>(bo + (uint32_t)L::SC_OFF + 4 * i); };

        // ---- S as B fragments over channels, one scale per column
        float iS[SPW];
        F sf[SPW][KSD];
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            float sS = 1.f;
            iS[j] = 1.f;
            if constexpr (!F32M) {
                float m = 0.f;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(S[j][cb][e]));
                m = colmax4(m);
                sS = pow2_scale_for(m);
                iS[j] = pow2_inv_scale_for(m);
            }
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const f32x4 bot = (2 * ks + 1 < CB) ? S[j][2 * ks + 1] : zero4();
                sf[j][ks] = to_frag<TM>(dtiles_to_frag(S[j][2 * ks], bot), sS);
            }
        }

        // ---- U = U~ - W S ;  O = (Gamma o Q) S
        f32x4 u[SPW][RB], ov[SPW][RB];
        {
            f32x4 wsum[SPW][RB], osum[SPW][RB];
#pragma unroll
            for (int j = 0; j < SPW; ++j)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) { wsum[j][rb] = zero4(); osum[j][rb] = zero4(); }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    const F wa = frag(L::W_OFF, rb * KSD + ks);
                    const F qa = frag(L::QG_OFF, rb * KSD + ks);
#pragma unroll
                    for (int j = 0; j < SPW; ++j) {
                        wsum[j][rb] = mma(wa, sf[j][ks], wsum[j][rb]);
                        osum[j][rb] = mma(qa, sf[j][ks], osum[j][rb]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                const uint32_t ub = bo + (uint32_t)L::BYTES + (uint32_t)((w * SPW + j) * L::USL);
                const float iUc = lds_ld<float>(bo + (uint32_t)L::SU_OFF + 4 * (uint32_t)col[j]);
                const float invWS = F32M ? 1.f : scl(SC_INV + SC_W) * iS[j];
                const float invQS = F32M ? 1.f : scl(SC_INV + SC_Q) * iS[j];
#pragma unroll
                for (int rb = 0; rb < RB; rb += UPR) {
                    typedef TM vu __attribute__((ext_vector_type(4 * UPR)));
                    const vu ut = lds_ld<vu>(ub + (uint32_t)L::u_off(rb, lane));
#pragma unroll
                    for (int r2 = 0; r2 < UPR; ++r2)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            u[j][rb + r2][e] = (float)ut[4 * r2 + e] * iUc - wsum[j][rb + r2][e] * invWS;
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) ov[j][rb] = osum[j][rb] * invQS;
            }
        }

        // ---- U as B fragments over tokens, one scale per column
        float iU[SPW];
        F uf[SPW][KSC];
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            float sU = 1.f;
            iU[j] = 1.f;
            if constexpr (!F32M) {
                float m = 0.f;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(u[j][rb][e]));
                m = colmax4(m);
                sU = pow2_scale_for(m);
                iU[j] = pow2_inv_scale_for(m);
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
                uf[j][ks] = to_frag<TM>(dtiles_to_frag(u[j][2 * ks], (2 * ks + 1 < RB) ? u[j][2 * ks + 1] : zero4()), sU);
        }

        // ---- O += P U: strictly lower part on MFMA, the diagonal in fp32.
        // Rows past the chunk end fall outside the store descriptor and are dropped.
        {
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(p.o + ((size_t)t0 * H + h) * DV, expired ? 0u : (uint32_t)(n - 1) * orow + (uint32_t)DV * 4);
            f32x4 pu[SPW][RB];
#pragma unroll
            for (int j = 0; j < SPW; ++j)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) pu[j][rb] = zero4();
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    if (ks > rb / 2) continue;
                    const F pa = frag(L::PS_OFF, rb * KSC + ks);
#pragma unroll
                    for (int j = 0; j < SPW; ++j) pu[j][rb] = mma(pa, uf[j][ks], pu[j][rb]);
                }
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                const float invPU = F32M ? 1.f : scl(SC_INV + SC_P) * iU[j];
                const uint32_t ovoff = (uint32_t)(4 * lg) * orow + (uint32_t)col[j] * 4;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const f32x4 pd4 = lds_ld<f32x4>(bo + (uint32_t)L::PD_OFF + 4 * (16 * rb + 4 * lg));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ovv = ov[j][rb][e] + pu[j][rb][e] * invPU + pd4[e] * u[j][rb][e];
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ovv), ro, ovoff, (16 * rb + e) * orow, 0);
                    }
                }
            }
        }

        // ---- S <- Diag(gamma_last) S + K_end^T U
        {
            float invKU[SPW];
#pragma unroll
            for (int j = 0; j < SPW; ++j) invKU[j] = F32M ? 1.f : scl(SC_INV + SC_K) * iU[j];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                f32x4 ku[SPW];
#pragma unroll
                for (int j = 0; j < SPW; ++j) ku[j] = zero4();
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    const F ka = frag(L::KE_OFF, cb * KSC + ks);
#pragma unroll
                    for (int j = 0; j < SPW; ++j) ku[j] = mma(ka, uf[j][ks], ku[j]);
                }
                const f32x4 g4 = lds_ld<f32x4>(bo + (uint32_t)L::GN_OFF + 4 * (16 * cb + 4 * lg));
#pragma unroll
                for (int j = 0; j < SPW; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[j][cb][e] = S[j][cb][e] * g4[e] + ku[j][e] * invKU[j];
            }
        }
        __syncthreads();
        if constexpr (SM::NBUF == 1) __syncthreads();
    }

    if (copier) {
        // keep the L2 touches alive: a store that no real input triggers
        // (H is positive for every launch)
        if (sink == 0x9e3779b9u && p.H < 0) p.o[0] = 0.f;
    }
    if (p.S_T && !copier) {
#pragma unroll
        for (int j = 0; j < SPW; ++j)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) p.S_T[sbase + (size_t)(16 * cb + 4 * lg + e) * DV + col[j]] = S[j][cb][e];
    }
}

// ------------------------------------------------------------------ state kernel, two waves per slice
//
// For 64-token chunks with bf16 inputs, each 16-column slice is shared by a
// pair of waves: wave hf of the pair keeps state rows (channels)
// 64 hf .. 64 hf + 63 (for dk = 128) and produces the outputs of token rows
// 32 hf .. 32 hf + 31. Per chunk the pair trades fp16 fragments through LDS:
// the halves of S (B operand over channels) before W S and (Gamma o Q) S, and
// the halves of U (B operand over tokens) before P U and K_end^T U. Each wave
// then reads half of the W, Gamma o Q and K_end^T fragments, which halves the
// LDS traffic per wave -- the limit of the one-wave form. Fragments keep one
// power-of-two scale per column and per half; partial products over the two
// halves go to separate accumulators and are combined in fp32.

template <int DK, int C, int NP>
struct PairSmem {
    using L = Lay<DK, C, false>;
    static constexpr int KH = L::KSD / 2;   // channel K steps per half
    static constexpr size_t UBYTES = ((size_t)NP * L::USL + 1023) / 1024 * 1024;
    static constexpr size_t BUF = L::BYTES + UBYTES;
    // per-slice exchange area
    static constexpr size_t X_S = 0;                                 // S halves [2][KH] fragment tiles
    static constexpr size_t X_U = X_S + (size_t)2 * KH * 1024;       // U halves [2] fragment tiles
    static constexpr size_t X_SI = X_U + 2 * 1024;                   // inverse S scales [2][16]
    static constexpr size_t X_UI = X_SI + 2 * 16 * 4;                // inverse U scales [2][16]
    static constexpr size_t X_F = X_UI + 2 * 16 * 4;                 // U-ready flags [2] (chunk index)
    static constexpr size_t XSL = X_F + 16;
    static constexpr size_t XCH = 2 * BUF;
    static constexpr size_t BYTES = XCH + (size_t)NP * XSL;
};

template <int DK, int C, int NP>
__global__ void __launch_bounds__(192 * NP) chunk_state_pair_kernel(StateParams p) {
    lds_poison((uint32_t)PairSmem<DK, C, NP>::BYTES);
    using L = Lay<DK, C, false>;
    using SM = PairSmem<DK, C, NP>;
    using F = f16x8;
    static_assert(C == 64 && DK >= 64, "pair form: 64-token chunks, dk >= 64");
    constexpr int KSD = L::KSD, KSC = L::KSC, KH = SM::KH;
    constexpr int CH = L::CB / 2;          // 16-row state tiles per wave
    constexpr int NCW = 2 * NP;            // compute waves

    const int item = walker_item(blockIdx.x, gridDim.x, p.NSG);
    const int sg = item % p.NSG;
    const int hs = item / p.NSG;
    const int H = p.H, DV = p.DV;
    const int h = hs % H, s = hs / H;
    const int lane = threadIdx.x % 64;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);   // wave index, uniform
    const bool copier = wv >= NCW;
    const int w = copier ? wv - NCW : wv;
    const int sl = w / 2, hf = w % 2;      // slice in the workgroup, half of the pair
    const int li = lane % 16, lg = lane / 16;
    const int col = 16 * (sg * NP + sl) + li;

    long bos, eos;
    int cs, ce;
    if (p.map.cu == nullptr) {
        bos = (long)s * p.map.T + (long)p.map.c0 * C;
        eos = (long)(s + 1) * p.map.T;
        cs = s * p.map.NC + p.map.c0;
        ce = s * p.map.NC + p.map.c1;
    } else {
        bos = p.map.cu[s];
        eos = p.map.cu[s + 1];
        cs = p.map.cstart[s];
        ce = p.map.cstart[s + 1];
    }

    const uint32_t xs = (uint32_t)(SM::XCH + (size_t)sl * SM::XSL);   // this slice's exchange area
    const uint32_t lfr = (uint32_t)lane * 16;
    int expired = 0;   // wave-uniform: set when a bounded wait ran out

    // own state rows 16 (CH hf + c) + 4 lg + e of column col
    f32x4 S[CH];
    const size_t sbase = ((size_t)s * H + h) * DK * DV;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[c][e] = (p.S0 && !copier) ? p.S0[sbase + (size_t)(16 * (CH * hf + c) + 4 * lg + e) * DV + col] : 0.f;

    // own half of S as fragments (channel steps KH hf + k), and its inverse scale
    F sfo[KH];
    float iSo = 1.f;
    auto make_s_frags = [&]() {
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(S[c][e]));
        m = colmax4(m);
        const float sc = pow2_scale_for(m);
        iSo = pow2_inv_scale_for(m);
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            sfo[k] = to_f16x8(dtiles_to_frag(S[2 * k], S[2 * k + 1]), sc);
            lds_st<F>(xs + (uint32_t)(SM::X_S + (size_t)(hf * KH + k) * 1024) + lfr, sfo[k]);
        }
        if (lg == 0) lds_st<float>(xs + (uint32_t)SM::X_SI + 4 * (16 * hf + li), iSo);
    };

    auto gblock = [&](int cg) { return p.ws + ((size_t)cg * H + h) * p.blk_bytes; };
    const uint32_t orow = (uint32_t)H * DV * 4;

    if (copier) {
        if (cs < ce) {
            stage_chunk<DK, C, false, NP, NP>(0, gblock(cs), p.blk_bytes, sg, w, lane);
            wait_vm_all();
        }
    } else {
        make_s_frags();
        if (lane == 0) lds_st<int>(xs + (uint32_t)SM::X_F + 4 * hf, -1);
    }
    __syncthreads();

    for (int cg = cs; cg < ce; ++cg) {
        if (copier) {
            // chunk cg+1 into the free buffer; the copy has the whole
            // iteration and must land before the barrier that ends it
            if (cg + 1 < ce)
                stage_chunk<DK, C, false, NP, NP>((uint32_t)(((cg + 1 - cs) % 2) * SM::BUF), gblock(cg + 1), p.blk_bytes,
                                                  sg, w, lane);
            wait_vm_all();
            __syncthreads();
            continue;
        }
        const long t0 = bos + (long)(cg - cs) * C;
        const int n = (int)min((long)C, eos - t0);
        const uint32_t bo = (uint32_t)(((cg - cs) % 2) * SM::BUF);
        auto frag = [&](size_t off, int tile) { return lds_ld<F>(bo + (uint32_t)off + (uint32_t)tile * 1024 + lfr); };
        auto scl = [&](int i) { return lds_ld<float>(bo + (uint32_t)L::SC_OFF + 4 * i); };
        const float iW = scl(SC_INV + SC_W), iQ = scl(SC_INV + SC_Q), iK = scl(SC_INV + SC_K), iP = scl(SC_INV + SC_P);

        // ---- the other half of S
        F sfx[KH];
#pragma unroll
        for (int k = 0; k < KH; ++k) sfx[k] = lds_ld<F>(xs + (uint32_t)(SM::X_S + (size_t)((1 - hf) * KH + k) * 1024) + lfr);
        const float iSx = lds_ld<float>(xs + (uint32_t)SM::X_SI + 4 * (16 * (1 - hf) + li));

        // ---- own token rows rb = 2 hf + r:  U = U~ - W S,  O = (Gamma o Q) S
        f32x4 u[2], ov[2];
        {
            const float iUc = lds_ld<float>(bo + (uint32_t)L::SU_OFF + 4 * (uint32_t)col);
            const F ut = lds_ld<F>(bo + (uint32_t)L::BYTES + (uint32_t)(sl * L::USL) + (uint32_t)L::u_off(2 * hf, lane));
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int rb = 2 * hf + r;
                f32x4 wo = zero4(), wx = zero4(), qo = zero4(), qx = zero4();
#pragma unroll
                for (int k = 0; k < KH; ++k) {
                    const int ko = hf * KH + k, kx = (1 - hf) * KH + k;
                    wo = mma(frag(L::W_OFF, rb * KSD + ko), sfo[k], wo);
                    wx = mma(frag(L::W_OFF, rb * KSD + kx), sfx[k], wx);
                    qo = mma(frag(L::QG_OFF, rb * KSD + ko), sfo[k], qo);
                    qx = mma(frag(L::QG_OFF, rb * KSD + kx), sfx[k], qx);
                }
                const float a1 = iW * iSo, a2 = iW * iSx, b1 = iQ * iSo, b2 = iQ * iSx;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u[r][e] = (float)ut[4 * r + e] * iUc - (wo[e] * a1 + wx[e] * a2);
                    ov[r][e] = qo[e] * b1 + qx[e] * b2;
                }
            }
        }

        // ---- own half of U (token step hf) as a fragment; trade halves
        F ufo;
        float iUo;
        {
            float m = 0.f;
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(u[r][e]));
            m = colmax4(m);
            const float sc = pow2_scale_for(m);
            iUo = pow2_inv_scale_for(m);
            ufo = to_f16x8(dtiles_to_frag(u[0], u[1]), sc);
            lds_st<F>(xs + (uint32_t)(SM::X_U + (size_t)hf * 1024) + lfr, ufo);
            if (lg == 0) lds_st<float>(xs + (uint32_t)SM::X_UI + 4 * (16 * hf + li), iUo);
        }
        // hand-off inside the pair: the LDS operations of one wave complete in
        // order, so the flag lands after the fragment; the wait is bounded
        // (both waves are resident, and the partner posts every chunk)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) lds_st<int>(xs + (uint32_t)SM::X_F + 4 * hf, cg);
        {
            extern __shared__ __align__(16) unsigned char smem[];
            typedef __attribute__((address_space(3))) const volatile int lds_flag_t;
            lds_flag_t* flag = (lds_flag_t*)(smem + xs + SM::X_F + 4 * (1 - hf));
            int spin = 0;
            for (; *flag != cg && spin < WAIT_POLLS; ++spin) __builtin_amdgcn_s_sleep(1);
            expired |= __builtin_amdgcn_readfirstlane(spin >= WAIT_POLLS ? 1 : 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const F ufx = lds_ld<F>(xs + (uint32_t)(SM::X_U + (size_t)(1 - hf) * 1024) + lfr);
        const float iUx = lds_ld<float>(xs + (uint32_t)SM::X_UI + 4 * (16 * (1 - hf) + li));

        // ---- O += P U for own rows (strictly lower part on MFMA, diagonal in
        // fp32); rows past the chunk end fall outside the store descriptor
        {
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(p.o + ((size_t)t0 * H + h) * DV, expired ? 0u : (uint32_t)(n - 1) * orow + (uint32_t)DV * 4);
            const uint32_t ovoff = (uint32_t)(4 * lg) * orow + (uint32_t)col * 4;
            const float po = iP * iUo, px = iP * iUx;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int rb = 2 * hf + r;
                // token step hf is this wave's own U half; step 0 for hf = 1 is the other's
                f32x4 pu_o = mma(frag(L::PS_OFF, rb * KSC + hf), ufo, zero4());
                f32x4 pu_x = zero4();
                if (hf == 1) pu_x = mma(frag(L::PS_OFF, rb * KSC + 0), ufx, pu_x);
                const f32x4 pd4 = lds_ld<f32x4>(bo + (uint32_t)L::PD_OFF + 4 * (16 * rb + 4 * lg));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ovv = ov[r][e] + pu_o[e] * po + pu_x[e] * px + pd4[e] * u[r][e];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ovv), ro, ovoff, (16 * rb + e) * orow, 0);
                }
            }
        }

        // ---- own state rows: S <- Diag(gamma_last) S + K_end^T U
        {
            const float ko = iK * iUo, kx = iK * iUx;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int cb = CH * hf + c;
                const f32x4 k_o = mma(frag(L::KE_OFF, cb * KSC + hf), ufo, zero4());
                const f32x4 k_x = mma(frag(L::KE_OFF, cb * KSC + (1 - hf)), ufx, zero4());
                const f32x4 g4 = lds_ld<f32x4>(bo + (uint32_t)L::GN_OFF + 4 * (16 * cb + 4 * lg));
#pragma unroll
                for (int e = 0; e < 4; ++e) S[c][e] = S[c][e] * g4[e] + (k_o[e] * ko + k_x[e] * kx);
            }
        }
        make_s_frags();
        __syncthreads();
    }

    if (!copier) raise_status(p.status, expired);
    if (!copier && p.S_T && !expired) {
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.S_T[sbase + (size_t)(16 * (CH * hf + c) + 4 * lg + e) * DV + col] = S[c][e];
    }
}

// ------------------------------------------------------------------ state kernel, four waves per slice
//
// dk = 128, 64-token chunks, bf16 inputs: each 16-column slice is shared by
// four waves. Wave q keeps state rows (channels) 32q .. 32q + 31 -- channel
// step q of the B operand over channels -- and produces token rows
// 16q .. 16q + 15. Per chunk the four waves trade, through LDS, their fp16
// fragment of S (before W S and (Gamma o Q) S) and their rows of U in fp32
// (before P U and K_end^T U; every wave then forms the same U fragments with
// the same scales). Each wave reads a quarter of the W, Gamma o Q and K_end^T
// fragments. Partial products over channel steps with different scales go to
// separate accumulators and are combined in fp32.

template <int NS>
struct QuadSmem {
    using L = Lay<128, 64, false>;
    static constexpr size_t UBYTES = ((size_t)NS * L::USL + 1023) / 1024 * 1024;
    static constexpr size_t BUF = L::BYTES + UBYTES;
    // per-slice exchange area
    static constexpr size_t X_S = 0;                     // S fragments [4 channel steps][64 lanes]
    static constexpr size_t X_U = X_S + 4 * 1024;        // U rows, fp32 [4 token blocks][64 lanes][4]
    static constexpr size_t X_SI = X_U + 4 * 1024;       // inverse S scales [4][16]
    static constexpr size_t X_F = X_SI + 4 * 16 * 4;     // U-posted flags [4] (chunk index)
    static constexpr size_t XSL = X_F + 16;
    static constexpr size_t XCH = 2 * BUF;
    static constexpr size_t BYTES = XCH + (size_t)NS * XSL;
};

template <int NS>
__device__ __forceinline__ void quad_walk(const StateParams& p, int item) {
    constexpr int DK = 128, C = 64;
    using L = Lay<DK, C, false>;
    using SM = QuadSmem<NS>;
    using F = f16x8;
    constexpr int KSD = L::KSD, KSC = L::KSC;   // 4 channel steps, 2 token steps
    constexpr int NCW = 4 * NS;                  // compute waves
    constexpr int NCP = 2 * NS;                  // copy waves

    const int sg = item % p.NSG;
    const int hs = item / p.NSG;
    const int H = p.H, DV = p.DV;
    const int h = hs % H, s = hs / H;
    const int lane = threadIdx.x % 64;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);   // wave index, uniform
    const bool copier = wv >= NCW;
    const int w = copier ? wv - NCW : wv;
    const int sl = w / 4, q = w % 4;       // slice in the workgroup, quarter of the slice
    const int li = lane % 16, lg = lane / 16;
    const int col = 16 * (sg * NS + sl) + li;

    long bos, eos;
    int cs, ce;
    if (p.map.cu == nullptr) {
        bos = (long)s * p.map.T + (long)p.map.c0 * C;
        eos = (long)(s + 1) * p.map.T;
        cs = s * p.map.NC + p.map.c0;
        ce = s * p.map.NC + p.map.c1;
    } else {
        bos = p.map.cu[s];
        eos = p.map.cu[s + 1];
        cs = p.map.cstart[s];
        ce = p.map.cstart[s + 1];
    }

    const uint32_t xs = (uint32_t)(SM::XCH + (size_t)sl * SM::XSL);   // this slice's exchange area
    const uint32_t lfr = (uint32_t)lane * 16;
    int expired = 0;   // wave-uniform: set when a bounded wait ran out

    // own state rows 16 (2q + c) + 4 lg + e of column col
    f32x4 S[2];
    const size_t sbase = ((size_t)s * H + h) * DK * DV;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[c][e] = (p.S0 && !copier) ? p.S0[sbase + (size_t)(16 * (2 * q + c) + 4 * lg + e) * DV + col] : 0.f;

    // own channel step of S as a fragment, its inverse scale, both posted
    F sfo;
    float iSo = 1.f;
    auto make_s_frag = [&]() {
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(S[c][e]));
        m = colmax4(m);
        const float sc = pow2_scale_for(m);
        iSo = pow2_inv_scale_for(m);
        sfo = to_f16x8(dtiles_to_frag(S[0], S[1]), sc);
        lds_st<F>(xs + (uint32_t)(SM::X_S + (size_t)q * 1024) + lfr, sfo);
        if (lg == 0) lds_st<float>(xs + (uint32_t)SM::X_SI + 4 * (16 * q + li), iSo);
    };

    auto gblock = [&](int cg) { return p.ws + ((size_t)cg * H + h) * p.blk_bytes; };
    const uint32_t orow = (uint32_t)H * DV * 4;

    uint32_t sink = 0;
    if (copier) {
        if (cs < ce) {
            stage_chunk<DK, C, false, NCP, NS>(0, gblock(cs), p.blk_bytes, sg, w, lane, sg);
            wait_vm_all();
        }
    } else {
        make_s_frag();
        if (lane == 0) lds_st<int>(xs + (uint32_t)SM::X_F + 4 * q, -1);
    }
    __syncthreads();

    for (int cg = cs; cg < ce; ++cg) {
        if (copier) {
            // chunk cg+1 into the free buffer; the copy has the whole
            // iteration and must land before the barrier that ends it. The
            // workgroups of one (sequence, head) start at different pieces,
            // so that one of them misses L2 on each line and the others hit.
            if (cg + 1 < ce)
                stage_chunk<DK, C, false, NCP, NS>((uint32_t)(((cg + 1 - cs) % 2) * SM::BUF), gblock(cg + 1), p.blk_bytes,
                                                   sg, w, lane, sg);
            // Pull this workgroup's share (one part in NSG) of chunk cg+2's
            // shared operands into L2 with one 4-byte load per 128-byte line:
            // the misses are spread over the workgroups of the (sequence,
            // head), and every workgroup's copy of chunk cg+2 then hits L2.
            if (cg + 2 < ce) {
                constexpr int L0 = (int)(L::BYTES / 128);
                const int per = (L0 + p.NSG - 1) / p.NSG;
                const int line = sg * per + w * 64 + lane;
                const bool mine = w * 64 + lane < per && line < L0;
                const __amdgpu_buffer_rsrc_t rt = make_rsrc(gblock(cg + 2), (uint32_t)L::BYTES);
                // other lanes point past the descriptor: no access, value 0
                sink ^= __builtin_amdgcn_raw_buffer_load_b32(rt, mine ? line * 128 : (int)L::BYTES, 0, 0);
                wait_vm_upto<1>();
            } else {
                wait_vm_all();
            }
            __syncthreads();
            continue;
        }
        const long t0 = bos + (long)(cg - cs) * C;
        const int n = (int)min((long)C, eos - t0);
        const uint32_t bo = (uint32_t)(((cg - cs) % 2) * SM::BUF);
        auto frag = [&](size_t off, int tile) { return lds_ld<F>(bo + (uint32_t)off + (uint32_t)tile * 1024 + lfr); };
        auto scl = [&](int i) { return lds_ld<float>(bo + (uint32_t)L::SC_OFF + 4 * i); };
        const float iW = scl(SC_INV + SC_W), iQ = scl(SC_INV + SC_Q), iK = scl(SC_INV + SC_K), iP = scl(SC_INV + SC_P);

        // ---- S over all channel steps (the other three from LDS)
        F sf[KSD];
        float iS[KSD];
#pragma unroll
        for (int k = 0; k < KSD; ++k) {
            if (k == q) continue;
            sf[k] = lds_ld<F>(xs + (uint32_t)(SM::X_S + (size_t)k * 1024) + lfr);
            iS[k] = lds_ld<float>(xs + (uint32_t)SM::X_SI + 4 * (16 * k + li));
        }
        // wave-uniform q: place the own step by selection (no dynamic register index)
#pragma unroll
        for (int k = 0; k < KSD; ++k)
            if (k == q) { sf[k] = sfo; iS[k] = iSo; }

        // ---- own token rows rb = q:  u = U~ - W S,  O = (Gamma o Q) S
        f32x4 uq, ov = zero4();
        {
            f32x4 ws = zero4();
#pragma unroll
            for (int k = 0; k < KSD; ++k) {
                const f32x4 wk = mma(frag(L::W_OFF, q * KSD + k), sf[k], zero4());
                const f32x4 qk = mma(frag(L::QG_OFF, q * KSD + k), sf[k], zero4());
                const float a = iW * iS[k], b = iQ * iS[k];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ws[e] += wk[e] * a;
                    ov[e] += qk[e] * b;
                }
            }
            typedef _Float16 h4 __attribute__((ext_vector_type(4)));
            const float iUc = lds_ld<float>(bo + (uint32_t)L::SU_OFF + 4 * (uint32_t)col);
            const h4 ut = lds_ld<h4>(bo + (uint32_t)L::BYTES + (uint32_t)(sl * L::USL) + (uint32_t)L::u_off(q, lane));
#pragma unroll
            for (int e = 0; e < 4; ++e) uq[e] = (float)ut[e] * iUc - ws[e];
        }
        // post own rows of U; the LDS operations of one wave complete in order,
        // so the flag lands after the rows; waits are bounded (all four waves
        // are resident and post every chunk)
        lds_st<f32x4>(xs + (uint32_t)(SM::X_U + (size_t)q * 1024) + lfr, uq);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) lds_st<int>(xs + (uint32_t)SM::X_F + 4 * q, cg);
        {
            extern __shared__ __align__(16) unsigned char smem[];
            typedef __attribute__((address_space(3))) const volatile int lds_flag_t;
            lds_flag_t* flags = (lds_flag_t*)(smem + xs + SM::X_F);
            int spin = 0;
            for (; spin < WAIT_POLLS; ++spin) {
                if (flags[0] == cg && flags[1] == cg && flags[2] == cg && flags[3] == cg) break;
                __builtin_amdgcn_s_sleep(1);
            }
            expired |= __builtin_amdgcn_readfirstlane(spin >= WAIT_POLLS ? 1 : 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        f32x4 u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = r == q ? uq : lds_ld<f32x4>(xs + (uint32_t)(SM::X_U + (size_t)r * 1024) + lfr);

        // ---- U over the two token steps, one scale per (step, column); every
        // wave of the slice forms the same fragments
        F uf[KSC];
        float iU[KSC];
#pragma unroll
        for (int t = 0; t < KSC; ++t) {
            float m = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(u[2 * t][e]), fabsf(u[2 * t + 1][e])));
            m = colmax4(m);
            iU[t] = pow2_inv_scale_for(m);
            uf[t] = to_f16x8(dtiles_to_frag(u[2 * t], u[2 * t + 1]), pow2_scale_for(m));
        }

        // ---- O += P U for token rows rb = q (strictly lower part on MFMA,
        // diagonal in fp32); rows past the chunk end fall outside the store
        // descriptor
        {
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(p.o + ((size_t)t0 * H + h) * DV, expired ? 0u : (uint32_t)(n - 1) * orow + (uint32_t)DV * 4);
            const uint32_t ovoff = (uint32_t)(4 * lg) * orow + (uint32_t)col * 4;
            f32x4 o4 = ov;
#pragma unroll
            for (int t = 0; t < KSC; ++t) {
                if (t > q / 2) continue;
                const f32x4 pu = mma(frag(L::PS_OFF, q * KSC + t), uf[t], zero4());
                const float pc = iP * iU[t];
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] += pu[e] * pc;
            }
            const f32x4 pd4 = lds_ld<f32x4>(bo + (uint32_t)L::PD_OFF + 4 * (16 * q + 4 * lg));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ovv = o4[e] + pd4[e] * uq[e];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ovv), ro, ovoff, (16 * q + e) * orow, 0);
            }
        }

        // ---- own state rows: S <- Diag(gamma_last) S + K_end^T U
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int cb = 2 * q + c;
            const f32x4 k0 = mma(frag(L::KE_OFF, cb * KSC + 0), uf[0], zero4());
            const f32x4 k1 = mma(frag(L::KE_OFF, cb * KSC + 1), uf[1], zero4());
            const float c0 = iK * iU[0], c1 = iK * iU[1];
            const f32x4 g4 = lds_ld<f32x4>(bo + (uint32_t)L::GN_OFF + 4 * (16 * cb + 4 * lg));
#pragma unroll
            for (int e = 0; e < 4; ++e) S[c][e] = S[c][e] * g4[e] + (k0[e] * c0 + k1[e] * c1);
        }
        make_s_frag();
        __syncthreads();
    }

    if (copier) {
        // keep the L2 touches alive: a store that no real input triggers
        // (H is positive for every launch)
        if (sink == 0x9e3779b9u && p.H < 0) p.o[0] = 0.f;
    } else {
        raise_status(p.status, expired);
    }
    if (!copier && p.S_T && !expired) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.S_T[sbase + (size_t)(16 * (2 * q + c) + 4 * lg + e) * DV + col] = S[c][e];
    }
}

template <int NS>
__global__ void __launch_bounds__(384 * NS) chunk_state_quad_kernel(StateParams p) {
    lds_poison((uint32_t)QuadSmem<NS>::BYTES);
    quad_walk<NS>(p, walker_item(blockIdx.x, gridDim.x, p.NSG));
}

// ------------------------------------------------------------------ slice walker

// One 16-column value slice of one (sequence, head) on one workgroup of four
// waves, with the chunk operands loaded straight into registers one chunk
// ahead (no LDS staging and no copy waves). Wave q keeps state rows 32q ..
// 32q + 31 and produces token rows 16q .. 16q + 15, and needs only its own
// quarter of W, Gamma o Q, K_end^T and P; the four waves trade their fp16
// S fragment and their fp32 U rows through LDS, as in the two-slice walker,
// whose arithmetic this repeats operation for operation. The eight slices of
// a (sequence, head) are consecutive workgroups (one XCD), so a block fetched
// from memory by one of them is served to the others by L2.
struct SliceLds {
    static constexpr size_t X_S = 0;                     // S fragments [4 channel steps][64 lanes]
    static constexpr size_t X_U = X_S + 4 * 1024;        // U rows, fp32 [4 token blocks][64 lanes][4]
    static constexpr size_t X_SI = X_U + 4 * 1024;       // inverse S scales [4][16]
    static constexpr size_t X_F = X_SI + 4 * 16 * 4;     // U-posted flags [4] (chunk index)
    static constexpr size_t BYTES = (X_F + 16 + 1023) / 1024 * 1024;
};

// A 16x32 fp16 fragment of a block: tile t, this lane's 16 bytes.
__device__ __forceinline__ f16x8 ld_frag(__amdgpu_buffer_rsrc_t r, uint32_t off, int tile, int lane) {
    return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + (uint32_t)tile * 1024 + (uint32_t)lane * 16), 0, 0));
}
__device__ __forceinline__ f32x4 ld_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float ld_f1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// The operands of one chunk that wave q reads, in the groups in which they
// are reloaded for the next chunk: each group right after its last use in
// this chunk, so that the loads spread over the chunk instead of stalling the
// wave's instruction stream in one burst.
struct SliceOps {
    f16x8 w[4], qg[4];            // group 0: W, Gamma o Q (first used)
    f32x4 isc;                    //          inverse scales of W, Gamma o Q, K_end^T, P
    float iUc;                    //          inverse scale of this U~ column
    _Float16 __attribute__((ext_vector_type(4))) ut;   // U~ rows
    f16x8 ps[2];                  // group 1: strictly lower P
    f32x4 pd;                     //          P diagonal rows
    f16x8 ke[2][2];               // group 2: K_end^T
    f32x4 g[2];                   //          gamma_last rows
};

struct SliceSrc {
    __amdgpu_buffer_rsrc_t r;
    int q, lane, col, slice;
};

__device__ __forceinline__ void slice_load0(SliceOps& o, const SliceSrc& x) {
    using L = Lay<128, 64, false>;
    constexpr int KSD = L::KSD;
#pragma unroll
    for (int k = 0; k < KSD; ++k) o.w[k] = ld_frag(x.r, (uint32_t)L::W_OFF, x.q * KSD + k, x.lane);
#pragma unroll
    for (int k = 0; k < KSD; ++k) o.qg[k] = ld_frag(x.r, (uint32_t)L::QG_OFF, x.q * KSD + k, x.lane);
    o.isc = ld_f4(x.r, (uint32_t)L::SC_OFF + 4 * SC_INV);
    o.iUc = ld_f1(x.r, (uint32_t)L::SU_OFF + 4 * (uint32_t)x.col);
    const uint32_t uo = (uint32_t)(L::BYTES + (size_t)x.slice * L::USL + L::u_off(x.q, x.lane));
    o.ut = __builtin_bit_cast(decltype(o.ut), __builtin_amdgcn_raw_buffer_load_b64(x.r, (int)uo, 0, 0));
}

__device__ __forceinline__ void slice_load1(SliceOps& o, const SliceSrc& x) {
    using L = Lay<128, 64, false>;
    constexpr int KSC = L::KSC;
#pragma unroll
    for (int t = 0; t < KSC; ++t)
        if (t <= x.q / 2) o.ps[t] = ld_frag(x.r, (uint32_t)L::PS_OFF, x.q * KSC + t, x.lane);
    o.pd = ld_f4(x.r, (uint32_t)L::PD_OFF + 4 * (16 * x.q + 4 * (x.lane / 16)));
}

__device__ __forceinline__ void slice_load2(SliceOps& o, const SliceSrc& x) {
    using L = Lay<128, 64, false>;
    constexpr int KSC = L::KSC;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int t = 0; t < KSC; ++t) o.ke[c][t] = ld_frag(x.r, (uint32_t)L::KE_OFF, (2 * x.q + c) * KSC + t, x.lane);
        o.g[c] = ld_f4(x.r, (uint32_t)L::GN_OFF + 4 * (16 * (2 * x.q + c) + 4 * (x.lane / 16)));
    }
}

__device__ __forceinline__ void slice_walk(const StateParams& p, int item) {
    constexpr int DK = 128, C = 64;
    using L = Lay<DK, C, false>;
    using SM = SliceLds;
    using F = f16x8;
    constexpr int KSD = L::KSD, KSC = L::KSC;   // 4 channel steps, 2 token steps

    const int nsl = p.NSG;                       // slices per (sequence, head)
    const int sl = item % nsl;
    const int hs = item / nsl;
    const int H = p.H, DV = p.DV;
    const int h = hs % H, s = hs / H;
    const int lane = threadIdx.x % 64;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);   // quarter, uniform
    const int li = lane % 16, lg = lane / 16;
    const int col = 16 * sl + li;

    long bos, eos;
    int cs, ce;
    if (p.map.cu == nullptr) {
        bos = (long)s * p.map.T + (long)p.map.c0 * C;
        eos = (long)(s + 1) * p.map.T;
        cs = s * p.map.NC + p.map.c0;
        ce = s * p.map.NC + p.map.c1;
    } else {
        bos = p.map.cu[s];
        eos = p.map.cu[s + 1];
        cs = p.map.cstart[s];
        ce = p.map.cstart[s + 1];
    }
    const uint32_t lfr = (uint32_t)lane * 16;
    int expired = 0;   // wave-uniform: set when a bounded wait ran out

    // own state rows 16 (2q + c) + 4 lg + e of column col
    f32x4 S[2];
    const size_t sbase = ((size_t)s * H + h) * DK * DV;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[c][e] = p.S0 ? p.S0[sbase + (size_t)(16 * (2 * q + c) + 4 * lg + e) * DV + col] : 0.f;

    // own channel step of S as an fp16 fragment and its inverse column
    // scales, posted for all four waves
    auto make_s_frag = [&]() {
        const float m = colmax4(absmax8(S[0], S[1]));
        const float iSo = pow2_inv_scale_for(m);
        const F sfo = to_f16x8(dtiles_to_frag(S[0], S[1]), pow2_scale_for(m));
        lds_st<F>((uint32_t)(SM::X_S + (size_t)q * 1024) + lfr, sfo);
        if (lg == 0) lds_st<float>((uint32_t)SM::X_SI + 4 * (16 * q + li), iSo);
    };

    auto gblock = [&](int cg) { return p.ws + ((size_t)cg * H + h) * p.blk_bytes; };
    const uint32_t orow = (uint32_t)H * DV * 4;

    auto src = [&](int cg) { return SliceSrc{make_rsrc(gblock(cg), (uint32_t)p.blk_bytes), q, lane, col, sl}; };
    SliceOps op;
    if (cs < ce) {
        const SliceSrc x = src(cs);
        slice_load0(op, x);
        slice_load1(op, x);
        slice_load2(op, x);
    }
    make_s_frag();
    if (lane == 0) lds_st<int>((uint32_t)SM::X_F + 4 * q, -1);
    __syncthreads();

    uint32_t sink = 0;
    // first touch of chunk cg+2: this slice's share of the shared operands'
    // lines (so that the slices of the (sequence, head) find them in L2) and
    // its own U~ lines; the lane's line offset within a block is fixed
    const bool toucher = q * 64 < (int)((L::BYTES / 128 + nsl - 1) / nsl + L::USL / 128);   // wave has lines
    int toff = (int)p.blk_bytes;   // past the descriptor: no access, value 0
    {
        constexpr int L0 = (int)(L::BYTES / 128), LU = (int)(L::USL / 128);
        const int per = (L0 + nsl - 1) / nsl;
        const int i = q * 64 + lane;
        if (i < per && sl * per + i < L0) toff = (sl * per + i) * 128;
        else if (i >= per && i < per + LU) toff = (int)(L::BYTES + (size_t)sl * L::USL) + (i - per) * 128;
    }
    for (int cg = cs; cg < ce; ++cg) {
        const long t0 = bos + (long)(cg - cs) * C;
        const int n = (int)min((long)C, eos - t0);
        // Issued before the loads below and consumed at the end of the
        // iteration: waiting for it then does not wait for them.
        uint32_t tch = 0;
        if (toucher) {
            const int off = cg + 2 < ce ? toff : (int)p.blk_bytes;
            const __amdgpu_buffer_rsrc_t rt = make_rsrc(gblock(cg + 2 < ce ? cg + 2 : cg), (uint32_t)p.blk_bytes);
            tch = __builtin_amdgcn_raw_buffer_load_b32(rt, off, 0, 0);
        }
        // operands of the next chunk (the last chunk reloads its own: a valid
        // block, never used)
        const int cn = cg + 1 < ce ? cg + 1 : cg;
        const SliceSrc xn = src(cn);
        const float iW = op.isc[SC_W], iQ = op.isc[SC_Q], iK = op.isc[SC_K], iP = op.isc[SC_P];

        // ---- S over all channel steps, read back from LDS (this wave's own
        // step too: one more read in parallel costs less than selecting it)
        F sf[KSD];
        float iS[KSD];
#pragma unroll
        for (int k = 0; k < KSD; ++k) {
            sf[k] = lds_ld<F>((uint32_t)(SM::X_S + (size_t)k * 1024) + lfr);
            iS[k] = lds_ld<float>((uint32_t)SM::X_SI + 4 * (16 * k + li));
        }

        // ---- own token rows rb = q:  u = U~ - W S,  O = (Gamma o Q) S
        f32x4 uq, ov = zero4();
        {
            f32x4 ws = zero4();
#pragma unroll
            for (int k = 0; k < KSD; ++k) {
                const f32x4 wk = mma(op.w[k], sf[k], zero4());
                const f32x4 qk = mma(op.qg[k], sf[k], zero4());
                const float a = iW * iS[k], b = iQ * iS[k];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ws[e] += wk[e] * a;
                    ov[e] += qk[e] * b;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) uq[e] = (float)op.ut[e] * op.iUc - ws[e];
        }
        lds_st<f32x4>((uint32_t)(SM::X_U + (size_t)q * 1024) + lfr, uq);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) lds_st<int>((uint32_t)SM::X_F + 4 * q, cg);
        // issuing loads stalls this wave for a while: do it only once U is
        // posted, while the other waves post theirs
        slice_load0(op, xn);
        {
            extern __shared__ __align__(16) unsigned char smem[];
            typedef __attribute__((address_space(3))) const volatile int lds_flag_t;
            lds_flag_t* fl = (lds_flag_t*)(smem + SM::X_F);
            // all four flags read before one wait (not one round trip each);
            // no sleep: the waits are short
            int spin = 0;
            for (; spin < WAIT_POLLS; ++spin) {
                const int f0 = fl[0], f1 = fl[1], f2 = fl[2], f3 = fl[3];
                if ((f0 == cg) & (f1 == cg) & (f2 == cg) & (f3 == cg)) break;
            }
            expired |= __builtin_amdgcn_readfirstlane(spin >= WAIT_POLLS ? 1 : 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        f32x4 u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = lds_ld<f32x4>((uint32_t)(SM::X_U + (size_t)r * 1024) + lfr);

        // ---- U over the two token steps, one scale per (step, column)
        F uf[KSC];
        float iU[KSC];
#pragma unroll
        for (int t = 0; t < KSC; ++t) {
            const float m = colmax4(absmax8(u[2 * t], u[2 * t + 1]));
            iU[t] = pow2_inv_scale_for(m);
            uf[t] = to_f16x8(dtiles_to_frag(u[2 * t], u[2 * t + 1]), pow2_scale_for(m));
        }

        // ---- O += P U for token rows rb = q, diagonal in fp32
        {
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(p.o + ((size_t)t0 * H + h) * DV, expired ? 0u : (uint32_t)(n - 1) * orow + (uint32_t)DV * 4);
            const uint32_t ovoff = (uint32_t)(4 * lg) * orow + (uint32_t)col * 4;
            f32x4 o4 = ov;
#pragma unroll
            for (int t = 0; t < KSC; ++t) {
                if (t > q / 2) continue;
                const f32x4 pu = mma(op.ps[t], uf[t], zero4());
                const float pc = iP * iU[t];
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] += pu[e] * pc;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ovv = o4[e] + op.pd[e] * uq[e];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ovv), ro, ovoff, (16 * q + e) * orow, 0);
            }
        }

        // ---- own state rows: S <- Diag(gamma_last) S + K_end^T U
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const f32x4 k0 = mma(op.ke[c][0], uf[0], zero4());
            const f32x4 k1 = mma(op.ke[c][1], uf[1], zero4());
            const float c0 = iK * iU[0], c1 = iK * iU[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) S[c][e] = S[c][e] * op.g[c][e] + (k0[e] * c0 + k1[e] * c1);
        }
        make_s_frag();
        // the rest of the next chunk's operands, once this wave's S is posted
        slice_load1(op, xn);
        slice_load2(op, xn);
        sink ^= tch;
        __syncthreads();
    }
    // keep the L2 touches alive: a store that no real input triggers
    if (sink == 0x9e3779b9u && p.H < 0) p.o[0] = 0.f;
    raise_status(p.status, expired);
    if (p.S_T && !expired) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.S_T[sbase + (size_t)(16 * (2 * q + c) + 4 * lg + e) * DV + col] = S[c][e];
    }
}

__global__ void __launch_bounds__(256) chunk_state_slice_kernel(StateParams p) {
    lds_poison((uint32_t)SliceLds::BYTES);
    slice_walk(p, walker_item(blockIdx.x, gridDim.x, p.NSG));
}

// ------------------------------------------------------------------ host side

template <int DK, int C>
static size_t block_bytes_t(int dv, bool bf16) {
    return bf16 ? Lay<DK, C, false>::BYTES + (size_t)(dv / 16) * Lay<DK, C, false>::USL
                : Lay<DK, C, true>::BYTES + (size_t)(dv / 16) * Lay<DK, C, true>::USL;
}

template <int DK>
static size_t block_bytes_c(int dv, int chunk, bool bf16) {
    switch (chunk) {
        case 16: return block_bytes_t<DK, 16>(dv, bf16);
        case 32: return block_bytes_t<DK, 32>(dv, bf16);
        default: return block_bytes_t<DK, 64>(dv, bf16);
    }
}

size_t chunk_block_bytes(int dk, int dv, int chunk, bool bf16) {
    switch (dk) {
        case 16: return block_bytes_c<16>(dv, chunk, bf16);
        case 32: return block_bytes_c<32>(dv, chunk, bf16);
        case 64: return block_bytes_c<64>(dv, chunk, bf16);
        default: return block_bytes_c<128>(dv, chunk, bf16);
    }
}

long chunk_count_bound(int B, int T, int chunk, bool varlen, int N) {
    if (!varlen) return (long)B * ((T + chunk - 1) / chunk);
    return (long)(T + chunk - 1) / chunk + N;
}

static size_t index_bytes(bool varlen, int N) { return varlen ? ((size_t)(N + 1) * 4 + 255) / 256 * 256 : 0; }

// Workspace: a 256-byte header whose first word is the call's status, the
// chunk index of packed sequences, then one block per (chunk, head).
constexpr size_t STATUS_BYTES = 256;

size_t chunk_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, bool varlen, int N, bool bf16) {
    return STATUS_BYTES + index_bytes(varlen, N) +
           (size_t)chunk_count_bound(B, T, chunk, varlen, N) * H * chunk_block_bytes(dk, dv, chunk, bf16);
}

__global__ void __launch_bounds__(64) status_clear_kernel(unsigned* status) {
    lds_poison(0);
    if (threadIdx.x == 0) *status = 0u;
}

// Compute units of the current device, queried on every call (a device
// attribute read; no state is kept between calls).
static int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

template <class K>
static hipError_t allow_lds(K kern, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <class TIn, int DK, int C, bool SG, bool EW>
static hipError_t launch_prep_t(const ChunkArgs& a, const ChunkMap& map, unsigned char* blocks, long nchunks) {
    constexpr bool F32M = std::is_same<TIn, float>::value;
    using SM = PrepLds<TIn, DK, C, F32M, EW>;
    static_assert(SM::BYTES <= 160 * 1024, "prep LDS");
    auto kern = chunk_prep_kernel<TIn, DK, C, SG, F32M, EW>;
    hipError_t e = allow_lds(kern, SM::BYTES);
    if (e != hipSuccess) return e;
    PrepParams pp{a.q, a.k, a.v, a.gate, a.beta, a.erase, a.write, (unsigned*)a.workspace, blocks,
                  chunk_block_bytes(DK, a.dv, C, !F32M), map, a.H, a.dv};
    const long grid = nchunks * a.H;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), SM::BYTES, a.stream, pp);
    return hipGetLastError();
}

template <class TIn, int DK, int C>
static hipError_t launch_prep(const ChunkArgs& a, const ChunkMap& map, unsigned char* blocks, long nchunks) {
    if (a.erase) {
        return a.scalar_gate ? launch_prep_t<TIn, DK, C, true, true>(a, map, blocks, nchunks)
                             : launch_prep_t<TIn, DK, C, false, true>(a, map, blocks, nchunks);
    }
    return a.scalar_gate ? launch_prep_t<TIn, DK, C, true, false>(a, map, blocks, nchunks)
                         : launch_prep_t<TIn, DK, C, false, false>(a, map, blocks, nchunks);
}

template <class TIn, int DK, int C, int NW, int SPW>
static hipError_t launch_state_w(const ChunkArgs& a, const ChunkMap& map, const unsigned char* blocks) {
    constexpr bool F32M = std::is_same<TIn, float>::value;
    using SM = StateSmem<DK, C, F32M, NW, SPW>;
    static_assert(SM::BYTES <= 160 * 1024, "state LDS");
    auto kern = chunk_state_kernel<DK, C, F32M, NW, SPW>;
    hipError_t e = allow_lds(kern, SM::BYTES);
    if (e != hipSuccess) return e;
    const int nsg = a.dv / 16 / SM::NSL;
    StateParams sp{a.S0, a.o, a.S_T, blocks, chunk_block_bytes(DK, a.dv, C, !F32M), map, a.H, a.dv, nsg,
                   (unsigned*)a.workspace};
    const long grid = (long)nsg * a.H * a.N;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(128 * NW), SM::BYTES, a.stream, sp);
    return hipGetLastError();
}

template <int DK, int C, int NP>
static hipError_t launch_state_pair(const ChunkArgs& a, const ChunkMap& map, const unsigned char* blocks) {
    using SM = PairSmem<DK, C, NP>;
    static_assert(SM::BYTES <= 160 * 1024, "pair state LDS");
    auto kern = chunk_state_pair_kernel<DK, C, NP>;
    hipError_t e = allow_lds(kern, SM::BYTES);
    if (e != hipSuccess) return e;
    const int nsg = a.dv / 16 / NP;
    StateParams sp{a.S0, a.o, a.S_T, blocks, chunk_block_bytes(DK, a.dv, C, true), map, a.H, a.dv, nsg,
                   (unsigned*)a.workspace};
    const long grid = (long)nsg * a.H * a.N;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(192 * NP), SM::BYTES, a.stream, sp);
    return hipGetLastError();
}

template <int NS>
static hipError_t launch_state_quad(const ChunkArgs& a, const ChunkMap& map, const unsigned char* blocks) {
    using SM = QuadSmem<NS>;
    static_assert(SM::BYTES <= 160 * 1024, "quad state LDS");
    auto kern = chunk_state_quad_kernel<NS>;
    hipError_t e = allow_lds(kern, SM::BYTES);
    if (e != hipSuccess) return e;
    const int nsg = a.dv / 16 / NS;
    StateParams sp{a.S0, a.o, a.S_T, blocks, chunk_block_bytes(128, a.dv, 64, true), map, a.H, a.dv, nsg,
                   (unsigned*)a.workspace};
    const long grid = (long)nsg * a.H * a.N;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(384 * NS), SM::BYTES, a.stream, sp);
    return hipGetLastError();
}

static hipError_t launch_state_slice(const ChunkArgs& a, const ChunkMap& map, const unsigned char* blocks) {
    const int nsl = a.dv / 16;
    StateParams sp{a.S0, a.o, a.S_T, blocks, chunk_block_bytes(128, a.dv, 64, true), map, a.H, a.dv, nsl,
                   (unsigned*)a.workspace};
    const long grid = (long)nsl * a.H * a.N;
    hipLaunchKernelGGL(chunk_state_slice_kernel, dim3((unsigned)grid), dim3(256), SliceLds::BYTES, a.stream, sp);
    return hipGetLastError();
}

// bf16 inputs, 64-token chunks: dk = 128 takes four waves per slice (two
// slices per workgroup), dk = 64 two waves per slice (four slices per
// workgroup). Otherwise one wave per slice: four compute waves of one
// slice each when the value width allows (more waves in flight shorten the
// sequential chunk loop more than sharing fragment reads between slices of
// one wave does).
template <class TIn, int DK, int C>
static hipError_t launch_state_t(const ChunkArgs& a, const ChunkMap& map, const unsigned char* blocks) {
    if constexpr (std::is_same<TIn, uint16_t>::value && C == 64 && DK == 128) {
        // one-slice walkers while they fit one per CU (measured faster
        // there); two-slice walkers when slices outnumber the CUs
        const long slices = (long)a.N * a.H * (a.dv / 16);
        if (slices <= device_cus()) return launch_state_slice(a, map, blocks);
        if (a.dv >= 32) return launch_state_quad<2>(a, map, blocks);
        return launch_state_quad<1>(a, map, blocks);
    }
    if constexpr (std::is_same<TIn, uint16_t>::value && C == 64 && DK >= 64) {
        if (a.dv >= 64) return launch_state_pair<DK, C, 4>(a, map, blocks);
        if (a.dv >= 32) return launch_state_pair<DK, C, 2>(a, map, blocks);
        return launch_state_pair<DK, C, 1>(a, map, blocks);
    }
    if (a.dv >= 64) return launch_state_w<TIn, DK, C, 4, 1>(a, map, blocks);
    if (a.dv >= 32) return launch_state_w<TIn, DK, C, 2, 1>(a, map, blocks);
    return launch_state_w<TIn, DK, C, 1, 1>(a, map, blocks);
}

template <class TIn, int DK, int C>
static hipError_t launch_pair(const ChunkArgs& a) {
    const bool varlen = a.cu_seqlens != nullptr;
    unsigned char* ws = (unsigned char*)a.workspace;
    const size_t ib = index_bytes(varlen, a.N);
    const int NC = (a.T + C - 1) / C;
    int32_t* cidx = (int32_t*)(ws + STATUS_BYTES);
    ChunkMap map{a.cu_seqlens, varlen ? cidx : nullptr, a.T, a.N, NC, 0, NC};
    unsigned char* blocks = ws + STATUS_BYTES + ib;
    const long nch = chunk_count_bound(a.B, a.T, C, varlen, a.N);
    if (a.stages & 1) {
        if (varlen) {
            hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens, cidx, a.N, C);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        // the prep's first workgroup clears the status word; without chunks a kernel of its own does
        hipError_t e;
        if (nch > 0) {
            e = launch_prep<TIn, DK, C>(a, map, blocks, nch);
        } else {
            hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, a.stream, (unsigned*)a.workspace);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    if (a.stages & 2) return launch_state_t<TIn, DK, C>(a, map, blocks);
    return hipSuccess;
}

template <class TIn, int DK>
static hipError_t launch_chunk_c(const ChunkArgs& a) {
    switch (a.chunk) {
        case 16: return launch_pair<TIn, DK, 16>(a);
        case 32: return launch_pair<TIn, DK, 32>(a);
        default: return launch_pair<TIn, DK, 64>(a);
    }
}

template <class TIn>
static hipError_t launch_chunk_dk(const ChunkArgs& a) {
    switch (a.dk) {
        case 16: return launch_chunk_c<TIn, 16>(a);
        case 32: return launch_chunk_c<TIn, 32>(a);
        case 64: return launch_chunk_c<TIn, 64>(a);
        default: return launch_chunk_c<TIn, 128>(a);
    }
}

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
    return a.bf16 ? launch_chunk_dk<uint16_t>(a) : launch_chunk_dk<float>(a);
}

}  // namespace kda
