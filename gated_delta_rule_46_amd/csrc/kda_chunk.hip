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
//    products, gated Gram matrices, the triangular inverse, and the operands
//    W, Gamma o Q, K_end^T, T, P written to a workspace as MFMA fragments.
//  * state -- one wavefront per 16 value columns of one (sequence, head),
//    up to four per workgroup. Walks the chunks of its sequence in order with its
//    slice of S in fp32 MFMA accumulator registers, while copy wavefronts of
//    the same workgroup stream the next chunk's operands into the other half
//    of a double-buffered LDS area.
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
// data, chosen so the largest entry lies in [0.5, 1)), products accumulate in
// fp32, and the state stays fp32. The one term that dominates an output --
// the current token's own update, P_rr u_r -- is applied in fp32.
// With fp32 inputs every contraction runs on fp32 MFMA instead.
#include <type_traits>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

__device__ __forceinline__ __bf16 bf16_from_bits(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

// vmcnt(0) with lgkmcnt and expcnt left alone (gfx9 s_waitcnt encoding).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// vmcnt(N): wait until at most N vector memory operations of this wave are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm_upto() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// ------------------------------------------------------------------ one (chunk, head) block of the workspace

enum { SC_W = 0, SC_Q = 1, SC_K = 2, SC_T = 3, SC_P = 4, SC_INV = 8 };

template <int DK, int C, bool F32M>
struct Lay {
    using TM = typename std::conditional<F32M, float, _Float16>::type;
    static constexpr int RB = C / 16, CB = DK / 16;
    static constexpr int KSD = (DK + 31) / 32, KSC = (C + 31) / 32;
    static constexpr int FRAG = 64 * 8 * (int)sizeof(TM);   // one 16x32 fragment tile
    static constexpr size_t W_OFF = 0;                                      // W       [RB][KSD] A frags
    static constexpr size_t QG_OFF = W_OFF + (size_t)RB * KSD * FRAG;       // Gamma o Q [RB][KSD]
    static constexpr size_t KE_OFF = QG_OFF + (size_t)RB * KSD * FRAG;      // K_end^T [CB][KSC]
    static constexpr size_t TT_OFF = KE_OFF + (size_t)CB * KSC * FRAG;      // T       [RB][KSC]
    static constexpr size_t PS_OFF = TT_OFF + (size_t)RB * KSC * FRAG;      // strictly lower P [RB][KSC]
    static constexpr size_t PD_OFF = PS_OFF + (size_t)RB * KSC * FRAG;      // diagonal of P, fp32 [C]
    static constexpr size_t GN_OFF = PD_OFF + (size_t)C * 4;                // gamma_last, fp32 [DK]
    static constexpr size_t SV_OFF = GN_OFF + (size_t)DK * 4;               // value column scales [128] + inverses [128]
    static constexpr size_t SC_OFF = SV_OFF + 256 * 4;                      // matrix scales [8] + inverses [8]
    static constexpr size_t BYTES = (SC_OFF + 64 + 1023) / 1024 * 1024;     // shared part
    static constexpr size_t VSL = (size_t)KSC * FRAG;                       // value B frags of one 16-column slice
};

// ------------------------------------------------------------------ fragments

template <class TM> struct FragOf;
template <> struct FragOf<_Float16> { using type = f16x8; };
template <> struct FragOf<float> { using type = f32x8; };

template <class TM>
__device__ __forceinline__ typename FragOf<TM>::type to_frag(const f32x8& x, float s) {
    if constexpr (std::is_same<TM, float>::value) {
        return x;
    } else {
        return to_f16x8(x, s);
    }
}

// Fragment from a row-major LDS array: row `row`, columns k0 + kpos(g, p),
// zero where the column is >= KLIM.
template <class TM, int KLIM>
__device__ __forceinline__ typename FragOf<TM>::type lds_frag(const TM* base, int ld, int row, int k0, int g) {
    using F = typename FragOf<TM>::type;
    const TM* p = base + (size_t)row * ld + k0 + 4 * g;
    F r;
    if constexpr (KLIM % 32 == 0) {
        if constexpr (std::is_same<TM, float>::value) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(p);
            const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16);
            r = F{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        } else {
            typedef _Float16 h4 __attribute__((ext_vector_type(4)));
            const h4 a = *reinterpret_cast<const h4*>(p);
            const h4 b = *reinterpret_cast<const h4*>(p + 16);
            r = F{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (k0 + 4 * g + j < KLIM) ? p[j] : (TM)0;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[4 + j] = (k0 + 16 + 4 * g + j < KLIM) ? p[16 + j] : (TM)0;
    }
    return r;
}

template <class TM>
__device__ __forceinline__ void st_frag(unsigned char* base, int tile, int lane, const typename FragOf<TM>::type& f) {
    *reinterpret_cast<typename FragOf<TM>::type*>(base + ((size_t)tile * 64 + lane) * sizeof(f)) = f;
}
template <class TM>
__device__ __forceinline__ typename FragOf<TM>::type ld_frag(const unsigned char* base, int tile, int lane) {
    using F = typename FragOf<TM>::type;
    return *reinterpret_cast<const F*>(base + ((size_t)tile * 64 + lane) * sizeof(F));
}

// 16-deep fp32 product on 16x16 tiles: step m takes K index 4g + m from lane group g.
__device__ __forceinline__ f32x4 mma16_f32(const f32x4& a, const f32x4& b, f32x4 c) {
#pragma unroll
    for (int m = 0; m < 4; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], c, 0, 0, 0);
    return c;
}

// ------------------------------------------------------------------ chunk addressing

struct ChunkMap {
    const int32_t* cu;      // null when every sequence has length T
    const int32_t* cstart;  // first chunk of each sequence (N+1), varlen only
    int T, N, NC;           // NC: chunks per sequence when not varlen
};

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

// cstart[s] = sum over earlier sequences of ceil(len / C); one workgroup.
__global__ void __launch_bounds__(256) chunk_index_kernel(const int32_t* __restrict__ cu, int32_t* __restrict__ cstart,
                                                          int N, int C) {
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

// ------------------------------------------------------------------ prep kernel

template <int DK, int C, bool F32M>
struct PrepSmem {
    using TM = typename Lay<DK, C, F32M>::TM;
    static constexpr int NBK = C / 16;
    static constexpr int LDM = DK + 8;   // [C][DK] arrays of TM
    static constexpr int LDT = C + 4;    // [DK][C] arrays of TM
    static constexpr int LDC = C + 4;    // [C][C] fp32
    static constexpr size_t al(size_t x) { return (x + 15) / 16 * 16; }
    static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t GKT = 0;                                       // (Gamma o K)^T
    static constexpr size_t BETA = al(GKT + (size_t)DK * LDT * sizeof(TM));
    static constexpr size_t TOT = al(BETA + (size_t)C * 4);                // block gate totals [NBK][DK]
    static constexpr size_t RED = al(TOT + (size_t)NBK * DK * 4);          // reductions [32]
    static constexpr size_t ROUND = al(RED + 32 * 4);
    // round A: Gamma o Q and K_end^T staging
    static constexpr size_t QGS = ROUND;
    static constexpr size_t KES = al(QGS + (size_t)C * LDM * sizeof(TM));
    static constexpr size_t END_A = al(KES + (size_t)DK * LDT * sizeof(TM));
    // one split level: K-side and Q-side scaled operands
    static constexpr size_t XS = ROUND;
    static constexpr size_t YS = al(XS + (size_t)C * LDM * sizeof(TM));
    static constexpr size_t END_L = al(YS + (size_t)C * LDM * sizeof(TM));
    // inverse
    static constexpr size_t XI = ROUND;
    static constexpr size_t AS = al(XI + (size_t)C * LDC * 4);
    static constexpr size_t PSM = al(AS + (size_t)C * LDC * 4);
    static constexpr size_t END_I = al(PSM + (size_t)C * LDC * 4);
    // staged value rows (value width up to 128, rounded to whole 1 KiB copies)
    static constexpr size_t END_V = ROUND + ((size_t)C * 128 * sizeof(TM) + 1023) / 1024 * 1024;
    static constexpr size_t BYTES = mx(mx(mx(END_A, END_L), END_I), END_V);
};

struct PrepParams {
    const void *q, *k, *v, *gate, *beta;
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

// Are 16-token blocks R (rows) and J (columns), R > J, separated at level hh >= 16?
__host__ __device__ constexpr bool blocks_sep_at(int R, int J, int hh) {
    return ((16 * R) / (2 * hh) == (16 * J) / (2 * hh)) && ((16 * R) % (2 * hh) >= hh) && ((16 * J) % (2 * hh) < hh);
}

// Two adjacent input elements (4- or 8-byte aligned) as floats.
__device__ __forceinline__ void ld2(const uint16_t* p, float& a, float& b) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    a = bf16_bits_to_f32((uint16_t)(u & 0xffffu));
    b = bf16_bits_to_f32((uint16_t)(u >> 16));
}
__device__ __forceinline__ void ld2(const float* p, float& a, float& b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 u = *reinterpret_cast<const f2*>(p);
    a = u[0];
    b = u[1];
}
// Two adjacent operand elements into LDS.
__device__ __forceinline__ void st2(_Float16* p, float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<h2*>(p) = h2{(_Float16)a, (_Float16)b};
}
__device__ __forceinline__ void st2(float* p, float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<f2*>(p) = f2{a, b};
}

template <class TIn, int DK, int C, bool SG, bool F32M>
__global__ void __launch_bounds__(256) chunk_prep_kernel(PrepParams p) {
    using L = Lay<DK, C, F32M>;
    using SM = PrepSmem<DK, C, F32M>;
    using TM = typename L::TM;
    constexpr int RB = L::RB, CB = L::CB, KSD = L::KSD, KSC = L::KSC;
    constexpr int NBK = C / 16;
    constexpr int CPL = DK >= 64 ? DK / 64 : 1;   // channels per lane in the gate phase
    constexpr int ACT = DK >= 64 ? 64 : DK;       // active lanes per wave in the gate phase
    constexpr int NOFF = NBK * (NBK - 1);         // off-diagonal output blocks (A and P)
    constexpr int OPW = NOFF > 0 ? (NOFF + 3) / 4 : 1;

    extern __shared__ __align__(16) unsigned char smem[];
    TM* s_gkt = reinterpret_cast<TM*>(smem + SM::GKT);
    float* s_beta = reinterpret_cast<float*>(smem + SM::BETA);
    float* s_tot = reinterpret_cast<float*>(smem + SM::TOT);
    float* s_red = reinterpret_cast<float*>(smem + SM::RED);
    TM* s_qg = reinterpret_cast<TM*>(smem + SM::QGS);
    TM* s_ke = reinterpret_cast<TM*>(smem + SM::KES);
    TM* s_x = reinterpret_cast<TM*>(smem + SM::XS);
    TM* s_y = reinterpret_cast<TM*>(smem + SM::YS);
    float* s_xi = reinterpret_cast<float*>(smem + SM::XI);
    float* s_a = reinterpret_cast<float*>(smem + SM::AS);
    float* s_p = reinterpret_cast<float*>(smem + SM::PSM);

    const int H = p.H, DV = p.DV;
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int h = item % H, gidx = item / H;
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

    // ---- gate phase layout: wave b owns tokens 16b..16b+15, lane owns CPL channels
    const bool gate_lane = (w < NBK) && (lane < ACT);
    const int blk_b = w;
    const int c0 = lane * CPL;
    float kk[16][CPL], qq[16][CPL], aa[16][CPL];
    float mk = 0.f, mq = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int tl = 16 * blk_b + t;
#pragma unroll
        for (int j = 0; j < CPL; ++j) { kk[t][j] = 0.f; qq[t][j] = 0.f; aa[t][j] = 1.f; }
        if (gate_lane && tl < n) {
            const size_t row = (size_t)(t0 + tl) * H + h;
            if constexpr (CPL == 2) {
                ld2(gk + row * DK + c0, kk[t][0], kk[t][1]);
                ld2(gq + row * DK + c0, qq[t][0], qq[t][1]);
                if constexpr (SG) {
                    aa[t][0] = aa[t][1] = ld_in(gg + row);
                } else {
                    ld2(gg + row * DK + c0, aa[t][0], aa[t][1]);
                }
            } else {
                kk[t][0] = ld_in(gk + row * DK + c0);
                qq[t][0] = ld_in(gq + row * DK + c0);
                aa[t][0] = SG ? ld_in(gg + row) : ld_in(gg + row * DK + c0);
            }
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            mk = fmaxf(mk, fabsf(kk[t][j]));
            mq = fmaxf(mq, fabsf(qq[t][j]));
        }
    }
    if (tid < C) s_beta[tid] = tid < n ? ld_in(gb + (size_t)(t0 + tid) * H + h) : 0.f;

    // ---- value rows of the chunk -> LDS, asynchronously; rows past the chunk
    // end fall outside the descriptor and arrive as zeros
    {
        const int rby = DV * (int)sizeof(TIn);            // bytes of one value row
        const int lpr = rby / 16, rpi = 64 / lpr;          // lanes per row, rows per instruction
        const uint32_t rowb = (uint32_t)H * (uint32_t)rby;
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(gv + ((size_t)t0 * H + h) * DV, (uint32_t)(n - 1) * rowb + (uint32_t)rby);
        const int ni = (C * rby + 1023) / 1024;
        for (int u = w; u < ni; u += 4) {
            const uint32_t voff = (uint32_t)(u * rpi + lane / lpr) * rowb + (uint32_t)(lane % lpr) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (__attribute__((address_space(3))) void*)(smem + SM::ROUND + (size_t)u * 1024), 16, voff, 0, 0, 0);
        }
    }

    if (gate_lane) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            float tot = 1.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) tot *= aa[t][j];
            s_tot[blk_b * DK + c0 + j] = tot;
        }
    }
    mk = wave_max(mk);
    mq = wave_max(mq);
    if (lane == 0) { s_red[w] = mk; s_red[4 + w] = mq; }
    wait_vm_all();
    __syncthreads();
    float sK = 1.f, sQ = 1.f, iK = 1.f, iQ = 1.f;
    if constexpr (!F32M) {
        const float m1 = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        const float m2 = fmaxf(fmaxf(s_red[4], s_red[5]), fmaxf(s_red[6], s_red[7]));
        sK = pow2_scale_for(m1);
        iK = pow2_inv_scale_for(m1);
        sQ = pow2_scale_for(m2);
        iQ = pow2_inv_scale_for(m2);
    }

    // ---- value fragments (B operand over tokens) from the staged rows, one
    // 16-column slice per wave, scaled per column
    {
        const TIn* vst = reinterpret_cast<const TIn*>(smem + SM::ROUND);
        for (int sl = w; sl < DV / 16; sl += 4) {
            f32x8 vf[KSC];
            float mv = 0.f;
            const int col = 16 * sl + li;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                for (int pp = 0; pp < 8; ++pp) {
                    const int t = 32 * ks + kpos(lg, pp);
                    const float x = t < C ? ld_in(vst + t * DV + col) : 0.f;
                    vf[ks][pp] = x;
                    mv = fmaxf(mv, fabsf(x));
                }
            float sv = 1.f;
            if constexpr (!F32M) {
                mv = colmax4(mv);
                sv = pow2_scale_for(mv);
                if (lg == 0) {
                    reinterpret_cast<float*>(blk + L::SV_OFF)[col] = sv;
                    reinterpret_cast<float*>(blk + L::SV_OFF)[128 + col] = pow2_inv_scale_for(mv);
                }
            }
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
                st_frag<TM>(blk + L::BYTES + (size_t)sl * L::VSL, ks, lane, to_frag<TM>(vf[ks], sv));
        }
    }
    __syncthreads();

    // ---- round A: Gamma o Q, K_end^T, (Gamma o K)^T, gamma_last
    if (gate_lane) {
        float pre[CPL], suf[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            pre[j] = 1.f;
            suf[j] = 1.f;
#pragma unroll
            for (int b = 0; b < NBK; ++b) {
                const float tb = s_tot[b * DK + c0 + j];
                if (b < blk_b) pre[j] *= tb;
                if (b > blk_b) suf[j] *= tb;
            }
        }
        float run[CPL], gkp[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) run[j] = pre[j];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int tl = 16 * blk_b + t;
            float qg[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                run[j] *= aa[t][j];
                qg[j] = qq[t][j] * run[j] * sQ;
                const float gk = kk[t][j] * run[j] * sK;
                if (t & 1) st2(&s_gkt[(c0 + j) * SM::LDT + tl - 1], gkp[j], gk);
                gkp[j] = gk;
            }
            if constexpr (CPL == 2) st2(&s_qg[tl * SM::LDM + c0], qg[0], qg[1]);
            else s_qg[tl * SM::LDM + c0] = (TM)qg[0];
        }
        if (blk_b == NBK - 1) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) reinterpret_cast<float*>(blk + L::GN_OFF)[c0 + j] = run[j];
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            float r = suf[j], nxt = 0.f;
#pragma unroll
            for (int t = 15; t >= 0; --t) {
                const float ke = kk[t][j] * r * sK;
                if (!(t & 1)) st2(&s_ke[(c0 + j) * SM::LDT + 16 * blk_b + t], ke, nxt);
                nxt = ke;
                r *= aa[t][j];
            }
        }
    }
    __syncthreads();
    for (int tt = w; tt < RB * KSD; tt += 4) {
        const int rb = tt / KSD, s = tt % KSD;
        st_frag<TM>(blk + L::QG_OFF, tt, lane, lds_frag<TM, DK>(s_qg, SM::LDM, 16 * rb + li, 32 * s, lg));
    }
    for (int tt = w; tt < CB * KSC; tt += 4) {
        const int cb = tt / KSC, s = tt % KSC;
        st_frag<TM>(blk + L::KE_OFF, tt, lane, lds_frag<TM, C>(s_ke, SM::LDT, 16 * cb + li, 32 * s, lg));
    }
    __syncthreads();

    // ---- gated Gram matrices, one split level per round
    f32x4 accA = zero4(), accP = zero4();   // diagonal block (w, w)
    f32x4 accO[OPW];                        // off-diagonal outputs o = w + 4 j
#pragma unroll
    for (int j = 0; j < OPW; ++j) accO[j] = zero4();

    auto off_out = [](int o, int& R, int& J, bool& isP) {
        isP = o >= NOFF / 2;
        int idx = isP ? o - NOFF / 2 : o;
        R = 1;
        while (idx >= R) { idx -= R; ++R; }
        J = idx;
    };

    constexpr int NLEV = (C == 64 ? 2 : (C == 32 ? 1 : 0)) + 5;
#pragma unroll
    for (int lev = 0; lev < NLEV; ++lev) {
        // half widths: C/2, ..., 16 (between blocks), then 8, 4, 2, 1, 0 (inside blocks)
        const int hh = lev < NLEV - 5 ? (C >> (lev + 1)) : (lev == NLEV - 1 ? 0 : (8 >> (lev - (NLEV - 5))));
        if (gate_lane) {
            float f[16][CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = c0 + j;
                if (hh >= 16) {
                    const int hb = hh / 16;
                    const int gs = (blk_b / (2 * hb)) * 2 * hb, midb = gs + hb;
                    if (blk_b >= midb) {
                        float run = 1.f;
                        for (int b = midb; b < blk_b; ++b) run *= s_tot[b * DK + c];
#pragma unroll
                        for (int t = 0; t < 16; ++t) { run *= aa[t][j]; f[t][j] = run; }
                    } else {
                        float run = 1.f;
                        for (int b = blk_b + 1; b < midb; ++b) run *= s_tot[b * DK + c];
#pragma unroll
                        for (int t = 15; t >= 0; --t) { f[t][j] = run; run *= aa[t][j]; }
                    }
                } else if (hh == 0) {
#pragma unroll
                    for (int t = 0; t < 16; ++t) f[t][j] = 1.f;
                } else {
#pragma unroll
                    for (int g0 = 0; g0 < 16; g0 += 2 * hh) {
                        float run = 1.f;
#pragma unroll
                        for (int t = g0 + hh; t < g0 + 2 * hh; ++t) { run *= aa[t][j]; f[t][j] = run; }
                        run = 1.f;
#pragma unroll
                        for (int t = g0 + hh - 1; t >= g0; --t) { f[t][j] = run; run *= aa[t][j]; }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int tl = 16 * blk_b + t;
                if constexpr (CPL == 2) {
                    st2(&s_x[tl * SM::LDM + c0], kk[t][0] * f[t][0] * sK, kk[t][1] * f[t][1] * sK);
                    st2(&s_y[tl * SM::LDM + c0], qq[t][0] * f[t][0] * sQ, qq[t][1] * f[t][1] * sQ);
                } else {
                    s_x[tl * SM::LDM + c0] = (TM)(kk[t][0] * f[t][0] * sK);
                    s_y[tl * SM::LDM + c0] = (TM)(qq[t][0] * f[t][0] * sQ);
                }
            }
        }
        __syncthreads();
        if (hh >= 16) {
#pragma unroll
            for (int j = 0; j < OPW; ++j) {
                const int o = w + 4 * j;
                if (o >= NOFF) continue;
                int R, J;
                bool isP;
                off_out(o, R, J, isP);
                if (!blocks_sep_at(R, J, hh)) continue;
#pragma unroll
                for (int s = 0; s < KSD; ++s) {
                    const auto af = lds_frag<TM, DK>(isP ? s_y : s_x, SM::LDM, 16 * R + li, 32 * s, lg);
                    const auto bf = lds_frag<TM, DK>(s_x, SM::LDM, 16 * J + li, 32 * s, lg);
                    accO[j] = mma(af, bf, accO[j]);
                }
            }
        } else if (w < NBK) {
            f32x4 ta = zero4(), tp = zero4();
#pragma unroll
            for (int s = 0; s < KSD; ++s) {
                const auto xf = lds_frag<TM, DK>(s_x, SM::LDM, 16 * w + li, 32 * s, lg);
                const auto yf = lds_frag<TM, DK>(s_y, SM::LDM, 16 * w + li, 32 * s, lg);
                if (hh > 0) ta = mma(xf, xf, ta);
                tp = mma(yf, xf, tp);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (sep_at(4 * lg + e, li, hh)) {
                    accA[e] += ta[e];
                    accP[e] += tp[e];
                }
            }
        }
        __syncthreads();
    }

    // ---- A = Diag(beta) A', P into LDS (upper blocks zero)
    for (int x = tid; x < C * SM::LDC; x += 256) { s_xi[x] = 0.f; s_a[x] = 0.f; s_p[x] = 0.f; }
    __syncthreads();
    {
        const float invKK = iK * iK, invQK = iQ * iK;
        if (w < NBK) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * lg + e, c = 16 * w + li;
                s_a[r * SM::LDC + c] = accA[e] * invKK * s_beta[r];
                s_p[r * SM::LDC + c] = accP[e] * invQK;
            }
        }
#pragma unroll
        for (int j = 0; j < OPW; ++j) {
            const int o = w + 4 * j;
            if (o >= NOFF) continue;
            int R, J;
            bool isP;
            off_out(o, R, J, isP);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * lg + e, c = 16 * J + li;
                if (isP) s_p[r * SM::LDC + c] = accO[j][e] * invQK;
                else s_a[r * SM::LDC + c] = accO[j][e] * invKK * s_beta[r];
            }
        }
    }
    __syncthreads();

    // ---- inverses of the 16x16 unit-lower diagonal blocks of I + A
    if (tid < RB * 16) {
        const int b = tid / 16, jj = tid % 16;
        const float* arow = s_a + (16 * b) * SM::LDC + 16 * b;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float v = rr == jj ? 1.f : 0.f;
            if (rr > jj) {
                float sacc = 0.f;
#pragma unroll
                for (int m = 0; m < rr; ++m)
                    if (m >= jj) sacc += arow[rr * SM::LDC + m] * x[m];
                v = -sacc;
            }
            x[rr] = v;
            s_xi[(16 * b + rr) * SM::LDC + 16 * b + jj] = v;
        }
    }
    __syncthreads();
    // ---- off-diagonal blocks, X_RJ = -X_RR sum_{J<=M<R} A_RM X_MJ
    for (int R = 1; R < RB; ++R) {
        for (int J = w; J < R; J += 4) {
            f32x4 tacc = zero4();
            for (int M = J; M < R; ++M) {
                f32x4 af, bf;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    af[m] = s_a[(16 * R + li) * SM::LDC + 16 * M + 4 * lg + m];
                    bf[m] = s_xi[(16 * M + 4 * lg + m) * SM::LDC + 16 * J + li];
                }
                tacc = mma16_f32(af, bf, tacc);
            }
            f32x4 xf;
#pragma unroll
            for (int m = 0; m < 4; ++m) xf[m] = s_xi[(16 * R + li) * SM::LDC + 16 * R + 4 * lg + m];
            const f32x4 xr = mma16_f32(xf, tacc, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) s_xi[(16 * R + 4 * lg + e) * SM::LDC + 16 * J + li] = -xr[e];
        }
        __syncthreads();
    }

    // ---- T = X Diag(beta), strictly lower P, diagonal of P; their scales
    auto t_frag = [&](int rb, int s) -> f32x8 {
        f32x8 r;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int c = 32 * s + kpos(lg, pp);
            r[pp] = c < C ? s_xi[(16 * rb + li) * SM::LDC + c] * s_beta[c] : 0.f;
        }
        return r;
    };
    auto p_frag = [&](int rb, int s) -> f32x8 {
        f32x8 r;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int c = 32 * s + kpos(lg, pp);
            const int row = 16 * rb + li;
            r[pp] = (c < C && c < row) ? s_p[row * SM::LDC + c] : 0.f;
        }
        return r;
    };
    float sT = 1.f, sP = 1.f, iT = 1.f, iP = 1.f;
    if constexpr (!F32M) {
        float mt = 0.f, mp = 0.f;
        for (int x = tid; x < C * C; x += 256) {
            const int r = x / C, c = x % C;
            mt = fmaxf(mt, fabsf(s_xi[r * SM::LDC + c] * s_beta[c]));
            if (c < r) mp = fmaxf(mp, fabsf(s_p[r * SM::LDC + c]));
        }
        mt = wave_max(mt);
        mp = wave_max(mp);
        if (lane == 0) { s_red[8 + w] = mt; s_red[12 + w] = mp; }
        __syncthreads();
        const float m1 = fmaxf(fmaxf(s_red[8], s_red[9]), fmaxf(s_red[10], s_red[11]));
        const float m2 = fmaxf(fmaxf(s_red[12], s_red[13]), fmaxf(s_red[14], s_red[15]));
        sT = pow2_scale_for(m1);
        iT = pow2_inv_scale_for(m1);
        sP = pow2_scale_for(m2);
        iP = pow2_inv_scale_for(m2);
    }
    for (int tt = w; tt < RB * KSC; tt += 4) {
        const int rb = tt / KSC, s = tt % KSC;
        st_frag<TM>(blk + L::TT_OFF, tt, lane, to_frag<TM>(t_frag(rb, s), sT));
        st_frag<TM>(blk + L::PS_OFF, tt, lane, to_frag<TM>(p_frag(rb, s), sP));
    }
    if (tid < C) reinterpret_cast<float*>(blk + L::PD_OFF)[tid] = s_p[tid * SM::LDC + tid];

    // ---- W = T (Gamma o K), computed as W^T = (Gamma o K)^T T^T: two stacked
    // 16x16 tiles of W^T (channel blocks 2s, 2s+1) are the A fragment of W for
    // token block rb and channel step s.
    constexpr int NWI = (RB * KSD + 3) / 4;
    f32x4 wt[NWI][2];
    float mw = 0.f;
    const float invKT = iK * iT;
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
            const auto bf = to_frag<TM>(t_frag(rb, s), sT);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int cb = 2 * s2 + half;
                if (cb >= CB) continue;
                const auto af = lds_frag<TM, C>(s_gkt, SM::LDT, 16 * cb + li, 32 * s, lg);
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

// ------------------------------------------------------------------ state kernel

struct StateParams {
    const float* S0;
    float* o;
    float* S_T;
    const unsigned char* ws;
    size_t blk_bytes;
    ChunkMap map;
    int H, DV, NSG;   // NSG: workgroups per (sequence, head)
};

// NW compute waves per workgroup, each owning SPW 16-column slices of the
// state; NW copy waves alongside.
template <int DK, int C, bool F32M, int NW, int SPW>
struct StateSmem {
    using L = Lay<DK, C, F32M>;
    static constexpr int NSL = NW * SPW;   // slices per workgroup
    static constexpr size_t BUF = L::BYTES + (size_t)NSL * L::VSL;
    static constexpr int NBUF = (2 * BUF <= 160 * 1024) ? 2 : 1;
    static constexpr size_t BYTES = NBUF * BUF;
};

// Copy one chunk's block -- the shared part and this workgroup's value
// slices -- into LDS with asynchronous buffer-to-LDS loads, 1 KiB per wave
// instruction; the block address lives in scalar registers. The NW copy
// waves split the work.
template <int DK, int C, bool F32M, int NW, int NSL>
__device__ __forceinline__ void stage_chunk(uint32_t lds_off, const unsigned char* gblk, size_t blk_bytes, int sg, int w,
                                            int lane) {
    using L = Lay<DK, C, F32M>;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int U0 = (int)(L::BYTES / 1024);
    constexpr int UV = (int)(NSL * L::VSL / 1024);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(gblk, (uint32_t)blk_bytes);
    const int vbase = (int)(L::BYTES + (size_t)sg * NSL * L::VSL) - U0 * 1024;
#pragma unroll
    for (int u = w; u < U0 + UV; u += NW) {
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
    const int vbase = (int)(L::BYTES + (size_t)sg * NSL * L::VSL) - L0 * 128;
#pragma unroll
    for (int k = 0; k < NPF; ++k) {
        const int line = (k * NW + w) * 64 + lane;
        const int off = line < L0 ? line * 128 : vbase + line * 128;
        pf[k] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
}

template <class F>
__device__ __forceinline__ F lds_ld(uint32_t off) {
    extern __shared__ __align__(16) unsigned char smem[];
    return *reinterpret_cast<const F*>(smem + off);
}

template <int DK, int C, bool F32M, int NW, int SPW>
__global__ void __launch_bounds__(128 * NW) chunk_state_kernel(StateParams p) {
    using L = Lay<DK, C, F32M>;
    using SM = StateSmem<DK, C, F32M, NW, SPW>;
    using TM = typename L::TM;
    using F = typename FragOf<TM>::type;
    constexpr int RB = L::RB, CB = L::CB, KSD = L::KSD, KSC = L::KSC;
    constexpr int NSL = SM::NSL;
    constexpr uint32_t FB = sizeof(F);   // bytes of one lane's fragment

    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int sg = item % p.NSG;
    const int hs = item / p.NSG;
    const int H = p.H, DV = p.DV;
    const int h = hs % H, s = hs / H;
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
        bos = (long)s * p.map.T;
        eos = bos + p.map.T;
        cs = s * p.map.NC;
        ce = cs + p.map.NC;
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

        // ---- U~ = T V ;  U = U~ - W S ;  O = (Gamma o Q) S
        f32x4 u[SPW][RB], ov[SPW][RB];
        {
            f32x4 tv[SPW][RB], wsum[SPW][RB], osum[SPW][RB];
#pragma unroll
            for (int j = 0; j < SPW; ++j)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) { tv[j][rb] = zero4(); wsum[j][rb] = zero4(); osum[j][rb] = zero4(); }
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
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    if (ks > rb / 2) continue;
                    const F ta = frag(L::TT_OFF, rb * KSC + ks);
#pragma unroll
                    for (int j = 0; j < SPW; ++j)
                        tv[j][rb] = mma(ta, lds_ld<F>(bo + (uint32_t)L::BYTES + (uint32_t)((w * SPW + j) * L::VSL) +
                                                      (uint32_t)ks * 64 * FB + lfr),
                                        tv[j][rb]);
                }
            }
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                float invTV = 1.f, invWS = 1.f, invQS = 1.f;
                if constexpr (!F32M) {
                    invTV = scl(SC_INV + SC_T) * lds_ld<float>(bo + (uint32_t)L::SV_OFF + 4 * (128 + col[j]));
                    invWS = scl(SC_INV + SC_W) * iS[j];
                    invQS = scl(SC_INV + SC_Q) * iS[j];
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    u[j][rb] = tv[j][rb] * invTV - wsum[j][rb] * invWS;
                    ov[j][rb] = osum[j][rb] * invQS;
                }
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
                make_rsrc(p.o + ((size_t)t0 * H + h) * DV, (uint32_t)(n - 1) * orow + (uint32_t)DV * 4);
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

// ------------------------------------------------------------------ host side

template <int DK, int C>
static size_t block_bytes_t(int dv, bool bf16) {
    return bf16 ? Lay<DK, C, false>::BYTES + (size_t)(dv / 16) * Lay<DK, C, false>::VSL
                : Lay<DK, C, true>::BYTES + (size_t)(dv / 16) * Lay<DK, C, true>::VSL;
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

size_t chunk_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, bool varlen, int N, bool bf16) {
    return index_bytes(varlen, N) +
           (size_t)chunk_count_bound(B, T, chunk, varlen, N) * H * chunk_block_bytes(dk, dv, chunk, bf16);
}

template <class K>
static hipError_t allow_lds(K kern, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <class TIn, int DK, int C, bool SG>
static hipError_t launch_prep_t(const ChunkArgs& a, const ChunkMap& map, unsigned char* blocks, long nchunks) {
    constexpr bool F32M = std::is_same<TIn, float>::value;
    using SM = PrepSmem<DK, C, F32M>;
    static_assert(SM::BYTES <= 160 * 1024, "prep LDS");
    auto kern = chunk_prep_kernel<TIn, DK, C, SG, F32M>;
    hipError_t e = allow_lds(kern, SM::BYTES);
    if (e != hipSuccess) return e;
    PrepParams pp{a.q, a.k, a.v, a.gate, a.beta, blocks, chunk_block_bytes(DK, a.dv, C, !F32M), map, a.H, a.dv};
    const long grid = nchunks * a.H;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), SM::BYTES, a.stream, pp);
    return hipGetLastError();
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
    StateParams sp{a.S0, a.o, a.S_T, blocks, chunk_block_bytes(DK, a.dv, C, !F32M), map, a.H, a.dv, nsg};
    const long grid = (long)nsg * a.H * a.N;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(128 * NW), SM::BYTES, a.stream, sp);
    return hipGetLastError();
}

// Slices per workgroup: four compute waves of one slice each when the value
// width allows (more waves in flight shorten the sequential chunk loop more
// than sharing fragment reads between slices of one wave does).
template <class TIn, int DK, int C>
static hipError_t launch_state_t(const ChunkArgs& a, const ChunkMap& map, const unsigned char* blocks) {
    if (a.dv >= 64) return launch_state_w<TIn, DK, C, 4, 1>(a, map, blocks);
    if (a.dv >= 32) return launch_state_w<TIn, DK, C, 2, 1>(a, map, blocks);
    return launch_state_w<TIn, DK, C, 1, 1>(a, map, blocks);
}

template <class TIn, int DK, int C>
static hipError_t launch_pair(const ChunkArgs& a) {
    const bool varlen = a.cu_seqlens != nullptr;
    unsigned char* ws = (unsigned char*)a.workspace;
    const size_t ib = index_bytes(varlen, a.N);
    ChunkMap map{a.cu_seqlens, varlen ? (const int32_t*)ws : nullptr, a.T, a.N, (a.T + C - 1) / C};
    unsigned char* blocks = ws + ib;
    if (a.stages & 1) {
        if (varlen) {
            hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens, (int32_t*)ws, a.N, C);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const long nch = chunk_count_bound(a.B, a.T, C, varlen, a.N);
        if (nch > 0) {
            hipError_t e = a.scalar_gate ? launch_prep_t<TIn, DK, C, true>(a, map, blocks, nch)
                                         : launch_prep_t<TIn, DK, C, false>(a, map, blocks, nch);
            if (e != hipSuccess) return e;
        }
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
