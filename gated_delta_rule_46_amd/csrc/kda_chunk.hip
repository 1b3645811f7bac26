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
//  * state -- one wavefront per (sequence, head, 16 value columns). Walks the
//    chunks of its sequence in order, keeps its slice of S in fp32 MFMA
//    accumulator registers, and writes o and the final state.
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
#include <type_traits>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

__device__ __forceinline__ __bf16 bf16_from_bits(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

template <int DK, int C, bool F32M>
struct Lay {
    using TM = typename std::conditional<F32M, float, _Float16>::type;
    static constexpr int RB = C / 16, CB = DK / 16;
    static constexpr int KSD = (DK + 31) / 32, KSC = (C + 31) / 32;
    static constexpr int FRAG = 64 * 8 * (int)sizeof(TM);   // one 16x32 fragment tile
    static constexpr int FRAG2 = 64 * 8 * 4;                // hi+lo bf16, or fp32
    static constexpr size_t W_OFF = 0;
    static constexpr size_t QG_OFF = W_OFF + (size_t)RB * KSD * FRAG;
    static constexpr size_t KE_OFF = QG_OFF + (size_t)RB * KSD * FRAG;
    static constexpr size_t TT_OFF = KE_OFF + (size_t)CB * KSC * FRAG;
    static constexpr size_t PP_OFF = TT_OFF + (size_t)RB * KSC * FRAG2;
    static constexpr size_t GN_OFF = PP_OFF + (size_t)RB * KSC * FRAG2;
    static constexpr size_t SC_OFF = GN_OFF + (size_t)DK * 4;
    static constexpr size_t BYTES = (SC_OFF + 16 + 255) / 256 * 256;
};

// ------------------------------------------------------------------ fragments

template <class TM> struct FragOf;
template <> struct FragOf<_Float16> { using type = f16x8; };
template <> struct FragOf<float> { using type = f32x8; };

// 8 values of row `row` of a row-major LDS array at columns k0 + kpos(g, p),
// zero where the column is >= klim.
template <class TM>
__device__ __forceinline__ f32x8 lds_row8(const TM* base, int ld, int row, int k0, int klim, int g) {
    f32x8 r;
    const TM* p = base + (size_t)row * ld + k0 + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (k0 + 4 * g + j < klim) ? (float)p[j] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[4 + j] = (k0 + 16 + 4 * g + j < klim) ? (float)p[16 + j] : 0.f;
    return r;
}

template <class TM>
__device__ __forceinline__ typename FragOf<TM>::type to_frag(const f32x8& x, float s) {
    if constexpr (std::is_same<TM, float>::value) {
        return x;
    } else {
        return to_f16x8(x, s);
    }
}

// Native-type fragment straight from an LDS array holding TM values.
template <class TM>
__device__ __forceinline__ typename FragOf<TM>::type lds_frag(const TM* base, int ld, int row, int k0, int klim, int g) {
    typename FragOf<TM>::type r;
    const TM* p = base + (size_t)row * ld + k0 + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (k0 + 4 * g + j < klim) ? p[j] : (TM)0;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[4 + j] = (k0 + 16 + 4 * g + j < klim) ? p[16 + j] : (TM)0;
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
    static constexpr int LDM = DK + 8;   // [C][DK] arrays of TM
    static constexpr int LDT = C + 8;    // [DK][C] arrays of TM
    static constexpr int LDC = C + 4;    // [C][C] fp32
    static constexpr int LDW = DK + 4;   // [C][DK] fp32 staging
    static constexpr size_t al(size_t x) { return (x + 15) / 16 * 16; }
    static constexpr size_t GKT = 0;
    static constexpr size_t ALT = al(GKT + (size_t)DK * LDT * sizeof(TM));
    // phase A
    static constexpr size_t QGS = ALT;
    static constexpr size_t KES = al(QGS + (size_t)C * LDM * sizeof(TM));
    static constexpr size_t END_A = al(KES + (size_t)DK * LDT * sizeof(TM));
    // phase B
    static constexpr size_t XS = ALT;
    static constexpr size_t YS = al(XS + (size_t)C * LDM * sizeof(TM));
    static constexpr size_t END_B = al(YS + (size_t)C * LDM * sizeof(TM));
    // phases C, D
    static constexpr size_t XI = ALT;
    static constexpr size_t AS = al(XI + (size_t)C * LDC * 4);
    static constexpr size_t PS = al(AS + (size_t)C * LDC * 4);
    static constexpr size_t END_AP = al(PS + (size_t)C * LDC * 4);
    static constexpr size_t WS = AS;
    static constexpr size_t END_W = al(WS + (size_t)C * LDW * 4);
    static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t SMALL = mx(mx(END_A, END_B), mx(END_AP, END_W));
    static constexpr size_t BETA = SMALL;
    static constexpr size_t RED = al(BETA + (size_t)C * 4);
    static constexpr size_t BYTES = al(RED + 16 * 4);
};

struct PrepParams {
    const void *q, *k, *gate, *beta;
    unsigned char* ws;
    ChunkMap map;
    int H;
};

// Is entry (r, j) of a 16x16 diagonal block separated at level h? h == 0 is
// the diagonal itself (P only).
__device__ __forceinline__ bool sep_at(int r, int j, int h) {
    if (h == 0) return r == j;
    const int w = 2 * h;
    return (r / w == j / w) && (r % w >= h) && (j % w < h);
}

template <class TIn, int DK, int C, bool SG, bool F32M>
__global__ void __launch_bounds__(256) chunk_prep_kernel(PrepParams p) {
    using L = Lay<DK, C, F32M>;
    using SM = PrepSmem<DK, C, F32M>;
    using TM = typename L::TM;
    constexpr int RB = L::RB, CB = L::CB, KSD = L::KSD, KSC = L::KSC;
    constexpr int NBLK = RB * (RB + 1) / 2;
    constexpr int NOUT = 2 * NBLK;
    constexpr int PER = (NOUT + 3) / 4;
    constexpr int LOGC = C == 16 ? 4 : (C == 32 ? 5 : 6);

    extern __shared__ __align__(16) unsigned char smem[];
    TM* s_gkt = reinterpret_cast<TM*>(smem + SM::GKT);
    TM* s_qg = reinterpret_cast<TM*>(smem + SM::QGS);
    TM* s_ke = reinterpret_cast<TM*>(smem + SM::KES);
    TM* s_x = reinterpret_cast<TM*>(smem + SM::XS);
    TM* s_y = reinterpret_cast<TM*>(smem + SM::YS);
    float* s_xi = reinterpret_cast<float*>(smem + SM::XI);
    float* s_a = reinterpret_cast<float*>(smem + SM::AS);
    float* s_p = reinterpret_cast<float*>(smem + SM::PS);
    float* s_w = reinterpret_cast<float*>(smem + SM::WS);
    float* s_beta = reinterpret_cast<float*>(smem + SM::BETA);
    float* s_red = reinterpret_cast<float*>(smem + SM::RED);

    const int H = p.H;
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int h = item % H, gidx = item / H;
    long t0;
    int n;
    if (!resolve_chunk(p.map, gidx, C, t0, n)) return;   // uniform over the workgroup

    const int tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
    const int li = lane % 16, lg = lane / 16;
    unsigned char* blk = p.ws + ((size_t)gidx * H + h) * L::BYTES;
    const TIn* gq = (const TIn*)p.q;
    const TIn* gk = (const TIn*)p.k;
    const TIn* gg = (const TIn*)p.gate;
    const TIn* gb = (const TIn*)p.beta;

    // ---- A1: this thread's channel over the chunk (padding: k = q = 0, alpha = 1, beta = 0)
    const int ch = tid;
    const bool has_ch = ch < DK;
    float a[C], kk[C], qq[C];
    float mk = 0.f, mq = 0.f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
        kk[t] = 0.f; qq[t] = 0.f; a[t] = 1.f;
        if (has_ch && t < n) {
            const size_t row = (size_t)(t0 + t) * H + h;
            kk[t] = ld_in(gk + row * DK + ch);
            qq[t] = ld_in(gq + row * DK + ch);
            a[t] = SG ? ld_in(gg + row) : ld_in(gg + row * DK + ch);
        }
        mk = fmaxf(mk, fabsf(kk[t]));
        mq = fmaxf(mq, fabsf(qq[t]));
    }
    if (tid < C) s_beta[tid] = tid < n ? ld_in(gb + (size_t)(t0 + tid) * H + h) : 0.f;
    mk = wave_max(mk);
    mq = wave_max(mq);
    if (lane == 0) { s_red[w] = mk; s_red[4 + w] = mq; }
    __syncthreads();
    float sK = 1.f, sQ = 1.f;
    if constexpr (!F32M) {
        sK = pow2_scale_for(fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3])));
        sQ = pow2_scale_for(fmaxf(fmaxf(s_red[4], s_red[5]), fmaxf(s_red[6], s_red[7])));
    }

    // ---- A2: Gamma o Q, K_end^T, (Gamma o K)^T, gamma_last
    if (has_ch) {
        float run = 1.f;
#pragma unroll
        for (int t = 0; t < C; ++t) {
            run *= a[t];
            s_qg[t * SM::LDM + ch] = (TM)(qq[t] * run * sQ);
            s_gkt[ch * SM::LDT + t] = (TM)(kk[t] * run * sK);
        }
        reinterpret_cast<float*>(blk + L::GN_OFF)[ch] = run;
        float suf = 1.f;
#pragma unroll
        for (int t = C - 1; t >= 0; --t) {
            s_ke[ch * SM::LDT + t] = (TM)(kk[t] * suf * sK);
            suf *= a[t];
        }
    }
    __syncthreads();
    // ---- A3: those two as MFMA fragments
    for (int tt = w; tt < RB * KSD; tt += 4) {
        const int rb = tt / KSD, s = tt % KSD;
        st_frag<TM>(blk + L::QG_OFF, tt, lane, lds_frag<TM>(s_qg, SM::LDM, 16 * rb + li, 32 * s, DK, lg));
    }
    for (int tt = w; tt < CB * KSC; tt += 4) {
        const int cb = tt / KSC, s = tt % KSC;
        st_frag<TM>(blk + L::KE_OFF, tt, lane, lds_frag<TM>(s_ke, SM::LDT, 16 * cb + li, 32 * s, C, lg));
    }
    if (tid == 0) {
        float* sc = reinterpret_cast<float*>(blk + L::SC_OFF);
        sc[1] = sQ;
        sc[2] = sK;
    }
    __syncthreads();

    // ---- B: gated Gram matrices A' (K side) and P (Q side), level by level
    f32x4 acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = zero4();

#pragma unroll
    for (int lev = 0; lev <= LOGC; ++lev) {
        const int hh = lev < LOGC ? (C >> (lev + 1)) : 0;   // half width of the split; 0 = diagonal
        if (has_ch) {
            float f[C];
            if (hh == 0) {
#pragma unroll
                for (int t = 0; t < C; ++t) f[t] = 1.f;
            } else {
#pragma unroll
                for (int g0 = 0; g0 < C; g0 += 2 * hh) {
                    float run = 1.f;
#pragma unroll
                    for (int t = g0 + hh; t < g0 + 2 * hh; ++t) { run *= a[t]; f[t] = run; }
                    run = 1.f;
#pragma unroll
                    for (int t = g0 + hh - 1; t >= g0; --t) { f[t] = run; run *= a[t]; }
                }
            }
#pragma unroll
            for (int t = 0; t < C; ++t) {
                s_x[t * SM::LDM + ch] = (TM)(kk[t] * f[t] * sK);
                s_y[t * SM::LDM + ch] = (TM)(qq[t] * f[t] * sQ);
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int o = w + 4 * j;
            if (o >= NOUT) continue;
            const bool isP = o >= NBLK;
            int idx = o % NBLK, R = 0;
            while (idx >= R + 1) { idx -= R + 1; ++R; }
            const int J = idx;
            bool on;
            if (hh >= 16) {
                const int w2 = 2 * hh;
                on = (R != J) && ((16 * R) / w2 == (16 * J) / w2) && ((16 * R) % w2 >= hh) && ((16 * J) % w2 < hh);
            } else {
                on = (R == J) && (hh > 0 || isP);
            }
            if (!on) continue;
            f32x4 tmp = zero4();
#pragma unroll
            for (int s = 0; s < KSD; ++s) {
                const auto af = lds_frag<TM>(isP ? s_y : s_x, SM::LDM, 16 * R + li, 32 * s, DK, lg);
                const auto bf = lds_frag<TM>(s_x, SM::LDM, 16 * J + li, 32 * s, DK, lg);
                tmp = mma(af, bf, tmp);
            }
            if (hh >= 16) {
                acc[j] += tmp;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (sep_at(4 * lg + e, li, hh)) acc[j][e] += tmp[e];
            }
        }
        __syncthreads();
    }

    // ---- B2: A = Diag(beta) A', P into LDS (upper blocks zero)
    for (int x = tid; x < C * SM::LDC; x += 256) { s_xi[x] = 0.f; s_a[x] = 0.f; s_p[x] = 0.f; }
    __syncthreads();
    {
        const float invKK = 1.f / (sK * sK), invQK = 1.f / (sQ * sK);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int o = w + 4 * j;
            if (o >= NOUT) continue;
            const bool isP = o >= NBLK;
            int idx = o % NBLK, R = 0;
            while (idx >= R + 1) { idx -= R + 1; ++R; }
            const int J = idx;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * lg + e, c = 16 * J + li;
                if (isP) s_p[r * SM::LDC + c] = acc[j][e] * invQK;
                else s_a[r * SM::LDC + c] = acc[j][e] * invKK * s_beta[r];
            }
        }
    }
    __syncthreads();

    // ---- C1: inverses of the 16x16 unit-lower diagonal blocks of I + A
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
    // ---- C2: off-diagonal blocks, X_RJ = -X_RR sum_{J<=M<R} A_RM X_MJ
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

    // ---- D1: scale of T = X Diag(beta)
    float sT = 1.f;
    if constexpr (!F32M) {
        float mt = 0.f;
        for (int x = tid; x < C * C; x += 256) {
            const int r = x / C, c = x % C;
            mt = fmaxf(mt, fabsf(s_xi[r * SM::LDC + c] * s_beta[c]));
        }
        mt = wave_max(mt);
        if (lane == 0) s_red[8 + w] = mt;
        __syncthreads();
        sT = pow2_scale_for(fmaxf(fmaxf(s_red[8], s_red[9]), fmaxf(s_red[10], s_red[11])));
    }

    // ---- D2: T and P fragments to the workspace; W = T (Gamma o K) tiles in registers
    auto t_frag = [&](int rb, int s) -> f32x8 {
        f32x8 r;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int c = 32 * s + kpos(lg, pp);
            r[pp] = c < C ? s_xi[(16 * rb + li) * SM::LDC + c] * s_beta[c] : 0.f;
        }
        return r;
    };
    for (int tt = w; tt < RB * KSC; tt += 4) {
        const int rb = tt / KSC, s = tt % KSC;
        const f32x8 tf = t_frag(rb, s);
        f32x8 pf;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int c = 32 * s + kpos(lg, pp);
            pf[pp] = c < C ? s_p[(16 * rb + li) * SM::LDC + c] : 0.f;
        }
        if constexpr (F32M) {
            st_frag<float>(blk + L::TT_OFF, tt, lane, tf);
            st_frag<float>(blk + L::PP_OFF, tt, lane, pf);
        } else {
            const bf16pair ts = split8(tf), ps = split8(pf);
            bf16x8* tp = reinterpret_cast<bf16x8*>(blk + L::TT_OFF) + (size_t)tt * 128;
            bf16x8* pq = reinterpret_cast<bf16x8*>(blk + L::PP_OFF) + (size_t)tt * 128;
            tp[lane] = ts.hi; tp[64 + lane] = ts.lo;
            pq[lane] = ps.hi; pq[64 + lane] = ps.lo;
        }
    }
    constexpr int NWT = (RB * CB + 3) / 4;
    f32x4 wacc[NWT];
    float mw = 0.f;
    const float invTK = 1.f / (sT * sK);
#pragma unroll
    for (int j = 0; j < NWT; ++j) {
        wacc[j] = zero4();
        const int tt = w + 4 * j;
        if (tt >= RB * CB) continue;
        const int rb = tt / CB, cb = tt % CB;
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
            if (s > rb / 2) continue;
            const auto af = to_frag<TM>(t_frag(rb, s), sT);
            const auto bf = lds_frag<TM>(s_gkt, SM::LDT, 16 * cb + li, 32 * s, C, lg);
            wacc[j] = mma(af, bf, wacc[j]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wacc[j][e] *= invTK;
            mw = fmaxf(mw, fabsf(wacc[j][e]));
        }
    }
    mw = wave_max(mw);
    if (lane == 0) s_red[12 + w] = mw;
    __syncthreads();   // T, P fragments done; A_s and P_s may now be overwritten
    float sW = 1.f;
    if constexpr (!F32M) sW = pow2_scale_for(fmaxf(fmaxf(s_red[12], s_red[13]), fmaxf(s_red[14], s_red[15])));
#pragma unroll
    for (int j = 0; j < NWT; ++j) {
        const int tt = w + 4 * j;
        if (tt >= RB * CB) continue;
        const int rb = tt / CB, cb = tt % CB;
#pragma unroll
        for (int e = 0; e < 4; ++e) s_w[(16 * rb + 4 * lg + e) * SM::LDW + 16 * cb + li] = wacc[j][e];
    }
    __syncthreads();
    for (int tt = w; tt < RB * KSD; tt += 4) {
        const int rb = tt / KSD, s = tt % KSD;
        st_frag<TM>(blk + L::W_OFF, tt, lane, to_frag<TM>(lds_row8<float>(s_w, SM::LDW, 16 * rb + li, 32 * s, DK, lg), sW));
    }
    if (tid == 0) reinterpret_cast<float*>(blk + L::SC_OFF)[0] = sW;
}

// ------------------------------------------------------------------ state kernel

struct StateParams {
    const void* v;
    const float* S0;
    float* o;
    float* S_T;
    const unsigned char* ws;
    ChunkMap map;
    int H, DV, NS;   // NS: value-column slices of 16
};

template <class TIn, int DK, int C, bool F32M>
__global__ void __launch_bounds__(64) chunk_state_kernel(StateParams p) {
    using L = Lay<DK, C, F32M>;
    using TM = typename L::TM;
    using F = typename FragOf<TM>::type;
    constexpr int RB = L::RB, CB = L::CB, KSD = L::KSD, KSC = L::KSC;

    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int slice = item % p.NS;
    const int hs = item / p.NS;
    const int H = p.H, DV = p.DV;
    const int h = hs % H, s = hs / H;
    const int lane = threadIdx.x, li = lane % 16, lg = lane / 16;
    const int col = 16 * slice + li;

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

    // state slice: rows 16*cb + 4*lg + e, column `col`
    f32x4 S[CB];
    const size_t sbase = ((size_t)s * H + h) * DK * DV;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[cb][e] = p.S0 ? p.S0[sbase + (size_t)(16 * cb + 4 * lg + e) * DV + col] : 0.f;

    const TIn* gv = (const TIn*)p.v;
    for (int cg = cs; cg < ce; ++cg) {
        const long t0 = bos + (long)(cg - cs) * C;
        const int n = (int)min((long)C, eos - t0);
        const unsigned char* blk = p.ws + ((size_t)cg * H + h) * L::BYTES;
        const float* sc = reinterpret_cast<const float*>(blk + L::SC_OFF);

        // ---- U~ = T V
        f32x4 u[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) u[rb] = zero4();
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            if constexpr (F32M) {
                f32x8 vf;
#pragma unroll
                for (int pp = 0; pp < 8; ++pp) {
                    const int t = 32 * ks + kpos(lg, pp);
                    vf[pp] = t < n ? ld_in(gv + ((size_t)(t0 + t) * H + h) * DV + col) : 0.f;
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if (ks > rb / 2) continue;
                    u[rb] = mma(ld_frag<float>(blk + L::TT_OFF, rb * KSC + ks, lane), vf, u[rb]);
                }
            } else {
                bf16x8 vb;
#pragma unroll
                for (int pp = 0; pp < 8; ++pp) {
                    const int t = 32 * ks + kpos(lg, pp);
                    const uint16_t bits = t < n ? reinterpret_cast<const uint16_t*>(gv)[((size_t)(t0 + t) * H + h) * DV + col] : (uint16_t)0;
                    vb[pp] = bf16_from_bits(bits);
                }
                const bf16x8* tp = reinterpret_cast<const bf16x8*>(blk + L::TT_OFF);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if (ks > rb / 2) continue;
                    const size_t tt = (size_t)(rb * KSC + ks) * 128;
                    u[rb] = mma(tp[tt + lane], vb, u[rb]);
                    u[rb] = mma(tp[tt + 64 + lane], vb, u[rb]);
                }
            }
        }

        // ---- S as B fragments (scaled fp16, or fp32)
        float sS = 1.f;
        if constexpr (!F32M) {
            float m = 0.f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(S[cb][e]));
            sS = pow2_scale_for(wave_max(m));
        }
        F sf[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const f32x4 bot = (2 * ks + 1 < CB) ? S[2 * ks + 1] : zero4();
            sf[ks] = to_frag<TM>(dtiles_to_frag(S[2 * ks], bot), sS);
        }

        // ---- U = U~ - W S ;  O = (Gamma o Q) S
        f32x4 ov[RB];
        const float invWS = F32M ? 1.f : 1.f / (sc[0] * sS);
        const float invQS = F32M ? 1.f : 1.f / (sc[1] * sS);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            f32x4 ws = zero4(), os = zero4();
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                ws = mma(ld_frag<TM>(blk + L::W_OFF, rb * KSD + ks, lane), sf[ks], ws);
                os = mma(ld_frag<TM>(blk + L::QG_OFF, rb * KSD + ks, lane), sf[ks], os);
            }
            u[rb] -= ws * invWS;
            ov[rb] = os * invQS;
        }

        // ---- U as B fragments over tokens
        float sU = 1.f;
        if constexpr (!F32M) {
            float m = 0.f;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(u[rb][e]));
            sU = pow2_scale_for(wave_max(m));
        }
        f32x8 uf[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) uf[ks] = dtiles_to_frag(u[2 * ks], (2 * ks + 1 < RB) ? u[2 * ks + 1] : zero4());

        // ---- O += P U (three bf16 products, or fp32)
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            if constexpr (F32M) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if (ks > rb / 2) continue;
                    ov[rb] = mma(ld_frag<float>(blk + L::PP_OFF, rb * KSC + ks, lane), uf[ks], ov[rb]);
                }
            } else {
                const bf16pair us = split8(uf[ks]);
                const bf16x8* pp = reinterpret_cast<const bf16x8*>(blk + L::PP_OFF);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if (ks > rb / 2) continue;
                    const size_t tt = (size_t)(rb * KSC + ks) * 128;
                    const bf16x8 phi = pp[tt + lane], plo = pp[tt + 64 + lane];
                    ov[rb] = mma(phi, us.hi, ov[rb]);
                    ov[rb] = mma(phi, us.lo, ov[rb]);
                    ov[rb] = mma(plo, us.hi, ov[rb]);
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * rb + 4 * lg + e;
                if (t < n) p.o[((size_t)(t0 + t) * H + h) * DV + col] = ov[rb][e];
            }

        // ---- S <- Diag(gamma_last) S + K_end^T U
        const float* gn = reinterpret_cast<const float*>(blk + L::GN_OFF);
        F ufr[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) ufr[ks] = to_frag<TM>(uf[ks], sU);
        const float invKU = F32M ? 1.f : 1.f / (sc[2] * sU);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            f32x4 ku = zero4();
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) ku = mma(ld_frag<TM>(blk + L::KE_OFF, cb * KSC + ks, lane), ufr[ks], ku);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[cb][e] = S[cb][e] * gn[16 * cb + 4 * lg + e] + ku[e] * invKU;
        }
    }

    if (p.S_T) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.S_T[sbase + (size_t)(16 * cb + 4 * lg + e) * DV + col] = S[cb][e];
    }
}

// ------------------------------------------------------------------ host side

template <int DK, int C>
static size_t block_bytes_t(bool bf16) { return bf16 ? Lay<DK, C, false>::BYTES : Lay<DK, C, true>::BYTES; }

template <int DK>
static size_t block_bytes_c(int chunk, bool bf16) {
    switch (chunk) {
        case 16: return block_bytes_t<DK, 16>(bf16);
        case 32: return block_bytes_t<DK, 32>(bf16);
        default: return block_bytes_t<DK, 64>(bf16);
    }
}

size_t chunk_block_bytes(int dk, int chunk, bool bf16) {
    switch (dk) {
        case 16: return block_bytes_c<16>(chunk, bf16);
        case 32: return block_bytes_c<32>(chunk, bf16);
        case 64: return block_bytes_c<64>(chunk, bf16);
        default: return block_bytes_c<128>(chunk, bf16);
    }
}

long chunk_count_bound(int B, int T, int chunk, bool varlen, int N) {
    if (!varlen) return (long)B * ((T + chunk - 1) / chunk);
    return (long)(T + chunk - 1) / chunk + N;
}

static size_t index_bytes(bool varlen, int N) { return varlen ? ((size_t)(N + 1) * 4 + 255) / 256 * 256 : 0; }

size_t chunk_workspace_bytes(int B, int H, int T, int dk, int chunk, bool varlen, int N, bool bf16) {
    return index_bytes(varlen, N) + (size_t)chunk_count_bound(B, T, chunk, varlen, N) * H * chunk_block_bytes(dk, chunk, bf16);
}

template <class TIn, int DK, int C, bool SG>
static hipError_t launch_prep_t(const ChunkArgs& a, const ChunkMap& map, unsigned char* blocks, long nchunks) {
    constexpr bool F32M = std::is_same<TIn, float>::value;
    using SM = PrepSmem<DK, C, F32M>;
    auto kern = chunk_prep_kernel<TIn, DK, C, SG, F32M>;
    static_assert(SM::BYTES <= 160 * 1024, "prep LDS");
    if (SM::BYTES > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)SM::BYTES);
        if (e != hipSuccess) return e;
    }
    PrepParams pp{a.q, a.k, a.gate, a.beta, blocks, map, a.H};
    const long grid = nchunks * a.H;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), SM::BYTES, a.stream, pp);
    return hipGetLastError();
}

template <class TIn, int DK, int C>
static hipError_t launch_state_t(const ChunkArgs& a, const ChunkMap& map, const unsigned char* blocks) {
    constexpr bool F32M = std::is_same<TIn, float>::value;
    StateParams sp{a.v, a.S0, a.o, a.S_T, blocks, map, a.H, a.dv, a.dv / 16};
    const long grid = (long)(a.dv / 16) * a.H * a.N;
    hipLaunchKernelGGL((chunk_state_kernel<TIn, DK, C, F32M>), dim3((unsigned)grid), dim3(64), 0, a.stream, sp);
    return hipGetLastError();
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
