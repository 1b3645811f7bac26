// Gradient of the gated delta-rule forward over whole sequences.
//
// Forward, per (sequence, head), state S in R^{dk x dv} (Complex KDA summary,
// background "diagonal-plus-rank-one transitions"; delta form of the CyFA blog
// post, section 2.2, gate first):
//   S' = Diag(alpha_t) S_{t-1};  pred = S'^T k_t;  u = beta_t (v_t - pred)
//   S_t = S' + k_t u^T;          o_t = S_t^T q_t
// With dS = dL/dS_t (dS_T, or zero, before the last token), the adjoint of
// one token, last token first:
//   dS += q dO^T                 dq = S_t dO
//   du = dS^T k                  dk = dS u + S' dpred,   dpred = -beta du
//   dbeta = du . (v - pred)      dv = beta du
//   dS' = dS + k dpred^T         dalpha_i = sum_j dS'_ij S_{t-1,ij}
//   dS  = Diag(alpha) dS'        (dL/dS_{t-1}; after the first token: dS0)
// The pages measure forward-plus-backward throughput of this family (Complex
// KDA summary, efficiency) without printing the backward; the lines above
// are the chain rule applied to the forward, nothing more.
// With decoupled erase and write gates (EW: erase e per key channel, write w
// per value channel; S_t = S' + k (w o v - S'^T (e o k))^T) the same adjoint
// reads with ke = e o k and drops beta:
//   du = dS^T k       dk = dS u + e o dke,   dke = S' dpred,  dpred = -du
//   dv = w o du       dw = du o v            de = k o dke
//   dS' = dS + ke dpred^T                    (dalpha, dS as above)
//
// Value columns of S never mix (the transition acts on the key side only),
// so each wave owns COLS value columns and all dk rows of S and dS: lane l
// holds rows l + 64 m. A column sum over the rows (pred, du) is then a
// wave-wide sum (DPP inside rows of 16 lanes, lane swaps across rows), with
// no barrier. Only dq, dk and dalpha (sums over value columns) cross waves,
// through per-wave partial sums in LDS, and workgroups, through
// per-workgroup partial sums in memory that a second kernel adds up.
//
// Pass A runs the forward from S0 and stores S at the start of every
// SUB-token block (the checkpoints) and the residual e = v - pred of every
// token. Pass B walks the blocks backwards: reload the checkpoint, replay the
// block forward with u = beta e (no reductions) keeping the SUB states
// S_{t-1} in registers, then the adjoint over the block. The adjoint takes
// S_t from the replay (the next block's checkpoint for the block's last
// token), and dk's S' dpred term as -Diag(alpha) (S_{t-1} dv), so S' is never
// formed. Each block's inputs are staged in LDS once, fetched one block ahead;
// one barrier per block. All arithmetic is fp32 (inputs converted exactly).
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int BW_SUB = 8;   // tokens per checkpoint interval
constexpr int BW_OOB = (int)0x80000000;   // buffer offset past any range used here: the store is dropped


// The four column sums of a wave (x[c] summed over the 64 lanes), returned
// in every lane (wave-uniform), with a reduce-scatter instead of four full
// reductions: swapping with the neighbour lane and then with the lane two
// away, each lane keeps half of what it has and adds its partner's copy of
// that half, until it holds one column (column 0, 2, 1, 3 in lanes 0, 1, 2, 3
// of every quad); row rotations by 4 and 8 then sum the four quads of each
// row of 16 lanes, two lane swaps sum the four rows, and lanes 0..3 hold the
// totals, which readlane makes scalars.
template <int CTRL>
__device__ __forceinline__ float dpp_of(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ void wave_sum4(const float (&x)[4], float (&out)[4], int lane) {
    const bool odd = lane & 1, hi = lane & 2;
    const float k0 = odd ? x[2] : x[0], k1 = odd ? x[3] : x[1];
    const float s0 = odd ? x[0] : x[2], s1 = odd ? x[1] : x[3];
    const float n0 = k0 + dpp_of<0xB1>(s0), n1 = k1 + dpp_of<0xB1>(s1);   // quad_perm [1,0,3,2]
    const float kk = hi ? n1 : n0, ss = hi ? n0 : n1;
    float m = kk + dpp_of<0x4E>(ss);                                      // quad_perm [2,3,0,1]
    m += dpp_of<0x124>(m);                                                // row_ror:4
    m += dpp_of<0x128>(m);                                                // row_ror:8
    const uint32_t u = __float_as_uint(m);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t u2 = __float_as_uint(m);
    const auto b = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
    m = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    const int mi = __float_as_int(m);
    out[0] = __int_as_float(__builtin_amdgcn_readlane(mi, 0));
    out[1] = __int_as_float(__builtin_amdgcn_readlane(mi, 2));
    out[2] = __int_as_float(__builtin_amdgcn_readlane(mi, 1));
    out[3] = __int_as_float(__builtin_amdgcn_readlane(mi, 3));
}

struct BwdParams {
    const void *q, *k, *v, *gate, *beta;
    const void *erase, *write;   // erase/write form only
    const float *S0, *dO, *dST;
    float *dv_out, *dS0, *ckpt, *part;
    float* dw_out;               // erase/write form: dL/dwrite
    float* resid;   // e = v - S'^T k of every token from pass A, [B*T*H][dv]
    const int32_t* cu;
    int H, T, dv, ncg;
    long nblk;   // checkpoint slots per (head, column group)
    long rows;   // B * T * H
};

template <int DK, int NC, bool SG, bool EW>
struct BwdStage {
    float k[BW_SUB][DK], q[BW_SUB][DK], a[BW_SUB][SG ? 1 : DK];
    float v[BW_SUB][NC], dO[BW_SUB][NC], e[BW_SUB][NC], b[BW_SUB];
    float er[BW_SUB][EW ? DK : 1], wr[BW_SUB][EW ? NC : 1];   // erase and write gates
};

// Partial sums per row kept per wave: dq, dk, dalpha (and de with erase/write gates).
template <bool EW> constexpr int bwd_nq() { return EW ? 4 : 3; }

// Dynamic LDS of one workgroup: the double-buffered input stage and, also
// double-buffered by block parity, each wave's per-token partial sums over its
// own value columns (dq, dk, dalpha per row; dbeta), written with plain
// stores and added up across the waves when the block is flushed. (LDS
// atomics from four waves onto the same rows took 40% of the kernel time.)
template <int DK, int NC, int NWV, bool SG, bool EW>
struct BwdLds {
    // partial-sum slots double-buffered by block parity, except for the
    // erase/write form at dk = 128, whose four slots fit LDS only once (its
    // block flush then ends with a barrier of its own)
    static constexpr int NSB = (EW && DK >= 128) ? 1 : 2;
    BwdStage<DK, NC, SG, EW> st[2];
    float slot[NSB][NWV][BW_SUB][bwd_nq<EW>()][DK];
    float slotb[2][NWV][BW_SUB];
    float vout[2][BW_SUB][NC];   // per-token wave-uniform results: e (pass A), dv (pass B)
    float vout2[2][BW_SUB][EW ? NC : 1];   // dw (pass B, erase/write form)
    // target of the lanes that do not store a wave-uniform value: lane l
    // writes 4 floats at 4 l + j NC for token j (the stride of vout), so one
    // base address per block serves every token
    float junk[4 * WAVE + BW_SUB * NC];
};

// Buffer resource over the SUB tokens starting at token `tok0` (flat token
// index b * T + t) of a [tokens][H][width] float array, so that per-element
// offsets stay small and tokens past the end of a sequence can be dropped
// with an out-of-range offset instead of a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(float* base, size_t tok0, int H, int width) {
    return make_rsrc(base + tok0 * H * width, (uint32_t)(BW_SUB * H * width * 4));
}

// One block's inputs, fetched into registers one block ahead, then written
// to LDS. Element e = tid + NT i of the [SUB][DK] key-side arrays and of the
// [SUB][NC] value-side arrays. Tokens past the sequence end get gate 1 and
// zeros everywhere else, which makes them exact no-ops in both directions
// (S' = S, u = 0; dS, dq, dk, dv and dbeta unchanged or zero), so the token
// loops run without branches and the compiler can overlap tokens.
// Inputs stay in their storage type between the load and the LDS store (the
// next block), so that nothing reads the loaded registers early and forces a
// wait for the memory latency inside the token loop.
__device__ __forceinline__ float in_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float in_f32(float x) { return x; }
template <class TIn> __device__ __forceinline__ TIn in_one();
template <> __device__ __forceinline__ uint16_t in_one<uint16_t>() { return 0x3F80; }   // bf16 1.0
template <> __device__ __forceinline__ float in_one<float>() { return 1.f; }

template <class TIn, int DK, int NC, int NT, int RPL, int COLS, bool SG, bool BWD, bool EW>
struct BwdFetch {
    static constexpr int KPT = (BW_SUB * DK + NT - 1) / NT;
    static constexpr int VPT = (BW_SUB * NC + NT - 1) / NT;
    static constexpr bool LV = !BWD || EW;   // v is staged (pass A; pass B of the erase/write form)
    TIn k[KPT], q[BWD ? KPT : 1], a[SG ? 1 : KPT], v[LV ? VPT : 1], b, ag;
    TIn er[EW ? KPT : 1], wr[EW ? VPT : 1];
    float dO[BWD ? VPT : 1], pr[BWD ? VPT : 1];
    f32x4 ck[BWD ? RPL * COLS / 4 : 1];   // this lane's part of the block's checkpoint

    __device__ __forceinline__ void fetch(const BwdParams& p, int tid, int b0, int h, int ts, int te, int cw0,
                                          const float* ckp) {
        const TIn* K = (const TIn*)p.k;
        const TIn* Q = (const TIn*)p.q;
        const TIn* A = (const TIn*)p.gate;
        const TIn* V = (const TIn*)p.v;
        const TIn* Bt = (const TIn*)p.beta;
        const TIn* E = (const TIn*)p.erase;
        const TIn* W = (const TIn*)p.write;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int e = tid + NT * i, j = e / DK, r = e % DK, t = ts + j;
            const bool ok = e < BW_SUB * DK && t < te;
            const size_t row = ((size_t)b0 * p.T + t) * p.H + h;
            k[i] = ok ? K[row * DK + r] : TIn(0);
            if (BWD) q[i] = ok ? Q[row * DK + r] : TIn(0);
            if (!SG) a[i] = ok ? A[row * DK + r] : in_one<TIn>();
            if (EW) er[i] = ok ? E[row * DK + r] : TIn(0);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int e = tid + NT * i, j = e / NC, c = e % NC, t = ts + j;
            const bool ok = e < BW_SUB * NC && t < te;
            const size_t row = ((size_t)b0 * p.T + t) * p.H + h;
            if (LV) v[i] = ok ? V[row * p.dv + cw0 + c] : TIn(0);
            if (EW) wr[i] = ok ? W[row * p.dv + cw0 + c] : TIn(0);
            if (BWD) dO[i] = ok ? p.dO[row * p.dv + cw0 + c] : 0.f;
            if (BWD) pr[i] = ok ? p.resid[row * p.dv + cw0 + c] : 0.f;
        }
        {
            const int t = ts + tid;
            const bool ok = tid < BW_SUB && t < te;
            const size_t row = ((size_t)b0 * p.T + t) * p.H + h;
            b = ok && !EW ? Bt[row] : TIn(0);
            ag = SG ? (ok ? A[row] : in_one<TIn>()) : TIn(0);
        }
        if (BWD) {
            const f32x4* c4 = reinterpret_cast<const f32x4*>(ckp);
#pragma unroll
            for (int m = 0; m < RPL * COLS / 4; ++m) ck[m] = c4[m];
        }
    }

    __device__ __forceinline__ void store(BwdStage<DK, NC, SG, EW>& s, int tid) const {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int e = tid + NT * i;
            if (e < BW_SUB * DK) {
                (&s.k[0][0])[e] = in_f32(k[i]);
                if (BWD) (&s.q[0][0])[e] = in_f32(q[i]);
                if (!SG) (&s.a[0][0])[e] = in_f32(a[i]);
                if (EW) (&s.er[0][0])[e] = in_f32(er[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int e = tid + NT * i;
            if (e < BW_SUB * NC) {
                if (LV) (&s.v[0][0])[e] = in_f32(v[i]);
                if (EW) (&s.wr[0][0])[e] = in_f32(wr[i]);
                if (BWD) (&s.dO[0][0])[e] = dO[i];
                if (BWD) (&s.e[0][0])[e] = pr[i];
            }
        }
        if (tid < BW_SUB) {
            s.b[tid] = in_f32(b);
            if (SG) s.a[tid][0] = in_f32(ag);
        }
    }
};

template <class TIn, int DK, int NWV, int COLS, bool SG, bool EW>
__global__ void __launch_bounds__(NWV * WAVE)
chunk_bwd_kernel(BwdParams p) {
    lds_poison((uint32_t)sizeof(BwdLds<DK, NWV * COLS, NWV, SG, EW>));
    constexpr int NT = NWV * WAVE, NC = NWV * COLS, SUB = BW_SUB, NQ = bwd_nq<EW>();
    constexpr int RPL = DK >= WAVE ? DK / WAVE : 1;        // state rows per lane
    constexpr int CKF = NT * RPL * COLS;                    // floats per checkpoint slot
    static_assert(COLS % 4 == 0, "float4 column groups");
    extern __shared__ __align__(16) unsigned char smem[];
    BwdLds<DK, NC, NWV, SG, EW>& L = *reinterpret_cast<BwdLds<DK, NC, NWV, SG, EW>*>(smem);

    const int tid = threadIdx.x, lane = tid % WAVE;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    // the column groups of one (sequence, head) run on one XCD and share its L2
    // for the inputs they all read
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int cg = item % p.ncg, pair = item / p.ncg;
    const int s = pair / p.H, h = pair % p.H;
    int t0, t1, b0;
    long base;
    if (p.cu) {
        t0 = p.cu[s];
        t1 = p.cu[s + 1];
        b0 = 0;
        base = t0 / SUB + s;
    } else {
        t0 = 0;
        t1 = p.T;
        b0 = s;
        base = (long)s * ((p.T + SUB - 1) / SUB);
    }
    const int nb = (t1 - t0 + SUB - 1) / SUB;
    const int cw0 = cg * NC, c0 = cw0 + w * COLS;          // first column of the workgroup / of this wave
    float* ck = p.ckpt + ((size_t)(h * p.ncg + cg) * p.nblk + base) * CKF + (size_t)tid * RPL * COLS;
    const size_t sbase = (size_t)(s * p.H + h) * DK * p.dv;

    bool rv[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) rv[m] = DK >= WAVE || lane < DK;

    float S[RPL][COLS];
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        const int r = lane + WAVE * m;
#pragma unroll
        for (int c4 = 0; c4 < COLS / 4; ++c4) {
            f32x4 x = zero4();
            if (p.S0 && rv[m]) x = *reinterpret_cast<const f32x4*>(p.S0 + sbase + (size_t)r * p.dv + c0 + 4 * c4);
#pragma unroll
            for (int c = 0; c < 4; ++c) S[m][4 * c4 + c] = x[c];
        }
    }

    // Wave-uniform per-token results of block fb, from LDS to memory (pass A: e)
    auto flush_vout = [&](int fb, float* dst, const float (*src)[NC]) {
        const int ts = t0 + fb * SUB;
        const __amdgpu_buffer_rsrc_t r = block_rsrc(dst, (size_t)b0 * p.T + ts, p.H, p.dv);
        for (int e = tid; e < SUB * NC; e += NT) {
            const int j = e / NC, c = e % NC;
            const int off = ts + j < t1 ? ((j * p.H + h) * p.dv + cw0 + c) * 4 : BW_OOB;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(src[j][c]), r, off, 0, 0);
        }
    };
    auto flush_resid = [&](int fb) { flush_vout(fb, p.resid, L.vout[fb & 1]); };

    // ------------------------------------------------ pass A: forward, checkpoints
    {
        BwdFetch<TIn, DK, NC, NT, RPL, COLS, SG, false, EW> f;
        if (nb > 0) f.fetch(p, tid, b0, h, t0, t1, cw0, nullptr);
        for (int blk = 0; blk < nb; ++blk) {
            BwdStage<DK, NC, SG, EW>& st = L.st[blk & 1];
            f.store(st, tid);
            __syncthreads();
            const int ts = t0 + blk * SUB;
            if (blk > 0) flush_resid(blk - 1);
            if (blk + 1 < nb) f.fetch(p, tid, b0, h, ts + SUB, t1, cw0, nullptr);
            f32x4* cp = reinterpret_cast<f32x4*>(ck + (size_t)blk * CKF);
            float* vb = lane == 0 ? &L.vout[blk & 1][0][w * COLS] : &L.junk[4 * lane];
#pragma unroll
            for (int m = 0; m < RPL; ++m)
#pragma unroll
                for (int c4 = 0; c4 < COLS / 4; ++c4)
                    cp[m * (COLS / 4) + c4] = f32x4{S[m][4 * c4], S[m][4 * c4 + 1], S[m][4 * c4 + 2], S[m][4 * c4 + 3]};
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                {
                    float kr[RPL], kx[RPL], part[COLS];   // write key k, read key (k, or e o k)
#pragma unroll
                    for (int m = 0; m < RPL; ++m) {
                        const int r = rv[m] ? lane + WAVE * m : 0;
                        kr[m] = rv[m] ? st.k[j][r] : 0.f;
                        kx[m] = EW ? kr[m] * (rv[m] ? st.er[j][r] : 0.f) : kr[m];
                        const float a = SG ? st.a[j][0] : (rv[m] ? st.a[j][r] : 0.f);
#pragma unroll
                        for (int c = 0; c < COLS; ++c) S[m][c] *= a;
                    }
                    {
                        float x[COLS];
#pragma unroll
                        for (int c = 0; c < COLS; ++c) {
                            x[c] = 0.f;
#pragma unroll
                            for (int m = 0; m < RPL; ++m) x[c] = fmaf(S[m][c], kx[m], x[c]);
                        }
                        wave_sum4(x, part, lane);
                    }
                    static_assert(COLS == 4, "one 16-byte LDS store of e per wave and token");
                    float e[COLS];
#pragma unroll
                    for (int c = 0; c < COLS; ++c) {
                        const float vv = st.v[j][w * COLS + c];
                        e[c] = (EW ? st.wr[j][w * COLS + c] * vv : vv) - part[c];
                    }
                    *reinterpret_cast<f32x4*>(vb + j * NC) = f32x4{e[0], e[1], e[2], e[3]};
                    const float bt = EW ? 1.f : st.b[j];
#pragma unroll
                    for (int c = 0; c < COLS; ++c) {
                        const float u = bt * e[c];
#pragma unroll
                        for (int m = 0; m < RPL; ++m) S[m][c] = fmaf(kr[m], u, S[m][c]);
                    }
                }
            }
        }
    }
    __syncthreads();
    if (nb > 0) flush_resid(nb - 1);
    __syncthreads();   // pass B reads e written by other threads

    // ------------------------------------------------ pass B: adjoint, blocks in reverse
    float dS[RPL][COLS];
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        const int r = lane + WAVE * m;
#pragma unroll
        for (int c4 = 0; c4 < COLS / 4; ++c4) {
            f32x4 x = zero4();
            if (p.dST && rv[m]) x = *reinterpret_cast<const f32x4*>(p.dST + sbase + (size_t)r * p.dv + c0 + 4 * c4);
#pragma unroll
            for (int c = 0; c < 4; ++c) dS[m][4 * c4 + c] = x[c];
        }
    }
    // S after the last token of the block being processed: pass A's final
    // state for the last block (padding tokens are exact no-ops), then each
    // block's checkpoint for the block before it
    float Sn[RPL][COLS];
#pragma unroll
    for (int m = 0; m < RPL; ++m)
#pragma unroll
        for (int c = 0; c < COLS; ++c) Sn[m][c] = S[m][c];
    const size_t nrk = (size_t)p.rows * DK;
    auto flush = [&](int fb) {   // block fb: dv (and dw), and the waves' partial sums added up, to memory
        const int ts = t0 + fb * SUB;
        const size_t tok0 = (size_t)b0 * p.T + ts;
        flush_vout(fb, p.dv_out, L.vout[fb & 1]);
        if constexpr (EW) flush_vout(fb, p.dw_out, L.vout2[fb & 1]);
#pragma unroll
        for (int qty = 0; qty < NQ; ++qty) {
            const __amdgpu_buffer_rsrc_t r = block_rsrc(p.part + ((size_t)cg * NQ + qty) * nrk, tok0, p.H, DK);
#pragma unroll
            for (int i = 0; i < (SUB * DK + NT - 1) / NT; ++i) {
                const int e = tid + NT * i, j = e / DK, ii = e % DK, jj = j < SUB ? j : SUB - 1;
                float x = 0.f;
#pragma unroll
                for (int ww = 0; ww < NWV; ++ww) x += L.slot[fb % L.NSB][ww][jj][qty][ii];
                const int off = e < SUB * DK && ts + j < t1 ? ((j * p.H + h) * DK + ii) * 4 : BW_OOB;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
            }
        }
        if constexpr (!EW) {
            const __amdgpu_buffer_rsrc_t r =
                block_rsrc(p.part + (size_t)p.ncg * 3 * nrk + (size_t)cg * p.rows, tok0, p.H, 1);
            float x = 0.f;
#pragma unroll
            for (int ww = 0; ww < NWV; ++ww) x += L.slotb[fb & 1][ww][tid < SUB ? tid : 0];
            const int off = tid < SUB && ts + tid < t1 ? (tid * p.H + h) * 4 : BW_OOB;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
        }
    };
    {
        BwdFetch<TIn, DK, NC, NT, RPL, COLS, SG, true, EW> f;
        if (nb > 0) f.fetch(p, tid, b0, h, t0 + (nb - 1) * SUB, t1, cw0, ck + (size_t)(nb - 1) * CKF);
        for (int blk = nb - 1; blk >= 0; --blk) {
            BwdStage<DK, NC, SG, EW>& st = L.st[blk & 1];
            f.store(st, tid);
            float Sb[RPL][COLS];
#pragma unroll
            for (int m = 0; m < RPL; ++m)
#pragma unroll
                for (int c = 0; c < COLS; ++c) Sb[m][c] = f.ck[m * (COLS / 4) + c / 4][c % 4];
            __syncthreads();
            if (blk + 1 < nb) flush(blk + 1);
            if constexpr (BwdLds<DK, NC, NWV, SG, EW>::NSB == 1) __syncthreads();   // slot read before rewritten
            const int ts = t0 + blk * SUB;
            if (blk > 0) f.fetch(p, tid, b0, h, ts - SUB, t1, cw0, ck + (size_t)(blk - 1) * CKF);

            // replay the block forward, keeping S_{t-1} and u for every token
            float Sh[SUB][RPL][COLS], uh[SUB][COLS];
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
#pragma unroll
                for (int m = 0; m < RPL; ++m)
#pragma unroll
                    for (int c = 0; c < COLS; ++c) Sh[j][m][c] = Sb[m][c];
                if (j + 1 < SUB) {   // e from pass A: the same values, no reduction
                    float kr[RPL];
#pragma unroll
                    for (int m = 0; m < RPL; ++m) {
                        const int r = rv[m] ? lane + WAVE * m : 0;
                        kr[m] = rv[m] ? st.k[j][r] : 0.f;
                        const float a = SG ? st.a[j][0] : (rv[m] ? st.a[j][r] : 0.f);
#pragma unroll
                        for (int c = 0; c < COLS; ++c) Sb[m][c] *= a;
                    }
                    const float bt = EW ? 1.f : st.b[j];
#pragma unroll
                    for (int c = 0; c < COLS; ++c) {
                        const float u = bt * st.e[j][w * COLS + c];
                        uh[j][c] = u;
#pragma unroll
                        for (int m = 0; m < RPL; ++m) Sb[m][c] = fmaf(kr[m], u, Sb[m][c]);
                    }
                }
            }

            float(*slot)[NQ][DK] = L.slot[blk % L.NSB][w];
            float* vb = lane == 0 ? &L.vout[blk & 1][0][w * COLS] : &L.junk[4 * lane];
            float* wb = EW && lane == 0 ? &L.vout2[blk & 1][0][w * COLS] : &L.junk[4 * lane];
            float* bb = lane == 0 ? &L.slotb[blk & 1][w][0] : &L.junk[lane];
#pragma unroll
            for (int j = SUB - 1; j >= 0; --j) {
                {
                    float kr[RPL], qr[RPL], ar[RPL], er[RPL], oo[COLS], ee[COLS];
#pragma unroll
                    for (int m = 0; m < RPL; ++m) {
                        const int r = rv[m] ? lane + WAVE * m : 0;
                        kr[m] = rv[m] ? st.k[j][r] : 0.f;
                        qr[m] = rv[m] ? st.q[j][r] : 0.f;
                        ar[m] = SG ? st.a[j][0] : (rv[m] ? st.a[j][r] : 0.f);
                        er[m] = EW && rv[m] ? st.er[j][r] : 0.f;
                    }
#pragma unroll
                    for (int c = 0; c < COLS; ++c) {
                        oo[c] = st.dO[j][w * COLS + c];
                        ee[c] = st.e[j][w * COLS + c];
                    }
                    const float bt = EW ? 1.f : st.b[j];
                    float du[COLS];
#pragma unroll
                    for (int m = 0; m < RPL; ++m)
#pragma unroll
                        for (int c = 0; c < COLS; ++c) dS[m][c] = fmaf(qr[m], oo[c], dS[m][c]);
                    {
                        float y[COLS];
#pragma unroll
                        for (int c = 0; c < COLS; ++c) {
                            y[c] = 0.f;
#pragma unroll
                            for (int m = 0; m < RPL; ++m) y[c] = fmaf(dS[m][c], kr[m], y[c]);
                        }
                        wave_sum4(y, du, lane);
                    }
                    // u = beta e; dv = beta du; dpred = -dv. Erase/write form:
                    // u = e; dv = w o du; dw = du o v; dpred = -du
                    float u[COLS], dvv[COLS], dpr[COLS], dww[COLS], dbt = 0.f;
#pragma unroll
                    for (int c = 0; c < COLS; ++c) {
                        u[c] = j + 1 < SUB ? uh[j + 1 < SUB ? j : 0][c] : bt * ee[c];
                        dvv[c] = (EW ? st.wr[j][w * COLS + c] : bt) * du[c];
                        dpr[c] = EW ? du[c] : dvv[c];   // -dpred
                        dww[c] = EW ? du[c] * st.v[j][w * COLS + c] : 0.f;
                        dbt = fmaf(du[c], ee[c], dbt);
                    }
#pragma unroll
                    for (int m = 0; m < RPL; ++m) {
                        float St[COLS];   // S_t
#pragma unroll
                        for (int c = 0; c < COLS; ++c) St[c] = j + 1 < SUB ? Sh[j + 1 < SUB ? j + 1 : 0][m][c] : Sn[m][c];
                        const float kx = EW ? er[m] * kr[m] : kr[m];   // the read key
                        float gq = 0.f, gk = 0.f, gs = 0.f, ga = 0.f;
#pragma unroll
                        for (int c = 0; c < COLS; ++c) {
                            gq = fmaf(St[c], oo[c], gq);
                            gk = fmaf(dS[m][c], u[c], gk);
                            gs = fmaf(Sh[j][m][c], dpr[c], gs);
                            const float dsp = fmaf(-kx, dpr[c], dS[m][c]);   // dS' = dS + kx dpred^T
                            ga = fmaf(dsp, Sh[j][m][c], ga);
                            dS[m][c] = ar[m] * dsp;
                        }
                        const float dke = -ar[m] * gs;   // S' dpred
                        if (rv[m]) {
                            const int r = lane + WAVE * m;
                            slot[j][0][r] = gq;
                            slot[j][1][r] = EW ? fmaf(er[m], dke, gk) : fmaf(-ar[m], gs, gk);
                            slot[j][2][r] = ga;
                            if constexpr (EW) slot[j][EW ? 3 : 0][r] = kr[m] * dke;
                        }
                    }
                    // wave-uniform values, stored by lane 0 without a branch (the other
                    // lanes write a junk area): dbeta and dv, flushed with the block
                    bb[j] = dbt;
                    *reinterpret_cast<f32x4*>(vb + j * NC) = f32x4{dvv[0], dvv[1], dvv[2], dvv[3]};
                    if constexpr (EW) *reinterpret_cast<f32x4*>(wb + j * NC) = f32x4{dww[0], dww[1], dww[2], dww[3]};
                }
            }
#pragma unroll
            for (int m = 0; m < RPL; ++m)
#pragma unroll
                for (int c = 0; c < COLS; ++c) Sn[m][c] = Sh[0][m][c];
        }
    }
    __syncthreads();
    if (nb > 0) flush(0);
    if (p.dS0) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            if (!rv[m]) continue;
            const int r = lane + WAVE * m;
#pragma unroll
            for (int c4 = 0; c4 < COLS / 4; ++c4)
                *reinterpret_cast<f32x4*>(p.dS0 + sbase + (size_t)r * p.dv + c0 + 4 * c4) =
                    f32x4{dS[m][4 * c4], dS[m][4 * c4 + 1], dS[m][4 * c4 + 2], dS[m][4 * c4 + 3]};
        }
    }
}

// Sums the per-workgroup partials: dq, dk, dalpha (and, with nq = 4, de)
// per (token, head, channel) and dbeta per (token, head) (db null: none, the
// erase/write form); the scalar gate's gradient also sums over the channels.
__global__ void __launch_bounds__(256)
chunk_bwd_reduce_kernel(const float* __restrict__ part, long rows, int dk, int ncg, bool sg, int nq,
                        float* __restrict__ dq, float* __restrict__ dkg, float* __restrict__ dg,
                        float* __restrict__ db, float* __restrict__ de) {
    lds_poison(0);
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    const long n = rows * dk;
    if (e < n) {
        float a = 0.f, b = 0.f, c = 0.f, d = 0.f;
        for (int g = 0; g < ncg; ++g) {
            a += part[(size_t)(nq * g) * n + e];
            b += part[(size_t)(nq * g + 1) * n + e];
            if (!sg) c += part[(size_t)(nq * g + 2) * n + e];
            if (nq > 3) d += part[(size_t)(nq * g + 3) * n + e];
        }
        dq[e] = a;
        dkg[e] = b;
        if (!sg) dg[e] = c;
        if (nq > 3) de[e] = d;
    }
    if (e < rows) {
        if (db) {
            float x = 0.f;
            for (int g = 0; g < ncg; ++g) x += part[(size_t)nq * ncg * n + (size_t)g * rows + e];
            db[e] = x;
        }
        if (sg) {
            float y = 0.f;
            for (int g = 0; g < ncg; ++g)
                for (int i = 0; i < dk; ++i) y += part[(size_t)(nq * g + 2) * n + (size_t)e * dk + i];
            dg[e] = y;
        }
    }
}

constexpr int BW_COLS = 4;   // value columns per wave
constexpr int BW_WAVES = 4;  // waves per workgroup: 16 value columns (dv >= 16 always)
int bwd_waves(int) { return BW_WAVES; }

template <class TIn, int DK, int NWV, bool SG, bool EW>
hipError_t launch_bwd_t(const BwdArgs& a, const BwdParams& p) {
    constexpr size_t bytes = sizeof(BwdLds<DK, NWV * BW_COLS, NWV, SG, EW>);
    static_assert(bytes <= 160 * 1024, "backward LDS");
    auto kern = chunk_bwd_kernel<TIn, DK, NWV, BW_COLS, SG, EW>;
    if (bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(a.N * a.H * p.ncg), dim3(NWV * WAVE), bytes, a.stream, p);
    return hipGetLastError();
}

template <class TIn, bool SG, bool EW>
hipError_t launch_bwd_dk(const BwdArgs& a, const BwdParams& p) {
    switch (a.dk) {
        case 16: return launch_bwd_t<TIn, 16, BW_WAVES, SG, EW>(a, p);
        case 32: return launch_bwd_t<TIn, 32, BW_WAVES, SG, EW>(a, p);
        case 64: return launch_bwd_t<TIn, 64, BW_WAVES, SG, EW>(a, p);
        default: return launch_bwd_t<TIn, 128, BW_WAVES, SG, EW>(a, p);
    }
}

template <class TIn, bool SG>
hipError_t launch_bwd_ew(const BwdArgs& a, const BwdParams& p) {
    return a.erase ? launch_bwd_dk<TIn, SG, true>(a, p) : launch_bwd_dk<TIn, SG, false>(a, p);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

long bwd_slots(int B, int T, bool varlen, int N) {
    return varlen ? (long)T / BW_SUB + N : (long)B * ((T + BW_SUB - 1) / BW_SUB);
}

size_t bwd_ckpt_bytes(int H, long slots, int dk, int dv) {
    const int rpl = dk >= WAVE ? dk / WAVE : 1;
    return align256((size_t)H * slots * dv * WAVE * rpl * sizeof(float));
}

// Per-workgroup partial sums: dq, dk, dalpha [ncg][3][rows][dk] and dbeta
// [ncg][rows]; the erase/write form keeps dq, dk, dalpha, de [ncg][4][rows][dk].
size_t bwd_part_bytes(int B, int H, int T, int dk, int dv, bool ew) {
    const int ncg = dv / (bwd_waves(dv) * BW_COLS);
    const size_t rows = (size_t)B * T * H;
    return align256((ew ? (size_t)ncg * 4 * rows * dk : (size_t)ncg * 3 * rows * dk + (size_t)ncg * rows) *
                    sizeof(float));
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int T, int dk, int dv, bool varlen, int N, bool ew) {
    const size_t resid = align256((size_t)B * T * H * dv * sizeof(float));
    return bwd_ckpt_bytes(H, bwd_slots(B, T, varlen, N), dk, dv) + bwd_part_bytes(B, H, T, dk, dv, ew) + resid;
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
    const bool varlen = a.cu_seqlens != nullptr;
    BwdParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.gate = a.gate;
    p.beta = a.beta;
    p.erase = a.erase;
    p.write = a.write;
    p.dw_out = a.g_write;
    p.S0 = a.S0;
    p.dO = a.dO;
    p.dST = a.dST;
    p.dv_out = a.g_v;
    p.dS0 = a.g_S0;
    p.cu = a.cu_seqlens;
    p.H = a.H;
    p.T = a.T;
    p.dv = a.dv;
    p.ncg = a.dv / (bwd_waves(a.dv) * BW_COLS);
    p.nblk = bwd_slots(a.B, a.T, varlen, a.N);
    p.rows = (long)a.B * a.T * a.H;
    char* ws = static_cast<char*>(a.workspace);
    p.ckpt = reinterpret_cast<float*>(ws);
    const bool ew = a.erase != nullptr;
    p.part = reinterpret_cast<float*>(ws + bwd_ckpt_bytes(a.H, p.nblk, a.dk, a.dv));
    p.resid = reinterpret_cast<float*>(ws + bwd_ckpt_bytes(a.H, p.nblk, a.dk, a.dv) +
                                      bwd_part_bytes(a.B, a.H, a.T, a.dk, a.dv, ew));
    hipError_t e = a.bf16 ? (a.scalar_gate ? launch_bwd_ew<uint16_t, true>(a, p) : launch_bwd_ew<uint16_t, false>(a, p))
                          : (a.scalar_gate ? launch_bwd_ew<float, true>(a, p) : launch_bwd_ew<float, false>(a, p));
    if (e != hipSuccess || p.rows == 0) return e;
    const long n = p.rows * a.dk;
    hipLaunchKernelGGL(chunk_bwd_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, a.stream, p.part,
                       p.rows, a.dk, p.ncg, a.scalar_gate, ew ? 4 : 3, a.g_q, a.g_k, a.g_gate,
                       ew ? nullptr : a.g_beta, ew ? a.g_erase : nullptr);
    return hipGetLastError();
}

}  // namespace kda
