// Device-side building blocks shared by the gated delta-rule kernels (gfx950).
//
// MFMA fragment convention used throughout (16x16 output tiles, 32-deep K
// steps, 64-lane wavefronts):
//   lane l = 16*g + i   (g = l / 16 in 0..3, i = l % 16)
//   A operand (16 rows x 32 K): lane holds row i, 8 values at K positions
//       kpos(g, p), p = 0..7
//   B operand (32 K x 16 cols): lane holds column i, the same 8 K positions
//   C/D (16 x 16 fp32):          lane holds column i, rows 4g .. 4g+3
// with kpos(g, p) = 4g + p for p < 4 and 16 + 4g + (p - 4) for p >= 4.
// The K order inside a step does not change a product as long as A and B
// agree, and this particular order makes two vertically stacked D tiles a
// ready B operand: a state or update matrix held in accumulator registers
// feeds the next contraction without an LDS round trip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

namespace kda {

constexpr int WAVE = 64;
constexpr int NXCD = 8;   // accelerator complex dies; consecutive workgroups round-robin over them

__host__ __device__ constexpr int kpos(int g, int p) { return p < 4 ? 4 * g + p : 12 + 4 * g + p; }

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <class TIn> __device__ __forceinline__ float ld_in(const TIn* p);
template <> __device__ __forceinline__ float ld_in<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }
template <> __device__ __forceinline__ float ld_in<float>(const float* p) { return *p; }

// Power-of-two scale for a block of values whose largest magnitude is m >= 0:
// m * scale lies in [0.5, 1). The exponent is clamped to [2^-62, 2^62] so that
// products and inverses of two scales stay normal fp32 numbers; blocks with
// m < 2^-63 are scaled up by 2^62 only, and m >= 2^78 is outside the range the
// fp16 operand path represents. Read straight from the exponent bits.
__device__ __forceinline__ int scale_exp(float m) {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);
    return min(max(e, 64), 188);
}
__device__ __forceinline__ float pow2_scale_for(float m) { return __uint_as_float((uint32_t)(253 - scale_exp(m)) << 23); }
__device__ __forceinline__ float pow2_inv_scale_for(float m) { return __uint_as_float((uint32_t)(scale_exp(m) + 1) << 23); }

// max(|a|, |b|, |c|) in one instruction (the compiler does not always fuse
// the chains itself)
__device__ __forceinline__ float absmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// Largest |x| over the eight values of two D-tile quads.
__device__ __forceinline__ float absmax8(const f32x4& a, const f32x4& b) {
    float m = absmax3(a[0], a[1], a[2]);
    m = absmax3(m, a[3], b[0]);
    m = absmax3(m, b[1], b[2]);
    return absmax3(m, b[3], b[3]);
}

// Largest value over the four lanes that hold one column of a 16x16 D tile
// (lanes i, i+16, i+32, i+48): two lane-swap steps, no LDS round trip. For
// v >= +0 (maxima of |x|, the only use): non-negative floats order as their
// bit patterns, so integer maxima do it without float canonicalisation.
__device__ __forceinline__ float colmax4(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t m = a[0] > a[1] ? a[0] : a[1];
    const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    return __uint_as_float(b[0] > b[1] ? b[0] : b[1]);
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4 mma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 operands: eight 16x16x4 steps; step m takes position m of every lane
// group, which covers the 32 K positions once each.
__device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
    for (int m = 0; m < 8; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Split an fp32 value into bf16 hi + lo (hi + lo carries 16 mantissa bits).
struct bf16pair { bf16x8 hi, lo; };
__device__ __forceinline__ bf16pair split8(const f32x8& x) {
    bf16pair r;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        __bf16 h = (__bf16)x[p];
        r.hi[p] = h;
        r.lo[p] = (__bf16)(x[p] - (float)h);
    }
    return r;
}

__device__ __forceinline__ f16x8 to_f16x8(const f32x8& x, float s) {
    f16x8 r;
#pragma unroll
    for (int p = 0; p < 8; ++p) r[p] = (_Float16)(x[p] * s);
    return r;
}

// Two stacked D tiles (rows 0-15 and 16-31 of a 32-deep K step) as the 8
// values of a B fragment, per the kpos order.
__device__ __forceinline__ f32x8 dtiles_to_frag(const f32x4& top, const f32x4& bot) {
    return f32x8{top[0], top[1], top[2], top[3], bot[0], bot[1], bot[2], bot[3]};
}

// ---------------------------------------------------------------- buffer resources
// A raw buffer descriptor (gfx9 family) over `bytes` bytes at `base`. Loads
// and stores through it take a 32-bit per-lane offset plus scalar offsets,
// and accesses past `bytes` are dropped by the hardware (stores) or return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------- wave reductions

// v from lane CTRL's DPP source within each row of 16 lanes
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum over the wave of v >= +0 (maxima of |x|), in every lane: within
// each row of 16 lanes by DPP (swap neighbours, swap pairs, mirror halves of
// 8, mirror the row), then across the four rows with colmax4; integer maxima
// on the bit patterns, no LDS round trips.
__device__ __forceinline__ float wave_max(float v) {
    uint32_t u = __float_as_uint(v), t;
    t = dpp_row<0xB1>(u);  u = u > t ? u : t;   // quad_perm [1,0,3,2]
    t = dpp_row<0x4E>(u);  u = u > t ? u : t;   // quad_perm [2,3,0,1]
    t = dpp_row<0x141>(u); u = u > t ? u : t;   // row_half_mirror
    t = dpp_row<0x140>(u); u = u > t ? u : t;   // row_mirror
    return colmax4(__uint_as_float(u));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
}

// ---------------------------------------------------------------- XCD-aware work order
// Workgroup ids are dispatched round-robin over the XCDs. Renumber them so
// that consecutive work items (e.g. the value-column slices of one head) land
// on one XCD and share its L2. A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int L, int total) {
    const int per = total / NXCD, rem = total % NXCD;
    const int x = L % NXCD, j = L / NXCD;
    return x * per + (x < rem ? x : rem) + j;
}

// ---------------------------------------------------------------- LDS poisoning (debug build)
// Built with -DKDA_LDS_POISON, every kernel first fills its workgroup's whole
// LDS allocation (static, then dyn_bytes of dynamic) with 0xFFFFFFFF -- a NaN
// as fp32 and as each fp16 or bf16 half -- so that a read of LDS the kernel
// has not written first turns into NaN in its results. Every thread calls it
// before anything else; in the normal build it does nothing.
__device__ __forceinline__ void lds_poison(uint32_t dyn_bytes) {
#ifdef KDA_LDS_POISON
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    const uint32_t total = __builtin_amdgcn_groupstaticsize() + dyn_bytes;
    const uint32_t nt = blockDim.x * blockDim.y * blockDim.z;
    for (uint32_t off = 4 * threadIdx.x; off < total; off += 4 * nt) *(lds_u32*)off = 0xFFFFFFFFu;
    __syncthreads();
#else
    (void)dyn_bytes;
#endif
}

}  // namespace kda
