// Device helpers shared by the gfx950 kernels of libslr.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16x2 (a in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2bf(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// ---- MFMA: D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16) ----------------
// Lane l supplies A[m = l%32][k-slot 8*(l/32)+e] and B[k-slot 8*(l/32)+e][n = l%32]
// for e = 0..7 (any fixed map of k-slots to contraction indices works as long
// as A and B agree). Result: lane l, reg v holds D[m = 8*(v/4) + 4*(l/32) + v%4][n = l%32].
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// fp32 MFMA: D(16x16) += A(16x4) * B(4x16); lane l supplies A[l%16][k=l/16], B[k=l/16][l%16];
// result lane l, reg v holds D[m = 4*(l/16) + v][n = l%16].
__device__ __forceinline__ f32x4_t mfma16f32(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- wave helpers --------------------------------------------------------
__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }
// Pairwise reductions of lanes l and l ^ 32 with v_permlane32_swap (a VALU
// op, no LDS round trip): the swap exchanges one 32-lane half between its
// two operands, so combining both results gives every lane f(x[l], x[l^32]).
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
// Swap with the adjacent lane (l ^ 1) through DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float lane_swap1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// s_waitcnt with only the vector-memory counter constrained (<= N outstanding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Order-preserving key of a float (larger float -> larger key); -0 maps to +0.
__device__ __forceinline__ uint32_t ordered_key(float f) {
    f = f + 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// phi(x) = elu(x) + 1
__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : expf(x); }
// the same with the hardware exp2 (relative error ~1e-7 for the x <= 0 branch; bf16 paths)
__device__ __forceinline__ float phi_elu1_fast(float x) {
    return x > 0.f ? x + 1.f : __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
// SiLU(x) = x / (1 + exp(-x)) (exp(-x) = inf for very negative x gives -0)
__device__ __forceinline__ float phi_silu(float x) { return x / (1.f + expf(-x)); }
__device__ __forceinline__ float phi_silu_fast(float x) {
    return x / (1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}
// per-component feature map of the low-rank branch: 0 = elu + 1, 1 = SiLU
// (FAVOR+, 2, mixes the components and is computed by the kernels themselves)
__device__ __forceinline__ float phi_feat(int fmap, float x) { return fmap == 1 ? phi_silu(x) : phi_elu1(x); }
__device__ __forceinline__ float phi_feat_fast(int fmap, float x) {
    return fmap == 1 ? phi_silu_fast(x) : phi_elu1_fast(x);
}

// Grid coordinates of token l + delta given those of token l (t-major, then
// h, then w), without divisions.
__device__ __forceinline__ void coords_advance(int& t, int& h, int& w, int delta, int Hg, int Wg) {
    w += delta;
    while (w >= Wg) {
        w -= Wg;
        if (++h == Hg) { h = 0; ++t; }
    }
}

// The same for 0 <= delta < Wg (at most one wrap of w), branch free.
__device__ __forceinline__ void coords_step(int& t, int& h, int& w, int delta, int Hg, int Wg) {
    w += delta;
    const bool ww = w >= Wg;
    w -= ww ? Wg : 0;
    h += ww ? 1 : 0;
    const bool hw = h >= Hg;
    h -= hw ? Hg : 0;
    t += hw ? 1 : 0;
}

// Position of key/token x (0..15) inside a 16-slot group in the order
// {0,1,2,3,8,9,10,11,4,5,6,7,12,13,14,15}: lane half h of a 32x32x16 MFMA
// holds slots 8h..8h+7, which is the order the 32x32 accumulator keeps rows
// (8*(v/4) + 4*h + v%4), so an accumulator can feed the next MFMA directly.
__host__ __device__ __forceinline__ int slot16(int x) {
    return (x & 3) | (((x >> 3) & 1) << 2) | (((x >> 2) & 1) << 3);
}

// Geometry of the 3D rotary schedule: per-axis pair counts and the offsets of
// the per-axis (cos, sin) tables, laid out [axis_len][pairs_axis].
struct RopeGeom {
    int T, Hg, Wg;
    int np[3];
    int tab_off[3];
};

__device__ __forceinline__ void token_coords(long l, int Hg, int Wg, int& t, int& h, int& w) {
    // token indices (padded rows included) stay below 2^32: 32-bit unsigned division
    const uint32_t lu = (uint32_t)l, hw = (uint32_t)Hg * (uint32_t)Wg;
    const uint32_t tq = lu / hw, rem = lu - tq * hw, hq = rem / (uint32_t)Wg;
    t = (int)tq;
    h = (int)hq;
    w = (int)(rem - hq * (uint32_t)Wg);
}

// Work-item order that keeps each XCD on a contiguous range of
// (slice, query block): hardware hands workgroup p to XCD p % 8.
__device__ __forceinline__ long xcd_remap(long p, long n) {
    const long per = n / 8, rem = n % 8, x = p % 8, loc = p / 8;
    return x * per + (x < rem ? x : rem) + loc;
}

// Fully pipelined global loads / LDS access as 16-byte vectors.
__device__ __forceinline__ u32x4_t ldg16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void stg16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

}  // namespace slr
