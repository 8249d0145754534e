// 3D RoPE tables and the fused rotate + block mean-pool kernel.
//
// RoLA (arXiv 2609.06712v3) §3 "3D RoPE", eq. 1: the head is split across
// the t, h, w axes; each axis rotates its own pairs by (coordinate) x
// (its frequency), so scores depend on per-axis offsets only. §4.2 reuses
// the backbone's cos/sin tensors in the low-rank branch, so the tables
// built here serve both branches.
#include "slr_common.h"
#include "slr_launch.h"

namespace slr {

// (cos, sin) of p * base^(-2j/(2n)) for every axis coordinate p and pair j,
// evaluated in fp64 and rounded once to fp32.
__global__ void k_rope_tables(float2* __restrict__ tab, int T, int Hg, int Wg, int nt, int nh, int nw,
                              double base) {
    const int n_t = T * nt, n_h = Hg * nh, n_w = Wg * nw;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n_t + n_h + n_w; e += gridDim.x * blockDim.x) {
        int p, j, n;
        if (e < n_t) {
            p = e / nt; j = e % nt; n = nt;
        } else if (e < n_t + n_h) {
            p = (e - n_t) / nh; j = (e - n_t) % nh; n = nh;
        } else {
            p = (e - n_t - n_h) / nw; j = (e - n_t - n_h) % nw; n = nw;
        }
        double theta = pow(base, -2.0 * (double)j / (2.0 * (double)n));
        double a = (double)p * theta;
        tab[e] = make_float2((float)cos(a), (float)sin(a));
    }
}

template <typename TIO> struct Io8;
template <> struct Io8<uint16_t> {
    // 8 bf16 values as fp32
    static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
        u32x4_t w = ldg16(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[2 * i] = bf_lo(w[i]); x[2 * i + 1] = bf_hi(w[i]); }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float* x) {
        u32x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf2(x[2 * i], x[2 * i + 1]);
        stg16(p, w);
    }
};
template <> struct Io8<float> {
    static __device__ __forceinline__ void load(const float* p, float* x) {
        f32x4_t a = *reinterpret_cast<const f32x4_t*>(p), b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
    }
    static __device__ __forceinline__ void store(float* p, const float* x) {
        f32x4_t a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) { a[i] = x[i]; b[i] = x[4 + i]; }
        *reinterpret_cast<f32x4_t*>(p) = a;
        *reinterpret_cast<f32x4_t*>(p + 4) = b;
    }
};

// One workgroup = one block of `bs` tokens of one (b, h) slice, for q and
// (optionally) k. Thread layout: 8 consecutive dims (4 pairs) of one token
// row per thread, D/8 threads per row, 256/(D/8) rows per pass.
// Writes the rotated rows when q_out / k_out are non-null (rows in
// [L, out_rows) of the block are written as zeros, which pads the workspace
// copy to whole blocks; the q copy is multiplied by qscale before rounding)
// and, when qbar is non-null, the block means of the fp32 rotated values
// over valid tokens (not scaled).
//
// Tiled mode (bf16, D = 128, 64-token blocks; the layout the block-sparse
// flash kernel streams): instead of a plain copy, rotated k and the
// transposed v of every block go to one contiguous 32 KB tile
// kv_tiles[bh][blk] = [ K part 16 KB | V^T part 16 KB ] in operand order:
// every 1 KB chunk is one wave's MFMA operand, lane l's 16 bytes at l * 16.
//   K chunk (kh, s), kh = key half, s = 16-dim step:
//       lane l holds K[key 32kh + l%32][dims 16s + 8(l/32) .. +7]
//   V^T chunk (kh, db, h2), db = 32-dim block, h2 = 16-key group of the half:
//       lane l holds V[keys (slot16 order) 32kh + 16h2 + 8(l/32) .. +7][dim 32db + l%32]
// Keys past L are zero.
template <typename TIO, int D, int BS, bool TWO, bool TILED>
__global__ __launch_bounds__(256) void k_rope_pool(const TIO* __restrict__ q, const TIO* __restrict__ k,
                                                   TIO* __restrict__ q_out, TIO* __restrict__ k_out,
                                                   float* __restrict__ qbar, float* __restrict__ kbar,
                                                   const float2* __restrict__ tab, RopeGeom g, long L,
                                                   long out_rows, int nblk, const TIO* __restrict__ v,
                                                   uint16_t* __restrict__ kv_tiles, float qscale) {
    constexpr int CH = D / 8;          // threads per row
    constexpr int RPP = 256 / CH;      // rows per pass
    constexpr int bs = BS;
    constexpr bool two = TWO;
    const int tid = threadIdx.x;
    const int c = tid % CH, rsub = tid / CH;
    const int blk = blockIdx.x;
    const long bh = blockIdx.y;

    // table entry of the 4 pairs this thread owns: base + (axis coordinate) * stride
    int pax[4], pbase[4], pstride[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int p = 4 * c + e;
        int a = 0, j = p;
        if (p >= g.np[0] + g.np[1]) { a = 2; j = p - g.np[0] - g.np[1]; }
        else if (p >= g.np[0]) { a = 1; j = p - g.np[0]; }
        pax[e] = a;
        pbase[e] = (a == 0 ? g.tab_off[0] : a == 1 ? g.tab_off[1] : g.tab_off[2]) + j;
        pstride[e] = a == 0 ? g.np[0] : a == 1 ? g.np[1] : g.np[2];
    }

    float sq[8], sk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { sq[i] = 0.f; sk[i] = 0.f; }

    const TIO* qs = q + bh * L * D;
    const TIO* ks = two ? k + bh * L * D : nullptr;
    TIO* qo = q_out ? q_out + bh * out_rows * D : nullptr;
    TIO* ko = (two && k_out) ? k_out + bh * out_rows * D : nullptr;
    uint16_t* tile = TILED ? kv_tiles + (bh * nblk + blk) * (long)kTileElems : nullptr;

    // All loads of the block first (rows past L are clamped to row L - 1 and
    // zeroed after), then the table gathers, then the arithmetic: no load
    // waits on another.
    constexpr int MAXP = BS / RPP;   // passes over the block
    constexpr int npass = MAXP;
    float xq[MAXP][8], xk[MAXP][8];
    float2 cs[MAXP][4];
    // V^T (tiled mode): thread tid < 128 takes 8 keys x 8 dims (keys = slots
    // 8vh..8vh+7 of 16-group vG); it transposes them in registers and stores
    // 8 rows of 16 bytes at the end
    // (threads 128..255 load the same rows as tid - 128, so the loads are not
    // under a divergent branch; those repeats are served by the caches)
    const int vc = tid & 15, vg = (tid >> 4) & 7, vG = vg >> 1, vh = vg & 1;
    uint32_t vrows[TILED ? 8 : 1][4];
    if (TILED) {
        const uint16_t* vs = reinterpret_cast<const uint16_t*>(v) + bh * L * D;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const long l = (long)blk * 64 + 16 * vG + 4 * vh + (e & 3) + 8 * (e >> 2);
            const u32x4_t w = ldg16(vs + (l < L ? l : L - 1) * D + 8 * vc);
#pragma unroll
            for (int i = 0; i < 4; ++i) vrows[e][i] = l < L ? w[i] : 0u;
        }
    }
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p < npass) {
            const long l = (long)blk * bs + p * RPP + rsub;
            const long lc = l < L ? l : L - 1;
            Io8<TIO>::load(qs + lc * D + 8 * c, xq[p]);
            if (two) Io8<TIO>::load(ks + lc * D + 8 * c, xk[p]);
        }
    }
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p < npass) {
            const long l = (long)blk * bs + p * RPP + rsub;
            int ct, chh, cw;
            token_coords(l < L ? l : L - 1, g.Hg, g.Wg, ct, chh, cw);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int cv = pax[e] == 2 ? cw : (pax[e] == 1 ? chh : ct);
                cs[p][e] = tab[pbase[e] + cv * pstride[e]];
            }
        }
    }
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p < npass) {
            const long l = (long)blk * bs + p * RPP + rsub;
            if (l >= out_rows) continue;
            const bool valid = l < L;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x0 = xq[p][2 * e], x1 = xq[p][2 * e + 1];
                xq[p][2 * e] = valid ? x0 * cs[p][e].x - x1 * cs[p][e].y : 0.f;
                xq[p][2 * e + 1] = valid ? x0 * cs[p][e].y + x1 * cs[p][e].x : 0.f;
                if (two) {
                    x0 = xk[p][2 * e]; x1 = xk[p][2 * e + 1];
                    xk[p][2 * e] = valid ? x0 * cs[p][e].x - x1 * cs[p][e].y : 0.f;
                    xk[p][2 * e + 1] = valid ? x0 * cs[p][e].y + x1 * cs[p][e].x : 0.f;
                } else {
#pragma unroll
                    for (int i = 0; i < 2; ++i) xk[p][2 * e + i] = 0.f;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) { sq[i] += xq[p][i]; sk[i] += xk[p][i]; }
            if (qo) {
                float xs[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) xs[i] = xq[p][i] * qscale;
                Io8<TIO>::store(qo + l * D + 8 * c, xs);
            }
            if (TILED) {
                const int r = p * RPP + rsub;   // key within the block; dims 8c .. 8c+7 = step c/2, lane half c%2
                const int kh = r >> 5, ln = (r & 31) + 32 * (c & 1);
                Io8<TIO>::store(reinterpret_cast<TIO*>(tile + ((kh * 8 + (c >> 1)) * 64 + ln) * 8), xk[p]);
            } else if (ko) {
                Io8<TIO>::store(ko + l * D + 8 * c, xk[p]);
            }
        }
    }

    if (TILED && tid < 128) {
        static_assert(!TILED || (D == 128 && sizeof(TIO) == 2), "tiled layout is bf16, D = 128");
        uint16_t* vt = tile + 64 * D;
        const int kh = vG >> 1, h2 = vG & 1;   // 16-key group vG = 2kh + h2, lane half vh
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            u32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t a0 = vrows[2 * i][f >> 1], a1 = vrows[2 * i + 1][f >> 1];
                o[i] = (f & 1) ? __builtin_amdgcn_perm(a1, a0, 0x07060302u)
                               : __builtin_amdgcn_perm(a1, a0, 0x05040100u);
            }
            const int d = 8 * vc + f;
            const int ln = (d & 31) + 32 * vh;
            stg16(vt + ((kh * 8 + (d >> 5) * 2 + h2) * 64 + ln) * 8, o);
        }
    }

    if (qbar == nullptr) return;
    // block means: reduce the RPP row groups through LDS, fixed order
    __shared__ float red[2][RPP][D];
#pragma unroll
    for (int i = 0; i < 8; ++i) { red[0][rsub][8 * c + i] = sq[i]; red[1][rsub][8 * c + i] = sk[i]; }
    __syncthreads();
    const long lo = (long)blk * bs;
    const long hi = lo + bs < L ? lo + bs : L;
    const float inv = 1.f / (float)(hi - lo);
    for (int e = tid; e < (two ? 2 : 1) * D; e += 256) {
        const int which = e / D, d = e % D;
        float s = 0.f;
        for (int r = 0; r < RPP; ++r) s += red[which][r][d];
        float* dst = which ? kbar : qbar;
        dst[(bh * nblk + blk) * D + d] = s * inv;
    }
}

// ---- launchers ----------------------------------------------------------
hipError_t launch_rope_tables(float2* tab, const RopeGeom& g, double base, hipStream_t st) {
    const int n = g.T * g.np[0] + g.Hg * g.np[1] + g.Wg * g.np[2];
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_rope_tables, dim3((n + 255) / 256), dim3(256), 0, st, tab, g.T, g.Hg, g.Wg, g.np[0],
                       g.np[1], g.np[2], base);
    return hipGetLastError();
}

template <typename TIO, int D, int BS, bool TWO>
static hipError_t rope_pool_t(const void* q, const void* k, void* qo, void* ko, float* qbar, float* kbar,
                              const float2* tab, const RopeGeom& g, long BH, long L, long out_rows, int nblk,
                              hipStream_t st, float qscale) {
    dim3 grid((unsigned)nblk, (unsigned)BH);
    hipLaunchKernelGGL((k_rope_pool<TIO, D, BS, TWO, false>), grid, dim3(256), 0, st, (const TIO*)q, (const TIO*)k,
                       (TIO*)qo, (TIO*)ko, qbar, kbar, tab, g, L, out_rows, nblk, (const TIO*)nullptr,
                       (uint16_t*)nullptr, qscale);
    return hipGetLastError();
}

template <typename TIO, int D>
static hipError_t rope_pool_d(const void* q, const void* k, void* qo, void* ko, float* qbar, float* kbar,
                              const float2* tab, const RopeGeom& g, long BH, long L, long out_rows, int bs,
                              int nblk, hipStream_t st, float qs) {
    if (bs == 32)
        return k ? rope_pool_t<TIO, D, 32, true>(q, k, qo, ko, qbar, kbar, tab, g, BH, L, out_rows, nblk, st, qs)
                 : rope_pool_t<TIO, D, 32, false>(q, k, qo, ko, qbar, kbar, tab, g, BH, L, out_rows, nblk, st, qs);
    return k ? rope_pool_t<TIO, D, 64, true>(q, k, qo, ko, qbar, kbar, tab, g, BH, L, out_rows, nblk, st, qs)
             : rope_pool_t<TIO, D, 64, false>(q, k, qo, ko, qbar, kbar, tab, g, BH, L, out_rows, nblk, st, qs);
}

hipError_t launch_rope_pool_tiled(const void* q, const void* k, const void* v, void* qo, uint16_t* kv_tiles,
                                  float* qbar, float* kbar, const float2* tab, const RopeGeom& g, long BH, long L,
                                  int nblk, float qscale, hipStream_t st) {
    dim3 grid((unsigned)nblk, (unsigned)BH);
    hipLaunchKernelGGL((k_rope_pool<uint16_t, 128, 64, true, true>), grid, dim3(256), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (uint16_t*)qo, (uint16_t*)nullptr, qbar, kbar, tab, g, L,
                       (long)nblk * 64, nblk, (const uint16_t*)v, kv_tiles, qscale);
    return hipGetLastError();
}

hipError_t launch_rope_pool(int dtype_bf16, int D, const void* q, const void* k, void* qo, void* ko, float* qbar,
                            float* kbar, const float2* tab, const RopeGeom& g, long BH, long L, long out_rows,
                            int bs, int nblk, hipStream_t st, float qs) {
    if (dtype_bf16) {
        if (D == 64)
            return rope_pool_d<uint16_t, 64>(q, k, qo, ko, qbar, kbar, tab, g, BH, L, out_rows, bs, nblk, st, qs);
        return rope_pool_d<uint16_t, 128>(q, k, qo, ko, qbar, kbar, tab, g, BH, L, out_rows, bs, nblk, st, qs);
    }
    if (D == 64) return rope_pool_d<float, 64>(q, k, qo, ko, qbar, kbar, tab, g, BH, L, out_rows, bs, nblk, st, qs);
    return rope_pool_d<float, 128>(q, k, qo, ko, qbar, kbar, tab, g, BH, L, out_rows, bs, nblk, st, qs);
}

}  // namespace slr
