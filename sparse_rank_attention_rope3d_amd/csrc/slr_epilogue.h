// Low-rank readout + gated combine epilogue shared by the attention kernels
// of libslr (internal header).
//
// RoLA (arXiv 2609.06712v3) App. A Algorithm 1 and §4.3-§4.4: the layer
// output adds the gated low-rank readout rho(w)^T S / (w . z + eps) with
// w = phi(q W_q) from the raw q; the absolute-PE variant (RoPeSLR, arXiv
// 2605.20659, abstract) adds per-axis tables before phi and skips rho.
#pragma once

#include "slr_common.h"
#include "slr_launch.h"

namespace slr {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float2 lr_cossin_q(const float2* __restrict__ tab, const LrGeom& g, int pr,
                                              const int* crd) {
    int a, j;
    if (pr < g.lp[0]) { a = 0; j = pr; }
    else if (pr < g.lp[0] + g.lp[1]) { a = 1; j = pr - g.lp[0]; }
    else { a = 2; j = pr - g.lp[0] - g.lp[1]; }
    return tab[g.rope.tab_off[a] + crd[a] * g.rope.np[a] + j];
}


// Epilogue shared by the flash kernels: lane owns query row q0 + l32 and the
// O^T accumulator dims 32db + 8(i/4) + 4hf + i%4. Normalises the sparse
// branch, evaluates the low-rank readout rho(w)^T S / (w . z + eps) with
// w = phi(q W_q [+ E]) on MFMA (hi/lo bf16 splits of w and S for ~fp32
// accuracy), combines with the per-head gate and stores bf16 rows.
template <int D, int RP, int LR>
__device__ __forceinline__ void flash_epilogue(const FlashArgs& a, long bh, int head, long q0, float lsum,
                                               const f32x16_t* oacc) {
    constexpr int NS = D / 16;
    constexpr int NDB = D / 32;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
    const long L = a.L;
    const long qrow = q0 + l32;
    const bool qval = qrow < L;
    const float inv = 1.f / lsum;
    float gsc = 0.f, rden = 0.f;
    constexpr int NRB = RP / 32;
    u32x4_t whi[NRB][2], wlo[NRB][2];
    if (LR != 0) {
        const uint16_t* qraw = (const uint16_t*)a.q + (bh * L + (qval ? qrow : 0)) * D;
        f32x16_t wacc[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 16; ++i) wacc[rb][i] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const u32x4_t qo2 = qval ? ldg16(qraw + 16 * s + 8 * hf) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const u32x4_t wa = ldg16(a.wqt + ((long)head * RP + 32 * rb + l32) * D + 16 * s + 8 * hf);
                wacc[rb] = mfma32(wa, qo2, wacc[rb]);
            }
        }
        int crd[3] = {0, 0, 0};
        if (qval) token_coords(qrow, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
        const float* zp = a.zp + bh * RP;
        float den = 0.f;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            float w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 32 * rb + 8 * (i >> 2) + 4 * hf + (i & 3);
                const bool ok = qval && r < a.g.R;
                float x = wacc[rb][i];
                if (LR == 2 && ok) x += a.Et[crd[0] * a.g.R + r] + a.Eh[crd[1] * a.g.R + r] + a.Ew[crd[2] * a.g.R + r];
                w[i] = ok ? phi_elu1(x) : 0.f;
                den += w[i] * zp[r];
            }
            if (LR == 1) {
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const int r = 32 * rb + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (qval && r < a.g.R) {
                        const float2 cs = lr_cossin_q(a.tab, a.g, r >> 1, crd);
                        const float w0 = w[i], w1 = w[i + 1];
                        w[i] = w0 * cs.x - w1 * cs.y;
                        w[i + 1] = w0 * cs.y + w1 * cs.x;
                    }
                }
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a0 = w[8 * h2 + 2 * i], a1 = w[8 * h2 + 2 * i + 1];
                    const uint32_t hi = pack_bf2(a0, a1);
                    whi[rb][h2][i] = hi;
                    wlo[rb][h2][i] = pack_bf2(a0 - bf_lo(hi), a1 - bf_hi(hi));
                }
        }
        den = sum_xor32(den);
        rden = 1.f / (den + a.eps);
        gsc = a.gate[head];
    }
    uint16_t* out = (uint16_t*)a.out + (bh * L + (qval ? qrow : 0)) * D;
    uint16_t* osp = a.o_sp ? (uint16_t*)a.o_sp + (bh * L + (qval ? qrow : 0)) * D : nullptr;
    uint16_t* olr = a.o_lr ? (uint16_t*)a.o_lr + (bh * L + (qval ? qrow : 0)) * D : nullptr;
    // one 32-dim block at a time: num^T = S^T rho(w)^T (m = d, k = r, n = query), combine, store
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        f32x16_t nacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) nacc[i] = 0.f;
        if (LR != 0) {
            const long so = (bh * D + 32 * db + l32) * RP + 8 * hf;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const u32x4_t sh = ldg16(a.st_hi + so + 32 * rb + 16 * h2);
                    const u32x4_t sl = ldg16(a.st_lo + so + 32 * rb + 16 * h2);
                    nacc = mfma32(sh, whi[rb][h2], nacc);
                    nacc = mfma32(sh, wlo[rb][h2], nacc);
                    nacc = mfma32(sl, whi[rb][h2], nacc);
                }
        }
        if (qval) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * db + 8 * g4 + 4 * hf;
                float vs[4], vl[4], vo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vs[i] = oacc[db][4 * g4 + i] * inv;
                    vl[i] = LR != 0 ? nacc[4 * g4 + i] * rden : 0.f;
                    vo[i] = vs[i] + gsc * vl[i];
                }
                *reinterpret_cast<u32x2_t*>(out + d0) = u32x2_t{pack_bf2(vo[0], vo[1]), pack_bf2(vo[2], vo[3])};
                if (osp)
                    *reinterpret_cast<u32x2_t*>(osp + d0) = u32x2_t{pack_bf2(vs[0], vs[1]), pack_bf2(vs[2], vs[3])};
                if (olr)
                    *reinterpret_cast<u32x2_t*>(olr + d0) = u32x2_t{pack_bf2(vl[0], vl[1]), pack_bf2(vl[2], vl[3])};
            }
        }
    }
}


}  // namespace slr
