// Block-sparse (and dense) flash attention with the low-rank readout and the
// gated combine fused into the epilogue, for the layer shapes outside the
// persistent tiled kernel (fp32 layers; bf16 with D = 64 or 32-token blocks).
//
// RoLA (arXiv 2609.06712v3) §4.1: exact softmax attention of each query
// block over the tokens of its kept key blocks; App. A Algorithm 1: the
// layer output adds the gated low-rank readout rho(w)^T S / (w . z + eps),
// w = phi(q W_q) from the raw q (§4.3); App. F: the sparse branch dominates
// the cost. Dense attention (§3 "Full attention") is the same loop over
// every key block.
//
// bf16 layers, per workgroup = one query block of BS rows, BS/32 waves of
// 32 query rows each. Scores are computed transposed, S^T = K Q^T, with the
// 32x32x16 bf16 MFMA: each lane then owns one query row (l % 32) and 16 of
// its keys per 32-key sub-block, so the online softmax (fp32, exp2 domain)
// needs one cross-lane step (lane ^ 32) per tile. O^T = V^T P^T is the
// second MFMA; the probabilities go straight from the score accumulator
// into the B operand because V^T is staged in LDS with keys in the same
// slot16 order. K and V^T tiles live in LDS (padded rows: conflict-free
// 16-byte reads); the next kept tile is fetched into registers while the
// current one is consumed.
#include "slr_common.h"
#include "slr_epilogue.h"
#include "slr_launch.h"

namespace slr {

template <int D, int BS, int RP, int LR, bool DENSE>
__global__ __launch_bounds__(BS * 2) void k_flash_bf16(FlashArgs a) {
    constexpr int NT = BS * 2;          // threads (BS/32 waves)
    constexpr int KLD = D + 8;          // K tile row stride (elements)
    constexpr int VLD = BS + 8;         // V^T tile row stride (elements)
    constexpr int NKB = BS / 32;        // 32-key sub-blocks per tile
    constexpr int NS = D / 16;          // k-steps over d
    constexpr int NDB = D / 32;         // 32-dim blocks of the output
    constexpr int KCH = D / 8;          // 16-byte chunks per row
    constexpr int KRPP = NT / KCH;      // K rows loaded per pass
    constexpr int KPASS = BS / KRPP;
    constexpr int VBLK = (BS / 8) * (D / 8);  // 8x8 V blocks per tile
    static_assert(VBLK <= NT, "one 8x8 V block per thread");
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[BS * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VLD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const long bh = wid / a.nblk;
    const int qb = (int)(wid % a.nblk);
    const int head = (int)(bh % a.H);
    const long rows = (long)a.nblk * BS;
    const long L = a.L;

    const uint16_t* qr = (const uint16_t*)a.qr + (bh * rows + (long)qb * BS + 32 * wave) * D;
    const uint16_t* kr = (const uint16_t*)a.kr + bh * rows * D;
    const uint16_t* vg = (const uint16_t*)a.v + bh * L * D;
    const int32_t* ix = DENSE ? nullptr : a.idx + (bh * a.nblk + qb) * (long)a.keep;
    const int ntile = DENSE ? a.nblk : a.keep;

    // B operand of S^T = K Q^T: q row l32, dims 16s + 8hf + e
    u32x4_t qop[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) qop[s] = ldg16(qr + l32 * D + 16 * s + 8 * hf);

    // tile loader assignment
    const int kc = tid % KCH, kr0 = tid / KCH;
    const int vc = tid % (D / 8), vgp = tid / (D / 8);
    const int vG = vgp >> 1, vh = vgp & 1;
    const bool vload = tid < VBLK;
    u32x4_t kreg[KPASS], vreg[8];

    auto fetch = [&](int j) {
        const uint16_t* kt = kr + (long)j * BS * D;
#pragma unroll
        for (int i = 0; i < KPASS; ++i) kreg[i] = ldg16(kt + (long)(kr0 + KRPP * i) * D + 8 * kc);
        if (vload) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const long row = (long)j * BS + 16 * vG + 4 * vh + (e & 3) + 8 * (e >> 2);
                vreg[e] = row < L ? ldg16(vg + row * D + 8 * vc) : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < KPASS; ++i)
            *reinterpret_cast<u32x4_t*>(k_lds + (kr0 + KRPP * i) * KLD + 8 * kc) = kreg[i];
        if (vload) {
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                u32x4_t o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a0 = vreg[2 * i][f >> 1], a1 = vreg[2 * i + 1][f >> 1];
                    o[i] = (f & 1) ? __builtin_amdgcn_perm(a1, a0, 0x07060302u)
                                   : __builtin_amdgcn_perm(a1, a0, 0x05040100u);
                }
                *reinterpret_cast<u32x4_t*>(vt_lds + (8 * vc + f) * VLD + 16 * vG + 8 * vh) = o;
            }
        }
    };

    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = a.scale * kLog2e;
    const bool ragged = (L % BS) != 0;

    int j = DENSE ? 0 : ix[0];
    fetch(j);
    stash();
    __syncthreads();

    for (int n = 0; n < ntile; ++n) {
        const int jn = (n + 1 < ntile) ? (DENSE ? n + 1 : ix[n + 1]) : -1;
        if (jn >= 0) fetch(jn);

        // ---- S^T = K Q^T over this tile
        f32x16_t sacc[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(k_lds + (32 * kb + l32) * KLD + 16 * s + 8 * hf);
                sacc[kb] = mfma32(ka, qop[s], sacc[kb]);
            }
        }
        // ---- online softmax (log2 domain); lane holds query l32
        const bool mask = ragged && j == a.nblk - 1;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = sacc[kb][i] * sl2;
                if (mask) {
                    const long key = (long)j * BS + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (key >= L) x = -INFINITY;
                }
                sacc[kb][i] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, wave_xor32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        u32x4_t pop[NKB][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = fast_exp2(sacc[kb][8 * h2 + 2 * i] - m_new);
                    const float p1 = fast_exp2(sacc[kb][8 * h2 + 2 * i + 1] - m_new);
                    l_run += p0 + p1;
                    pop[kb][h2][i] = pack_bf2(p0, p1);
                }
        // ---- O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const u32x4_t va =
                        *reinterpret_cast<const u32x4_t*>(vt_lds + (32 * db + l32) * VLD + 32 * kb + 16 * h2 + 8 * hf);
                    oacc[db] = mfma32(va, pop[kb][h2], oacc[db]);
                }
        __syncthreads();
        if (jn >= 0) {
            stash();
            j = jn;
        }
        __syncthreads();
    }

    flash_epilogue<D, RP, LR>(a, bh, head, (long)qb * BS + 32 * wave, l_run + wave_xor32(l_run), oacc);
}


// fp32 layers: one thread per query row, K / V tiles staged in LDS, fp32
// VALU throughout (the precision the tiny fp32 check layer asks for).
template <int D, int RP, int LR, bool DENSE>
__global__ __launch_bounds__(64) void k_flash_f32(FlashArgs a, int BS) {
    __shared__ float k_lds[64][D + 1];
    __shared__ float v_lds[64][D];
    const int tid = threadIdx.x;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const long bh = wid / a.nblk;
    const int qb = (int)(wid % a.nblk);
    const int head = (int)(bh % a.H);
    const long rows = (long)a.nblk * BS;
    const long L = a.L;
    const float* qr = (const float*)a.qr + (bh * rows + (long)qb * BS) * D;
    const float* kr = (const float*)a.kr + bh * rows * D;
    const float* vv = (const float*)a.v + bh * L * D;
    const int32_t* ix = DENSE ? nullptr : a.idx + (bh * a.nblk + qb) * (long)a.keep;
    const int ntile = DENSE ? a.nblk : a.keep;
    const bool act = tid < BS;

    float q[D], o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) { q[d] = act ? qr[(long)tid * D + d] : 0.f; o[d] = 0.f; }
    float m_run = -INFINITY, l_run = 0.f;
    for (int n = 0; n < ntile; ++n) {
        const int j = DENSE ? n : ix[n];
        __syncthreads();
        for (int e = tid; e < BS * D; e += 64) {
            const int r = e / D, d = e % D;
            const long row = (long)j * BS + r;
            k_lds[r][d] = kr[row * D + d];
            v_lds[r][d] = row < L ? vv[row * D + d] : 0.f;
        }
        __syncthreads();
        float s[64];
        float mx = -INFINITY;
        for (int r = 0; r < BS; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc += q[d] * k_lds[r][d];
            acc *= a.scale;
            if ((long)j * BS + r >= L) acc = -INFINITY;
            s[r] = acc;
            mx = fmaxf(mx, acc);
        }
        const float m_new = fmaxf(m_run, mx);
        const float alpha = expf(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
        for (int r = 0; r < BS; ++r) {
            const float p = expf(s[r] - m_new);
            l_run += p;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] += p * v_lds[r][d];
        }
        m_run = m_new;
    }
    const long qrow = (long)qb * BS + tid;
    if (!act || qrow >= L) return;
    const float inv = 1.f / l_run;
    float* out = (float*)a.out + (bh * L + qrow) * D;
    float* osp = a.o_sp ? (float*)a.o_sp + (bh * L + qrow) * D : nullptr;
    float* olr = a.o_lr ? (float*)a.o_lr + (bh * L + qrow) * D : nullptr;
    if (LR == 0) {
        for (int d = 0; d < D; ++d) {
            out[d] = o[d] * inv;
            if (osp) osp[d] = o[d] * inv;
        }
        return;
    }
    const int R = a.g.R;
    const float* qraw = (const float*)a.q + (bh * L + qrow) * D;
    const float* W = a.wq + (long)head * D * R;
    int crd[3];
    token_coords(qrow, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
    float w[RP], f[RP];
    float den = 0.f;
    for (int r = 0; r < RP; ++r) {
        float x = 0.f;
        if (r < R) {
            for (int d = 0; d < D; ++d) x += qraw[d] * W[d * R + r];
            if (LR == 2) x += a.Et[crd[0] * R + r] + a.Eh[crd[1] * R + r] + a.Ew[crd[2] * R + r];
        }
        w[r] = r < R ? phi_elu1(x) : 0.f;
        den += r < R ? w[r] * a.zp[bh * R + r] : 0.f;
    }
    for (int r = 0; r < RP; r += 2) {
        if (LR == 1 && r < R) {
            const float2 cs = lr_cossin_q(a.tab, a.g, r >> 1, crd);
            f[r] = w[r] * cs.x - w[r + 1] * cs.y;
            f[r + 1] = w[r] * cs.y + w[r + 1] * cs.x;
        } else {
            f[r] = w[r];
            f[r + 1] = w[r + 1];
        }
    }
    const float rd = 1.f / (den + a.eps);
    const float gs = a.gate[head];
    const float* S = a.S + bh * (long)R * D;
    for (int d = 0; d < D; ++d) {
        float num = 0.f;
        for (int r = 0; r < R; ++r) num += f[r] * S[(long)r * D + d];
        const float sp = o[d] * inv, lr = num * rd;
        out[d] = sp + gs * lr;
        if (osp) osp[d] = sp;
        if (olr) olr[d] = lr;
    }
}

// ---- launcher ------------------------------------------------------------
template <int D, int BS, int RP, int LR, bool DENSE>
static hipError_t flash_bf16_t(const FlashArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_flash_bf16<D, BS, RP, LR, DENSE>), dim3((unsigned)a.nwg), dim3(BS * 2), 0, st, a);
    return hipGetLastError();
}

template <int D, int BS, int RP>
static hipError_t flash_bf16_mode(int lr_mode, bool dense, const FlashArgs& a, hipStream_t st) {
    if (dense) return flash_bf16_t<D, BS, RP, 0, true>(a, st);
    if (lr_mode == 1) return flash_bf16_t<D, BS, RP, 1, false>(a, st);
    if (lr_mode == 2) return flash_bf16_t<D, BS, RP, 2, false>(a, st);
    return flash_bf16_t<D, BS, RP, 0, false>(a, st);
}

template <int D, int RP>
static hipError_t flash_f32_t(int lr_mode, bool dense, const FlashArgs& a, int BS, hipStream_t st) {
    dim3 grid((unsigned)a.nwg);
    if (dense)
        hipLaunchKernelGGL((k_flash_f32<D, RP, 0, true>), grid, dim3(64), 0, st, a, BS);
    else if (lr_mode == 1)
        hipLaunchKernelGGL((k_flash_f32<D, RP, 1, false>), grid, dim3(64), 0, st, a, BS);
    else if (lr_mode == 2)
        hipLaunchKernelGGL((k_flash_f32<D, RP, 2, false>), grid, dim3(64), 0, st, a, BS);
    else
        hipLaunchKernelGGL((k_flash_f32<D, RP, 0, false>), grid, dim3(64), 0, st, a, BS);
    return hipGetLastError();
}

hipError_t launch_flash(int dtype_bf16, int D, int BS, int RP, int lr_mode, bool dense, const FlashArgs& a, long BH,
                        hipStream_t st) {
    (void)BH;
    if (!dtype_bf16) {
        if (D == 64) return RP == 64 ? flash_f32_t<64, 64>(lr_mode, dense, a, BS, st)
                                     : flash_f32_t<64, 32>(lr_mode, dense, a, BS, st);
        return RP == 64 ? flash_f32_t<128, 64>(lr_mode, dense, a, BS, st)
                        : flash_f32_t<128, 32>(lr_mode, dense, a, BS, st);
    }
    if (D == 128 && BS == 64)
        return RP == 64 ? flash_bf16_mode<128, 64, 64>(lr_mode, dense, a, st)
                        : flash_bf16_mode<128, 64, 32>(lr_mode, dense, a, st);
    if (D == 128 && BS == 32)
        return RP == 64 ? flash_bf16_mode<128, 32, 64>(lr_mode, dense, a, st)
                        : flash_bf16_mode<128, 32, 32>(lr_mode, dense, a, st);
    if (D == 64 && BS == 64)
        return RP == 64 ? flash_bf16_mode<64, 64, 64>(lr_mode, dense, a, st)
                        : flash_bf16_mode<64, 64, 32>(lr_mode, dense, a, st);
    return RP == 64 ? flash_bf16_mode<64, 32, 64>(lr_mode, dense, a, st)
                    : flash_bf16_mode<64, 32, 32>(lr_mode, dense, a, st);
}

}  // namespace slr
