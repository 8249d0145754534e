// Block-sparse (and dense) flash attention with the low-rank readout and the
// gated combine fused into the epilogue.
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
// accuracy), combines with the gate and stores bf16 rows. The gate is the
// head's scalar, or (token gate, RoLA §4.4) sigmoid(q . W_g + b_g) of the
// token's raw query row times RMS(O_sparse) / (RMS(O_lowrank) + eps), both
// RMS over the head dims of the row.
// FAV: 0 = elu + 1 / SiLU features only, 1 = FAVOR+ features only, 2 = either (picked from a.g.fmap).
template <int D, int RP, int LR, int FAV = 2>
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
        const bool fav = FAV == 2 ? a.g.fmap == 2 : FAV == 1;
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
        // FAVOR+: |p|^2 of the row's projection p = q W_q [+ E] (this lane's
        // 16 ranks of each block, then the pair lane's)
        float sq = 0.f;
        if (fav) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = 32 * rb + 8 * (i >> 2) + 4 * hf + (i & 3);
                    const bool ok = qval && r < a.g.R;
                    float x = wacc[rb][i];
                    if (LR == 2 && ok) x += a.Et[crd[0] * a.g.R + r] + a.Eh[crd[1] * a.g.R + r] + a.Ew[crd[2] * a.g.R + r];
                    x = ok ? x : 0.f;
                    sq += x * x;
                }
            sq = sum_xor32(sq);
        }
        const float rsr = 1.f / sqrtf((float)a.g.R);
        const int na = a.g.rope.T + a.g.rope.Hg + a.g.rope.Wg;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            float w[16];
            // FAVOR+ exponent omega_c . (q W_q) = q . (W_q omega^T)_c for this
            // rank block, hi and lo weight parts (q re-read: L2-resident)
            f32x16_t yacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) yacc[i] = 0.f;
            if (fav) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const u32x4_t qo2 = qval ? ldg16(qraw + 16 * s + 8 * hf) : u32x4_t{0u, 0u, 0u, 0u};
                    const long wo = ((long)head * RP + 32 * rb + l32) * D + 16 * s + 8 * hf;
                    yacc = mfma32(ldg16(a.wqot_hi + wo), qo2, yacc);
                    yacc = mfma32(ldg16(a.wqot_lo + wo), qo2, yacc);
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 32 * rb + 8 * (i >> 2) + 4 * hf + (i & 3);
                const bool ok = qval && r < a.g.R;
                if (fav) {
                    float y = yacc[i];
                    if (LR == 2 && ok) {
                        const float* eoh = a.g.eo + (long)head * na * a.g.R + r;
                        y += eoh[crd[0] * a.g.R] + eoh[(a.g.rope.T + crd[1]) * a.g.R] +
                             eoh[(a.g.rope.T + a.g.rope.Hg + crd[2]) * a.g.R];
                    }
                    w[i] = ok ? __builtin_amdgcn_exp2f((y - 0.5f * sq) * kLog2e) * rsr : 0.f;
                } else {
                    float x = wacc[rb][i];
                    if (LR == 2 && ok) x += a.Et[crd[0] * a.g.R + r] + a.Eh[crd[1] * a.g.R + r] + a.Ew[crd[2] * a.g.R + r];
                    w[i] = ok ? phi_feat(a.g.fmap, x) : 0.f;
                }
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
        // sign-indefinite SiLU features (fmap 1): the readout is the mean over the L tokens
        rden = a.g.fmap == 1 ? 1.f / (float)L : 1.f / (den + a.eps);
        if (a.gate_mode == 0) {
            gsc = a.gate[head];
        } else {
            // token gate logit: this lane's dims 16s + 8hf .. +7, then the pair lane's
            float t = 0.f;
            if (qval) {
                const float* wgh = a.wg + (long)head * D;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const u32x4_t qv = ldg16(qraw + 16 * s + 8 * hf);
                    const float4 w0 = *reinterpret_cast<const float4*>(wgh + 16 * s + 8 * hf);
                    const float4 w1 = *reinterpret_cast<const float4*>(wgh + 16 * s + 8 * hf + 4);
                    t += bf_lo(qv[0]) * w0.x + bf_hi(qv[0]) * w0.y + bf_lo(qv[1]) * w0.z + bf_hi(qv[1]) * w0.w;
                    t += bf_lo(qv[2]) * w1.x + bf_hi(qv[2]) * w1.y + bf_lo(qv[3]) * w1.z + bf_hi(qv[3]) * w1.w;
                }
            }
            gsc = 1.f / (1.f + __expf(-(sum_xor32(t) + a.bg[head])));
        }
    }
    uint16_t* out = (uint16_t*)a.out + (bh * L + (qval ? qrow : 0)) * D;
    uint16_t* osp = a.o_sp ? (uint16_t*)a.o_sp + (bh * L + (qval ? qrow : 0)) * D : nullptr;
    uint16_t* olr = a.o_lr ? (uint16_t*)a.o_lr + (bh * L + (qval ? qrow : 0)) * D : nullptr;
    // num^T = S^T rho(w)^T, one 32-dim block per accumulator (m = d, k = r, n = query)
    f32x16_t nall[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        f32x16_t& nacc = nall[db];
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
    }
    if (LR != 0 && a.gate_mode != 0) {
        // token gate: scale the low-rank rows to the sparse rows' RMS
        float ss = 0.f, sl = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float xs = oacc[db][i] * inv, xl = nall[db][i] * rden;
                ss += xs * xs;
                sl += xl * xl;
            }
        ss = sum_xor32(ss);
        sl = sum_xor32(sl);
        gsc *= sqrtf(ss * (1.f / D)) / (sqrtf(sl * (1.f / D)) + a.eps);
    }
    // combine, store
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const f32x16_t& nacc = nall[db];
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

    const float lrow = l_run + wave_xor32(l_run);
    // training forward: log2 of the row's softmax normaliser over its scaled scores
    if (a.lse && hf == 0 && (long)qb * BS + 32 * wave + l32 < L)
        a.lse[bh * L + (long)qb * BS + 32 * wave + l32] = m_run + __log2f(lrow);
    flash_epilogue<D, RP, LR>(a, bh, head, (long)qb * BS + 32 * wave, lrow, oacc);
}


// ---------------------------------------------------------------------------
// Streaming variant for bf16, D = 128, 64-token blocks (every workload shape).
//
// Each kept key block is one contiguous 32 KB tile in operand order (see the
// rotate kernel): a 16 KB K part and a 16 KB V^T part whose 1 KB chunks are
// each one wave's MFMA operand, so the LDS image equals the memory image and
// is filled by direct global-to-LDS copies with no repacking. Workgroup = 4
// waves = one 64-row query block; wave (rh, kh) owns query rows 32rh.. and
// keys 32kh.. of every tile, with S^T = K Q^T computed so that each lane holds
// one query row. The K and V^T parts stream through separate LDS rings (K
// three deep, V^T two deep; one barrier per tile). The key halves of each row
// are merged once at the end through LDS. q comes pre-scaled into log2 units
// and the score accumulator starts at minus the row's reference, so the
// common tile needs only exp2 of the MFMA results; the reference moves only
// when a tile's probabilities could overflow, so the accumulator rescale is
// rare.

// Online softmax of one 32-row block's scores -> bf16 probabilities, exp2
// domain. q arrives multiplied by 1/sqrt(D) * log2(e) and the score
// accumulator of a tile starts at -m_run (0 while the row has no reference
// yet: m_run = -inf), so s already holds score - reference in log2 units and
// p = exp2(s) needs no max or FMA. The reference is raised only when some
// probability of the tile could exceed ~2^36 (its sum passes 2^40, or is not
// finite), and set from the tile when the row has none; O and l are scaled
// by the same factor, so the result after normalisation is unchanged. negm
// holds -m_run (0 without a reference) in all 16 accumulator slots: it is
// the C operand of a tile's first score MFMA and changes only with m_run.
__device__ __forceinline__ void softmax_tile(f32x16_t& s, f32x16_t* o, float& m_run, float& l_run, u32x4_t* pop,
                                             f32x16_t& negm) {
    float p[16];
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(s[i]);
        l += p[i];
    }
    const bool noref = m_run == -INFINITY;
    if (__ballot(!(l <= 1.0995116e12f) || noref)) {
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
        mx = max_xor32(mx);
        // shift of the reference: to the tile max for a row without one (it
        // stays -inf while every key seen is masked), else up to the tile max
        // when that is higher
        const float shift = noref ? mx : fmaxf(mx, 0.f);
        const bool none = shift == -INFINITY;
        const float ref = noref ? 0.f : m_run;
        const float alpha = noref ? 0.f : fast_exp2(-shift);
        m_run = none ? -INFINITY : ref + shift;
        {
            const float init = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
            for (int i = 0; i < 16; ++i) negm[i] = init;
        }
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        l = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = none ? 0.f : fast_exp2(s[i] - shift);
            l += p[i];
        }
    }
    l_run += l;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) pop[h2][i] = pack_bf2(p[8 * h2 + 2 * i], p[8 * h2 + 2 * i + 1]);
}

// Eight 16-byte LDS reads (1 KB apart) into registers; the block waits for
// them itself, so no read is left in flight when it ends (early-clobber
// outputs: no destination can alias the address register the later reads use).
__device__ __forceinline__ void lds_read8(u32x4_t* r, const uint16_t* lds_base) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)lds_base;
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\t"
        "ds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\t"
        "ds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a)
        : "memory");
}

template <int RP, int LR, bool DENSE, bool FAV = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_flash_tiled(
    FlashArgs a, const int32_t* __restrict__ idx_all, const uint16_t* __restrict__ kvt_all) {
    constexpr int D = 128, BS = 64;
    constexpr int PART = kTileElems / 2;                 // K or V^T part of a tile (elements)
    constexpr int PLOADS = PART * 2 / (256 * 16);        // 16-byte copies per thread per part (4)
    // K ring (3 parts) | V^T ring (2 parts), 80 KB; the start is reused as the
    // key-half exchange area at the end
    __shared__ __attribute__((aligned(16))) uint16_t lds[5 * PART];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rh = wave & 1, kh = wave >> 1;
    const int l32 = lane & 31, hf = lane >> 5;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const long bh = wid / a.nblk;
    const int qb = (int)(wid % a.nblk);
    const int head = (int)(bh % a.H);
    const long L = a.L;
    const int nblk = a.nblk;
    const uint16_t* tiles = kvt_all + bh * (long)nblk * kTileElems + (long)tid * 8;
    const int32_t* ix = DENSE ? nullptr : idx_all + (bh * nblk + qb) * (long)a.keep;
    const int ntile = DENSE ? nblk : a.keep;
    auto tile_of = [&](int n) -> int { return DENSE ? n : ix[n]; };

    // B operand of S^T = K Q^T: query row 32rh + l32 of the block
    u32x4_t qop[8];
    const uint16_t* qr = (const uint16_t*)a.qr + (bh * (long)nblk * BS + (long)qb * BS + 32 * rh + l32) * D + 8 * hf;
#pragma unroll
    for (int s = 0; s < 8; ++s) qop[s] = ldg16(qr + 16 * s);
    wait_vmcnt<0>();

    // part (0 = K, 1 = V^T) of tile j -> LDS: the LDS image equals the memory
    // image (operand order)
    auto issue = [&](int j, int part, uint16_t* dst) {
        const uint16_t* src = tiles + (long)j * kTileElems + part * PART;
#pragma unroll
        for (int m = 0; m < PLOADS; ++m)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(src + m * 256 * 8),
                (__attribute__((address_space(3))) void*)(dst + (m * 256 + wave * 64) * 8), 16, 0, 0);
    };
    const int rd = ((kh * 8) * 64 + lane) * 8;   // this lane's operand chunks (kh, 0..7) within a part

    f32x16_t oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;   // reference (log2 units), partial row sum
    f32x16_t negm;                           // -m_run (0 without a reference): C of the first score MFMA
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = 0.f;
    const bool ragged = (L % BS) != 0;

    // K of tile t lives in K slot t % 3, V^T in V slot t % 2. The barrier that
    // opens tile t also certifies that every wave is done with tile t - 1, so
    // V^T of t + 1 and K of t + 2 are requested into those slots right away:
    // K parts land two tiles ahead (they are needed first), V^T parts one.
    issue(tile_of(0), 0, lds);
    issue(tile_of(0), 1, lds + 3 * PART);
    if (ntile > 1) issue(tile_of(1), 0, lds + PART);
    int ks = 0;   // K slot of tile t
    for (int t = 0; t < ntile; ++t) {
        const int jcur = tile_of(t);
        // outstanding in issue order: ..., V^T(t), K(t + 1) -> keep K(t + 1) in flight
        if (t + 1 < ntile) wait_vmcnt<PLOADS>(); else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (t + 1 < ntile) issue(tile_of(t + 1), 1, lds + (3 + ((t + 1) & 1)) * PART);
        if (t + 2 < ntile) issue(tile_of(t + 2), 0, lds + (ks == 0 ? 2 : ks - 1) * PART);
        const uint16_t* kcur = lds + ks * PART;
        const uint16_t* vcur = lds + (3 + (t & 1)) * PART;
        ks = ks == 2 ? 0 : ks + 1;
        u32x4_t op[8], vop[8];
        lds_read8(op, kcur + rd);                 // K chunks (kh, s)
        __builtin_amdgcn_s_setprio(1);   // matrix phase first when two waves share a SIMD
        // First score MFMA with C = -m into a distinct accumulator (the builtin
        // form makes the compiler copy negm into the accumulator first). Its
        // inputs are old: op from an asm read that waited for itself, qop from
        // loads waited before the loop, negm written a tile earlier at most;
        // the next MFMA reads the result as C with exact overlap, which the
        // hardware chains back to back.
        f32x16_t sacc;
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(sacc) : "v"(op[0]), "v"(qop[0]), "v"(negm));
#pragma unroll
        for (int s = 1; s < 8; ++s) sacc = mfma32(op[s], qop[s], sacc);
        __builtin_amdgcn_s_setprio(0);
        // V^T chunks (kh, db, h2): read while the score MFMAs run, into
        // registers other than the K operands those MFMAs still read
        lds_read8(vop, vcur + rd);
        asm volatile("" ::"v"(op[0]), "v"(op[1]), "v"(op[2]), "v"(op[3]), "v"(op[4]), "v"(op[5]), "v"(op[6]),
                     "v"(op[7]));
        if (ragged && jcur == nblk - 1) {
            const long key0 = (long)jcur * BS + 32 * kh;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key0 + 8 * (i >> 2) + 4 * hf + (i & 3) >= L) sacc[i] = -INFINITY;
        }
        u32x4_t pop[2];
        softmax_tile(sacc, oacc, m_run, l_run, pop, negm);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) oacc[db] = mfma32(vop[db * 2 + h2], pop[h2], oacc[db]);
        __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    float (*mrg)[66 * 64] = reinterpret_cast<float (*)[66 * 64]>(&lds[0]);

    // ---- merge the two key halves of each row half through LDS
    float* m_lds = mrg[rh];
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) m_lds[(16 * db + i) * 64 + lane] = oacc[db][i];
        m_lds[64 * 64 + lane] = m_run;
        m_lds[65 * 64 + lane] = l_run;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = m_lds[64 * 64 + lane], l1 = m_lds[65 * 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float f0 = fast_exp2(m_run - m), f1 = fast_exp2(m1 - m);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = oacc[db][i] * f0 + m_lds[(16 * db + i) * 64 + lane] * f1;
    const float lsum = sum_xor32(l_run * f0 + l1 * f1);
    // training forward: log2 of the row's softmax normaliser (q arrives in log2 units)
    if (a.lse && hf == 0 && (long)qb * BS + 32 * rh + l32 < L)
        a.lse[bh * L + (long)qb * BS + 32 * rh + l32] = m + __log2f(lsum);
    flash_epilogue<D, RP, LR, FAV ? 1 : 0>(a, bh, head, (long)qb * BS + 32 * rh, lsum, oacc);
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
    if (a.lse) a.lse[bh * L + qrow] = (m_run + logf(l_run)) * kLog2e;   // log2 of the normaliser
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
        w[r] = r < R ? (a.g.fmap == 2 ? x : phi_feat(a.g.fmap, x)) : 0.f;
    }
    if (a.g.fmap == 2) {
        // FAVOR+: w_c = exp(omega_c . p - |p|^2 / 2) / sqrt(R) of the projection p (held in w)
        float sq = 0.f;
        for (int r = 0; r < R; ++r) sq += w[r] * w[r];
        const float* om = a.g.omega + (long)head * R * R;
        for (int c = 0; c < R; ++c) {
            float y = 0.f;
            for (int j = 0; j < R; ++j) y += om[c * R + j] * w[j];
            f[c] = expf(y - 0.5f * sq) / sqrtf((float)R);
        }
        for (int c = 0; c < R; ++c) w[c] = f[c];
    }
    for (int r = 0; r < R; ++r) den += w[r] * a.zp[bh * R + r];
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
    const float rd = a.g.fmap == 1 ? 1.f / (float)L : 1.f / (den + a.eps);
    const float* S = a.S + bh * (long)R * D;
    float gs;
    if (a.gate_mode == 0) {
        gs = a.gate[head];
    } else {
        // token gate (RoLA §4.4): sigmoid(q . W_g + b_g) * RMS(O_sparse) / (RMS(O_lowrank) + eps)
        const float* wgh = a.wg + (long)head * D;
        float t = a.bg[head], ss = 0.f, sl = 0.f;
        for (int d = 0; d < D; ++d) t += qraw[d] * wgh[d];
        for (int d = 0; d < D; ++d) {
            float num = 0.f;
            for (int r = 0; r < R; ++r) num += f[r] * S[(long)r * D + d];
            const float sp = o[d] * inv, lr = num * rd;
            ss += sp * sp;
            sl += lr * lr;
        }
        gs = 1.f / (1.f + expf(-t)) * sqrtf(ss / D) / (sqrtf(sl / D) + a.eps);
    }
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

template <int RP>
static hipError_t flash_tiled_t(int lr_mode, bool dense, const FlashArgs& a, hipStream_t st) {
    dim3 grid((unsigned)a.nwg), blk(256);
    if (dense) hipLaunchKernelGGL((k_flash_tiled<RP, 0, true>), grid, blk, 0, st, a, a.idx, a.kvt);
    else if (lr_mode == 1 && a.g.fmap == 2)
        hipLaunchKernelGGL((k_flash_tiled<RP, 1, false, true>), grid, blk, 0, st, a, a.idx, a.kvt);
    else if (lr_mode == 2 && a.g.fmap == 2)
        hipLaunchKernelGGL((k_flash_tiled<RP, 2, false, true>), grid, blk, 0, st, a, a.idx, a.kvt);
    else if (lr_mode == 1) hipLaunchKernelGGL((k_flash_tiled<RP, 1, false>), grid, blk, 0, st, a, a.idx, a.kvt);
    else if (lr_mode == 2) hipLaunchKernelGGL((k_flash_tiled<RP, 2, false>), grid, blk, 0, st, a, a.idx, a.kvt);
    else hipLaunchKernelGGL((k_flash_tiled<RP, 0, false>), grid, blk, 0, st, a, a.idx, a.kvt);
    return hipGetLastError();
}

hipError_t launch_flash(int dtype_bf16, int D, int BS, int RP, int lr_mode, bool dense, const FlashArgs& a, long BH,
                        hipStream_t st) {
    (void)BH;
    if (dtype_bf16 && D == 128 && BS == 64 && a.kvt)
        return RP == 64 ? flash_tiled_t<64>(lr_mode, dense, a, st) : flash_tiled_t<32>(lr_mode, dense, a, st);
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
