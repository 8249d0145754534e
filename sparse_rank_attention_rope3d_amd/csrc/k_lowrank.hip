// Low-rank global branch: the reusable per-head summary.
//
// RoLA (arXiv 2609.06712v3) §4.1 / App. B.1: the global context is one
// query-independent sum per head, O(L r D). §4.2-4.3: features are
// u = phi(k W_k) (phi = elu + 1, position-free content), rotated after phi
// by the backbone's first rotary pairs of each axis; RoPeSLR (arXiv
// 2605.20659) abstract: the absolute-PE variant adds E_t[t]+E_h[h]+E_w[w]
// before phi and does not rotate. S = sum f v^T, z = sum u over the L valid
// tokens.
//
// bf16 layers: u = K W_k on bf16 MFMA (exact products, fp32 sums); phi, the
// rotation and z in fp32; S = sum f v^T on bf16 MFMA with f split into
// bf16 hi + lo parts (about 16 mantissa bits), fp32 accumulation.
// Split-L partials [BH][nsplit][RP*D + RP] are reduced in a fixed order, so
// results are bitwise reproducible.
#include <atomic>

#include "slr_common.h"
#include "slr_launch.h"

namespace slr {

// W [H][D][R] fp32 -> Wt [H][RP][D] bf16 (transposed, rows r >= R zero).
__global__ void k_lr_prep(const float* __restrict__ W, uint16_t* __restrict__ Wt, int H, int D, int R, int RP) {
    const long n = (long)H * RP * D;
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
        const int d = (int)(e % D);
        const int r = (int)((e / D) % RP);
        const long h = e / ((long)D * RP);
        Wt[e] = r < R ? f2bf(W[(h * D + d) * R + r]) : (uint16_t)0;
    }
}

// FAVOR+ projections (positive random features of the exponential kernel,
// RoPeSLR appendix): the feature exponent omega_c . (x W) is x . (W omega^T)_c,
// so one more projection matrix per side serves it on MFMA. Writes
// (W omega^T)^T [H][RP][D] as bf16 hi + lo parts (about 16 mantissa bits;
// rows c >= R zero), W rounded to bf16 first for bf16 layers (the layer uses
// the rounded W), sums over j in fp32.
__global__ void k_lr_prep_favor(const float* __restrict__ W, const float* __restrict__ omega, int round_bf16, int H,
                                int D, int R, int RP, uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
    const long n = (long)H * RP * D;
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
        const int d = (int)(e % D);
        const int c = (int)((e / D) % RP);
        const long h = e / ((long)D * RP);
        float s = 0.f;
        if (c < R) {
            const float* wr = W + (h * D + d) * R;
            const float* om = omega + (h * R + c) * R;
            for (int j = 0; j < R; ++j) {
                const float w = round_bf16 ? bf2f(f2bf(wr[j])) : wr[j];
                s = fmaf(w, om[j], s);
            }
        }
        const uint16_t h16 = f2bf(s);
        hi[e] = h16;
        lo[e] = f2bf(s - bf2f(h16));
    }
}

// FAVOR+ with absolute PE: eo[h][n][c] = sum_j omega[h][c][j] E[n][j] over the
// concatenated axis tables n in [0, T + Hg + Wg) (E_t rows, then E_h, E_w).
__global__ void k_lr_prep_favor_e(const float* __restrict__ Et, const float* __restrict__ Eh,
                                  const float* __restrict__ Ew, const float* __restrict__ omega, int H, int T,
                                  int Hg, int Wg, int R, float* __restrict__ eo) {
    const int na = T + Hg + Wg;
    const long n = (long)H * na * R;
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
        const int c = (int)(e % R);
        const int row = (int)((e / R) % na);
        const long h = e / ((long)R * na);
        const float* er = row < T ? Et + (long)row * R : row < T + Hg ? Eh + (long)(row - T) * R
                                                                        : Ew + (long)(row - T - Hg) * R;
        const float* om = omega + (h * R + c) * R;
        float s = 0.f;
        for (int j = 0; j < R; ++j) s = fmaf(om[j], er[j], s);
        eo[e] = s;
    }
}

// Rotation of low-rank feature pair index pr (0 .. R/2-1) at token coords.
__device__ __forceinline__ float2 lr_cossin(const float2* __restrict__ tab, const LrGeom& g, int pr, const int* crd) {
    int a, j;
    if (pr < g.lp[0]) { a = 0; j = pr; }
    else if (pr < g.lp[0] + g.lp[1]) { a = 1; j = pr - g.lp[0]; }
    else { a = 2; j = pr - g.lp[0] - g.lp[1]; }
    return tab[g.rope.tab_off[a] + crd[a] * g.rope.np[a] + j];
}

// One workgroup (4 waves) = `chunk` consecutive tokens of one (b, h) slice;
// each wave takes 32-token sub-tiles. Per sub-tile:
//   U (32 tok x RP) = K_sub W_k              MFMA m=tok, n=r, k=d
//   U -> E, phi, rotation (pairs are adjacent lanes), z partial
//   S (RP x D) += U^T V_sub                  MFMA m=r, n=d, k=tok
// The U accumulator already has the token slots a 32x32x16 A operand needs
// (slot16 order), so V is staged in LDS transposed [d][slot16(tok)].
//
// TILEDV (D = 128, used inside the layer forward): V is not read from v but
// from the rotate kernel's [K | V^T] tiles, whose V^T chunks already hold a
// wave's B operand in this kernel's token-slot order, so no LDS transpose is
// needed (the tail block's padded keys are zero there).
//
// PF (TILEDV, rotary variant, rank <= 32, rotation table of at most kLrTabMax
// entries; the FAVOR+ instance would spill, so only elu + 1 / SiLU use it):
// each wave keeps its next sub-tile in flight while it works on the current
// one. The V^T chunks go straight from memory into a two-slot LDS ring of the
// wave (direct global -> LDS copies, no registers), the next K rows into the
// registers the U MFMAs just released, and the cos/sin rows of the low-rank
// pairs sit in LDS, so no global load is issued between the prefetch and the
// next sub-tile (vector loads complete in issue order: waiting for a later
// load would also wait for the prefetch). The ring aliases the reduction
// buffer, which is used only after the loop. (Copying the K rows into LDS as
// well, one slot each for K and V^T, measured 1% slower.)
//
// FAV (FAVOR+ features): besides U = K W_k (the exponent's |p|^2 term, per
// token a sum over the r lanes of a 32-lane half), Y = K (W_k omega^T) on
// MFMA with bf16 hi + lo weights gives omega_c . p; u_c = exp(y_c -
// |p|^2 / 2) / sqrt(R).
// Largest rotation table (float2 entries) the prefetching summary stages in LDS.
constexpr int kLrTabMax = 1920;

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Eight 16-byte LDS reads at 1 KB spacing (the chunks of one operand-order
// sub-tile), waiting for their own completion only. Written as one asm block
// so the compiler does not first wait for every copy still landing in LDS.
__device__ __forceinline__ void lds_read8_1k(u32x4_t* r, const uint16_t* lds_base) {
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

// Eight 8-byte LDS reads at per-lane byte addresses a[0..7], same waiting rule.
__device__ __forceinline__ void lds_gather8(f32x2_t* r, const uint32_t* a) {
    asm volatile(
        "ds_read_b64 %0, %8\n\t"
        "ds_read_b64 %1, %9\n\t"
        "ds_read_b64 %2, %10\n\t"
        "ds_read_b64 %3, %11\n\t"
        "ds_read_b64 %4, %12\n\t"
        "ds_read_b64 %5, %13\n\t"
        "ds_read_b64 %6, %14\n\t"
        "ds_read_b64 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

#define SLR_SUMMARY_PARAMS                                                                                      \
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const uint16_t *__restrict__ kv_tiles, int nblk, \
        const uint16_t *__restrict__ wkt, const float *__restrict__ Et, const float *__restrict__ Eh,            \
        const float *__restrict__ Ew, const float2 *__restrict__ tab, LrGeom g, long L, int H, int chunk,        \
        int nsplit, float *__restrict__ part, const uint16_t *__restrict__ wkot_hi,                              \
        const uint16_t *__restrict__ wkot_lo
#define SLR_SUMMARY_ARGS k, v, kv_tiles, nblk, wkt, Et, Eh, Ew, tab, g, L, H, chunk, nsplit, part, wkot_hi, wkot_lo

template <int D, int RP, bool ABSPE, bool TILEDV, bool FAV, bool PF>
__device__ __forceinline__ void lr_summary_bf16_body(SLR_SUMMARY_PARAMS) {
    constexpr int NRB = RP / 32;   // r blocks
    constexpr int NDB = D / 32;    // d blocks
    constexpr int NKS = D / 16;    // k steps over d
    constexpr int VLD = 32 + 8;    // LDS row stride (elements) of V^T
    static_assert(!PF || (TILEDV && !ABSPE && D == 128), "prefetching summary: tiled V^T, rotary variant");
    constexpr int RED_N = RP * D + RP;
    constexpr int RING_F = PF ? 4 * 2 * 4096 / 2 : 0;   // 4 waves x 2 slots x 8 KB, in floats
    __shared__ __attribute__((aligned(16))) uint16_t vt[TILEDV ? 1 : 4][TILEDV ? 8 : D * VLD];
    __shared__ __attribute__((aligned(16))) float red[RING_F > RED_N ? RING_F : RED_N];
    __shared__ __attribute__((aligned(16))) float2 ltab[PF ? kLrTabMax : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const long bh = blockIdx.y;
    const int head = (int)(bh % H);
    const int split = blockIdx.x;
    const long tok_lo = (long)split * chunk;
    const long tok_hi = tok_lo + chunk < L ? tok_lo + chunk : L;
    const uint16_t* ks = k + bh * L * D;
    const uint16_t* vs = v + bh * L * D;

    // B operand of U = K W: W[d = 16s + 8hf + e][r = 32rb + l32]
    u32x4_t wop[NRB][NKS];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int s = 0; s < NKS; ++s)
            wop[rb][s] = ldg16(wkt + ((long)head * RP + 32 * rb + l32) * D + 16 * s + 8 * hf);

    f32x16_t sacc[NRB][NDB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[rb][db][i] = 0.f;
    float zacc[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) zacc[rb] = 0.f;

    // V transpose assignment: 8 tokens x 8 dims per lane
    constexpr int VCH = D / 8;                 // dim chunks
    const int vc = lane % VCH, vg = lane / VCH;  // vg: 8-token group (valid if < 4)
    const int vG = vg >> 1, vh = vg & 1;
    uint16_t* myvt = vt[TILEDV ? 0 : wave];
    const uint16_t* tiles = TILEDV ? kv_tiles + bh * (long)nblk * kTileElems : nullptr;

    // each wave walks its own 32-token sub-tiles (wave, wave + 4, ...) with
    // its own LDS area, so the loop has no workgroup barrier
    // rotation of this lane's feature pair (r = 32rb + l32 is fixed per lane)
    // table row of this lane's pair: entry = base + (its axis coordinate) * stride
    int rax[NRB], rbase[NRB], rstride[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int pr = (32 * rb + l32) >> 1;
        int a = 0, j = pr;
        if (pr >= g.lp[0] + g.lp[1]) { a = 2; j = pr - g.lp[0] - g.lp[1]; }
        else if (pr >= g.lp[0]) { a = 1; j = pr - g.lp[0]; }
        rax[rb] = a;
        rbase[rb] = (a == 0 ? g.rope.tab_off[0] : a == 1 ? g.rope.tab_off[1] : g.rope.tab_off[2]) + j;
        rstride[rb] = a == 0 ? g.rope.np[0] : a == 1 ? g.rope.np[1] : g.rope.np[2];
    }
    u32x4_t kop[NKS];
    // K rows of sub-tile t0 (rows past the chunk clamped to its last token)
    auto load_k = [&](long t0) {
        const long tk = t0 + l32;
        const long tkc = tk < tok_hi ? tk : tok_hi - 1;
#pragma unroll
        for (int s = 0; s < NKS; ++s) kop[s] = ldg16(ks + tkc * D + 16 * s + 8 * hf);
    };
    // PF: V^T chunks of sub-tile t0 -> ring slot sl of this wave (the LDS
    // image equals the memory image: chunk i at 1 KB * i, lane at 16 B * lane)
    uint16_t* const vring = reinterpret_cast<uint16_t*>(red) + (PF ? wave * 8192 : 0);
    auto issue_v = [&](long t0, int sl) {
        const uint16_t* vp = tiles + (t0 >> 6) * (long)kTileElems + 64 * 128 + ((((t0 >> 5) & 1) * 8) * 64 + lane) * 8;
        uint16_t* dst = vring + sl * 4096;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vp + i * 512),
                                             (__attribute__((address_space(3))) void*)(dst + i * 512), 16, 0, 0);
    };
    // PF: LDS rotation table, entry (axis a, coordinate c, pair j < lp[a]) at
    // loff[a] + c lp[a] + j; the lanes of padding features (r >= R) read entry 0
    int lbase[NRB], lstride[NRB];
    const uint32_t tbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float2*)ltab;
    if constexpr (PF) {
        const int n0 = g.rope.T * g.lp[0], n1 = g.rope.Hg * g.lp[1], n2 = g.rope.Wg * g.lp[2];
        for (int e = tid; e < n0 + n1 + n2; e += 256) {
            const int a = e < n0 ? 0 : (e < n0 + n1 ? 1 : 2);
            const int r = e - (a == 0 ? 0 : (a == 1 ? n0 : n0 + n1));
            const int c = r / g.lp[a], j = r - c * g.lp[a];
            ltab[e] = tab[g.rope.tab_off[a] + c * g.rope.np[a] + j];
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const int r = 32 * rb + l32, pr = r >> 1, a = rax[rb];
            const int j = pr - (a == 0 ? 0 : (a == 1 ? g.lp[0] : g.lp[0] + g.lp[1]));
            const bool live = r < g.R;
            lbase[rb] = live ? (a == 0 ? 0 : (a == 1 ? n0 : n0 + n1)) + j : 0;
            lstride[rb] = live ? g.lp[a] : 0;
        }
        __syncthreads();
        const long tf = tok_lo + 32 * wave;
        if (tf < tok_hi) {
            issue_v(tf, 0);
            load_k(tf);
        }
    }
    int slot = 0;   // PF: ring slot of the current sub-tile
    // PF: cos/sin of this lane's pair for the 16 tokens of sub-tile t0 from LDS
    auto lds_cs = [&](int rb, const int* ca, long t0, float2* cs) {
        uint32_t ad[16];
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
            const bool okt = t0 + 4 * hf + 8 * (vv >> 2) + (vv & 3) < tok_hi;
            ad[vv] = tbase + 8u * (uint32_t)(lbase[rb] + (okt ? ca[vv] : 0) * lstride[rb]);
        }
        f32x2_t cv[16];
        lds_gather8(cv, ad);
        lds_gather8(cv + 8, ad + 8);
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) cs[vv] = make_float2(cv[vv].x, cv[vv].y);
    };
    // Every load below is unconditional: rows past the chunk are clamped to
    // its last token (their features are zeroed), so the loads of a sub-tile
    // issue back to back instead of one predicated round trip each.
    for (long t0 = tok_lo + 32 * wave; t0 < tok_hi; t0 += 128) {
        // ---- U = K_sub W_k (PF: K rows and the V^T chunks were requested one
        // sub-tile earlier, and nothing else is in flight)
        if constexpr (PF) wait_vmcnt<0>();
        else load_k(t0);
        f32x16_t uacc[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 16; ++i) uacc[rb][i] = 0.f;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) uacc[rb] = mfma32(kop[s], wop[rb][s], uacc[rb]);
        }
        // FAVOR+: Y = K_sub (W_k omega^T), hi and lo weight parts
        f32x16_t yacc[FAV ? NRB : 1];
        if constexpr (FAV) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int i = 0; i < 16; ++i) yacc[rb][i] = 0.f;
#pragma unroll
            for (int s = 0; s < NKS; ++s)
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    const long wo = ((long)head * RP + 32 * rb + l32) * D + 16 * s + 8 * hf;
                    yacc[rb] = mfma32(kop[s], ldg16(wkot_hi + wo), yacc[rb]);
                    yacc[rb] = mfma32(kop[s], ldg16(wkot_lo + wo), yacc[rb]);
                }
        }
        // PF: the next sub-tile's requests, now that kop is free
        if constexpr (PF) {
            if (t0 + 128 < tok_hi) {
                issue_v(t0 + 128, slot ^ 1);
                load_k(t0 + 128);
            }
        }
        // ---- V sub-tile -> this wave's LDS area, transposed to [d][slot16(tok)]
        u32x4_t vop[TILEDV ? 8 : 1];
        if (TILEDV) {
            // sub-tile = key half ((t0 / 32) & 1) of block t0 / 64; chunk (kh, db, h2)
            if constexpr (!PF) {
                const uint16_t* vp = tiles + (t0 >> 6) * (long)kTileElems + 64 * 128 + ((((t0 >> 5) & 1) * 8) * 64 + lane) * 8;
#pragma unroll
                for (int i = 0; i < 8; ++i) vop[i] = ldg16(vp + i * 512);
            }
        } else if (vg < 4) {
            uint32_t rows[8][4];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const long tv = t0 + 16 * vG + 4 * vh + (e & 3) + 8 * (e >> 2);
                const u32x4_t w = ldg16(vs + (tv < tok_hi ? tv : tok_hi - 1) * D + 8 * vc);
#pragma unroll
                for (int i = 0; i < 4; ++i) rows[e][i] = w[i];
            }
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                u32x4_t o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a0 = rows[2 * i][f >> 1], a1 = rows[2 * i + 1][f >> 1];
                    o[i] = (f & 1) ? __builtin_amdgcn_perm(a1, a0, 0x07060302u)
                                   : __builtin_amdgcn_perm(a1, a0, 0x05040100u);
                }
                stg16(myvt + (8 * vc + f) * VLD + 16 * vG + 8 * vh, o);
            }
        }
        // ---- features: lane holds r = 32rb + l32 for tokens t0 + 4hf + {0..3, 8..11, 16..19, 24..27}
        // coordinates of the 16 tokens (division free after the first): the three
        // axes for the absolute embeddings, else this lane's rotation axis only
        int cT[16], cH[16], cW[16], cA[NRB][16];
        {
            int ct, chh, cw;
            token_coords(t0 + 4 * hf, g.rope.Hg, g.rope.Wg, ct, chh, cw);
            if (g.rope.Wg > 5) {   // steps are at most 5 tokens: one wrap of w at most
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    if (vv > 0) coords_step(ct, chh, cw, (vv & 3) ? 1 : 5, g.rope.Hg, g.rope.Wg);
                    cT[vv] = ct; cH[vv] = chh; cW[vv] = cw;
                }
            } else {
                for (int vv = 0; vv < 16; ++vv) {
                    if (vv > 0) coords_advance(ct, chh, cw, (vv & 3) ? 1 : 5, g.rope.Hg, g.rope.Wg);
                    cT[vv] = ct; cH[vv] = chh; cW[vv] = cw;
                }
            }
#pragma unroll
            for (int vv = 0; vv < 16; ++vv)
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
                    cA[rb][vv] = rax[rb] == 2 ? cW[vv] : (rax[rb] == 1 ? cH[vv] : cT[vv]);
        }
        float fv[NRB][16];
        if constexpr (FAV) {
            // |p|^2 per token: this lane's r, then the other 31 lanes of its half
            float sqv[16];
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) sqv[vv] = 0.f;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const int r = 32 * rb + l32;
                float ev[16];
                if (ABSPE) {
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv) {
                        const bool ok = t0 + 4 * hf + 8 * (vv >> 2) + (vv & 3) < tok_hi && r < g.R;
                        const int rr = r < g.R ? r : 0;
                        const int it = ok ? cT[vv] : 0, ih = ok ? cH[vv] : 0, iw = ok ? cW[vv] : 0;
                        ev[vv] = Et[it * g.R + rr] + Eh[ih * g.R + rr] + Ew[iw * g.R + rr];
                    }
                }
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const bool ok = t0 + 4 * hf + 8 * (vv >> 2) + (vv & 3) < tok_hi && r < g.R;
                    float x = uacc[rb][vv];
                    if (ABSPE) x += ev[vv];
                    x = ok ? x : 0.f;
                    sqv[vv] += x * x;
                }
            }
#pragma unroll
            for (int vv = 0; vv < 16; ++vv)
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) sqv[vv] += __shfl_xor(sqv[vv], o, 64);
            const float rs = 1.f / sqrtf((float)g.R);
            const int na = g.rope.T + g.rope.Hg + g.rope.Wg;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const int r = 32 * rb + l32;
                float2 cs[16];
                float eo[16];
                if constexpr (PF) lds_cs(rb, cA[rb], t0, cs);
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const bool ok = t0 + 4 * hf + 8 * (vv >> 2) + (vv & 3) < tok_hi && r < g.R;
                    if (ABSPE) {
                        const int rr = r < g.R ? r : 0;
                        const int it = ok ? cT[vv] : 0, ih = ok ? cH[vv] : 0, iw = ok ? cW[vv] : 0;
                        const float* eoh = g.eo + (long)head * na * g.R + rr;
                        eo[vv] = eoh[it * g.R] + eoh[(g.rope.T + ih) * g.R] + eoh[(g.rope.T + g.rope.Hg + iw) * g.R];
                    } else if (!PF) {
                        cs[vv] = tab[rbase[rb] + (ok ? cA[rb][vv] : 0) * rstride[rb]];
                    }
                }
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const bool ok = t0 + 4 * hf + 8 * (vv >> 2) + (vv & 3) < tok_hi && r < g.R;
                    float y = yacc[rb][vv];
                    if (ABSPE) y += eo[vv];
                    float u = ok ? __builtin_amdgcn_exp2f((y - 0.5f * sqv[vv]) * kLog2e) * rs : 0.f;
                    zacc[rb] += u;
                    if (!ABSPE) {
                        const float p = lane_swap1(u);  // partner dim r ^ 1
                        u = (r & 1) ? (p * cs[vv].y + u * cs[vv].x) : (u * cs[vv].x - p * cs[vv].y);
                    }
                    fv[rb][vv] = u;
                }
            }
        } else {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const int r = 32 * rb + l32;
            // gathers first (all independent), arithmetic after
            float2 cs[16];
            float ev[16];
            if constexpr (PF) lds_cs(rb, cA[rb], t0, cs);
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const bool ok = t0 + 4 * hf + 8 * (vv >> 2) + (vv & 3) < tok_hi && r < g.R;
                if (ABSPE) {
                    const int rr = r < g.R ? r : 0;
                    const int it = ok ? cT[vv] : 0, ih = ok ? cH[vv] : 0, iw = ok ? cW[vv] : 0;
                    ev[vv] = Et[it * g.R + rr] + Eh[ih * g.R + rr] + Ew[iw * g.R + rr];
                } else if (!PF) {
                    cs[vv] = tab[rbase[rb] + (ok ? cA[rb][vv] : 0) * rstride[rb]];
                }
            }
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const bool ok = t0 + 4 * hf + 8 * (vv >> 2) + (vv & 3) < tok_hi && r < g.R;
                float x = uacc[rb][vv];
                if (ABSPE) x += ev[vv];
                float u = ok ? phi_feat_fast(g.fmap, x) : 0.f;
                zacc[rb] += u;
                if (!ABSPE) {
                    const float p = lane_swap1(u);  // partner dim r ^ 1
                    u = (r & 1) ? (p * cs[vv].y + u * cs[vv].x) : (u * cs[vv].x - p * cs[vv].y);
                }
                fv[rb][vv] = u;
            }
        }
        }
        u32x4_t fhi[NRB][2], flo[NRB][2];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a0 = fv[rb][8 * ks2 + 2 * i], a1 = fv[rb][8 * ks2 + 2 * i + 1];
                    const uint32_t hi = pack_bf2(a0, a1);
                    fhi[rb][ks2][i] = hi;
                    flo[rb][ks2][i] = pack_bf2(a0 - bf_lo(hi), a1 - bf_hi(hi));
                }
        // this wave's LDS writes before its reads (lanes read other lanes' data)
        if (!TILEDV) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        // ---- S += F^T V
        if constexpr (PF) lds_read8_1k(vop, vring + slot * 4096 + lane * 8);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
                const u32x4_t vb = TILEDV ? vop[(db * 2 + ks2) & (TILEDV ? 7 : 0)]
                                          : *reinterpret_cast<const u32x4_t*>(myvt + (32 * db + l32) * VLD + 16 * ks2 + 8 * hf);
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    sacc[rb][db] = mfma32(fhi[rb][ks2], vb, sacc[rb][db]);
                    sacc[rb][db] = mfma32(flo[rb][ks2], vb, sacc[rb][db]);
                }
            }
        // reads done before the next sub-tile overwrites the area
        if (!TILEDV) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        slot ^= 1;
    }
    // PF: the ring aliases red; no copy is requested past the last sub-tile
    if constexpr (PF) wait_vmcnt<0>();
    __syncthreads();

    // ---- reduce the 4 waves in a fixed order, then write the partial
    // sacc[rb][db][vv]: r = 32rb + 8(vv/4) + 4hf + vv%4, d = 32db + l32
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv) {
                        const int r = 32 * rb + 8 * (vv >> 2) + 4 * hf + (vv & 3);
                        const int e = r * D + 32 * db + l32;
                        red[e] = (w == 0 ? 0.f : red[e]) + sacc[rb][db][vv];
                    }
            // z: lanes l32 and l32+32 hold the same r, different tokens
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const float zz = zacc[rb] + wave_xor32(zacc[rb]);
                if (hf == 0) {
                    const int e = RP * D + 32 * rb + l32;
                    red[e] = (w == 0 ? 0.f : red[e]) + zz;
                }
            }
        }
        __syncthreads();
    }
    float* dst = part + (bh * nsplit + split) * (long)(RP * D + RP);
    for (int e = tid; e < RP * D + RP; e += 256) dst[e] = red[e];
}

template <int D, int RP, bool ABSPE, bool TILEDV, bool FAV = false>
__global__ __launch_bounds__(256) void k_lr_summary_bf16(SLR_SUMMARY_PARAMS) {
    lr_summary_bf16_body<D, RP, ABSPE, TILEDV, FAV, false>(SLR_SUMMARY_ARGS);
}

// The prefetching instance (elu + 1 or SiLU features, rank <= 32), held to
// two waves per SIMD: two workgroups per CU with its 79 KB of LDS.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_lr_summary_bf16_pf(
    SLR_SUMMARY_PARAMS) {
    lr_summary_bf16_body<128, 32, false, true, false, true>(SLR_SUMMARY_ARGS);
}

// fp32 layers: the same sums on fp32 VALU (tokens staged through LDS).
template <int D, int RP>
__global__ __launch_bounds__(256) void k_lr_summary_f32(const float* __restrict__ k, const float* __restrict__ v,
                                                        const float* __restrict__ W, const float* __restrict__ Et,
                                                        const float* __restrict__ Eh, const float* __restrict__ Ew,
                                                        const float2* __restrict__ tab, LrGeom g, long L, int H,
                                                        int absPE, int chunk, int nsplit, float* __restrict__ part) {
    constexpr int TS = 16;  // tokens per step
    __shared__ float ksh[TS][D], vsh[TS][D], fsh[TS][RP], ush[TS][RP], xsh[TS][RP];
    const int tid = threadIdx.x;
    const long bh = blockIdx.y;
    const int head = (int)(bh % H);
    const int split = blockIdx.x;
    const long tok_lo = (long)split * chunk;
    const long tok_hi = tok_lo + chunk < L ? tok_lo + chunk : L;
    const int R = g.R;
    const float* Wh = W + (long)head * D * R;
    constexpr int NE = (RP * D + 255) / 256;
    float sacc[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) sacc[i] = 0.f;
    float zacc = 0.f;

    for (long t0 = tok_lo; t0 < tok_hi; t0 += TS) {
        for (int e = tid; e < TS * D; e += 256) {
            const int tl = e / D, d = e % D;
            const long t = t0 + tl;
            ksh[tl][d] = t < tok_hi ? k[(bh * L + t) * D + d] : 0.f;
            vsh[tl][d] = t < tok_hi ? v[(bh * L + t) * D + d] : 0.f;
        }
        __syncthreads();
        const bool fav = g.fmap == 2;
        if (fav) {
            // FAVOR+: the projections p = k W [+ E] of the step's tokens first
            for (int e = tid; e < TS * RP; e += 256) {
                const int tl = e / RP, r = e % RP;
                const long t = t0 + tl;
                float acc = 0.f;
                if (t < tok_hi && r < R) {
                    for (int d = 0; d < D; ++d) acc += ksh[tl][d] * Wh[d * R + r];
                    if (absPE) {
                        int crd[3];
                        token_coords(t, g.rope.Hg, g.rope.Wg, crd[0], crd[1], crd[2]);
                        acc += Et[crd[0] * R + r] + Eh[crd[1] * R + r] + Ew[crd[2] * R + r];
                    }
                }
                xsh[tl][r] = acc;
            }
            __syncthreads();
        }
        // features, one (token, pair) per thread
        for (int e = tid; e < TS * (RP / 2); e += 256) {
            const int tl = e / (RP / 2), pr = e % (RP / 2);
            const long t = t0 + tl;
            float u[2] = {0.f, 0.f};
            int crd[3] = {0, 0, 0};
            const bool tv = t < tok_hi;
            if (tv) token_coords(t, g.rope.Hg, g.rope.Wg, crd[0], crd[1], crd[2]);
            for (int q = 0; q < 2; ++q) {
                const int r = 2 * pr + q;
                if (!tv || r >= R) continue;
                if (fav) {
                    // u_r = exp(omega_r . p - |p|^2 / 2) / sqrt(R)
                    const float* om = g.omega + ((long)head * R + r) * R;
                    float y = 0.f, sq = 0.f;
                    for (int j = 0; j < R; ++j) {
                        y += om[j] * xsh[tl][j];
                        sq += xsh[tl][j] * xsh[tl][j];
                    }
                    u[q] = expf(y - 0.5f * sq) / sqrtf((float)R);
                    continue;
                }
                float acc = 0.f;
                for (int d = 0; d < D; ++d) acc += ksh[tl][d] * Wh[d * R + r];
                if (absPE) acc += Et[crd[0] * R + r] + Eh[crd[1] * R + r] + Ew[crd[2] * R + r];
                u[q] = phi_feat(g.fmap, acc);
            }
            ush[tl][2 * pr] = u[0];
            ush[tl][2 * pr + 1] = u[1];
            if (!absPE && tv && 2 * pr < R) {
                const float2 cs = lr_cossin(tab, g, pr, crd);
                fsh[tl][2 * pr] = u[0] * cs.x - u[1] * cs.y;
                fsh[tl][2 * pr + 1] = u[0] * cs.y + u[1] * cs.x;
            } else {
                fsh[tl][2 * pr] = u[0];
                fsh[tl][2 * pr + 1] = u[1];
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = tid + 256 * i;
            if (e < RP * D) {
                const int r = e / D, d = e % D;
                float s = sacc[i];
                for (int tl = 0; tl < TS; ++tl) s += fsh[tl][r] * vsh[tl][d];
                sacc[i] = s;
            }
        }
        if (tid < RP)
            for (int tl = 0; tl < TS; ++tl) zacc += ush[tl][tid];
        __syncthreads();
    }
    float* dst = part + (bh * nsplit + split) * (long)(RP * D + RP);
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int e = tid + 256 * i;
        if (e < RP * D) dst[e] = sacc[i];
    }
    if (tid < RP) dst[RP * D + tid] = zacc;
}

// Sum the split partials in split order. Writes S [BH][R][D] and z [BH][R]
// (fp32), and for bf16 layers the readout operand St_hi/St_lo [BH][D][RP]
// (bf16 hi + lo of S, r in slot16 order inside each 16-group) and zp [BH][RP].
__global__ __launch_bounds__(256) void k_lr_reduce(const float* __restrict__ part, int nsplit, int D, int R, int RP,
                                                   float* __restrict__ S, float* __restrict__ z,
                                                   uint16_t* __restrict__ st_hi, uint16_t* __restrict__ st_lo,
                                                   float* __restrict__ zp) {
    const long bh = blockIdx.y;
    const int n = RP * D + RP;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const float* p = part + bh * nsplit * (long)n + e;
    float s = 0.f;
    for (int i = 0; i < nsplit; ++i) s += p[(long)i * n];
    if (e < RP * D) {
        const int r = e / D, d = e % D;
        if (r < R && S) S[(bh * R + r) * D + d] = s;
        if (st_hi) {
            const uint16_t hi = f2bf(s);
            const uint16_t lo = f2bf(s - bf2f(hi));
            const long o = (bh * D + d) * RP + 16 * (r >> 4) + slot16(r & 15);
            st_hi[o] = hi;
            st_lo[o] = lo;
        }
    } else {
        const int r = e - RP * D;
        if (r < R && z) z[bh * R + r] = s;
        if (zp) zp[bh * RP + r] = s;
    }
}

// ---- launchers ----------------------------------------------------------
hipError_t launch_lr_prep(const float* W, uint16_t* Wt, int H, int D, int R, int RP, hipStream_t st) {
    const long n = (long)H * RP * D;
    hipLaunchKernelGGL(k_lr_prep, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, W, Wt, H, D, R, RP);
    return hipGetLastError();
}

hipError_t launch_lr_prep_favor(const float* W, const float* omega, int round_bf16, int H, int D, int R, int RP,
                                uint16_t* wot_hi, uint16_t* wot_lo, const float* Et, const float* Eh, const float* Ew,
                                int T, int Hg, int Wg, float* eo, hipStream_t st) {
    if (wot_hi) {
        const long n = (long)H * RP * D;
        hipLaunchKernelGGL(k_lr_prep_favor, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, W, omega, round_bf16,
                           H, D, R, RP, wot_hi, wot_lo);
    }
    if (Et && eo) {
        const long n = (long)H * (T + Hg + Wg) * R;
        hipLaunchKernelGGL(k_lr_prep_favor_e, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Et, Eh, Ew, omega,
                           H, T, Hg, Wg, R, eo);
    }
    return hipGetLastError();
}

template <int D, int RP, bool TILEDV>
static hipError_t summary_bf16_t(bool abspe, const void* k, const void* v, const uint16_t* kvt, int nblk,
                                 const uint16_t* wkt, const float* Et, const float* Eh, const float* Ew,
                                 const float2* tab, const LrGeom& g, long BH, long L, int H, int chunk, int nsplit,
                                 float* part, hipStream_t st, const uint16_t* woh, const uint16_t* wol) {
    dim3 grid((unsigned)nsplit, (unsigned)BH);
    const bool fav = g.fmap == 2;
    const bool pf = lr_summary_prefetch(1, D, abspe, TILEDV, g);
#define SLR_SUMB(KERNEL)                                                                                    \
    hipLaunchKernelGGL((KERNEL), grid, dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v, kvt, nblk, wkt, \
                       Et, Eh, Ew, tab, g, L, H, chunk, nsplit, part, woh, wol)
    if (abspe) {
        if (fav) SLR_SUMB((k_lr_summary_bf16<D, RP, true, TILEDV, true>));
        else SLR_SUMB((k_lr_summary_bf16<D, RP, true, TILEDV, false>));
    } else if (pf) {
        if constexpr (TILEDV && D == 128 && RP == 32) SLR_SUMB(k_lr_summary_bf16_pf);
    } else {
        if (fav) SLR_SUMB((k_lr_summary_bf16<D, RP, false, TILEDV, true>));
        else SLR_SUMB((k_lr_summary_bf16<D, RP, false, TILEDV, false>));
    }
#undef SLR_SUMB
    return hipGetLastError();
}

bool lr_summary_prefetch(int dtype_bf16, int D, bool abspe, bool tiled, const LrGeom& g) {
    const long n = (long)g.rope.T * g.lp[0] + (long)g.rope.Hg * g.lp[1] + (long)g.rope.Wg * g.lp[2];
    return dtype_bf16 && D == 128 && tiled && !abspe && g.R <= 32 && g.fmap != 2 && n <= kLrTabMax;
}

// The kernel instance launch_lr_summary picks for these arguments.
static const void* summary_kernel(int dtype_bf16, int D, int RP, bool abspe, bool tiled, bool favor, bool pf) {
#define SLR_PICK(...) return reinterpret_cast<const void*>(&__VA_ARGS__)
    if (pf) SLR_PICK(k_lr_summary_bf16_pf);
    if (dtype_bf16 && favor) {
        // FAVOR+ instances (their occupancy is what sizes the split)
        if (tiled && D == 128) {
            if (RP == 32) { if (abspe) SLR_PICK(k_lr_summary_bf16<128, 32, true, true, true>); SLR_PICK(k_lr_summary_bf16<128, 32, false, true, true>); }
            if (abspe) SLR_PICK(k_lr_summary_bf16<128, 64, true, true, true>);
            SLR_PICK(k_lr_summary_bf16<128, 64, false, true, true>);
        }
        if (D == 64 && RP == 32) { if (abspe) SLR_PICK(k_lr_summary_bf16<64, 32, true, false, true>); SLR_PICK(k_lr_summary_bf16<64, 32, false, false, true>); }
        if (D == 64) { if (abspe) SLR_PICK(k_lr_summary_bf16<64, 64, true, false, true>); SLR_PICK(k_lr_summary_bf16<64, 64, false, false, true>); }
        if (RP == 32) { if (abspe) SLR_PICK(k_lr_summary_bf16<128, 32, true, false, true>); SLR_PICK(k_lr_summary_bf16<128, 32, false, false, true>); }
        if (abspe) SLR_PICK(k_lr_summary_bf16<128, 64, true, false, true>);
        SLR_PICK(k_lr_summary_bf16<128, 64, false, false, true>);
    }
    if (dtype_bf16) {
        if (tiled && D == 128) {
            if (RP == 32) { if (abspe) SLR_PICK(k_lr_summary_bf16<128, 32, true, true>); SLR_PICK(k_lr_summary_bf16<128, 32, false, true>); }
            if (abspe) SLR_PICK(k_lr_summary_bf16<128, 64, true, true>);
            SLR_PICK(k_lr_summary_bf16<128, 64, false, true>);
        }
        if (D == 64 && RP == 32) { if (abspe) SLR_PICK(k_lr_summary_bf16<64, 32, true, false>); SLR_PICK(k_lr_summary_bf16<64, 32, false, false>); }
        if (D == 64) { if (abspe) SLR_PICK(k_lr_summary_bf16<64, 64, true, false>); SLR_PICK(k_lr_summary_bf16<64, 64, false, false>); }
        if (RP == 32) { if (abspe) SLR_PICK(k_lr_summary_bf16<128, 32, true, false>); SLR_PICK(k_lr_summary_bf16<128, 32, false, false>); }
        if (abspe) SLR_PICK(k_lr_summary_bf16<128, 64, true, false>);
        SLR_PICK(k_lr_summary_bf16<128, 64, false, false>);
    }
    if (D == 64 && RP == 32) SLR_PICK(k_lr_summary_f32<64, 32>);
    if (D == 64) SLR_PICK(k_lr_summary_f32<64, 64>);
    if (RP == 32) SLR_PICK(k_lr_summary_f32<128, 32>);
    SLR_PICK(k_lr_summary_f32<128, 64>);
#undef SLR_PICK
}

hipError_t lr_summary_slots(int dtype_bf16, int D, int RP, bool abspe, bool tiled, int* slots, bool favor, bool pf) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev][128];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    pf = pf && dtype_bf16 && D == 128 && RP == 32 && tiled && !abspe && !favor;
    const int key = (pf ? 64 : 0) | (favor && dtype_bf16 ? 32 : 0) | (dtype_bf16 ? 16 : 0) | (D == 128 ? 8 : 0) |
                    (RP == 64 ? 4 : 0) | (abspe ? 2 : 0) | (tiled ? 1 : 0);
    if (dev >= 0 && dev < kMaxDev) {
        const int c = cache[dev][key].load(std::memory_order_relaxed);
        if (c > 0) { *slots = c; return hipSuccess; }
    }
    int cus = 0, per = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, summary_kernel(dtype_bf16, D, RP, abspe, tiled, favor, pf), 256,
                                                          0)) != hipSuccess)
        return e;
    const int n = (cus > 0 ? cus : 1) * (per > 0 ? per : 1);
    if (dev >= 0 && dev < kMaxDev) cache[dev][key].store(n, std::memory_order_relaxed);
    *slots = n;
    return hipSuccess;
}

hipError_t launch_lr_summary(int dtype_bf16, int D, int RP, bool abspe, const void* k, const void* v,
                             const uint16_t* kvt, int nblk, const float* W, const uint16_t* wkt, const float* Et,
                             const float* Eh, const float* Ew, const float2* tab, const LrGeom& g, long BH, long L,
                             int H, int chunk, int nsplit, float* part, hipStream_t st, const uint16_t* wkot_hi,
                             const uint16_t* wkot_lo) {
    if (dtype_bf16) {
        if (kvt && D == 128) {
            if (RP == 32)
                return summary_bf16_t<128, 32, true>(abspe, k, v, kvt, nblk, wkt, Et, Eh, Ew, tab, g, BH, L, H, chunk,
                                                     nsplit, part, st, wkot_hi, wkot_lo);
            return summary_bf16_t<128, 64, true>(abspe, k, v, kvt, nblk, wkt, Et, Eh, Ew, tab, g, BH, L, H, chunk,
                                                 nsplit, part, st, wkot_hi, wkot_lo);
        }
        if (D == 64 && RP == 32)
            return summary_bf16_t<64, 32, false>(abspe, k, v, nullptr, 0, wkt, Et, Eh, Ew, tab, g, BH, L, H, chunk,
                                                 nsplit, part, st, wkot_hi, wkot_lo);
        if (D == 64)
            return summary_bf16_t<64, 64, false>(abspe, k, v, nullptr, 0, wkt, Et, Eh, Ew, tab, g, BH, L, H, chunk,
                                                 nsplit, part, st, wkot_hi, wkot_lo);
        if (RP == 32)
            return summary_bf16_t<128, 32, false>(abspe, k, v, nullptr, 0, wkt, Et, Eh, Ew, tab, g, BH, L, H, chunk,
                                                  nsplit, part, st, wkot_hi, wkot_lo);
        return summary_bf16_t<128, 64, false>(abspe, k, v, nullptr, 0, wkt, Et, Eh, Ew, tab, g, BH, L, H, chunk,
                                              nsplit, part, st, wkot_hi, wkot_lo);
    }
    dim3 grid((unsigned)nsplit, (unsigned)BH);
#define SLR_SUMF32(DD, RR)                                                                                     \
    hipLaunchKernelGGL((k_lr_summary_f32<DD, RR>), grid, dim3(256), 0, st, (const float*)k, (const float*)v, W, \
                       Et, Eh, Ew, tab, g, L, H, (int)abspe, chunk, nsplit, part)
    if (D == 64 && RP == 32) SLR_SUMF32(64, 32);
    else if (D == 64) SLR_SUMF32(64, 64);
    else if (RP == 32) SLR_SUMF32(128, 32);
    else SLR_SUMF32(128, 64);
#undef SLR_SUMF32
    return hipGetLastError();
}

hipError_t launch_lr_reduce(const float* part, long BH, int nsplit, int D, int R, int RP, float* S, float* z,
                            uint16_t* st_hi, uint16_t* st_lo, float* zp, hipStream_t st) {
    const int n = RP * D + RP;
    dim3 grid((unsigned)((n + 255) / 256), (unsigned)BH);
    hipLaunchKernelGGL(k_lr_reduce, grid, dim3(256), 0, st, part, nsplit, D, R, RP, S, z, st_hi, st_lo, zp);
    return hipGetLastError();
}

}  // namespace slr
