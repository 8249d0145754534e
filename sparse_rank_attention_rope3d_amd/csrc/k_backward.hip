// Backward pass of the hybrid layer (either gate, every feature map; bf16 on
// MFMA, fp32 on VALU).
//
// The pages fine-tune this layer (RoLA, arXiv 2609.06712v3, §4.4 and
// App. E.2: the low-rank projections and the gate are trained), so its
// gradients are those of the forward by the chain rule, with the block
// selection (a top-k, piecewise constant) held fixed.
//
// Sparse branch (RoLA §4.1, exact softmax over the kept key blocks): per
// query row, P = softmax(q K^T / sqrt(D)) over the kept keys, dP = dO V^T,
// dS = P (dP - dO . O), dq = dS K / sqrt(D); every kept key receives
// dk += dS q / sqrt(D) and dv += P dO. Two kernels, no atomics:
//   k_bwd_dq    one workgroup per query block: with each row's log-sum-exp
//               saved by the forward, it forms dS tile by tile on MFMA
//               (S^T = K Q^T and dP^T = V dO^T, so each lane owns one query
//               row) and accumulates dQ^T = K^T dS^T;
//   k_bwd_dkdv  one workgroup per key block, over the query blocks that keep
//               it (an inverse of the kept lists, built deterministically from
//               a bitmap): S = Q K^T and dP = dO V^T with each lane owning one
//               key, dV^T += dO^T P and dK^T += Q^T dS.
// The rotated-space gradients go back through the 3D RoPE by its transpose
// (each pair turned by the opposite angle) in the epilogues, where the
// low-rank parts are added.
//
// Low-rank branch (RoLA §4.1-4.3, App. A; RoPeSLR abstract and appendix):
// per-token kernels and sums over tokens, split along L with fixed-order
// reductions of the partial sums; on bf16 MFMA for the per-head gate at
// ranks 8-64 with D = 128, fp32 VALU kernels for the other settings (the
// token gate, D = 64, fp32 layers). elu + 1 and SiLU features are
// elementwise; FAVOR+ features take their full Jacobian, du_c/dp =
// u_c (omega_c - p).
#include "slr_common.h"
#include "slr_launch.h"
#include "slr_backward.h"

namespace slr {

// (cos, sin) of backbone rotary pair p (0 .. D/2-1) at token coordinates crd.
// The axis is picked by selects over the three candidate entries rather than
// by indexing the geometry with it: a lane-dependent index into the kernel
// arguments turns into a memory load per call, ahead of the table load.
__device__ __forceinline__ float2 rope_cs(const float2* __restrict__ tab, const RopeGeom& g, int p, const int* crd) {
    const int n0 = g.np[0], n01 = g.np[0] + g.np[1];
    const int i0 = g.tab_off[0] + crd[0] * g.np[0] + p;
    const int i1 = g.tab_off[1] + crd[1] * g.np[1] + (p - n0);
    const int i2 = g.tab_off[2] + crd[2] * g.np[2] + (p - n01);
    return tab[p < n0 ? i0 : (p < n01 ? i1 : i2)];
}

// (cos, sin) of low-rank pair pr: the axis chunks hold lp[] pairs that reuse
// the backbone's schedule of their axis (axis picked as in rope_cs)
__device__ __forceinline__ float2 lowrank_cs(const float2* __restrict__ tab, const LrGeom& g, int pr, const int* crd) {
    const int n0 = g.lp[0], n01 = g.lp[0] + g.lp[1];
    const int i0 = g.rope.tab_off[0] + crd[0] * g.rope.np[0] + pr;
    const int i1 = g.rope.tab_off[1] + crd[1] * g.rope.np[1] + (pr - n0);
    const int i2 = g.rope.tab_off[2] + crd[2] * g.rope.np[2] + (pr - n01);
    return tab[pr < n0 ? i0 : (pr < n01 ? i1 : i2)];
}

// y -> R^T y for one pair: turned by minus its angle
__device__ __forceinline__ void rot_t(float& y0, float& y1, float2 cs) {
    const float x0 = y0 * cs.x + y1 * cs.y;
    const float x1 = -y0 * cs.y + y1 * cs.x;
    y0 = x0;
    y1 = x1;
}

// Epilogue of the streaming dQ and dK/dV kernels for one lane's row: out[d] =
// bf16((R^T (scale acc))[d] + lr[d]) over dims 32db + 8g4 + 4hf + 0..3
// (group q = 4db + g4), the low-rank part taken from lrp (the accumulator
// layout) when FUSED, else read from the fp32 row lr. The loads of NB
// groups are issued before their stores: the compiler keeps loads behind
// earlier stores that might alias them, so group by group each would wait
// for its own loads.
template <bool FUSED, int NB>
__device__ __forceinline__ void rotate_store_row(const float2* __restrict__ tab, const RopeGeom& g, const int* crd,
                                                 const f32x16_t* acc, float scale, const f32x16_t* lrp,
                                                 const float* __restrict__ lr, uint16_t* __restrict__ out, int hf) {
#pragma unroll
    for (int h = 0; h < 16 / NB; ++h) {
        float2 cs[2 * NB];
        float4 l[FUSED ? 1 : NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int q = NB * h + k, d0 = 32 * (q >> 2) + 8 * (q & 3) + 4 * hf;
            cs[2 * k] = rope_cs(tab, g, d0 >> 1, crd);
            cs[2 * k + 1] = rope_cs(tab, g, (d0 >> 1) + 1, crd);
            if (!FUSED) l[FUSED ? 0 : k] = *reinterpret_cast<const float4*>(lr + d0);
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int q = NB * h + k, d0 = 32 * (q >> 2) + 8 * (q & 3) + 4 * hf, e = 4 * (q & 3);
            const float4 lk = FUSED ? make_float4(lrp[q >> 2][e], lrp[q >> 2][e + 1], lrp[q >> 2][e + 2],
                                                  lrp[q >> 2][e + 3])
                                    : l[FUSED ? 0 : k];
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = acc[q >> 2][e + i] * scale;
            rot_t(y[0], y[1], cs[2 * k]);
            rot_t(y[2], y[3], cs[2 * k + 1]);
            *reinterpret_cast<u32x2_t*>(out + d0) =
                u32x2_t{pack_bf2(y[0] + lk.x, y[1] + lk.y), pack_bf2(y[2] + lk.z, y[3] + lk.w)};
        }
    }
}

// ---------------------------------------------------------------------------
// Staging of one BS x D bf16 block of rows into LDS, in two steps so the
// global loads of the next block can be in flight while the current one is
// consumed. Thread tid < (BS/8)(D/8) takes 8 rows x 8 dims: rows
// 16G + 4h + (e & 3) + 8(e >> 2) (e = 0..7) of 16-row group G with lane half
// h, dims 8c .. 8c+7. `rm` (optional) receives the rows row-major with
// stride D + 8; `tr` (optional) receives the transpose [D][BS + 8] with the
// rows of each 16-group at positions 16G + 8h + e, the slot order in which a
// 32x32 MFMA accumulator holds its rows, so an accumulator packs straight
// into the B operand that meets it. Rows at or past `limit` read as zeros.
template <int D, int BS>
struct Stager {
    static constexpr int KLD = D + 8, VLD = BS + 8, NB = (BS / 8) * (D / 8);
    int c, G, h;
    bool on;
    __device__ explicit Stager(int tid) {
        on = tid < NB;
        c = tid % (D / 8);
        const int gp = tid / (D / 8);
        G = gp >> 1;
        h = gp & 1;
    }
    __device__ __forceinline__ int row(int e) const { return 16 * G + 4 * h + (e & 3) + 8 * (e >> 2); }
    // Branch free: a row past `limit` loads row limit - 1 (always in bounds);
    // bit e of the returned mask marks row e valid, and stash() zeroes the
    // others (after the loads have landed, so no wait is forced here).
    __device__ __forceinline__ uint32_t fetch(u32x4_t* x, const uint16_t* __restrict__ src, long row0,
                                              long limit) const {
        uint32_t ok = 0;
        if (!on) return ok;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const long r = row0 + row(e);
            ok |= (r < limit ? 1u : 0u) << e;
            x[e] = ldg16(src + (r < limit ? r : limit - 1) * D + 8 * c);
        }
        return ok;
    }
    __device__ __forceinline__ void stash(u32x4_t* x, uint32_t ok, uint16_t* rm, uint16_t* tr) const {
        if (!on) return;
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[e][i] = ((ok >> e) & 1u) ? x[e][i] : 0u;
        if (rm) {
#pragma unroll
            for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4_t*>(rm + row(e) * KLD + 8 * c) = x[e];
        }
        if (tr) {
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                u32x4_t o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a0 = x[2 * i][f >> 1], a1 = x[2 * i + 1][f >> 1];
                    o[i] = (f & 1) ? __builtin_amdgcn_perm(a1, a0, 0x07060302u)
                                   : __builtin_amdgcn_perm(a1, a0, 0x05040100u);
                }
                *reinterpret_cast<u32x4_t*>(tr + (8 * c + f) * VLD + 16 * G + 8 * h) = o;
            }
        }
    }
};

// Eight 16-byte LDS reads into distinct registers, read i at byte offset
// (i & 1) * SI + (i >> 1) * SO from base; the block waits for them itself
// (early-clobber outputs: no destination can alias the address register).
template <int SI, int SO>
__device__ __forceinline__ void lds_read8x(u32x4_t* r, const uint16_t* base) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)base;
    asm volatile(
        "ds_read_b128 %0, %8 offset:%9\n\t"
        "ds_read_b128 %1, %8 offset:%10\n\t"
        "ds_read_b128 %2, %8 offset:%11\n\t"
        "ds_read_b128 %3, %8 offset:%12\n\t"
        "ds_read_b128 %4, %8 offset:%13\n\t"
        "ds_read_b128 %5, %8 offset:%14\n\t"
        "ds_read_b128 %6, %8 offset:%15\n\t"
        "ds_read_b128 %7, %8 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a), "n"(0), "n"(SI), "n"(SO), "n"(SI + SO), "n"(2 * SO), "n"(SI + 2 * SO), "n"(3 * SO),
          "n"(SI + 3 * SO)
        : "memory");
}

// ---------------------------------------------------------------------------
// dQ. Workgroup = one query block, BS/32 waves of 32 rows.
template <int D, int BS>
__global__ __launch_bounds__(BS * 2) void k_bwd_dq(BwdArgs a, const int32_t* __restrict__ idx_all) {
    constexpr int KLD = D + 8, VLD = BS + 8, NKB = BS / 32, NS = D / 16, NDB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[BS * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[BS * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t kt_lds[D * VLD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const long bh = wid / a.nblk;
    const int qb = (int)(wid % a.nblk);
    const long rows = (long)a.nblk * BS;
    const long L = a.L;
    const long qrow = (long)qb * BS + 32 * wave + l32;
    const bool qval = qrow < L;
    const uint16_t* kr = a.kr + bh * rows * D;
    const uint16_t* vg = a.v + bh * L * D;
    const int32_t* ix = idx_all + (bh * a.nblk + qb) * (long)a.keep;

    // B operands: rotated q row and dO row (dims 16s + 8hf + e); delta = dO . O
    u32x4_t qop[NS], doop[NS];
    float dl = 0.f;
    {
        const uint16_t* qp = a.qr + (bh * rows + qrow) * D + 8 * hf;
        const long orow = bh * L + (qval ? qrow : 0);
        const uint16_t* dp = a.dout + orow * D + 8 * hf;
        const uint16_t* op = a.o_sp + orow * D + 8 * hf;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qop[s] = ldg16(qp + 16 * s);
            doop[s] = qval ? ldg16(dp + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
            if (qval) {
                const u32x4_t o = ldg16(op + 16 * s);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dl += bf_lo(doop[s][i]) * bf_lo(o[i]) + bf_hi(doop[s][i]) * bf_hi(o[i]);
            }
        }
    }
    dl = sum_xor32(dl);

    const bool ragged = (L % BS) != 0;

    // kept tiles in list order, entries outside [0, nblk) skipped; the list
    // is read with scalar loads (uniform per workgroup)
    auto next_tile = [&](int n) {
        while (n < a.keep) {
            const int j = __builtin_amdgcn_readfirstlane(ix[n]);
            if (j >= 0 && j < a.nblk) break;
            ++n;
        }
        return n;
    };
    auto tile_at = [&](int n) { return __builtin_amdgcn_readfirstlane(ix[n]); };
    const Stager<D, BS> stg(tid);
    u32x4_t xk[8], xv[8];   // next tile's rows, in flight while the current one is consumed
    uint32_t okk = 0, okv = 0;

    // the forward's log2 normaliser of the row (zero on padded rows, whose
    // dO and delta are zero); kept for the key-side kernel
    const float lse2 = qval ? a.lse_in[bh * L + qrow] : 0.f;
    if (hf == 0) {
        a.lse2[bh * rows + qrow] = lse2;
        a.delta[bh * rows + qrow] = qval ? dl : 0.f;
    }
    int n;

    // ---- dS and dQ^T = K^T dS^T, tile by tile
    f32x16_t dqacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;
    n = next_tile(0);
    if (n < a.keep) {
        okk = stg.fetch(xk, kr, (long)tile_at(n) * BS, rows);
        okv = stg.fetch(xv, vg, (long)tile_at(n) * BS, L);
    }
    wait_vmcnt<0>();
    while (n < a.keep) {
        const int j = tile_at(n);
        __syncthreads();
        stg.stash(xk, okk, k_lds, kt_lds);
        stg.stash(xv, okv, v_lds, nullptr);
        __syncthreads();
        n = next_tile(n + 1);
        if (n < a.keep) {
            okk = stg.fetch(xk, kr, (long)tile_at(n) * BS, rows);
            okv = stg.fetch(xv, vg, (long)tile_at(n) * BS, L);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16_t sacc, dpacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
            if constexpr (NS == 8) {
                u32x4_t ak[8], av[8];
                lds_read8x<32, 64>(ak, k_lds + (32 * kb + l32) * KLD + 8 * hf);
                lds_read8x<32, 64>(av, v_lds + (32 * kb + l32) * KLD + 8 * hf);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    sacc = mfma32(ak[s], qop[s], sacc);
                    dpacc = mfma32(av[s], doop[s], dpacc);
                }
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const int o = (32 * kb + l32) * KLD + 16 * s + 8 * hf;
                    sacc = mfma32(*reinterpret_cast<const u32x4_t*>(k_lds + o), qop[s], sacc);
                    dpacc = mfma32(*reinterpret_cast<const u32x4_t*>(v_lds + o), doop[s], dpacc);
                }
            }
            float ds[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const long key = (long)j * BS + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
                const float p = (ragged && key >= L) ? 0.f : exp2f(sacc[i] * a.qmul - lse2);
                ds[i] = p * (dpacc[i] - dl);
            }
            u32x4_t dsop[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) dsop[h2][i] = pack_bf2(ds[8 * h2 + 2 * i], ds[8 * h2 + 2 * i + 1]);
            if constexpr (NDB == 4) {
                u32x4_t at[8];   // (db, h2) = (i / 2, i % 2)
                lds_read8x<32, 64 * VLD>(at, kt_lds + l32 * VLD + 32 * kb + 8 * hf);
#pragma unroll
                for (int i = 0; i < 8; ++i) dqacc[i >> 1] = mfma32(at[i], dsop[i & 1], dqacc[i >> 1]);
            } else {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
                        dqacc[db] = mfma32(*reinterpret_cast<const u32x4_t*>(kt_lds + (32 * db + l32) * VLD + 32 * kb +
                                                                             16 * h2 + 8 * hf),
                                           dsop[h2], dqacc[db]);
            }
        }
    }

    // ---- epilogue: dq = R^T (dQ_rot / sqrt(D)) + dq_lowrank; lane owns row qrow,
    // dims 32db + 8g4 + 4hf + 0..3
    if (!qval) return;
    int crd[3];
    token_coords(qrow, a.g.Hg, a.g.Wg, crd[0], crd[1], crd[2]);
    const float* lr = a.dq_lr + (bh * L + qrow) * D;
    uint16_t* out = a.dq + (bh * L + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * db + 8 * g4 + 4 * hf;
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = dqacc[db][4 * g4 + i] * a.scale;
            rot_t(y[0], y[1], rope_cs(a.tab, a.g, d0 >> 1, crd));
            rot_t(y[2], y[3], rope_cs(a.tab, a.g, (d0 >> 1) + 1, crd));
            const float4 l4 = *reinterpret_cast<const float4*>(lr + d0);
            *reinterpret_cast<u32x2_t*>(out + d0) =
                u32x2_t{pack_bf2(y[0] + l4.x, y[1] + l4.y), pack_bf2(y[2] + l4.z, y[3] + l4.w)};
        }
}

// ---------------------------------------------------------------------------
// Streaming dQ for bf16, D = 128, 64-token blocks (every workload shape).
//
// Each key block has one contiguous 32 KB tile [K | V] in operand order,
// written once per backward call (k_bwd_dq_tiles): every 1 KB chunk is one
// wave's MFMA operand, lane l's 16 bytes in slot opslot(l, s) of the chunk, so
// the LDS image equals the memory image and direct global-to-LDS copies fill
// it.
//   K chunk (kh, s): lane l holds K[key 32kh + l%32][dims 16s + 8(l/32) .. +7]
//   V chunk (kh, s): lane l holds V[key 32kh + l%32][dims 16s + 8(l/32) .. +7]
// The transposed operand K^T is read out of the K part with gfx950's
// transposing LDS reads (lds_read_t8). Keys past L are zero (K from the
// zero-padded rotated copy).
constexpr int kDqPart = 64 * 128;           // elements of one part
constexpr int kDqTileElems = 2 * kDqPart;   // [K | V]
// Query-side tiles of the streaming dK/dV kernel: [Q | dO | stats] per query
// block, the same chunk layout with query rows in place of keys, written by
// the dQ kernel (which holds those rows); stats = 2 KB of floats: the rows'
// log2 normalisers [64], delta = dO . O [64], and 384 unused (one 4-byte copy
// per lane of each of eight waves).
constexpr int kQtStatsElems = 1024;
constexpr int kQtTileElems = 2 * kDqPart + kQtStatsElems;
static_assert(kDqTileElems * 2 == kBwdDqTileBytes && kQtTileElems * 2 == kBwdQtTileBytes, "tile sizes");

// Slot of lane l's 16 bytes within operand chunk s of a part: l with bit 2
// flipped in the upper half-wave and bit 3 flipped in odd chunks. Each aligned
// group of 16 lanes keeps its 256 bytes, so a wave's 16-byte operand reads of
// a chunk stay conflict-free, and the transposed 8-byte reads of lds_read_t8
// (four rows x 16 dims of two neighbouring chunks per 32 lanes) fall on
// distinct banks.
__device__ __forceinline__ int opslot(int l, int s) { return l ^ ((l >> 3) & 4) ^ ((s & 1) << 3); }

// Eight 16-byte LDS reads into distinct registers, read i at byte offset
// (i >> 1) * SO from base0 (i even) or base1 (i odd); the block waits for
// them itself.
template <int SO>
__device__ __forceinline__ void lds_read8x2(u32x4_t* r, const uint16_t* base0, const uint16_t* base1) {
    const uint32_t a0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)base0;
    const uint32_t a1 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)base1;
    asm volatile(
        "ds_read_b128 %0, %8 offset:0\n\t"
        "ds_read_b128 %1, %9 offset:0\n\t"
        "ds_read_b128 %2, %8 offset:%10\n\t"
        "ds_read_b128 %3, %9 offset:%10\n\t"
        "ds_read_b128 %4, %8 offset:%11\n\t"
        "ds_read_b128 %5, %9 offset:%11\n\t"
        "ds_read_b128 %6, %8 offset:%12\n\t"
        "ds_read_b128 %7, %9 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a0), "v"(a1), "n"(SO), "n"(2 * SO), "n"(3 * SO)
        : "memory");
}

// Operand chunks (h, 0 .. 7) of a part into r[0 .. 7] (this lane's slots)
__device__ __forceinline__ void lds_read_chunks(u32x4_t* r, const uint16_t* part, int h, int lane) {
    lds_read8x2<2048>(r, part + ((h * 8) * 64 + opslot(lane, 0)) * 8, part + ((h * 8 + 1) * 64 + opslot(lane, 1)) * 8);
}

// Element offset, within the 32-row half h = 0 of a part, that this lane
// addresses in the transposed read x (rows 8x ..) of chunk (db, h2) = (0, 0).
// ds_read_tr16_b64 gives lane i of each 16-lane group the 16-bit element i % 4
// of the 8 bytes addressed by lanes 4j + i / 4, j = 0 .. 3; lane c of group g
// therefore addresses row 16h2 + 8x + 4(g / 2) + c / 4 at dims
// 32db + 16(g % 2) + 4(c % 4) .. +3, and lane i receives those four rows at
// dim 32db + 16(g % 2) + i.
__device__ __forceinline__ int tr_lane_off(int lane, int x) {
    const int c = lane & 15, gd = (lane >> 4) & 1, hf = lane >> 5, hh = (c & 3) >> 1;
    // chunk s = 2db + gd; slot opslot(row + 32hh, s) = 32hh + 16h2 + 8(x ^ gd) + 4(hf ^ hh) + c / 4
    return gd * 512 + (32 * hh + 8 * (x ^ gd) + 4 * (hf ^ hh) + (c >> 2)) * 8 + 4 * (c & 1);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2_t lds_tr8(const uint16_t* p) {
    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
    return __builtin_bit_cast(u32x2_t, r);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS accesses inside the streaming loops, whose next tile is being copied
// into the other ring slot meanwhile. The compiler cannot tell that such an
// access stays clear of the copy's slot, so before any LDS access it can see
// it waits for all copies in flight (the prefetch would then have to land
// before the current tile's math); these helpers issue their accesses in one
// asm block, and the reads wait for themselves inside it.
//
// The eight A operand chunks (h, db, h2), i = 2db + h2, of X^T from a part
// holding X: lane l gets X[rows 32h + 16h2 + 8(e / 4) + 4(l / 32) + e % 4,
// e = 0 .. 7][dim 32db + l % 32], the row order in which a 32x32 score
// accumulator holds its rows; t0 / t1 = part + 4096h + tr_lane_off(lane, 0 / 1).
// Chunk i takes the transposing reads at element offset 1024(i / 2) +
// 128(i % 2) from t0 (its first four rows) and from t1.
__device__ __forceinline__ void lds_read_t8(u32x4_t* at, const uint16_t* t0, const uint16_t* t1) {
    u32x2_t r[16];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %17 offset:0\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:256\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:256\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:2048\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:2048\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:2304\n\t"
        "ds_read_b64_tr_b16 %7, %17 offset:2304\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:4096\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:4096\n\t"
        "ds_read_b64_tr_b16 %10, %16 offset:4352\n\t"
        "ds_read_b64_tr_b16 %11, %17 offset:4352\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:6144\n\t"
        "ds_read_b64_tr_b16 %13, %17 offset:6144\n\t"
        "ds_read_b64_tr_b16 %14, %16 offset:6400\n\t"
        "ds_read_b64_tr_b16 %15, %17 offset:6400\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
        : "v"(lds_addr(t0)), "v"(lds_addr(t1))
        : "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) at[i] = u32x4_t{r[2 * i][0], r[2 * i][1], r[2 * i + 1][0], r[2 * i + 1][1]};
}

// Four float4 at p, p + 8, p + 16, p + 24 (p 16-byte aligned).
__device__ __forceinline__ void lds_read_f4x4(float4* v, const float* p) {
    u32x4_t r[4];
    asm volatile(
        "ds_read_b128 %0, %4 offset:0\n\t"
        "ds_read_b128 %1, %4 offset:32\n\t"
        "ds_read_b128 %2, %4 offset:64\n\t"
        "ds_read_b128 %3, %4 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(lds_addr(p))
        : "memory");
#pragma unroll
    for (int g = 0; g < 4; ++g) v[g] = __builtin_bit_cast(float4, r[g]);
}

// v[e] = p[64 e], e = 0 .. 15. (The pairs come out as float2: taking the
// second word of an integer pair output and bit-casting it to float compiles
// to the first word.)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_read_col16(float* v, const float* p) {
    f32x2_t r[8];
    asm volatile(
        "ds_read2st64_b32 %0, %8 offset0:0 offset1:1\n\t"
        "ds_read2st64_b32 %1, %8 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %2, %8 offset0:4 offset1:5\n\t"
        "ds_read2st64_b32 %3, %8 offset0:6 offset1:7\n\t"
        "ds_read2st64_b32 %4, %8 offset0:8 offset1:9\n\t"
        "ds_read2st64_b32 %5, %8 offset0:10 offset1:11\n\t"
        "ds_read2st64_b32 %6, %8 offset0:12 offset1:13\n\t"
        "ds_read2st64_b32 %7, %8 offset0:14 offset1:15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(lds_addr(p))
        : "memory");
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        v[2 * k] = r[k][0];
        v[2 * k + 1] = r[k][1];
    }
}

// p[64 e] = v[e], e = 0 .. 15 (the caller waits for the stores before it
// signals them to other waves).
__device__ __forceinline__ void lds_write_col16(float* p, const float* v) {
    asm volatile(
        "ds_write2st64_b32 %0, %1, %2 offset0:0 offset1:1\n\t"
        "ds_write2st64_b32 %0, %3, %4 offset0:2 offset1:3\n\t"
        "ds_write2st64_b32 %0, %5, %6 offset0:4 offset1:5\n\t"
        "ds_write2st64_b32 %0, %7, %8 offset0:6 offset1:7\n\t"
        "ds_write2st64_b32 %0, %9, %10 offset0:8 offset1:9\n\t"
        "ds_write2st64_b32 %0, %11, %12 offset0:10 offset1:11\n\t"
        "ds_write2st64_b32 %0, %13, %14 offset0:12 offset1:13\n\t"
        "ds_write2st64_b32 %0, %15, %16 offset0:14 offset1:15"
        :
        : "v"(lds_addr(p)), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15])
        : "memory");
}

// The dQ kernel's tile [K | V] of every key block, from the rotated k rows
// (zero-padded to whole blocks) and v [L] (rows past L read as zero).
// Grid (nblk, BH).
__global__ __launch_bounds__(256) void k_bwd_dq_tiles(const uint16_t* __restrict__ kr, const uint16_t* __restrict__ v,
                                                      long L, int nblk, uint16_t* __restrict__ tiles) {
    constexpr int D = 128;
    const int tid = threadIdx.x, blk = blockIdx.x;
    const long bh = blockIdx.y;
    const uint16_t* ks = kr + (bh * nblk + blk) * 64l * D;   // zero rows past L
    const uint16_t* vs = v + bh * L * D;
    uint16_t* t = tiles + (bh * nblk + blk) * (long)kDqTileElems;
    // thread takes dims 8c .. 8c+7 of rows 16p + tid/16
    const int c = tid & 15, rs = tid >> 4;
    u32x4_t xk[4], xv[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = 16 * p + rs;
        const long l = (long)blk * 64 + r;
        xk[p] = ldg16(ks + (long)r * D + 8 * c);
        const u32x4_t w = ldg16(vs + (l < L ? l : L - 1) * D + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[p][i] = l < L ? w[i] : 0u;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = 16 * p + rs;
        const int o = (((r >> 5) * 8 + (c >> 1)) * 64 + opslot((r & 31) + 32 * (c & 1), c >> 1)) * 8;
        stg16(t + o, xk[p]);
        stg16(t + kDqPart + o, xv[p]);
    }
}

// Low-rank part of a streaming kernel's output rows, formed in its epilogue
// instead of read back from fp32 copies: y[db] (the accumulator layout of the
// wave's 32 rows: lane row l % 32, register i = dim 32db + 8(i/4) + 4hf + i%4)
// = A x, with x the row's rank vector stored by the low-rank kernels (bf16
// hi + lo at xh / xl + row * rv; in the slot16 order of a product over r,
// lane half hf takes ranks 16ks + 4hf + 0..3 and 16ks + 8 + 4hf + 0..3 of
// k-step ks) and A [128][R] given as operand blocks (block (db, ks) =
// db * KS + ks, 64 lanes x 16 bytes, KS = R / 16; as k_bwd_lr_opblocks lays
// them out): W rounded to bf16 (alo null), or dS^T as hi + lo parts (three
// products), as the low-rank kernels form them. Run by the whole wave (each
// lane supplies its A row); rows with valid false add zero. The operands of
// two k-steps are loaded together (LrOps), so that a kernel can request the
// first pair before the barriers of its partial-sum merge and the load
// latency overlaps them.
struct LrOps {
    u32x4_t bh[2], bl[2], wh[2][4], wl[2][4];   // wl used only with the lo part (LO)
};
struct LrSrc {
    const u32x4_t* ahi;
    const u32x4_t* alo;
    const uint16_t* xh;
    const uint16_t* xl;
    long row;
    bool valid;
    int rv;
};
template <bool LO>
__device__ __forceinline__ void lr_rows_load(const LrSrc& src, int ks0, int lane, int hf, LrOps& o) {
    const int KS = src.rv <= 32 ? 2 : 4;   // rank padded to 32 or 64
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int ks = ks0 + k;
        o.bh[k] = u32x4_t{0u, 0u, 0u, 0u};
        o.bl[k] = u32x4_t{0u, 0u, 0u, 0u};
        const int r0 = 16 * ks + 4 * hf, r1 = r0 + 8;
        if (src.valid && r0 < src.rv) {
            const u32x2_t h = *reinterpret_cast<const u32x2_t*>(src.xh + src.row * src.rv + r0);
            const u32x2_t l = *reinterpret_cast<const u32x2_t*>(src.xl + src.row * src.rv + r0);
            o.bh[k][0] = h[0]; o.bh[k][1] = h[1]; o.bl[k][0] = l[0]; o.bl[k][1] = l[1];
        }
        if (src.valid && r1 < src.rv) {
            const u32x2_t h = *reinterpret_cast<const u32x2_t*>(src.xh + src.row * src.rv + r1);
            const u32x2_t l = *reinterpret_cast<const u32x2_t*>(src.xl + src.row * src.rv + r1);
            o.bh[k][2] = h[0]; o.bh[k][3] = h[1]; o.bl[k][2] = l[0]; o.bl[k][3] = l[1];
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            o.wh[k][db] = src.ahi[(db * KS + ks) * 64 + lane];
            if (LO) o.wl[k][db] = src.alo[(db * KS + ks) * 64 + lane];
        }
    }
}
template <bool LO>
__device__ __forceinline__ void lr_rows_mfma(const LrOps& o, f32x16_t* y) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            y[db] = mfma32(o.wh[k][db], o.bh[k], y[db]);
            y[db] = mfma32(o.wh[k][db], o.bl[k], y[db]);
            if (LO) y[db] = mfma32(o.wl[k][db], o.bh[k], y[db]);
        }
}
// Adds the product to y given the operands of k-steps 0 and 1 (loaded by the
// caller); loads the rest at rank 64.
template <bool LO>
__device__ __forceinline__ void lr_rows_finish(const LrSrc& src, LrOps& o, int lane, int hf, f32x16_t* y) {
    lr_rows_mfma<LO>(o, y);
    if (src.rv > 32) {
        lr_rows_load<LO>(src, 2, lane, hf, o);
        lr_rows_mfma<LO>(o, y);
    }
}

// Workgroup = 4 waves = one 64-row query block; wave (rh, kh) owns query rows
// 32rh .. and keys 32kh .. of every kept tile: S^T = K Q^T and dP^T = V dO^T
// (a lane owns one query row), dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T.
// The tiles stream through a two-slot LDS ring (64 KB: two workgroups per
// CU), each requested one tile ahead, one barrier per tile; K^T comes from
// the K part by transposing reads. The two key halves' dQ^T are added through
// LDS at the end. The tiled path scores with q pre-multiplied by
// log2(e)/sqrt(D), so p = exp2(score - lse2).
__global__ __launch_bounds__(256, 2) void k_bwd_dq_tiled(BwdArgs a, const int32_t* __restrict__ idx_all,
                                                      const uint16_t* __restrict__ tiles_all) {
    constexpr int D = 128, BS = 64, PART = kDqPart, PLOADS = PART * 2 / (256 * 16);
    __shared__ __attribute__((aligned(16))) uint16_t lds[4 * PART];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rh = wave & 1, kh = wave >> 1;
    const int l32 = lane & 31, hf = lane >> 5;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const int nblk = a.nblk;
    const long bh = wid / nblk;
    const int qb = (int)(wid % nblk);
    const long rows = (long)nblk * BS;
    const long L = a.L;
    const long qrow = (long)qb * BS + 32 * rh + l32;
    const bool qval = qrow < L;
    const uint16_t* tiles = tiles_all + bh * (long)nblk * kDqTileElems + (long)tid * 8;
    const int32_t* ix = idx_all + (bh * nblk + qb) * (long)a.keep;
    const int ntile = a.keep;

    // B operands: rotated (scaled) q row and dO row (dims 16s + 8hf + e); delta = dO . O
    u32x4_t qop[8], doop[8];
    float dl = 0.f;
    {
        const uint16_t* qp = a.qr + (bh * rows + qrow) * D + 8 * hf;
        const long orow = bh * L + (qval ? qrow : 0);
        const uint16_t* dp = a.dout + orow * D + 8 * hf;
        const uint16_t* op = a.o_sp + orow * D + 8 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            qop[s] = ldg16(qp + 16 * s);
            const u32x4_t dd = ldg16(dp + 16 * s);
            const u32x4_t o = ldg16(op + 16 * s);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                doop[s][i] = qval ? dd[i] : 0u;
                dl += bf_lo(doop[s][i]) * bf_lo(o[i]) + bf_hi(doop[s][i]) * bf_hi(o[i]);
            }
        }
    }
    dl = sum_xor32(dl);
    const float lse2 = qval ? a.lse_in[bh * L + (qval ? qrow : 0)] : 0.f;
    wait_vmcnt<0>();
    // the row statistics, zero on padded rows, for the key-side kernel
    if (kh == 0 && hf == 0) {
        a.lse2[bh * rows + qrow] = lse2;
        a.delta[bh * rows + qrow] = qval ? dl : 0.f;
    }
    if (a.qtt) {
        // this query block's tile [Q | dO | stats] for the streaming dK/dV
        // kernel: qop / doop already are the Q / dO chunks (rh, s) of this lane
        // (waves kh = 0 store Q, kh = 1 dO)
        uint16_t* qt = const_cast<uint16_t*>(a.qtt) + (bh * nblk + qb) * (long)kQtTileElems;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            stg16(qt + kh * PART + ((rh * 8 + s) * 64 + opslot(lane, s)) * 8, kh == 0 ? qop[s] : doop[s]);
        if (hf == 0) {
            float* st = reinterpret_cast<float*>(qt + 2 * PART);
            st[(kh == 0 ? 0 : 64) + 32 * rh + l32] = kh == 0 ? lse2 : (qval ? dl : 0.f);
        }
    }

    // entries outside [0, nblk) contribute nothing (their slot streams tile 0)
    auto tile_of = [&](int n) -> int {
        const int j = ix[n];
        return (unsigned)j < (unsigned)nblk ? j : 0;
    };
    // tile j -> ring slot sl: K to part sl, V to part 2 + sl
    auto issue = [&](int j, int sl) {
        const uint16_t* src = tiles + (long)j * kDqTileElems;
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int m = 0; m < PLOADS; ++m)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(src + p * PART + m * 256 * 8),
                    (__attribute__((address_space(3))) void*)(lds + (2 * p + sl) * PART + (m * 256 + wave * 64) * 8),
                    16, 0, 0);
    };
    const bool ragged = (L % BS) != 0;
    const int tr0 = kh * 4096 + tr_lane_off(lane, 0), tr1 = kh * 4096 + tr_lane_off(lane, 1);

    f32x16_t dqacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

    // tile t in slot t % 2; tile t + 1 is requested right after the barrier
    // that opens tile t (which certifies that every wave is done with tile
    // t - 1, whose slot it takes)
    if (ntile > 0) issue(tile_of(0), 0);
    for (int t = 0; t < ntile; ++t) {
        const int jraw = ix[t];
        const bool jok = (unsigned)jraw < (unsigned)nblk;
        const int sl = t & 1;
        wait_vmcnt<0>();   // tile t landed (the only copies in flight)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t + 1 < ntile) issue(tile_of(t + 1), sl ^ 1);
        const uint16_t* kp = lds + sl * PART;
        f32x16_t sacc, dpacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
        u32x4_t op[8];
        lds_read_chunks(op, kp, kh, lane);
#pragma unroll
        for (int s = 0; s < 8; ++s) sacc = mfma32(op[s], qop[s], sacc);
        u32x4_t vop[8];
        lds_read_chunks(vop, lds + (2 + sl) * PART, kh, lane);
#pragma unroll
        for (int s = 0; s < 8; ++s) dpacc = mfma32(vop[s], doop[s], dpacc);
        u32x4_t at[8];   // K^T chunks (kh, db, h2) = (kh, i / 2, i % 2)
        lds_read_t8(at, kp + tr0, kp + tr1);
        // entry i of this lane is key 64 jraw + 32 kh + 4 hf + 8(i / 4) + i % 4: the number of
        // keys from the first one that lie in the layer (0 .. 64)
        const int kleft =
            ragged ? (int)max(0l, min(L - ((long)jraw * BS + 32 * kh + 4 * hf), (long)BS)) : BS;
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            // an entry off the layer or of a skipped block gets exp2(-inf) = 0 (its dP is
            // finite: a skipped entry streams tile 0): the select sits before the exp, so the
            // compiler has no reason to branch around the exp of each entry
            const bool off = !jok || 8 * (i >> 2) + (i & 3) >= kleft;
            ds[i] = __builtin_amdgcn_exp2f(off ? -__builtin_inff() : sacc[i] - lse2) * (dpacc[i] - dl);
        }
        u32x4_t dsop[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < 4; ++i) dsop[h2][i] = pack_bf2(ds[8 * h2 + 2 * i], ds[8 * h2 + 2 * i + 1]);
#pragma unroll
        for (int i = 0; i < 8; ++i) dqacc[i >> 1] = mfma32(at[i], dsop[i & 1], dqacc[i >> 1]);
    }

    // the low-rank part W_q dpq of the wave's rows, unless it was stored in fp32: the key-half-0
    // waves request its first operands now (whole wave)
    const bool fused = a.lr_ph != nullptr;
    const LrSrc lrs{reinterpret_cast<const u32x4_t*>(a.lr_w) + (bh % a.H) * (a.lr_rv <= 32 ? 512 : 1024), nullptr,
                    a.lr_ph, a.lr_pl, bh * L + (qval ? qrow : 0), qval, a.lr_rv};
    LrOps lro;
    if (fused && kh == 0) lr_rows_load<false>(lrs, 0, lane, hf, lro);

    // ---- add the key halves through LDS (no copy is in flight: the last tile waited for all)
    __syncthreads();
    float* mrg = reinterpret_cast<float*>(lds) + rh * (64 * 64);
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) mrg[(16 * db + i) * 64 + lane] = dqacc[db][i];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqacc[db][i] += mrg[(16 * db + i) * 64 + lane];
    f32x16_t lrp[4];
    if (fused) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) lrp[db][i] = 0.f;
        lr_rows_finish<false>(lrs, lro, lane, hf, lrp);
    }
    if (!qval) return;

    // ---- epilogue: dq = R^T (dQ_rot / sqrt(D)) + dq_lowrank; lane owns row qrow
    int crd[3];
    token_coords(qrow, a.g.Hg, a.g.Wg, crd[0], crd[1], crd[2]);
    uint16_t* out = a.dq + (bh * L + qrow) * D;
    if (fused)
        rotate_store_row<true, 8>(a.tab, a.g, crd, dqacc, a.scale, lrp, nullptr, out, hf);
    else
        rotate_store_row<false, 8>(a.tab, a.g, crd, dqacc, a.scale, lrp, a.dq_lr + (bh * L + qrow) * D, out, hf);
}

// ---------------------------------------------------------------------------
// Streaming dK, dV for bf16, D = 128, 64-token blocks. Workgroup = 8 waves =
// one 64-key block; waves 0..3 accumulate dV^T, waves 4..7 dK^T, and wave
// w & 3 = (kw, qh) takes keys 32kw .. and query rows 32qh .. of every query
// block that keeps the key block. A lane owns one key, register e of an
// accumulator the row 32qh + 8(e/4) + 4hf + e%4. The dV wave computes
// S = Q K^T and P, passes P (fp32) to the dK wave of the same (kw, qh)
// through LDS and adds dO^T P; the dK wave meanwhile computes dP = dO V^T,
// then dS = P (dP - delta), and adds Q^T dS: 16 MFMAs per wave per tile.
// Waves w and w + 4 share a SIMD, one of each role (two waves per SIMD). The
// query-side tiles [Q | dO | stats] stream through a two-slot LDS ring
// (68 KB, and 16 KB for P), requested one tile ahead; Q^T and dO^T come from
// the Q and dO parts by transposing reads. Two barriers per tile (tile
// landed, P handed over). The query halves' partial sums are added through
// LDS at the end.
template <int ROLE>
__device__ __forceinline__ void dkdv_tiled_loop(const BwdArgs& a, uint16_t* lds, const uint16_t* qt,
                                                const int32_t* list, int n0, int n1, int tid, int wave, int lane,
                                                int qh, int hf, const u32x4_t* op, float* pex,
                                                f32x16_t* acc) {
    constexpr int PART = kDqPart, TILE = kQtTileElems, PL = PART * 2 / (512 * 16);
    constexpr int FSZ = 2 * PART + kQtStatsElems;   // one slot: [Q | dO | stats]
    // Tile i -> a slot: Q, dO (two 16-byte copies per lane each) and the 2 KB
    // of row statistics (one 4-byte copy per lane)
    auto issue_f = [&](int i, uint16_t* slot) {
        const uint16_t* src = qt + (long)i * TILE;
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int m = 0; m < PL; ++m)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(src + p * PART + (m * 512 + tid) * 8),
                    (__attribute__((address_space(3))) void*)(slot + p * PART + (m * 512 + wave * 64) * 8), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + 2 * PART + tid * 2),
                                         (__attribute__((address_space(3))) void*)(slot + 2 * PART + wave * 128), 4,
                                         0, 0);
    };
    auto qblock = [&](int n) { return __builtin_amdgcn_readfirstlane(list[n]); };
    const int ntile = n1 - n0;
    // transposed reads of Q (dK waves) or dO (dV waves): this lane's addresses in part 0
    const int tpart = ROLE == 0 ? PART : 0;
    const int tr0 = tpart + qh * 4096 + tr_lane_off(lane, 0), tr1 = tpart + qh * 4096 + tr_lane_off(lane, 1);
    // Tile t in slot t % 2; tile t + 1 is requested right after the barrier
    // that opens tile t (which certifies that every wave is done with tile
    // t - 1, whose slot it takes).
    if (ntile > 0) issue_f(qblock(n0), lds);
    for (int t = 0; t < ntile; ++t) {
        wait_vmcnt<0>();   // tile t landed (the only copies in flight)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t + 1 < ntile) issue_f(qblock(n0 + t + 1), lds + ((t + 1) & 1) * FSZ);
        const uint16_t* cur = lds + (t & 1) * FSZ;
        const float* st = reinterpret_cast<const float*>(cur + 2 * PART) + 32 * qh + 4 * hf;
        // dV waves: S = Q K^T and P, handed to the dK wave of the same (kw, qh)
        // through LDS; dK waves meanwhile: dP = dO V^T
        f32x16_t sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
        u32x4_t aq[8];
        lds_read_chunks(aq, cur + (ROLE == 0 ? 0 : PART), qh, lane);
#pragma unroll
        for (int s = 0; s < 8; ++s) sacc = mfma32(aq[s], op[s], sacc);
        u32x4_t bop[2];   // P (dV waves) or dS (dK waves): the keys' B operand of the second product
        if constexpr (ROLE == 0) {
            float p[16];
            float4 l4[4];   // the rows' log2 normalisers
            lds_read_f4x4(l4, st);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                p[4 * g + 0] = __builtin_amdgcn_exp2f(sacc[4 * g + 0] * a.qmul - l4[g].x);
                p[4 * g + 1] = __builtin_amdgcn_exp2f(sacc[4 * g + 1] * a.qmul - l4[g].y);
                p[4 * g + 2] = __builtin_amdgcn_exp2f(sacc[4 * g + 2] * a.qmul - l4[g].z);
                p[4 * g + 3] = __builtin_amdgcn_exp2f(sacc[4 * g + 3] * a.qmul - l4[g].w);
            }
            lds_write_col16(pex + lane, p);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int e = 0; e < 4; ++e) bop[h2][e] = pack_bf2(p[8 * h2 + 2 * e], p[8 * h2 + 2 * e + 1]);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // P stored before the barrier below
        }
        __builtin_amdgcn_s_barrier();   // P is in LDS
        asm volatile("" ::: "memory");
        if constexpr (ROLE == 1) {
            float ds[16], pv[16];
            float4 d4[4];   // the rows' delta = dO . O
            lds_read_f4x4(d4, st + 64);
            lds_read_col16(pv, pex + lane);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                ds[4 * g + 0] = pv[4 * g + 0] * (sacc[4 * g + 0] - d4[g].x);
                ds[4 * g + 1] = pv[4 * g + 1] * (sacc[4 * g + 1] - d4[g].y);
                ds[4 * g + 2] = pv[4 * g + 2] * (sacc[4 * g + 2] - d4[g].z);
                ds[4 * g + 3] = pv[4 * g + 3] * (sacc[4 * g + 3] - d4[g].w);
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int e = 0; e < 4; ++e) bop[h2][e] = pack_bf2(ds[8 * h2 + 2 * e], ds[8 * h2 + 2 * e + 1]);
        }
        u32x4_t at[8];   // dO^T (dV waves) or Q^T (dK waves) chunks (qh, db, h2) = (qh, i / 2, i % 2)
        lds_read_t8(at, cur + tr0, cur + tr1);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i >> 1] = mfma32(at[i], bop[i & 1], acc[i >> 1]);
    }
}

// The end of k_bwd_dkdv_tiled for the waves of one role: the query halves'
// partial sums added through LDS, then dv = dV + dv_lowrank (dV waves) or
// dk = R^T (kscale dK_rot) + dk_lowrank (dK waves); the lane owns key `key`,
// dims 32db + 8g4 + 4hf + 0..3. The low-rank part (unless it was stored in
// fp32) is dS^T fk, accumulated onto dV by the MFMAs, or W_k dpk; the
// query-half-0 waves request the operands of its first two k-steps before
// the merge, so that their latency overlaps it.
template <int ROLE>
__device__ __forceinline__ void dkdv_tiled_tail(const BwdArgs& a, uint16_t* lds, f32x16_t* acc, long bh, long key,
                                                bool kval, int kw, int qh, int lane, int hf) {
    constexpr int D = 128;
    const long L = a.L;
    const bool fused = a.lr_ph != nullptr;
    const long nb = a.lr_rv <= 32 ? 512 : 1024;   // 16-byte entries of one operand matrix
    const long lrow = bh * L + (kval ? key : 0);
    const LrSrc lrs = ROLE == 0 ? LrSrc{reinterpret_cast<const u32x4_t*>(a.lr_sh) + bh * nb,
                                        reinterpret_cast<const u32x4_t*>(a.lr_sl) + bh * nb, a.lr_fh, a.lr_fl,
                                        lrow, kval, a.lr_rv}
                                : LrSrc{reinterpret_cast<const u32x4_t*>(a.lr_w) + (bh % a.H) * nb, nullptr, a.lr_ph,
                                        a.lr_pl, lrow, kval, a.lr_rv};
    LrOps lro;
    if (fused && qh == 0) lr_rows_load<ROLE == 0>(lrs, 0, lane, hf, lro);

    // ---- add the query halves through LDS (no copy is in flight: the last tile waited for all)
    __syncthreads();
    float* mrg = reinterpret_cast<float*>(lds) + (ROLE * 2 + kw) * (64 * 64);
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) mrg[(16 * db + i) * 64 + lane] = acc[db][i];
    }
    __syncthreads();
    if (qh == 1) return;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] += mrg[(16 * db + i) * 64 + lane];

    const long ro = (bh * L + key) * D;
    if (ROLE == 0) {
        if (fused) lr_rows_finish<true>(lrs, lro, lane, hf, acc);   // whole wave
        if (!kval) return;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * db + 8 * g4 + 4 * hf;
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = acc[db][4 * g4 + i];
                if (!fused) {
                    const float4 vl = *reinterpret_cast<const float4*>(a.dv_lr + ro + d0);
                    y[0] += vl.x; y[1] += vl.y; y[2] += vl.z; y[3] += vl.w;
                }
                *reinterpret_cast<u32x2_t*>(a.dv + ro + d0) = u32x2_t{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
            }
        return;
    }
    f32x16_t lrp[4];
    if (fused) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) lrp[db][i] = 0.f;
        lr_rows_finish<false>(lrs, lro, lane, hf, lrp);   // whole wave
    }
    if (!kval) return;
    int crd[3];
    token_coords(key, a.g.Hg, a.g.Wg, crd[0], crd[1], crd[2]);
    if (fused)
        rotate_store_row<true, 4>(a.tab, a.g, crd, acc, a.kscale, lrp, nullptr, a.dk + ro, hf);
    else
        rotate_store_row<false, 4>(a.tab, a.g, crd, acc, a.kscale, lrp, a.dk_lr + ro, a.dk + ro, hf);
}

__global__ __launch_bounds__(512) void k_bwd_dkdv_tiled(BwdArgs a, const int32_t* __restrict__ inv_off,
                                                        const int32_t* __restrict__ inv_list,
                                                        const int32_t* __restrict__ order,
                                                        const uint16_t* __restrict__ qt_all) {
    constexpr int D = 128, BS = 64, TILE = kQtTileElems;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (2 * kDqPart + kQtStatsElems)];
    __shared__ float pex_all[4][16 * 64];   // P of each (kw, qh), from the dV wave to the dK wave

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = wave >> 2, kw = wave & 1, qh = (wave >> 1) & 1;
    const int l32 = lane & 31, hf = lane >> 5;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const int nblk = a.nblk;
    const long bh = wid / nblk;
    // key blocks of a slice run longest list first
    const int jb = __builtin_amdgcn_readfirstlane(order[bh * nblk + wid % nblk]);
    const long rows = (long)nblk * BS;
    const long L = a.L;
    const long key = (long)jb * BS + 32 * kw + l32;
    const bool kval = key < L;
    const uint16_t* qt = qt_all + bh * (long)nblk * TILE;
    const int32_t* off = inv_off + bh * (long)(nblk + 1);
    const int32_t* list = inv_list + bh * (long)nblk * a.keep;
    const int n0 = __builtin_amdgcn_readfirstlane(off[jb]), n1 = __builtin_amdgcn_readfirstlane(off[jb + 1]);

    f32x16_t acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    // B operand of the first product: rotated k row of this lane's key (dV
    // waves: S = Q K^T) or its v row (dK waves: dP = dO V^T); dims 16s + 8hf + e
    u32x4_t op[8];
    {
        const uint16_t* src = role == 0 ? a.kr + (bh * rows + key) * D : a.v + (bh * L + (kval ? key : 0)) * D;
        const bool zero = role == 1 && !kval;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4_t w = ldg16(src + 8 * hf + 16 * s);
#pragma unroll
            for (int i = 0; i < 4; ++i) op[s][i] = zero ? 0u : w[i];
        }
    }
    wait_vmcnt<0>();
    float* pex = pex_all[kw * 2 + qh];
    if (role == 0)
        dkdv_tiled_loop<0>(a, lds, qt, list, n0, n1, tid, wave, lane, qh, hf, op, pex, acc);
    else
        dkdv_tiled_loop<1>(a, lds, qt, list, n0, n1, tid, wave, lane, qh, hf, op, pex, acc);

    if (role == 0)
        dkdv_tiled_tail<0>(a, lds, acc, bh, key, kval, kw, qh, lane, hf);
    else
        dkdv_tiled_tail<1>(a, lds, acc, bh, key, kval, kw, qh, lane, hf);
}

// ---------------------------------------------------------------------------
// dK, dV. Workgroup = one key block, BS/32 waves of 32 keys.
template <int D, int BS>
__global__ __launch_bounds__(BS * 2) void k_bwd_dkdv(BwdArgs a, const int32_t* __restrict__ inv_off,
                                                   const int32_t* __restrict__ inv_list,
                                                   const int32_t* __restrict__ order) {
    constexpr int KLD = D + 8, VLD = BS + 8, NQB = BS / 32, NS = D / 16, NDB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[BS * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t do_lds[BS * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t qt_lds[D * VLD];
    __shared__ __attribute__((aligned(16))) uint16_t dot_lds[D * VLD];
    __shared__ float lse_lds[BS], dl_lds[BS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const long bh = wid / a.nblk;
    // key blocks of a slice run longest list first
    const int jb = order ? __builtin_amdgcn_readfirstlane(order[bh * a.nblk + wid % a.nblk]) : (int)(wid % a.nblk);
    const long rows = (long)a.nblk * BS;
    const long L = a.L;
    const long key = (long)jb * BS + 32 * wave + l32;
    const bool kval = key < L;
    const uint16_t* qr = a.qr + bh * rows * D;
    const uint16_t* dg = a.dout + bh * L * D;

    // B operands: rotated k row and v row of this lane's key (dims 16s + 8hf + e)
    u32x4_t kop[NS], vop[NS];
    {
        const uint16_t* kp = a.kr + (bh * rows + key) * D + 8 * hf;
        const uint16_t* vp = a.v + (bh * L + (kval ? key : 0)) * D + 8 * hf;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kop[s] = ldg16(kp + 16 * s);
            vop[s] = kval ? ldg16(vp + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    f32x16_t dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) { dkacc[db][i] = 0.f; dvacc[db][i] = 0.f; }

    const int32_t* off = inv_off + bh * (long)(a.nblk + 1);
    const int32_t* list = inv_list + bh * (long)a.nblk * a.keep;
    const int n0 = __builtin_amdgcn_readfirstlane(off[jb]), n1 = __builtin_amdgcn_readfirstlane(off[jb + 1]);
    auto qblock_at = [&](int n) { return __builtin_amdgcn_readfirstlane(list[n]); };
    const Stager<D, BS> stg(tid);
    u32x4_t xq[8], xd[8];   // next query block's rows, in flight while the current one is consumed
    float xl = 0.f, xdl = 0.f;
    uint32_t okq = 0, okd = 0;
    auto fetch = [&](int i) {
        okq = stg.fetch(xq, qr, (long)i * BS, rows);
        okd = stg.fetch(xd, dg, (long)i * BS, L);
        if (tid < BS) {
            xl = a.lse2[bh * rows + (long)i * BS + tid];
            xdl = a.delta[bh * rows + (long)i * BS + tid];
        }
    };
    if (n0 < n1) fetch(qblock_at(n0));
    // nothing from the prologue stays in flight into the loop
    wait_vmcnt<0>();
    for (int n = n0; n < n1; ++n) {
        __syncthreads();
        stg.stash(xq, okq, q_lds, qt_lds);
        stg.stash(xd, okd, do_lds, dot_lds);
        if (tid < BS) {
            lse_lds[tid] = xl;
            dl_lds[tid] = xdl;
        }
        __syncthreads();
        if (n + 1 < n1) fetch(qblock_at(n + 1));
#pragma unroll
        for (int qs = 0; qs < NQB; ++qs) {
            f32x16_t sacc, dpacc;
#pragma unroll
            for (int e = 0; e < 16; ++e) { sacc[e] = 0.f; dpacc[e] = 0.f; }
            if constexpr (NS == 8) {
                u32x4_t aq[8], ad[8];
                lds_read8x<32, 64>(aq, q_lds + (32 * qs + l32) * KLD + 8 * hf);
                lds_read8x<32, 64>(ad, do_lds + (32 * qs + l32) * KLD + 8 * hf);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    sacc = mfma32(aq[s], kop[s], sacc);
                    dpacc = mfma32(ad[s], vop[s], dpacc);
                }
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const int o = (32 * qs + l32) * KLD + 16 * s + 8 * hf;
                    sacc = mfma32(*reinterpret_cast<const u32x4_t*>(q_lds + o), kop[s], sacc);
                    dpacc = mfma32(*reinterpret_cast<const u32x4_t*>(do_lds + o), vop[s], dpacc);
                }
            }
            // lane = key, register e = query row 32qs + 8(e/4) + 4hf + e%4
            float p[16], ds[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 32 * qs + 8 * (e >> 2) + 4 * hf + (e & 3);
                p[e] = exp2f(sacc[e] * a.qmul - lse_lds[r]);
                ds[e] = p[e] * (dpacc[e] - dl_lds[r]);
            }
            u32x4_t pb[2], dsb[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pb[h2][e] = pack_bf2(p[8 * h2 + 2 * e], p[8 * h2 + 2 * e + 1]);
                    dsb[h2][e] = pack_bf2(ds[8 * h2 + 2 * e], ds[8 * h2 + 2 * e + 1]);
                }
            if constexpr (NDB == 4) {
                u32x4_t at[8], aq[8];   // (db, h2) = (i / 2, i % 2)
                lds_read8x<32, 64 * VLD>(at, dot_lds + l32 * VLD + 32 * qs + 8 * hf);
                lds_read8x<32, 64 * VLD>(aq, qt_lds + l32 * VLD + 32 * qs + 8 * hf);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    dvacc[i >> 1] = mfma32(at[i], pb[i & 1], dvacc[i >> 1]);
                    dkacc[i >> 1] = mfma32(aq[i], dsb[i & 1], dkacc[i >> 1]);
                }
            } else {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int o = (32 * db + l32) * VLD + 32 * qs + 16 * h2 + 8 * hf;
                        dvacc[db] = mfma32(*reinterpret_cast<const u32x4_t*>(dot_lds + o), pb[h2], dvacc[db]);
                        dkacc[db] = mfma32(*reinterpret_cast<const u32x4_t*>(qt_lds + o), dsb[h2], dkacc[db]);
                    }
            }
        }
    }

    // ---- epilogue: dk = R^T (dK_rot / sqrt(D)) + dk_lowrank, dv = dV + dv_lowrank
    if (!kval) return;
    int crd[3];
    token_coords(key, a.g.Hg, a.g.Wg, crd[0], crd[1], crd[2]);
    const long ro = (bh * L + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * db + 8 * g4 + 4 * hf;
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = dkacc[db][4 * g4 + i] * a.kscale;
            rot_t(y[0], y[1], rope_cs(a.tab, a.g, d0 >> 1, crd));
            rot_t(y[2], y[3], rope_cs(a.tab, a.g, (d0 >> 1) + 1, crd));
            const float4 kl = *reinterpret_cast<const float4*>(a.dk_lr + ro + d0);
            const float4 vl = *reinterpret_cast<const float4*>(a.dv_lr + ro + d0);
            *reinterpret_cast<u32x2_t*>(a.dk + ro + d0) =
                u32x2_t{pack_bf2(y[0] + kl.x, y[1] + kl.y), pack_bf2(y[2] + kl.z, y[3] + kl.w)};
            const f32x16_t& dv = dvacc[db];
            *reinterpret_cast<u32x2_t*>(a.dv + ro + d0) =
                u32x2_t{pack_bf2(dv[4 * g4] + vl.x, dv[4 * g4 + 1] + vl.y),
                        pack_bf2(dv[4 * g4 + 2] + vl.z, dv[4 * g4 + 3] + vl.w)};
        }
}

// ---------------------------------------------------------------------------
// fp32 layers: the same two kernels in fp32 VALU (the precision the tiny fp32
// check layer asks for). Thread (row, c) owns the 32 dims 32c .. 32c+31 of one
// row (NC = D/32 threads per row); a row's dot products add the NC partial
// sums with lane swaps. Key (dq) or query (dk, dv) rows of a block are staged
// in LDS as fp32.
template <int NC>
__device__ __forceinline__ float sum_lanes(float x) {
    x += __shfl_xor(x, 1, 64);
    if (NC == 4) x += __shfl_xor(x, 2, 64);
    return x;
}

template <int D>
__global__ __launch_bounds__(256) void k_bwd_dq_f32(BwdArgs a, const int32_t* __restrict__ idx_all, int BS) {
    constexpr int NC = D / 32;
    __shared__ float k_s[64 * (D + 1)];
    __shared__ float v_s[64 * (D + 1)];
    const int tid = threadIdx.x, row = tid / NC, c = tid % NC;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const long bh = wid / a.nblk;
    const int qb = (int)(wid % a.nblk);
    const long rows = (long)a.nblk * BS;
    const long L = a.L;
    const bool act = row < BS;
    const long qrow = (long)qb * BS + (act ? row : 0);
    const bool qval = act && qrow < L;
    const float* qr = (const float*)(const void*)a.qr + bh * rows * D;
    const float* kr = (const float*)(const void*)a.kr + bh * rows * D;
    const float* vg = (const float*)(const void*)a.v + bh * L * D;
    const float* dg = (const float*)(const void*)a.dout + bh * L * D;
    const float* og = (const float*)(const void*)a.o_sp + bh * L * D;
    const int32_t* ix = idx_all + (bh * a.nblk + qb) * (long)a.keep;
    float q[32], g[32], acc[32];
    float dl = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int d = 32 * c + i;
        q[i] = qr[qrow * D + d];
        g[i] = qval ? dg[qrow * D + d] : 0.f;
        dl += qval ? g[i] * og[qrow * D + d] : 0.f;
        acc[i] = 0.f;
    }
    dl = sum_lanes<NC>(dl);
    const float lse2 = qval ? a.lse_in[bh * L + qrow] : 0.f;
    if (act && c == 0) {
        a.lse2[bh * rows + qrow] = lse2;
        a.delta[bh * rows + qrow] = qval ? dl : 0.f;
    }
    for (int n = 0; n < a.keep; ++n) {
        const int j = ix[n];
        if (j < 0 || j >= a.nblk) continue;
        __syncthreads();
        for (int e = tid; e < BS * D; e += 256) {
            const int r = e / D, d = e % D;
            const long key = (long)j * BS + r;
            k_s[r * (D + 1) + d] = kr[key * D + d];
            v_s[r * (D + 1) + d] = key < L ? vg[key * D + d] : 0.f;
        }
        __syncthreads();
        for (int r = 0; r < BS; ++r) {
            if ((long)j * BS + r >= L) break;
            const float* kk = k_s + r * (D + 1) + 32 * c;
            const float* vv = v_s + r * (D + 1) + 32 * c;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                s += q[i] * kk[i];
                dp += g[i] * vv[i];
            }
            s = sum_lanes<NC>(s);
            dp = sum_lanes<NC>(dp);
            const float ds = exp2f(s * a.qmul - lse2) * (dp - dl);
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] += ds * kk[i];
        }
    }
    if (!qval) return;
    int crd[3];
    token_coords(qrow, a.g.Hg, a.g.Wg, crd[0], crd[1], crd[2]);
    float* out = (float*)(void*)a.dq + (bh * L + qrow) * D;
    const float* lr = a.dq_lr + (bh * L + qrow) * D;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
        const int d = 32 * c + i;
        float y0 = acc[i] * a.scale, y1 = acc[i + 1] * a.scale;
        rot_t(y0, y1, rope_cs(a.tab, a.g, d >> 1, crd));
        out[d] = y0 + lr[d];
        out[d + 1] = y1 + lr[d + 1];
    }
}

template <int D>
__global__ __launch_bounds__(256) void k_bwd_dkdv_f32(BwdArgs a, const int32_t* __restrict__ inv_off,
                                                      const int32_t* __restrict__ inv_list, int BS) {
    constexpr int NC = D / 32;
    __shared__ float q_s[64 * (D + 1)];
    __shared__ float g_s[64 * (D + 1)];
    __shared__ float lse_s[64], dl_s[64];
    const int tid = threadIdx.x, row = tid / NC, c = tid % NC;
    const long wid = xcd_remap(blockIdx.x, a.nwg);
    const long bh = wid / a.nblk;
    const int jb = (int)(wid % a.nblk);
    const long rows = (long)a.nblk * BS;
    const long L = a.L;
    const bool act = row < BS;
    const long key = (long)jb * BS + (act ? row : 0);
    const bool kval = act && key < L;
    const float* qr = (const float*)(const void*)a.qr + bh * rows * D;
    const float* kr = (const float*)(const void*)a.kr + bh * rows * D;
    const float* vg = (const float*)(const void*)a.v + bh * L * D;
    const float* dg = (const float*)(const void*)a.dout + bh * L * D;
    float k[32], v[32], dk[32], dv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int d = 32 * c + i;
        k[i] = kr[key * D + d];
        v[i] = kval ? vg[key * D + d] : 0.f;
        dk[i] = 0.f;
        dv[i] = 0.f;
    }
    const int32_t* off = inv_off + bh * (long)(a.nblk + 1);
    const int32_t* list = inv_list + bh * (long)a.nblk * a.keep;
    for (int n = off[jb]; n < off[jb + 1]; ++n) {
        const int ib = list[n];
        __syncthreads();
        for (int e = tid; e < BS * D; e += 256) {
            const int r = e / D, d = e % D;
            const long qrow = (long)ib * BS + r;
            q_s[r * (D + 1) + d] = qr[qrow * D + d];
            g_s[r * (D + 1) + d] = qrow < L ? dg[qrow * D + d] : 0.f;
        }
        if (tid < BS) {
            lse_s[tid] = a.lse2[bh * rows + (long)ib * BS + tid];
            dl_s[tid] = a.delta[bh * rows + (long)ib * BS + tid];
        }
        __syncthreads();
        for (int r = 0; r < BS; ++r) {
            if ((long)ib * BS + r >= L) break;
            const float* qq = q_s + r * (D + 1) + 32 * c;
            const float* gg = g_s + r * (D + 1) + 32 * c;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                s += qq[i] * k[i];
                dp += gg[i] * v[i];
            }
            s = sum_lanes<NC>(s);
            dp = sum_lanes<NC>(dp);
            const float p = exp2f(s * a.qmul - lse_s[r]);
            const float ds = p * (dp - dl_s[r]);
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                dv[i] += p * gg[i];
                dk[i] += ds * qq[i];
            }
        }
    }
    if (!kval) return;
    int crd[3];
    token_coords(key, a.g.Hg, a.g.Wg, crd[0], crd[1], crd[2]);
    const long ro = (bh * L + key) * D;
    float* dko = (float*)(void*)a.dk + ro;
    float* dvo = (float*)(void*)a.dv + ro;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
        const int d = 32 * c + i;
        float y0 = dk[i] * a.kscale, y1 = dk[i + 1] * a.kscale;
        rot_t(y0, y1, rope_cs(a.tab, a.g, d >> 1, crd));
        dko[d] = y0 + a.dk_lr[ro + d];
        dko[d + 1] = y1 + a.dk_lr[ro + d + 1];
        dvo[d] = dv[i] + a.dv_lr[ro + d];
        dvo[d + 1] = dv[i + 1] + a.dv_lr[ro + d + 1];
    }
}

// ---------------------------------------------------------------------------
// Inverse of the kept lists: for each key block, the query blocks that keep
// it, ascending. A bitmap [BH][key block][query-block bits] is set with
// atomic ORs (the result does not depend on their order), counted, scanned
// and read back in bit order.
__global__ void k_inv_zero(uint32_t* __restrict__ bits, long n) {
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) bits[e] = 0u;
}

__global__ void k_inv_mark(const int32_t* __restrict__ idx, long BH, int nblk, int keep, int W,
                           uint32_t* __restrict__ bits) {
    const long per = (long)nblk * keep;
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < BH * per; e += (long)gridDim.x * blockDim.x) {
        const long bh = e / per;
        const int i = (int)((e % per) / keep);
        const int j = idx[e];
        if (j >= 0 && j < nblk) atomicOr(bits + (bh * nblk + j) * W + (i >> 5), 1u << (i & 31));
    }
}

__global__ void k_inv_count(const uint32_t* __restrict__ bits, long n, int W, int32_t* __restrict__ cnt) {
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
        int c = 0;
        for (int w = 0; w < W; ++w) c += __popc(bits[e * W + w]);
        cnt[e] = c;
    }
}

// One workgroup per slice: exclusive scan of the counts into off[0 .. nblk].
__global__ __launch_bounds__(256) void k_inv_scan(const int32_t* __restrict__ cnt, int nblk,
                                                  int32_t* __restrict__ off) {
    __shared__ int part[256];
    const long bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int per = (nblk + 255) / 256;
    const int lo = tid * per, hi = min(lo + per, nblk);
    int s = 0;
    for (int j = lo; j < hi; ++j) s += cnt[bh * nblk + j];
    part[tid] = s;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int t = 0; t < 256; ++t) {
            const int x = part[t];
            part[t] = run;
            run += x;
        }
    }
    __syncthreads();
    int run = part[tid];
    int32_t* o = off + bh * (nblk + 1);
    for (int j = lo; j < hi; ++j) {
        o[j] = run;
        run += cnt[bh * nblk + j];
    }
    if (tid == 255) o[nblk] = run;
}

// Order of the key blocks of a slice for the dK/dV kernel: longest query-block
// list first (lists are skewed; the longest runs ~4x the mean), ties by index:
// rank(j) = #{i : cnt_i > cnt_j} + #{i < j : cnt_i = cnt_j}, so order is a
// deterministic permutation and each workgroup still computes one key block.
__global__ __launch_bounds__(256) void k_inv_order(const int32_t* __restrict__ cnt, int nblk,
                                                   int32_t* __restrict__ order) {
    const long bh = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= nblk) return;
    const int32_t* c = cnt + bh * nblk;
    const int cj = c[j];
    int rank = 0;
    for (int i = 0; i < nblk; ++i) {
        const int ci = c[i];
        rank += (ci > cj || (ci == cj && i < j)) ? 1 : 0;
    }
    order[bh * nblk + rank] = j;
}

__global__ void k_inv_fill(const uint32_t* __restrict__ bits, const int32_t* __restrict__ off, long BH, int nblk,
                           int keep, int W, int32_t* __restrict__ list) {
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < BH * nblk; e += (long)gridDim.x * blockDim.x) {
        const long bh = e / nblk;
        const int j = (int)(e % nblk);
        int pos = off[bh * (nblk + 1) + j];
        int32_t* dst = list + bh * (long)nblk * keep;
        for (int w = 0; w < W; ++w) {
            uint32_t m = bits[e * W + w];
            while (m) {
                const int b = __ffs(m) - 1;
                dst[pos++] = 32 * w + b;
                m &= m - 1u;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Low-rank branch. phi and its derivative: elu + 1 (x + 1 | e^x) or SiLU
// (FAVOR+ features depend on the whole projected row: lr_features_favor).
__device__ __forceinline__ void phi_grad(bool silu, float x, float& f, float& df) {
    if (silu) {
        const float sg = 1.f / (1.f + expf(-x));
        f = x * sg;
        df = sg * (1.f + x * (1.f - sg));
    } else if (x > 0.f) {
        f = x + 1.f;
        df = 1.f;
    } else {
        f = expf(x);
        df = f;
    }
}

__device__ __forceinline__ float round_bf(float x) { return bf2f(f2bf(x)); }

// Shared tile machinery of the two low-rank kernels: fp32 LDS copies of the
// weights W [D][R + 4] and of S (or dS) [R][D], a tile of TT token rows of
// two inputs [TT][D + 4], and per-token rank vectors [TT][R + 4]. Every
// product is register-blocked over float4 LDS reads: work items take the
// token index fastest (lanes then read rows 16 bytes apart mod 256: no bank
// conflicts) and 4 outputs each; the partial sums over tokens take 4x4
// blocks per thread.
template <int D, int R>
struct LrTile {
    static constexpr int TT = 16, XLD = D + 4, RW = R + 4, RLD = R + 4;
    static constexpr int NBLK = D * R / 16;                  // 4x4 blocks of a [D][R] or [R][D] sum
    static constexpr int NB16 = (NBLK + 255) / 256;          // blocks per thread
};

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void fma4(float4& acc, float s, const float4& v) {
    acc.x += s * v.x; acc.y += s * v.y; acc.z += s * v.z; acc.w += s * v.w;
}

// y[t][4g .. 4g+3] = sum_r v[t][r] M[4g + i][r] (M rows of length R, stride ld)
template <int R>
__device__ __forceinline__ float4 rowdot4(const float* vrow, const float* M, int ld, int g) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 2
    for (int r = 0; r < R; r += 4) {
        const float4 v = ld4(vrow + r);
        const float4 m0 = ld4(M + (4 * g) * ld + r), m1 = ld4(M + (4 * g + 1) * ld + r);
        const float4 m2 = ld4(M + (4 * g + 2) * ld + r), m3 = ld4(M + (4 * g + 3) * ld + r);
        acc.x += v.x * m0.x + v.y * m0.y + v.z * m0.z + v.w * m0.w;
        acc.y += v.x * m1.x + v.y * m1.y + v.z * m1.z + v.w * m1.w;
        acc.z += v.x * m2.x + v.y * m2.y + v.z * m2.z + v.w * m2.w;
        acc.w += v.x * m3.x + v.y * m3.y + v.z * m3.z + v.w * m3.w;
    }
    return acc;
}

// y[t][4g .. 4g+3] = sum_k v[t][k] M[k][4g .. 4g+3] (M rows of length >= 4g + 4, stride ld), K terms
template <int K>
__device__ __forceinline__ float4 vecmat4(const float* vrow, const float* M, int ld, int g) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 2
    for (int k = 0; k < K; k += 4) {
        const float4 v = ld4(vrow + k);
        fma4(acc, v.x, ld4(M + k * ld + 4 * g));
        fma4(acc, v.y, ld4(M + (k + 1) * ld + 4 * g));
        fma4(acc, v.z, ld4(M + (k + 2) * ld + 4 * g));
        fma4(acc, v.w, ld4(M + (k + 3) * ld + 4 * g));
    }
    return acc;
}

// Load TT token rows of two [L][D] inputs (bf16 when BF, else fp32) into fp32
// LDS tiles (zeros past t_hi).
template <int D, int R, bool BF>
__device__ __forceinline__ void lr_load_rows(const void* a_src, const void* b_src, long t0, long t_hi, float* xa,
                                             float* xb, int tid) {
    using Tl = LrTile<D, R>;
    for (int e = tid; e < Tl::TT * D / 8; e += 256) {
        const int t = e / (D / 8), c = e % (D / 8);
        const long l = t0 + t;
        float* pa = xa + t * Tl::XLD + 8 * c;
        float* pb = xb + t * Tl::XLD + 8 * c;
        if constexpr (BF) {
            u32x4_t ua{0u, 0u, 0u, 0u}, ub{0u, 0u, 0u, 0u};
            if (l < t_hi) {
                ua = ldg16((const uint16_t*)a_src + l * D + 8 * c);
                ub = ldg16((const uint16_t*)b_src + l * D + 8 * c);
            }
            *reinterpret_cast<float4*>(pa) = make_float4(bf_lo(ua[0]), bf_hi(ua[0]), bf_lo(ua[1]), bf_hi(ua[1]));
            *reinterpret_cast<float4*>(pa + 4) = make_float4(bf_lo(ua[2]), bf_hi(ua[2]), bf_lo(ua[3]), bf_hi(ua[3]));
            *reinterpret_cast<float4*>(pb) = make_float4(bf_lo(ub[0]), bf_hi(ub[0]), bf_lo(ub[1]), bf_hi(ub[1]));
            *reinterpret_cast<float4*>(pb + 4) = make_float4(bf_lo(ub[2]), bf_hi(ub[2]), bf_lo(ub[3]), bf_hi(ub[3]));
        } else {
            float4 z = make_float4(0.f, 0.f, 0.f, 0.f), a0 = z, a1 = z, b0 = z, b1 = z;
            if (l < t_hi) {
                const float* fa = (const float*)a_src + l * D + 8 * c;
                const float* fb = (const float*)b_src + l * D + 8 * c;
                a0 = ld4(fa); a1 = ld4(fa + 4); b0 = ld4(fb); b1 = ld4(fb + 4);
            }
            *reinterpret_cast<float4*>(pa) = a0;
            *reinterpret_cast<float4*>(pa + 4) = a1;
            *reinterpret_cast<float4*>(pb) = b0;
            *reinterpret_cast<float4*>(pb + 4) = b1;
        }
    }
}

// Projection and feature map of a token tile: p = x W, f_raw = phi(p) -> wt,
// phi'(p) -> dt; then the rotation after phi -> ft (pairs of one token).
template <int D, int R>
__device__ __forceinline__ void lr_features(const LrBwdArgs& a, const float* x, const float* w_s, float* wt,
                                            float* ft, float* dt, long t0, long t_hi, int tid) {
    using Tl = LrTile<D, R>;
    for (int e = tid; e < Tl::TT * (R / 4); e += 256) {
        const int t = e % Tl::TT, g = e / Tl::TT;
        float4 p = vecmat4<D>(x + t * Tl::XLD, w_s, Tl::RW, g);
        const long l = t0 + t;
        int crd[3] = {0, 0, 0};
        if (l < t_hi) token_coords(l, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
        if (a.abspe && l < t_hi) {
            // absolute PE: E_t[t] + E_h[h] + E_w[w] added before phi (tables only 4-byte aligned)
            const float* et = a.Et + crd[0] * R + 4 * g;
            const float* eh = a.Eh + crd[1] * R + 4 * g;
            const float* ew = a.Ew + crd[2] * R + 4 * g;
            p.x += et[0] + eh[0] + ew[0];
            p.y += et[1] + eh[1] + ew[1];
            p.z += et[2] + eh[2] + ew[2];
            p.w += et[3] + eh[3] + ew[3];
        }
        float f[4], df[4];
        const bool silu = a.g.fmap == 1;
        phi_grad(silu, p.x, f[0], df[0]);
        phi_grad(silu, p.y, f[1], df[1]);
        phi_grad(silu, p.z, f[2], df[2]);
        phi_grad(silu, p.w, f[3], df[3]);
        *reinterpret_cast<float4*>(wt + t * Tl::RLD + 4 * g) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(dt + t * Tl::RLD + 4 * g) = make_float4(df[0], df[1], df[2], df[3]);
        // rotation after phi of the two pairs (4g, 4g+1), (4g+2, 4g+3) (rotary variant)
        if (!a.abspe && l < t_hi) {
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const float2 cs = lowrank_cs(a.tab, a.g, 2 * g + q2, crd);
                const float f0 = f[2 * q2], f1 = f[2 * q2 + 1];
                f[2 * q2] = f0 * cs.x - f1 * cs.y;
                f[2 * q2 + 1] = f0 * cs.y + f1 * cs.x;
            }
        }
        *reinterpret_cast<float4*>(ft + t * Tl::RLD + 4 * g) = make_float4(f[0], f[1], f[2], f[3]);
    }
}

// d_pre[t][r] = (rho_t^T (sum_d M[r][d] v[t][d] * scale_t) + add_t z[r]) * phi'[t][r]
// (dt holds phi' on entry and the result on exit), pairs of one token per item.
template <int D, int R>
__device__ __forceinline__ void lr_back_features(const LrBwdArgs& a, const float* vtile, const float* m_s,
                                                 const float* z_s, const float* scale_t, const float* add_t,
                                                 float* dt, long t0, long t_hi, int tid) {
    using Tl = LrTile<D, R>;
    for (int e = tid; e < Tl::TT * (R / 2); e += 256) {
        const int t = e % Tl::TT, pr = e / Tl::TT;
        const float* vr = vtile + t * Tl::XLD;
        const float* m0 = m_s + (2 * pr) * D;
        const float* m1 = m0 + D;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll 4
        for (int d = 0; d < D; d += 4) {
            const float4 v = ld4(vr + d), x0 = ld4(m0 + d), x1 = ld4(m1 + d);
            a0 += v.x * x0.x + v.y * x0.y + v.z * x0.z + v.w * x0.w;
            a1 += v.x * x1.x + v.y * x1.y + v.z * x1.z + v.w * x1.w;
        }
        const float sc = scale_t ? scale_t[t] : 1.f;
        a0 *= sc;
        a1 *= sc;
        const long l = t0 + t;
        if (!a.abspe && l < t_hi) {
            int crd[3];
            token_coords(l, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
            rot_t(a0, a1, lowrank_cs(a.tab, a.g, pr, crd));
        }
        const float ad = add_t ? add_t[t] : 1.f;
        dt[t * Tl::RLD + 2 * pr] *= a0 + ad * z_s[2 * pr];
        dt[t * Tl::RLD + 2 * pr + 1] *= a1 + ad * z_s[2 * pr + 1];
    }
}

// FAVOR+ features of a token tile (RoPeSLR appendix): p = x W (+ E) -> pt,
// u_c = exp(omega_c . p - |p|^2 / 2) / sqrt(R) -> wt, and u also -> dt (the
// elementwise factor lr_back_features multiplies by; lr_favor_back then
// applies the rest of du/dp), the rotation after the features -> ft. om_s
// holds the head's omega [R][R + 4]. One (token, 4 ranks) item per thread;
// called by every thread of the workgroup.
template <int D, int R>
__device__ __forceinline__ void lr_features_favor(const LrBwdArgs& a, const float* x, const float* w_s,
                                                  const float* om_s, float* pt, float* wt, float* ft, float* dt,
                                                  long t0, long t_hi, int tid) {
    using Tl = LrTile<D, R>;
    static_assert(Tl::TT * (R / 4) <= 256, "one item per thread");
    const bool own = tid < Tl::TT * (R / 4);
    const int t = tid % Tl::TT, g = tid / Tl::TT;
    const long l = t0 + t;
    int crd[3] = {0, 0, 0};
    if (l < t_hi) token_coords(l, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
    if (own) {
        float4 p = vecmat4<D>(x + t * Tl::XLD, w_s, Tl::RW, g);
        if (a.abspe && l < t_hi) {
            const float* et = a.Et + crd[0] * R + 4 * g;
            const float* eh = a.Eh + crd[1] * R + 4 * g;
            const float* ew = a.Ew + crd[2] * R + 4 * g;
            p.x += et[0] + eh[0] + ew[0];
            p.y += et[1] + eh[1] + ew[1];
            p.z += et[2] + eh[2] + ew[2];
            p.w += et[3] + eh[3] + ew[3];
        }
        *reinterpret_cast<float4*>(pt + t * Tl::RLD + 4 * g) = p;
    }
    __syncthreads();
    if (own) {
        const float* pr = pt + t * Tl::RLD;
        const float4 y = rowdot4<R>(pr, om_s, Tl::RW, g);   // omega_c . p for c = 4g .. 4g + 3
        float sq = 0.f;
#pragma unroll 4
        for (int j = 0; j < R; j += 4) {
            const float4 v = ld4(pr + j);
            sq += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        const float h = 0.5f * sq, isr = 1.f / sqrtf((float)R);
        float f[4] = {expf(y.x - h) * isr, expf(y.y - h) * isr, expf(y.z - h) * isr, expf(y.w - h) * isr};
        *reinterpret_cast<float4*>(wt + t * Tl::RLD + 4 * g) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(dt + t * Tl::RLD + 4 * g) = make_float4(f[0], f[1], f[2], f[3]);
        if (!a.abspe && l < t_hi) {
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const float2 cs = lowrank_cs(a.tab, a.g, 2 * g + q2, crd);
                const float f0 = f[2 * q2], f1 = f[2 * q2 + 1];
                f[2 * q2] = f0 * cs.x - f1 * cs.y;
                f[2 * q2 + 1] = f0 * cs.y + f1 * cs.x;
            }
        }
        *reinterpret_cast<float4*>(ft + t * Tl::RLD + 4 * g) = make_float4(f[0], f[1], f[2], f[3]);
    }
}

// The rest of the FAVOR+ Jacobian: with e = du * u in dt (du/dp_j = u_c
// (omega_cj - p_j)), dp_j = sum_c omega_cj e_c - p_j sum_c e_c -> dt. Called
// by every thread of the workgroup after the barrier that follows
// lr_back_features; ends with dt written (a barrier must follow).
template <int D, int R>
__device__ __forceinline__ void lr_favor_back(const float* om_s, const float* pt, float* dt, int tid) {
    using Tl = LrTile<D, R>;
    const bool own = tid < Tl::TT * (R / 4);
    const int t = tid % Tl::TT, g = tid / Tl::TT;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    if (own) {
        const float* er = dt + t * Tl::RLD;
        y = vecmat4<R>(er, om_s, Tl::RW, g);   // (omega^T e)_j for j = 4g .. 4g + 3
        float se = 0.f;
#pragma unroll 4
        for (int c = 0; c < R; c += 4) {
            const float4 v = ld4(er + c);
            se += v.x + v.y + v.z + v.w;
        }
        const float4 p = ld4(pt + t * Tl::RLD + 4 * g);
        y.x -= p.x * se; y.y -= p.y * se; y.z -= p.z * se; y.w -= p.w * se;
    }
    __syncthreads();
    if (own) *reinterpret_cast<float4*>(dt + t * Tl::RLD + 4 * g) = y;
}

// Query side, per token l (O_l = rho_l(w_l)^T S / n_l, w_l = phi(q_l W_q),
// n_l = w_l . z + eps, or L for SiLU), given dO_lr = g_h dout:
//   dfq = S dO / n, dn = -(dO . O) / n, dw = rho^T dfq + dn z, dpq = dw phi',
//   dq_lr = W_q dpq; partial sums of dW_q = q^T dpq, dS = fq dO^T / n,
//   dz = dn w and dg = dout . O over the workgroup's tokens.
// Partial layout per (slice, split): [dW_q D*R | dS R*D | dz R | dg 1 | pad 3]
// (a stride of 2DR + R + 4 floats keeps every block 16-byte aligned).
template <int D, int R, bool BF, bool FV>
__global__ __launch_bounds__(256) void k_bwd_lr_q(LrBwdArgs a) {
    using Tl = LrTile<D, R>;
    constexpr int TT = Tl::TT, XLD = Tl::XLD, RW = Tl::RW, RLD = Tl::RLD, NB16 = Tl::NB16;
    __shared__ __attribute__((aligned(16))) float w_s[D * RW];
    // FAVOR+: the head's omega and the tile's projected rows p
    __shared__ __attribute__((aligned(16))) float om_s[FV ? R * RW : 4];
    __shared__ __attribute__((aligned(16))) float p_t[FV ? TT * RLD : 4];
    __shared__ __attribute__((aligned(16))) float s_s[R * D];
    __shared__ float z_s[R];
    __shared__ __attribute__((aligned(16))) float x_s[TT * XLD];
    __shared__ __attribute__((aligned(16))) float g_s[TT * XLD];
    __shared__ __attribute__((aligned(16))) float w_t[TT * RLD];
    __shared__ __attribute__((aligned(16))) float f_t[TT * RLD];
    __shared__ __attribute__((aligned(16))) float d_t[TT * RLD];
    __shared__ float part_s[(D / 4) * TT];
    __shared__ float n_s[TT], dn_s[TT], sc_s[TT];
    __shared__ float red[256];
    // token gate: per-row sums of O.O and O_sp.O_sp, and the gate's row coefficients
    __shared__ float part2_s[(D / 4) * TT], part3_s[(D / 4) * TT];
    __shared__ float G_s[TT], kl_s[TT], ks_s[TT], dtt_s[TT];
    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const long bh = blockIdx.y;
    const int head = (int)(bh % a.H);
    const long L = a.L;
    const long t_lo = (long)split * a.chunk;
    const long t_hi = t_lo + a.chunk < L ? t_lo + a.chunk : L;
    const bool token = a.token != 0;
    // the per-head gate exists only in head mode (the token gate passes no gate array)
    const float gh = token ? 0.f : a.gate[head];
    const bool silu = a.g.fmap == 1;   // SiLU's readout divides by L
    for (int e = tid; e < D * R; e += 256) {
        const float x = a.Wq[(long)head * D * R + e];
        w_s[(e / R) * RW + e % R] = BF ? round_bf(x) : x;
    }
    if constexpr (FV)
        for (int e = tid; e < R * R; e += 256) om_s[(e / R) * RW + e % R] = a.g.omega[(long)head * R * R + e];
    for (int e = tid; e < R * D; e += 256) s_s[e] = a.S[bh * R * D + e];
    for (int e = tid; e < R; e += 256) z_s[e] = a.z[bh * R + e];
    float4 accW[NB16][4], accS[NB16][4];
#pragma unroll
    for (int c = 0; c < NB16; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            accW[c][i] = make_float4(0.f, 0.f, 0.f, 0.f);
            accS[c][i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    float accz = 0.f, accg = 0.f, accwg = 0.f;
    const size_t es = BF ? 2 : 4;
    const void* qs = (const char*)(const void*)a.q + bh * L * D * es;
    const void* gs = (const char*)(const void*)a.dout + bh * L * D * es;
    const float* wgh = token ? a.wg + (long)head * D : nullptr;
    const float bgh = token ? a.bg[head] : 0.f;
    // 4 dims of the forward's O_sparse (zero past t_hi)
    auto osp4 = [&](long l, int g) -> float4 {
        if (l >= t_hi) return make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (BF) {
            const u32x2_t u = *reinterpret_cast<const u32x2_t*>((const uint16_t*)a.o_sp + (bh * L + l) * D + 4 * g);
            return make_float4(bf_lo(u[0]), bf_hi(u[0]), bf_lo(u[1]), bf_hi(u[1]));
        } else {
            return ld4((const float*)a.o_sp + (bh * L + l) * D + 4 * g);
        }
    };

    for (long t0 = t_lo; t0 < t_hi; t0 += TT) {
        __syncthreads();
        lr_load_rows<D, R, BF>(qs, gs, t0, t_hi, x_s, g_s, tid);
        __syncthreads();
        if constexpr (FV)
            lr_features_favor<D, R>(a, x_s, w_s, om_s, p_t, w_t, f_t, d_t, t0, t_hi, tid);
        else
            lr_features<D, R>(a, x_s, w_s, w_t, f_t, d_t, t0, t_hi, tid);
        __syncthreads();
        if (tid < TT) {
            float n = 0.f;
            for (int r = 0; r < R; ++r) n += w_t[tid * RLD + r] * z_s[r];
            n_s[tid] = silu ? (float)L : n + a.eps;
        }
        // readout O = fq S / n (unnormalised here) and its dot with dout, per (token, 4 dims)
        for (int e = tid; e < TT * (D / 4); e += 256) {
            const int t = e % TT, g = e / TT;
            const float4 o = vecmat4<R>(f_t + t * RLD, s_s, D, g);
            const float4 go = ld4(g_s + t * XLD + 4 * g);
            part_s[g * TT + t] = go.x * o.x + go.y * o.y + go.z * o.z + go.w * o.w;
            if (token) {
                const float4 sp = osp4(t0 + t, g);
                part2_s[g * TT + t] = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
                part3_s[g * TT + t] = sp.x * sp.x + sp.y * sp.y + sp.z * sp.z + sp.w * sp.w;
            }
        }
        __syncthreads();
        if (tid < TT) {
            float dot = 0.f;
            for (int g = 0; g < D / 4; ++g) dot += part_s[g * TT + tid];
            const float invn = 1.f / n_s[tid];
            dot *= invn;
            if (!token) {
                dn_s[tid] = silu ? 0.f : -gh * dot * invn;
                sc_s[tid] = gh * invn;
                accg += dot;
            } else {
                // out = O_sp + G O_lr, G = sigmoid(q . W_g + b_g) RMS(O_sp) / (RMS(O_lr) + eps):
                // dO_lr = G dout + kl O_lr, dO_sp = dout + ks O_sp, d(logit) = dtt
                float oo = 0.f, ss = 0.f, lg = bgh;
                for (int g = 0; g < D / 4; ++g) {
                    oo += part2_s[g * TT + tid];
                    ss += part3_s[g * TT + tid];
                }
                oo *= invn * invn;
                for (int d = 0; d < D; ++d) lg += x_s[tid * XLD + d] * wgh[d];
                const float gg = 1.f / (1.f + expf(-lg));
                const float rl = sqrtf(oo / D), rs = sqrtf(ss / D);
                const float c = rs / (rl + a.eps), G = gg * c;
                const float dc = dot * gg;
                const float drs = dc / (rl + a.eps), drl = -dc * rs / ((rl + a.eps) * (rl + a.eps));
                const float kl = rl > 0.f ? drl / (D * rl) : 0.f;
                G_s[tid] = G;
                kl_s[tid] = kl;
                ks_s[tid] = rs > 0.f ? drs / (D * rs) : 0.f;
                const float dtt = dot * c * gg * (1.f - gg);
                dtt_s[tid] = dtt;
                // dO_lr . O = G (dout . O) + kl (O . O)
                dn_s[tid] = silu ? 0.f : -(G * dot + kl * oo) * invn;
                sc_s[tid] = invn;
                accg += dtt;
            }
        }
        __syncthreads();
        if (token) {
            // dO_lr replaces dout in the tile; dO_sp goes out for the sparse branch
            for (int e = tid; e < TT * (D / 4); e += 256) {
                const int t = e % TT, g = e / TT;
                const long l = t0 + t;
                const float invn = 1.f / n_s[t];
                float4 o = vecmat4<R>(f_t + t * RLD, s_s, D, g);
                o.x *= invn; o.y *= invn; o.z *= invn; o.w *= invn;
                float* gp = g_s + t * XLD + 4 * g;
                const float4 go = ld4(gp);
                const float G = G_s[t], kl = kl_s[t], ks = ks_s[t];
                *reinterpret_cast<float4*>(gp) = make_float4(G * go.x + kl * o.x, G * go.y + kl * o.y,
                                                             G * go.z + kl * o.z, G * go.w + kl * o.w);
                if (l < t_hi) {
                    const float4 sp = osp4(l, g);
                    const float4 y = make_float4(go.x + ks * sp.x, go.y + ks * sp.y, go.z + ks * sp.z, go.w + ks * sp.w);
                    if constexpr (BF) {
                        *reinterpret_cast<u32x2_t*>((uint16_t*)a.dosp + (bh * L + l) * D + 4 * g) =
                            u32x2_t{pack_bf2(y.x, y.y), pack_bf2(y.z, y.w)};
                    } else {
                        *reinterpret_cast<float4*>((float*)a.dosp + (bh * L + l) * D + 4 * g) = y;
                    }
                }
            }
            for (int d = tid; d < D; d += 256) {
                float acc = 0.f;
                for (int t = 0; t < TT; ++t) acc += dtt_s[t] * x_s[t * XLD + d];
                accwg += acc;
            }
            __syncthreads();
        }
        // dfq = S (g dout) / n -> rho^T, + dn z, * phi'  (d_t becomes dpq)
        lr_back_features<D, R>(a, g_s, s_s, z_s, sc_s, dn_s, d_t, t0, t_hi, tid);
        __syncthreads();
        if constexpr (FV) {
            lr_favor_back<D, R>(om_s, p_t, d_t, tid);
            __syncthreads();
        }
        if (a.abspe) {
            // gradient w.r.t. q W_q + E of each valid token (the E tables' share)
            for (int e = tid; e < TT * R; e += 256) {
                const int t = e / R, r = e % R;
                if (t0 + t < t_hi) a.dpre[(bh * L + t0 + t) * R + r] = d_t[t * RLD + r];
            }
        }
        // dq_lr = W_q dpq per (token, 4 dims)
        for (int e = tid; e < TT * (D / 4); e += 256) {
            const int t = e % TT, g = e / TT;
            const long l = t0 + t;
            float4 y = rowdot4<R>(d_t + t * RLD, w_s, RW, g);
            if (token) {
                // the gate's logit reads the raw query row: + dtt W_g
                const float dt = dtt_s[t];
                y.x += dt * wgh[4 * g]; y.y += dt * wgh[4 * g + 1]; y.z += dt * wgh[4 * g + 2]; y.w += dt * wgh[4 * g + 3];
            }
            if (l < t_hi) *reinterpret_cast<float4*>(a.dq_lr + (bh * L + l) * D + 4 * g) = y;
        }
        // partial sums over the tile's tokens, 4x4 blocks
#pragma unroll
        for (int c = 0; c < NB16; ++c) {
            const int blk = tid + 256 * c;
            if (blk < Tl::NBLK) {
                const int bd = blk / (R / 4), br = blk % (R / 4);     // dW_q block (4 d) x (4 r)
                const int sr = blk / (D / 4), sd = blk % (D / 4);     // dS block (4 r) x (4 d)
#pragma unroll 4
                for (int t = 0; t < TT; ++t) {
                    const float4 xv = ld4(x_s + t * XLD + 4 * bd), dv = ld4(d_t + t * RLD + 4 * br);
                    fma4(accW[c][0], xv.x, dv);
                    fma4(accW[c][1], xv.y, dv);
                    fma4(accW[c][2], xv.z, dv);
                    fma4(accW[c][3], xv.w, dv);
                    const float sc = sc_s[t];
                    const float4 fv = ld4(f_t + t * RLD + 4 * sr), gv = ld4(g_s + t * XLD + 4 * sd);
                    fma4(accS[c][0], fv.x * sc, gv);
                    fma4(accS[c][1], fv.y * sc, gv);
                    fma4(accS[c][2], fv.z * sc, gv);
                    fma4(accS[c][3], fv.w * sc, gv);
                }
            }
        }
        if (tid < R) {
            float acc = 0.f;
            for (int t = 0; t < TT; ++t) acc += dn_s[t] * w_t[t * RLD + tid];
            accz += acc;
        }
    }
    float* part = a.part + (bh * a.nsplit + split) * (long)(2 * D * R + R + 4);
#pragma unroll
    for (int c = 0; c < NB16; ++c) {
        const int blk = tid + 256 * c;
        if (blk < Tl::NBLK) {
            const int bd = blk / (R / 4), br = blk % (R / 4);
            const int sr = blk / (D / 4), sd = blk % (D / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<float4*>(part + (4 * bd + i) * R + 4 * br) = accW[c][i];
                *reinterpret_cast<float4*>(part + D * R + (4 * sr + i) * D + 4 * sd) = accS[c][i];
            }
        }
    }
    if (tid < R) part[2 * D * R + tid] = accz;
    red[tid] = accg;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int t = 0; t < 256; ++t) s += red[t];
        if (token) a.gpart[(bh * a.nsplit + split) * (long)(D + 4) + D] = s;   // db_g
        else part[2 * D * R + R] = s;                                           // dg_h
    }
    if (token && tid < D) a.gpart[(bh * a.nsplit + split) * (long)(D + 4) + tid] = accwg;
}

// Key side, per token m (S = sum rho_m(u_m) v_m^T, z = sum u_m, u = phi(k W_k)),
// given the reduced dS, dz: dv_lr = dS^T fk, dfk = dS v, du = rho^T dfk + dz,
// dpk = du phi', dk_lr = W_k dpk; partial sums of dW_k = k^T dpk [D*R].
template <int D, int R, bool BF, bool FV>
__global__ __launch_bounds__(256) void k_bwd_lr_k(LrBwdArgs a) {
    using Tl = LrTile<D, R>;
    constexpr int TT = Tl::TT, XLD = Tl::XLD, RW = Tl::RW, RLD = Tl::RLD, NB16 = Tl::NB16;
    __shared__ __attribute__((aligned(16))) float w_s[D * RW];
    __shared__ __attribute__((aligned(16))) float om_s[FV ? R * RW : 4];
    __shared__ __attribute__((aligned(16))) float p_t[FV ? TT * RLD : 4];
    __shared__ __attribute__((aligned(16))) float s_s[R * D];
    __shared__ float z_s[R];
    __shared__ __attribute__((aligned(16))) float x_s[TT * XLD];
    __shared__ __attribute__((aligned(16))) float v_s[TT * XLD];
    __shared__ __attribute__((aligned(16))) float u_t[TT * RLD];
    __shared__ __attribute__((aligned(16))) float f_t[TT * RLD];
    __shared__ __attribute__((aligned(16))) float d_t[TT * RLD];
    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const long bh = blockIdx.y;
    const int head = (int)(bh % a.H);
    const long L = a.L;
    const long t_lo = (long)split * a.chunk;
    const long t_hi = t_lo + a.chunk < L ? t_lo + a.chunk : L;
    const float* dsz = a.dSz + bh * (long)(R * D + R);
    for (int e = tid; e < D * R; e += 256) {
        const float x = a.Wk[(long)head * D * R + e];
        w_s[(e / R) * RW + e % R] = BF ? round_bf(x) : x;
    }
    if constexpr (FV)
        for (int e = tid; e < R * R; e += 256) om_s[(e / R) * RW + e % R] = a.g.omega[(long)head * R * R + e];
    for (int e = tid; e < R * D; e += 256) s_s[e] = dsz[e];
    for (int e = tid; e < R; e += 256) z_s[e] = dsz[R * D + e];
    float4 accW[NB16][4];
#pragma unroll
    for (int c = 0; c < NB16; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) accW[c][i] = make_float4(0.f, 0.f, 0.f, 0.f);
    const size_t es = BF ? 2 : 4;
    const void* ks = (const char*)(const void*)a.k + bh * L * D * es;
    const void* vs = (const char*)(const void*)a.v + bh * L * D * es;

    for (long t0 = t_lo; t0 < t_hi; t0 += TT) {
        __syncthreads();
        lr_load_rows<D, R, BF>(ks, vs, t0, t_hi, x_s, v_s, tid);
        __syncthreads();
        if constexpr (FV)
            lr_features_favor<D, R>(a, x_s, w_s, om_s, p_t, u_t, f_t, d_t, t0, t_hi, tid);
        else
            lr_features<D, R>(a, x_s, w_s, u_t, f_t, d_t, t0, t_hi, tid);
        __syncthreads();
        // dv_lr = dS^T fk per (token, 4 dims)
        for (int e = tid; e < TT * (D / 4); e += 256) {
            const int t = e % TT, g = e / TT;
            const long l = t0 + t;
            const float4 y = vecmat4<R>(f_t + t * RLD, s_s, D, g);
            if (l < t_hi) *reinterpret_cast<float4*>(a.dv_lr + (bh * L + l) * D + 4 * g) = y;
        }
        // dfk = dS v -> rho^T, + dz, * phi'  (d_t becomes dpk)
        lr_back_features<D, R>(a, v_s, s_s, z_s, nullptr, nullptr, d_t, t0, t_hi, tid);
        __syncthreads();
        if constexpr (FV) {
            lr_favor_back<D, R>(om_s, p_t, d_t, tid);
            __syncthreads();
        }
        if (a.abspe) {
            // adds the key side's share (the query side wrote its own first)
            for (int e = tid; e < TT * R; e += 256) {
                const int t = e / R, r = e % R;
                if (t0 + t < t_hi) a.dpre[(bh * L + t0 + t) * R + r] += d_t[t * RLD + r];
            }
        }
        for (int e = tid; e < TT * (D / 4); e += 256) {
            const int t = e % TT, g = e / TT;
            const long l = t0 + t;
            const float4 y = rowdot4<R>(d_t + t * RLD, w_s, RW, g);
            if (l < t_hi) *reinterpret_cast<float4*>(a.dk_lr + (bh * L + l) * D + 4 * g) = y;
        }
#pragma unroll
        for (int c = 0; c < NB16; ++c) {
            const int blk = tid + 256 * c;
            if (blk < Tl::NBLK) {
                const int bd = blk / (R / 4), br = blk % (R / 4);
#pragma unroll 4
                for (int t = 0; t < TT; ++t) {
                    const float4 xv = ld4(x_s + t * XLD + 4 * bd), dv = ld4(d_t + t * RLD + 4 * br);
                    fma4(accW[c][0], xv.x, dv);
                    fma4(accW[c][1], xv.y, dv);
                    fma4(accW[c][2], xv.z, dv);
                    fma4(accW[c][3], xv.w, dv);
                }
            }
        }
    }
    float* part = a.part + (bh * a.nsplit + split) * (long)(D * R);
#pragma unroll
    for (int c = 0; c < NB16; ++c) {
        const int blk = tid + 256 * c;
        if (blk < Tl::NBLK) {
            const int bd = blk / (R / 4), br = blk % (R / 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<float4*>(part + (4 * bd + i) * R + 4 * br) = accW[c][i];
        }
    }
}

// ---------------------------------------------------------------------------
// Low-rank branch on MFMA (lr_bwd_on_mfma: bf16, D = 128, R = 32 or 64,
// per-head gate; rotary or absolute-PE features: with absolute PE,
// p = x W + E_t[t] + E_h[h] + E_w[w], rho is the identity, and each token's
// dp is also stored (dpre) for the tables' sums). Tokens sit on the MFMA column axis: lane
// l owns token l % 32 of its wave's 32, and a product over d leaves rank
// r = 32rb + 8(v/4) + 4(l/32) + v%4 in register v of block rb (the slot16
// order), which is the B operand layout of a product over r, and keeps each
// rank pair (2j, 2j+1) of a token in one lane for the rotations. q, k, v,
// dout and the bf16-rounded W are exact in bf16; fp32 operands (S, dS and
// the per-token rank vectors) enter as hi + lo bf16 pairs (hi = bf16(x),
// lo = bf16(x - hi)), and the products take hi*hi + lo*hi (+ hi*lo), about
// 16 significant bits. Workgroup = 4 waves, 32 tokens per wave per step.
//
//   k_bwd_lrm_q    p^T = W_q^T q^T, f = phi(p), fq = rho(f), n = f . z + eps
//                  (L for SiLU), sg = S dout (dout . O_un = fq . sg),
//                  dot = fq . sg / n, dpq = (rho^T(g sg / n) - (g dot / n) z) phi',
//                  dq_lr = W_q dpq; stores dpq and fq g / n (hi, lo) per token,
//                  and the workgroup's sums of dn f (dz) and dot (dg).
//   k_bwd_lrm_k    u = phi(k W_k), fk = rho(u), dv_lr = dS^T fk,
//                  dpk = (rho^T(dS v) + dz) phi', dk_lr = W_k dpk; stores dpk.
//   k_bwd_lrm_red  per (slice, split): sum over the split's tokens of
//                  x^T y (x [t][128] bf16, y [t][R] hi + lo): dW_q = q^T dpq,
//                  dS^T = dout^T (fq g / n), dW_k = k^T dpk.

// Operand-order LDS copies of an R x 128 matrix m(r, d) (1 KB blocks, lane
// l's 16 bytes at l * 16):
//   rd: A[row r][k = d], block (rb, s) = 8rb + s, lane l: m(32rb + l%32, 16s + 8(l/32) + e)
//   dr: A[row d][k = r], block (db, ks) = db (R/16) + ks, lane l:
//       m(16ks + 8(e/4) + 4(l/32) + e%4, 32db + l%32)
// SPLIT: hi to `hi`, lo to `lo`; else the bf16 rounding to `hi`.
template <int R, bool DR, bool SPLIT, typename M>
__device__ __forceinline__ void lrm_build(u32x4_t* hi, u32x4_t* lo, M m, int tid) {
    constexpr int NBLK = R / 4;   // (R / 32) * 8 = 4 * (R / 16)
    for (int it = tid; it < NBLK * 64; it += 256) {
        const int blk = it >> 6, l = it & 63, h = l >> 5;
        float x[8];
        if constexpr (!DR) {
            const int rb = blk >> 3, s = blk & 7;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = m(32 * rb + (l & 31), 16 * s + 8 * h + e);
        } else {
            const int db = blk / (R / 16), ks = blk % (R / 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = m(16 * ks + 8 * (e >> 2) + 4 * h + (e & 3), 32 * db + (l & 31));
        }
        u32x4_t a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = pack_bf2(x[2 * i], x[2 * i + 1]);
            if constexpr (SPLIT)
                b[i] = pack_bf2(x[2 * i] - bf_lo(a[i]), x[2 * i + 1] - bf_hi(a[i]));
        }
        hi[it] = a;
        if constexpr (SPLIT) lo[it] = b;
    }
}

// B operands (hi, lo) of k-step ks = (rb, h2) of a product over r from a
// rank vector in accumulator layout: registers 8h2 .. 8h2 + 7 of block rb
__device__ __forceinline__ void lrm_bop(const f32x16_t& y, int h2, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x0 = y[8 * h2 + 2 * i], x1 = y[8 * h2 + 2 * i + 1];
        hi[i] = pack_bf2(x0, x1);
        lo[i] = pack_bf2(x0 - bf_lo(hi[i]), x1 - bf_hi(hi[i]));
    }
}

// The 8 B operands of a product over d (lane: token row t, dims 16s + 8(l/32) .. +7); zero past t_hi
__device__ __forceinline__ void lrm_rowops(u32x4_t* b, const uint16_t* row, bool valid, int hf) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const u32x4_t w = ldg16(row + 16 * s + 8 * hf);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[s][i] = valid ? w[i] : 0u;
    }
}

// Stores of a rank vector in accumulator layout to y [t][rv] as bf16 hi + lo (ranks < rv)
template <int NR>
__device__ __forceinline__ void lrm_store_rank(const f32x16_t* y, uint16_t* dh, uint16_t* dl, int hf, int rv) {
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int r0 = 32 * rb + 8 * g4 + 4 * hf;
            if (r0 >= rv) continue;
            uint32_t h[2], l[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float x0 = y[rb][4 * g4 + 2 * i], x1 = y[rb][4 * g4 + 2 * i + 1];
                h[i] = pack_bf2(x0, x1);
                l[i] = pack_bf2(x0 - bf_lo(h[i]), x1 - bf_hi(h[i]));
            }
            *reinterpret_cast<u32x2_t*>(dh + r0) = u32x2_t{h[0], h[1]};
            *reinterpret_cast<u32x2_t*>(dl + r0) = u32x2_t{l[0], l[1]};
        }
}

// Operand-order LDS copies of the head's FAVOR+ directions omega [rv][rv]
// (zero past rv), hi and lo parts, blocks (cb, ks) = cb (R/16) + ks:
//   !TR: A[row c][k = j]: lane l: omega[32cb + l%32][16ks + 8(e/4) + 4(l/32) + e%4]  (y = omega p)
//    TR: A[row j][k = c]: lane l: omega[16ks + 8(e/4) + 4(l/32) + e%4][32cb + l%32]  (omega^T g)
template <int R, bool TR>
__device__ __forceinline__ void lrm_build_omega(u32x4_t* hi, u32x4_t* lo, const float* om, int rv, int tid) {
    constexpr int KS = R / 16, NBLK = (R / 32) * KS;
    for (int it = tid; it < NBLK * 64; it += 256) {
        const int blk = it >> 6, l = it & 63, h = l >> 5, cb = blk / KS, ks = blk % KS;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int a = 32 * cb + (l & 31), b = 16 * ks + 8 * (e >> 2) + 4 * h + (e & 3);
            const int c = TR ? b : a, j = TR ? a : b;
            x[e] = c < rv && j < rv ? om[c * rv + j] : 0.f;
        }
        u32x4_t u, v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u[i] = pack_bf2(x[2 * i], x[2 * i + 1]);
            v[i] = pack_bf2(x[2 * i] - bf_lo(u[i]), x[2 * i + 1] - bf_hi(u[i]));
        }
        hi[it] = u;
        lo[it] = v;
    }
}

// out = M x over ranks (M an R x R operand copy in hi / lo parts, x a rank
// vector in accumulator layout): three products per k-step (hi hi, lo hi, hi lo)
template <int NR>
__device__ __forceinline__ void lrm_rank_mat(const u32x4_t* mhi, const u32x4_t* mlo, const f32x16_t* x, int lane,
                                             f32x16_t* out) {
    constexpr int KS = NR * 2;
    u32x4_t xh[KS], xl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) lrm_bop(x[ks >> 1], ks & 1, xh[ks], xl[ks]);
#pragma unroll
    for (int cb = 0; cb < NR; ++cb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) out[cb][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int bi = (cb * KS + ks) * 64 + lane;
            const u32x4_t h = mhi[bi];
            out[cb] = mfma32(h, xh[ks], out[cb]);
            out[cb] = mfma32(mlo[bi], xh[ks], out[cb]);
            out[cb] = mfma32(h, xl[ks], out[cb]);
        }
    }
}

// FAVOR+ features of p (rank layout, zero past rv): u = exp(omega p - |p|^2 / 2) / sqrt(rv)
template <int NR>
__device__ __forceinline__ void lrm_favor(const u32x4_t* oh, const u32x4_t* ol, const f32x16_t* p, int lane, int hf,
                                          int rv, f32x16_t* u) {
    float sq = 0.f;
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sq += p[rb][v] * p[rb][v];
    sq = sum_xor32(sq);
    lrm_rank_mat<NR>(oh, ol, p, lane, u);
    const float rs = 1.f / sqrtf((float)rv);
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const bool rok = 32 * rb + 8 * (v >> 2) + 4 * hf + (v & 3) < rv;
            u[rb][v] = rok ? __builtin_amdgcn_exp2f((u[rb][v] - 0.5f * sq) * kLog2e) * rs : 0.f;
        }
}

// Gradient w.r.t. p of sum(du * u(p)) for FAVOR+ features: omega^T (du * u) - p sum(du * u); in place in du
template <int NR>
__device__ __forceinline__ void lrm_favor_back(const u32x4_t* th, const u32x4_t* tl, const f32x16_t* p,
                                               const f32x16_t* u, int lane, f32x16_t* du) {
    float gs = 0.f;
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            du[rb][v] *= u[rb][v];
            gs += du[rb][v];
        }
    gs = sum_xor32(gs);
    f32x16_t og[NR];
    lrm_rank_mat<NR>(th, tl, du, lane, og);
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) du[rb][v] = og[rb][v] - p[rb][v] * gs;
}

// phi and phi' without branches: elu + 1 or SiLU
template <bool SILU>
__device__ __forceinline__ void lrm_phi(float x, float& f, float& df) {
    if constexpr (SILU) {
        const float sg = 1.f / (1.f + expf(-x));
        f = x * sg;
        df = sg * (1.f + x * (1.f - sg));
    } else {
        const float e = expf(fminf(x, 0.f));
        f = x > 0.f ? x + 1.f : e;
        df = x > 0.f ? 1.f : e;
    }
}

// fp32 rank vector in accumulator layout -> dst [rv] (ADD: dst += it; ranks < rv)
template <int NR, bool ADD>
__device__ __forceinline__ void lrm_store_dpre(const f32x16_t* y, float* dst, int hf, int rv) {
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            if (32 * rb + 8 * g4 + 4 * hf >= rv) continue;
            float4* p = reinterpret_cast<float4*>(dst + 32 * rb + 8 * g4 + 4 * hf);
            float4 x = make_float4(y[rb][4 * g4], y[rb][4 * g4 + 1], y[rb][4 * g4 + 2], y[rb][4 * g4 + 3]);
            if constexpr (ADD) {
                const float4 o = *p;
                x.x += o.x; x.y += o.y; x.z += o.z; x.w += o.w;
            }
            *p = x;
        }
}

// z (or dz) at the ranks register v of block rb holds: 4 consecutive floats per group v / 4
__device__ __forceinline__ float4 lrm_z4(const float* z_s, int rb, int g4, int hf) {
    return *reinterpret_cast<const float4*>(z_s + 32 * rb + 8 * g4 + 4 * hf);
}

// Absolute PE: E_t[t] + E_h[h] + E_w[w] ([.][rv] tables, only 4-byte aligned) at the ranks
// register v of block rb holds (ranks < rv)
__device__ __forceinline__ void lrm_add_e(const LrBwdArgs& a, const int* crd, int hf, f32x16_t& p, int rb, int rv) {
    const float* et = a.Et + crd[0] * rv;
    const float* eh = a.Eh + crd[1] * rv;
    const float* ew = a.Ew + crd[2] * rv;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int r = 32 * rb + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (r < rv) p[v] += et[r] + eh[r] + ew[r];
    }
}

// (cos, sin) of the rank pairs (v, v + 1), v even, of block rb at token coordinates crd
// (the identity for the padding pairs past rv / 2)
template <int NR>
__device__ __forceinline__ void lrm_pairs_cs(const LrBwdArgs& a, const int* crd, int hf, float2 (*cs)[8], int rv) {
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int pr = 16 * rb + 4 * (j >> 1) + 2 * hf + (j & 1);
            cs[rb][j] = 2 * pr < rv ? lowrank_cs(a.tab, a.g, pr, crd) : make_float2(1.f, 0.f);
        }
}

// y = W dpq (or dS^T fk ...): the 4 column blocks of a [128] x [R] product over r, one at a
// time, each stored (for valid tokens) as it completes; bh / bl: hi / lo B operands of the
// k-steps. Called by the whole wave: lane l supplies the A operand's row l % 32 for every
// token, so the products must not sit under a branch on the lane's own token.
template <int KS, bool THREE>
__device__ __forceinline__ void lrm_apply_store(const u32x4_t* ahi, const u32x4_t* alo, const u32x4_t* bh,
                                                const u32x4_t* bl, int lane, float* dst, int hf, bool valid) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        f32x16_t y;
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4_t w = ahi[(db * KS + ks) * 64 + lane];
            y = mfma32(w, bh[ks], y);
            y = mfma32(w, bl[ks], y);
            if constexpr (THREE) y = mfma32(alo[(db * KS + ks) * 64 + lane], bh[ks], y);
        }
        if (valid) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *reinterpret_cast<float4*>(dst + 32 * db + 8 * g4 + 4 * hf) =
                    make_float4(y[4 * g4], y[4 * g4 + 1], y[4 * g4 + 2], y[4 * g4 + 3]);
        }
    }
}

template <int R, int FM, bool ABSPE>
__global__ __launch_bounds__(256) void k_bwd_lrm_q(LrBwdArgs a) {
    constexpr int D = 128, NR = R / 32, NB = R / 4, KS = R / 16;
    constexpr bool SILU = FM == 1, FAV = FM == 2;   // feature map: elu + 1, SiLU, FAVOR+
    constexpr int OB = FAV ? NR * KS * 64 : 1;
    __shared__ u32x4_t w_rd[NB * 64], w_dr[NB * 64], s_hi[NB * 64], s_lo[NB * 64];
    __shared__ u32x4_t om_hi[OB], om_lo[OB], omt_hi[OB], omt_lo[OB];   // FAVOR+: omega, omega^T
    __shared__ __attribute__((aligned(16))) float z_s[R];
    __shared__ float red[4][R + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5;
    const int split = blockIdx.x;
    const long bh = blockIdx.y;
    const int head = (int)(bh % a.H);
    const long L = a.L;
    const long t_lo = (long)split * a.chunk;
    const long t_hi = t_lo + a.chunk < L ? t_lo + a.chunk : L;
    const float gh = a.gate[head];
    // rv = the layer's rank (8, 16, 32 or 64); ranks rv .. R - 1 are padding with zero weights
    const int rv = a.g.R;
    const float* W = a.Wq + (long)head * D * rv;
    const float* S = a.S + bh * rv * D;
    lrm_build<R, false, false>(w_rd, nullptr, [&](int r, int d) { return r < rv ? W[d * rv + r] : 0.f; }, tid);
    lrm_build<R, true, false>(w_dr, nullptr, [&](int r, int d) { return r < rv ? W[d * rv + r] : 0.f; }, tid);
    lrm_build<R, false, true>(s_hi, s_lo, [&](int r, int d) { return r < rv ? S[r * D + d] : 0.f; }, tid);
    if constexpr (FAV) {
        lrm_build_omega<R, false>(om_hi, om_lo, a.g.omega + (long)head * rv * rv, rv, tid);
        lrm_build_omega<R, true>(omt_hi, omt_lo, a.g.omega + (long)head * rv * rv, rv, tid);
    }
    for (int e = tid; e < R; e += 256) z_s[e] = e < rv ? a.z[bh * rv + e] : 0.f;
    __syncthreads();
    float accz[NR][16];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) accz[rb][v] = 0.f;
    float accg = 0.f;

    for (long t0 = t_lo + 32 * wave; t0 < t_hi; t0 += 128) {
        // the operand copies are re-read from LDS each step rather than held in registers
        asm volatile("" ::: "memory");
        const long t = t0 + (lane & 31);
        const bool valid = t < t_hi;
        const long row = bh * L + (valid ? t : t_lo);
        int crd[3];
        token_coords(valid ? t : 0, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
        // p = q W_q (+ E), f = phi(p), phi' (FAVOR+: f from all of p, p kept for the backward), n
        f32x16_t f[NR], df[NR], pp[FAV ? NR : 1];
        float nz = 0.f;
        {
            u32x4_t xb[8];
            lrm_rowops(xb, a.q + row * D, valid, hf);
#pragma unroll
            for (int rb = 0; rb < NR; ++rb) {
                f32x16_t p;
#pragma unroll
                for (int i = 0; i < 16; ++i) p[i] = 0.f;
#pragma unroll
                for (int s = 0; s < 8; ++s) p = mfma32(w_rd[(8 * rb + s) * 64 + lane], xb[s], p);
                if constexpr (ABSPE) lrm_add_e(a, crd, hf, p, rb, rv);
                if constexpr (FAV) {
                    pp[rb] = p;
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        float fv, dv;
                        lrm_phi<SILU>(p[v], fv, dv);
                        const bool rok = 32 * rb + 8 * (v >> 2) + 4 * hf + (v & 3) < rv;
                        f[rb][v] = rok ? fv : 0.f;
                        df[rb][v] = rok ? dv : 0.f;
                    }
                }
            }
        }
        if constexpr (FAV) lrm_favor<NR>(om_hi, om_lo, pp, lane, hf, rv, f);
#pragma unroll
        for (int rb = 0; rb < NR; ++rb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 z4 = lrm_z4(z_s, rb, g4, hf);
                nz += f[rb][4 * g4] * z4.x + f[rb][4 * g4 + 1] * z4.y + f[rb][4 * g4 + 2] * z4.z +
                      f[rb][4 * g4 + 3] * z4.w;
            }
        // sg = S dout
        f32x16_t sg[NR];
        {
            u32x4_t gb[8];
            lrm_rowops(gb, a.dout + row * D, valid, hf);
#pragma unroll
            for (int rb = 0; rb < NR; ++rb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sg[rb][i] = 0.f;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int bi = (8 * rb + s) * 64 + lane;
                    sg[rb] = mfma32(s_hi[bi], gb[s], sg[rb]);
                    sg[rb] = mfma32(s_lo[bi], gb[s], sg[rb]);
                }
            }
        }
        // fq = rho(f) (f itself for absolute PE) and dout . O_un = fq . sg
        float2 cs[NR][8];
        if constexpr (!ABSPE) lrm_pairs_cs<NR>(a, crd, hf, cs, rv);
        f32x16_t fq[NR];
        float dsum = 0.f;
#pragma unroll
        for (int rb = 0; rb < NR; ++rb)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float f0 = f[rb][2 * j], f1 = f[rb][2 * j + 1];
                fq[rb][2 * j] = ABSPE ? f0 : f0 * cs[rb][j].x - f1 * cs[rb][j].y;
                fq[rb][2 * j + 1] = ABSPE ? f1 : f0 * cs[rb][j].y + f1 * cs[rb][j].x;
                dsum += fq[rb][2 * j] * sg[rb][2 * j] + fq[rb][2 * j + 1] * sg[rb][2 * j + 1];
            }
        const float n = SILU ? (float)L : sum_xor32(nz) + a.eps;
        const float invn = 1.f / n;
        const float dot = valid ? sum_xor32(dsum) * invn : 0.f;
        const float dn = SILU ? 0.f : -gh * dot * invn;
        const float sc = valid ? gh * invn : 0.f;
        if (hf == 0) accg += dot;
        // dz terms; dpq = (rho^T(sg sc) + dn z) phi' in place in sg; fq sc in place in fq
#pragma unroll
        for (int rb = 0; rb < NR; ++rb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                accz[rb][v] += dn * f[rb][v];
                fq[rb][v] *= sc;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 z4 = lrm_z4(z_s, rb, j >> 1, hf);
                const float za = (j & 1) ? z4.z : z4.x, zb = (j & 1) ? z4.w : z4.y;
                float y0 = sg[rb][2 * j] * sc, y1 = sg[rb][2 * j + 1] * sc;
                if constexpr (!ABSPE) rot_t(y0, y1, cs[rb][j]);
                sg[rb][2 * j] = (y0 + dn * za) * (FAV ? 1.f : df[rb][2 * j]);
                sg[rb][2 * j + 1] = (y1 + dn * zb) * (FAV ? 1.f : df[rb][2 * j + 1]);
            }
        }
        // FAVOR+: dw -> dp through the features' Jacobian
        if constexpr (FAV) lrm_favor_back<NR>(omt_hi, omt_lo, pp, f, lane, sg);
        if (valid) {
            lrm_store_rank<NR>(sg, a.y1h + row * rv, a.y1l + row * rv, hf, rv);
            lrm_store_rank<NR>(fq, a.y2h + row * rv, a.y2l + row * rv, hf, rv);
            // absolute PE: each token's gradient of q W_q + E (the query side's share of the E sums)
            if constexpr (ABSPE) lrm_store_dpre<NR, false>(sg, a.dpre + row * rv, hf, rv);
        }
        // dq_lr = W_q dpq (unless the streaming dQ kernel forms it from dpq)
        if (a.dq_lr) {
            u32x4_t bh_[KS], bl_[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) lrm_bop(sg[ks >> 1], ks & 1, bh_[ks], bl_[ks]);
            lrm_apply_store<KS, false>(w_dr, nullptr, bh_, bl_, lane, a.dq_lr + row * D, hf, valid);
        }
    }
    // workgroup sums: dz over the 32 tokens of each lane half, then the waves in order; dg
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float x = accz[rb][v];
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o, 64);
            if ((lane & 31) == 0) red[wave][32 * rb + 8 * (v >> 2) + 4 * hf + (v & 3)] = x;
        }
    float g = accg;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) g += __shfl_xor(g, o, 64);
    if (lane == 0) red[wave][R] = g;
    __syncthreads();
    // [dW_q | dS | dz | dg | pad] partials of rank rv: dz (rv), then dg
    float* part = a.part + (bh * a.nsplit + split) * (long)(2 * D * rv + rv + 4);
    if (tid <= rv) {
        const int j = tid < rv ? tid : R;
        part[2 * D * rv + tid] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
    }
}

template <int R, int FM, bool ABSPE>
__global__ __launch_bounds__(256) void k_bwd_lrm_k(LrBwdArgs a) {
    constexpr int D = 128, NR = R / 32, NB = R / 4, KS = R / 16;
    constexpr bool SILU = FM == 1, FAV = FM == 2;   // feature map: elu + 1, SiLU, FAVOR+
    constexpr int OB = FAV ? NR * KS * 64 : 1;
    __shared__ u32x4_t w_rd[NB * 64], w_dr[NB * 64], s_rd_hi[NB * 64], s_rd_lo[NB * 64], s_dr_hi[NB * 64],
        s_dr_lo[NB * 64];
    __shared__ u32x4_t om_hi[OB], om_lo[OB], omt_hi[OB], omt_lo[OB];   // FAVOR+: omega, omega^T
    __shared__ __attribute__((aligned(16))) float z_s[R];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5;
    const int split = blockIdx.x;
    const long bh = blockIdx.y;
    const int head = (int)(bh % a.H);
    const long L = a.L;
    const long t_lo = (long)split * a.chunk;
    const long t_hi = t_lo + a.chunk < L ? t_lo + a.chunk : L;
    // rv = the layer's rank (8, 16, 32 or 64); ranks rv .. R - 1 are padding with zero weights
    const int rv = a.g.R;
    const float* W = a.Wk + (long)head * D * rv;
    const float* dS = a.dSz + bh * (long)(rv * D + rv);
    lrm_build<R, false, false>(w_rd, nullptr, [&](int r, int d) { return r < rv ? W[d * rv + r] : 0.f; }, tid);
    lrm_build<R, true, false>(w_dr, nullptr, [&](int r, int d) { return r < rv ? W[d * rv + r] : 0.f; }, tid);
    lrm_build<R, false, true>(s_rd_hi, s_rd_lo, [&](int r, int d) { return r < rv ? dS[r * D + d] : 0.f; }, tid);
    lrm_build<R, true, true>(s_dr_hi, s_dr_lo, [&](int r, int d) { return r < rv ? dS[r * D + d] : 0.f; }, tid);
    if constexpr (FAV) {
        lrm_build_omega<R, false>(om_hi, om_lo, a.g.omega + (long)head * rv * rv, rv, tid);
        lrm_build_omega<R, true>(omt_hi, omt_lo, a.g.omega + (long)head * rv * rv, rv, tid);
    }
    for (int e = tid; e < R; e += 256) z_s[e] = e < rv ? dS[rv * D + e] : 0.f;
    __syncthreads();

    for (long t0 = t_lo + 32 * wave; t0 < t_hi; t0 += 128) {
        // the operand copies are re-read from LDS each step rather than held in registers
        asm volatile("" ::: "memory");
        const long t = t0 + (lane & 31);
        const bool valid = t < t_hi;
        const long row = bh * L + (valid ? t : t_lo);
        int crd[3];
        token_coords(valid ? t : 0, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
        float2 cs[NR][8];
        if constexpr (!ABSPE) lrm_pairs_cs<NR>(a, crd, hf, cs, rv);
        // p = k W_k (+ E), u = phi(p) and phi' (FAVOR+: u from all of p, kept in du, and p kept),
        // fk = rho(u) (u itself for absolute PE); zero past rank rv
        f32x16_t fk[NR], du[NR], pp[FAV ? NR : 1];
        {
            u32x4_t xb[8];
            lrm_rowops(xb, a.k + row * D, valid, hf);
#pragma unroll
            for (int rb = 0; rb < NR; ++rb) {
                f32x16_t p;
#pragma unroll
                for (int i = 0; i < 16; ++i) p[i] = 0.f;
#pragma unroll
                for (int s = 0; s < 8; ++s) p = mfma32(w_rd[(8 * rb + s) * 64 + lane], xb[s], p);
                if constexpr (ABSPE) lrm_add_e(a, crd, hf, p, rb, rv);
                if constexpr (FAV) {
                    pp[rb] = p;
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        float f0, f1, d0, d1;
                        lrm_phi<SILU>(p[2 * j], f0, d0);
                        lrm_phi<SILU>(p[2 * j + 1], f1, d1);
                        // ranks 2j, 2j + 1 of this lane's group: both valid or both padding (rv % 8 == 0)
                        if (32 * rb + 8 * (j >> 1) + 4 * hf + 2 * (j & 1) >= rv) f0 = f1 = d0 = d1 = 0.f;
                        du[rb][2 * j] = d0;
                        du[rb][2 * j + 1] = d1;
                        fk[rb][2 * j] = !valid ? 0.f : ABSPE ? f0 : f0 * cs[rb][j].x - f1 * cs[rb][j].y;
                        fk[rb][2 * j + 1] = !valid ? 0.f : ABSPE ? f1 : f0 * cs[rb][j].y + f1 * cs[rb][j].x;
                    }
                }
            }
        }
        if constexpr (FAV) {
            lrm_favor<NR>(om_hi, om_lo, pp, lane, hf, rv, du);   // du holds u
#pragma unroll
            for (int rb = 0; rb < NR; ++rb)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float f0 = du[rb][2 * j], f1 = du[rb][2 * j + 1];
                    fk[rb][2 * j] = !valid ? 0.f : ABSPE ? f0 : f0 * cs[rb][j].x - f1 * cs[rb][j].y;
                    fk[rb][2 * j + 1] = !valid ? 0.f : ABSPE ? f1 : f0 * cs[rb][j].y + f1 * cs[rb][j].x;
                }
        }
        // dv_lr = dS^T fk, or fk stored for the streaming dK/dV kernel to form it
        if (a.dv_lr) {
            u32x4_t bh_[KS], bl_[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) lrm_bop(fk[ks >> 1], ks & 1, bh_[ks], bl_[ks]);
            lrm_apply_store<KS, true>(s_dr_hi, s_dr_lo, bh_, bl_, lane, a.dv_lr + row * D, hf, valid);
        } else if (valid) {
            lrm_store_rank<NR>(fk, a.y2h + row * rv, a.y2l + row * rv, hf, rv);
        }
        // dpk = (rho^T(dS v) + dz) phi'
        f32x16_t sv[NR];
        {
            u32x4_t vb[8];
            lrm_rowops(vb, a.v + row * D, valid, hf);
#pragma unroll
            for (int rb = 0; rb < NR; ++rb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sv[rb][i] = 0.f;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int bi = (8 * rb + s) * 64 + lane;
                    sv[rb] = mfma32(s_rd_hi[bi], vb[s], sv[rb]);
                    sv[rb] = mfma32(s_rd_lo[bi], vb[s], sv[rb]);
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < NR; ++rb)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 z4 = lrm_z4(z_s, rb, j >> 1, hf);
                const float za = (j & 1) ? z4.z : z4.x, zb = (j & 1) ? z4.w : z4.y;
                float y0 = sv[rb][2 * j], y1 = sv[rb][2 * j + 1];
                if constexpr (!ABSPE) rot_t(y0, y1, cs[rb][j]);
                sv[rb][2 * j] = valid ? (y0 + za) * (FAV ? 1.f : du[rb][2 * j]) : 0.f;
                sv[rb][2 * j + 1] = valid ? (y1 + zb) * (FAV ? 1.f : du[rb][2 * j + 1]) : 0.f;
            }
        // FAVOR+: du -> dp through the features' Jacobian (u in du)
        if constexpr (FAV) lrm_favor_back<NR>(omt_hi, omt_lo, pp, du, lane, sv);
        if (valid) {
            lrm_store_rank<NR>(sv, a.y1h + row * rv, a.y1l + row * rv, hf, rv);
            // absolute PE: adds the key side's share (the query side wrote its own first)
            if constexpr (ABSPE) lrm_store_dpre<NR, true>(sv, a.dpre + row * rv, hf, rv);
        }
        // dk_lr = W_k dpk (unless the streaming dK/dV kernel forms it from dpk)
        if (a.dk_lr) {
            u32x4_t bh_[KS], bl_[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) lrm_bop(sv[ks >> 1], ks & 1, bh_[ks], bl_[ks]);
            lrm_apply_store<KS, false>(w_dr, nullptr, bh_, bl_, lane, a.dk_lr + row * D, hf, valid);
        }
    }
}

// out[d][r] = sum over the split's tokens t of x[t][d] y[t][r] (y = yh + yl,
// [t][rv], rv <= R: the columns past rv are zero in LDS), written to
// part + (slice * nsplit + split) * stride + off as [128][rv], or as
// [rv][128] when `trans`. Wave w owns rows d = 32w ..; 64-token stages go
// through LDS (rows padded to 288 / (2R + 32) bytes: the transposing reads
// of 4 rows x 16 columns per 16 lanes hit distinct banks), loaded one stage
// ahead into registers.
template <int R>
__global__ __launch_bounds__(256) void k_bwd_lrm_red(const uint16_t* __restrict__ x, const uint16_t* __restrict__ yh,
                                                     const uint16_t* __restrict__ yl, int rv, long L, int chunk,
                                                     int nsplit, float* __restrict__ part, long stride, long off,
                                                     int trans) {
    constexpr int D = 128, NR = R / 32, XP = D + 16, YP = R + 16, YC = R / 8;
    constexpr int NY = (2 * 64 * YC + 255) / 256;   // 16-byte pieces of y per thread
    __shared__ __attribute__((aligned(16))) uint16_t xs[64 * XP];
    __shared__ __attribute__((aligned(16))) uint16_t ys[2][64 * YP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x;
    const long bh = blockIdx.y;
    const long t_lo = (long)split * chunk;
    const long t_hi = t_lo + chunk < L ? t_lo + chunk : L;
    const uint16_t* xb = x + bh * L * D;
    const uint16_t* yhb = yh + bh * L * rv;
    const uint16_t* ylb = yl + bh * L * rv;
    f32x16_t acc[NR];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rb][i] = 0.f;
    u32x4_t rx[4], ry[NY];
    auto load = [&](long t0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int it = tid + 256 * m, r = it >> 4, c = it & 15;
            const long t = t0 + r;
            const u32x4_t w = ldg16(xb + (t < t_hi ? t : t_lo) * D + 8 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) rx[m][i] = t < t_hi ? w[i] : 0u;
        }
#pragma unroll
        for (int m = 0; m < NY; ++m) {
            const int it = tid + 256 * m;
            const int which = it / (64 * YC), r = (it % (64 * YC)) / YC, c = it % YC;
            const long t = t0 + r;
            if (it < 2 * 64 * YC) {
                const bool ok = t < t_hi && 8 * c < rv;
                const u32x4_t w = ok ? ldg16((which ? ylb : yhb) + t * rv + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < 4; ++i) ry[m][i] = w[i];
            }
        }
    };
    // transposing-read addresses: lane c of group g reads row 4x + c/4 (+ 16ks + 8(l/32)) at
    // columns 16(g % 2) + 4(c % 4) .. +3 (+ 32 * column block)
    const int g = lane >> 4, c = lane & 15, hf = lane >> 5;
    const int xr = (8 * hf + (c >> 2)) * XP + 32 * wave + 16 * (g & 1) + 4 * (c & 3);
    const int yr = (8 * hf + (c >> 2)) * YP + 16 * (g & 1) + 4 * (c & 3);
    if (t_lo < t_hi) load(t_lo);
    for (long t0 = t_lo; t0 < t_hi; t0 += 64) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int it = tid + 256 * m;
            *reinterpret_cast<u32x4_t*>(xs + (it >> 4) * XP + 8 * (it & 15)) = rx[m];
        }
#pragma unroll
        for (int m = 0; m < NY; ++m) {
            const int it = tid + 256 * m;
            if (it < 2 * 64 * YC) {
                const int which = it / (64 * YC), r = (it % (64 * YC)) / YC, cc = it % YC;
                *reinterpret_cast<u32x4_t*>(ys[which] + r * YP + 8 * cc) = ry[m];
            }
        }
        __syncthreads();
        if (t0 + 64 < t_hi) load(t0 + 64);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x2_t a0 = lds_tr8(xs + xr + 16 * ks * XP), a1 = lds_tr8(xs + xr + (16 * ks + 4) * XP);
            const u32x4_t av = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
            for (int rb = 0; rb < NR; ++rb) {
                const int o = 16 * ks * YP + 32 * rb;
                const u32x2_t h0 = lds_tr8(ys[0] + yr + o), h1 = lds_tr8(ys[0] + yr + o + 4 * YP);
                const u32x2_t l0 = lds_tr8(ys[1] + yr + o), l1 = lds_tr8(ys[1] + yr + o + 4 * YP);
                acc[rb] = mfma32(av, u32x4_t{h0[0], h0[1], h1[0], h1[1]}, acc[rb]);
                acc[rb] = mfma32(av, u32x4_t{l0[0], l0[1], l1[0], l1[1]}, acc[rb]);
            }
        }
        __syncthreads();
    }
    float* dst = part + (bh * nsplit + split) * stride + off;
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int d = 32 * wave + 8 * (v >> 2) + 4 * hf + (v & 3), r = 32 * rb + (lane & 31);
            if (r < rv) dst[trans ? r * D + d : d * rv + r] = acc[rb][v];
        }
}

// Per-axis sums for the absolute-PE tables: workgroup (c, bh) adds dpre over
// the tokens of slice bh whose coordinate on `axis` is c, in a fixed order
// (thread (j, r) takes every (256/R)-th such token from j, then the j's are
// added in order).
// Operand blocks of the streaming kernels' low-rank epilogue products, laid
// out as the low-rank kernels hold them in LDS (lrm_build, A[row d][k = r],
// R = 32 or 64 padded with zeros): W [D][rv] of each head rounded to bf16
// (DS false), or dS^T of each slice as hi + lo parts (DS: dS [rv][D] at
// src + g (rv D + rv)). Grid = matrices.
template <int R, bool DS>
__global__ __launch_bounds__(256) void k_bwd_lr_opblocks(const float* __restrict__ src, int rv, u32x4_t* __restrict__ hi,
                                                         u32x4_t* __restrict__ lo) {
    constexpr int D = 128, NB = R / 4 * 64;
    const long g = blockIdx.x;
    if constexpr (DS) {
        const float* dS = src + g * (long)(rv * D + rv);
        lrm_build<R, true, true>(hi + g * NB, lo + g * NB, [&](int r, int d) { return r < rv ? dS[r * D + d] : 0.f; },
                                 (int)threadIdx.x);
    } else {
        const float* W = src + g * (long)D * rv;
        lrm_build<R, true, false>(hi + g * NB, nullptr, [&](int r, int d) { return r < rv ? W[d * rv + r] : 0.f; },
                                  (int)threadIdx.x);
    }
}

__global__ __launch_bounds__(256) void k_bwd_e_sum(const float* __restrict__ dpre, long L, int Hg, int Wg, int axis,
                                                   int R, float* __restrict__ part) {
    __shared__ float red[256];
    const int c = blockIdx.x;
    const long bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int step = 256 / R, r = tid % R, j0 = tid / R;
    const long HW = (long)Hg * Wg;
    const long n = axis == 0 ? HW : (axis == 1 ? L / HW * Wg : L / HW * Hg);
    const float* src = dpre + bh * L * R;
    float acc = 0.f;
    for (long k = j0; k < n; k += step) {
        long l;
        if (axis == 0) l = (long)c * HW + k;
        else if (axis == 1) l = (k / Wg) * HW + (long)c * Wg + k % Wg;
        else l = k * Wg + c;
        acc += src[l * R + r];
    }
    red[tid] = acc;
    __syncthreads();
    if (tid < R) {
        float s = 0.f;
        for (int j = 0; j < step; ++j) s += red[j * R + tid];
        part[(bh * gridDim.x + c) * R + tid] = s;
    }
}

__global__ void k_bwd_sum_parts(const float* __restrict__ part, int B, int H, int nsplit, long stride, long off,
                                long n, int per_head, float* __restrict__ out) {
    const long nout = (per_head ? (long)H : (long)B * H) * n;
    for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < nout; e += (long)gridDim.x * blockDim.x) {
        const long o = e / n, x = e % n;
        float s = 0.f;
        if (per_head) {
            for (int b = 0; b < B; ++b)
                for (int sp = 0; sp < nsplit; ++sp) s += part[(((long)b * H + o) * nsplit + sp) * stride + off + x];
        } else {
            for (int sp = 0; sp < nsplit; ++sp) s += part[(o * nsplit + sp) * stride + off + x];
        }
        out[e] = s;
    }
}

// ---- launchers ------------------------------------------------------------
static unsigned grid_for(long n) {
    long g = (n + 255) / 256;
    if (g > 65536) g = 65536;
    return (unsigned)(g < 1 ? 1 : g);
}

template <int D, int R, bool BF>
static hipError_t bwd_lr_t(bool key_side, const LrBwdArgs& a, long BH, hipStream_t st) {
    dim3 grid((unsigned)a.nsplit, (unsigned)BH);
    const bool fv = a.g.fmap == 2;
    if (key_side) {
        if (fv) hipLaunchKernelGGL((k_bwd_lr_k<D, R, BF, true>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_bwd_lr_k<D, R, BF, false>), grid, dim3(256), 0, st, a);
    } else {
        if (fv) hipLaunchKernelGGL((k_bwd_lr_q<D, R, BF, true>), grid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_bwd_lr_q<D, R, BF, false>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

template <int D, bool BF>
static hipError_t bwd_lr_d(int R, bool key_side, const LrBwdArgs& a, long BH, hipStream_t st) {
    switch (R) {
        case 8: return bwd_lr_t<D, 8, BF>(key_side, a, BH, st);
        case 16: return bwd_lr_t<D, 16, BF>(key_side, a, BH, st);
        case 32: return bwd_lr_t<D, 32, BF>(key_side, a, BH, st);
        default: return bwd_lr_t<D, 64, BF>(key_side, a, BH, st);
    }
}

template <int R, int FM, bool ABSPE>
static hipError_t bwd_lrm(bool key_side, const LrBwdArgs& a, long BH, hipStream_t st) {
    constexpr int D = 128;
    const dim3 grid((unsigned)a.nsplit, (unsigned)BH);
    const int rv = a.g.R;   // the layer's rank; R is its padded width (32 or 64)
    if (!key_side) {
        // per token, then the [dW_q | dS | dz | dg] partials' dW_q and dS (stored transposed)
        const long qs = 2l * D * rv + rv + 4;
        hipLaunchKernelGGL((k_bwd_lrm_q<R, FM, ABSPE>), grid, dim3(256), 0, st, a);
        hipLaunchKernelGGL((k_bwd_lrm_red<R>), grid, dim3(256), 0, st, a.q, a.y1h, a.y1l, rv, a.L, a.chunk,
                           a.nsplit, a.part, qs, 0l, 0);
        hipLaunchKernelGGL((k_bwd_lrm_red<R>), grid, dim3(256), 0, st, a.dout, a.y2h, a.y2l, rv, a.L, a.chunk,
                           a.nsplit, a.part, qs, (long)D * rv, 1);
    } else {
        hipLaunchKernelGGL((k_bwd_lrm_k<R, FM, ABSPE>), grid, dim3(256), 0, st, a);
        hipLaunchKernelGGL((k_bwd_lrm_red<R>), grid, dim3(256), 0, st, a.k, a.y1h, a.y1l, rv, a.L, a.chunk,
                           a.nsplit, a.part, (long)D * rv, 0l, 0);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_lr(int dtype_bf16, int D, int R, bool key_side, const LrBwdArgs& a, long BH, hipStream_t st) {
    if (lr_bwd_on_mfma(dtype_bf16, D, R, key_side, a.token != 0)) {
        if (!a.y1h || !a.y1l || !a.y2h || !a.y2l) return hipErrorInvalidValue;
        if (a.g.R != R || (a.g.fmap == 2 && !a.g.omega)) return hipErrorInvalidValue;
        if (a.abspe && !a.dpre) return hipErrorInvalidValue;
        const bool w32 = R <= 32;   // ranks 8, 16 run padded to 32
#define SLR_LRM(FM_, AB_) \
    return w32 ? bwd_lrm<32, FM_, AB_>(key_side, a, BH, st) : bwd_lrm<64, FM_, AB_>(key_side, a, BH, st)
        switch (a.g.fmap * 2 + (a.abspe ? 1 : 0)) {
            case 0: SLR_LRM(0, false);
            case 1: SLR_LRM(0, true);
            case 2: SLR_LRM(1, false);
            case 3: SLR_LRM(1, true);
            case 4: SLR_LRM(2, false);
            default: SLR_LRM(2, true);
        }
#undef SLR_LRM
    }
    if (a.g.fmap == 2 && !a.g.omega) return hipErrorInvalidValue;
    if (dtype_bf16)
        return D == 64 ? bwd_lr_d<64, true>(R, key_side, a, BH, st) : bwd_lr_d<128, true>(R, key_side, a, BH, st);
    return D == 64 ? bwd_lr_d<64, false>(R, key_side, a, BH, st) : bwd_lr_d<128, false>(R, key_side, a, BH, st);
}

hipError_t launch_bwd_lr_opblocks(bool ds, int rv, const float* src, long n, uint16_t* hi, uint16_t* lo,
                                  hipStream_t st) {
    u32x4_t* h = reinterpret_cast<u32x4_t*>(hi);
    u32x4_t* l = reinterpret_cast<u32x4_t*>(lo);
    const dim3 grid((unsigned)n);
    if (rv <= 32) {
        if (ds) hipLaunchKernelGGL((k_bwd_lr_opblocks<32, true>), grid, dim3(256), 0, st, src, rv, h, l);
        else hipLaunchKernelGGL((k_bwd_lr_opblocks<32, false>), grid, dim3(256), 0, st, src, rv, h, l);
    } else {
        if (ds) hipLaunchKernelGGL((k_bwd_lr_opblocks<64, true>), grid, dim3(256), 0, st, src, rv, h, l);
        else hipLaunchKernelGGL((k_bwd_lr_opblocks<64, false>), grid, dim3(256), 0, st, src, rv, h, l);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_sum_parts(const float* part, int B, int H, int nsplit, long stride, long off, long n,
                                bool per_head, float* out, hipStream_t st) {
    const long nout = (per_head ? (long)H : (long)B * H) * n;
    hipLaunchKernelGGL(k_bwd_sum_parts, dim3(grid_for(nout)), dim3(256), 0, st, part, B, H, nsplit, stride, off, n,
                       per_head ? 1 : 0, out);
    return hipGetLastError();
}

hipError_t launch_bwd_e_sum(const float* dpre, long BH, long L, int T, int Hg, int Wg, int axis, int R, float* part,
                            hipStream_t st) {
    const int n = axis == 0 ? T : (axis == 1 ? Hg : Wg);
    hipLaunchKernelGGL(k_bwd_e_sum, dim3((unsigned)n, (unsigned)BH), dim3(256), 0, st, dpre, L, Hg, Wg, axis, R, part);
    return hipGetLastError();
}

hipError_t launch_bwd_inverse(const int32_t* idx, long BH, int nblk, int keep, uint32_t* bits, int32_t* cnt,
                              int32_t* off, int32_t* list, int32_t* order, hipStream_t st) {
    const int W = (nblk + 31) / 32;
    const long nbits = BH * nblk * (long)W;
    hipLaunchKernelGGL(k_inv_zero, dim3(grid_for(nbits)), dim3(256), 0, st, bits, nbits);
    hipLaunchKernelGGL(k_inv_mark, dim3(grid_for(BH * nblk * (long)keep)), dim3(256), 0, st, idx, BH, nblk, keep, W,
                       bits);
    hipLaunchKernelGGL(k_inv_count, dim3(grid_for(BH * nblk)), dim3(256), 0, st, bits, BH * nblk, W, cnt);
    hipLaunchKernelGGL(k_inv_scan, dim3((unsigned)BH), dim3(256), 0, st, cnt, nblk, off);
    hipLaunchKernelGGL(k_inv_fill, dim3(grid_for(BH * nblk)), dim3(256), 0, st, bits, off, BH, nblk, keep, W, list);
    if (order)
        hipLaunchKernelGGL(k_inv_order, dim3((unsigned)((nblk + 255) / 256), (unsigned)BH), dim3(256), 0, st, cnt, nblk,
                           order);
    return hipGetLastError();
}

template <int D, int BS>
static hipError_t bwd_sparse_t(bool dkdv, const BwdArgs& a, hipStream_t st) {
    if (dkdv)
        hipLaunchKernelGGL((k_bwd_dkdv<D, BS>), dim3((unsigned)a.nwg), dim3(BS * 2), 0, st, a, a.inv_off, a.inv_list,
                           a.order);
    else
        hipLaunchKernelGGL((k_bwd_dq<D, BS>), dim3((unsigned)a.nwg), dim3(BS * 2), 0, st, a, a.idx);
    return hipGetLastError();
}

static hipError_t bwd_sparse(int D, int BS, bool dkdv, const BwdArgs& a, hipStream_t st) {
    if (D == 128) return BS == 64 ? bwd_sparse_t<128, 64>(dkdv, a, st) : bwd_sparse_t<128, 32>(dkdv, a, st);
    return BS == 64 ? bwd_sparse_t<64, 64>(dkdv, a, st) : bwd_sparse_t<64, 32>(dkdv, a, st);
}

hipError_t launch_bwd_dq_tiles(const uint16_t* kr, const uint16_t* v, long BH, long L, int nblk, uint16_t* tiles,
                               hipStream_t st) {
    hipLaunchKernelGGL(k_bwd_dq_tiles, dim3((unsigned)nblk, (unsigned)BH), dim3(256), 0, st, kr, v, L, nblk, tiles);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(int dtype_bf16, int D, int BS, const BwdArgs& a, hipStream_t st) {
    if (dtype_bf16 && D == 128 && BS == 64 && a.dqt) {
        hipLaunchKernelGGL(k_bwd_dq_tiled, dim3((unsigned)a.nwg), dim3(256), 0, st, a, a.idx, a.dqt);
        return hipGetLastError();
    }
    if (dtype_bf16) return bwd_sparse(D, BS, false, a, st);
    if (D == 64)
        hipLaunchKernelGGL((k_bwd_dq_f32<64>), dim3((unsigned)a.nwg), dim3(256), 0, st, a, a.idx, BS);
    else
        hipLaunchKernelGGL((k_bwd_dq_f32<128>), dim3((unsigned)a.nwg), dim3(256), 0, st, a, a.idx, BS);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(int dtype_bf16, int D, int BS, const BwdArgs& a, hipStream_t st) {
    if (dtype_bf16 && D == 128 && BS == 64 && a.qtt) {
        hipLaunchKernelGGL(k_bwd_dkdv_tiled, dim3((unsigned)a.nwg), dim3(512), 0, st, a, a.inv_off, a.inv_list, a.order,
                           a.qtt);
        return hipGetLastError();
    }
    if (dtype_bf16) return bwd_sparse(D, BS, true, a, st);
    if (D == 64)
        hipLaunchKernelGGL((k_bwd_dkdv_f32<64>), dim3((unsigned)a.nwg), dim3(256), 0, st, a, a.inv_off, a.inv_list, BS);
    else
        hipLaunchKernelGGL((k_bwd_dkdv_f32<128>), dim3((unsigned)a.nwg), dim3(256), 0, st, a, a.inv_off, a.inv_list,
                           BS);
    return hipGetLastError();
}

}  // namespace slr
