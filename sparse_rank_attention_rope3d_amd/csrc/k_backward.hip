// Backward pass of the hybrid layer (bf16 layers, per-head gate).
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
//   k_bwd_dq    one workgroup per query block: a first pass over its kept
//               tiles gives each row's log-sum-exp, a second forms dS tile by
//               tile on MFMA (S^T = K Q^T and dP^T = V dO^T, so each lane owns
//               one query row) and accumulates dQ^T = K^T dS^T;
//   k_bwd_dkdv  one workgroup per key block, over the query blocks that keep
//               it (an inverse of the kept lists, built deterministically from
//               a bitmap): S = Q K^T and dP = dO V^T with each lane owning one
//               key, dV^T += dO^T P and dK^T += Q^T dS.
// The rotated-space gradients go back through the 3D RoPE by its transpose
// (each pair turned by the opposite angle) in the epilogues, where the
// low-rank parts are added.
//
// Low-rank branch (RoLA §4.1-4.3, App. A): fp32 VALU kernels over token
// tiles, split along L with fixed-order reductions of the partial sums.
#include "slr_common.h"
#include "slr_launch.h"

namespace slr {

// (cos, sin) of backbone rotary pair p (0 .. D/2-1) at token coordinates crd
__device__ __forceinline__ float2 rope_cs(const float2* __restrict__ tab, const RopeGeom& g, int p, const int* crd) {
    int a, j;
    if (p < g.np[0]) { a = 0; j = p; }
    else if (p < g.np[0] + g.np[1]) { a = 1; j = p - g.np[0]; }
    else { a = 2; j = p - g.np[0] - g.np[1]; }
    return tab[g.tab_off[a] + crd[a] * g.np[a] + j];
}

// (cos, sin) of low-rank pair pr: the axis chunks hold lp[] pairs that reuse
// the backbone's schedule of their axis
__device__ __forceinline__ float2 lowrank_cs(const float2* __restrict__ tab, const LrGeom& g, int pr, const int* crd) {
    int a, j;
    if (pr < g.lp[0]) { a = 0; j = pr; }
    else if (pr < g.lp[0] + g.lp[1]) { a = 1; j = pr - g.lp[0]; }
    else { a = 2; j = pr - g.lp[0] - g.lp[1]; }
    return tab[g.rope.tab_off[a] + crd[a] * g.rope.np[a] + j];
}

// y -> R^T y for one pair: turned by minus its angle
__device__ __forceinline__ void rot_t(float& y0, float& y1, float2 cs) {
    const float x0 = y0 * cs.x + y1 * cs.y;
    const float x1 = -y0 * cs.y + y1 * cs.x;
    y0 = x0;
    y1 = x1;
}

// ---------------------------------------------------------------------------
// Staging of one BS x D bf16 block of rows into LDS. Thread tid < (BS/8)(D/8)
// takes 8 rows x 8 dims: rows 16G + 4h + (e & 3) + 8(e >> 2) (e = 0..7) of
// 16-row group G with lane half h, dims 8c .. 8c+7. `rm` (optional) receives
// the rows row-major with stride D + 8; `tr` (optional) receives the
// transpose [D][BS + 8] with the rows of each 16-group at positions
// 16G + 8h + e, the slot order in which a 32x32 MFMA accumulator holds its
// rows, so an accumulator packs straight into the B operand that meets it.
// Rows at or past `limit` read as zeros.
template <int D, int BS>
__device__ __forceinline__ void stage_block(const uint16_t* __restrict__ src, long row0, long limit, uint16_t* rm,
                                            uint16_t* tr, int tid) {
    constexpr int KLD = D + 8, VLD = BS + 8, NB = (BS / 8) * (D / 8);
    if (tid >= NB) return;
    const int c = tid % (D / 8), gp = tid / (D / 8), G = gp >> 1, h = gp & 1;
    u32x4_t x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int r = 16 * G + 4 * h + (e & 3) + 8 * (e >> 2);
        x[e] = row0 + r < limit ? ldg16(src + (row0 + r) * D + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
    }
    if (rm) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int r = 16 * G + 4 * h + (e & 3) + 8 * (e >> 2);
            *reinterpret_cast<u32x4_t*>(rm + r * KLD + 8 * c) = x[e];
        }
    }
    if (tr) {
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            u32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t a0 = x[2 * i][f >> 1], a1 = x[2 * i + 1][f >> 1];
                o[i] = (f & 1) ? __builtin_amdgcn_perm(a1, a0, 0x07060302u) : __builtin_amdgcn_perm(a1, a0, 0x05040100u);
            }
            *reinterpret_cast<u32x4_t*>(tr + (8 * c + f) * VLD + 16 * G + 8 * h) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// dQ. Workgroup = one query block, BS/32 waves of 32 rows.
template <int D, int BS>
__global__ __launch_bounds__(BS * 2) void k_bwd_dq(BwdArgs a) {
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
    const int32_t* ix = a.idx + (bh * a.nblk + qb) * (long)a.keep;

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

    const float sl2 = a.scale * kLog2e;
    const bool ragged = (L % BS) != 0;

    // ---- pass 1: log-sum-exp of each row over its kept keys (log2 units)
    float m_run = -INFINITY, l_run = 0.f;
    for (int n = 0; n < a.keep; ++n) {
        const int j = ix[n];
        if (j < 0 || j >= a.nblk) continue;
        __syncthreads();
        stage_block<D, BS>(kr, (long)j * BS, rows, k_lds, nullptr, tid);
        __syncthreads();
        float x[NKB][16];
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16_t sacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s)
                sacc = mfma32(*reinterpret_cast<const u32x4_t*>(k_lds + (32 * kb + l32) * KLD + 16 * s + 8 * hf),
                              qop[s], sacc);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const long key = (long)j * BS + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
                x[kb][i] = (ragged && key >= L) ? -INFINITY : sacc[i] * sl2;
                mx = fmaxf(mx, x[kb][i]);
            }
        }
        const float mn = fmaxf(m_run, mx);
        if (mn != -INFINITY) {
            float l = l_run * exp2f(m_run - mn);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) l += exp2f(x[kb][i] - mn);
            l_run = l;
            m_run = mn;
        }
    }
    float lse2;
    {
        const float mo = wave_xor32(m_run), lo = wave_xor32(l_run);
        const float m = fmaxf(m_run, mo);
        const float l = (m_run == -INFINITY ? 0.f : l_run * exp2f(m_run - m)) +
                        (mo == -INFINITY ? 0.f : lo * exp2f(mo - m));
        lse2 = m + log2f(l);
    }
    if (hf == 0) {
        a.lse2[bh * rows + qrow] = lse2;
        a.delta[bh * rows + qrow] = qval ? dl : 0.f;
    }

    // ---- pass 2: dS and dQ^T = K^T dS^T
    f32x16_t dqacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;
    for (int n = 0; n < a.keep; ++n) {
        const int j = ix[n];
        if (j < 0 || j >= a.nblk) continue;
        __syncthreads();
        stage_block<D, BS>(kr, (long)j * BS, rows, k_lds, kt_lds, tid);
        stage_block<D, BS>(vg, (long)j * BS, L, v_lds, nullptr, tid);
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16_t sacc, dpacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int o = (32 * kb + l32) * KLD + 16 * s + 8 * hf;
                sacc = mfma32(*reinterpret_cast<const u32x4_t*>(k_lds + o), qop[s], sacc);
                dpacc = mfma32(*reinterpret_cast<const u32x4_t*>(v_lds + o), doop[s], dpacc);
            }
            float ds[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const long key = (long)j * BS + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
                const float p = (ragged && key >= L) ? 0.f : exp2f(sacc[i] * sl2 - lse2);
                ds[i] = p * (dpacc[i] - dl);
            }
            u32x4_t dsop[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) dsop[h2][i] = pack_bf2(ds[8 * h2 + 2 * i], ds[8 * h2 + 2 * i + 1]);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    dqacc[db] = mfma32(
                        *reinterpret_cast<const u32x4_t*>(kt_lds + (32 * db + l32) * VLD + 32 * kb + 16 * h2 + 8 * hf),
                        dsop[h2], dqacc[db]);
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
// dK, dV. Workgroup = one key block, BS/32 waves of 32 keys.
template <int D, int BS>
__global__ __launch_bounds__(BS * 2) void k_bwd_dkdv(BwdArgs a) {
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
    const int jb = (int)(wid % a.nblk);
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
    const float sl2 = a.scale * kLog2e;
    f32x16_t dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) { dkacc[db][i] = 0.f; dvacc[db][i] = 0.f; }

    const int32_t* off = a.inv_off + bh * (long)(a.nblk + 1);
    const int32_t* list = a.inv_list + bh * (long)a.nblk * a.keep;
    const int n0 = off[jb], n1 = off[jb + 1];
    for (int n = n0; n < n1; ++n) {
        const int i = list[n];
        __syncthreads();
        stage_block<D, BS>(qr, (long)i * BS, rows, q_lds, qt_lds, tid);
        stage_block<D, BS>(dg, (long)i * BS, L, do_lds, dot_lds, tid);
        if (tid < BS) {
            lse_lds[tid] = a.lse2[bh * rows + (long)i * BS + tid];
            dl_lds[tid] = a.delta[bh * rows + (long)i * BS + tid];
        }
        __syncthreads();
#pragma unroll
        for (int qs = 0; qs < NQB; ++qs) {
            f32x16_t sacc, dpacc;
#pragma unroll
            for (int e = 0; e < 16; ++e) { sacc[e] = 0.f; dpacc[e] = 0.f; }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int o = (32 * qs + l32) * KLD + 16 * s + 8 * hf;
                sacc = mfma32(*reinterpret_cast<const u32x4_t*>(q_lds + o), kop[s], sacc);
                dpacc = mfma32(*reinterpret_cast<const u32x4_t*>(do_lds + o), vop[s], dpacc);
            }
            // lane = key, register e = query row 32qs + 8(e/4) + 4hf + e%4
            float p[16], ds[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 32 * qs + 8 * (e >> 2) + 4 * hf + (e & 3);
                p[e] = exp2f(sacc[e] * sl2 - lse_lds[r]);
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
            for (int i = 0; i < 4; ++i) y[i] = dkacc[db][4 * g4 + i] * a.scale;
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
// Low-rank branch. phi and its derivative: elu + 1 (x + 1 | e^x) or SiLU.
__device__ __forceinline__ void phi_grad(int fmap, float x, float& f, float& df) {
    if (fmap) {
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

// Query side, per token l (O_l = rho_l(w_l)^T S / n_l, w_l = phi(q_l W_q),
// n_l = w_l . z + eps, or L for SiLU), given dO_lr = g_h dout:
//   dfq = S dO / n, dn = -(dO . O) / n, dw = rho^T dfq + dn z, dpq = dw phi',
//   dq_lr = W_q dpq; partial sums of dW_q = q^T dpq, dS = fq dO^T / n,
//   dz = dn w and dg = dout . O over the workgroup's tokens.
// Partial layout per (slice, split): [dW_q D*R | dS R*D | dz R | dg 1].
template <int D, int R>
__global__ __launch_bounds__(256) void k_bwd_lr_q(LrBwdArgs a) {
    constexpr int TT = 32, XLD = D + 1, RLD = R + 1, NW = D * R / 256;
    static_assert(NW >= 1 && D * R % 256 == 0, "partials per thread");
    __shared__ float w_s[D * R];
    __shared__ float s_s[R * D];
    __shared__ float z_s[R];
    __shared__ float x_s[TT * XLD];
    __shared__ float g_s[TT * XLD];
    __shared__ float w_t[TT * RLD];
    __shared__ float f_t[TT * RLD];
    __shared__ float d_t[TT * RLD];
    __shared__ float n_s[TT], dn_s[TT];
    __shared__ float red[256];
    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const long bh = blockIdx.y;
    const int head = (int)(bh % a.H);
    const long L = a.L;
    const long t_lo = (long)split * a.chunk;
    const long t_hi = t_lo + a.chunk < L ? t_lo + a.chunk : L;
    const float gh = a.gate[head];
    const bool silu = a.g.fmap != 0;
    for (int e = tid; e < D * R; e += 256) w_s[e] = round_bf(a.Wq[(long)head * D * R + e]);
    for (int e = tid; e < R * D; e += 256) s_s[e] = a.S[bh * R * D + e];
    for (int e = tid; e < R; e += 256) z_s[e] = a.z[bh * R + e];
    float accW[NW], accS[NW], accz = 0.f, accg = 0.f;
#pragma unroll
    for (int c = 0; c < NW; ++c) { accW[c] = 0.f; accS[c] = 0.f; }
    const uint16_t* qs = a.q + bh * L * D;
    const uint16_t* gs = a.dout + bh * L * D;
    __syncthreads();

    for (long t0 = t_lo; t0 < t_hi; t0 += TT) {
        for (int e = tid; e < TT * D / 8; e += 256) {
            const int t = e / (D / 8), c = e % (D / 8);
            const long l = t0 + t;
            u32x4_t xq{0u, 0u, 0u, 0u}, xg{0u, 0u, 0u, 0u};
            if (l < t_hi) {
                xq = ldg16(qs + l * D + 8 * c);
                xg = ldg16(gs + l * D + 8 * c);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x_s[t * XLD + 8 * c + 2 * i] = bf_lo(xq[i]);
                x_s[t * XLD + 8 * c + 2 * i + 1] = bf_hi(xq[i]);
                g_s[t * XLD + 8 * c + 2 * i] = bf_lo(xg[i]);
                g_s[t * XLD + 8 * c + 2 * i + 1] = bf_hi(xg[i]);
            }
        }
        __syncthreads();
        for (int e = tid; e < TT * R; e += 256) {
            const int t = e / R, r = e % R;
            float acc = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) acc += x_s[t * XLD + d] * w_s[d * R + r];
            float f, df;
            phi_grad(a.g.fmap, acc, f, df);
            w_t[t * RLD + r] = f;
            d_t[t * RLD + r] = df;
        }
        __syncthreads();
        for (int e = tid; e < TT * R / 2; e += 256) {
            const int t = e / (R / 2), pr = e % (R / 2);
            const long l = t0 + t;
            float f0 = w_t[t * RLD + 2 * pr], f1 = w_t[t * RLD + 2 * pr + 1];
            if (l < t_hi) {
                int crd[3];
                token_coords(l, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
                const float2 cs = lowrank_cs(a.tab, a.g, pr, crd);
                const float y0 = f0 * cs.x - f1 * cs.y, y1 = f0 * cs.y + f1 * cs.x;
                f0 = y0;
                f1 = y1;
            }
            f_t[t * RLD + 2 * pr] = f0;
            f_t[t * RLD + 2 * pr + 1] = f1;
        }
        if (tid < TT) {
            float n = 0.f;
            for (int r = 0; r < R; ++r) n += w_t[tid * RLD + r] * z_s[r];
            n_s[tid] = silu ? (float)L : n + a.eps;
        }
        __syncthreads();
        {
            // 8 threads per row: readout O and dout . O
            const int t = tid >> 3, c = tid & 7;
            const float invn = 1.f / n_s[t];
            float dot = 0.f;
            for (int dd = 0; dd < D / 8; ++dd) {
                const int d = c + 8 * dd;
                float o = 0.f;
                for (int r = 0; r < R; ++r) o += f_t[t * RLD + r] * s_s[r * D + d];
                dot += g_s[t * XLD + d] * (o * invn);
            }
            dot += __shfl_xor(dot, 1, 64);
            dot += __shfl_xor(dot, 2, 64);
            dot += __shfl_xor(dot, 4, 64);
            if (c == 0) {
                dn_s[t] = silu ? 0.f : -gh * dot * invn;
                accg += dot;
            }
        }
        __syncthreads();
        for (int e = tid; e < TT * R / 2; e += 256) {
            const int t = e / (R / 2), pr = e % (R / 2);
            const long l = t0 + t;
            const float sc = gh / n_s[t];
            float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) {
                const float go = g_s[t * XLD + d];
                a0 += s_s[(2 * pr) * D + d] * go;
                a1 += s_s[(2 * pr + 1) * D + d] * go;
            }
            a0 *= sc;
            a1 *= sc;
            if (l < t_hi) {
                int crd[3];
                token_coords(l, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
                rot_t(a0, a1, lowrank_cs(a.tab, a.g, pr, crd));
            }
            const float dn = dn_s[t];
            d_t[t * RLD + 2 * pr] *= a0 + dn * z_s[2 * pr];
            d_t[t * RLD + 2 * pr + 1] *= a1 + dn * z_s[2 * pr + 1];
        }
        __syncthreads();
        for (int e = tid; e < TT * D; e += 256) {
            const int t = e / D, d = e % D;
            const long l = t0 + t;
            if (l < t_hi) {
                float acc = 0.f;
                for (int r = 0; r < R; ++r) acc += w_s[d * R + r] * d_t[t * RLD + r];
                a.dq_lr[(bh * L + l) * D + d] = acc;
            }
        }
        // partial sums: element tid + 256c of dW_q [D][R] and of dS [R][D]
#pragma unroll 1
        for (int t = 0; t < TT; ++t) {
            const float sc = gh / n_s[t];
#pragma unroll
            for (int c = 0; c < NW; ++c) {
                const int e = tid + 256 * c;
                accW[c] += x_s[t * XLD + e / R] * d_t[t * RLD + e % R];
                accS[c] += f_t[t * RLD + e / D] * (g_s[t * XLD + e % D] * sc);
            }
        }
        if (tid < R) {
            float acc = 0.f;
            for (int t = 0; t < TT; ++t) acc += dn_s[t] * w_t[t * RLD + tid];
            accz += acc;
        }
        __syncthreads();
    }
    float* part = a.part + (bh * a.nsplit + split) * (long)(2 * D * R + R + 1);
#pragma unroll
    for (int c = 0; c < NW; ++c) {
        part[tid + 256 * c] = accW[c];
        part[D * R + tid + 256 * c] = accS[c];
    }
    if (tid < R) part[2 * D * R + tid] = accz;
    red[tid] = accg;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int t = 0; t < 256; ++t) s += red[t];
        part[2 * D * R + R] = s;
    }
}

// Key side, per token m (S = sum rho_m(u_m) v_m^T, z = sum u_m, u = phi(k W_k)),
// given the reduced dS, dz: dv_lr = dS^T fk, dfk = dS v, du = rho^T dfk + dz,
// dpk = du phi', dk_lr = W_k dpk; partial sums of dW_k = k^T dpk [D*R].
template <int D, int R>
__global__ __launch_bounds__(256) void k_bwd_lr_k(LrBwdArgs a) {
    constexpr int TT = 32, XLD = D + 1, RLD = R + 1, NW = D * R / 256;
    __shared__ float w_s[D * R];
    __shared__ float s_s[R * D];
    __shared__ float z_s[R];
    __shared__ float x_s[TT * XLD];
    __shared__ float v_s[TT * XLD];
    __shared__ float f_t[TT * RLD];
    __shared__ float d_t[TT * RLD];
    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const long bh = blockIdx.y;
    const int head = (int)(bh % a.H);
    const long L = a.L;
    const long t_lo = (long)split * a.chunk;
    const long t_hi = t_lo + a.chunk < L ? t_lo + a.chunk : L;
    const float* dsz = a.dSz + bh * (long)(R * D + R);
    for (int e = tid; e < D * R; e += 256) w_s[e] = round_bf(a.Wk[(long)head * D * R + e]);
    for (int e = tid; e < R * D; e += 256) s_s[e] = dsz[e];
    for (int e = tid; e < R; e += 256) z_s[e] = dsz[R * D + e];
    float accW[NW];
#pragma unroll
    for (int c = 0; c < NW; ++c) accW[c] = 0.f;
    const uint16_t* ks = a.k + bh * L * D;
    const uint16_t* vs = a.v + bh * L * D;
    __syncthreads();

    for (long t0 = t_lo; t0 < t_hi; t0 += TT) {
        for (int e = tid; e < TT * D / 8; e += 256) {
            const int t = e / (D / 8), c = e % (D / 8);
            const long l = t0 + t;
            u32x4_t xk{0u, 0u, 0u, 0u}, xv{0u, 0u, 0u, 0u};
            if (l < t_hi) {
                xk = ldg16(ks + l * D + 8 * c);
                xv = ldg16(vs + l * D + 8 * c);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x_s[t * XLD + 8 * c + 2 * i] = bf_lo(xk[i]);
                x_s[t * XLD + 8 * c + 2 * i + 1] = bf_hi(xk[i]);
                v_s[t * XLD + 8 * c + 2 * i] = bf_lo(xv[i]);
                v_s[t * XLD + 8 * c + 2 * i + 1] = bf_hi(xv[i]);
            }
        }
        __syncthreads();
        // features, rotated features and phi' (pairs in one thread)
        for (int e = tid; e < TT * R / 2; e += 256) {
            const int t = e / (R / 2), pr = e % (R / 2);
            const long l = t0 + t;
            float p0 = 0.f, p1 = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) {
                const float x = x_s[t * XLD + d];
                p0 += x * w_s[d * R + 2 * pr];
                p1 += x * w_s[d * R + 2 * pr + 1];
            }
            float u0, u1, g0, g1;
            phi_grad(a.g.fmap, p0, u0, g0);
            phi_grad(a.g.fmap, p1, u1, g1);
            float f0 = u0, f1 = u1;
            if (l < t_hi) {
                int crd[3];
                token_coords(l, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
                const float2 cs = lowrank_cs(a.tab, a.g, pr, crd);
                f0 = u0 * cs.x - u1 * cs.y;
                f1 = u0 * cs.y + u1 * cs.x;
            }
            f_t[t * RLD + 2 * pr] = f0;
            f_t[t * RLD + 2 * pr + 1] = f1;
            d_t[t * RLD + 2 * pr] = g0;
            d_t[t * RLD + 2 * pr + 1] = g1;
        }
        __syncthreads();
        // dv_lr = dS^T fk
        for (int e = tid; e < TT * D; e += 256) {
            const int t = e / D, d = e % D;
            const long l = t0 + t;
            if (l < t_hi) {
                float acc = 0.f;
                for (int r = 0; r < R; ++r) acc += s_s[r * D + d] * f_t[t * RLD + r];
                a.dv_lr[(bh * L + l) * D + d] = acc;
            }
        }
        // dfk = dS v, back through the rotation, + dz, times phi'
        for (int e = tid; e < TT * R / 2; e += 256) {
            const int t = e / (R / 2), pr = e % (R / 2);
            const long l = t0 + t;
            float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) {
                const float vv = v_s[t * XLD + d];
                a0 += s_s[(2 * pr) * D + d] * vv;
                a1 += s_s[(2 * pr + 1) * D + d] * vv;
            }
            if (l < t_hi) {
                int crd[3];
                token_coords(l, a.g.rope.Hg, a.g.rope.Wg, crd[0], crd[1], crd[2]);
                rot_t(a0, a1, lowrank_cs(a.tab, a.g, pr, crd));
            }
            d_t[t * RLD + 2 * pr] *= a0 + z_s[2 * pr];
            d_t[t * RLD + 2 * pr + 1] *= a1 + z_s[2 * pr + 1];
        }
        __syncthreads();
        for (int e = tid; e < TT * D; e += 256) {
            const int t = e / D, d = e % D;
            const long l = t0 + t;
            if (l < t_hi) {
                float acc = 0.f;
                for (int r = 0; r < R; ++r) acc += w_s[d * R + r] * d_t[t * RLD + r];
                a.dk_lr[(bh * L + l) * D + d] = acc;
            }
        }
#pragma unroll 1
        for (int t = 0; t < TT; ++t) {
#pragma unroll
            for (int c = 0; c < NW; ++c) {
                const int e = tid + 256 * c;
                accW[c] += x_s[t * XLD + e / R] * d_t[t * RLD + e % R];
            }
        }
        __syncthreads();
    }
    float* part = a.part + (bh * a.nsplit + split) * (long)(D * R);
#pragma unroll
    for (int c = 0; c < NW; ++c) part[tid + 256 * c] = accW[c];
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

template <int D, int R>
static hipError_t bwd_lr_t(bool key_side, const LrBwdArgs& a, long BH, hipStream_t st) {
    dim3 grid((unsigned)a.nsplit, (unsigned)BH);
    if (key_side)
        hipLaunchKernelGGL((k_bwd_lr_k<D, R>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_bwd_lr_q<D, R>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int D>
static hipError_t bwd_lr_d(int R, bool key_side, const LrBwdArgs& a, long BH, hipStream_t st) {
    switch (R) {
        case 8: return bwd_lr_t<D, 8>(key_side, a, BH, st);
        case 16: return bwd_lr_t<D, 16>(key_side, a, BH, st);
        case 32: return bwd_lr_t<D, 32>(key_side, a, BH, st);
        default: return bwd_lr_t<D, 64>(key_side, a, BH, st);
    }
}

hipError_t launch_bwd_lr(int D, int R, bool key_side, const LrBwdArgs& a, long BH, hipStream_t st) {
    return D == 64 ? bwd_lr_d<64>(R, key_side, a, BH, st) : bwd_lr_d<128>(R, key_side, a, BH, st);
}

hipError_t launch_bwd_sum_parts(const float* part, int B, int H, int nsplit, long stride, long off, long n,
                                bool per_head, float* out, hipStream_t st) {
    const long nout = (per_head ? (long)H : (long)B * H) * n;
    hipLaunchKernelGGL(k_bwd_sum_parts, dim3(grid_for(nout)), dim3(256), 0, st, part, B, H, nsplit, stride, off, n,
                       per_head ? 1 : 0, out);
    return hipGetLastError();
}

hipError_t launch_bwd_inverse(const int32_t* idx, long BH, int nblk, int keep, uint32_t* bits, int32_t* cnt,
                              int32_t* off, int32_t* list, hipStream_t st) {
    const int W = (nblk + 31) / 32;
    const long nbits = BH * nblk * (long)W;
    hipLaunchKernelGGL(k_inv_zero, dim3(grid_for(nbits)), dim3(256), 0, st, bits, nbits);
    hipLaunchKernelGGL(k_inv_mark, dim3(grid_for(BH * nblk * (long)keep)), dim3(256), 0, st, idx, BH, nblk, keep, W,
                       bits);
    hipLaunchKernelGGL(k_inv_count, dim3(grid_for(BH * nblk)), dim3(256), 0, st, bits, BH * nblk, W, cnt);
    hipLaunchKernelGGL(k_inv_scan, dim3((unsigned)BH), dim3(256), 0, st, cnt, nblk, off);
    hipLaunchKernelGGL(k_inv_fill, dim3(grid_for(BH * nblk)), dim3(256), 0, st, bits, off, BH, nblk, keep, W, list);
    return hipGetLastError();
}

template <int D, int BS>
static hipError_t bwd_sparse_t(bool dkdv, const BwdArgs& a, hipStream_t st) {
    if (dkdv)
        hipLaunchKernelGGL((k_bwd_dkdv<D, BS>), dim3((unsigned)a.nwg), dim3(BS * 2), 0, st, a);
    else
        hipLaunchKernelGGL((k_bwd_dq<D, BS>), dim3((unsigned)a.nwg), dim3(BS * 2), 0, st, a);
    return hipGetLastError();
}

static hipError_t bwd_sparse(int D, int BS, bool dkdv, const BwdArgs& a, hipStream_t st) {
    if (D == 128) return BS == 64 ? bwd_sparse_t<128, 64>(dkdv, a, st) : bwd_sparse_t<128, 32>(dkdv, a, st);
    return BS == 64 ? bwd_sparse_t<64, 64>(dkdv, a, st) : bwd_sparse_t<64, 32>(dkdv, a, st);
}

hipError_t launch_bwd_dq(int D, int BS, const BwdArgs& a, hipStream_t st) { return bwd_sparse(D, BS, false, a, st); }
hipError_t launch_bwd_dkdv(int D, int BS, const BwdArgs& a, hipStream_t st) { return bwd_sparse(D, BS, true, a, st); }

}  // namespace slr
