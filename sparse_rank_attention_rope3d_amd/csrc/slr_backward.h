// Host-side launch wrappers of the backward-pass kernels (internal to the library).
#pragma once

#include "slr_launch.h"

namespace slr {

// ---- backward pass ---------------------------------------------------------

// Bytes per block of the streaming kernels' tiles (bf16, D = 128, 64-token
// blocks): [K | V] for dQ, [Q | dO | 2 KB of row statistics] for dK/dV.
constexpr size_t kBwdDqTileBytes = 2ul * 64 * 128 * 2;
constexpr size_t kBwdQtTileBytes = (2ul * 64 * 128 + 1024) * 2;

// Sparse branch: softmax attention over the kept blocks, differentiated.
struct BwdArgs {
    const uint16_t* qr;        // [BH][nblk*BS][D] rotated q, zero rows past L (unscaled)
    const uint16_t* kr;        // same layout, rotated k
    const uint16_t* v;         // [BH][L][D]
    const uint16_t* o_sp;      // [BH][L][D] the forward's sparse-branch output
    const uint16_t* dout;      // [BH][L][D] gradient of the layer output
    const int32_t* idx;        // [BH][nblk][keep] kept key blocks per query block
    const int32_t* inv_off;    // [BH][nblk + 1] query-block list offsets per key block
    const int32_t* inv_list;   // [BH][nblk * keep] query blocks keeping each key block, ascending
    const int32_t* order;      // [BH][nblk] key blocks by list length, longest first (dK/dV launch order)
    const uint16_t* dqt;       // bf16, D = 128, 64-token blocks: [BH][nblk][K | V] 32 KB operand-order
                               // tiles of the streaming dQ kernel (null: the staging kernel)
    const uint16_t* qtt;       // same shapes: [BH][nblk][Q | dO | stats] 34 KB tiles of the streaming
                               // dK/dV kernel, written by the dQ kernel (null: staging kernels)
    const float* lse_in;       // [BH][L] the forward's log2 normalisers
    float* lse2;               // [BH][nblk*BS] the same, zero on padded rows
    float qmul;                // score (log2 units) = qmul * (q_rot . k_rot): log2(e)/sqrt(D), or 1
                               // when q_rot already carries that factor
    float kscale;              // dk_rot = kscale * sum dS q_rot: 1/sqrt(D), or ln 2 for scaled q
    float* delta;              // [BH][nblk*BS] dO . O_sparse per row
    const float* dq_lr;        // [BH][L][D] low-rank parts of the gradients (fp32), read when the
    const float* dk_lr;        // streaming kernel does not form them itself (lr_ph null)
    const float* dv_lr;
    // Streaming kernels (dqt / qtt set): the low-rank parts formed in the epilogue from the
    // per-token rank vectors the MFMA low-rank kernels stored (bf16 hi + lo, [BH][L][lr_rv]):
    // dq_lr = W_q dpq (dQ kernel), dk_lr = W_k dpk and dv_lr = dS^T fk (dK/dV kernel).
    const uint16_t *lr_ph, *lr_pl;   // dpq or dpk (null: read dq_lr / dk_lr, dv_lr)
    const uint16_t *lr_fh, *lr_fl;   // fk (dK/dV kernel)
    const uint16_t* lr_w;            // [H] operand blocks of W_q or W_k (launch_bwd_lr_opblocks)
    const uint16_t *lr_sh, *lr_sl;   // [BH] operand blocks of dS^T, hi and lo (dK/dV kernel)
    int lr_rv, H;
    uint16_t* dq;              // [BH][L][D] outputs
    uint16_t* dk;
    uint16_t* dv;
    const float2* tab;         // rotary (cos, sin) tables
    RopeGeom g;
    long L;
    int nblk, keep;
    float scale;               // 1/sqrt(D)
    long nwg;
};

// Low-rank branch (per-head gate): gradients of O_lr given g_h dout.
struct LrBwdArgs {
    const uint16_t *q, *k, *v, *dout;   // [BH][L][D]
    const float *Wq, *Wk;               // [H][D][R] (used rounded to bf16)
    const float *S, *z;                 // [BH][R][D], [BH][R] the forward summary
    const float* gate;                  // [H]
    const float* dSz;                   // [BH][R*D + R] reduced dS, dz (key side input)
    const float2* tab;
    LrGeom g;
    float eps;
    long L;
    int H, chunk, nsplit;
    float *dq_lr, *dk_lr, *dv_lr;       // [BH][L][D] (MFMA kernels: null when the streaming
                                        // sparse kernels form them; the key side then stores fk in y2)
    float* part;                        // split partials
    int abspe;                          // absolute-PE variant: E added before phi, no rotation
    const float *Et, *Eh, *Ew;          // [T|Hg|Wg][R] (absolute PE)
    float* dpre;                        // absolute PE: [BH][L][R] gradient w.r.t. x W + E (q side + k side)
    int token;                          // token-wise gate (RoLA §4.4) instead of g_h
    const float *wg, *bg;               // [H][D], [H]
    const void* o_sp;                   // [BH][L][D] the forward's O_sparse (layer dtype)
    void* dosp;                         // [BH][L][D] (layer dtype): the sparse branch's upstream gradient
    float* gpart;                       // [BH][nsplit][D + 4]: dW_g, db_g partials
    // MFMA kernels (lr_bwd_on_mfma): per-token rank vectors as bf16 hi + lo pairs, [BH][L][R] each:
    // y1 = dpq (query side) or dpk (key side), y2 = fq g / n (query side)
    uint16_t *y1h, *y1l, *y2h, *y2l;
};

// The low-rank backward runs on MFMA for bf16 layers with D = 128 and rank
// 8, 16, 32 or 64 (8 and 16 padded to 32 with zero weights), rotary or
// absolute-PE features, any feature map: both sides with the per-head gate;
// with the token gate only the key side (the gate changes only the query
// side's upstream gradient), the query side taking the VALU kernel. fp32
// layers and D = 64 take the VALU kernels on both sides.
inline bool lr_bwd_key_on_mfma(int dtype_bf16, long D, int R) {
    return dtype_bf16 && D == 128 && (R == 8 || R == 16 || R == 32 || R == 64);
}
inline bool lr_bwd_on_mfma(int dtype_bf16, long D, int R, bool key_side, bool token) {
    return lr_bwd_key_on_mfma(dtype_bf16, D, R) && (key_side || !token);
}

// The streaming dQ (dK/dV) kernel forms the low-rank part itself when its
// side of the low-rank backward runs on MFMA (whose kernels then store only
// the rank vectors, not the [B,H,L,D] fp32 parts).
inline bool lr_fused_in_sparse(bool tiled, int dtype_bf16, long D, int R, bool key_side, bool token) {
    return tiled && lr_bwd_on_mfma(dtype_bf16, D, R, key_side, token);
}

hipError_t launch_bwd_lr(int dtype_bf16, int D, int R, bool key_side, const LrBwdArgs& a, long BH, hipStream_t st);
// Operand blocks of the streaming kernels' low-rank products (bf16, D = 128, rank padded to 32
// or 64: kBwdLrOpBytes(rv) bytes per matrix): n heads' W [D][rv] (ds false; lo unused) or n
// slices' dS^T from the reduced [rv*D + rv] records (ds: hi and lo parts); grid n.
constexpr size_t kBwdLrOpBytes(int rv) { return (rv <= 32 ? 512ul : 1024ul) * 16; }
hipError_t launch_bwd_lr_opblocks(bool ds, int rv, const float* src, long n, uint16_t* hi, uint16_t* lo,
                                  hipStream_t st);
// out[o][e] = sum over (b < nb, split < nsplit) of part[((b*H + h)*nsplit + split)*stride + off + e]:
// per_head sums the batches into [H][n], else [BH][n] (nb = 1, h = slice).
hipError_t launch_bwd_sum_parts(const float* part, int B, int H, int nsplit, long stride, long off, long n,
                                bool per_head, float* out, hipStream_t st);
// Absolute PE: part[bh][c][r] = sum over the tokens l of slice bh with coordinate c on `axis`
// (0 = t, 1 = h, 2 = w) of dpre[bh][l][r]; grid (axis length, BH).
hipError_t launch_bwd_e_sum(const float* dpre, long BH, long L, int T, int Hg, int Wg, int axis, int R, float* part,
                            hipStream_t st);
// Inverse of the kept-block lists, deterministic: bits [BH][nblk][ceil(nblk/32)] scratch.
hipError_t launch_bwd_inverse(const int32_t* idx, long BH, int nblk, int keep, uint32_t* bits, int32_t* cnt,
                              int32_t* off, int32_t* list, int32_t* order, hipStream_t st);
// [K | V] operand-order tiles of every key block for the streaming dQ kernel, from the
// zero-padded rotated k copy kr [BH][nblk*64][128] and v [BH][L][128] (bf16); grid (nblk, BH).
hipError_t launch_bwd_dq_tiles(const uint16_t* kr, const uint16_t* v, long BH, long L, int nblk, uint16_t* tiles,
                               hipStream_t st);
hipError_t launch_bwd_dq(int dtype_bf16, int D, int BS, const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dkdv(int dtype_bf16, int D, int BS, const BwdArgs& a, hipStream_t st);

}  // namespace slr
