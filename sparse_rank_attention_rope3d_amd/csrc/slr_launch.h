// Host-side launch wrappers of the libslr kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "slr_common.h"

namespace slr {

struct LrGeom {
    RopeGeom rope;
    int lp[3];
    int R;
    int fmap;   // feature map: 0 = elu + 1 (readout / (w . z + eps)), 1 = SiLU (readout / L)
};

// Everything the fused sparse/dense flash kernel reads.
struct FlashArgs {
    const void* qr;          // [BH][nblk*BS][D] rotated q, zero rows past L
    const void* kr;          // same layout, rotated k
    const uint16_t* kvt;     // tiled K / V^T (bf16, D = 128, 64-token blocks)
    const void* v;           // [BH][L][D]
    const int32_t* idx;      // [BH][nblk][keep] (sparse only)
    const void* q;           // raw q [BH][L][D] (low-rank readout)
    const uint16_t* wqt;     // bf16 layers: W_q^T [H][RP][D]
    const float* wq;         // fp32 layers: W_q [H][D][R]
    const uint16_t* st_hi;   // bf16 layers: S^T hi/lo [BH][D][RP], r in slot16 order
    const uint16_t* st_lo;
    const float* S;          // fp32 layers: S [BH][R][D]
    const float* zp;         // [BH][RP] (bf16 layers) or [BH][R] (fp32 layers)
    const float* gate;       // [H] per-head gate (gate_mode 0)
    int gate_mode;           // 0: per-head gate; 1: per-token gate from wg, bg
    const float* wg;         // [H, D] token-gate weights
    const float* bg;         // [H] token-gate biases
    const float *Et, *Eh, *Ew;
    const float2* tab;
    LrGeom g;
    void* out;               // [BH][L][D]
    void* o_sp;              // optional debug outputs, same layout
    void* o_lr;
    float* lse;              // optional [BH][L]: log2 of each row's softmax normaliser over its
                             // scores in log2 units (training forward)
    long L;
    int H, nblk, keep;
    float scale;             // 1/sqrt(D)
    float eps;
    long nwg;                // workgroups in the grid
};

hipError_t launch_rope_tables(float2* tab, const RopeGeom& g, double base, hipStream_t st);
hipError_t launch_rope_pool(int dtype_bf16, int D, const void* q, const void* k, void* qo, void* ko, float* qbar,
                            float* kbar, const float2* tab, const RopeGeom& g, long BH, long L, long out_rows,
                            int bs, int nblk, hipStream_t st, float qscale = 1.f);
// Tiled K / V^T layout of the block-sparse flash kernel (bf16, D = 128, 64-token blocks).
constexpr int kTileElems = 2 * 64 * 128;
// qscale multiplies the rotated q copy (the flash kernel's scores then come
// out in log2 units), not the block means.
hipError_t launch_rope_pool_tiled(const void* q, const void* k, const void* v, void* qo, uint16_t* kv_tiles,
                                  float* qbar, float* kbar, const float2* tab, const RopeGeom& g, long BH, long L,
                                  int nblk, float qscale, hipStream_t st);
size_t select_scores_bytes(long BH, int nblk);
hipError_t launch_select(int D, const float* qbar, const float* kbar, float* scores, int32_t* idx, long BH, int nblk,
                         int keep, hipStream_t st);
hipError_t launch_lr_prep(const float* W, uint16_t* Wt, int H, int D, int R, int RP, hipStream_t st);
// Workgroups of the summary kernel chosen for these arguments that the
// current device holds at once (CUs x resident workgroups per CU; cached).
hipError_t lr_summary_slots(int dtype_bf16, int D, int RP, bool abspe, bool tiled, int* slots);

// kvt: when non-null (bf16, D = 128, 64-token blocks), V operands come from the [K | V^T] tiles
hipError_t launch_lr_summary(int dtype_bf16, int D, int RP, bool abspe, const void* k, const void* v,
                             const uint16_t* kvt, int nblk, const float* W, const uint16_t* wkt, const float* Et,
                             const float* Eh, const float* Ew, const float2* tab, const LrGeom& g, long BH, long L,
                             int H, int chunk, int nsplit, float* part, hipStream_t st);
hipError_t launch_lr_reduce(const float* part, long BH, int nsplit, int D, int R, int RP, float* S, float* z,
                            uint16_t* st_hi, uint16_t* st_lo, float* zp, hipStream_t st);
// lr_mode: 0 = no low-rank term (plain attention), 1 = rotary after phi, 2 = absolute PE
hipError_t launch_flash(int dtype_bf16, int D, int BS, int RP, int lr_mode, bool dense, const FlashArgs& a,
                        long BH, hipStream_t st);

// ---- backward pass (bf16 layers) -----------------------------------------

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
    const float* lse_in;       // [BH][L] the forward's log2 normalisers
    float* lse2;               // [BH][nblk*BS] the same, zero on padded rows
    float qmul;                // score (log2 units) = qmul * (q_rot . k_rot): log2(e)/sqrt(D), or 1
                               // when q_rot already carries that factor
    float kscale;              // dk_rot = kscale * sum dS q_rot: 1/sqrt(D), or ln 2 for scaled q
    float* delta;              // [BH][nblk*BS] dO . O_sparse per row
    const float* dq_lr;        // [BH][L][D] low-rank parts of the gradients (fp32)
    const float* dk_lr;
    const float* dv_lr;
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
    float *dq_lr, *dk_lr, *dv_lr;       // [BH][L][D]
    float* part;                        // split partials
};

hipError_t launch_bwd_lr(int D, int R, bool key_side, const LrBwdArgs& a, long BH, hipStream_t st);
// out[o][e] = sum over (b < nb, split < nsplit) of part[((b*H + h)*nsplit + split)*stride + off + e]:
// per_head sums the batches into [H][n], else [BH][n] (nb = 1, h = slice).
hipError_t launch_bwd_sum_parts(const float* part, int B, int H, int nsplit, long stride, long off, long n,
                                bool per_head, float* out, hipStream_t st);
// Inverse of the kept-block lists, deterministic: bits [BH][nblk][ceil(nblk/32)] scratch.
hipError_t launch_bwd_inverse(const int32_t* idx, long BH, int nblk, int keep, uint32_t* bits, int32_t* cnt,
                              int32_t* off, int32_t* list, hipStream_t st);
hipError_t launch_bwd_dq(int D, int BS, const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dkdv(int D, int BS, const BwdArgs& a, hipStream_t st);

}  // namespace slr
