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
    int fmap;   // feature map: 0 = elu + 1 (readout / (w . z + eps)), 1 = SiLU (readout / L),
                // 2 = FAVOR+ positive random features exp(omega p - |p|^2 / 2) / sqrt(R), p = x W [+ E]
                // (readout / (w . z + eps))
    const float* omega;   // FAVOR+: [H][R][R] random directions (row c = omega_c)
    const float* eo;      // FAVOR+ with absolute PE: [H][T + Hg + Wg][R], the axis tables times omega^T
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
    const uint16_t* wqot_hi;   // FAVOR+, bf16 layers: (W_q omega^T)^T [H][RP][D] as bf16 hi + lo parts
    const uint16_t* wqot_lo;
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
// FAVOR+: (W omega^T)^T [H][RP][D] as bf16 hi + lo parts (W rounded to bf16 first when round_bf16), and, when
// Et is non-null, eo [H][T + Hg + Wg][R] = the concatenated axis tables times omega^T
hipError_t launch_lr_prep_favor(const float* W, const float* omega, int round_bf16, int H, int D, int R, int RP,
                                uint16_t* wot_hi, uint16_t* wot_lo, const float* Et, const float* Eh, const float* Ew,
                                int T, int Hg, int Wg, float* eo, hipStream_t st);
// Whether the summary runs its prefetching instance for these arguments
// (bf16, D = 128, tiled V^T, rotary variant, rank <= 32, elu + 1 or SiLU features,
// rotation table fits its LDS copy).
bool lr_summary_prefetch(int dtype_bf16, int D, bool abspe, bool tiled, const LrGeom& g);
// Workgroups of the summary kernel chosen for these arguments that the
// current device holds at once (CUs x resident workgroups per CU; cached).
hipError_t lr_summary_slots(int dtype_bf16, int D, int RP, bool abspe, bool tiled, int* slots, bool favor = false,
                            bool pf = false);

// kvt: when non-null (bf16, D = 128, 64-token blocks), V operands come from the [K | V^T] tiles
// wkot_hi / wkot_lo: FAVOR+ on bf16 layers, (W_k omega^T)^T from launch_lr_prep_favor (else null)
hipError_t launch_lr_summary(int dtype_bf16, int D, int RP, bool abspe, const void* k, const void* v,
                             const uint16_t* kvt, int nblk, const float* W, const uint16_t* wkt, const float* Et,
                             const float* Eh, const float* Ew, const float2* tab, const LrGeom& g, long BH, long L,
                             int H, int chunk, int nsplit, float* part, hipStream_t st,
                             const uint16_t* wkot_hi = nullptr, const uint16_t* wkot_lo = nullptr);
hipError_t launch_lr_reduce(const float* part, long BH, int nsplit, int D, int R, int RP, float* S, float* z,
                            uint16_t* st_hi, uint16_t* st_lo, float* zp, hipStream_t st);
// lr_mode: 0 = no low-rank term (plain attention), 1 = rotary after phi, 2 = absolute PE
hipError_t launch_flash(int dtype_bf16, int D, int BS, int RP, int lr_mode, bool dense, const FlashArgs& a,
                        long BH, hipStream_t st);

}  // namespace slr
