/*
 * slr.h -- C ABI of the MI355X (gfx950) 3D-RoPE sparse + low-rank hybrid
 * attention forward library (libslr.so).
 *
 * The layer (RoLA, arXiv 2609.06712v3, App. A Algorithm 1 and Fig. 2;
 * RoPeSLR, arXiv 2605.20659, abstract) combines
 *   - a block-sparse softmax branch: 3D RoPE of q and k, block mean-pool,
 *     per-query-block top-k key blocks, exact softmax over the kept blocks;
 *   - a head-wise rank-r linear-attention branch: phi(x W) with phi = elu+1
 *     (or SiLU, RoLA §5.3, read out as a mean over the tokens),
 *     and either the backbone's rotary schedule truncated to r dims applied
 *     after phi (RoLA §4.2-4.3) or learnable per-axis absolute embeddings
 *     added before phi (RoPeSLR abstract), read out through one reusable
 *     per-head summary S = sum rho(phi(k)) v^T, z = sum phi(k);
 *   - an additive gated combine: per head,  O = O_sparse + g_h * O_lowrank,
 *     or per token (RoLA §4.4 "Feature Alignment and Gated Fusion"),
 *     O = O_sparse + sigmoid(q . W_g + b_g) * RMS(O_sparse) / (RMS(O_lowrank)
 *     + eps) * O_lowrank, with q the token's raw query row and the RMS taken
 *     over the head dims.
 *
 * Conventions shared by every entry point
 *   Tensors q, k, v, out are [B, H, L, D] contiguous, L = T*Hg*Wg tokens
 *   flattened t-major, then h, then w. Element type is fp32 (SLR_F32) or
 *   bf16 stored as raw 16-bit patterns (SLR_BF16). Every pointer argument
 *   is a DEVICE pointer (including weights, gate and tables), 16-byte
 *   aligned, owned by the caller; the library never allocates, frees or
 *   retains memory and keeps no state between calls. Scratch comes from the
 *   caller's workspace (size from slr_workspace_bytes, 256-byte aligned).
 *   All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *   stream) with no host synchronisation; SLR_OK means "enqueued". Calls
 *   that share a workspace must be ordered on one stream.
 *   Every argument is checked on the host before anything is launched; a
 *   failed check returns a negative status and touches no memory. A HIP
 *   launch failure returns SLR_EHIP. Nothing throws across the ABI.
 *
 * Readings of points the pages leave open (fixed here, documented with the
 * design notes): rotary pairs are adjacent dims (2i, 2i+1) in contiguous
 * t | h | w chunks; pair j of an axis with n pairs turns by
 * p * base^(-2j/(2n)) at integer coordinate p; block scores are
 * mean(rotated q) . mean(rotated k) / sqrt(D) over valid tokens; ties go to
 * the lower block index; kept indices are stored ascending; the softmax
 * scale is 1/sqrt(D); the normaliser is phi(q W_q) . z + eps with the
 * un-rotated features.
 */
#ifndef SLR_H
#define SLR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SLR_OK 0
#define SLR_EINVAL (-1)        /* bad shape, config, pointer or alignment */
#define SLR_EUNSUPPORTED (-2)  /* valid but not built (e.g. D not 64/128) */
#define SLR_EWORKSPACE (-3)    /* workspace missing or too small          */
#define SLR_EHIP (-4)          /* a HIP call or kernel launch failed      */
#define SLR_ESCRATCH (-5)      /* needs more than the fixed scratch of a
                                  *_noalloc entry point                   */

/* element types */
#define SLR_F32 0
#define SLR_BF16 1

/* low-rank branch variants */
#define SLR_LR_ROPE_OUTSIDE 0  /* RoLA: truncated rotary schedule after phi      */
#define SLR_LR_ABS_PE 1        /* RoPeSLR: E_t[t]+E_h[h]+E_w[w] added before phi */

/* Feature map of the low-rank branch (slr_lowrank_cfg.feature_map) */
#define SLR_FMAP_ELU1 0        /* phi = elu + 1; readout / (w . z + eps)            */
#define SLR_FMAP_SILU 1        /* RoLA §5.3 / Table 6: phi = SiLU (sign-indefinite);
                                  readout / L, the mean over the valid tokens        */
#define SLR_FMAP_FAVOR 2       /* RoPeSLR appendix: positive random features (FAVOR+)
                                  of the exponential kernel, feature c of p = x W [+ E]:
                                  exp(omega_c . p - |p|^2 / 2) / sqrt(r), omega from
                                  slr_lowrank_cfg.omega; readout / (w . z + eps) */

/* Gate of the combine (slr_lowrank_cfg.gate_mode) */
#define SLR_GATE_HEAD 0        /* one scalar g_h per head: gate[H]                 */
#define SLR_GATE_TOKEN 1       /* RoLA §4.4: per token, from Wg[H, D] and bg[H]    */

/* operations, for slr_workspace_bytes */
#define SLR_OP_ROPE3D 0
#define SLR_OP_SELECT 1
#define SLR_OP_LOWRANK_SUMMARY 2
#define SLR_OP_ATTENTION 3
#define SLR_OP_DENSE 4
#define SLR_OP_ATTENTION_BWD 5

typedef struct {
    int32_t B, H, D;       /* batch, heads, head dim (64 or 128)      */
    int32_t T, Hg, Wg;     /* token grid; L = T*Hg*Wg                 */
    int32_t dtype;         /* SLR_F32 or SLR_BF16                     */
} slr_shape;

typedef struct {
    double base;                         /* rotary base, > 1           */
    int32_t pairs_t, pairs_h, pairs_w;   /* sum = D/2, each >= 0        */
} slr_rope_cfg;

typedef struct {
    int32_t block;   /* tokens per block: 32 or 64; nblk = ceil(L/block) */
    int32_t keep;    /* kept key blocks per query block, 1..nblk         */
} slr_sparse_cfg;

typedef struct {
    int32_t rank;                /* r: 8, 16, 32 or 64                              */
    int32_t mode;                /* SLR_LR_ROPE_OUTSIDE or SLR_LR_ABS_PE            */
    int32_t lr_pairs_t, lr_pairs_h, lr_pairs_w; /* ROPE_OUTSIDE: sum = r/2, each
                                    <= the backbone pairs of its axis; ignored for ABS_PE */
    float eps;                   /* normaliser epsilon (> 0), e.g. 1e-6             */
    const float *Wq, *Wk;        /* [H, D, r] fp32; bf16 layers use them rounded to bf16 */
    const float *gate;           /* [H] fp32, the per-head gate g_h (SLR_GATE_HEAD)   */
    const float *Et, *Eh, *Ew;   /* ABS_PE only: [T, r], [Hg, r], [Wg, r] fp32; else NULL */
    int32_t gate_mode;           /* SLR_GATE_HEAD or SLR_GATE_TOKEN                 */
    const float *Wg;             /* SLR_GATE_TOKEN: [H, D] fp32 gate weights, else NULL */
    const float *bg;             /* SLR_GATE_TOKEN: [H] fp32 gate biases, else NULL */
    int32_t feature_map;         /* SLR_FMAP_ELU1, SLR_FMAP_SILU or SLR_FMAP_FAVOR   */
    const float *omega;          /* SLR_FMAP_FAVOR: [H, r, r] fp32 random directions, row c
                                    = omega_c of the head (the caller draws them, e.g. from
                                    N(0, I_r)); else NULL                              */
} slr_lowrank_cfg;

/*
 * Workspace size in bytes for operation `op` (SLR_OP_*) at this shape.
 * `sparse` may be NULL for SLR_OP_ROPE3D / SLR_OP_LOWRANK_SUMMARY /
 * SLR_OP_DENSE; `lowrank` may be NULL unless op is SLR_OP_ATTENTION or
 * SLR_OP_LOWRANK_SUMMARY. Pure host arithmetic: no HIP call.
 */
int slr_workspace_bytes(int op, const slr_shape *shape, const slr_rope_cfg *rope,
                        const slr_sparse_cfg *sparse, const slr_lowrank_cfg *lowrank,
                        size_t *bytes);

/*
 * 3D RoPE (RoLA §3 "3D RoPE", eq. 1): x_rot = R(t,h,w) x for every token.
 * x, x_rot: [B,H,L,D] of shape->dtype (x_rot may not alias x). Rotation in
 * fp32 with fp32 cos/sin tables built from fp64 values.
 */
int slr_rope3d(const slr_shape *shape, const slr_rope_cfg *rope, const void *x, void *x_rot,
               void *ws, size_t ws_bytes, void *stream);

/*
 * Block selection of the sparse branch (RoLA Fig. 2, the top-k spike blocks of the sparse branch;
 * §4.1): rotate q and k, mean-pool each block over its valid tokens (from
 * the fp32 rotated values), score s_ij = qbar_i . kbar_j / sqrt(D) in fp32
 * and keep the `keep` largest per query block (ties: lower index).
 * idx: int32 [B,H,nblk,keep], ascending per row.
 * q_rot, k_rot: optional [B,H,L,D] outputs of the rotated q, k (NULL to skip).
 */
int slr_select_blocks(const slr_shape *shape, const slr_rope_cfg *rope, const slr_sparse_cfg *sparse,
                      const void *q, const void *k, int32_t *idx, void *q_rot, void *k_rot,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * The low-rank branch's reusable per-head summary (RoLA §4.1, App. B.1):
 *   S = sum_l f_l v_l^T  [B,H,r,D] fp32,   z = sum_l u_l  [B,H,r] fp32,
 * u_l = phi(k_l W_k [+ E]) from the raw (un-rotated) k, f_l = rho_l(u_l)
 * (ROPE_OUTSIDE) or u_l (ABS_PE); sums over the L valid tokens, reduced in
 * a fixed order (bitwise reproducible).
 */
int slr_lowrank_summary(const slr_shape *shape, const slr_rope_cfg *rope, const slr_lowrank_cfg *lowrank,
                        const void *k, const void *v, float *S, float *z,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * slr_lowrank_summary for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same sums with no workspace argument. Its scratch (rotary
 * tables, projection copies, split-L partial sums) is a fixed per-GPU buffer
 * of SLR_NOALLOC_SCRATCH_BYTES inside the library, held by every GPU the
 * library runs on until the process ends; the call allocates nothing (no
 * hipMalloc, no library allocation). When the partial sums would not fit,
 * fewer splits are used (S and z then differ from slr_lowrank_summary's only
 * by rounding order); a shape whose scratch exceeds the buffer even with one
 * split per slice returns SLR_ESCRATCH before anything is launched. Every call
 * on one GPU shares that buffer: calls that overlap on one GPU (different
 * streams, or host threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe. The first call on a device
 * looks up the buffer's device address (hipGetSymbolAddress).
 */
#define SLR_NOALLOC_SCRATCH_BYTES (32u << 20)
int slr_lowrank_summary_noalloc(const slr_shape *shape, const slr_rope_cfg *rope, const slr_lowrank_cfg *lowrank,
                                const void *k, const void *v, float *S, float *z, void *stream);

/*
 * The whole hybrid layer forward (RoLA App. A, Algorithm 1):
 *   out = O_sparse + g_h * (rho(w)^T S) / (w . z + eps),  w = phi(q W_q [+ E]).
 * out: [B,H,L,D] of shape->dtype. Optional outputs (NULL to skip):
 *   idx_out [B,H,nblk,keep] int32 (the selection used),
 *   o_sparse_out, o_lowrank_out [B,H,L,D] of shape->dtype (the two branches
 *   before the combine; for tests and diagnostics).
 */
int slr_attention_fwd(const slr_shape *shape, const slr_rope_cfg *rope, const slr_sparse_cfg *sparse,
                      const slr_lowrank_cfg *lowrank, const void *q, const void *k, const void *v,
                      void *out, int32_t *idx_out, void *o_sparse_out, void *o_lowrank_out,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * slr_attention_fwd, plus timing marks: events[0..4] are hipEvent_t handles
 * created by the caller; they are recorded on `stream` before the first
 * launch, after the rotate + pool step, after the block selection, after the
 * low-rank summary (projection prep, split-L partials, reduce) and after the
 * fused sparse flash + readout + combine kernel. Same results, same errors.
 */
int slr_attention_fwd_staged(const slr_shape *shape, const slr_rope_cfg *rope, const slr_sparse_cfg *sparse,
                             const slr_lowrank_cfg *lowrank, const void *q, const void *k, const void *v,
                             void *out, int32_t *idx_out, void *o_sparse_out, void *o_lowrank_out,
                             void *ws, size_t ws_bytes, void *const events[5], void *stream);

/*
 * slr_attention_fwd for a training step: also saves what slr_attention_bwd
 * needs. idx_out, o_sparse_out (as in slr_attention_fwd) and lse_out are
 * required: lse_out [B,H,L] fp32 receives, per query row, log2 of the
 * softmax normaliser over its kept keys, sum_j 2^(s_j) with s_j the row's
 * scores in log2 units (q.k / sqrt(D) * log2(e)). S_out [B,H,r,D] and
 * z_out [B,H,r] fp32 (optional: both or neither, 4-byte aligned, else
 * SLR_EINVAL) receive the low-rank summary the layer used (RoLA App. A
 * Algorithm 1: S = sum over tokens of rho(phi(k W_k)) v^T, z = sum of
 * phi(k W_k)), so that slr_attention_bwd need not recompute it. Same results
 * otherwise.
 */
int slr_attention_fwd_train(const slr_shape *shape, const slr_rope_cfg *rope, const slr_sparse_cfg *sparse,
                            const slr_lowrank_cfg *lowrank, const void *q, const void *k, const void *v, void *out,
                            int32_t *idx_out, void *o_sparse_out, float *lse_out, float *S_out, float *z_out,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Dense softmax attention with 3D RoPE applied inside (RoLA §3 "Full
 * attention"; the baseline the sparse branch is measured against):
 *   out = softmax(R q (R k)^T / sqrt(D)) v  over all L keys.
 */
int slr_dense_attention_fwd(const slr_shape *shape, const slr_rope_cfg *rope, const void *q,
                            const void *k, const void *v, void *out,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Backward pass of the layer (gradients of slr_attention_fwd's output; the
 * pages fine-tune this layer, RoLA §4.4 and App. E.2). Given dout = dL/dout:
 *   sparse branch (RoLA §4.1): per query row, P = softmax over the kept keys
 *     of (R q).(R k) / sqrt(D), dP = dout V^T, dS = P (dP - dout . O_sparse);
 *     dq += R^T (dS K_rot) / sqrt(D), dk += R^T (dS^T Q_rot) / sqrt(D),
 *     dv += P^T dout, with R^T the transpose of the 3D RoPE;
 *   low-rank branch (RoLA §4.1-4.3, App. A; RoPeSLR abstract): the chain
 *     rule through phi(x W [+ E]), the rotation after phi (rotary variant),
 *     S, z and the normaliser, with dO_lowrank = g_h dout;
 *   dgate[h] = sum over b and rows of dout . O_lowrank (per-head gate);
 *   with the token gate (RoLA §4.4; out = O_sparse + G O_lowrank, G =
 *     sigmoid(q . W_g + b_g) RMS(O_sparse) / (RMS(O_lowrank) + eps)) the
 *     gradient also flows through both RMS terms and the gate's logit:
 *     dWg [H,D] and dbg [H] fp32 (sums over batch and rows) replace dgate.
 * The selection is held fixed: idx [B,H,nblk,keep] int32 is the forward's
 * (idx_out of slr_attention_fwd_train); each row must list distinct blocks
 * in [0, nblk): entries outside that range are skipped, and a row that
 * lists a block twice gives undefined gradients (the forward's selection
 * never does). o_sparse [B,H,L,D] and lse [B,H,L] fp32 are that call's
 * o_sparse_out and lse_out (the softmax normalisers are reused, not
 * recomputed), for the same q, k, v and configuration. S [B,H,r,D] and z
 * [B,H,r] fp32 are that call's S_out, z_out (optional: both or neither;
 * with neither, the summary is recomputed from k and v; the workspace size
 * does not depend on the choice). dout, dq, dk, dv:
 * [B,H,L,D] of shape->dtype (bf16 or fp32, like q, k, v); the byte ranges
 * of dq, dk and dv may not overlap each other or those of q, k, v,
 * o_sparse, dout (SLR_EINVAL). dWq, dWk: [H,D,r]
 * fp32, all overwritten (sums over the batch); dgate [H] fp32 for
 * SLR_GATE_HEAD (dWg, dbg ignored, may be NULL), dWg [H,D] and dbg [H]
 * fp32 for SLR_GATE_TOKEN (dgate ignored, may be NULL).
 * SLR_LR_ABS_PE layers also get the tables' gradients dEt [T,r], dEh [Hg,r],
 * dEw [Wg,r] fp32 (overwritten; sums over batch, heads and tokens; required,
 * 4-byte aligned); for SLR_LR_ROPE_OUTSIDE they are ignored (may be NULL).
 * Every setting of the forward is covered: either gate, either low-rank
 * variant, bf16 or fp32, and each feature map (elu + 1, SiLU, FAVOR+; the
 * FAVOR+ gradient takes the features' full Jacobian, du_c/dp =
 * u_c (omega_c - p), with omega held fixed). Workspace:
 * slr_workspace_bytes(SLR_OP_ATTENTION_BWD, ...). Results are bitwise
 * reproducible (fixed reduction orders, no floating-point atomics).
 */
int slr_attention_bwd(const slr_shape *shape, const slr_rope_cfg *rope, const slr_sparse_cfg *sparse,
                      const slr_lowrank_cfg *lowrank, const void *q, const void *k, const void *v,
                      const int32_t *idx, const void *o_sparse, const float *lse, const float *S, const float *z,
                      const void *dout, void *dq, void *dk, void *dv, float *dWq, float *dWk, float *dgate,
                      float *dWg, float *dbg, float *dEt, float *dEh, float *dEw, void *ws, size_t ws_bytes,
                      void *stream);

/* Static text for a status code. */
const char *slr_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SLR_H */
