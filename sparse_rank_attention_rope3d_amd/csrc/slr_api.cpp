// libslr C ABI: argument checks, workspace layout and the launch sequence.
//
// Every check runs on the host before the first HIP call, so a rejected call
// has no side effect. Launch order of the layer forward (one stream):
//   rope tables -> (bf16) projection prep -> rotate + pool q, k -> block
//   top-k -> low-rank split-L summary -> fixed-order reduce -> fused
//   sparse flash + low-rank readout + gated combine.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/slr.h"
#include "slr_launch.h"
#include "slr_backward.h"

using namespace slr;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
// The tiled path stores q already multiplied by 1/sqrt(D) * log2(e): the
// flash kernel's scores then come out of the MFMAs in log2 units.
float tiled_qscale(long D) { return (float)(1.4426950408889634 / std::sqrt((double)D)); }

struct Dims {
    long B, H, BH, D, L;
    int T, Hg, Wg, bf16, es;
};

int check_shape(const slr_shape* s, Dims* d) {
    if (!s) return SLR_EINVAL;
    if (s->B < 1 || s->H < 1 || s->T < 1 || s->Hg < 1 || s->Wg < 1) return SLR_EINVAL;
    if (s->dtype != SLR_F32 && s->dtype != SLR_BF16) return SLR_EINVAL;
    if (s->D < 2 || (s->D & 1)) return SLR_EINVAL;
    if (s->D != 64 && s->D != 128) return SLR_EUNSUPPORTED;
    const long L = (long)s->T * s->Hg * s->Wg;
    if (L > 0x7fffffffL || (long)s->Hg * s->Wg > 0x7fffffffL) return SLR_EUNSUPPORTED;
    const long BH = (long)s->B * s->H;
    if (BH > 65535) return SLR_EUNSUPPORTED;
    d->B = s->B; d->H = s->H; d->BH = BH; d->D = s->D; d->L = L;
    d->T = s->T; d->Hg = s->Hg; d->Wg = s->Wg;
    d->bf16 = s->dtype == SLR_BF16;
    d->es = d->bf16 ? 2 : 4;
    return SLR_OK;
}

int check_rope(const slr_rope_cfg* r, const Dims& d, RopeGeom* g) {
    if (!r) return SLR_EINVAL;
    if (!std::isfinite(r->base) || !(r->base > 1.0)) return SLR_EINVAL;
    if (r->pairs_t < 0 || r->pairs_h < 0 || r->pairs_w < 0) return SLR_EINVAL;
    if ((long)r->pairs_t + r->pairs_h + r->pairs_w != d.D / 2) return SLR_EINVAL;
    g->T = d.T; g->Hg = d.Hg; g->Wg = d.Wg;
    g->np[0] = r->pairs_t; g->np[1] = r->pairs_h; g->np[2] = r->pairs_w;
    g->tab_off[0] = 0;
    g->tab_off[1] = d.T * r->pairs_t;
    g->tab_off[2] = g->tab_off[1] + d.Hg * r->pairs_h;
    return SLR_OK;
}

long rope_tab_entries(const RopeGeom& g) { return (long)g.T * g.np[0] + (long)g.Hg * g.np[1] + (long)g.Wg * g.np[2]; }

int check_sparse(const slr_sparse_cfg* sp, const Dims& d, int* nblk) {
    if (!sp) return SLR_EINVAL;
    if (sp->block != 32 && sp->block != 64) return SLR_EINVAL;
    const long nb = (d.L + sp->block - 1) / sp->block;
    if (sp->keep < 1 || sp->keep > nb) return SLR_EINVAL;
    if (nb > 16383 || d.BH * nb > 0x7fffffffL) return SLR_EUNSUPPORTED;
    *nblk = (int)nb;
    return SLR_OK;
}

int check_lowrank(const slr_lowrank_cfg* lr, const slr_rope_cfg* rope, const Dims& d, bool need_q, LrGeom* lg,
                  int* RP) {
    if (!lr) return SLR_EINVAL;
    if (lr->rank != 8 && lr->rank != 16 && lr->rank != 32 && lr->rank != 64) return SLR_EINVAL;
    if (lr->mode != SLR_LR_ROPE_OUTSIDE && lr->mode != SLR_LR_ABS_PE) return SLR_EINVAL;
    if (!std::isfinite(lr->eps) || !(lr->eps > 0.f)) return SLR_EINVAL;
    if (!lr->Wk || !aligned(lr->Wk, 4)) return SLR_EINVAL;
    if (need_q) {
        if (!lr->Wq || !aligned(lr->Wq, 4)) return SLR_EINVAL;
        if (lr->gate_mode == SLR_GATE_HEAD) {
            if (!lr->gate || !aligned(lr->gate, 4)) return SLR_EINVAL;
        } else if (lr->gate_mode == SLR_GATE_TOKEN) {
            if (!lr->Wg || !aligned(lr->Wg, 16) || !lr->bg || !aligned(lr->bg, 4)) return SLR_EINVAL;
        } else {
            return SLR_EINVAL;
        }
    }
    if (lr->feature_map != SLR_FMAP_ELU1 && lr->feature_map != SLR_FMAP_SILU && lr->feature_map != SLR_FMAP_FAVOR)
        return SLR_EINVAL;
    if (lr->feature_map == SLR_FMAP_FAVOR && (!lr->omega || !aligned(lr->omega, 4))) return SLR_EINVAL;
    lg->fmap = lr->feature_map;
    lg->omega = lr->feature_map == SLR_FMAP_FAVOR ? lr->omega : nullptr;
    lg->eo = nullptr;
    lg->lp[0] = lg->lp[1] = lg->lp[2] = 0;
    if (lr->mode == SLR_LR_ROPE_OUTSIDE) {
        if (lr->lr_pairs_t < 0 || lr->lr_pairs_h < 0 || lr->lr_pairs_w < 0) return SLR_EINVAL;
        if (lr->lr_pairs_t + lr->lr_pairs_h + lr->lr_pairs_w != lr->rank / 2) return SLR_EINVAL;
        if (lr->lr_pairs_t > rope->pairs_t || lr->lr_pairs_h > rope->pairs_h || lr->lr_pairs_w > rope->pairs_w)
            return SLR_EINVAL;
        lg->lp[0] = lr->lr_pairs_t; lg->lp[1] = lr->lr_pairs_h; lg->lp[2] = lr->lr_pairs_w;
    } else {
        if (!lr->Et || !lr->Eh || !lr->Ew) return SLR_EINVAL;
        if (!aligned(lr->Et, 4) || !aligned(lr->Eh, 4) || !aligned(lr->Ew, 4)) return SLR_EINVAL;
    }
    lg->R = lr->rank;
    *RP = lr->rank <= 32 ? 32 : 64;
    (void)d;
    return SLR_OK;
}

bool tensor_ok(const void* p) { return p && aligned(p, 16); }

// Split-L partition of the summary: each of the BH slices is cut into nsplit
// chunks of a multiple of 128 tokens, one workgroup per chunk. At most
// max(1, 2048 / BH) splits (this bounds the partial-sum workspace).
int summary_split_cap(const Dims& d) {
    long cap = 2048 / d.BH;
    const long most = (d.L + 127) / 128;
    if (cap > most) cap = most;
    return cap < 1 ? 1 : (int)cap;
}

// The split that minimises the modelled time when `slots` workgroups run at
// once: rounds of workgroups x (128-token steps per workgroup + a fixed
// per-workgroup cost of about three steps); ties go to fewer splits.
// slots = 0 gives the cap. max_split (> 0) lowers the cap.
void summary_split(const Dims& d, int slots, int* chunk, int* nsplit, int max_split = 0) {
    int cap = summary_split_cap(d);
    if (max_split > 0 && max_split < cap) cap = max_split;
    long best_cost = -1, best_c = 0, best_n = 0;
    for (int n = 1; n <= cap; ++n) {
        const long c = ((d.L + n - 1) / n + 127) / 128 * 128;
        const long ne = (d.L + c - 1) / c;
        if (ne != n) continue;
        const long rounds = slots > 0 ? (d.BH * ne + slots - 1) / slots : 1;
        const long cost = rounds * (c / 128 + 3);
        if (slots <= 0 || best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best_c = c;
            best_n = ne;
        }
    }
    *chunk = (int)best_c;
    *nsplit = (int)best_n;
}

// Whether the byte ranges [a, a + n) and [b, b + n) share a byte.
bool overlaps(const void* a, const void* b, size_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + n && y < x + n;
}

// Workspace layout (byte offsets, each 256-byte aligned).
struct Layout {
    size_t tab, qr, kr, kvt, qbar, kbar, scores, idx, wqt, wkt, part, S, z, sthi, stlo, zp, total;
    // FAVOR+ (bf16 layers): (W omega^T)^T hi/lo parts of both sides, the projected axis tables
    size_t wqo_hi, wqo_lo, wko_hi, wko_lo, eo;
    size_t opwq, opwk, opsh, opsl;   // backward: operand blocks of the fused low-rank products
    // backward
    size_t lse, delta, dqlr, dklr, dvlr, lrpart, dsz, bits, cnt, off, list, order, dpre, epart, dosp, gpart, dqt, qtt;
    size_t lry;   // MFMA low-rank backward: 4 bf16 [BH][L][R] per-token rank vectors
    bool tiled;
};

// bf16, D = 128, 64-token blocks: K and V^T go to contiguous per-block tiles
// that the streaming flash kernel copies straight into LDS.
bool use_tiles(const Dims& d, int bs) { return d.bf16 && d.D == 128 && bs == 64; }

// Split-L partition of the low-rank backward: about 1024 workgroups over the
// BH slices, chunks of a multiple of 32 tokens.
void lr_bwd_split(const Dims& d, int* chunk, int* nsplit) {
    const long tiles = (d.L + 31) / 32;
    long n = 1024 / d.BH;
    if (n < 1) n = 1;
    if (n > tiles) n = tiles;
    const long c = ((d.L + n - 1) / n + 31) / 32 * 32;
    *chunk = (int)c;
    *nsplit = (int)((d.L + c - 1) / c);
}

Layout layout(int op, const Dims& d, const RopeGeom& g, int bs, int nblk, int keep, int R, int RP,
              bool abspe = false, bool token = false, bool favor = false, int max_split = 0) {
    Layout w;
    std::memset(&w, 0, sizeof(w));
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    w.tab = take(sizeof(float2) * (size_t)rope_tab_entries(g));
    if (op == SLR_OP_SELECT || op == SLR_OP_ATTENTION) {
        w.qbar = take(4ul * d.BH * nblk * d.D);
        w.kbar = take(4ul * d.BH * nblk * d.D);
        w.scores = take(select_scores_bytes(d.BH, nblk));
        w.idx = take(4ul * d.BH * nblk * keep);
    }
    w.tiled = false;
    if (op == SLR_OP_ATTENTION_BWD) {
        // rotated q, k (rows padded to whole blocks), the summary (recomputed when
        // the caller does not pass the forward's),
        // per-row softmax statistics, the low-rank gradient parts and the
        // inverse of the kept lists
        const size_t rows = (size_t)nblk * bs;
        w.qr = take((size_t)d.es * d.BH * rows * d.D);
        w.kr = take((size_t)d.es * d.BH * rows * d.D);
        w.wkt = take(2ul * d.H * RP * d.D);
        if (favor && d.bf16) {
            // FAVOR+: the summary's (W_k omega^T) parts and, for absolute PE, the projected axis tables
            w.wko_hi = take(2ul * d.H * RP * d.D);
            w.wko_lo = take(2ul * d.H * RP * d.D);
            if (abspe) w.eo = take(4ul * d.H * ((long)d.T + d.Hg + d.Wg) * R);
        }
        w.part = take(4ul * d.BH * summary_split_cap(d) * (RP * d.D + RP));
        w.S = take(4ul * d.BH * R * d.D);
        w.z = take(4ul * d.BH * R);
        w.lse = take(4ul * d.BH * rows);
        w.delta = take(4ul * d.BH * rows);
        // fp32 low-rank gradient parts, unless the streaming sparse kernels form them
        if (!lr_fused_in_sparse(use_tiles(d, bs), d.bf16, d.D, R, false, token)) w.dqlr = take(4ul * d.BH * d.L * d.D);
        if (!lr_fused_in_sparse(use_tiles(d, bs), d.bf16, d.D, R, true, token)) {
            w.dklr = take(4ul * d.BH * d.L * d.D);
            w.dvlr = take(4ul * d.BH * d.L * d.D);
        }
        if (lr_fused_in_sparse(use_tiles(d, bs), d.bf16, d.D, R, true, token)) {
            // operand blocks of the fused products: W_q, W_k per head; dS^T hi, lo per slice
            w.opwq = take(kBwdLrOpBytes(R) * d.H);
            w.opwk = take(kBwdLrOpBytes(R) * d.H);
            w.opsh = take(kBwdLrOpBytes(R) * d.BH);
            w.opsl = take(kBwdLrOpBytes(R) * d.BH);
        }
        int chunk, nsplit;
        lr_bwd_split(d, &chunk, &nsplit);
        w.lrpart = take(4ul * d.BH * nsplit * (2ul * d.D * R + R + 4));
        if (lr_bwd_key_on_mfma(d.bf16, d.D, R)) w.lry = take(8ul * d.BH * d.L * R);
        w.dsz = take(4ul * d.BH * ((size_t)R * d.D + R));
        if (abspe) {
            // per-token gradient of x W + E and the per-slice axis sums of it
            w.dpre = take(4ul * d.BH * d.L * R);
            const int na = d.T > d.Hg ? (d.T > d.Wg ? d.T : d.Wg) : (d.Hg > d.Wg ? d.Hg : d.Wg);
            w.epart = take(4ul * d.BH * na * R);
        }
        if (token) {
            // the sparse branch's upstream gradient and the gate parameters' partials
            w.dosp = take((size_t)d.es * d.BH * d.L * d.D);
            w.gpart = take(4ul * d.BH * nsplit * (d.D + 4));
        }
        w.bits = take(4ul * d.BH * nblk * ((nblk + 31) / 32));
        w.cnt = take(4ul * d.BH * nblk);
        w.off = take(4ul * d.BH * (nblk + 1));
        w.list = take(4ul * d.BH * nblk * keep);
        w.order = take(4ul * d.BH * nblk);
        if (use_tiles(d, bs)) {
            w.dqt = take(d.BH * nblk * kBwdDqTileBytes);
            w.qtt = take(d.BH * nblk * kBwdQtTileBytes);
        }
        w.total = off;
        return w;
    }
    if (op == SLR_OP_ATTENTION || op == SLR_OP_DENSE) {
        const size_t rows = (size_t)nblk * bs;
        w.qr = take((size_t)d.es * d.BH * rows * d.D);
        if (use_tiles(d, bs)) {
            w.tiled = true;
            w.kvt = take(2ul * d.BH * nblk * kTileElems);
        } else {
            w.kr = take((size_t)d.es * d.BH * rows * d.D);
        }
    }
    if (op == SLR_OP_ATTENTION || op == SLR_OP_LOWRANK_SUMMARY) {
        int nsplit = summary_split_cap(d);
        if (max_split > 0 && max_split < nsplit) nsplit = max_split;
        if (d.bf16) {
            w.wqt = take(2ul * d.H * RP * d.D);
            w.wkt = take(2ul * d.H * RP * d.D);
            if (favor) {
                w.wqo_hi = take(2ul * d.H * RP * d.D);
                w.wqo_lo = take(2ul * d.H * RP * d.D);
                w.wko_hi = take(2ul * d.H * RP * d.D);
                w.wko_lo = take(2ul * d.H * RP * d.D);
                if (abspe) w.eo = take(4ul * d.H * ((long)d.T + d.Hg + d.Wg) * R);
            }
        }
        w.part = take(4ul * d.BH * nsplit * (RP * d.D + RP));
        w.S = take(4ul * d.BH * R * d.D);
        w.z = take(4ul * d.BH * R);
        if (d.bf16) {
            w.sthi = take(2ul * d.BH * d.D * RP);
            w.stlo = take(2ul * d.BH * d.D * RP);
            w.zp = take(4ul * d.BH * RP);
        }
    }
    w.total = off;
    return w;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return SLR_OK;
    if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return SLR_EWORKSPACE;
    return SLR_OK;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

#define SLR_TRY(expr)                                  \
    do {                                               \
        if ((expr) != hipSuccess) return SLR_EHIP;     \
    } while (0)

// The fixed scratch of slr_lowrank_summary_noalloc: one copy per GPU, held
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the address hipGetSymbolAddress returns for
// the current device (kept per device below), never the name.
constexpr size_t kScratchBytes = (size_t)SLR_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// Device address of this GPU's scratch, looked up once per device (with that
// device current) on the first call there.
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SLR_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return SLR_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SLR_EHIP;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return SLR_OK;
}

}  // namespace

extern "C" {

const char* slr_status_string(int status) {
    switch (status) {
        case SLR_OK: return "SLR_OK: success";
        case SLR_EINVAL: return "SLR_EINVAL: invalid shape, configuration, pointer or alignment";
        case SLR_EUNSUPPORTED: return "SLR_EUNSUPPORTED: valid arguments outside the built kernel set";
        case SLR_EWORKSPACE: return "SLR_EWORKSPACE: workspace missing, misaligned or too small";
        case SLR_EHIP: return "SLR_EHIP: a HIP runtime call or kernel launch failed";
        case SLR_ESCRATCH: return "SLR_ESCRATCH: the call needs more than the library's fixed scratch buffer";
        default: return "unknown slr status";
    }
}

int slr_workspace_bytes(int op, const slr_shape* shape, const slr_rope_cfg* rope, const slr_sparse_cfg* sparse,
                        const slr_lowrank_cfg* lowrank, size_t* bytes) {
    if (!bytes) return SLR_EINVAL;
    Dims d;
    RopeGeom g;
    int st = check_shape(shape, &d);
    if (st) return st;
    if ((st = check_rope(rope, d, &g))) return st;
    int nblk = 0, keep = 0, bs = 64, R = 0, RP = 32;
    switch (op) {
        case SLR_OP_ROPE3D:
        case SLR_OP_DENSE:
            nblk = (int)((d.L + bs - 1) / bs);
            break;
        case SLR_OP_SELECT:
        case SLR_OP_ATTENTION:
        case SLR_OP_ATTENTION_BWD:
            if ((st = check_sparse(sparse, d, &nblk))) return st;
            bs = sparse->block;
            keep = sparse->keep;
            break;
        case SLR_OP_LOWRANK_SUMMARY:
            break;
        default:
            return SLR_EINVAL;
    }
    if (op == SLR_OP_ATTENTION || op == SLR_OP_LOWRANK_SUMMARY || op == SLR_OP_ATTENTION_BWD) {
        if (!lowrank) return SLR_EINVAL;
        LrGeom lg;
        // pointer fields are not needed for sizing
        slr_lowrank_cfg probe = *lowrank;
        float dummy[4] __attribute__((aligned(16)));
        probe.Wq = probe.Wk = probe.gate = dummy;
        probe.Et = probe.Eh = probe.Ew = dummy;
        probe.Wg = probe.bg = dummy;
        probe.omega = dummy;
        if ((st = check_lowrank(&probe, rope, d, op != SLR_OP_LOWRANK_SUMMARY, &lg, &RP))) return st;
        R = lowrank->rank;
    }
    *bytes = layout(op, d, g, bs, nblk, keep, R, RP, lowrank && lowrank->mode == SLR_LR_ABS_PE,
                    lowrank && lowrank->gate_mode == SLR_GATE_TOKEN,
                    lowrank && lowrank->feature_map == SLR_FMAP_FAVOR).total;
    return SLR_OK;
}

int slr_rope3d(const slr_shape* shape, const slr_rope_cfg* rope, const void* x, void* x_rot, void* ws,
               size_t ws_bytes, void* stream) {
    Dims d;
    RopeGeom g;
    int st = check_shape(shape, &d);
    if (st) return st;
    if ((st = check_rope(rope, d, &g))) return st;
    if (!tensor_ok(x) || !tensor_ok(x_rot) || x == x_rot) return SLR_EINVAL;
    const int bs = 64;
    const int nblk = (int)((d.L + bs - 1) / bs);
    Layout w = layout(SLR_OP_ROPE3D, d, g, bs, nblk, 0, 0, 32);
    if ((st = check_ws(ws, ws_bytes, w.total))) return st;
    hipStream_t s = (hipStream_t)stream;
    float2* tab = at<float2>(ws, w.tab);
    SLR_TRY(launch_rope_tables(tab, g, rope->base, s));
    SLR_TRY(launch_rope_pool(d.bf16, (int)d.D, x, nullptr, x_rot, nullptr, nullptr, nullptr, tab, g, d.BH, d.L, d.L,
                             bs, nblk, s));
    return SLR_OK;
}

int slr_select_blocks(const slr_shape* shape, const slr_rope_cfg* rope, const slr_sparse_cfg* sparse, const void* q,
                      const void* k, int32_t* idx, void* q_rot, void* k_rot, void* ws, size_t ws_bytes,
                      void* stream) {
    Dims d;
    RopeGeom g;
    int nblk;
    int st = check_shape(shape, &d);
    if (st) return st;
    if ((st = check_rope(rope, d, &g))) return st;
    if ((st = check_sparse(sparse, d, &nblk))) return st;
    if (!tensor_ok(q) || !tensor_ok(k) || !idx || !aligned(idx, 4)) return SLR_EINVAL;
    if ((q_rot && !tensor_ok(q_rot)) || (k_rot && !tensor_ok(k_rot))) return SLR_EINVAL;
    Layout w = layout(SLR_OP_SELECT, d, g, sparse->block, nblk, sparse->keep, 0, 32);
    if ((st = check_ws(ws, ws_bytes, w.total))) return st;
    hipStream_t s = (hipStream_t)stream;
    float2* tab = at<float2>(ws, w.tab);
    float* qbar = at<float>(ws, w.qbar);
    float* kbar = at<float>(ws, w.kbar);
    SLR_TRY(launch_rope_tables(tab, g, rope->base, s));
    SLR_TRY(launch_rope_pool(d.bf16, (int)d.D, q, k, q_rot, k_rot, qbar, kbar, tab, g, d.BH, d.L, d.L, sparse->block,
                             nblk, s));
    SLR_TRY(launch_select((int)d.D, qbar, kbar, at<float>(ws, w.scores), idx, d.BH, nblk, sparse->keep, s));
    return SLR_OK;
}

namespace {

// Shared by the summary entry point and the layer forward.
// FAVOR+ on bf16 layers: the projected axis tables of the absolute-PE
// variant (shared by both sides), placed in the geometry the kernels get.
static int favor_tables(const Dims& d, LrGeom* lg, const slr_lowrank_cfg* lr, void* ws, const Layout& w, hipStream_t s) {
    if (lr->feature_map != SLR_FMAP_FAVOR || !d.bf16 || lr->mode != SLR_LR_ABS_PE) return SLR_OK;
    float* eo = at<float>(ws, w.eo);
    SLR_TRY(launch_lr_prep_favor(nullptr, lr->omega, 1, (int)d.H, (int)d.D, lg->R, 0, nullptr, nullptr, lr->Et,
                                 lr->Eh, lr->Ew, d.T, d.Hg, d.Wg, eo, s));
    lg->eo = eo;
    return SLR_OK;
}

static int run_summary(const Dims& d, const RopeGeom& g, const LrGeom& lg, int RP, const slr_lowrank_cfg* lr, const void* k,
                const void* v, const uint16_t* kvt, int nblk, void* ws, const Layout& w, float* S, float* z,
                bool want_st, hipStream_t s, int max_split = 0) {
    const bool abspe = lr->mode == SLR_LR_ABS_PE;
    const bool favor = lr->feature_map == SLR_FMAP_FAVOR;
    int slots = 0, chunk, nsplit;
    SLR_TRY(lr_summary_slots(d.bf16, (int)d.D, RP, abspe, kvt != nullptr, &slots, favor,
                             lr_summary_prefetch(d.bf16, (int)d.D, abspe, kvt != nullptr, lg)));
    summary_split(d, slots, &chunk, &nsplit, max_split);
    const float2* tab = at<float2>(ws, w.tab);
    uint16_t* wkt = d.bf16 ? at<uint16_t>(ws, w.wkt) : nullptr;
    if (d.bf16) SLR_TRY(launch_lr_prep(lr->Wk, wkt, (int)d.H, (int)d.D, lg.R, RP, s));
    uint16_t *woh = nullptr, *wol = nullptr;
    if (favor && d.bf16) {
        woh = at<uint16_t>(ws, w.wko_hi);
        wol = at<uint16_t>(ws, w.wko_lo);
        SLR_TRY(launch_lr_prep_favor(lr->Wk, lr->omega, 1, (int)d.H, (int)d.D, lg.R, RP, woh, wol, nullptr, nullptr,
                                     nullptr, d.T, d.Hg, d.Wg, nullptr, s));
    }
    float* part = at<float>(ws, w.part);
    SLR_TRY(launch_lr_summary(d.bf16, (int)d.D, RP, abspe, k, v, kvt, nblk, lr->Wk, wkt, lr->Et, lr->Eh, lr->Ew, tab,
                              lg, d.BH, d.L, (int)d.H, chunk, nsplit, part, s, woh, wol));
    uint16_t* sthi = want_st ? at<uint16_t>(ws, w.sthi) : nullptr;
    uint16_t* stlo = want_st ? at<uint16_t>(ws, w.stlo) : nullptr;
    float* zp = want_st ? at<float>(ws, w.zp) : nullptr;
    SLR_TRY(launch_lr_reduce(part, d.BH, nsplit, (int)d.D, lg.R, RP, S, z, sthi, stlo, zp, s));
    (void)g;
    return SLR_OK;
}

}  // namespace

int slr_lowrank_summary(const slr_shape* shape, const slr_rope_cfg* rope, const slr_lowrank_cfg* lowrank,
                        const void* k, const void* v, float* S, float* z, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    RopeGeom g;
    LrGeom lg;
    int RP;
    int st = check_shape(shape, &d);
    if (st) return st;
    if ((st = check_rope(rope, d, &g))) return st;
    if ((st = check_lowrank(lowrank, rope, d, false, &lg, &RP))) return st;
    if (!tensor_ok(k) || !tensor_ok(v) || !S || !z || !aligned(S, 4) || !aligned(z, 4)) return SLR_EINVAL;
    lg.rope = g;
    Layout w = layout(SLR_OP_LOWRANK_SUMMARY, d, g, 64, 0, 0, lowrank->rank, RP, lowrank->mode == SLR_LR_ABS_PE,
                      false, lowrank->feature_map == SLR_FMAP_FAVOR);
    if ((st = check_ws(ws, ws_bytes, w.total))) return st;
    hipStream_t s = (hipStream_t)stream;
    SLR_TRY(launch_rope_tables(at<float2>(ws, w.tab), g, rope->base, s));
    if ((st = favor_tables(d, &lg, lowrank, ws, w, s))) return st;
    return run_summary(d, g, lg, RP, lowrank, k, v, nullptr, 0, ws, w, S, z, false, s);
}

int slr_lowrank_summary_noalloc(const slr_shape* shape, const slr_rope_cfg* rope, const slr_lowrank_cfg* lowrank,
                                const void* k, const void* v, float* S, float* z, void* stream) {
    Dims d;
    RopeGeom g;
    LrGeom lg;
    int RP;
    int st = check_shape(shape, &d);
    if (st) return st;
    if ((st = check_rope(rope, d, &g))) return st;
    if ((st = check_lowrank(lowrank, rope, d, false, &lg, &RP))) return st;
    if (!tensor_ok(k) || !tensor_ok(v) || !S || !z || !aligned(S, 4) || !aligned(z, 4)) return SLR_EINVAL;
    lg.rope = g;
    // the most splits whose partial sums fit the fixed scratch (fewer splits:
    // the same sums in a coarser fixed order)
    const bool abspe = lowrank->mode == SLR_LR_ABS_PE, favor = lowrank->feature_map == SLR_FMAP_FAVOR;
    int max_split = summary_split_cap(d);
    Layout w = layout(SLR_OP_LOWRANK_SUMMARY, d, g, 64, 0, 0, lowrank->rank, RP, abspe, false, favor, max_split);
    while (w.total > kScratchBytes && max_split > 1) {
        --max_split;
        w = layout(SLR_OP_LOWRANK_SUMMARY, d, g, 64, 0, 0, lowrank->rank, RP, abspe, false, favor, max_split);
    }
    if (w.total > kScratchBytes) return SLR_ESCRATCH;
    void* ws = nullptr;
    if ((st = scratch_address(&ws))) return st;
    hipStream_t s = (hipStream_t)stream;
    SLR_TRY(launch_rope_tables(at<float2>(ws, w.tab), g, rope->base, s));
    if ((st = favor_tables(d, &lg, lowrank, ws, w, s))) return st;
    return run_summary(d, g, lg, RP, lowrank, k, v, nullptr, 0, ws, w, S, z, false, s, max_split);
}

namespace {

static int attention_fwd(const slr_shape* shape, const slr_rope_cfg* rope, const slr_sparse_cfg* sparse,
                  const slr_lowrank_cfg* lowrank, const void* q, const void* k, const void* v, void* out,
                  int32_t* idx_out, void* o_sparse_out, void* o_lowrank_out, float* lse_out, float* S_out,
                  float* z_out, void* ws, size_t ws_bytes, void* const* events, void* stream) {
    Dims d;
    RopeGeom g;
    LrGeom lg;
    int nblk, RP;
    int st = check_shape(shape, &d);
    if (st) return st;
    if ((st = check_rope(rope, d, &g))) return st;
    if ((st = check_sparse(sparse, d, &nblk))) return st;
    if ((st = check_lowrank(lowrank, rope, d, true, &lg, &RP))) return st;
    if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out)) return SLR_EINVAL;
    if (idx_out && !aligned(idx_out, 4)) return SLR_EINVAL;
    if ((o_sparse_out && !tensor_ok(o_sparse_out)) || (o_lowrank_out && !tensor_ok(o_lowrank_out)))
        return SLR_EINVAL;
    if (lse_out && !aligned(lse_out, 4)) return SLR_EINVAL;
    lg.rope = g;
    const int bs = sparse->block;
    const bool favor = lowrank->feature_map == SLR_FMAP_FAVOR;
    Layout w = layout(SLR_OP_ATTENTION, d, g, bs, nblk, sparse->keep, lowrank->rank, RP,
                      lowrank->mode == SLR_LR_ABS_PE, false, favor);
    if ((st = check_ws(ws, ws_bytes, w.total))) return st;
    hipStream_t s = (hipStream_t)stream;

    float2* tab = at<float2>(ws, w.tab);
    void* qr = at<void>(ws, w.qr);
    void* kr = w.tiled ? nullptr : at<void>(ws, w.kr);
    uint16_t* kvt = w.tiled ? at<uint16_t>(ws, w.kvt) : nullptr;
    float* qbar = at<float>(ws, w.qbar);
    float* kbar = at<float>(ws, w.kbar);
    int32_t* idx = idx_out ? idx_out : at<int32_t>(ws, w.idx);
    // the summary goes to the caller's S_out, z_out when given (training forward)
    float* S = S_out ? S_out : at<float>(ws, w.S);
    float* z = z_out ? z_out : at<float>(ws, w.z);

    auto mark = [&](int i) { return events ? hipEventRecord((hipEvent_t)events[i], s) : hipSuccess; };
    SLR_TRY(mark(0));
    SLR_TRY(launch_rope_tables(tab, g, rope->base, s));
    if (w.tiled)
        SLR_TRY(launch_rope_pool_tiled(q, k, v, qr, kvt, qbar, kbar, tab, g, d.BH, d.L, nblk, tiled_qscale(d.D), s));
    else
        SLR_TRY(launch_rope_pool(d.bf16, (int)d.D, q, k, qr, kr, qbar, kbar, tab, g, d.BH, d.L, (long)nblk * bs, bs,
                                 nblk, s));
    SLR_TRY(mark(1));
    SLR_TRY(launch_select((int)d.D, qbar, kbar, at<float>(ws, w.scores), idx, d.BH, nblk, sparse->keep, s));
    SLR_TRY(mark(2));
    if ((st = favor_tables(d, &lg, lowrank, ws, w, s))) return st;
    if ((st = run_summary(d, g, lg, RP, lowrank, k, v, kvt, nblk, ws, w, S, z, d.bf16 != 0, s))) return st;
    uint16_t* wqt = nullptr;
    uint16_t *wqoh = nullptr, *wqol = nullptr;
    if (d.bf16) {
        wqt = at<uint16_t>(ws, w.wqt);
        SLR_TRY(launch_lr_prep(lowrank->Wq, wqt, (int)d.H, (int)d.D, lg.R, RP, s));
        if (favor) {
            wqoh = at<uint16_t>(ws, w.wqo_hi);
            wqol = at<uint16_t>(ws, w.wqo_lo);
            SLR_TRY(launch_lr_prep_favor(lowrank->Wq, lowrank->omega, 1, (int)d.H, (int)d.D, lg.R, RP, wqoh, wqol,
                                         nullptr, nullptr, nullptr, d.T, d.Hg, d.Wg, nullptr, s));
        }
    }
    SLR_TRY(mark(3));

    FlashArgs a;
    std::memset(&a, 0, sizeof(a));
    a.qr = qr; a.kr = kr; a.kvt = kvt; a.v = v; a.idx = idx; a.q = q;
    a.wqt = wqt; a.wq = lowrank->Wq;
    a.st_hi = d.bf16 ? at<uint16_t>(ws, w.sthi) : nullptr;
    a.st_lo = d.bf16 ? at<uint16_t>(ws, w.stlo) : nullptr;
    a.S = S;
    a.zp = d.bf16 ? at<float>(ws, w.zp) : z;
    a.gate = lowrank->gate;
    a.gate_mode = lowrank->gate_mode;
    a.wg = lowrank->Wg;
    a.bg = lowrank->bg;
    a.Et = lowrank->Et; a.Eh = lowrank->Eh; a.Ew = lowrank->Ew;
    a.wqot_hi = wqoh; a.wqot_lo = wqol;
    a.tab = tab;
    a.g = lg;
    a.out = out; a.o_sp = o_sparse_out; a.o_lr = o_lowrank_out; a.lse = lse_out;
    a.L = d.L; a.H = (int)d.H; a.nblk = nblk; a.keep = sparse->keep;
    a.scale = (float)(1.0 / std::sqrt((double)d.D));
    a.eps = lowrank->eps;
    a.nwg = d.BH * nblk;
    const int lr_mode = lowrank->mode == SLR_LR_ABS_PE ? 2 : 1;
    SLR_TRY(launch_flash(d.bf16, (int)d.D, bs, RP, lr_mode, false, a, d.BH, s));
    SLR_TRY(mark(4));
    return SLR_OK;
}

}  // namespace

int slr_attention_fwd(const slr_shape* shape, const slr_rope_cfg* rope, const slr_sparse_cfg* sparse,
                      const slr_lowrank_cfg* lowrank, const void* q, const void* k, const void* v, void* out,
                      int32_t* idx_out, void* o_sparse_out, void* o_lowrank_out, void* ws, size_t ws_bytes,
                      void* stream) {
    return attention_fwd(shape, rope, sparse, lowrank, q, k, v, out, idx_out, o_sparse_out, o_lowrank_out, nullptr,
                         nullptr, nullptr, ws, ws_bytes, nullptr, stream);
}

int slr_attention_fwd_train(const slr_shape* shape, const slr_rope_cfg* rope, const slr_sparse_cfg* sparse,
                            const slr_lowrank_cfg* lowrank, const void* q, const void* k, const void* v, void* out,
                            int32_t* idx_out, void* o_sparse_out, float* lse_out, float* S_out, float* z_out,
                            void* ws, size_t ws_bytes, void* stream) {
    if (!idx_out || !o_sparse_out || !lse_out) return SLR_EINVAL;
    if ((S_out == nullptr) != (z_out == nullptr) || (S_out && (!aligned(S_out, 4) || !aligned(z_out, 4))))
        return SLR_EINVAL;
    return attention_fwd(shape, rope, sparse, lowrank, q, k, v, out, idx_out, o_sparse_out, nullptr, lse_out, S_out,
                         z_out, ws, ws_bytes, nullptr, stream);
}

int slr_attention_fwd_staged(const slr_shape* shape, const slr_rope_cfg* rope, const slr_sparse_cfg* sparse,
                             const slr_lowrank_cfg* lowrank, const void* q, const void* k, const void* v, void* out,
                             int32_t* idx_out, void* o_sparse_out, void* o_lowrank_out, void* ws, size_t ws_bytes,
                             void* const events[5], void* stream) {
    if (!events) return SLR_EINVAL;
    for (int i = 0; i < 5; ++i)
        if (!events[i]) return SLR_EINVAL;
    return attention_fwd(shape, rope, sparse, lowrank, q, k, v, out, idx_out, o_sparse_out, o_lowrank_out, nullptr,
                         nullptr, nullptr, ws, ws_bytes, events, stream);
}

int slr_dense_attention_fwd(const slr_shape* shape, const slr_rope_cfg* rope, const void* q, const void* k,
                            const void* v, void* out, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    RopeGeom g;
    int st = check_shape(shape, &d);
    if (st) return st;
    if ((st = check_rope(rope, d, &g))) return st;
    if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out)) return SLR_EINVAL;
    const int bs = 64;
    const long nb = (d.L + bs - 1) / bs;
    if (d.BH * nb > 0x7fffffffL) return SLR_EUNSUPPORTED;
    const int nblk = (int)nb;
    Layout w = layout(SLR_OP_DENSE, d, g, bs, nblk, 0, 0, 32);
    if ((st = check_ws(ws, ws_bytes, w.total))) return st;
    hipStream_t s = (hipStream_t)stream;
    float2* tab = at<float2>(ws, w.tab);
    void* qr = at<void>(ws, w.qr);
    void* kr = w.tiled ? nullptr : at<void>(ws, w.kr);
    uint16_t* kvt = w.tiled ? at<uint16_t>(ws, w.kvt) : nullptr;
    SLR_TRY(launch_rope_tables(tab, g, rope->base, s));
    if (w.tiled)
        SLR_TRY(launch_rope_pool_tiled(q, k, v, qr, kvt, nullptr, nullptr, tab, g, d.BH, d.L, nblk, tiled_qscale(d.D),
                                       s));
    else
        SLR_TRY(launch_rope_pool(d.bf16, (int)d.D, q, k, qr, kr, nullptr, nullptr, tab, g, d.BH, d.L, (long)nblk * bs,
                                 bs, nblk, s));
    FlashArgs a;
    std::memset(&a, 0, sizeof(a));
    a.qr = qr; a.kr = kr; a.kvt = kvt; a.v = v; a.out = out;
    a.L = d.L; a.H = (int)d.H; a.nblk = nblk; a.keep = nblk;
    a.scale = (float)(1.0 / std::sqrt((double)d.D));
    a.nwg = d.BH * nblk;
    SLR_TRY(launch_flash(d.bf16, (int)d.D, bs, 32, 0, true, a, d.BH, s));
    return SLR_OK;
}

int slr_attention_bwd(const slr_shape* shape, const slr_rope_cfg* rope, const slr_sparse_cfg* sparse,
                      const slr_lowrank_cfg* lowrank, const void* q, const void* k, const void* v, const int32_t* idx,
                      const void* o_sparse, const float* lse, const float* S_in, const float* z_in, const void* dout,
                      void* dq, void* dk, void* dv,
                      float* dWq, float* dWk, float* dgate, float* dWg, float* dbg, float* dEt, float* dEh,
                      float* dEw, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    RopeGeom g;
    LrGeom lg;
    int nblk, RP;
    int st = check_shape(shape, &d);
    if (st) return st;
    if ((st = check_rope(rope, d, &g))) return st;
    if ((st = check_sparse(sparse, d, &nblk))) return st;
    if ((st = check_lowrank(lowrank, rope, d, true, &lg, &RP))) return st;
    const bool favor = lowrank->feature_map == SLR_FMAP_FAVOR;
    if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o_sparse) || !tensor_ok(dout)) return SLR_EINVAL;
    if (!tensor_ok(dq) || !tensor_ok(dk) || !tensor_ok(dv) || !idx || !aligned(idx, 4)) return SLR_EINVAL;
    if (!lse || !aligned(lse, 4)) return SLR_EINVAL;
    if ((S_in == nullptr) != (z_in == nullptr) || (S_in && (!aligned(S_in, 4) || !aligned(z_in, 4))))
        return SLR_EINVAL;
    const bool token = lowrank->gate_mode == SLR_GATE_TOKEN;
    if (!dWq || !dWk || !aligned(dWq, 4) || !aligned(dWk, 4)) return SLR_EINVAL;
    if (!token && (!dgate || !aligned(dgate, 4))) return SLR_EINVAL;
    if (token && (!dWg || !dbg || !aligned(dWg, 4) || !aligned(dbg, 4))) return SLR_EINVAL;
    const bool abspe = lowrank->mode == SLR_LR_ABS_PE;
    if (abspe && (!dEt || !dEh || !dEw || !aligned(dEt, 4) || !aligned(dEh, 4) || !aligned(dEw, 4)))
        return SLR_EINVAL;
    {
        // dq, dk, dv ([B,H,L,D] each) may share no byte with each other or
        // with the [B,H,L,D] inputs
        const size_t nb = (size_t)d.es * d.BH * d.L * d.D;
        const void* outs[3] = {dq, dk, dv};
        const void* ins[5] = {q, k, v, o_sparse, dout};
        for (int i = 0; i < 3; ++i) {
            for (int j = 0; j < 5; ++j)
                if (overlaps(outs[i], ins[j], nb)) return SLR_EINVAL;
            for (int j = i + 1; j < 3; ++j)
                if (overlaps(outs[i], outs[j], nb)) return SLR_EINVAL;
        }
    }
    lg.rope = g;
    const int bs = sparse->block, keep = sparse->keep, R = lowrank->rank;
    Layout w = layout(SLR_OP_ATTENTION_BWD, d, g, bs, nblk, keep, R, RP, abspe, token, favor);
    if ((st = check_ws(ws, ws_bytes, w.total))) return st;
    hipStream_t s = (hipStream_t)stream;
    float2* tab = at<float2>(ws, w.tab);
    uint16_t* qr = at<uint16_t>(ws, w.qr);
    uint16_t* kr = at<uint16_t>(ws, w.kr);
    // the forward's summary when the caller saved it, else recomputed here
    const float* S = S_in ? S_in : at<float>(ws, w.S);
    const float* z = z_in ? z_in : at<float>(ws, w.z);

    // q scaled exactly as the forward scored it (pre-scaled into log2 units on
    // the tiled path), so the saved normalisers match the recomputed scores
    const bool tiled_fwd = use_tiles(d, bs);
    const float log2e = 1.4426950408889634f, inv_sqrt_d = (float)(1.0 / std::sqrt((double)d.D));
    SLR_TRY(launch_rope_tables(tab, g, rope->base, s));
    SLR_TRY(launch_rope_pool(d.bf16, (int)d.D, q, k, qr, kr, nullptr, nullptr, tab, g, d.BH, d.L, (long)nblk * bs, bs,
                             nblk, s, tiled_fwd ? tiled_qscale(d.D) : 1.f));
    if (!S_in) {
        if ((st = favor_tables(d, &lg, lowrank, ws, w, s))) return st;
        if ((st = run_summary(d, g, lg, RP, lowrank, k, v, nullptr, 0, ws, w, at<float>(ws, w.S), at<float>(ws, w.z),
                              false, s)))
            return st;
    }

    // low-rank branch: query side, reductions, key side
    LrBwdArgs la;
    std::memset(&la, 0, sizeof(la));
    la.q = (const uint16_t*)q; la.k = (const uint16_t*)k; la.v = (const uint16_t*)v; la.dout = (const uint16_t*)dout;
    la.Wq = lowrank->Wq; la.Wk = lowrank->Wk; la.S = S; la.z = z; la.gate = lowrank->gate;
    float* dsz = at<float>(ws, w.dsz);
    la.dSz = dsz;
    la.tab = tab; la.g = lg; la.eps = lowrank->eps; la.L = d.L; la.H = (int)d.H;
    lr_bwd_split(d, &la.chunk, &la.nsplit);
    // the streaming dQ (dK/dV) kernel forms the low-rank part of its rows itself when that side
    // runs on the MFMA low-rank kernels; they then store only the rank vectors
    const bool fuse_q = lr_fused_in_sparse(tiled_fwd, d.bf16, d.D, R, false, token);
    const bool fuse_k = lr_fused_in_sparse(tiled_fwd, d.bf16, d.D, R, true, token);
    la.dq_lr = fuse_q ? nullptr : at<float>(ws, w.dqlr);
    la.dk_lr = fuse_k ? nullptr : at<float>(ws, w.dklr);
    la.dv_lr = fuse_k ? nullptr : at<float>(ws, w.dvlr);
    la.part = at<float>(ws, w.lrpart);
    la.abspe = abspe ? 1 : 0;
    la.Et = lowrank->Et; la.Eh = lowrank->Eh; la.Ew = lowrank->Ew;
    la.dpre = abspe ? at<float>(ws, w.dpre) : nullptr;
    la.token = token ? 1 : 0;
    la.wg = lowrank->Wg; la.bg = lowrank->bg; la.o_sp = o_sparse;
    la.dosp = token ? at<void>(ws, w.dosp) : nullptr;
    la.gpart = token ? at<float>(ws, w.gpart) : nullptr;
    if (lr_bwd_key_on_mfma(d.bf16, d.D, R)) {
        const size_t n = (size_t)d.BH * d.L * R;
        la.y1h = at<uint16_t>(ws, w.lry);
        la.y1l = la.y1h + n;
        la.y2h = la.y1l + n;
        la.y2l = la.y2h + n;
    }
    const long qstride = 2l * d.D * R + R + 4;   // [dW_q | dS | dz | dg | pad]
    SLR_TRY(launch_bwd_lr(d.bf16, (int)d.D, R, false, la, d.BH, s));
    // [dW_q | dS | dz | dg] partials -> dS, dz per slice; dW_q, dg per head
    SLR_TRY(launch_bwd_sum_parts(la.part, (int)d.B, (int)d.H, la.nsplit, qstride, d.D * R, (long)R * d.D + R, false,
                                 dsz, s));
    SLR_TRY(launch_bwd_sum_parts(la.part, (int)d.B, (int)d.H, la.nsplit, qstride, 0, d.D * R, true, dWq, s));
    if (!token) {
        SLR_TRY(launch_bwd_sum_parts(la.part, (int)d.B, (int)d.H, la.nsplit, qstride, 2l * d.D * R + R, 1, true, dgate,
                                     s));
    } else {
        // token gate: dW_g [H][D] and db_g [H] from the [dW_g | db_g | pad] partials
        SLR_TRY(launch_bwd_sum_parts(la.gpart, (int)d.B, (int)d.H, la.nsplit, d.D + 4, 0, d.D, true, dWg, s));
        SLR_TRY(launch_bwd_sum_parts(la.gpart, (int)d.B, (int)d.H, la.nsplit, d.D + 4, d.D, 1, true, dbg, s));
    }
    // sparse branch, dQ first (and the row statistics): with fuse_q it forms W_q dpq from the
    // query side's rank vectors, which the key side's overwrite next
    BwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.qr = qr; a.kr = kr; a.v = (const uint16_t*)v; a.o_sp = (const uint16_t*)o_sparse;
    // with the token gate the sparse branch's upstream gradient is dout plus the RMS term
    a.dout = (const uint16_t*)(token ? la.dosp : dout); a.idx = idx;
    a.inv_off = at<int32_t>(ws, w.off); a.inv_list = at<int32_t>(ws, w.list);
    a.lse_in = lse; a.lse2 = at<float>(ws, w.lse); a.delta = at<float>(ws, w.delta);
    a.qmul = tiled_fwd ? 1.f : log2e * inv_sqrt_d;
    a.kscale = tiled_fwd ? 0.6931471805599453f : inv_sqrt_d;
    a.dq_lr = la.dq_lr; a.dk_lr = la.dk_lr; a.dv_lr = la.dv_lr;
    a.dq = (uint16_t*)dq; a.dk = (uint16_t*)dk; a.dv = (uint16_t*)dv;
    a.tab = tab; a.g = g; a.L = d.L; a.nblk = nblk; a.keep = keep;
    a.scale = (float)(1.0 / std::sqrt((double)d.D));
    a.nwg = d.BH * nblk;
    a.lr_rv = R; a.H = (int)d.H;
    if (fuse_q) {
        a.lr_ph = la.y1h; a.lr_pl = la.y1l;
        uint16_t* opw = at<uint16_t>(ws, w.opwq);
        SLR_TRY(launch_bwd_lr_opblocks(false, R, lowrank->Wq, d.H, opw, nullptr, s));
        a.lr_w = opw;
    }
    if (tiled_fwd) {
        uint16_t* dqt = at<uint16_t>(ws, w.dqt);
        SLR_TRY(launch_bwd_dq_tiles(kr, (const uint16_t*)v, d.BH, d.L, nblk, dqt, s));
        a.dqt = dqt;
        a.qtt = at<uint16_t>(ws, w.qtt);   // written by the dQ kernel for the dK/dV kernel
    }
    SLR_TRY(launch_bwd_dq(d.bf16, (int)d.D, bs, a, s));

    // low-rank key side (with fuse_k it stores dpk and fk for the dK/dV kernel), its sums
    SLR_TRY(launch_bwd_lr(d.bf16, (int)d.D, R, true, la, d.BH, s));
    SLR_TRY(launch_bwd_sum_parts(la.part, (int)d.B, (int)d.H, la.nsplit, d.D * R, 0, d.D * R, true, dWk, s));
    if (abspe) {
        // E tables: per-axis sums of the per-token gradient, per slice, then over the slices
        float* ep = at<float>(ws, w.epart);
        const int na[3] = {d.T, d.Hg, d.Wg};
        float* outs[3] = {dEt, dEh, dEw};
        for (int ax = 0; ax < 3; ++ax) {
            SLR_TRY(launch_bwd_e_sum(la.dpre, d.BH, d.L, d.T, d.Hg, d.Wg, ax, R, ep, s));
            SLR_TRY(launch_bwd_sum_parts(ep, (int)d.BH, 1, 1, (long)na[ax] * R, 0, (long)na[ax] * R, true, outs[ax], s));
        }
    }

    // the inverse lists, dK and dV
    a.lr_ph = a.lr_pl = a.lr_fh = a.lr_fl = a.lr_w = a.lr_sh = a.lr_sl = nullptr;
    if (fuse_k) {
        a.lr_ph = la.y1h; a.lr_pl = la.y1l; a.lr_fh = la.y2h; a.lr_fl = la.y2l;
        uint16_t* opw = at<uint16_t>(ws, w.opwk);
        uint16_t* osh = at<uint16_t>(ws, w.opsh);
        uint16_t* osl = at<uint16_t>(ws, w.opsl);
        SLR_TRY(launch_bwd_lr_opblocks(false, R, lowrank->Wk, d.H, opw, nullptr, s));
        SLR_TRY(launch_bwd_lr_opblocks(true, R, dsz, d.BH, osh, osl, s));
        a.lr_w = opw; a.lr_sh = osh; a.lr_sl = osl;
    }
    a.order = at<int32_t>(ws, w.order);
    SLR_TRY(launch_bwd_inverse(idx, d.BH, nblk, keep, at<uint32_t>(ws, w.bits), at<int32_t>(ws, w.cnt),
                               at<int32_t>(ws, w.off), at<int32_t>(ws, w.list), at<int32_t>(ws, w.order), s));
    SLR_TRY(launch_bwd_dkdv(d.bf16, (int)d.D, bs, a, s));
    return SLR_OK;
}

}  // extern "C"
