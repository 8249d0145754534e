// Persistent block-sparse (and dense) flash attention for bf16 layers with
// D = 128 and 64-token blocks, the key-range segments it streams, and the
// partial merge + gated low-rank apply.
//
// RoLA (arXiv 2609.06712v3) §4.1: every query block attends, with an exact
// softmax, to the tokens of its kept key blocks; App. F: this sparse branch is
// the dominant cost of the layer. §3 "Full attention" is the same loop over
// every key block. App. A Algorithm 1 with §4.3-§4.4: the gated low-rank
// readout is added to the sparse output (k_lr_apply).
//
// Work decomposition. A task is (query block, key range): the kept list of a
// query block (ascending) is cut at the range boundaries r * nblk / ksplit.
// Every XCD serves its own key ranges, so its L2 only ever holds the tiles of
// those ranges; a task writes its normalised partial output and the row max
// and row sum, and k_lr_apply merges the partials (exact: softmax over a
// union of disjoint key sets). With ksplit = 1 a task is a whole query block.
//
// Kernel shape. Persistent: two workgroups per CU, each of two waves (one
// wave per SIMD). Wave kh owns keys 32kh..+31 of every tile and all 64 query
// rows, so the waves share no operand and each loads its own 1 KB operand
// chunks of the operand-order [K | V^T] tile straight into registers (a tile
// enters the CU once; no LDS staging, no barrier per tile). The loop over a
// workgroup's tile stream (its tasks back to back) is software-pipelined:
// step t issues the K loads of tile t + 2, the P V MFMAs of tile t - 1 next
// to the softmax of tile t, the V^T loads of tile t + 1 and the score MFMAs
// of tile t + 1. The rotated q copy is pre-scaled by scale * log2(e) and the
// score accumulator starts at -m (the running row max), so the MFMA yields
// the exp2 argument directly; the running max is only raised when a tile's
// probabilities would pass 2^40 (checked through their sum).
#include <type_traits>

#include "slr_common.h"
#include "slr_epilogue.h"
#include "slr_launch.h"

namespace slr {

// ---- key-range segments ----------------------------------------------------
// seg[row][r] = number of kept blocks of the row below r * nblk / ksplit
// (r = 0 .. ksplit); kept lists are ascending. One wave per row.
__global__ __launch_bounds__(256) void k_segments(const int32_t* __restrict__ idx, int32_t* __restrict__ seg,
                                                  long rows, int keep, int nblk, int ksplit) {
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int32_t* ix = idx + row * keep;
    int cnt = 0;   // lane r (1 <= r < ksplit) counts the kept blocks below boundary r
    for (int c0 = 0; c0 < keep; c0 += 64) {
        const int n = c0 + lane;
        const int v = n < keep ? ix[n] : 0x7fffffff;
        for (int r = 1; r < ksplit; ++r) {
            const int bound = (int)((long)r * nblk / ksplit);
            const int m = __popcll(__ballot(v < bound));
            if (lane == r) cnt += m;
        }
    }
    int32_t* out = seg + row * (ksplit + 1);
    if (lane < ksplit) out[lane] = lane == 0 ? 0 : cnt;
    if (lane == ksplit) out[lane] = keep;
}

// ---- task list of one workgroup ----------------------------------------------
// ksplit <= 8 (a divisor of 8): XCD x serves range x % ksplit over its share
// (x / ksplit) of the query blocks; ksplit = 8p: XCD x serves ranges x, x + 8,
// ... one after the other over all query blocks. The workgroups of an XCD
// take the tasks round robin, so at any time they work on neighbouring
// query blocks of one range.
struct TaskList {
    long N;     // query blocks (BH * nblk)
    long lo;    // first query block of this XCD's share (ksplit <= 8)
    long NT;    // tasks of this XCD
    int r0;     // range (ksplit <= 8) or range of the first phase (ksplit > 8)
};

struct Cur {
    long k;      // task number in the list (>= NT: stream exhausted)
    long qidx;   // query block: bh * nblk + qb
    int r;       // key range
    int n, e;    // position and end in the kept list (dense: block index)
    bool fst;    // n is the first position of the task
};

template <bool DENSE>
__device__ __forceinline__ void cur_task(Cur& c, long k, long stride, const TaskList& tl, const FlashArgs& a) {
    const int ks = a.ksplit;
    for (; k < tl.NT; k += stride) {
        long qidx;
        int r;
        if (ks <= 8) {
            qidx = tl.lo + k;
            r = tl.r0;
        } else {
            const long p = k / tl.N;
            qidx = k - p * tl.N;
            r = (int)(8 * p) + tl.r0;
        }
        int b, e;
        if (DENSE) {
            b = (int)((long)r * a.nblk / ks);
            e = (int)((long)(r + 1) * a.nblk / ks);
        } else if (ks == 1) {
            b = 0;
            e = a.keep;
        } else {
            const int32_t* sg = a.seg + qidx * (ks + 1) + r;
            b = sg[0];
            e = sg[1];
        }
        if (b < e) {
            c.k = k; c.qidx = qidx; c.r = r; c.n = b; c.e = e; c.fst = true;
            return;
        }
    }
    c.k = tl.NT;
    c.fst = false;
}

template <bool DENSE>
__device__ __forceinline__ void cur_next(Cur& c, long stride, const TaskList& tl, const FlashArgs& a) {
    if (c.k >= tl.NT) return;
    c.fst = false;
    if (++c.n >= c.e) cur_task<DENSE>(c, c.k + stride, stride, tl, a);
}

// Eight 16-byte LDS reads (1 KB apart) into registers; the block waits for
// them itself (the compiler would otherwise wait for every copy in flight
// before any LDS read), so no read is left in flight when it ends. Outputs
// are early-clobber: a read must not land in the address register while
// later reads of the block still use it.
__device__ __forceinline__ void lds_rd8(u32x4_t* r, const void* lds_base) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
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
// Four 16-byte LDS writes / reads at 1 KB spacing (the key-half exchange),
// each completed inside the block.
__device__ __forceinline__ void lds_wr4(const void* lds_base, u32x4_t x0, u32x4_t x1, u32x4_t x2, u32x4_t x3) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
    asm volatile(
        "ds_write_b128 %0, %1\n\t"
        "ds_write_b128 %0, %2 offset:1024\n\t"
        "ds_write_b128 %0, %3 offset:2048\n\t"
        "ds_write_b128 %0, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        :
        : "v"(a), "v"(x0), "v"(x1), "v"(x2), "v"(x3)
        : "memory");
}
__device__ __forceinline__ void lds_rd4(u32x4_t* r, const void* lds_base) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a)
        : "memory");
}
__device__ __forceinline__ void lds_wr2f(const void* lds_base, float x, float y) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
    asm volatile("s_nop 1\n\tds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 :
                 : "v"(a), "v"(u32x2_t{__float_as_uint(x), __float_as_uint(y)})
                 : "memory");
}
// The hazard tracking of the compiler does not look into asm blocks: before
// an asm block reads MFMA results, wait out the MFMA result latency (19 wait
// states cover the longest MFMA). The accumulators pass through as in/out
// operands, so no read of them can move above the wait.
__device__ __forceinline__ void mfma_results_ready(f32x16_t (&o)[4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
}
__device__ __forceinline__ void lds_rd2f(const void* lds_base, float& x, float& y) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
    u32x2_t r;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(a) : "memory");
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

// Online softmax, exp2 domain, one 32-row block; a lane holds one query row
// and 16 of its keys. m_run is the row's reference (its running max up to a
// slack); -inf means "no valid key seen yet" (a task whose first tile is the
// ragged tail block can mask a whole key half). The score accumulator of a
// tile starts at -m_run (0 while there is no reference), so s holds
// scaled score - reference.

// a task's first tile: the row max becomes the reference
__device__ __forceinline__ void softmax_first(f32x16_t& s, float& m_run, float& l_run, u32x4_t* pop) {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = max_xor32(mx);
    const bool none = mx == -INFINITY;   // every key of this half masked
    float l = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p0 = none ? 0.f : fast_exp2(s[8 * h2 + 2 * i] - mx);
            const float p1 = none ? 0.f : fast_exp2(s[8 * h2 + 2 * i + 1] - mx);
            l += p0 + p1;
            pop[h2][i] = pack_bf2(p0, p1);
        }
    m_run = mx;
    l_run = l;
}

// later tiles: p = exp2(s) directly; the reference is raised only when some
// probability of the tile would exceed ~2^36 (sum > 2^40), and set from the
// tile when the row has none yet
__device__ __forceinline__ void softmax_next(f32x16_t& s, f32x16_t* o, float& m_run, float& l_run, u32x4_t* pop) {
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
        // shift of the reference: to the tile max for a row without one (may
        // stay -inf), else up to the tile max when that is higher
        const float shift = noref ? mx : fmaxf(mx, 0.f);
        const bool none = shift == -INFINITY;
        const float ref = noref ? 0.f : m_run;
        const float alpha = noref ? 0.f : fast_exp2(-shift);
        m_run = none ? -INFINITY : ref + shift;
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

// Workgroup = 4 waves = one 64-row query block of the current task; wave
// (rh, kh) owns query rows 32rh..+31 and keys 32kh..+31 of every tile. K and
// V^T parts of the tile stream (the workgroup's tasks back to back) go
// through LDS rings filled by direct global-to-LDS copies: K three parts deep
// (requested two tiles ahead), V^T two deep (one tile ahead); one barrier per
// tile. At the end of a task the key halves are merged through the ring slots
// that are free at that point: K slot of the last tile (query rows 0-31), K
// slot two tiles ahead (rows 32-63; its copy is issued one tile later) and
// the V^T slot of the last tile (row maxima and sums).
template <bool DENSE, bool DIRECT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_sparse_flash(
    FlashArgs a, const int32_t* __restrict__ idx_all, const uint16_t* __restrict__ kvt_all) {
    constexpr int D = 128, BS = 64;
    constexpr int PART = kTileElems / 2;                 // K or V^T part of a tile (elements)
    constexpr int PLOADS = PART * 2 / (256 * 16);        // 16-byte copies per thread per part (4)
    __shared__ __attribute__((aligned(16))) uint16_t lds[5 * PART];   // K ring (3) | V^T ring (2)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rh = wave & 1, kh = wave >> 1;
    const int l32 = lane & 31, hf = lane >> 5;
    const int nblk = a.nblk, keep = a.keep, ks = a.ksplit;
    const long L = a.L;
    const bool ragged = (L % BS) != 0;

    TaskList tl;
    const int x = (int)(blockIdx.x % 8);
    const long stride = gridDim.x / 8;
    const long first = blockIdx.x / 8;
    tl.N = a.nwg;
    if (ks <= 8) {
        const int G = 8 / ks, g = x / ks;
        tl.r0 = x % ks;
        tl.lo = g * tl.N / G;
        tl.NT = (g + 1) * tl.N / G - tl.lo;
    } else {
        tl.r0 = x;
        tl.lo = 0;
        tl.NT = (long)(ks / 8) * tl.N;
    }

    Cur c0, c1, c2;
    cur_task<DENSE>(c0, first, stride, tl, a);
    if (c0.k >= tl.NT) return;
    c1 = c0;
    cur_next<DENSE>(c1, stride, tl, a);
    c2 = c1;
    cur_next<DENSE>(c2, stride, tl, a);

    auto tile_of = [&](const Cur& c) -> const uint16_t* {
        const long bhn = c.qidx - c.qidx % nblk;   // first block of the slice
        const int j = DENSE ? c.n : idx_all[c.qidx * keep + c.n];
        return kvt_all + (bhn + j) * (long)kTileElems + (long)tid * 8;
    };
    // part (0 = K, 1 = V^T) of a tile -> LDS (same image as in memory)
    auto issue = [&](const uint16_t* src, int part, uint16_t* dst) {
        src += part * PART;
#pragma unroll
        for (int m = 0; m < PLOADS; ++m)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(src + m * 256 * 8),
                (__attribute__((address_space(3))) void*)(dst + (m * 256 + wave * 64) * 8), 16, 0, 0);
    };
    const int rd = ((kh * 8) * 64 + lane) * 8;   // this lane's operand chunks (kh, 0..7) within a part

    // B operands of S^T = K Q^T: query row 32rh + l32 of the task's block,
    // dims 16s + 8hf + e. The next task's operands replace them as soon as
    // the last score MFMAs of the current task have read them.
    u32x4_t qop[8];
    auto load_q = [&](u32x4_t* dst, long qidx) {
        const uint16_t* qr = (const uint16_t*)a.qr + (qidx * BS + 32 * rh + l32) * D + 8 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) dst[s] = ldg16(qr + 16 * s);
    };
    load_q(qop, c0.qidx);

    f32x16_t oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = 0.f, l_run = 0.f;

    // ring: K of stream position t in K slot t % 3, V^T in V slot t % 2
    {
        const uint16_t* p0 = tile_of(c0);
        issue(p0, 0, lds);
        issue(p0, 1, lds + 3 * PART);
    }
    bool k_ahead = c1.k < tl.NT;   // K of position t + 1 was the last copy requested
    if (k_ahead) issue(tile_of(c1), 0, lds + PART);
    bool k_pend = false;           // K of position t + 1 still to request (deferred by a task end)
    int t3 = 0, t2 = 0;            // t % 3, t % 2

    for (;;) {
        const bool v1 = c1.k < tl.NT, v2 = c2.k < tl.NT;
        const bool task_end = !v1 || c1.fst;
        if (k_ahead) wait_vmcnt<PLOADS>(); else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        const int t3n = t3 == 2 ? 0 : t3 + 1, t3nn = t3 == 0 ? 2 : t3 - 1;
        if (k_pend) issue(tile_of(c1), 0, lds + t3n * PART);   // K of t + 1 (deferred)
        if (v1) issue(tile_of(c1), 1, lds + (3 + (t2 ^ 1)) * PART);
        k_ahead = false;
        k_pend = false;
        if (v2) {
            if (task_end) k_pend = true;   // its slot carries the exchange first
            else {
                issue(tile_of(c2), 0, lds + t3nn * PART);
                k_ahead = true;
            }
        }
        const uint16_t* kcur = lds + t3 * PART;
        const uint16_t* vcur = lds + (3 + t2) * PART;

        u32x4_t op[8], vop[8];
        lds_rd8(op, kcur + rd);
        f32x16_t sacc;
        {
            const float init = (c0.fst || m_run == -INFINITY) ? 0.f : -m_run;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = init;
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 8; ++s) sacc = mfma32(op[s], qop[s], sacc);
        __builtin_amdgcn_s_setprio(0);
        if (task_end && v1) load_q(qop, c1.qidx);
        lds_rd8(vop, vcur + rd);
        asm volatile("" ::"v"(op[0]), "v"(op[1]), "v"(op[2]), "v"(op[3]), "v"(op[4]), "v"(op[5]), "v"(op[6]),
                     "v"(op[7]));
        const int jc = DENSE ? c0.n : idx_all[c0.qidx * keep + c0.n];
        if (ragged && jc == nblk - 1) {
            const long key0 = (long)jc * BS + 32 * kh;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key0 + 8 * (i >> 2) + 4 * hf + (i & 3) >= L) sacc[i] = -INFINITY;
        }
        u32x4_t pop[2];
        if (c0.fst) softmax_first(sacc, m_run, l_run, pop);
        else softmax_next(sacc, oacc, m_run, l_run, pop);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) oacc[db] = mfma32(vop[db * 2 + h2], pop[h2], oacc[db]);
        __builtin_amdgcn_s_setprio(0);

        if (task_end) {
            // ---- merge the key halves through the free slots, store the task
            // (plain barriers: the LDS accesses complete inside their asm blocks,
            // and the copies in flight go to other slots)
            __builtin_amdgcn_s_barrier();
            uint16_t* xo = lds + (rh == 0 ? t3 : t3nn) * PART;       // this row half's O exchange
            uint16_t* xml = lds + (3 + t2) * PART + rh * 512;         // its m, l exchange
            if (kh == 1) {
                mfma_results_ready(oacc);
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    u32x4_t w[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int e = 0; e < 4; ++e) w[g][e] = __float_as_uint(oacc[db][4 * g + e]);
                    lds_wr4(xo + (db * 4 * 64 + lane) * 8, w[0], w[1], w[2], w[3]);
                }
                lds_wr2f(xml + lane * 4, m_run, l_run);
            }
            __builtin_amdgcn_s_barrier();
            if (kh == 0) {
                float m1, l1;
                lds_rd2f(xml + lane * 4, m1, l1);
                const float m = fmaxf(m_run, m1);
                const float f0 = fast_exp2(m_run - m), f1 = fast_exp2(m1 - m);
                const float lrow = sum_xor32(l_run * f0 + l1 * f1);
                const float inv = 1.f / lrow;
                const float g0 = f0 * inv, g1 = f1 * inv;
                const long part = (c0.qidx * ks + c0.r) * 2 + rh;
                const long bh = c0.qidx / nblk;
                const long row = (c0.qidx - bh * nblk) * BS + 32 * rh + l32;
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    u32x4_t w[4];
                    lds_rd4(w, xo + (db * 4 * 64 + lane) * 8);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float o4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * g + e] * g0 + __uint_as_float(w[g][e]) * g1;
                        const u32x2_t pk = u32x2_t{pack_bf2(o4[0], o4[1]), pack_bf2(o4[2], o4[3])};
                        if (DIRECT) {
                            if (row < L)
                                *reinterpret_cast<u32x2_t*>((uint16_t*)a.out + (bh * L + row) * D + 32 * db + 8 * g +
                                                            4 * hf) = pk;
                        } else {
                            *reinterpret_cast<u32x2_t*>(a.part_o + part * (16 * 64 * 4) + ((db * 4 + g) * 64 + lane) * 4) =
                                pk;
                        }
                    }
                }
                if (!DIRECT) a.part_ml[part * 64 + lane] = hf ? lrow : m;
            }
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
            if (!v1) break;
        }
        // advance the stream
        c0 = c1;
        c1 = c2;
        cur_next<DENSE>(c2, stride, tl, a);
        t3 = t3n;
        t2 ^= 1;
    }
}

// ---- partial merge + low-rank readout + gated combine -------------------------
// One workgroup = one query block, wave h = query rows 32h..+31 (the lane
// layout of the partials). Partials of the ranges with kept blocks are merged
// with their row maxima and sums; the flash epilogue then adds the low-rank
// readout and the gate and writes the rows below L.
template <int RP, int LR>
__global__ __launch_bounds__(128) void k_lr_apply(FlashArgs a) {
    const int lane = threadIdx.x & 63;
    const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const long qidx = blockIdx.x;
    const int nblk = a.nblk, ks = a.ksplit;
    const long bh = qidx / nblk;
    const int qb = (int)(qidx - bh * nblk);
    const int head = (int)(bh % a.H);

    auto load_part = [&](long part, f32x16_t* o, float c, bool acc) __attribute__((always_inline)) {
        const uint16_t* po = a.part_o + part * (16 * 64 * 4) + lane * 4;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const u32x2_t w = *reinterpret_cast<const u32x2_t*>(po + (db * 4 + g4) * 256);
                const float v0 = bf_lo(w[0]), v1 = bf_hi(w[0]), v2 = bf_lo(w[1]), v3 = bf_hi(w[1]);
                if (acc) {
                    o[db][4 * g4] += c * v0;
                    o[db][4 * g4 + 1] += c * v1;
                    o[db][4 * g4 + 2] += c * v2;
                    o[db][4 * g4 + 3] += c * v3;
                } else {
                    o[db][4 * g4] = c * v0;
                    o[db][4 * g4 + 1] = c * v1;
                    o[db][4 * g4 + 2] = c * v2;
                    o[db][4 * g4 + 3] = c * v3;
                }
            }
    };
    f32x16_t oacc[4];
    float lsum;
    if (ks == 1) {
        load_part(qidx * 2 + h, oacc, 1.f, false);
        lsum = 1.f;
    } else {
        const int32_t* sg = a.seg + qidx * (ks + 1);
        float m = -INFINITY;
        for (int r = 0; r < ks; ++r)
            if (sg[r] < sg[r + 1]) m = fmaxf(m, a.part_ml[((qidx * ks + r) * 2 + h) * 64 + l32]);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
        lsum = 0.f;
        for (int r = 0; r < ks; ++r) {
            if (sg[r] >= sg[r + 1]) continue;
            const long part = (qidx * ks + r) * 2 + h;
            const float mr = a.part_ml[part * 64 + l32], lr = a.part_ml[part * 64 + 32 + l32];
            const float c = lr * fast_exp2(mr - m);
            lsum += c;
            load_part(part, oacc, c, true);
        }
    }
    flash_epilogue<128, RP, LR>(a, bh, head, (long)qb * 64 + 32 * h, lsum, oacc);
}

// ---- launchers -------------------------------------------------------------------
static int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Key ranges per query block: the tiles of one range of a slice should fit
// comfortably in one XCD's L2 (4 MB); ranges are split over the 8 XCDs.
int sparse_flash_ksplit(long BH, int nblk, int keep, bool dense) {
    (void)BH;
    (void)keep;
    if (dense) return 1;
    const long slice_bytes = (long)nblk * kTileElems * 2;
    const long target = 3l << 20;
    if (slice_bytes <= 8 * target) return 8;
    long ks = (slice_bytes + target - 1) / target;
    ks = (ks + 7) / 8 * 8;
    return ks > 32 ? 32 : (int)ks;
}

hipError_t launch_segments(const int32_t* idx, int32_t* seg, long rows, int keep, int nblk, int ksplit,
                           hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_segments, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, idx, seg, rows, keep, nblk,
                       ksplit);
    return hipGetLastError();
}

hipError_t launch_sparse_flash(const FlashArgs& a, bool dense, bool direct_out, hipStream_t st) {
    const int wgs = (2 * device_cus() + 7) / 8 * 8;
    dim3 grid((unsigned)wgs), blk(256);
    if (dense && direct_out)
        hipLaunchKernelGGL((k_sparse_flash<true, true>), grid, blk, 0, st, a, a.idx, a.kvt);
    else if (dense)
        hipLaunchKernelGGL((k_sparse_flash<true, false>), grid, blk, 0, st, a, a.idx, a.kvt);
    else
        hipLaunchKernelGGL((k_sparse_flash<false, false>), grid, blk, 0, st, a, a.idx, a.kvt);
    return hipGetLastError();
}

template <int RP>
static hipError_t lr_apply_t(int lr_mode, const FlashArgs& a, long nq, hipStream_t st) {
    dim3 grid((unsigned)nq), blk(128);
    if (lr_mode == 1) hipLaunchKernelGGL((k_lr_apply<RP, 1>), grid, blk, 0, st, a);
    else if (lr_mode == 2) hipLaunchKernelGGL((k_lr_apply<RP, 2>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_lr_apply<RP, 0>), grid, blk, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_lr_apply(int RP, int lr_mode, const FlashArgs& a, long BH, hipStream_t st) {
    const long nq = BH * a.nblk;
    return RP == 64 ? lr_apply_t<64>(lr_mode, a, nq, st) : lr_apply_t<32>(lr_mode, a, nq, st);
}

}  // namespace slr
