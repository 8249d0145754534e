// Per-query-block top-k selection of key blocks.
//
// RoLA (arXiv 2609.06712v3) Fig. 2 / §4.1: the sparse branch keeps the
// top-k key blocks of every query block. Scores are
// s_ij = qbar_i . kbar_j / sqrt(D) of the fp32 block means; the k-th largest
// is found exactly by bisection over order-preserving 32-bit keys, ties go to
// the lower block index, and the kept indices are written in ascending order.
//
// Two kernels: a tiled score GEMM per (b, h) slice and a one-wave-per-row
// top-k. The GEMM runs on bf16 MFMA with each fp32 operand split into a bf16
// hi + lo pair (three products: hi*hi + hi*lo + lo*hi, fp32 accumulation);
// the dropped lo*lo term and the residual of the split are ~2^-16 relative,
// about 1e-7 on these scores -- two orders below the near-tie window the
// selection is specified with.
#include "slr_common.h"
#include "slr_launch.h"

namespace slr {

// 8 fp32 values -> bf16 hi and lo parts (packed pairs)
__device__ __forceinline__ void split8(const float* x, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h = pack_bf2(x[2 * i], x[2 * i + 1]);
        hi[i] = h;
        lo[i] = pack_bf2(x[2 * i] - bf_lo(h), x[2 * i + 1] - bf_hi(h));
    }
}

// One workgroup (4 waves) = 32 complete rows of the score matrix of one
// slice, so its output is one contiguous stretch of memory. A = qbar rows
// (m = i, k = d), split once and kept in registers; the waves take the 32-key
// column tiles round robin, B = kbar rows (k = d, n = j) from L2. The grid is
// remapped so that all row blocks of a slice run on one XCD.
template <int D>
__global__ __launch_bounds__(256) void k_block_scores(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                      float* __restrict__ scores, int nblk, float scale, int nrb,
                                                      long nwg) {
    constexpr int NS = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const long wg = xcd_remap(blockIdx.x, nwg);
    const long bh = wg / nrb;
    const int i0 = (int)(wg % nrb) * 32;
    const float* qb = qbar + bh * (long)nblk * D;
    const float* kb = kbar + bh * (long)nblk * D;
    // rows / columns past nblk read the last one; they are never stored
    const int ia = i0 + l32 < nblk ? i0 + l32 : nblk - 1;
    u32x4_t ahi[NS], alo[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const f32x4_t* p = reinterpret_cast<const f32x4_t*>(qb + (long)ia * D + 16 * s + 8 * hf);
        const f32x4_t u = p[0], w = p[1];
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[e] = u[e]; x[4 + e] = w[e]; }
        split8(x, ahi[s], alo[s]);
    }
    const int ntile = (nblk + 31) / 32;
    float* out_rows = scores + bh * (long)nblk * nblk;
    for (int jt = wave; jt < ntile; jt += 4) {
        const int j0 = jt * 32;
        const int jb = j0 + l32 < nblk ? j0 + l32 : nblk - 1;
        f32x4_t braw[2 * NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x4_t* p = reinterpret_cast<const f32x4_t*>(kb + (long)jb * D + 16 * s + 8 * hf);
            braw[2 * s] = p[0];
            braw[2 * s + 1] = p[1];
        }
        f32x16_t acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = braw[2 * s][e]; x[4 + e] = braw[2 * s + 1][e]; }
            u32x4_t bhi, blo;
            split8(x, bhi, blo);
            acc = mfma32(ahi[s], bhi, acc);
            acc = mfma32(ahi[s], blo, acc);
            acc = mfma32(alo[s], bhi, acc);
        }
        // lane holds rows i0 + 8(v/4) + 4hf + v%4 of column j0 + l32
        if (j0 + l32 < nblk) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = i0 + 8 * (v >> 2) + 4 * hf + (v & 3);
                if (i < nblk) out_rows[(long)i * nblk + j0 + l32] = acc[v] * scale;
            }
        }
    }
}

// Top-k of one score row per wave. KPL = keys per lane held in registers
// (column j = 64 m + lane); KPL = 0 reads the row from memory on every pass.
//
// The k-th largest key is found exactly, bit by bit from the top. With keys
// in registers this runs in two phases: the upper 16 bits over all keys, then
// the lower 16 bits over only the keys that share the upper 16 bits with the
// threshold (compacted into LDS), since every other key is decided by then.
template <int KPL>
__global__ __launch_bounds__(256) void k_topk_rows(const float* __restrict__ scores, int32_t* __restrict__ idx,
                                                   long nrows, int nblk, int keep) {
    constexpr int CMAX = KPL > 0 ? 64 * KPL : 1;
    __shared__ uint32_t cand_all[4][CMAX];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long row = (long)blockIdx.x * 4 + wave;
    if (row >= nrows) return;
    const float* s = scores + row * nblk;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t key[KPL > 0 ? KPL : 1];
    if (KPL > 0) {
        // unconditional loads (columns past nblk read the last one, then get
        // key 0, which is below every finite key)
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const int j = 64 * m + lane;
            const uint32_t kk = ordered_key(s[j < nblk ? j : nblk - 1]);
            key[m] = j < nblk ? kk : 0u;
        }
    }
    auto count_ge = [&](uint32_t cand) -> int {
        int cnt = 0;
        if (KPL > 0) {
#pragma unroll
            for (int m = 0; m < KPL; ++m) cnt += __popcll(__ballot(key[m] >= cand));
        } else {
            for (int j0 = 0; j0 < nblk; j0 += 64) {
                const int j = j0 + lane;
                cnt += __popcll(__ballot(j < nblk && ordered_key(s[j]) >= cand));
            }
        }
        return cnt;
    };
    // thr = the largest key value t with #(key >= t) >= keep
    uint32_t thr = 0;
    if (KPL > 0) {
        // phase 1: upper 16 bits
        uint32_t hi = 0;
        for (int bit = 15; bit >= 0; --bit) {
            const uint32_t c = hi | (1u << bit);
            if (count_ge(c << 16) >= keep) hi = c;
        }
        const int n_above = hi == 0xffffu ? 0 : count_ge((hi + 1) << 16);
        // keys in bucket hi -> this wave's LDS list
        uint32_t* cand = cand_all[wave];
        int nc = 0;
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const bool in = (key[m] >> 16) == hi;
            const uint64_t msk = __ballot(in);
            if (in) cand[nc + __popcll(msk & below)] = key[m];
            nc += __popcll(msk);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // phase 2: lower 16 bits, counting the bucket only
        thr = hi << 16;
        for (int bit = 15; bit >= 0; --bit) {
            const uint32_t c = thr | (1u << bit);
            int cnt = n_above;
            for (int j0 = 0; j0 < nc; j0 += 64) {
                const int j = j0 + lane;
                cnt += __popcll(__ballot(j < nc && cand[j < nc ? j : 0] >= c));
            }
            if (cnt >= keep) thr = c;
        }
    } else {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            if (count_ge(cand) >= keep) thr = cand;
        }
    }
    const int need = keep - (thr == 0xffffffffu ? 0 : count_ge(thr + 1));  // ties at thr, lowest index first
    int32_t* out = idx + row * (long)keep;
    int pos = 0, eqseen = 0;
    auto emit = [&](int j, uint32_t k) {
        const bool valid = j < nblk;
        const bool isgt = valid && k > thr;
        const bool iseq = valid && k == thr;
        const uint64_t eqm = __ballot(iseq);
        const bool sel = isgt || (iseq && eqseen + __popcll(eqm & below) < need);
        const uint64_t selm = __ballot(sel);
        if (sel) out[pos + __popcll(selm & below)] = j;
        pos += __popcll(selm);
        eqseen += __popcll(eqm);
    };
    if (KPL > 0) {
#pragma unroll
        for (int m = 0; m < (KPL > 0 ? KPL : 1); ++m)
            if (64 * m < nblk) emit(64 * m + lane, key[m]);
    } else {
        for (int j0 = 0; j0 < nblk; j0 += 64) {
            const int j = j0 + lane;
            emit(j, j < nblk ? ordered_key(s[j]) : 0u);
        }
    }
}

size_t select_scores_bytes(long BH, int nblk) { return sizeof(float) * (size_t)BH * nblk * nblk; }

hipError_t launch_select(int D, const float* qbar, const float* kbar, float* scores, int32_t* idx, long BH, int nblk,
                         int keep, hipStream_t st) {
    const float scale = 1.0f / sqrtf((float)D);
    const int nrb = (nblk + 31) / 32;
    const long nwg = (long)nrb * BH;
    dim3 g1((unsigned)nwg);
    if (D == 64)
        hipLaunchKernelGGL(k_block_scores<64>, g1, dim3(256), 0, st, qbar, kbar, scores, nblk, scale, nrb, nwg);
    else
        hipLaunchKernelGGL(k_block_scores<128>, g1, dim3(256), 0, st, qbar, kbar, scores, nblk, scale, nrb, nwg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long rows = BH * nblk;
    dim3 g2((unsigned)((rows + 3) / 4));
    const int kpl = (nblk + 63) / 64;
    if (kpl <= 8)
        hipLaunchKernelGGL(k_topk_rows<8>, g2, dim3(256), 0, st, scores, idx, rows, nblk, keep);
    else if (kpl <= 16)
        hipLaunchKernelGGL(k_topk_rows<16>, g2, dim3(256), 0, st, scores, idx, rows, nblk, keep);
    else if (kpl <= 20)
        hipLaunchKernelGGL(k_topk_rows<20>, g2, dim3(256), 0, st, scores, idx, rows, nblk, keep);
    else if (kpl <= 24)
        hipLaunchKernelGGL(k_topk_rows<24>, g2, dim3(256), 0, st, scores, idx, rows, nblk, keep);
    else if (kpl <= 32)
        hipLaunchKernelGGL(k_topk_rows<32>, g2, dim3(256), 0, st, scores, idx, rows, nblk, keep);
    else if (kpl <= 64)
        hipLaunchKernelGGL(k_topk_rows<64>, g2, dim3(256), 0, st, scores, idx, rows, nblk, keep);
    else
        hipLaunchKernelGGL(k_topk_rows<0>, g2, dim3(256), 0, st, scores, idx, rows, nblk, keep);
    return hipGetLastError();
}

}  // namespace slr
