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

// One workgroup (4 waves) = a 64 x 64 tile of the score matrix of one slice;
// wave (wi, wj) owns the 32 x 32 sub-tile. A = qbar rows (m = i, k = d),
// B = kbar rows (k = d, n = j), both read straight from global memory.
template <int D>
__global__ __launch_bounds__(256) void k_block_scores(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                      float* __restrict__ scores, int nblk, float scale) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const long bh = blockIdx.z;
    const int i0 = blockIdx.y * 64 + 32 * (wave & 1);
    const int j0 = blockIdx.x * 64 + 32 * (wave >> 1);
    const float* qb = qbar + bh * (long)nblk * D;
    const float* kb = kbar + bh * (long)nblk * D;
    const int ia = i0 + l32, jb = j0 + l32;
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        float xa[8], xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { xa[e] = 0.f; xb[e] = 0.f; }
        if (ia < nblk) {
            const f32x4_t* p = reinterpret_cast<const f32x4_t*>(qb + (long)ia * D + 16 * s + 8 * hf);
            const f32x4_t u = p[0], w = p[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) { xa[e] = u[e]; xa[4 + e] = w[e]; }
        }
        if (jb < nblk) {
            const f32x4_t* p = reinterpret_cast<const f32x4_t*>(kb + (long)jb * D + 16 * s + 8 * hf);
            const f32x4_t u = p[0], w = p[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) { xb[e] = u[e]; xb[4 + e] = w[e]; }
        }
        u32x4_t ah, al, bhi, blo;
        split8(xa, ah, al);
        split8(xb, bhi, blo);
        acc = mfma32(ah, bhi, acc);
        acc = mfma32(ah, blo, acc);
        acc = mfma32(al, bhi, acc);
    }
    // lane holds rows i0 + 8(v/4) + 4hf + v%4 of column j0 + l32
    if (jb < nblk) {
        float* out = scores + bh * (long)nblk * nblk + jb;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = i0 + 8 * (v >> 2) + 4 * hf + (v & 3);
            if (i < nblk) out[(long)i * nblk] = acc[v] * scale;
        }
    }
}

// Top-k of one score row per wave. KPL = keys per lane held in registers
// (column j = 64 m + lane); KPL = 0 reads the row from memory on every pass.
template <int KPL>
__global__ __launch_bounds__(256) void k_topk_rows(const float* __restrict__ scores, int32_t* __restrict__ idx,
                                                   long nrows, int nblk, int keep) {
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= nrows) return;
    const float* s = scores + row * nblk;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t key[KPL > 0 ? KPL : 1];
    if (KPL > 0) {
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const int j = 64 * m + lane;
            key[m] = j < nblk ? ordered_key(s[j]) : 0u;   // 0 is below every finite key
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
    // largest key value t with #(key >= t) >= keep, built bit by bit
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        if (count_ge(cand) >= keep) thr = cand;
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
    const int nt = (nblk + 63) / 64;
    dim3 g1((unsigned)nt, (unsigned)nt, (unsigned)BH);
    if (D == 64)
        hipLaunchKernelGGL(k_block_scores<64>, g1, dim3(256), 0, st, qbar, kbar, scores, nblk, scale);
    else
        hipLaunchKernelGGL(k_block_scores<128>, g1, dim3(256), 0, st, qbar, kbar, scores, nblk, scale);
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
