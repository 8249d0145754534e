// Per-query-block top-k selection of key blocks.
//
// RoLA (arXiv 2609.06712v3) Fig. 2 / §4.1: the sparse branch keeps the
// top-k key blocks of every query block. Scores are
// s_ij = qbar_i . kbar_j / sqrt(D) of the fp32 block means, computed in fp32
// (fp32 MFMA); the k-th largest is found exactly with a bitwise search over
// order-preserving 32-bit keys, ties go to the lower block index, and the
// kept indices are written in ascending order.
#include "slr_common.h"
#include "slr_launch.h"

namespace slr {

// One workgroup (4 waves) = `qt` consecutive query blocks of one (b, h)
// slice. Phase 1 fills an LDS score tile [qt][nblk] with 16x16x4 fp32 MFMAs
// (rows beyond qt are zero operands); phase 2 gives each wave whole rows.
template <int D>
__global__ __launch_bounds__(256) void k_select(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                int32_t* __restrict__ idx, int nblk, int keep, int qt,
                                                int ld, float scale) {
    extern __shared__ float sc[];  // [qt][ld]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long bh = blockIdx.y;
    const int i0 = blockIdx.x * qt;
    const float* qb = qbar + bh * nblk * D;
    const float* kb = kbar + bh * nblk * D;

    // A operand: query block i0 + lane%16, dims 16p + 4*(lane/16) + {0..3}
    const int arow = lane & 15, kq = 4 * (lane >> 4);
    const bool aval = arow < qt && i0 + arow < nblk;
    f32x4_t a[D / 16];
#pragma unroll
    for (int p = 0; p < D / 16; ++p) {
        a[p] = aval ? *reinterpret_cast<const f32x4_t*>(qb + (long)(i0 + arow) * D + 16 * p + kq)
                    : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int c0 = wave * 16; c0 < nblk; c0 += 64) {
        const int col = c0 + (lane & 15);
        const bool bval = col < nblk;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < D / 16; ++p) {
            f32x4_t b = bval ? *reinterpret_cast<const f32x4_t*>(kb + (long)col * D + 16 * p + kq)
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc = mfma16f32(a[p][0], b[0], acc);
            acc = mfma16f32(a[p][1], b[1], acc);
            acc = mfma16f32(a[p][2], b[2], acc);
            acc = mfma16f32(a[p][3], b[3], acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 4 * (lane >> 4) + v;
            if (row < qt && bval) sc[row * ld + col] = acc[v] * scale;
        }
    }
    __syncthreads();

    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int row = wave; row < qt; row += 4) {
        const int i = i0 + row;
        if (i >= nblk) break;
        const float* s = sc + row * ld;
        // largest key value t with #(key >= t) >= keep, built bit by bit
        uint32_t thr = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int cnt = 0;
            for (int j = lane; j < nblk; j += 64) cnt += ordered_key(s[j]) >= cand;
            if (wave_sum_int(cnt) >= keep) thr = cand;
        }
        int gt = 0;
        for (int j = lane; j < nblk; j += 64) gt += ordered_key(s[j]) > thr;
        const int need = keep - wave_sum_int(gt);  // ties at the threshold to keep, lowest index first
        int pos = 0, eqseen = 0;
        int32_t* out = idx + (bh * nblk + i) * (long)keep;
        for (int j0 = 0; j0 < nblk; j0 += 64) {
            const int j = j0 + lane;
            const uint32_t key = j < nblk ? ordered_key(s[j]) : 0u;
            const bool isgt = j < nblk && key > thr;
            const bool iseq = j < nblk && key == thr;
            const uint64_t eqm = __ballot(iseq);
            const bool sel = isgt || (iseq && eqseen + __popcll(eqm & below) < need);
            const uint64_t selm = __ballot(sel);
            if (sel) out[pos + __popcll(selm & below)] = j;
            pos += __popcll(selm);
            eqseen += __popcll(eqm);
        }
    }
}

// rows per workgroup: as many as fit 64 KB of scores, at most 16
int select_rows_per_wg(int nblk) {
    const int ld = nblk + 1;
    int qt = 16;
    while (qt > 1 && (size_t)qt * ld * sizeof(float) > 64 * 1024) qt >>= 1;
    return qt;
}

size_t select_lds_bytes(int nblk) { return (size_t)select_rows_per_wg(nblk) * (nblk + 1) * sizeof(float); }

hipError_t launch_select(int D, const float* qbar, const float* kbar, int32_t* idx, long BH, int nblk, int keep,
                         hipStream_t st) {
    const int qt = select_rows_per_wg(nblk);
    const int ld = nblk + 1;
    const size_t lds = (size_t)qt * ld * sizeof(float);
    dim3 grid((unsigned)((nblk + qt - 1) / qt), (unsigned)BH);
    const float scale = 1.0f / sqrtf((float)D);
    if (D == 64)
        hipLaunchKernelGGL(k_select<64>, grid, dim3(256), lds, st, qbar, kbar, idx, nblk, keep, qt, ld, scale);
    else
        hipLaunchKernelGGL(k_select<128>, grid, dim3(256), lds, st, qbar, kbar, idx, nblk, keep, qt, ld, scale);
    return hipGetLastError();
}

}  // namespace slr
