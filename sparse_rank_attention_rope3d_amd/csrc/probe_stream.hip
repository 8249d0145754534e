// Probes of what the part sustains (a measurement utility of the bench, built
// as its own small library, libslr_probe.so; not part of the layer's ABI):
// the read bandwidth of the memory hierarchy, and the issue rate of the
// 32x32x16 bf16 MFMA with operands in registers.
//
// Read bandwidth:
// Each workgroup streams 16-byte vectors of a device buffer, `passes` times
// over, either into registers (ordinary vector loads, folded into one value
// per thread so none is dead) or straight into LDS with the direct
// global -> LDS copy the block-sparse flash kernel streams its tiles with.
// With the buffer larger than the L2 share of an XCD (4 MB each; workgroup p
// runs on XCD p % 8, and consecutive workgroups read consecutive 4 KB
// pieces, so an XCD touches one eighth of every 32 KB) the reads are served
// by the 256 MB memory-side cache (MALL) while the buffer fits in it, and by
// HBM beyond that: the rate at a few sizes tells which level bounds a
// kernel whose working set sits between the two.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool TO_LDS>
__global__ __launch_bounds__(256) void k_stream_read(const u32x4_t* __restrict__ buf, long nvec, int passes,
                                                     uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[4 * 256 * 4];   // 4 slots of 4 KB
    const long stride = (long)gridDim.x * 256;
    const long first = (long)blockIdx.x * 256 + threadIdx.x;
    const int wave = threadIdx.x >> 6;
    uint32_t acc = 0;
    int slot = 0;
    for (int p = 0; p < passes; ++p) {
        long i = first;
        // four independent loads in flight per thread
        for (; i + 3 * stride < nvec; i += 4 * stride) {
            if (TO_LDS) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void*)(buf + i + u * stride),
                        (__attribute__((address_space(3))) void*)(lds + (slot * 256 + wave * 64) * 4), 16, 0, 0);
                    slot = (slot + 1) & 3;
                }
                // at most eight copies of this wave in flight (the compiler does not count them)
                __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
            } else {
                const u32x4_t a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
                const u32x4_t x = a ^ b ^ c ^ d;
                acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
            }
        }
        for (; i < nvec; i += stride) {
            const u32x4_t a = buf[i];
            acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
        }
    }
    if (TO_LDS) {
        __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
        __syncthreads();
        acc ^= lds[threadIdx.x * 4];
    }
    sink[(long)blockIdx.x * 256 + threadIdx.x] = acc;
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// MFMA issue rate: each wave runs `iters` rounds of eight independent
// 32x32x16 bf16 accumulation chains on register operands (non-zero bf16
// values that vary by lane, so the multipliers toggle as on real data); the
// accumulators are folded into one value per thread at the end so no chain
// is dead. 32768 flops per MFMA.
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* __restrict__ sink) {
    const uint32_t lane = threadIdx.x;
    u32x4_t a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // two bf16 values in [0.5, 2): exponent 126 or 127, mantissa from a hash
            uint32_t h = (lane * 2654435761u) ^ ((uint32_t)(s * 4 + i) * 40503u) ^ (blockIdx.x * 97u);
            h ^= h >> 13;
            h *= 0x5bd1e995u;
            const uint32_t lo = 0x3f00u | (h & 0xffu) | ((h >> 8) & 0x80u);
            const uint32_t hi = 0x3f00u | ((h >> 16) & 0xffu) | ((h >> 24) & 0x80u);
            a[s][i] = lo | (hi << 16);
            b[s][i] = hi | (lo << 16);
        }
    f32x16_t c[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) c[s][i] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
            c[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(__attribute__((ext_vector_type(8))) __bf16, a[s]),
                __builtin_bit_cast(__attribute__((ext_vector_type(8))) __bf16, b[s ^ 1]), c[s], 0, 0, 0);
    }
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += c[s][i];
    sink[(long)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Launches the probe on `stream`: `nwg` workgroups of 256 threads read the
// `bytes` of `buf` (16-byte aligned; bytes a multiple of 16) `passes` times;
// sink receives nwg * 256 uint32 values. Returns 0, or -1 for bad arguments,
// -4 when the launch fails.
int slrprobe_stream_read(const void* buf, size_t bytes, int passes, int to_lds, int nwg, uint32_t* sink,
                         void* stream) {
    if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15) || bytes == 0 || passes < 1 ||
        nwg < 1 || nwg > 65536)
        return -1;
    const long nvec = (long)(bytes / 16);
    hipStream_t s = (hipStream_t)stream;
    if (to_lds)
        hipLaunchKernelGGL(k_stream_read<true>, dim3(nwg), dim3(256), 0, s, (const u32x4_t*)buf, nvec, passes, sink);
    else
        hipLaunchKernelGGL(k_stream_read<false>, dim3(nwg), dim3(256), 0, s, (const u32x4_t*)buf, nvec, passes, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Launches the MFMA probe on `stream`: `nwg` workgroups of 256 threads, each
// wave `iters` rounds of 8 MFMAs; sink receives nwg * 256 floats. Returns 0,
// or -1 for bad arguments, -4 when the launch fails.
int slrprobe_mfma_loop(int nwg, int iters, float* sink, void* stream) {
    if (!sink || nwg < 1 || nwg > 65536 || iters < 1) return -1;
    hipLaunchKernelGGL(k_mfma_loop, dim3(nwg), dim3(256), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
