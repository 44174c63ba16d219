// Reference kernels for the benchmark's HBM ceilings (not part of the fp8
// library's interface; built into libfp8bench.so, which only bench.py
// loads).  They move the same bytes as the library's bandwidth-bound kernels
// with no arithmetic, so their rates are the practical ceilings those kernels
// are measured against on this GPU:
//   * fp8bench_empty: a launch that does nothing (the per-launch floor);
//   * fp8bench_read: every byte of a buffer read once, 256 workgroups each
//     streaming a contiguous slab (the short-A GEMM's weight stream);
//   * fp8bench_stream21: the quantize's access pattern without the
//     conversion, the amax or the fold (read 2 bytes, write 1 byte per
//     element: the high byte of each bf16), in the quantize's launch shape
//     (grid, chunks per lane per round) and chunk order.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void empty_kernel() {}

// Each lane keeps kU 16-byte loads in flight; a contiguous slab per
// workgroup.  The xor of everything read is stored only in the (never
// taken) case that it equals a fixed pattern, so the loads cannot be
// dropped and nothing is written.
template <int kU, bool NT>
__global__ __launch_bounds__(512) void read_kernel(const uint4* b, int64_t nvec, uint32_t* sink) {
    const int64_t per = (nvec + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < nvec ? lo + per : nvec;
    uint32_t acc = 0;
    for (int64_t c0 = lo + threadIdx.x; c0 < hi; c0 += (int64_t)kU * blockDim.x) {
        uint4 r[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t c = c0 + (int64_t)u * blockDim.x;
            const int64_t cl = c < hi ? c : lo;
            if constexpr (NT) {
                typedef int v4i __attribute__((ext_vector_type(4)));
                const v4i t = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(b + cl));
                r[u] = make_uint4((uint32_t)t[0], (uint32_t)t[1], (uint32_t)t[2], (uint32_t)t[3]);
            } else {
                r[u] = b[cl];
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
    }
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

// 16 bf16 -> their 16 high bytes.
__device__ __forceinline__ uint32_t hi_bytes(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07050301u);
}

// The quantize's sweep: 256-lane workgroups, the grid's lanes taking
// consecutive 16-element chunks in each round, kUnroll chunks in flight per
// lane (4 below 2^25 elements, 1 from there, with the grid the caller
// passes).
constexpr int kThreads = 256;

template <int kUnroll>
__global__ __launch_bounds__(kThreads) void stream21_kernel(const uint4* x, int64_t nvec,
                                                           uint4* out) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const int64_t slot = (int64_t)gridDim.x * kThreads;  // chunks per slot of a round
    const int64_t round = slot * kUnroll;
    const int64_t nr = (nvec + round - 1) / round;
    const int64_t mine = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (int64_t rd = 0; rd < nr; ++rd) {
        const int64_t c0 = rd * round + mine;
        uint4 r[kUnroll][2];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t c = c0 + u * slot;
            const int64_t cl = c < nvec ? c : 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const v4i t = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(x + 2 * cl + i));
                r[u][i] = make_uint4((uint32_t)t[0], (uint32_t)t[1], (uint32_t)t[2], (uint32_t)t[3]);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t c = c0 + u * slot;
            if (c < nvec)
                out[c] = make_uint4(hi_bytes(r[u][0].x, r[u][0].y), hi_bytes(r[u][0].z, r[u][0].w),
                                    hi_bytes(r[u][1].x, r[u][1].y), hi_bytes(r[u][1].z, r[u][1].w));
        }
    }
}

}  // namespace

extern "C" {

// Returns 0 on success, else the HIP error code of the launch.
int fp8bench_empty(int grid, int threads, hipStream_t stream) {
    if (grid < 1 || threads < 1 || threads > 1024) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(threads), 0, stream);
    return (int)hipGetLastError();
}

// bytes: a multiple of 16; b 16-byte aligned; sink: 512 uint32 (never
// written in practice).
int fp8bench_read(const void* b, int64_t bytes, uint32_t* sink, int grid, int nontemporal,
                  hipStream_t stream) {
    if (!b || !sink || bytes < 16 || (bytes % 16) || grid < 1 ||
        (reinterpret_cast<uintptr_t>(b) & 15))
        return (int)hipErrorInvalidValue;
    const int64_t nvec = bytes / 16;
    if (nontemporal)
        hipLaunchKernelGGL((read_kernel<8, true>), dim3(grid), dim3(512), 0, stream,
                           static_cast<const uint4*>(b), nvec, sink);
    else
        hipLaunchKernelGGL((read_kernel<8, false>), dim3(grid), dim3(512), 0, stream,
                           static_cast<const uint4*>(b), nvec, sink);
    return (int)hipGetLastError();
}

// numel: a multiple of 16; x, out 16-byte aligned; unroll: 1 or 4 chunks
// per lane per round.
int fp8bench_stream21(const uint16_t* x, int64_t numel, uint8_t* out, int grid, int unroll,
                      hipStream_t stream) {
    if (!x || !out || numel < 16 || (numel % 16) || grid < 1 ||
        (unroll != 1 && unroll != 4) ||
        ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) & 15))
        return (int)hipErrorInvalidValue;
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    uint4* ov = reinterpret_cast<uint4*>(out);
    if (unroll == 1)
        hipLaunchKernelGGL(stream21_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, xv,
                           numel / 16, ov);
    else
        hipLaunchKernelGGL(stream21_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, xv,
                           numel / 16, ov);
    return (int)hipGetLastError();
}

}  // extern "C"
