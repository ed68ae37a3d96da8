// pkv_probe.hip -- a measurement probe, not part of the attention path: the simplest kernel that moves a decode
// launch's bytes in the same work decomposition.  Workgroup g (512 threads, one per tile, in the order the decode
// launch dispatches its tiles) streams its own contiguous slice of x -- len16[g] 16-byte chunks from chunk off16[g],
// eight of them in flight per thread, non-temporal -- and, if write_bytes > 0, writes that many bytes of y at its end
// (the tile's output), so
// bench.py can time what the tiles' sizes alone cost on this GPU with the plainest kernel of that decomposition (a
// reference, not a bound: eight pipelined waves per tile keep more bytes in flight on long tiles than its one
// pass).  Built into its own library (libpkvprobe.so); all HIP code here is built with packed-fp32
// instructions disabled.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_probe.h"

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u4 *__restrict__ x, int64_t x16,
                                                               const int64_t *__restrict__ off16,
                                                               const int32_t *__restrict__ len16, u4 *__restrict__ y,
                                                               int32_t write16) {
    const int64_t g = blockIdx.x;
    // a run is clamped into x, so no offset or length reads outside it
    int64_t off = off16[g];
    off = off < 0 ? 0 : (off > x16 ? x16 : off);
    int64_t n = len16[g] < 0 ? 0 : len16[g];
    n = n < x16 - off ? n : x16 - off;
    const u4 *xs = x + off;
    uint32_t acc = 0;
    int64_t i = threadIdx.x;
    for (; i + (kInFlight - 1) * kThreads < n; i += kInFlight * kThreads) {
        u4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            v[u] = __builtin_nontemporal_load(xs + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += kThreads) {
        const u4 v = xs[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // the tile's output (the loaded data folded in, so that no load can be dropped)
    u4 *ys = y + g * write16;
    for (int64_t j = threadIdx.x; j < write16; j += kThreads)
        ys[j] = (u4){acc, acc ^ 1u, acc ^ 2u, (uint32_t)j};
}

}  // namespace

extern "C" {

int pkv_probe_stream_read(const void *x, int64_t x_bytes, const int64_t *off16, const int32_t *len16, void *y,
                          int32_t groups, int32_t write_bytes, void *stream) {
    if (groups < 0 || x_bytes < 0 || write_bytes < 0 || write_bytes % 16 != 0)
        return 1;
    if (groups == 0)
        return 0;
    if (!x || !off16 || !len16 || (write_bytes > 0 && !y) || ((uintptr_t)x % 16) ||
        (write_bytes > 0 && ((uintptr_t)y % 16)))
        return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)groups), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u4 *>(x), x_bytes / 16, off16, len16, static_cast<u4 *>(y),
                       write_bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
