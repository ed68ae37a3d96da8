// pkv_check.hip -- cold-path checks of the device-resident indices the hot-path kernels read without validating
// them (block tables, context lengths, prefix sums, positions, slot mappings).  Each check counts the offending
// entries on the device and reports through a small device array the caller reads after synchronising: the
// debug facility for inputs that would otherwise give unspecified results.  [ferrum-kernels 0.7.7,
// src/backend/cuda/paged.rs: paged_decode_attention's cold path copies the final lengths back to the host to
// check them against q_len; here the check stays on the device and costs no synchronisation of its own.]
//
// Report layout (int32[4]): [0] bad lengths / positions / prefix sums, [1] table entries (among those a call
// reads) outside [0, num_blocks), [2] the first sequence (or token) with a problem, INT32_MAX when none,
// [3] slots at or past num_blocks * block_size (slot checks only).
//
// All HIP code here is built with packed-fp32 instructions disabled.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(64) void report_clear_kernel(int32_t *report) {
    if (threadIdx.x < 4)
        report[threadIdx.x] = threadIdx.x == 2 ? INT32_MAX : 0;
}

// Adds this wave's count to report[slot] with one atomic (lane 0).
__device__ __forceinline__ void add_count(int32_t *report, int slot, int count) {
    for (int o = 32; o > 0; o >>= 1)
        count += __shfl_xor(count, o, 64);
    if ((threadIdx.x & 63) == 0 && count > 0)
        atomicAdd(report + slot, count);
}

// One workgroup per sequence.  Decode mode (cu == null): length L = lens[s] must lie in [0, BS * M]; the table
// entries a call reads are those of blocks [max(0, L - window) / BS, ceil(L / BS)).  Varlen mode: sequence s's
// new rows are cu[s] .. cu[s+1]-1 at positions pos[s] + i; cu must start at 0, not decrease and end at T, pos must
// be >= 0 with pos[s] + (new rows) <= BS * M, and the entries read are those of blocks [0, ceil((pos + n) / BS)).
__global__ __launch_bounds__(kCheckThreads) void check_indices_kernel(CheckParams p) {
    const int s = (int)blockIdx.x;
    const int cap = p.M * p.BS;
    int end_row;  // rows 0 .. end_row - 1 are read
    int first_row = 0;
    bool bad = false;
    if (p.cu_seqlens_q) {
        const int c0 = p.cu_seqlens_q[s], c1 = p.cu_seqlens_q[s + 1];
        const int pos = p.pos_offsets[s];
        bad = c1 < c0 || (s == 0 && c0 != 0) || (s == p.B - 1 && c1 != p.T) || pos < 0 ||
              (int64_t)pos + (c1 - c0) > cap;
        end_row = bad ? 0 : pos + (c1 - c0);
    } else {
        const int L = p.context_lens[s];
        bad = L < 0 || L > cap;
        end_row = bad ? 0 : L;
        if (p.window > 0 && end_row > p.window)
            first_row = end_row - p.window;
    }
    const int b0 = first_row / p.BS, b1 = (end_row + p.BS - 1) / p.BS;
    int count = 0;
    for (int j = b0 + (int)threadIdx.x; j < b1; j += kCheckThreads) {
        const int32_t b = p.block_tables[(int64_t)s * p.M + j];
        count += (b < 0 || b >= p.N) ? 1 : 0;
    }
    add_count(p.report, 1, count);
    if (threadIdx.x == 0 && bad)
        atomicAdd(p.report + 0, 1);
    // the first sequence with any problem
    __shared__ int any;
    if (threadIdx.x == 0)
        any = bad ? 1 : 0;
    __syncthreads();
    if (count > 0)
        atomicOr(&any, 1);
    __syncthreads();
    if (threadIdx.x == 0 && any)
        atomicMin(p.report + 2, s);
}

// One thread per token: slots at or past N * BS (negative slots mark padding and are allowed).
__global__ __launch_bounds__(kCheckThreads) void check_slots_kernel(CheckParams p) {
    const int i = (int)(blockIdx.x * kCheckThreads + threadIdx.x);
    bool bad = false;
    if (i < p.T) {
        const int64_t slot = p.slot_mapping[i];
        bad = slot >= (int64_t)p.N * p.BS;
        if (bad)
            atomicMin(p.report + 2, i);
    }
    add_count(p.report, 3, bad ? 1 : 0);
}

}  // namespace

hipError_t launch_check(const CheckParams &p, hipStream_t stream) {
    hipLaunchKernelGGL(report_clear_kernel, dim3(1), dim3(64), 0, stream, p.report);
    if (p.slot_mapping) {
        if (p.T > 0)
            hipLaunchKernelGGL(check_slots_kernel, dim3((unsigned)((p.T + kCheckThreads - 1) / kCheckThreads)),
                               dim3(kCheckThreads), 0, stream, p);
    } else if (p.B > 0) {
        hipLaunchKernelGGL(check_indices_kernel, dim3((unsigned)p.B), dim3(kCheckThreads), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace pkv
