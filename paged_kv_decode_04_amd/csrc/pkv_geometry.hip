// pkv_geometry.hip -- host-side facts about the compiled kernels that the dispatcher plans with: which head dims
// and block sizes have kernels, how many wavefronts a workgroup of each may have, and how much LDS a launch asks
// for.  They follow the kernels' own layout constants (pkv_unit.h, pkv_internal.h); kept apart from the kernel
// sources so that host-only builds of the API (the CPU sanitizer test) link them without any device code.
#include "pkv_internal.h"
#include "pkv_unit.h"

namespace pkv {

size_t decode_lds_bytes(int head_dim, int G, int waves) {
    // the merge area, then the fused step's copy of the new row (K and V, head_dim halves each)
    return sizeof(float) * merge_floats(head_dim, G, waves) + 4 * (size_t)head_dim;
}

size_t varlen_lds_bytes(int head_dim, int waves, bool fused) {
    // the merge area, then (fused step) kFusedUnits units of new K and V rows
    return sizeof(float) * (size_t)merge_floats(head_dim, 16, waves) +
           (fused ? sizeof(_Float16) * (size_t)kFusedUnits * 32 * head_dim : 0);
}

bool decode_geometry_supported(int head_dim, int block_size) {
    return (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
           (block_size == 16 || block_size == 32 || block_size == 64);
}

// Two K/V fragment sets of head dim 256 need more registers than a wave of an 8-wave group has, so that variant
// would spill and is not compiled.
int max_waves_per_group(int head_dim) { return head_dim >= 256 ? 4 : kMaxWaves; }

}  // namespace pkv
