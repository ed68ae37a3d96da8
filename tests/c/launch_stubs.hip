// Kernel-launch stubs for the host-only sanitizer build of the library: the host code of pkv_api.hip,
// pkv_check.hip and pkv_geometry.hip is linked with these in place of the kernel sources, so that building it with
// AddressSanitizer and UndefinedBehaviorSanitizer takes seconds and runs without a GPU.  Every stub counts its call
// and fails as an unsupported launch; the host-path checks expect no call at all (every error they provoke must be
// found before anything is enqueued).
#include <stdio.h>

#include "pkv_internal.h"

namespace {
int g_launches = 0;
hipError_t stub(const char *name) {
    ++g_launches;
    fprintf(stderr, "stub launch: %s\n", name);
    return hipErrorNotSupported;
}
}  // namespace

extern "C" __attribute__((visibility("default"))) int pkv_test_stub_launches(void) { return g_launches; }

namespace pkv {
hipError_t launch_decode(const DecodeParams &, int, int, int, int, bool, hipStream_t) { return stub("decode"); }
hipError_t launch_combine(const CombineParams &, int, hipStream_t) { return stub("combine"); }
hipError_t launch_varlen(const VarlenParams &, int, int, int, int, bool, hipStream_t) { return stub("varlen"); }
hipError_t launch_append(const AppendParams &, hipStream_t) { return stub("append"); }
hipError_t launch_append_newest(const AppendParams &, hipStream_t) { return stub("append_newest"); }
hipError_t launch_order(const int32_t *, const int32_t *, int, int, int, int, int32_t *, const PieceRule &, hipStream_t) {
    return stub("order");
}
hipError_t launch_order_varlen(const int32_t *, const int32_t *, const int32_t *, int, int, int, int32_t *,
                               hipStream_t) {
    return stub("order_varlen");
}
hipError_t launch_append_varlen(const AppendParams &, const int32_t *, const int32_t *, int, int, hipStream_t) {
    return stub("append_varlen");
}
hipError_t launch_qkv_cache(const QkvParams &, int, hipStream_t) { return stub("qkv_cache"); }
}  // namespace pkv
