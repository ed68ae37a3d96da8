// pkv_api.hip -- host side of libpkv: argument checks, the split dispatcher,
// the library-owned split-K workspace and the extern "C" entry points
// declared in include/pkv.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

thread_local char g_error[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_error[0] = '\0';
    return PKV_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(PKV_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---------------------------------------------------------------------------
// device facts, cached per device ordinal

struct DeviceFacts {
    int cu_count = 0;
    int lds_per_block = 0;
};

std::mutex g_dev_mutex;
std::map<int, DeviceFacts> g_dev;

int device_facts(DeviceFacts *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> g(g_dev_mutex);
    auto it = g_dev.find(dev);
    if (it != g_dev.end()) {
        *out = it->second;
        return PKV_OK;
    }
    DeviceFacts f;
    e = hipDeviceGetAttribute(&f.cu_count, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
    e = hipDeviceGetAttribute(&f.lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipDeviceGetAttribute(MaxSharedMemoryPerBlock)");
    g_dev[dev] = f;
    *out = f;
    return PKV_OK;
}

// ---------------------------------------------------------------------------
// split-K workspace owned by the library: grow-only, one per (device, stream)

struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Buffers replaced by growth.  They stay allocated until the process exits: a HIP graph captured while one of them
// was current holds its address in its kernel arguments and may be replayed after the growth.
std::vector<void *> g_ws_retired;

int library_workspace(size_t need, hipStream_t stream, void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> g(g_ws_mutex);
    Workspace &w = g_ws[std::make_pair(dev, stream)];
    if (w.bytes < need) {
        // Growing allocates (hipMalloc), which a stream under graph capture must not do: the caller warms the
        // workspace up with one call on this stream before capturing, or passes its own (the _ws variants).
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamIsCapturing");
        if (cap != hipStreamCaptureStatusNone)
            return fail(PKV_EWORKSPACE, "the library workspace of this stream holds %zu bytes, the call needs %zu, and "
                        "the stream is being captured: make one call on this stream before capture, or pass a "
                        "workspace", w.bytes, need);
        // The old buffer is retired, not freed: queued kernels and captured graphs may still use it.
        size_t grown = need + need / 4;  // slack so that small growth does not reallocate every call
        void *fresh = nullptr;
        e = hipMalloc(&fresh, grown);
        if (e != hipSuccess)
            return fail(PKV_ENOMEM, "hipMalloc of %zu workspace bytes failed: %s", grown, hipGetErrorString(e));
        if (w.ptr)
            g_ws_retired.push_back(w.ptr);
        w.ptr = fresh;
        w.bytes = grown;
    }
    *ptr = w.ptr;
    return PKV_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bytes of the library workspace of this (device, stream) now, without growing it.
size_t library_workspace_bytes(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    std::lock_guard<std::mutex> g(g_ws_mutex);
    auto it = g_ws.find(std::make_pair(dev, stream));
    return it == g_ws.end() ? 0 : it->second.bytes;
}

struct WsLayout {
    size_t o_off, m_off, l_off, order_off, count_off, total;
};

// Split-K partials (S > 1), then order_ints int32 of dispatch-order records.
WsLayout ws_layout(int64_t B, int64_t Hq, int64_t D, int64_t S, int64_t order_ints = 0) {
    WsLayout L;
    const size_t o = S > 1 ? round256((size_t)(B * Hq * S * D) * sizeof(float)) : 0;
    const size_t ml = S > 1 ? round256((size_t)(B * Hq * S) * sizeof(float)) : 0;
    L.o_off = 0;
    L.m_off = o;
    L.l_off = o + ml;
    L.order_off = o + 2 * ml;
    L.count_off = 0;
    L.total = L.order_off + round256((size_t)order_ints * sizeof(int32_t));
    return L;
}

// An ordered single pass with pieces (see pkv::PieceRule): the pieces' partials ([records][Hq][D] outputs, then
// [records][Hq] maxima and sums), the records, then the [B][Hkv] piece counters.
WsLayout ws_layout_pieces(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t records) {
    WsLayout L;
    const size_t o = round256((size_t)(records * Hq * D) * sizeof(float));
    const size_t ml = round256((size_t)(records * Hq) * sizeof(float));
    L.o_off = 0;
    L.m_off = o;
    L.l_off = o + ml;
    L.order_off = o + 2 * ml;
    L.count_off = L.order_off + round256((size_t)(records * pkv::kOrderRecord) * sizeof(int32_t));
    L.total = L.count_off + round256((size_t)(B * Hkv) * sizeof(int32_t));
    return L;
}

// Where a call's split-K partials and dispatch-order records live.
enum WsKind {
    kCallerWs = 0,   // a workspace the caller passes (the _ws / _planned variants)
    kLibraryWs = 1,  // the library-owned, grow-only buffer of the (device, stream)
    kFixedWs = 2,    // the fixed device array below (pkv_paged_decode_attention_noalloc)
};

// ---------------------------------------------------------------------------
// Fixed device scratch for callers that cannot allocate (pkv_paged_decode_attention_noalloc).  Each device that
// loads the library holds its own copy of the array until the process exits.  In host code `scratch` names a host
// stand-in, not device memory: kernels get the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
std::map<int, void *> g_scratch_ptr;  // device ordinal -> that device's address of `scratch`

int scratch_address(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> g(g_scratch_mutex);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *ptr = it->second;
        return PKV_OK;
    }
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256))
        return fail(PKV_EHIP, "hipGetSymbolAddress(scratch) returned %p, not a 256-byte aligned device address", p);
    g_scratch_ptr[dev] = p;
    *ptr = p;
    return PKV_OK;
}

// ---------------------------------------------------------------------------
// checks shared by the attention entry points

int check_pool(const pkv_pool_desc &pool) {
    if (pool.num_kv_heads <= 0 || pool.head_dim <= 0 || pool.block_size <= 0 || pool.num_blocks < 0)
        return fail(PKV_EINVAL, "bad pool geometry (Hkv=%d, D=%d, BS=%d, N=%d)", pool.num_kv_heads,
                    pool.head_dim, pool.block_size, pool.num_blocks);
    return PKV_OK;
}

int check_decode_geometry(int32_t num_seqs, int32_t num_q_heads, const pkv_pool_desc &pool,
                          int32_t max_blocks_per_seq) {
    int rc = check_pool(pool);
    if (rc)
        return rc;
    if (num_seqs < 0)
        return fail(PKV_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
    if (num_q_heads <= 0 || num_q_heads % pool.num_kv_heads != 0)
        return fail(PKV_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", num_q_heads,
                    pool.num_kv_heads);
    if (max_blocks_per_seq <= 0)
        return fail(PKV_EINVAL, "max_blocks_per_seq must be > 0 (got %d)", max_blocks_per_seq);
    if (!pkv::decode_geometry_supported(pool.head_dim, pool.block_size))
        return fail(PKV_EUNSUPPORTED, "head_dim %d / block_size %d not compiled (head_dim 64|128|256, "
                    "block_size 16|32|64)", pool.head_dim, pool.block_size);
    const int G = num_q_heads / pool.num_kv_heads;
    if (G > 16)
        return fail(PKV_EUNSUPPORTED, "group size %d > 16 query heads per kv head is not compiled", G);
    if ((int64_t)max_blocks_per_seq * pool.block_size > INT32_MAX)
        return fail(PKV_EINVAL, "max_blocks_per_seq * block_size overflows int32");
    if ((int64_t)num_seqs * pool.num_kv_heads > INT32_MAX)
        return fail(PKV_EINVAL, "num_seqs * num_kv_heads overflows the grid");
    return PKV_OK;
}

int check_decode_pointers(const void *q, const void *k_pool, const void *v_pool, const void *block_tables,
                          const void *context_lens, const void *out) {
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
        return fail(PKV_EINVAL, "null device pointer (q=%p k_pool=%p v_pool=%p block_tables=%p "
                    "context_lens=%p out=%p)", q, k_pool, v_pool, block_tables, context_lens, out);
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16))
        return fail(PKV_EINVAL, "q, k_pool, v_pool and out must be 16-byte aligned");
    if (!aligned(block_tables, 4) || !aligned(context_lens, 4))
        return fail(PKV_EINVAL, "block_tables and context_lens must be 4-byte aligned");
    return PKV_OK;
}

// The dispatcher.  Work per (sequence, kv head) tile is read once, so the
// question is only how many workgroups the grid needs.  One workgroup streams
// at most ~50 GB/s (one CU's share of outstanding misses), so a single pass
// reaches the HBM roofline once about half the CUs hold a tile; with fewer
// tiles each is split into about CUs / tiles ranges (one round of the CUs, each
// range at least 8 blocks).  A split costs a combine launch and
// G*(D+2)*4 bytes written and read per split.  The pages' 128-SM constants
// become the device's CU count; the rules and waves per workgroup come from
// measurements on MI355X.
int plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t max_blocks_per_seq, int32_t max_context_hint, int32_t num_splits, int32_t cu_count,
                int32_t lds_limit, pkv_decode_plan *plan) {
    if (!plan)
        return fail(PKV_EINVAL, "plan is null");
    if (num_splits < 0)
        return fail(PKV_EINVAL, "num_splits must be >= 0 (got %d)", num_splits);
    if (max_context_hint < 0)
        return fail(PKV_EINVAL, "max_context_hint must be >= 0 (got %d)", max_context_hint);
    pkv_pool_desc pool = {num_kv_heads, head_dim, block_size, 0};
    int rc = check_decode_geometry(num_seqs, num_q_heads, pool, max_blocks_per_seq);
    if (rc)
        return rc;
    const int G = num_q_heads / num_kv_heads;
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    const int64_t lmax = max_context_hint > 0 ? (max_context_hint < cap ? max_context_hint : cap) : cap;
    const int64_t nbmax = (lmax + block_size - 1) / block_size;
    const int64_t tiles = (int64_t)num_seqs * num_kv_heads;
    int S = 1;
    if (num_splits >= 1) {
        S = num_splits;
    } else if (tiles > 0) {
        // One workgroup streams at most ~50 GB/s (one CU's share of outstanding misses), so a single pass needs
        // about half the CUs busy to reach the HBM roofline; with fewer tiles, split each into about CUs / tiles
        // ranges (one round of the CUs; each range at least 8 blocks).  Measured on MI355X: with as many tiles as
        // CUs or more, a single pass beats every split (the combine launch and the partials cost more than the
        // ragged tail they remove).
        const int64_t cu = cu_count > 0 ? cu_count : 256;
        if (nbmax > 8 && 2 * tiles < cu) {
            int64_t want = (cu + tiles - 1) / tiles;
            if (want > nbmax / 8)
                want = nbmax / 8;
            if (want > 64)
                want = 64;
            S = (int)(want < 1 ? 1 : want);
        }
    }
    if (S > 65535)
        return fail(PKV_EINVAL, "num_splits %d exceeds the grid limit 65535", S);
    if ((int64_t)num_seqs * num_kv_heads * S > INT32_MAX)
        return fail(PKV_EINVAL, "num_seqs * num_kv_heads * num_splits overflows the grid");
    int waves = 8;  // measured best for head_dim <= 128, single pass and splits alike
    if (waves > pkv::max_waves_per_group(head_dim))
        waves = pkv::max_waves_per_group(head_dim);
    const size_t limit = lds_limit > 0 ? (size_t)lds_limit : (size_t)65536;
    while (waves > 1 && pkv::decode_lds_bytes(head_dim, G, waves) > limit)
        waves >>= 1;
    if (pkv::decode_lds_bytes(head_dim, G, waves) > limit)
        return fail(PKV_EUNSUPPORTED, "LDS need %zu exceeds the device limit %zu",
                    pkv::decode_lds_bytes(head_dim, G, waves), limit);
    plan->num_splits = S;
    plan->chunk_blocks = 0;
    plan->waves_per_group = waves;
    plan->reserved = 0;
    plan->workspace_bytes = S > 1 ? ws_layout(num_seqs, num_q_heads, head_dim, S).total : 0;
    return PKV_OK;
}

pkv::DecodeParams decode_params(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                const pkv_pool_desc &pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                const int32_t *context_lens, int32_t num_q_heads, float scale) {
    pkv::DecodeParams p;
    memset(&p, 0, sizeof p);
    p.q = reinterpret_cast<const _Float16 *>(q);
    p.k_pool = reinterpret_cast<const _Float16 *>(k_pool);
    p.v_pool = reinterpret_cast<const _Float16 *>(v_pool);
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.Hq = num_q_heads;
    p.Hkv = pool.num_kv_heads;
    p.G = num_q_heads / pool.num_kv_heads;
    p.N = pool.num_blocks;
    p.M = max_blocks_per_seq;
    p.num_splits = 1;
    p.chunk_blocks = 0;
    p.scale_log2 = scale * 1.44269504088896340736f;
    return p;
}

// Checks a plan against the geometry and the device; S == 1 is a single pass (chunk ignored).
int check_plan(const pkv_decode_plan &plan, int32_t num_seqs, int32_t num_q_heads, const pkv_pool_desc &pool,
               int32_t max_blocks_per_seq, int lds_limit) {
    if (plan.num_splits < 1 || plan.num_splits > 65535)
        return fail(PKV_EINVAL, "plan.num_splits must be in [1, 65535] (got %d)", plan.num_splits);
    if (plan.chunk_blocks < 0)
        return fail(PKV_EINVAL, "plan.chunk_blocks must be >= 0 (got %d)", plan.chunk_blocks);
    if (plan.num_splits > 1 && plan.chunk_blocks > 0 &&
        (int64_t)plan.num_splits * plan.chunk_blocks < max_blocks_per_seq)
        return fail(PKV_EINVAL, "plan: num_splits * chunk_blocks (%d * %d) does not cover max_blocks_per_seq %d",
                    plan.num_splits, plan.chunk_blocks, max_blocks_per_seq);
    if ((int64_t)num_seqs * pool.num_kv_heads * plan.num_splits > INT32_MAX)
        return fail(PKV_EINVAL, "num_seqs * num_kv_heads * num_splits overflows the grid");
    const int w = plan.waves_per_group;
    if (w != 1 && w != 2 && w != 4 && w != 8)
        return fail(PKV_EINVAL, "plan.waves_per_group must be 1, 2, 4 or 8 (got %d)", w);
    if (w > pkv::max_waves_per_group(pool.head_dim))
        return fail(PKV_EUNSUPPORTED, "plan.waves_per_group %d exceeds the %d compiled for head_dim %d", w,
                    pkv::max_waves_per_group(pool.head_dim), pool.head_dim);
    if (lds_limit < 0)
        return PKV_OK;  // the device-free checks only (the LDS limit is the device's)
    const size_t need = pkv::decode_lds_bytes(pool.head_dim, num_q_heads / pool.num_kv_heads, w);
    const size_t limit = lds_limit > 0 ? (size_t)lds_limit : (size_t)65536;
    if (need > limit)
        return fail(PKV_EUNSUPPORTED, "plan needs %zu LDS bytes per workgroup, the device allows %zu", need, limit);
    return PKV_OK;
}

// Where the decode step from QKV rows takes q and the new K/V rows (pkv_paged_decode_step_qkv).
struct QkvSource {
    const uint16_t *qkv;
    const uint16_t *q_norm_w;
    const uint16_t *k_norm_w;
    const float *cos_t;
    const float *sin_t;
    int32_t P;
    int32_t qk_mode;
    float eps;
    uint16_t *q_out;
};

// Checks of the QKV-row arguments shared by the QKV entry points.
int check_qkv_source(const QkvSource &q, int32_t head_dim) {
    if (q.P <= 0)
        return fail(PKV_EINVAL, "max_positions must be > 0 (got %d)", q.P);
    if (q.qk_mode != 0 && q.qk_mode != 1)
        return fail(PKV_EINVAL, "qk_mode must be 0 (rotate only) or 1 (RMS norm, then rotate); got %d", q.qk_mode);
    if (!(q.eps >= 0.f) || !isfinite(q.eps))
        return fail(PKV_EINVAL, "eps must be finite and >= 0");
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return fail(PKV_EUNSUPPORTED, "head_dim %d not compiled (64|128|256)", head_dim);
    return PKV_OK;
}

int check_qkv_pointers(const QkvSource &q) {
    if (!q.qkv || !q.cos_t || !q.sin_t || !q.q_out || (q.qk_mode == 1 && (!q.q_norm_w || !q.k_norm_w)))
        return fail(PKV_EINVAL, "null device pointer (qkv=%p cos=%p sin=%p q_out=%p q_norm_w=%p k_norm_w=%p)", q.qkv,
                    q.cos_t, q.sin_t, q.q_out, q.q_norm_w, q.k_norm_w);
    if (!aligned(q.qkv, 16) || !aligned(q.q_out, 16) || !aligned(q.cos_t, 16) || !aligned(q.sin_t, 16) ||
        (q.qk_mode == 1 && (!aligned(q.q_norm_w, 16) || !aligned(q.k_norm_w, 16))))
        return fail(PKV_EINVAL, "qkv, q_out, the cos/sin tables and the norm weights must be 16-byte aligned");
    return PKV_OK;
}

// Enqueues the kernels of a checked plan.
int run_plan(const pkv_decode_plan &plan, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
             const pkv_pool_desc &pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
             const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, float scale, uint16_t *out,
             void *workspace, size_t workspace_bytes, WsKind ws_kind, hipStream_t stream, int cu_count,
             const uint16_t *k_new = nullptr, const uint16_t *v_new = nullptr, int32_t window = 0,
             const QkvSource *qsrc = nullptr, const pkv::AppendParams *pre_append = nullptr) {
    pkv::DecodeParams p = decode_params(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens,
                                        num_q_heads, scale);
    p.window = window;
    p.out = reinterpret_cast<_Float16 *>(out);
    if (qsrc) {  // decode step from QKV rows, one launch: q and the new rows are formed in the kernel
        p.qkv = reinterpret_cast<const _Float16 *>(qsrc->qkv);
        p.q_norm_w = reinterpret_cast<const _Float16 *>(qsrc->q_norm_w);
        p.k_norm_w = reinterpret_cast<const _Float16 *>(qsrc->k_norm_w);
        p.cos_t = qsrc->cos_t;
        p.sin_t = qsrc->sin_t;
        p.P = qsrc->P;
        p.qk_mode = qsrc->qk_mode;
        p.eps = qsrc->eps;
        p.q_out = reinterpret_cast<_Float16 *>(qsrc->q_out);
        p.k_dst = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(k_pool));
        p.v_dst = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(v_pool));
    }
    if (k_new) {  // fused decode step: the pools are written too
        p.k_new = reinterpret_cast<const _Float16 *>(k_new);
        p.v_new = reinterpret_cast<const _Float16 *>(v_new);
        p.k_dst = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(k_pool));
        p.v_dst = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(v_pool));
    }
    // A grid of more than one round of the CUs runs longest sequences first (a launch of order_kernel fills the
    // order array in the library workspace): the longest workgroups otherwise tend to start in a late round and
    // finish alone.  Only with the library workspace, and not where it would have to grow under graph capture.
    const int64_t grid = (int64_t)num_seqs * pool.num_kv_heads * plan.num_splits;
    bool order = ws_kind != kCallerWs && num_seqs > 1 && num_seqs <= pkv::kOrderMaxSeqs && cu_count > 0 &&
                 grid > cu_count;
    // An ordered single pass also splits the longest sequences into pieces (pkv::PieceRule): fewer than
    // cu_count / Hkv extra records.
    bool pieces = order && plan.num_splits == 1 && window <= 0;
    const int64_t records = num_seqs + (cu_count + pool.num_kv_heads - 1) / pool.num_kv_heads;
    auto layout = [&]() {
        if (pieces)
            return ws_layout_pieces(num_seqs, num_q_heads, pool.num_kv_heads, pool.head_dim, records);
        return ws_layout(num_seqs, num_q_heads, pool.head_dim, plan.num_splits,
                         order ? (int64_t)num_seqs * pkv::kOrderRecord : 0);
    };
    WsLayout L = layout();
    if (pieces && ws_kind == kFixedWs && L.total > workspace_bytes) {
        pieces = false;  // the pieces' partials do not fit: whole sequences in order
        L = layout();
    }
    if (order && ws_kind == kFixedWs && L.total > workspace_bytes) {
        order = false;  // the records do not fit beside the partials: id order
        L = layout();
    }
    if (order && ws_kind == kLibraryWs && library_workspace_bytes(stream) < L.total) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamIsCapturing");
        if (cap != hipStreamCaptureStatusNone) {
            order = pieces = false;  // dispatch order is an optimisation: never worth a failed capture
            L = layout();
        }
    }
    if (plan.num_splits == 1 && !order) {
        if (pre_append) {
            hipError_t e = pkv::launch_append_newest(*pre_append, stream);
            if (e != hipSuccess)
                return hip_fail(e, "append kernel launch");
        }
        hipError_t e = pkv::launch_decode(p, num_seqs, pool.head_dim, pool.block_size, plan.waves_per_group, false,
                                          stream);
        if (e != hipSuccess)
            return hip_fail(e, "decode kernel launch");
        return ok();
    }
    void *ws = workspace;
    if (ws_kind == kLibraryWs) {
        int rc = library_workspace(L.total, stream, &ws);
        if (rc)
            return rc;
    } else if (ws_kind == kFixedWs) {
        if (L.total > workspace_bytes)
            return fail(PKV_EWORKSPACE, "the plan (%d splits, %d sequences) needs %zu bytes of split-K partials; the "
                        "fixed scratch of the no-allocation entry point holds %zu", plan.num_splits, num_seqs,
                        L.total, workspace_bytes);
    } else {
        if (!ws || workspace_bytes < L.total)
            return fail(PKV_EWORKSPACE, "workspace of %zu bytes at %p; the plan (%d splits) needs %zu",
                        workspace_bytes, ws, plan.num_splits, L.total);
        if (!aligned(ws, 256))
            return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
    }
    char *base = static_cast<char *>(ws);
    int32_t *ord = order ? reinterpret_cast<int32_t *>(base + L.order_off) : nullptr;
    pkv::PieceRule rule{};
    if (pieces) {
        rule.records = (int32_t)records;
        rule.cus = cu_count;
        rule.hkv = pool.num_kv_heads;
        rule.block_size = pool.block_size;
        rule.counters = reinterpret_cast<int32_t *>(base + L.count_off);
        p.order_records = rule.records;
        p.piece_count = rule.counters;
        p.part_o = reinterpret_cast<float *>(base + L.o_off);
        p.part_m = reinterpret_cast<float *>(base + L.m_off);
        p.part_l = reinterpret_cast<float *>(base + L.l_off);
    }
    if (pre_append) {  // the decode step's append launch, which also writes the order records
        pkv::AppendParams a = *pre_append;
        a.order = ord;
        a.order_cap = max_blocks_per_seq * pool.block_size;
        a.order_window = window;
        a.pieces = rule;
        hipError_t e = pkv::launch_append_newest(a, stream);
        if (e != hipSuccess)
            return hip_fail(e, "append kernel launch");
    } else if (ord) {
        hipError_t e = pkv::launch_order(context_lens, block_tables, num_seqs, max_blocks_per_seq,
                                         max_blocks_per_seq * pool.block_size, window, ord, rule, stream);
        if (e != hipSuccess)
            return hip_fail(e, "order kernel launch");
    }
    p.order = ord;
    if (plan.num_splits == 1) {
        hipError_t e = pkv::launch_decode(p, num_seqs, pool.head_dim, pool.block_size, plan.waves_per_group, false,
                                          stream);
        if (e != hipSuccess)
            return hip_fail(e, "decode kernel launch");
        return ok();
    }
    p.part_o = reinterpret_cast<float *>(base + L.o_off);
    p.part_m = reinterpret_cast<float *>(base + L.m_off);
    p.part_l = reinterpret_cast<float *>(base + L.l_off);
    p.num_splits = plan.num_splits;
    p.chunk_blocks = plan.chunk_blocks;
    hipError_t e = pkv::launch_decode(p, num_seqs, pool.head_dim, pool.block_size, plan.waves_per_group, true,
                                      stream);
    if (e != hipSuccess)
        return hip_fail(e, "split-K phase-1 kernel launch");
    pkv::CombineParams c;
    c.part_o = p.part_o;
    c.part_m = p.part_m;
    c.part_l = p.part_l;
    c.context_lens = context_lens;
    c.out = p.out;
    c.B = num_seqs;
    c.Hq = num_q_heads;
    c.BS = pool.block_size;
    c.M = max_blocks_per_seq;
    c.num_splits = plan.num_splits;
    c.chunk_blocks = plan.chunk_blocks;
    c.window = window;
    e = pkv::launch_combine(c, pool.head_dim, stream);
    if (e != hipSuccess)
        return hip_fail(e, "split-K combine kernel launch");
    return ok();
}

int decode_impl(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool, pkv_pool_desc pool,
                const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                int32_t num_seqs, int32_t num_q_heads, float scale, uint16_t *out, int32_t num_splits,
                int32_t max_context_hint, const pkv_decode_plan *given, void *workspace, size_t workspace_bytes,
                WsKind ws_kind, hipStream_t stream, const uint16_t *k_new = nullptr,
                const uint16_t *v_new = nullptr, int32_t window = 0, const QkvSource *qsrc = nullptr) {
    int rc = check_decode_geometry(num_seqs, num_q_heads, pool, max_blocks_per_seq);
    if (rc)
        return rc;
    if (window < 0)
        return fail(PKV_EINVAL, "window must be >= 0 (got %d)", window);
    if (window > 0 && (max_context_hint == 0 || max_context_hint > window))
        max_context_hint = window;  // the dispatcher sizes splits for at most `window` rows per sequence
    if (num_splits < 0)
        return fail(PKV_EINVAL, "num_splits must be >= 0 (got %d)", num_splits);
    if (!isfinite(scale))
        return fail(PKV_EINVAL, "scale must be finite");
    if (num_seqs == 0)
        return ok();
    rc = check_decode_pointers(q, k_pool, v_pool, block_tables, context_lens, out);
    if (rc)
        return rc;
    if (given && (rc = check_plan(*given, num_seqs, num_q_heads, pool, max_blocks_per_seq, -1)) != 0)
        return rc;  // every argument error is reported before the first device query
    DeviceFacts facts;
    rc = device_facts(&facts);
    if (rc)
        return rc;
    if (ws_kind == kFixedWs && workspace == nullptr) {
        rc = scratch_address(&workspace);  // once per device: the address of that device's copy of `scratch`
        if (rc)
            return rc;
    }
    pkv_decode_plan plan;
    if (given) {
        plan = *given;
        rc = check_plan(plan, num_seqs, num_q_heads, pool, max_blocks_per_seq, facts.lds_per_block);
    } else {
        rc = plan_decode(num_seqs, num_q_heads, pool.num_kv_heads, pool.head_dim, pool.block_size,
                         max_blocks_per_seq, max_context_hint, num_splits, facts.cu_count, facts.lds_per_block,
                         &plan);
    }
    if (rc)
        return rc;
    if (qsrc && (int64_t)num_seqs * pool.num_kv_heads * plan.num_splits > facts.cu_count) {
        // The step from QKV rows over more than one round of CUs: the QKV kernel (one new token per sequence, at
        // row L-1), then attention reading its q_out.
        pkv::QkvParams a;
        memset(&a, 0, sizeof a);
        a.qkv = reinterpret_cast<const _Float16 *>(qsrc->qkv);
        a.q_norm_w = reinterpret_cast<const _Float16 *>(qsrc->q_norm_w);
        a.k_norm_w = reinterpret_cast<const _Float16 *>(qsrc->k_norm_w);
        a.cos_t = qsrc->cos_t;
        a.sin_t = qsrc->sin_t;
        a.block_tables = block_tables;
        a.decode_lens = context_lens;
        a.B = a.T = num_seqs;
        a.Hq = num_q_heads;
        a.Hkv = pool.num_kv_heads;
        a.G = num_q_heads / pool.num_kv_heads;
        a.N = pool.num_blocks;
        a.M = max_blocks_per_seq;
        a.BS = pool.block_size;
        a.P = qsrc->P;
        a.qk_mode = qsrc->qk_mode;
        a.eps = qsrc->eps;
        a.hpp = a.G + 2;
        a.parts = 1;
        a.q_out = reinterpret_cast<_Float16 *>(qsrc->q_out);
        a.k_pool = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(k_pool));
        a.v_pool = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(v_pool));
        hipError_t e = pkv::launch_qkv_cache(a, pool.head_dim, stream);
        if (e != hipSuccess)
            return hip_fail(e, "qkv-to-cache kernel launch");
        q = qsrc->q_out;
        qsrc = nullptr;
    }
    if (k_new && (int64_t)num_seqs * pool.num_kv_heads * plan.num_splits > facts.cu_count) {
        // Decode step over more workgroups than one round of the device's CUs: the append kernel, then attention.
        // Writes issued from inside a long, read-saturated launch cost far more than a launch of their own.
        pkv::AppendParams a;
        memset(&a, 0, sizeof a);
        a.k = reinterpret_cast<const _Float16 *>(k_new);
        a.v = reinterpret_cast<const _Float16 *>(v_new);
        a.block_tables = block_tables;
        a.context_lens = context_lens;
        a.k_pool = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(k_pool));
        a.v_pool = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(v_pool));
        a.T = num_seqs;
        a.Hkv = pool.num_kv_heads;
        a.D = pool.head_dim;
        a.BS = pool.block_size;
        a.N = pool.num_blocks;
        a.M = max_blocks_per_seq;
        k_new = v_new = nullptr;
        // run_plan launches it first, with the dispatch-order records folded in when the grid is ordered
        return run_plan(plan, q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                        num_q_heads, scale, out, workspace, workspace_bytes, ws_kind, stream, facts.cu_count,
                        nullptr, nullptr, window, qsrc, &a);
    }
    return run_plan(plan, q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                    num_q_heads, scale, out, workspace, workspace_bytes, ws_kind, stream, facts.cu_count, k_new,
                    v_new, window, qsrc);
}

// Paged varlen attention (several new query rows per sequence): plan, checks, launches.
int varlen_impl(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool, pkv_pool_desc pool,
                const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q,
                const int32_t *pos_offsets, int32_t num_seqs, int32_t total_q, int32_t num_q_heads, float scale,
                uint16_t *out, int32_t num_splits, int32_t max_q_len, int32_t max_context_hint, hipStream_t stream,
                const uint16_t *k_new = nullptr, const uint16_t *v_new = nullptr) {
    int rc = check_decode_geometry(num_seqs, num_q_heads, pool, max_blocks_per_seq);
    if (rc)
        return rc;
    if (total_q < 0 || num_splits < 0 || max_q_len < 0 || max_context_hint < 0)
        return fail(PKV_EINVAL, "total_q_tokens, num_splits, max_q_len and max_context_hint must be >= 0 "
                    "(got %d, %d, %d, %d)", total_q, num_splits, max_q_len, max_context_hint);
    if (!isfinite(scale))
        return fail(PKV_EINVAL, "scale must be finite");
    if (num_seqs == 0 || total_q == 0)
        return ok();
    if (!q || !k_pool || !v_pool || !block_tables || !cu_seqlens_q || !pos_offsets || !out)
        return fail(PKV_EINVAL, "null device pointer (q=%p k_pool=%p v_pool=%p block_tables=%p cu_seqlens_q=%p "
                    "pos_offsets=%p out=%p)", q, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets, out);
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16))
        return fail(PKV_EINVAL, "q, k_pool, v_pool and out must be 16-byte aligned");
    if (!aligned(block_tables, 4) || !aligned(cu_seqlens_q, 4) || !aligned(pos_offsets, 4))
        return fail(PKV_EINVAL, "block_tables, cu_seqlens_q and pos_offsets must be 4-byte aligned");
    const bool step = k_new != nullptr || v_new != nullptr;
    if (step) {
        if (!k_new || !v_new)
            return fail(PKV_EINVAL, "null device pointer (k_new=%p v_new=%p)", k_new, v_new);
        if (!aligned(k_new, 16) || !aligned(v_new, 16))
            return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
        if (max_q_len < 1)
            return fail(PKV_EINVAL, "max_q_len must bound every sequence's new rows (>= 1, got %d)", max_q_len);
    }
    DeviceFacts facts;
    rc = device_facts(&facts);
    if (rc)
        return rc;
    const int G = num_q_heads / pool.num_kv_heads;
    const int R = 16 / G;
    const int64_t qmax = max_q_len > 0 && max_q_len < total_q ? max_q_len : total_q;
    // Two tiles per workgroup (one K/V stream for both) once a sequence can have more than one tile.
    const int QT = qmax > R ? 2 : 1;
    const int64_t tiles_per_seq = (qmax + QT * R - 1) / (QT * R);  // tile-group slots
    // workgroups that find work: at most one per QT * R new rows plus one partial group per sequence
    int64_t active = (int64_t)num_seqs * tiles_per_seq;
    const int64_t bound = ((int64_t)total_q + QT * R - 1) / (QT * R) + num_seqs;
    if (active > bound)
        active = bound;
    active *= pool.num_kv_heads;
    const int64_t cap = (int64_t)max_blocks_per_seq * pool.block_size;
    const int64_t lmax = max_context_hint > 0 && max_context_hint < cap ? max_context_hint : cap;
    const int64_t nbmax = (lmax + pool.block_size - 1) / pool.block_size;
    int S = num_splits;
    if (S == 0) {
        S = 1;
        const int64_t cu = facts.cu_count > 0 ? facts.cu_count : 256;
        if (nbmax > 8 && 2 * active < cu) {
            int64_t want = (cu + active - 1) / active;
            if (want > nbmax / 8)
                want = nbmax / 8;
            if (want > 64)
                want = 64;
            S = (int)(want < 1 ? 1 : want);
        }
    }
    if ((int64_t)num_seqs * tiles_per_seq * pool.num_kv_heads * S > INT32_MAX || S > 65535)
        return fail(PKV_EINVAL, "varlen grid (%d sequences x %lld tiles x %d kv heads x %d splits) is too large",
                    num_seqs, (long long)tiles_per_seq, pool.num_kv_heads, S);
    // The varlen step in one launch: one pass, at most kStepFusedRows new rows per sequence (the launch keeps
    // them in LDS), one tile per group at head dim 256 (two would spill), and no more workgroups than one round of
    // the CUs -- as for the decode step, writes issued from inside a long, read-saturated launch cost more than a
    // launch of their own.
    const bool fused = step && S == 1 && max_q_len <= pkv::kStepFusedRows && (QT == 1 || pool.head_dim <= 128) &&
                       (int64_t)num_seqs * tiles_per_seq * pool.num_kv_heads <= facts.cu_count;
    int waves = pkv::max_waves_per_group(pool.head_dim);
    const size_t limit = facts.lds_per_block > 0 ? (size_t)facts.lds_per_block : (size_t)65536;
    while (waves > 1 && pkv::varlen_lds_bytes(pool.head_dim, waves, fused) > limit)
        waves >>= 1;
    if (pkv::varlen_lds_bytes(pool.head_dim, waves, fused) > limit)
        return fail(PKV_EUNSUPPORTED, "varlen needs %zu LDS bytes, the device allows %zu",
                    pkv::varlen_lds_bytes(pool.head_dim, waves, fused), limit);
    pkv::VarlenParams p;
    memset(&p, 0, sizeof p);
    p.q = reinterpret_cast<const _Float16 *>(q);
    p.block_tables = block_tables;
    p.cu_seqlens_q = cu_seqlens_q;
    p.pos_offsets = pos_offsets;
    p.Hq = num_q_heads;
    p.Hkv = pool.num_kv_heads;
    p.G = G;
    p.N = pool.num_blocks;
    p.M = max_blocks_per_seq;
    p.T = total_q;
    p.R = R;
    p.QT = QT;
    p.tiles_per_seq = (int32_t)tiles_per_seq;
    p.num_splits = S;
    p.chunk_blocks = 0;
    p.scale_log2 = scale * 1.44269504088896340736f;
    p.k_pool = reinterpret_cast<const _Float16 *>(k_pool);
    p.v_pool = reinterpret_cast<const _Float16 *>(v_pool);
    p.out = reinterpret_cast<_Float16 *>(out);
    if (fused) {
        p.k_new = reinterpret_cast<const _Float16 *>(k_new);
        p.v_new = reinterpret_cast<const _Float16 *>(v_new);
        p.k_dst = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(k_pool));
        p.v_dst = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(v_pool));
    }
    // A grid of more than one round runs its sequences longest first, as in decode (the records live in the
    // library workspace; skipped where the workspace would have to grow under graph capture).
    const int64_t grid = (int64_t)num_seqs * tiles_per_seq * pool.num_kv_heads * S;
    bool order = !fused && num_seqs > 1 && num_seqs <= pkv::kOrderMaxSeqs && grid > facts.cu_count;
    WsLayout L = ws_layout(total_q, num_q_heads, pool.head_dim, S, order ? (int64_t)num_seqs * pkv::kOrderRecord : 0);
    if (order && library_workspace_bytes(stream) < L.total) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamIsCapturing");
        if (cap != hipStreamCaptureStatusNone) {
            order = false;
            L = ws_layout(total_q, num_q_heads, pool.head_dim, S);
        }
    }
    void *ws = nullptr;
    if (S > 1 || order) {
        rc = library_workspace(L.total, stream, &ws);
        if (rc)
            return rc;
    }
    char *base = static_cast<char *>(ws);
    int32_t *ord = order ? reinterpret_cast<int32_t *>(base + L.order_off) : nullptr;
    if (step && !fused) {
        // the new rows' own launch (which also writes the order records), then attention over the updated pools
        pkv::AppendParams a;
        memset(&a, 0, sizeof a);
        a.k = reinterpret_cast<const _Float16 *>(k_new);
        a.v = reinterpret_cast<const _Float16 *>(v_new);
        a.block_tables = block_tables;
        a.k_pool = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(k_pool));
        a.v_pool = reinterpret_cast<_Float16 *>(const_cast<uint16_t *>(v_pool));
        a.T = total_q;
        a.Hkv = pool.num_kv_heads;
        a.D = pool.head_dim;
        a.BS = pool.block_size;
        a.N = pool.num_blocks;
        a.M = max_blocks_per_seq;
        a.order = ord;
        a.order_cap = max_blocks_per_seq * pool.block_size;
        hipError_t e = pkv::launch_append_varlen(a, cu_seqlens_q, pos_offsets, num_seqs, (int)qmax, stream);
        if (e != hipSuccess)
            return hip_fail(e, "varlen append kernel launch");
    } else if (order) {
        hipError_t e = pkv::launch_order_varlen(cu_seqlens_q, pos_offsets, block_tables, num_seqs, max_blocks_per_seq,
                                                max_blocks_per_seq * pool.block_size, ord, stream);
        if (e != hipSuccess)
            return hip_fail(e, "varlen order kernel launch");
    }
    p.order = ord;
    if (S == 1) {
        hipError_t e = pkv::launch_varlen(p, num_seqs, pool.head_dim, pool.block_size, waves, false, stream);
        if (e != hipSuccess)
            return hip_fail(e, "varlen kernel launch");
        return ok();
    }
    p.part_o = reinterpret_cast<float *>(base + L.o_off);
    p.part_m = reinterpret_cast<float *>(base + L.m_off);
    p.part_l = reinterpret_cast<float *>(base + L.l_off);
    hipError_t e = pkv::launch_varlen(p, num_seqs, pool.head_dim, pool.block_size, waves, true, stream);
    if (e != hipSuccess)
        return hip_fail(e, "varlen split phase-1 kernel launch");
    pkv::CombineParams c;
    memset(&c, 0, sizeof c);
    c.part_o = p.part_o;
    c.part_m = p.part_m;
    c.part_l = p.part_l;
    c.context_lens = nullptr;  // every split of every row was written
    c.out = p.out;
    c.B = total_q;
    c.Hq = num_q_heads;
    c.BS = pool.block_size;
    c.M = max_blocks_per_seq;
    c.num_splits = S;
    c.chunk_blocks = 0;
    e = pkv::launch_combine(c, pool.head_dim, stream);
    if (e != hipSuccess)
        return hip_fail(e, "varlen combine kernel launch");
    return ok();
}

// Split QKV + q/k RMSNorm + RoPE + paged-cache write: checks and the launch.  varlen == false is the one-sequence
// form (no cu_seqlens_q / pos_offsets; rope_base / cache_base are host values, checked here).
int qkv_impl(const uint16_t *qkv, const uint16_t *q_norm_w, const uint16_t *k_norm_w, const float *cos_table,
             const float *sin_table, int32_t max_positions, uint16_t *q_out, uint16_t *k_pool, uint16_t *v_pool,
             pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
             const int32_t *cu_seqlens_q, const int32_t *pos_offsets, int32_t num_seqs, int32_t total_tokens,
             int32_t num_q_heads, bool varlen, int32_t rope_base, int32_t cache_base, float eps,
             int32_t qk_mode, hipStream_t stream) {
    int rc = check_pool(pool);
    if (rc)
        return rc;
    if (num_seqs < 0 || total_tokens < 0)
        return fail(PKV_EINVAL, "num_seqs and the token count must be >= 0 (got %d, %d)", num_seqs, total_tokens);
    if (num_q_heads <= 0 || num_q_heads % pool.num_kv_heads != 0)
        return fail(PKV_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", num_q_heads,
                    pool.num_kv_heads);
    const QkvSource src = {qkv, q_norm_w, k_norm_w, cos_table, sin_table, max_positions, qk_mode, eps, q_out};
    rc = check_qkv_source(src, pool.head_dim);
    if (rc)
        return rc;
    if (num_q_heads / pool.num_kv_heads > 16)
        return fail(PKV_EUNSUPPORTED, "group size %d > 16 query heads per kv head is not compiled",
                    num_q_heads / pool.num_kv_heads);
    if (pool.block_size % 16 != 0)
        return fail(PKV_EUNSUPPORTED, "block_size %d must be a multiple of 16", pool.block_size);
    if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * pool.block_size > INT32_MAX)
        return fail(PKV_EINVAL, "max_blocks_per_seq must be > 0 with max_blocks_per_seq * block_size in int32 "
                    "(got %d)", max_blocks_per_seq);
    if (!varlen) {
        if (rope_base < 0 || (int64_t)rope_base + total_tokens > max_positions)
            return fail(PKV_EINVAL, "positions %d .. %d + %d exceed the %d table rows", rope_base, rope_base,
                        total_tokens, max_positions);
        if (cache_base < 0 || (int64_t)cache_base + total_tokens > (int64_t)max_blocks_per_seq * pool.block_size)
            return fail(PKV_EINVAL, "cache rows %d .. %d + %d exceed the table capacity %lld", cache_base,
                        cache_base, total_tokens, (long long)max_blocks_per_seq * pool.block_size);
    }
    if (num_seqs == 0 || total_tokens == 0)
        return ok();
    rc = check_qkv_pointers(src);
    if (rc)
        return rc;
    if (!k_pool || !v_pool || !block_tables || (varlen && (!cu_seqlens_q || !pos_offsets)))
        return fail(PKV_EINVAL, "null device pointer (k_pool=%p v_pool=%p block_tables=%p cu_seqlens_q=%p "
                    "pos_offsets=%p)", k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets);
    if (!aligned(k_pool, 16) || !aligned(v_pool, 16))
        return fail(PKV_EINVAL, "k_pool and v_pool must be 16-byte aligned");
    if (!aligned(block_tables, 4) || (varlen && (!aligned(cu_seqlens_q, 4) || !aligned(pos_offsets, 4))))
        return fail(PKV_EINVAL, "block_tables, cu_seqlens_q and pos_offsets must be 4-byte aligned");
    if ((int64_t)total_tokens + 32 * (int64_t)num_seqs > INT32_MAX || pool.num_kv_heads * 18 > 65535)
        return fail(PKV_EINVAL, "total_tokens + 32 * num_seqs or num_kv_heads overflows the grid");
    if ((int64_t)total_tokens * (num_q_heads + 2 * pool.num_kv_heads) * pool.head_dim > INT32_MAX)
        return fail(PKV_EINVAL, "qkv holds more than 2^31 values");
    pkv::QkvParams p;
    memset(&p, 0, sizeof p);
    p.qkv = reinterpret_cast<const _Float16 *>(qkv);
    p.q_norm_w = reinterpret_cast<const _Float16 *>(q_norm_w);
    p.k_norm_w = reinterpret_cast<const _Float16 *>(k_norm_w);
    p.cos_t = cos_table;
    p.sin_t = sin_table;
    p.cu_seqlens_q = varlen ? cu_seqlens_q : nullptr;
    p.pos_offsets = varlen ? pos_offsets : nullptr;
    p.block_tables = block_tables;
    p.B = num_seqs;
    p.T = total_tokens;
    p.Hq = num_q_heads;
    p.Hkv = pool.num_kv_heads;
    p.G = num_q_heads / pool.num_kv_heads;
    p.N = pool.num_blocks;
    p.M = max_blocks_per_seq;
    p.BS = pool.block_size;
    p.P = max_positions;
    p.qk_mode = qk_mode;
    p.rope_base = rope_base;
    p.cache_base = cache_base;
    // Head slots per workgroup: all G + 2 of a kv head when units hold a row or two (decode), else two passes of
    // 256 threads over a full 16-row unit (hpp * 16 rows * head_dim/8 lanes <= 512; measured on a 2048-token
    // prefill chunk, Qwen3-8B heads: 16.2 us against 16.8-17.1 with four passes and 17.8 with two units a group).
    {
        const int G = p.G;
        const int cap = 512 / (2 * pool.head_dim);
        const bool decode_like = (int64_t)total_tokens <= 2 * (int64_t)num_seqs;
        int parts = decode_like ? 1 : (G + 2 + cap - 1) / cap;
        p.hpp = (G + 2 + parts - 1) / parts;
        p.parts = (G + 2 + p.hpp - 1) / p.hpp;
    }
    p.eps = eps;
    p.q_out = reinterpret_cast<_Float16 *>(q_out);
    p.k_pool = reinterpret_cast<_Float16 *>(k_pool);
    p.v_pool = reinterpret_cast<_Float16 *>(v_pool);
    hipError_t e = pkv::launch_qkv_cache(p, pool.head_dim, stream);
    if (e != hipSuccess)
        return hip_fail(e, "qkv-to-cache kernel launch");
    return ok();
}

}  // namespace

extern "C" {

int pkv_paged_kv_append(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping, int32_t num_tokens,
                        uint16_t *k_pool, uint16_t *v_pool, pkv_pool_desc pool, void *stream) {
    int rc = check_pool(pool);
    if (rc)
        return rc;
    if (num_tokens < 0)
        return fail(PKV_EINVAL, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (pool.head_dim % 32 != 0 || pool.block_size % 16 != 0)
        return fail(PKV_EUNSUPPORTED, "head_dim %d must be a multiple of 32 and block_size %d a multiple of 16",
                    pool.head_dim, pool.block_size);
    if (num_tokens == 0)
        return ok();
    if (!k || !v || !slot_mapping || !k_pool || !v_pool)
        return fail(PKV_EINVAL, "null device pointer (k=%p v=%p slot_mapping=%p k_pool=%p v_pool=%p)", k, v,
                    slot_mapping, k_pool, v_pool);
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 2) ||
        !aligned(slot_mapping, 4))
        return fail(PKV_EINVAL, "k, v and k_pool must be 16-byte aligned");
    if ((int64_t)num_tokens * pool.num_kv_heads * (pool.head_dim / 8) > (int64_t)INT32_MAX * 256)
        return fail(PKV_EINVAL, "append too large for one launch");
    pkv::AppendParams p;
    memset(&p, 0, sizeof p);
    p.k = reinterpret_cast<const _Float16 *>(k);
    p.v = reinterpret_cast<const _Float16 *>(v);
    p.slot_mapping = slot_mapping;
    p.k_pool = reinterpret_cast<_Float16 *>(k_pool);
    p.v_pool = reinterpret_cast<_Float16 *>(v_pool);
    p.T = num_tokens;
    p.Hkv = pool.num_kv_heads;
    p.D = pool.head_dim;
    p.BS = pool.block_size;
    p.N = pool.num_blocks;
    hipError_t e = pkv::launch_append(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "append kernel launch");
    return ok();
}

int pkv_paged_decode_attention(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                               pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                               uint16_t *out, int32_t num_splits, int32_t max_context_hint, void *stream) {
    return decode_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, out, num_splits, max_context_hint, nullptr, nullptr, 0, kLibraryWs,
                       static_cast<hipStream_t>(stream));
}

int pkv_paged_decode_attention_ws(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                  pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                                  uint16_t *out, int32_t num_splits, int32_t max_context_hint, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return decode_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, out, num_splits, max_context_hint, nullptr, workspace, workspace_bytes,
                       kCallerWs, static_cast<hipStream_t>(stream));
}

int pkv_paged_decode_attention_noalloc(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                       pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                       float scale, uint16_t *out, int32_t num_splits, int32_t max_context_hint,
                                       void *stream) {
    // the fixed array's address is looked up inside, once the arguments have passed their checks
    return decode_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, out, num_splits, max_context_hint, nullptr, nullptr,
                       (size_t)PKV_NOALLOC_SCRATCH_BYTES, kFixedWs, static_cast<hipStream_t>(stream));
}

int pkv_paged_decode_attention_planned(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                       pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                       float scale, uint16_t *out, const pkv_decode_plan *plan, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    if (!plan)
        return fail(PKV_EINVAL, "plan is null");
    return decode_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, out, 0, 0, plan, workspace, workspace_bytes,
                       workspace == nullptr ? kLibraryWs : kCallerWs,
                       static_cast<hipStream_t>(stream));
}

int pkv_paged_decode_step(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                          uint16_t *v_pool, pkv_pool_desc pool, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                          int32_t num_q_heads, float scale, uint16_t *out, int32_t num_splits,
                          int32_t max_context_hint, void *stream) {
    if (num_seqs > 0 && (!k_new || !v_new))
        return fail(PKV_EINVAL, "null device pointer (k_new=%p v_new=%p)", k_new, v_new);
    if (num_seqs > 0 && (!aligned(k_new, 16) || !aligned(v_new, 16)))
        return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
    return decode_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, out, num_splits, max_context_hint, nullptr, nullptr, 0, kLibraryWs,
                       static_cast<hipStream_t>(stream), k_new, v_new);
}

int pkv_paged_decode_step_window(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                                 uint16_t *v_pool, pkv_pool_desc pool, const int32_t *block_tables,
                                 int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, float scale, uint16_t *out, int32_t num_splits, int32_t window,
                                 int32_t max_context_hint, void *stream) {
    if (num_seqs > 0 && (!k_new || !v_new))
        return fail(PKV_EINVAL, "null device pointer (k_new=%p v_new=%p)", k_new, v_new);
    if (num_seqs > 0 && (!aligned(k_new, 16) || !aligned(v_new, 16)))
        return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
    return decode_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, out, num_splits, max_context_hint, nullptr, nullptr, 0, kLibraryWs,
                       static_cast<hipStream_t>(stream), k_new, v_new, window);
}

int pkv_plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_hint, int32_t num_splits,
                    int32_t cu_count, pkv_decode_plan *plan) {
    int lds = 0;
    if (cu_count <= 0) {
        DeviceFacts f;
        int rc = device_facts(&f);
        if (rc)
            return rc;
        cu_count = f.cu_count;
        lds = f.lds_per_block;
    }
    int rc = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                         max_context_hint, num_splits, cu_count, lds, plan);
    return rc ? rc : ok();
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t num_splits) {
    if (num_splits <= 1 || num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0)
        return 0;
    return ws_layout(num_seqs, num_q_heads, head_dim, num_splits).total;
}

int pkv_paged_decode_split_partials(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                    pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                    float scale, int32_t num_splits, int32_t chunk_blocks, float *partial_out,
                                    float *partial_m, float *partial_l, void *stream) {
    int rc = check_decode_geometry(num_seqs, num_q_heads, pool, max_blocks_per_seq);
    if (rc)
        return rc;
    if (num_splits < 1 || num_splits > 65535)
        return fail(PKV_EINVAL, "num_splits must be in [1, 65535] (got %d)", num_splits);
    if (chunk_blocks < 0)
        return fail(PKV_EINVAL, "chunk_blocks must be >= 0 (got %d)", chunk_blocks);
    if ((int64_t)num_seqs * pool.num_kv_heads * num_splits > INT32_MAX)
        return fail(PKV_EINVAL, "num_seqs * num_kv_heads * num_splits overflows the grid");
    if (chunk_blocks > 0 && (int64_t)num_splits * chunk_blocks < max_blocks_per_seq)
        return fail(PKV_EINVAL, "num_splits * chunk_blocks (%d * %d) does not cover max_blocks_per_seq %d",
                    num_splits, chunk_blocks, max_blocks_per_seq);
    if (!isfinite(scale))
        return fail(PKV_EINVAL, "scale must be finite");
    if (num_seqs == 0)
        return ok();
    rc = check_decode_pointers(q, k_pool, v_pool, block_tables, context_lens, q);
    if (rc)
        return rc;
    if (!partial_out || !partial_m || !partial_l || !aligned(partial_out, 16) || !aligned(partial_m, 4) ||
        !aligned(partial_l, 4))
        return fail(PKV_EINVAL, "partial buffers must be non-null (partial_out 16-byte aligned)");
    DeviceFacts facts;
    rc = device_facts(&facts);
    if (rc)
        return rc;
    pkv_decode_plan plan;
    rc = plan_decode(num_seqs, num_q_heads, pool.num_kv_heads, pool.head_dim, pool.block_size, max_blocks_per_seq,
                     0, num_splits > 1 ? num_splits : 2, facts.cu_count, facts.lds_per_block, &plan);
    if (rc)
        return rc;
    pkv::DecodeParams p = decode_params(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens,
                                        num_q_heads, scale);
    p.part_o = partial_out;
    p.part_m = partial_m;
    p.part_l = partial_l;
    p.num_splits = num_splits;
    p.chunk_blocks = chunk_blocks;
    hipError_t e = pkv::launch_decode(p, num_seqs, pool.head_dim, pool.block_size, plan.waves_per_group, true,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "split-K phase-1 kernel launch");
    return ok();
}

int pkv_paged_decode_split_combine(const float *partial_out, const float *partial_m, const float *partial_l,
                                   const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                   int32_t num_splits, int32_t chunk_blocks, uint16_t *out, void *stream) {
    if (num_seqs < 0 || num_q_heads <= 0 || block_size <= 0 || max_blocks_per_seq <= 0)
        return fail(PKV_EINVAL, "bad geometry (num_seqs=%d Hq=%d BS=%d M=%d)", num_seqs, num_q_heads, block_size,
                    max_blocks_per_seq);
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return fail(PKV_EUNSUPPORTED, "head_dim %d not compiled (64|128|256)", head_dim);
    if (num_splits < 1 || chunk_blocks < 0)
        return fail(PKV_EINVAL, "num_splits must be >= 1 and chunk_blocks >= 0");
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX || (int64_t)num_seqs * num_q_heads > INT32_MAX)
        return fail(PKV_EINVAL, "geometry overflows int32");
    if (num_seqs == 0)
        return ok();
    if (!partial_out || !partial_m || !partial_l || !context_lens || !out)
        return fail(PKV_EINVAL, "null device pointer");
    if (!aligned(out, 2) || !aligned(partial_out, 4))
        return fail(PKV_EINVAL, "misaligned buffer");
    pkv::CombineParams c;
    c.part_o = partial_out;
    c.part_m = partial_m;
    c.part_l = partial_l;
    c.context_lens = context_lens;
    c.out = reinterpret_cast<_Float16 *>(out);
    c.B = num_seqs;
    c.Hq = num_q_heads;
    c.BS = block_size;
    c.M = max_blocks_per_seq;
    c.num_splits = num_splits;
    c.chunk_blocks = chunk_blocks;
    hipError_t e = pkv::launch_combine(c, head_dim, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "split-K combine kernel launch");
    return ok();
}

int pkv_split_qkv_norm_rope_into_paged_cache_varlen(const uint16_t *qkv, const uint16_t *q_norm_w,
                                                    const uint16_t *k_norm_w, const float *cos_table,
                                                    const float *sin_table, int32_t max_positions, uint16_t *q_out,
                                                    uint16_t *k_pool, uint16_t *v_pool, pkv_pool_desc pool,
                                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                                    const int32_t *cu_seqlens_q, const int32_t *pos_offsets,
                                                    int32_t num_seqs, int32_t total_tokens, int32_t num_q_heads,
                                                    float eps, int32_t qk_mode, void *stream) {
    return qkv_impl(qkv, q_norm_w, k_norm_w, cos_table, sin_table, max_positions, q_out, k_pool, v_pool, pool,
                    block_tables, max_blocks_per_seq, cu_seqlens_q, pos_offsets, num_seqs, total_tokens,
                    num_q_heads, true, 0, 0, eps, qk_mode, static_cast<hipStream_t>(stream));
}

int pkv_split_qkv_norm_rope_into_paged_cache(const uint16_t *qkv, const uint16_t *q_norm_w, const uint16_t *k_norm_w,
                                             const float *cos_table, const float *sin_table, int32_t max_positions,
                                             uint16_t *q_out, uint16_t *k_pool, uint16_t *v_pool,
                                             pkv_pool_desc pool, const int32_t *block_table,
                                             int32_t max_blocks_per_seq, int32_t num_tokens, int32_t num_q_heads,
                                             int32_t pos_offset, int32_t cache_len, float eps, int32_t qk_mode,
                                             void *stream) {
    return qkv_impl(qkv, q_norm_w, k_norm_w, cos_table, sin_table, max_positions, q_out, k_pool, v_pool, pool,
                    block_table, max_blocks_per_seq, nullptr, nullptr, 1, num_tokens, num_q_heads, false,
                    pos_offset, cache_len, eps, qk_mode, static_cast<hipStream_t>(stream));
}

int pkv_paged_decode_step_qkv(const uint16_t *qkv, const uint16_t *q_norm_w, const uint16_t *k_norm_w,
                              const float *cos_table, const float *sin_table, int32_t max_positions, float eps,
                              int32_t qk_mode, uint16_t *q_out, uint16_t *k_pool, uint16_t *v_pool,
                              pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                              const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                              uint16_t *out, int32_t num_splits, int32_t max_context_hint, void *stream) {
    const QkvSource src = {qkv, q_norm_w, k_norm_w, cos_table, sin_table, max_positions, qk_mode, eps, q_out};
    int rc = check_pool(pool);
    if (rc)
        return rc;
    rc = check_qkv_source(src, pool.head_dim);
    if (rc)
        return rc;
    if (num_seqs > 0) {
        rc = check_qkv_pointers(src);
        if (rc)
            return rc;
    }
    return decode_impl(q_out, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, out, num_splits, max_context_hint, nullptr, nullptr, 0, kLibraryWs,
                       static_cast<hipStream_t>(stream), nullptr, nullptr, 0, &src);
}

// ---------------------------------------------------------------------------
// cold-path input checks

static int check_common(const pkv_pool_desc &pool, int32_t *report) {
    int rc = check_pool(pool);
    if (rc)
        return rc;
    if (!report || !aligned(report, 4))
        return fail(PKV_EINVAL, "report must be a 4-byte aligned device array of 4 int32");
    if (pool.block_size % 16 != 0)
        return fail(PKV_EUNSUPPORTED, "block_size %d must be a multiple of 16", pool.block_size);
    return PKV_OK;
}

static int run_check(const pkv::CheckParams &c, hipStream_t stream) {
    hipError_t e = pkv::launch_check(c, stream);
    if (e != hipSuccess)
        return hip_fail(e, "input check kernel launch");
    return ok();
}

int pkv_check_decode_inputs(const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t num_seqs, pkv_pool_desc pool, int32_t window, int32_t *report, void *stream) {
    int rc = check_common(pool, report);
    if (rc)
        return rc;
    if (num_seqs < 0 || max_blocks_per_seq <= 0 || window < 0 ||
        (int64_t)max_blocks_per_seq * pool.block_size > INT32_MAX)
        return fail(PKV_EINVAL, "num_seqs and window must be >= 0 and max_blocks_per_seq > 0 (got %d, %d, %d)",
                    num_seqs, window, max_blocks_per_seq);
    if (num_seqs > 0 && (!block_tables || !context_lens || !aligned(block_tables, 4) || !aligned(context_lens, 4)))
        return fail(PKV_EINVAL, "block_tables and context_lens must be non-null, 4-byte aligned device arrays");
    pkv::CheckParams c;
    memset(&c, 0, sizeof c);
    c.block_tables = block_tables;
    c.context_lens = context_lens;
    c.B = num_seqs;
    c.M = max_blocks_per_seq;
    c.N = pool.num_blocks;
    c.BS = pool.block_size;
    c.window = window;
    c.report = report;
    return run_check(c, static_cast<hipStream_t>(stream));
}

int pkv_check_varlen_inputs(const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q,
                            const int32_t *pos_offsets, int32_t num_seqs, int32_t total_q_tokens, pkv_pool_desc pool,
                            int32_t *report, void *stream) {
    int rc = check_common(pool, report);
    if (rc)
        return rc;
    if (num_seqs < 0 || total_q_tokens < 0 || max_blocks_per_seq <= 0 ||
        (int64_t)max_blocks_per_seq * pool.block_size > INT32_MAX)
        return fail(PKV_EINVAL, "num_seqs and total_q_tokens must be >= 0 and max_blocks_per_seq > 0 (got %d, %d, %d)",
                    num_seqs, total_q_tokens, max_blocks_per_seq);
    if (num_seqs > 0 && (!block_tables || !cu_seqlens_q || !pos_offsets || !aligned(block_tables, 4) ||
                         !aligned(cu_seqlens_q, 4) || !aligned(pos_offsets, 4)))
        return fail(PKV_EINVAL, "block_tables, cu_seqlens_q and pos_offsets must be non-null, 4-byte aligned device "
                    "arrays");
    pkv::CheckParams c;
    memset(&c, 0, sizeof c);
    c.block_tables = block_tables;
    c.cu_seqlens_q = cu_seqlens_q;
    c.pos_offsets = pos_offsets;
    c.B = num_seqs;
    c.T = total_q_tokens;
    c.M = max_blocks_per_seq;
    c.N = pool.num_blocks;
    c.BS = pool.block_size;
    c.report = report;
    return run_check(c, static_cast<hipStream_t>(stream));
}

int pkv_check_slot_mapping(const int32_t *slot_mapping, int32_t num_tokens, pkv_pool_desc pool, int32_t *report,
                           void *stream) {
    int rc = check_common(pool, report);
    if (rc)
        return rc;
    if (num_tokens < 0)
        return fail(PKV_EINVAL, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (num_tokens > 0 && (!slot_mapping || !aligned(slot_mapping, 4)))
        return fail(PKV_EINVAL, "slot_mapping must be a non-null, 4-byte aligned device array");
    pkv::CheckParams c;
    memset(&c, 0, sizeof c);
    c.slot_mapping = slot_mapping ? slot_mapping : reinterpret_cast<const int32_t *>(report);  // marks the mode
    c.T = num_tokens;
    c.N = pool.num_blocks;
    c.BS = pool.block_size;
    c.report = report;
    return run_check(c, static_cast<hipStream_t>(stream));
}

int pkv_device_cu_count(int32_t *cu_count) {
    if (!cu_count)
        return fail(PKV_EINVAL, "cu_count is null");
    DeviceFacts f;
    int rc = device_facts(&f);
    if (rc)
        return rc;
    *cu_count = f.cu_count;
    return ok();
}

const char *pkv_last_error(void) { return g_error; }

const char *pkv_version(void) { return "pkv 0.1.0 (gfx950)"; }

int pkv_paged_decode_attention_window(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                      pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                      float scale, uint16_t *out, int32_t num_splits, int32_t window,
                                      int32_t max_context_hint, void *stream) {
    return decode_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, scale, out, num_splits, max_context_hint, nullptr, nullptr, 0, kLibraryWs,
                       static_cast<hipStream_t>(stream), nullptr, nullptr, window);
}

int pkv_paged_varlen_attention(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                               pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *cu_seqlens_q, const int32_t *pos_offsets, int32_t num_seqs,
                               int32_t total_q_tokens, int32_t num_q_heads, float scale, uint16_t *out,
                               int32_t num_splits, int32_t max_q_len, int32_t max_context_hint, void *stream) {
    return varlen_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, cu_seqlens_q, pos_offsets, num_seqs,
                       total_q_tokens, num_q_heads, scale, out, num_splits, max_q_len, max_context_hint,
                       static_cast<hipStream_t>(stream));
}

int pkv_paged_varlen_step(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                          uint16_t *v_pool, pkv_pool_desc pool, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q, const int32_t *pos_offsets,
                          int32_t num_seqs, int32_t total_q_tokens, int32_t num_q_heads, float scale, uint16_t *out,
                          int32_t num_splits, int32_t max_q_len, int32_t max_context_hint, void *stream) {
    if (num_seqs > 0 && total_q_tokens > 0 && (!k_new || !v_new))
        return fail(PKV_EINVAL, "null device pointer (k_new=%p v_new=%p)", k_new, v_new);
    return varlen_impl(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq, cu_seqlens_q, pos_offsets, num_seqs,
                       total_q_tokens, num_q_heads, scale, out, num_splits, max_q_len, max_context_hint,
                       static_cast<hipStream_t>(stream), k_new, v_new);
}

}  // extern "C"

