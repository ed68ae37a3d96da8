// pkv_qkv.hip -- gfx950 kernel of the step that feeds paged attention: split the fused QKV projection rows,
// RMS-normalise the query and key heads, rotate them (RoPE), and leave q in q_out and the new K/V rows in the
// paged cache.
// [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: split_qkv_norm_rope_into_paged_cache (one sequence) and
// split_qkv_norm_rope_into_paged_cache_varlen (cu_seqlens_q / pos_offsets); ferrum-kernels 0.7.1, cuda.rs:
// qk_norm_rope]
//
// Per token (sequence s, i-th new token, RoPE position p = pos + i, cache row r = cache + i), for every head of the
// row qkv[token] = [Hq query heads | Hkv key heads | Hkv value heads] x D:
//   query/key head: x <- x / sqrt(mean(x^2) + eps) * w   (qk_mode 1; w = q_norm_w or k_norm_w)
//                   (x_j, x_{j+D/2}) <- (x_j c - x_{j+D/2} s, x_{j+D/2} c + x_j s),  c, s = cos_t[p][j], sin_t[p][j]
//   query head  -> q_out[token][head]; key head -> K row r; value head -> V row r (copied).
// f32 arithmetic, each output rounded once to fp16 (nearest even).
//
// Work decomposition (MI355X-first: the pool's 16-row panels are written whole):
//   * one workgroup per (16-row cache unit holding new rows, kv head h, part).  The grid's x runs over unit slots, at
//     least floor(n_s / 16) + 2 of them per sequence (enough for the units its n_s new rows touch, wherever the
//     first starts); a slot finds its sequence by a wave-wide search of the prefix sums, and slots past a
//     sequence's last unit return at once.  The unit's head slots of kv head h (its G query heads, key head h,
//     value head h) are split over `parts` workgroups of `hpp` slots each (the host picks them: one part when
//     units hold a row or two, as in decode; parts of two passes of 256 threads each when units are full), the
//     part holding K and V dispatched first; items are (new row, head slot) pairs.  Every load of the unit is
//     issued before the first wait (the norm weights, the unit's rows of the cos/sin tables, each thread's qkv
//     pieces of the first two passes, the old panels of a partly written unit);
//   * a head row is D/8 lanes; lane l holds dims 4l .. 4l+3 and D/2 + 4l .. +3, so each RoPE pair (j, j + D/2)
//     lives in one lane.  The sum of squares is reduced across the group's lanes on the VALU (DPP row rotations,
//     and a v_permlane16_swap for 32-lane groups);
//   * q goes straight to q_out (8-byte stores, coalesced per half head row).  The unit's new K and V rows are
//     staged in LDS row-major (padded rows); each thread then writes 16-byte chunks of the panels (each put in its
//     panel order on the way): the new rows' K runs (64 bytes per row and 32-dim piece), and the V quads of 4 rows
//     that hold new rows, whole 128-byte lines whose old rows come from the quad as loaded at the start (so that
//     load overlaps everything else).  The pools thus see whole sectors and lines only -- scattered 2-byte V stores
//     cost far more at the memory than their bytes -- and nothing that holds no new row is rewritten;
//   * decode mode (decode_lens set): slot g is sequence g, whose one new token sits at row decode_lens[g] - 1 --
//     the QKV half of the decode step from QKV rows when it runs as two launches.
//
// The other rows of a quad that holds new rows are rewritten with their own values: no other work may write the
// panel meanwhile (the block holding a sequence's new rows belongs to that sequence alone).
//
// All HIP code here is built with packed-fp32 instructions disabled.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_internal.h"
#include "pkv_lanes.h"
#include "pkv_unit.h"

namespace pkv {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBatch = 2;  // passes whose qkv pieces are loaded together (1 and 4 measured slower)

// Sequence s's unit slots are [V_s / 16, V_{s+1} / 16) with V_s = cu[s] + 32 s: at least floor(n_s / 16) + 2 slots
// for its n_s new rows, enough for the 16-row cache units they touch wherever the first one starts.  The slot
// count is (T + 32 B) / 16, a host value, and a slot finds its sequence without a table.
__device__ __forceinline__ int slot_key(const int32_t *cu, int s) { return cu[s] + 32 * s; }

// The sequence of unit slot g -- the last s in [0, B] with slot_key(s) <= 16 g + 15 -- with its first token, new
// token count and first position.  The 64 lanes of the wave test 64 evenly spaced candidates per round; with
// B < 64 one round holds every candidate (SlotKeys) and the answer's neighbours come from lane exchanges.  Keys increase, so the lanes that pass are a prefix; with malformed prefix
// sums s still lies in [0, B].
struct SeqOfSlot {
    int s, first, n, pos;
};

struct SlotKeys {
    int c, q;  // lane l: cu[l] (l <= B) and pos[l]
};

__device__ __forceinline__ SlotKeys load_slot_keys(const int32_t *cu, const int32_t *pos, int B) {
    const int lane = threadIdx.x & 63;
    return SlotKeys{cu[lane <= B ? lane : B], pos[lane < B ? lane : B - 1]};
}

__device__ __forceinline__ SeqOfSlot lookup_slot(const SlotKeys &key, int B, int g) {  // B < 64
    const int lane = threadIdx.x & 63;
    const bool pass = lane <= B && key.c + 32 * lane <= 16 * g + 15;
    int k = __popcll(__ballot(pass)) - 1;
    k = k > 0 ? k : 0;
    SeqOfSlot r;
    r.s = k;
    r.first = __shfl(key.c, k, 64);
    r.n = __shfl(key.c, k + 1 <= B ? k + 1 : B, 64) - r.first;
    r.pos = __shfl(key.q, k < B ? k : B - 1, 64);
    return r;
}

__device__ __forceinline__ SeqOfSlot search_slot(const int32_t *cu, const int32_t *pos, int B, int g) {  // any B
    const int lane = threadIdx.x & 63;
    const int target = 16 * g + 15;
    int lo = 0, hi = B;
    while (lo < hi) {
        const int stride = (hi - lo + 64) / 64;
        const int idx = lo + lane * stride;
        const bool pass = idx <= hi && slot_key(cu, idx) <= target;
        const int k = __popcll(__ballot(pass)) - 1;
        lo += (k > 0 ? k : 0) * stride;
        hi = min(hi, lo + stride - 1);
    }
    SeqOfSlot r{lo, 0, 0, 0};
    if (lo < B) {
        r.first = cu[lo];
        r.n = cu[lo + 1] - r.first;
        r.pos = pos[lo];
    }
    return r;
}

// One 16-row cache unit of a workgroup: new rows r0 .. r0 + rows - 1 (rows == 0: the slot has nothing to write),
// of sequence s, token m0 first; lo is the cache row of row r0 in the sequence and rp0 its RoPE position.
struct Unit {
    int s, r0, rows, m0;
    int64_t lo, rp0;
};

// The j-th unit slot of sequence s (first token `first`, n new tokens, the first of them at RoPE position rope0 and
// cache row cache0): its unit and the new rows in it, or rows == 0 when the slot lies past the sequence's units or
// its tokens or positions fall outside the arrays (malformed prefix sums, positions outside the tables: those
// tokens are not written).
__device__ __forceinline__ Unit unit_of_slot(const QkvParams &p, int s, int first, int n, int rope0, int cache0,
                                             int j) {
    Unit un{s, 0, 0, 0, 0, 0};
    const int64_t u = (int64_t)(cache0 >> 4) + j;
    const int64_t lo = max((int64_t)cache0, 16 * u);
    const int64_t hi = min((int64_t)cache0 + n, 16 * u + 16);
    if (j < 0 || lo >= hi)
        return un;
    const int i0 = (int)(lo - cache0);  // index of row r0 among the sequence's new tokens
    const int m0 = first + i0;
    int rows = (int)(hi - lo);
    rows = rows < p.T - m0 ? rows : p.T - m0;
    const int64_t rp0 = (int64_t)rope0 + i0;
    if (m0 < 0 || rows <= 0 || rp0 < 0 || rp0 + rows > p.P)
        return un;
    un.r0 = (int)(lo - 16 * u);
    un.rows = rows;
    un.m0 = m0;
    un.lo = lo;
    un.rp0 = rp0;
    return un;
}

// The same values in every lane (they come from wave-wide searches), made scalar so that the buffer resources
// built from them stay in scalar registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni(int64_t x) {
    return (int64_t)(((uint64_t)(uint32_t)uni((int)(x >> 32)) << 32) | (uint32_t)uni((int)x));
}
__device__ __forceinline__ Unit uniform(const Unit &u) {
    return Unit{uni(u.s), uni(u.r0), uni(u.rows), uni(u.m0), uni(u.lo), uni(u.rp0)};
}

template <int D>
__global__ __launch_bounds__(kThreads) void qkv_cache_kernel(QkvParams p) {
    constexpr int LPR = D / 8;       // lanes per head row, 8 dims each
    constexpr int HALF = D / 2;
    constexpr int CHUNKS = 2 * D;    // 16-byte chunks of one 16-row panel (16 * D halves)
    constexpr int CPT = (CHUNKS + kThreads - 1) / kThreads;
    constexpr int TAB = 16 * HALF / 4;  // float4 chunks of 16 rows of one table
    constexpr int TPT = (TAB + kThreads - 1) / kThreads;  // chunks of each table per thread
    constexpr int VS = D + 4;  // row stride of the V staging (the pad spreads a dim's 16 rows over distinct banks)
    constexpr int KS = D + 8;  // row stride of the K staging (16-byte chunks of 16 rows read back together)
    __shared__ __attribute__((aligned(16))) _Float16 sk[16 * KS];  // new K rows, row-major [16][D + 8]
    __shared__ __attribute__((aligned(16))) _Float16 sv[16 * VS];  // new V rows, row-major [16][D + 4]
    __shared__ __attribute__((aligned(16))) float scos[16 * HALF];  // the unit's rows of the tables
    __shared__ __attribute__((aligned(16))) float ssin[16 * HALF];
    __shared__ __attribute__((aligned(16))) _Float16 sw[2 * D];     // q_norm_w, k_norm_w
    typedef float f4 __attribute__((ext_vector_type(4)));

    // (kv head, part): the part holding K and V, the heaviest, is dispatched first, so that the workgroups that
    // wait for a free slot are light ones
    const int yy = (int)gridDim.y - 1 - (int)blockIdx.y;
    const int part = yy / p.Hkv;  // which of the kv head's head slots (G query heads, K, V) this group does
    const int h = yy - part * p.Hkv;
    // head slots [hs0, hs1) of kv head h: < G query heads, G the key head, G + 1 the value head
    const int hs0 = part * p.hpp;
    const int hs1 = min(hs0 + p.hpp, p.G + 2);
    const int nh = hs1 - hs0;
    const bool has_k = hs0 <= p.G && p.G < hs1;
    const bool has_v = hs1 == p.G + 2;
    const bool rotates = hs0 <= p.G;  // the group holds a query or key head
    const int tid = threadIdx.x;
    const int width = (p.Hq + 2 * p.Hkv) * D;

    // Every load is a buffer load whose resource bounds the bytes it may touch: a lane with nothing to load passes
    // an offset past the bound and gets zeros without a memory access, so no load sits under a branch and all of
    // them are in flight before the first wait.  (With per-lane branches the compiler waited for each load where
    // its value left the branch: the block id, then each table chunk, then each qkv piece, a chain of round trips
    // before the unit's data was all requested.)
    constexpr uint32_t kPast = 0x7ffffff0u;  // an offset past every bound below
    auto rsrc = [](const void *base, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kRsrcWord3);
    };
    // the norm weights first: they depend on nothing
    const int w_bytes = rotates && p.qk_mode == 1 ? 2 * D : 0;
    const h8 wq = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(
                                             rsrc(p.q_norm_w, w_bytes), tid < LPR ? (uint32_t)(16 * tid) : kPast, 0, 0));
    const h8 wk = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(
                                             rsrc(p.k_norm_w, w_bytes),
                                             tid >= LPR && tid < 2 * LPR ? (uint32_t)(16 * (tid - LPR)) : kPast, 0, 0));

    // this slot's unit
    const int g = (int)blockIdx.x;
    Unit w;
    if (p.decode_lens) {
        // one new token per sequence: slot g is sequence g, its row at position L - 1
        const int L = p.decode_lens[g];
        w = unit_of_slot(p, g, g, L > 0 ? 1 : 0, L - 1, L - 1, 0);
    } else {
        SeqOfSlot q{0, 0, p.T, p.rope_base};
        int cache0 = p.cache_base;
        if (p.cu_seqlens_q) {
            q = p.B < 64 ? lookup_slot(load_slot_keys(p.cu_seqlens_q, p.pos_offsets, p.B), p.B, g)
                         : search_slot(p.cu_seqlens_q, p.pos_offsets, p.B, g);
            cache0 = q.pos;
            q.n = q.s < p.B ? q.n : 0;
        }
        w = unit_of_slot(p, q.s, q.first, q.n, q.pos, cache0, g - ((q.first + 32 * q.s) >> 4));
    }
    w = uniform(w);
    if (w.rows <= 0)
        return;  // (wave-uniform, and the same in every wave of the group)
    const bool whole = w.r0 == 0 && w.rows == 16;
    const int lanes = w.rows * nh * LPR;

    // the unit's block id: a scalar load (its wait never holds back the vector loads), used once they are in flight
    const bool in_table = (has_k || has_v) && w.lo >= 0 && w.lo < (int64_t)p.M * p.BS;
    const int blk = in_table ? uniform_load(p.block_tables, (int64_t)w.s * p.M + w.lo / p.BS) : -1;
    // the unit's rows of the cos/sin tables (LDS copies below), before its qkv pieces, so that the copies and the
    // barrier after them wait for the older loads only
    const int tab_bytes = rotates ? w.rows * HALF * 4 : 0;
    const __amdgpu_buffer_rsrc_t cos_r = rsrc(p.cos_t + w.rp0 * HALF, tab_bytes);
    const __amdgpu_buffer_rsrc_t sin_r = rsrc(p.sin_t + w.rp0 * HALF, tab_bytes);
    f4 cv[TPT], sv4[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int t = tid + kThreads * i;  // float4 t of the unit's 16 table rows
        const uint32_t off = t < TAB ? (uint32_t)(16 * t) : kPast;
        cv[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(cos_r, off, 0, 0));
        sv4[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(sin_r, off, 0, 0));
    }
    // this thread's qkv pieces: rows m0 .. m0 + rows - 1 of qkv
    const __amdgpu_buffer_rsrc_t qkv_r = rsrc(p.qkv + (int64_t)w.m0 * width, w.rows * width * 2);
    auto source = [&](int idx, int &rr, int &hs, int &piece) {
        const int item = idx / LPR;
        piece = idx - item * LPR;
        rr = item / nh;
        hs = hs0 + (item - rr * nh);
    };
    // lane `piece` of a head row holds dims 4 piece .. +4 and D/2 + 4 piece .. +4: each RoPE pair in one lane
    auto fetch = [&](int idx) {
        int rr, hs, piece;
        source(idx, rr, hs, piece);
        const int head = hs < p.G ? h * p.G + hs : (hs == p.G ? p.Hq + h : p.Hq + p.Hkv + h);
        const uint32_t off = idx < lanes ? (uint32_t)(2 * (rr * width + head * D + 4 * piece)) : kPast;
        // the QKV rows are read once: non-temporal, as the attention kernels stream K and V (r2: 15.16 -> 14.61 us)
        const h4 a = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(qkv_r, off, 0, kKvLoadPolicy));
        const h4 b = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(qkv_r, off, 2 * HALF,
                                                                                 kKvLoadPolicy));
        return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    };
    h8 raw[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
        raw[b] = fetch(b * kThreads + tid);
    // the old panels, once the block id is in (rows outside [r0, r0 + rows) are written back unchanged)
    int64_t panel = -1;  // the unit's panel (element offset of its first half) in both pools
    if (in_table && blk >= 0 && blk < p.N)
        panel = (((int64_t)blk * p.Hkv + h) * p.BS + ((int)w.lo % p.BS - w.r0)) * D;
    // Only the new rows are written: their K runs, and the V quads (4 rows, whole 128-byte lines) that hold them; a
    // quad that also holds old rows is read here and written back with those unchanged.
    const bool keep_old = panel >= 0 && !whole;
    auto quad_new = [&](int q) {  // V chunk q's quad of rows holds a new row
        const int vr = 4 * (q / (D / 2));
        return vr + 3 >= w.r0 && vr < w.r0 + w.rows;
    };
    const __amdgpu_buffer_rsrc_t ov_r = rsrc(keep_old ? p.v_pool + panel : p.v_pool, keep_old && has_v ? 32 * D : 0);
    h8 ov[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int q = tid + kThreads * c;
        const uint32_t off = q < CHUNKS && quad_new(q) ? (uint32_t)(16 * q) : kPast;
        ov[c] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(ov_r, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int t = tid + kThreads * i;
        if (rotates && t < TAB) {
            *reinterpret_cast<f4 *>(scos + 4 * t) = cv[i];
            *reinterpret_cast<f4 *>(ssin + 4 * t) = sv4[i];
        }
    }
    if (rotates && p.qk_mode == 1 && tid < 2 * LPR)
        *reinterpret_cast<h8 *>(sw + 8 * tid) = tid < LPR ? wq : wk;
    __syncthreads();

    const float inv_d = 1.0f / (float)D;
    for (int base = 0; base < lanes; base += kBatch * kThreads) {
        if (base > 0) {
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                raw[b] = fetch(base + b * kThreads + tid);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int idx = base + b * kThreads + tid;
            if (idx >= lanes)
                break;  // lanes below `lanes` form whole head-row groups, so every group sum has all its lanes
            int rr, hs, piece;
            source(idx, rr, hs, piece);
            const int rin = w.r0 + rr;
            if (hs > p.G) {
                // value head: staged row-major, put into the panel's quad order on the way out
                const h8 v = raw[b];
                *reinterpret_cast<h4 *>(sv + rin * VS + 4 * piece) = h4{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<h4 *>(sv + rin * VS + HALF + 4 * piece) = h4{v[4], v[5], v[6], v[7]};
                continue;
            }
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = (float)raw[b][e];
            if (p.qk_mode == 1) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ss += x[e] * x[e];
                const float r = rsqrtf(lanes_sum<LPR>(ss) * inv_d + p.eps);
                const _Float16 *wp = sw + (hs < p.G ? 0 : D) + 4 * piece;
                const h4 wa = *reinterpret_cast<const h4 *>(wp);
                const h4 wb = *reinterpret_cast<const h4 *>(wp + HALF);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = x[e] * r * (float)wa[e];
                    x[4 + e] = x[4 + e] * r * (float)wb[e];
                }
            }
            const f4 c = *reinterpret_cast<const f4 *>(scos + rr * HALF + 4 * piece);
            const f4 sn = *reinterpret_cast<const f4 *>(ssin + rr * HALF + 4 * piece);
            h4 ya, yb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ya[e] = (_Float16)(x[e] * c[e] - x[4 + e] * sn[e]);
                yb[e] = (_Float16)(x[4 + e] * c[e] + x[e] * sn[e]);
            }
            if (hs < p.G) {
                _Float16 *dst = p.q_out + ((int64_t)(w.m0 + rr) * p.Hq + h * p.G + hs) * D + 4 * piece;
                *reinterpret_cast<h4 *>(dst) = ya;
                *reinterpret_cast<h4 *>(dst + HALF) = yb;
            } else {
                *reinterpret_cast<h4 *>(sk + rin * KS + 4 * piece) = ya;
                *reinterpret_cast<h4 *>(sk + rin * KS + HALF + 4 * piece) = yb;
            }
        }
    }
    __syncthreads();
    if (panel < 0)
        return;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int q = tid + kThreads * c;
        if (q >= CHUNKS)
            break;
        if (has_k) {
            // K panel [D/32][16][32], chunk q: dims 8 * (4 * (q / 64) + q % 4) .. +8 of row (q / 4) % 16
            const int kr = (q >> 2) & 15;
            if (whole || (kr >= w.r0 && kr < w.r0 + w.rows))
                *reinterpret_cast<h8 *>(p.k_pool + panel + 8 * q) =
                    *reinterpret_cast<const h8 *>(sk + kr * KS + 8 * (4 * (q >> 6) + (q & 3)));
        }
        if (has_v && (whole || quad_new(q))) {
            // V panel [4][D][4], chunk q: dims d0 = 2 * (q % (D/2)) and d0 + 1 of quad q / (D/2); element x is dim
            // d0 + x / 4 of row 4 * (q / (D/2)) + x % 4
            const int vq = q / (D / 2), d0 = 2 * (q % (D / 2));
            h8 vn;
#pragma unroll
            for (int x = 0; x < 8; ++x)
                vn[x] = sv[(4 * vq + (x & 3)) * VS + d0 + (x >> 2)];
            if (!whole) {
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const int vr = 4 * vq + (x & 3);
                    vn[x] = (vr >= w.r0 && vr < w.r0 + w.rows) ? vn[x] : ov[c][x];
                }
            }
            *reinterpret_cast<h8 *>(p.v_pool + panel + 8 * q) = vn;
        }
    }
}

}  // namespace

hipError_t launch_qkv_cache(const QkvParams &p, int head_dim, hipStream_t stream) {
    if (p.T <= 0)
        return hipSuccess;
    const int64_t slots = p.decode_lens ? p.B : ((int64_t)p.T + 32 * (int64_t)(p.cu_seqlens_q ? p.B : 1)) / 16;
    const dim3 grid((unsigned)slots, (unsigned)(p.Hkv * p.parts)), block(kThreads);
    switch (head_dim) {
    case 64: hipLaunchKernelGGL(qkv_cache_kernel<64>, grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL(qkv_cache_kernel<128>, grid, block, 0, stream, p); break;
    case 256: hipLaunchKernelGGL(qkv_cache_kernel<256>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
