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
//     units hold a row or two, as in decode; a few, about four passes of 256 threads each, when units are full);
//     items are (new row, head slot) pairs.  The first loads are issued at once (the old panels, the unit's rows
//     of the cos/sin tables and the norm weights into LDS, each thread's qkv pieces of the first pass);
//   * a head row is D/8 lanes; lane l holds dims 4l .. 4l+3 and D/2 + 4l .. +3, so each RoPE pair (j, j + D/2)
//     lives in one lane.  The sum of squares is reduced across the group's lanes on the VALU (DPP row rotations,
//     and a v_permlane16_swap for 32-lane groups);
//   * q goes straight to q_out (8-byte stores, coalesced per half head row).  The unit's new K and V rows are
//     staged in LDS row-major (padded rows); each thread then writes 16-byte chunks of the two panels (each put in
//     its panel order on the way), taking rows
//     outside the new range from the old panel, which it loaded at the start (so that load overlaps everything
//     else).  The pools thus see only whole 16-byte chunks of whole panels -- scattered 2-byte V stores and
//     16-byte K row pieces cost far more at the memory than their bytes;
//   * decode mode (decode_lens set): slot g is sequence g, whose one new token sits at row decode_lens[g] - 1 --
//     the QKV half of the decode step from QKV rows when it runs as two launches.
//
// A unit's other rows are rewritten with their own values: no other work may write the panel meanwhile (the
// block holding a sequence's new rows belongs to that sequence alone).
//
// All HIP code here is built with packed-fp32 instructions disabled.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_internal.h"
#include "pkv_lanes.h"

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
// B < 64 one round loads every candidate and its position at once, and the answer's neighbours come from lane
// exchanges.  Keys increase, so the lanes that pass are a prefix; with malformed prefix sums s still lies in
// [0, B].
struct SeqOfSlot {
    int s, first, n, pos;
};

__device__ __forceinline__ SeqOfSlot find_sequence(const int32_t *cu, const int32_t *pos, int B, int g) {
    const int lane = threadIdx.x & 63;
    const int target = 16 * g + 15;
    SeqOfSlot r;
    if (B < 64) {
        const int c = cu[lane <= B ? lane : B];
        const int q = pos[lane < B ? lane : B - 1];
        const bool pass = lane <= B && c + 32 * lane <= target;
        int k = __popcll(__ballot(pass)) - 1;
        k = k > 0 ? k : 0;
        r.s = k;
        r.first = __shfl(c, k, 64);
        r.n = __shfl(c, k + 1 <= B ? k + 1 : B, 64) - r.first;
        r.pos = __shfl(q, k < B ? k : B - 1, 64);
        return r;
    }
    int lo = 0, hi = B;
    while (lo < hi) {
        const int stride = (hi - lo + 64) / 64;
        const int idx = lo + lane * stride;
        const bool pass = idx <= hi && slot_key(cu, idx) <= target;
        const int k = __popcll(__ballot(pass)) - 1;
        lo += (k > 0 ? k : 0) * stride;
        hi = min(hi, lo + stride - 1);
    }
    r.s = lo;
    if (lo < B) {
        r.first = cu[lo];
        r.n = cu[lo + 1] - r.first;
        r.pos = pos[lo];
    }
    return r;
}

template <int D>
__global__ __launch_bounds__(kThreads) void qkv_cache_kernel(QkvParams p) {
    constexpr int LPR = D / 8;       // lanes per head row, 8 dims each
    constexpr int HALF = D / 2;
    constexpr int CHUNKS = 2 * D;    // 16-byte chunks of one 16-row panel (16 * D halves)
    constexpr int CPT = (CHUNKS + kThreads - 1) / kThreads;
    constexpr int TAB = 16 * HALF / 4;  // float4 chunks of 16 rows of one table
    constexpr int VS = D + 4;  // row stride of the V staging (the pad spreads a dim's 16 rows over distinct banks)
    constexpr int KS = D + 8;  // row stride of the K staging (16-byte chunks of 16 rows read back together)
    __shared__ __attribute__((aligned(16))) _Float16 sk[16 * KS];  // new K rows, row-major [16][D + 8]
    __shared__ __attribute__((aligned(16))) _Float16 sv[16 * VS];  // new V rows, row-major [16][D + 4]
    __shared__ __attribute__((aligned(16))) float scos[16 * HALF];  // the unit's rows of the tables
    __shared__ __attribute__((aligned(16))) float ssin[16 * HALF];
    __shared__ __attribute__((aligned(16))) _Float16 sw[2 * D];     // q_norm_w, k_norm_w

    const int g = (int)blockIdx.x;                  // unit slot
    const int h = (int)blockIdx.y / p.parts;        // kv head
    const int part = (int)blockIdx.y - h * p.parts;  // which of its head slots (G query heads, K, V) this group does
    int s = 0, first = 0, n = p.T, rope0 = p.rope_base, cache0 = p.cache_base;
    int j;  // index of this slot's cache unit among the sequence's units
    if (p.decode_lens) {
        // one new token per sequence: slot g is sequence g, its row at position L - 1
        s = first = g;
        const int L = p.decode_lens[s];
        n = L > 0 ? 1 : 0;
        rope0 = cache0 = L - 1;
        j = 0;
    } else {
        if (p.cu_seqlens_q) {
            const SeqOfSlot q = find_sequence(p.cu_seqlens_q, p.pos_offsets, p.B, g);
            if (q.s >= p.B)
                return;
            s = q.s;
            first = q.first;
            n = q.n;
            rope0 = cache0 = q.pos;
        }
        j = g - ((first + 32 * s) >> 4);
    }
    // this slot's 16-row cache unit and the new rows in it
    const int64_t u = (int64_t)(cache0 >> 4) + j;
    const int64_t lo = max((int64_t)cache0, 16 * u);
    const int64_t hi = min((int64_t)cache0 + n, 16 * u + 16);
    if (j < 0 || lo >= hi)
        return;
    const int r0 = (int)(lo - 16 * u);  // first new row inside the unit
    int rows = (int)(hi - lo);
    const int i0 = (int)(lo - cache0);  // its index among the sequence's new tokens
    const int m0 = first + i0;          // its token
    rows = rows < p.T - m0 ? rows : p.T - m0;
    const int64_t rp0 = (int64_t)rope0 + i0;
    if (m0 < 0 || rows <= 0 || rp0 < 0 || rp0 + rows > p.P)
        return;  // positions outside the tables (or malformed prefix sums): the unit's tokens are not written

    // head slots [hs0, hs1) of kv head h: < G query heads, G the key head, G + 1 the value head
    const int hs0 = part * p.hpp;
    const int hs1 = min(hs0 + p.hpp, p.G + 2);
    const int nh = hs1 - hs0;
    const bool has_k = hs0 <= p.G && p.G < hs1;
    const bool has_v = hs1 == p.G + 2;
    int64_t panel = -1;  // the unit's panel (element offset of its first half) in both pools
    if ((has_k || has_v) && lo >= 0 && lo < (int64_t)p.M * p.BS) {
        const int row = (int)lo;
        const int blk = p.block_tables[(int64_t)s * p.M + row / p.BS];
        if (blk >= 0 && blk < p.N)
            panel = (((int64_t)blk * p.Hkv + h) * p.BS + (row % p.BS - r0)) * D;
    }
    const bool whole = r0 == 0 && rows == 16;
    const int tid = threadIdx.x;
    const int width = (p.Hq + 2 * p.Hkv) * D;
    const int lanes = rows * nh * LPR;
    const bool rotates = hs0 <= p.G;  // the group holds a query or key head

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
        const _Float16 *src = p.qkv + (int64_t)(m0 + rr) * width + (int64_t)head * D + 4 * piece;
        const h4 a = *reinterpret_cast<const h4 *>(src);
        const h4 b = *reinterpret_cast<const h4 *>(src + HALF);
        return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    };

    // The first batch of global loads at once: the old panels (rows outside [r0, r0 + rows) are written back
    // unchanged), the unit's rows of the cos/sin tables and the norm weights (to LDS), this thread's qkv pieces.
    h8 ok[CPT], ov[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int q = tid + kThreads * c;
        if (panel >= 0 && !whole && q < CHUNKS) {
            if (has_k)
                ok[c] = *reinterpret_cast<const h8 *>(p.k_pool + panel + 8 * q);
            if (has_v)
                ov[c] = *reinterpret_cast<const h8 *>(p.v_pool + panel + 8 * q);
        }
    }
    if (rotates) {
        for (int c = tid; c < 2 * TAB; c += kThreads) {
            const int t = c < TAB ? c : c - TAB;  // float4 t of the unit's 16 table rows
            if (t < rows * (HALF / 4)) {
                const float *src = (c < TAB ? p.cos_t : p.sin_t) + rp0 * HALF + 4 * t;
                *reinterpret_cast<float4 *>((c < TAB ? scos : ssin) + 4 * t) =
                    *reinterpret_cast<const float4 *>(src);
            }
        }
        if (p.qk_mode == 1 && tid < 2 * LPR)
            *reinterpret_cast<h8 *>(sw + 8 * tid) =
                *reinterpret_cast<const h8 *>((tid < LPR ? p.q_norm_w : p.k_norm_w) + 8 * (tid % LPR));
    }
    h8 raw[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
        if (b * kThreads + tid < lanes)
            raw[b] = fetch(b * kThreads + tid);
    __syncthreads();

    const float inv_d = 1.0f / (float)D;
    for (int base = 0; base < lanes; base += kBatch * kThreads) {
        if (base > 0) {
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (base + b * kThreads + tid < lanes)
                    raw[b] = fetch(base + b * kThreads + tid);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int idx = base + b * kThreads + tid;
            if (idx >= lanes)
                break;  // lanes below `lanes` form whole head-row groups, so every group sum has all its lanes
            int rr, hs, piece;
            source(idx, rr, hs, piece);
            const int rin = r0 + rr;
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
            const float4 c = *reinterpret_cast<const float4 *>(scos + rr * HALF + 4 * piece);
            const float4 sn = *reinterpret_cast<const float4 *>(ssin + rr * HALF + 4 * piece);
            const float cs[4] = {c.x, c.y, c.z, c.w};
            const float ss4[4] = {sn.x, sn.y, sn.z, sn.w};
            h4 ya, yb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ya[e] = (_Float16)(x[e] * cs[e] - x[4 + e] * ss4[e]);
                yb[e] = (_Float16)(x[4 + e] * cs[e] + x[e] * ss4[e]);
            }
            if (hs < p.G) {
                _Float16 *dst = p.q_out + ((int64_t)(m0 + rr) * p.Hq + h * p.G + hs) * D + 4 * piece;
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
            const h8 kn = *reinterpret_cast<const h8 *>(sk + kr * KS + 8 * (4 * (q >> 6) + (q & 3)));
            const bool knew = whole || (kr >= r0 && kr < r0 + rows);
            *reinterpret_cast<h8 *>(p.k_pool + panel + 8 * q) = knew ? kn : ok[c];
        }
        if (has_v) {
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
                    vn[x] = (vr >= r0 && vr < r0 + rows) ? vn[x] : ov[c][x];
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
