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
//   * one workgroup per (16-row cache unit holding new rows, kv head h).  The grid has one workgroup per (token,
//     kv head); the workgroup of the first new token of each unit does the unit, the others return at once.  Its
//     items are the (new row, head) pairs of the unit: the G query heads of h, key head h and value head h;
//   * a head row is D/8 lanes, each holding one 16-byte piece.  The sum of squares is reduced across those lanes,
//     and RoPE's partner dim j + D/2 sits D/16 lanes away, so both are lane exchanges inside the group;
//   * q goes straight to q_out (16-byte stores, coalesced per head row).  The unit's new K and V rows are staged
//     in LDS in the pool's panel layout (K [D/8][16][8], V [D][16]); each thread then writes 16-byte chunks of
//     the two panels, taking rows outside the new range from the old panel, which it loaded at the start (so that
//     load overlaps everything else).  The pools thus see only whole 16-byte chunks of whole panels -- scattered
//     2-byte V stores and 16-byte K row pieces cost far more at the memory than their bytes.
//
// A unit's other rows are rewritten with their own values: no other work may write the panel meanwhile (the
// block holding a sequence's new rows belongs to that sequence alone).
//
// All HIP code here is built with packed-fp32 instructions disabled.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

template <int D>
__global__ __launch_bounds__(256) void qkv_cache_kernel(QkvParams p) {
    constexpr int LPR = D / 8;       // lanes per head row, one 16-byte piece each
    constexpr int PARTNER = D / 16;  // lane distance from dim j to dim j + D/2
    constexpr int HALF = D / 2;
    constexpr int CHUNKS = 2 * D;    // 16-byte chunks of one 16-row panel (16 * D halves)
    constexpr int CPT = (CHUNKS + 255) / 256;
    __shared__ __attribute__((aligned(16))) _Float16 sk[16 * D];  // new K rows, panel layout [D/8][16][8]
    __shared__ __attribute__((aligned(16))) _Float16 sv[16 * D];  // new V rows, panel layout [D][16]

    const int m = (int)(blockIdx.x / (unsigned)p.Hkv);
    const int h = (int)(blockIdx.x - (unsigned)m * p.Hkv);
    int s = 0, first = 0, n = p.T, rope0 = p.rope_base, cache0 = p.cache_base;
    if (p.cu_seqlens_q) {
        // the sequence of token m: the last s with cu[s] <= m
        int lo = 0, hi = p.B;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.cu_seqlens_q[mid] <= m)
                lo = mid;
            else
                hi = mid - 1;
        }
        s = lo;
        if (s >= p.B)
            return;
        first = p.cu_seqlens_q[s];
        n = p.cu_seqlens_q[s + 1] - first;
        rope0 = cache0 = p.pos_offsets[s];
    }
    const int i = m - first;
    if (i < 0 || i >= n)
        return;
    const int row = cache0 + i;  // cache row of token m
    const int r0 = row & 15;     // its row inside the 16-row unit
    if (i > 0 && r0 != 0)
        return;                  // not the unit's first new token: another workgroup writes this unit
    int rows = 16 - r0;          // new rows of the unit, from r0 on
    rows = rows < n - i ? rows : n - i;
    rows = rows < p.T - m ? rows : p.T - m;
    const int64_t rp0 = (int64_t)rope0 + i;
    if (rp0 < 0 || rp0 + rows > p.P)
        return;                  // positions outside the tables: the unit's tokens are not written

    int64_t panel = -1;          // the unit's panel (element offset of its first half) in both pools
    if (row >= 0 && (int64_t)row < (int64_t)p.M * p.BS) {
        const int blk = p.block_tables[(int64_t)s * p.M + row / p.BS];
        if (blk >= 0 && blk < p.N)
            panel = (((int64_t)blk * p.Hkv + h) * p.BS + (row % p.BS - r0)) * D;
    }
    const bool whole = r0 == 0 && rows == 16;
    const int tid = threadIdx.x;

    // old panel contents first: rows outside [r0, r0 + rows) are written back unchanged
    h8 ok[CPT], ov[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + 256 * j;
        if (panel >= 0 && !whole && c < CHUNKS) {
            ok[j] = *reinterpret_cast<const h8 *>(p.k_pool + panel + 8 * c);
            ov[j] = *reinterpret_cast<const h8 *>(p.v_pool + panel + 8 * c);
        }
    }

    const int width = (p.Hq + 2 * p.Hkv) * D;
    const int heads = p.G + 2;
    const int lanes = rows * heads * LPR;
    const float inv_d = 1.0f / (float)D;
    for (int base = 0; base < lanes; base += 256) {
        const int idx = base + tid;
        if (idx >= lanes)
            break;  // lanes >= idx form whole head-row groups, so every exchange below has its partner
        const int item = idx / LPR;
        const int piece = idx - item * LPR;
        const int rr = item / heads;
        const int hh = item - rr * heads;
        const int tok = m + rr;
        const int rin = r0 + rr;
        const int head = hh < p.G ? h * p.G + hh : (hh == p.G ? p.Hq + h : p.Hq + p.Hkv + h);
        const h8 raw = *reinterpret_cast<const h8 *>(p.qkv + (int64_t)tok * width + (int64_t)head * D + 8 * piece);
        if (hh > p.G) {
            // value head: copied into the staged V panel (dim-major, 16 rows per dim)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sv[(8 * piece + e) * 16 + rin] = raw[e];
            continue;
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            x[e] = (float)raw[e];
        if (p.qk_mode == 1) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ss += x[e] * x[e];
#pragma unroll
            for (int o = 1; o < LPR; o <<= 1)
                ss += __shfl_xor(ss, o, 64);
            const float r = rsqrtf(ss * inv_d + p.eps);
            const h8 w = *reinterpret_cast<const h8 *>((hh < p.G ? p.q_norm_w : p.k_norm_w) + 8 * piece);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = x[e] * r * (float)w[e];
        }
        const int64_t t0 = (rp0 + rr) * HALF + (8 * piece) % HALF;
        const float4 c0 = *reinterpret_cast<const float4 *>(p.cos_t + t0);
        const float4 c1 = *reinterpret_cast<const float4 *>(p.cos_t + t0 + 4);
        const float4 s0 = *reinterpret_cast<const float4 *>(p.sin_t + t0);
        const float4 s1 = *reinterpret_cast<const float4 *>(p.sin_t + t0 + 4);
        const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const bool low = piece < PARTNER;  // this lane holds dims j < D/2; its partner holds j + D/2
        h8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xp = __shfl_xor(x[e], PARTNER, 64);
            y[e] = (_Float16)(low ? x[e] * cs[e] - xp * sn[e] : x[e] * cs[e] + xp * sn[e]);
        }
        if (hh < p.G)
            *reinterpret_cast<h8 *>(p.q_out + ((int64_t)tok * p.Hq + head) * D + 8 * piece) = y;
        else
            *reinterpret_cast<h8 *>(sk + (piece * 16 + rin) * 8) = y;
    }
    __syncthreads();
    if (panel < 0)
        return;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + 256 * j;
        if (c >= CHUNKS)
            break;
        // K chunk c: piece c / 16 of row c % 16
        const int kr = c & 15;
        const h8 kn = *reinterpret_cast<const h8 *>(sk + 8 * c);
        const bool knew = whole || (kr >= r0 && kr < r0 + rows);
        *reinterpret_cast<h8 *>(p.k_pool + panel + 8 * c) = knew ? kn : ok[j];
        // V chunk c: dim c / 2, rows 8 * (c % 2) .. + 8
        h8 vn = *reinterpret_cast<const h8 *>(sv + 8 * c);
        if (!whole) {
            const int vr = 8 * (c & 1);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vn[e] = (vr + e >= r0 && vr + e < r0 + rows) ? vn[e] : ov[j][e];
        }
        *reinterpret_cast<h8 *>(p.v_pool + panel + 8 * c) = vn;
    }
}

}  // namespace

hipError_t launch_qkv_cache(const QkvParams &p, int head_dim, hipStream_t stream) {
    if (p.T <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((int64_t)p.T * p.Hkv)), block(256);
    switch (head_dim) {
    case 64: hipLaunchKernelGGL(qkv_cache_kernel<64>, grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL(qkv_cache_kernel<128>, grid, block, 0, stream, p); break;
    case 256: hipLaunchKernelGGL(qkv_cache_kernel<256>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
