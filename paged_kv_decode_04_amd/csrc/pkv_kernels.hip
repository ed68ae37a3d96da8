// pkv_kernels.hip -- gfx950 kernels for paged-KV decode attention and the
// paged KV append.
//
// Decode attention [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
// paged_batched_decode_single_pass, paged_batched_flash_dispatch]:
//   out[s][hq] = softmax(scale * q[s][hq] . K_s^T) . V_s over the context_lens[s]
//   rows of sequence s, gathered through block_tables[s].
//
// Work decomposition (MI355X-first, not the pages' CTA-per-query-head):
//   * one workgroup per (sequence, kv head[, split]); the G query heads of the
//     kv head share every K/V byte the workgroup reads, so each KV tile crosses
//     HBM once per decode step, not G times;
//   * inside the workgroup, wavefront w takes the 16-row units w, w+NW, ... of
//     the range and keeps its own running max / sum / output; the waves merge
//     through LDS at the end (no partials in HBM for a single pass);
//   * per 16-row unit, the two products run on the matrix cores:
//       S^T[t][h] = sum_d K[t][d] Q[h][d]     v_mfma_f32_16x16x32_f16, D/32 steps
//       O^T[d][h] += sum_t V^T[d][t] P^T[t][h] v_mfma_f32_16x16x16_f16, D/16 tiles
//     The first product's accumulator layout (lane = 16*g + h holds rows
//     t = 4g..4g+3 of column h) is exactly the B-operand layout the second
//     product needs (lane 16*g + h holds k = 4g..4g+3 of column h), so the
//     probabilities never leave registers.  Query heads beyond G are zero
//     columns.  The reduction dimension of the first product is permuted the
//     same way in both operands (lane group g owns dims 32c + 8g .. +8), which
//     lets every lane load a 16-byte piece of a K row straight from HBM, each
//     K load of the wave one 1 KB run; V is stored in quads of 4 rows, so a
//     lane's 4 consecutive rows of one dim are 8 contiguous bytes and each V
//     load of the wave is four whole 128-byte lines.
//   * online softmax in f32, in the log2 domain (scores pre-multiplied by
//     scale*log2(e)); the running max starts at a finite -1e30 so that an
//     all-masked unit never forms inf - inf.
//   * each wave double-buffers its K/V fragments: the next unit's loads are in
//     flight while the current one is computed.
//
// Split-K phase 1 is the same kernel restricted to a block range, writing
// f32 (O_j unnormalised, m_j in natural units, l_j) instead of fp16 out; the
// combine kernel below is phase 2.
//
// All HIP code here is built with packed-fp32 instructions disabled.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv_internal.h"
#include "pkv_lanes.h"
#include "pkv_unit.h"

namespace pkv {

// FUSED: the fused decode step (p.k_new / p.v_new hold each sequence's new row); otherwise attention alone.
// QKV (with FUSED): the decode step from the QKV projection rows -- q and the new K/V rows are taken from p.qkv,
// the query and key heads RMS-normalised (qk_mode 1) and rotated at position L-1 in the prologue [ferrum-kernels
// 0.7.7, src/backend/cuda/paged.rs: split_qkv_norm_rope_into_paged_cache_varlen, then paged_decode_attention].
template <int D, int BS, int NW, bool SPLIT, bool FUSED, bool QKV = false, bool ORDERED = false>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeParams p) {
    constexpr int KC = D / 32;
    constexpr int VC = D / 16;
    constexpr int NS = pipeline_stages<D, NW>();
    constexpr int SPB = BS / 16;
    constexpr int DP = D + 4;  // padded LDS row of one head's output
    extern __shared__ float smem[];

    // 1-D grid.  With splits, the S splits of one (sequence, kv head) tile are consecutive workgroup ids: the
    // dispatcher deals consecutive ids to different XCDs and CUs, so a long tile's splits stream through many CUs
    // (each CU's outstanding-miss budget, not HBM, bounds one workgroup), and each CU's co-resident workgroups come
    // from unrelated tiles.
    const int tile = SPLIT ? (int)(blockIdx.x / (unsigned)p.num_splits) : (int)blockIdx.x;
    const int split = SPLIT ? (int)(blockIdx.x - (unsigned)tile * p.num_splits) : 0;
    const int rank = tile / p.Hkv;
    const int hk = tile - rank * p.Hkv;
    // ORDERED (a grid of several rounds): the sequences run longest first, tile t taking the sequence of order
    // record t / Hkv -- the dispatcher starts workgroups in id order as CUs free up, so the longest ones no longer
    // start last and finish alone.  The record also holds the length and the first block ids, so the first K/V
    // loads still wait for one dependent load.  A record may be one piece of a sequence (a range of its units, see
    // PieceRule): the pieces' partials are merged by the last of them to finish (the epilogue below).
    const int32_t *rec = ORDERED ? p.order + (int64_t)rank * kOrderRecord : nullptr;
    int s_rec = 0, L_rec = 0;          // the record's sequence and length
    int u0_rec = 0, u1_rec = 0;        // its unit range
    int pc_rec = 1 << 16, base_rec = 0;  // piece index | pieces << 16; the record of piece 0
    if (ORDERED) {
        uniform_load_pair(rec, 0, s_rec, L_rec);
        uniform_load_pair(rec, 2, u0_rec, u1_rec);
        uniform_load_pair(rec, 4, pc_rec, base_rec);
    }
    const bool unused_rec = ORDERED && s_rec < 0;  // a record past the last piece (wave-uniform)
    const int s = ORDERED ? (unused_rec ? 0 : s_rec) : rank;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r = lane & 15;
    const int g4 = lane >> 4;

    const int32_t *bt = p.block_tables + (int64_t)s * p.M;
    const int max_units = p.M * SPB;  // units the table can name
    // Block ids are read with scalar loads (wave-uniform index), one pipeline step ahead of the unit that needs
    // them.  When the range start is known from the launch alone (a single pass starts at block 0, a fixed-size
    // split j at j*chunk_blocks), the ids of this wave's first NS units are requested together with the length,
    // so the first K/V loads wait for one dependent load, not two.
    const int u_known = (SPLIT ? split * p.chunk_blocks : 0) * SPB + wave;
    constexpr int NSPEC = 2 * NS - 1;  // the prologue's NS-1 units and the NS block ids requested ahead
    const bool start_known = (!SPLIT || p.chunk_blocks > 0) && p.window <= 0 &&
                             (!ORDERED || (u_known + (NSPEC - 1) * NW) / SPB < kOrderRecBlocks);
    int spec_raw[NSPEC];
#pragma unroll
    for (int j = 0; j < NSPEC; ++j) {
        const int bi = min(u_known + j * NW, max_units - 1) / SPB;
        spec_raw[j] = start_known ? (ORDERED ? uniform_load(rec, kOrderRecHead + bi) : uniform_load(bt, bi)) : -1;
    }
    int L = ORDERED ? L_rec : uniform_load(p.context_lens, s);

    // Q^T as the B operand: lane (g4, r) holds head r, dims 32c + 8*g4 .. +8.  Columns r >= G (no such head in
    // the group) repeat head 0; every column of the matrix-core tiles is independent and those are never stored.
    // From QKV rows (QKV): the raw query head, rotated below once the position is known.
    const int64_t qkv_row = (int64_t)s * (p.Hq + 2 * p.Hkv) * D;  // QKV: sequence s's row (its one new token)
    f16x8 qf[KC];
    {
        const int hq = hk * p.G + (r < p.G ? r : 0);
        const _Float16 *qrow = (QKV ? p.qkv + qkv_row + (int64_t)hq * D : p.q + ((int64_t)s * p.Hq + hq) * D) + 8 * g4;
#pragma unroll
        for (int c = 0; c < KC; ++c)
            qf[c] = *reinterpret_cast<const f16x8 *>(qrow + 32 * c);
    }
    f16x8 qw[KC];  // QKV, qk_mode 1: the query norm weights of this lane's dims
    if (QKV && p.qk_mode == 1) {
#pragma unroll
        for (int c = 0; c < KC; ++c)
            qw[c] = *reinterpret_cast<const f16x8 *>(p.q_norm_w + 32 * c + 8 * g4);
    }

    // Every request above depends on the launch alone; an empty asm statement that reads L and the first block
    // ids keeps them all ahead of the first use of the length, so one wait covers all the scalar loads.
    static_assert(NSPEC <= 5, "the barrier below names at most five block ids");
    asm volatile("" ::"s"(L), "s"(spec_raw[0]), "s"(spec_raw[NSPEC > 1 ? 1 : 0]), "s"(spec_raw[NSPEC > 2 ? 2 : 0]),
                 "s"(spec_raw[NSPEC > 3 ? 3 : 0]), "s"(spec_raw[NSPEC > 4 ? 4 : 0])
                 : "memory");

    if (unused_rec)
        return;
    if (ORDERED && !SPLIT && start_known && (pc_rec & 0xffff) != 0) {
        // a later piece's record holds no block ids: its first ones come from the table (one more dependent load,
        // for the few workgroups of the pieces past the first)
#pragma unroll
        for (int j = 0; j < NSPEC; ++j)
            spec_raw[j] = uniform_load(bt, min(u0_rec + u_known + j * NW, max_units - 1) / SPB);
    }
    L = L < 0 ? 0 : (L > p.M * BS ? p.M * BS : L);
    if (p.N <= 0)
        L = 0;  // an empty pool holds no rows
    const int nb = (L + BS - 1) / BS;
    // sliding window: rows lo .. L-1, from block lo / BS [cortiq-engine 0.8.80, src/gpu_cuda.rs: the decode
    // attend's first row, stored - window]
    const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
    const int b_lo = lo / BS;
    int b0 = b_lo, b1 = nb;
    if (SPLIT) {
        const int chunk = p.chunk_blocks > 0 ? p.chunk_blocks : (nb - b_lo + p.num_splits - 1) / p.num_splits;
        b0 = b_lo + split * chunk;
        b1 = min(nb, b0 + chunk);
        if (b0 >= b1)
            return;  // empty split: the combine never reads it
    }
    // units wholly before the window are skipped; an ordered piece reads its own range of units
    const int u_begin = max(max(b0 * SPB, lo >> 4), ORDERED && !SPLIT ? u0_rec : 0);
    const int u_end = min(min(b1 * SPB, (L + 15) >> 4), ORDERED && !SPLIT ? u1_rec : INT32_MAX);
    const int npieces = ORDERED && !SPLIT ? (pc_rec >> 16) : 1;
    const bool piece = npieces > 1;  // this tile is one piece of a split sequence: it writes a partial
    const RowLimits lim = {L - 1, L - 1, L - 1, lo};
    const int u_first = u_begin + wave;  // wave w takes units u_begin + w, + w + NW, ...
    const int n_units = u_first < u_end ? (u_end - u_first + NW - 1) / NW : 0;
    // Fused decode step: the workgroup whose range holds row L-1 writes the sequence's new K/V row there (the slot
    // the callers form from the table: block bt[(L-1)/BS], row (L-1)%BS).  The wave that computes the unit holding
    // row L-1 loads the row, keeps a copy in LDS and, when it computes that unit, patches it into the fragments and
    // writes its K runs and V quad back (see compute_unit).
    const bool appending = FUSED && L > 0 && (L - 1) / BS >= b0 && (L - 1) / BS < b1;
    const int patch_unit = appending ? (L - 1) >> 4 : -1;
    const int prow_row = (L - 1) & 15;
    const bool patch_owner = appending && wave == (patch_unit - u_begin) % NW;

    f32x4 o[VC];
#pragma unroll
    for (int c = 0; c < VC; ++c)
        o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = kNegBig;
    float l_run = 0.f;

    const uint32_t k_lane = k_lane_offset(r, g4);             // bytes into a K panel
    const uint32_t v_lane = v_lane_offset(D, r, g4);          // bytes into a V panel
    const int64_t head_off = (int64_t)hk * (BS * D);
    const int64_t block_stride = (int64_t)p.Hkv * (BS * D);

    // LDS copy of the new row (fused step): K then V, D halves each, after the merge area (which other waves may
    // fill while the owner wave still computes).
    _Float16 *sm_pk = reinterpret_cast<_Float16 *>(smem + merge_floats(D, p.G, NW));
    _Float16 *sm_pv = sm_pk + D;
    // Owner wave: load the new row (lane t < D/8 takes dims 8t .. 8t+7 of K and of V) ahead of its first K/V loads
    // and copy it to LDS for the unit that holds it (see compute_unit).  From QKV rows, lane t < D/16 takes K dims
    // 8t .. 8t+7 and D/2 + 8t .. +7 instead, so that each rotated pair (j, j + D/2) is in one lane.
    f16x8 new_k = (f16x8)(_Float16)0.0f, new_v = (f16x8)(_Float16)0.0f, new_k2 = (f16x8)(_Float16)0.0f;
    f16x8 kwa = new_k, kwb = new_k;  // QKV, qk_mode 1: the key norm weights of those dims
    if (patch_owner) {
        if (QKV) {
            const _Float16 *krow = p.qkv + qkv_row + (int64_t)(p.Hq + hk) * D;
            if (lane < D / 16) {
                new_k = *reinterpret_cast<const f16x8 *>(krow + 8 * lane);
                new_k2 = *reinterpret_cast<const f16x8 *>(krow + D / 2 + 8 * lane);
                if (p.qk_mode == 1) {
                    kwa = *reinterpret_cast<const f16x8 *>(p.k_norm_w + 8 * lane);
                    kwb = *reinterpret_cast<const f16x8 *>(p.k_norm_w + D / 2 + 8 * lane);
                }
            }
            if (lane < D / 8)
                new_v = *reinterpret_cast<const f16x8 *>(p.qkv + qkv_row + (int64_t)(p.Hq + p.Hkv + hk) * D + 8 * lane);
        } else if (lane < D / 8) {
            const int64_t row_off = ((int64_t)s * p.Hkv + hk) * D + 8 * lane;
            new_k = *reinterpret_cast<const f16x8 *>(p.k_new + row_off);
            new_v = *reinterpret_cast<const f16x8 *>(p.v_new + row_off);
        }
    }
    // QKV: the rotation's table row is position L-1 (clamped into the table: a length past it gives unspecified
    // results, never an access outside it).  Query lanes need cos/sin of dims 32c + 8*g4 .. +8 (c < KC/2), the
    // owner's key lanes those of dims 8t .. 8t+7.
    float4 qcs[KC / 2][2], qsn[KC / 2][2], kcs[2], ksn[2];
    if (QKV) {
        const int64_t trow = (int64_t)min(max(L - 1, 0), p.P - 1) * (D / 2);
#pragma unroll
        for (int c = 0; c < KC / 2; ++c) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                qcs[c][h] = *reinterpret_cast<const float4 *>(p.cos_t + trow + 32 * c + 8 * g4 + 4 * h);
                qsn[c][h] = *reinterpret_cast<const float4 *>(p.sin_t + trow + 32 * c + 8 * g4 + 4 * h);
            }
        }
        if (patch_owner && lane < D / 16) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                kcs[h] = *reinterpret_cast<const float4 *>(p.cos_t + trow + 8 * lane + 4 * h);
                ksn[h] = *reinterpret_cast<const float4 *>(p.sin_t + trow + 8 * lane + 4 * h);
            }
        }
    }
    // QKV: norm (qk_mode 1) and rotation of this lane's query dims; the first wave of the first split also stores
    // the rotated heads to q_out.  Dims 32c + 8*g4 + e and 32(c + KC/2) + 8*g4 + e are a RoPE pair (D/2 apart).
    auto rotate_q = [&]() {
        float x[KC][8];
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[c][e] = (float)qf[c][e];
        if (p.qk_mode == 1) {
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < KC; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ss += x[c][e] * x[c][e];
            const float rn = rsqrtf(rows_sum(ss) * (1.0f / D) + p.eps);  // lanes r, r+16, r+32, r+48: head r
#pragma unroll
            for (int c = 0; c < KC; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[c][e] = x[c][e] * rn * (float)qw[c][e];
        }
#pragma unroll
        for (int c = 0; c < KC / 2; ++c) {
            const float cs[8] = {qcs[c][0].x, qcs[c][0].y, qcs[c][0].z, qcs[c][0].w,
                                 qcs[c][1].x, qcs[c][1].y, qcs[c][1].z, qcs[c][1].w};
            const float sn[8] = {qsn[c][0].x, qsn[c][0].y, qsn[c][0].z, qsn[c][0].w,
                                 qsn[c][1].x, qsn[c][1].y, qsn[c][1].z, qsn[c][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = x[c][e], b = x[c + KC / 2][e];
                x[c][e] = a * cs[e] - b * sn[e];
                x[c + KC / 2][e] = b * cs[e] + a * sn[e];
            }
        }
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                qf[c][e] = (_Float16)x[c][e];
        if (wave == 0 && split == 0 && r < p.G) {
            _Float16 *qo = p.q_out + ((int64_t)s * p.Hq + hk * p.G + r) * D + 8 * g4;
#pragma unroll
            for (int c = 0; c < KC; ++c)
                *reinterpret_cast<f16x8 *>(qo + 32 * c) = qf[c];
        }
    };
    auto copy_new_row = [&]() {
        if (QKV) {
            if (lane < D / 16) {
                float a[8], b[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a[e] = (float)new_k[e];
                    b[e] = (float)new_k2[e];
                }
                if (p.qk_mode == 1) {
                    float ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        ss += a[e] * a[e] + b[e] * b[e];
                    const float rn = rsqrtf(lanes_sum<D / 16>(ss) * (1.0f / D) + p.eps);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        a[e] = a[e] * rn * (float)kwa[e];
                        b[e] = b[e] * rn * (float)kwb[e];
                    }
                }
                const float cs[8] = {kcs[0].x, kcs[0].y, kcs[0].z, kcs[0].w, kcs[1].x, kcs[1].y, kcs[1].z, kcs[1].w};
                const float sn[8] = {ksn[0].x, ksn[0].y, ksn[0].z, ksn[0].w, ksn[1].x, ksn[1].y, ksn[1].z, ksn[1].w};
                f16x8 ya, yb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ya[e] = (_Float16)(a[e] * cs[e] - b[e] * sn[e]);
                    yb[e] = (_Float16)(b[e] * cs[e] + a[e] * sn[e]);
                }
                *reinterpret_cast<f16x8 *>(sm_pk + 8 * lane) = ya;
                *reinterpret_cast<f16x8 *>(sm_pk + D / 2 + 8 * lane) = yb;
            }
            if (lane < D / 8)
                *reinterpret_cast<f16x8 *>(sm_pv + 8 * lane) = new_v;
        } else if (lane < D / 8) {
            *reinterpret_cast<f16x8 *>(sm_pk + 8 * lane) = new_k;
            *reinterpret_cast<f16x8 *>(sm_pv + 8 * lane) = new_v;
        }
    };

    if (n_units > 0) {
        // Block id of unit u, clamped to block 0 when the table names no pool block (the unit is then loaded as
        // zeros and computed fully masked).
        auto raw_block = [&](int u) -> int { return uniform_load(bt, min(u, max_units - 1) / SPB); };
        auto resolve = [&](int raw, bool &dead) -> int {
            const int b = __builtin_amdgcn_readfirstlane(raw);
            dead = (unsigned)b >= (unsigned)p.N;
            return dead ? 0 : b;
        };
        auto k_ptr = [&](int blk, int u) {
            return p.k_pool + (int64_t)blk * block_stride + head_off + (u % SPB) * (16 * D);
        };
        auto v_ptr = [&](int blk, int u) {
            return p.v_pool + (int64_t)blk * block_stride + head_off + (u % SPB) * (16 * D);
        };
        // NS-stage pipeline: while unit k is computed, units k+1 .. k+NS-1 are in flight, and the block ids of the
        // next NS units to issue are already requested (ring raw_q, slot k % NS holds unit k+NS-1's id at step k).
        // Every step issues its prefetch unconditionally -- past a wave's last unit as loads that touch no memory
        // (see load_unit) -- so the wait counts the compiler derives are exact on every path.  Slot indices are
        // compile-time constants in the unrolled step loop, so every fragment stays in registers.  Pipeline slots
        // past the wave's last unit are never computed, so their block ids may be anything in range.
        Frag<D, BS> f[NS];
        bool dead[NS];
        int uu[NS];
        int raw_q[NS];
        int bk[NS];  // block of each slot (the fused step writes the patched panel back there)
#pragma unroll
        for (int j = 0; j < NS - 1; ++j) {
            uu[j] = u_first + j * NW;
            const int blk = resolve(start_known ? spec_raw[j] : raw_block(uu[j]), dead[j]);
            bk[j] = blk;
            load_unit<D, BS>(f[j], k_ptr(blk, uu[j]), v_ptr(blk, uu[j]), k_lane, v_lane, j < n_units && !dead[j]);
        }
#pragma unroll
        for (int j = 0; j < NS; ++j)
            raw_q[j] = start_known ? spec_raw[NS - 1 + j] : raw_block(u_first + min(NS - 1 + j, n_units - 1) * NW);
        if (QKV)
            rotate_q();
        if (patch_owner)
            copy_new_row();
        int k = 0;
        for (;;) {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const int jn = (j + NS - 1) % NS;  // the slot freed by the unit computed one step ago
                uu[jn] = u_first + min(k + NS - 1, n_units - 1) * NW;
                const int blk = resolve(raw_q[j], dead[jn]);
                bk[jn] = blk;
                load_unit<D, BS>(f[jn], k_ptr(blk, uu[jn]), v_ptr(blk, uu[jn]), k_lane, v_lane,
                                 k + NS - 1 < n_units && !dead[jn]);
                raw_q[j] = raw_block(u_first + min(k + 2 * NS - 1, n_units - 1) * NW);
                compute_unit<D, BS>(f[j], qf, o, m_run, l_run, uu[j], lim, dead[j], r, g4, p.scale_log2,
                                    FUSED && uu[j] == patch_unit ? prow_row : -1, sm_pk, sm_pv,
                                    FUSED ? p.k_dst + (k_ptr(bk[j], uu[j]) - p.k_pool) : nullptr,
                                    FUSED ? p.v_dst + (v_ptr(bk[j], uu[j]) - p.v_pool) : nullptr, k_lane, v_lane);
                if (++k >= n_units)
                    goto units_done;
            }
        }
    units_done:;
    }

    l_run = rows_sum(l_run);

    // Cross-wave merge.  Each lane first forms its column's merged max M and denominator from every wave's (m, l),
    // then scales its own registers by a = 2^(m - M) (and by 1 / denominator for a single pass), so the final pass
    // is a plain sum over the waves per output element.
    float *sm_m = smem;
    float *sm_l = smem + NW * 16;
    float *sm_o = smem + 2 * NW * 16;
    if (g4 == 0) {
        sm_m[wave * 16 + r] = m_run;
        sm_l[wave * 16 + r] = l_run;
    }
    __syncthreads();
    float Mc = kNegBig;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        Mc = fmaxf(Mc, sm_m[w * 16 + r]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        den += exp2_fast(sm_m[w * 16 + r] - Mc) * sm_l[w * 16 + r];
    {
        const float a = exp2_fast(m_run - Mc);
        const float f = SPLIT || piece ? a : (den > 0.f ? a / den : 0.f);
        if (r < p.G) {  // 16-byte writes: with DP = D + 4 the eight lanes of a pass hit distinct banks
            float *dst = sm_o + (wave * p.G + r) * DP + 4 * g4;
#pragma unroll
            for (int c = 0; c < VC; ++c)
                *reinterpret_cast<f32x4 *>(dst + 16 * c) = o[c] * f;
        }
        if (SPLIT && wave == 0 && g4 == 0 && r < p.G) {
            const int64_t base = ((int64_t)s * p.Hq + hk * p.G + r) * p.num_splits + split;
            p.part_m[base] = Mc * kLn2;
            p.part_l[base] = den;
        }
        if (piece && wave == 0 && g4 == 0 && r < p.G) {  // the piece's (max in log2 units, sum) per query head
            const int64_t slot = (int64_t)rank * p.Hq + hk * p.G + r;
            store_agent(p.part_m + slot, Mc);
            store_agent(p.part_l + slot, den);
        }
    }
    __syncthreads();

    // Four dims per thread: 16-byte LDS reads, the waves summed in order from 0 (the same sums as one dim at a time)
    const int total4 = p.G * (D / 4);
    for (int idx = threadIdx.x; idx < total4; idx += NW * 64) {
        const int h = idx / (D / 4);
        const int d = 4 * (idx - h * (D / 4));
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w)
            num += *reinterpret_cast<const f32x4 *>(sm_o + (w * p.G + h) * DP + d);
        const int64_t row = (int64_t)s * p.Hq + hk * p.G + h;
        if (SPLIT) {
            *reinterpret_cast<f32x4 *>(p.part_o + (row * p.num_splits + split) * D + d) = num;
        } else if (piece) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                store_agent(p.part_o + ((int64_t)rank * p.Hq + hk * p.G + h) * D + d + e, num[e]);
        } else {
            f16x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y[e] = (_Float16)num[e];
            *reinterpret_cast<f16x4 *>(p.out + row * D + d) = y;
        }
    }
    if (piece) {
        // The pieces of a (sequence, kv head) meet at their ends only: each stores its partial with agent-coherent
        // stores (coherent across the XCDs' L2 caches), waits until they are complete, then counts itself in; the
        // piece that counts in last reads every piece's partial and merges them in piece order, whoever it is,
        // so the output does not depend on which piece ends last.  No workgroup waits for another, and no
        // cache-wide write-back is needed.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int *seen = reinterpret_cast<int *>(smem);
        if (threadIdx.x == 0)
            seen[0] = __hip_atomic_fetch_add(p.piece_count + (int64_t)s * p.Hkv + hk, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (seen[0] == npieces - 1) {
            for (int idx = threadIdx.x; idx < p.G * D; idx += NW * 64) {
                const int h = idx / D;
                const int d = idx - h * D;
                const int64_t hq = (int64_t)hk * p.G + h;
                float Mx = kNegBig;
                for (int pc = 0; pc < npieces; ++pc) {
                    const int64_t slot = (int64_t)(base_rec + pc) * p.Hq + hq;
                    if (load_agent(p.part_l + slot) > 0.f)
                        Mx = fmaxf(Mx, load_agent(p.part_m + slot));
                }
                float num = 0.f, dsum = 0.f;
                for (int pc = 0; pc < npieces; ++pc) {
                    const int64_t slot = (int64_t)(base_rec + pc) * p.Hq + hq;
                    const float l = load_agent(p.part_l + slot);
                    if (l > 0.f) {
                        const float a = exp2_fast(load_agent(p.part_m + slot) - Mx);
                        num += a * load_agent(p.part_o + slot * D + d);
                        dsum += a * l;
                    }
                }
                p.out[((int64_t)s * p.Hq + hq) * D + d] = (_Float16)(dsum > 0.f ? num / dsum : 0.f);
            }
        }
    }
}

// Paged varlen attention [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: paged_varlen_attention,
// paged_varlen_split_k_dispatch and the tiled_q4 variant's shared KV reads]: sequence s owns query rows
// cu[s] .. cu[s+1]-1 of the token-major q, its i-th new row at position pos[s] + i attending rows 0 .. pos[s] + i.
// One workgroup per (sequence, tile slot, kv head[, split]).  A tile is R = 16 / G consecutive new rows of one
// sequence; its 16 matrix-core columns are the (row, head) pairs c = row * G + head, so every K/V byte a workgroup
// loads serves all R rows and the whole GQA group; each column carries its own causal limit (RowLimits).  Tile slot
// j takes the sequence's tile groups j, j + tiles_per_seq, ... (any q length is covered whatever the host's
// estimate).  A group is QT consecutive tiles that share every K/V load: each unit's fragments feed QT tiles' score
// and P.V products (QT = 2 when a sequence has more than one tile: half the K/V traffic of one tile per workgroup).
// With splits, phase 1 writes every split of every valid column -- an empty one as m = -1e30, l = 0, O = 0 -- so
// the combine needs no per-row split count.
// FUSED (the fused varlen step, single pass): the new rows' K/V (k_new / v_new, token-major) are written into the
// pools by this launch -- each 16-row unit holding new rows is patched from an LDS copy of its new rows whenever it
// is computed, and the new rows' K runs and V quads are written back, so any interleaving of workgroups leaves the
// same bytes -- for the first
// kFusedUnits units of a sequence's new rows: any kStepFusedRows consecutive rows fit.

template <int D, int BS, int NW, bool SPLIT, int QT, bool FUSED = false, bool ORDERED = false>
__global__ __launch_bounds__(NW * 64) void varlen_kernel(VarlenParams p) {
    constexpr int KC = D / 32;
    constexpr int VC = D / 16;
    constexpr int SPB = BS / 16;
    constexpr int DP = D + 4;
    constexpr int NS = pipeline_stages<D, NW>();
    extern __shared__ float smem[];

    unsigned id = blockIdx.x;
    const int split = SPLIT ? (int)(id % (unsigned)p.num_splits) : 0;
    if (SPLIT)
        id /= (unsigned)p.num_splits;
    const int hk = (int)(id % (unsigned)p.Hkv);
    id /= (unsigned)p.Hkv;
    const int slot = (int)(id % (unsigned)p.tiles_per_seq);
    const int rank = (int)(id / (unsigned)p.tiles_per_seq);
    // ORDERED (a grid of several rounds): the sequences run longest first, their prefix sums, position and first
    // block ids read from the order record (see the decode kernel)
    const int32_t *rec = ORDERED ? p.order + (int64_t)rank * kOrderRecord : nullptr;
    int s_rec = 0, q0_rec = 0, q1_rec = 0, pos_rec = 0;
    if (ORDERED) {
        uniform_load_pair(rec, 0, s_rec, q0_rec);
        uniform_load_pair(rec, 2, q1_rec, pos_rec);
    }
    const int s = ORDERED ? s_rec : rank;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r = lane & 15;
    const int g4 = lane >> 4;

    const int32_t *bt = p.block_tables + (int64_t)s * p.M;
    const int max_units = p.M * SPB;
    const int cap = p.M * BS;  // rows the table can name
    // Every tile's key range starts at row 0 (in split mode with fixed chunks, at split * chunk_blocks), so the
    // block ids of this wave's first units are requested together with the prefix sums and the position.
    const int u_known = (SPLIT ? split * p.chunk_blocks : 0) * SPB + wave;
    constexpr int NSPEC = 2 * NS - 1;
    const bool start_known = (!SPLIT || p.chunk_blocks > 0) &&
                             (!ORDERED || (u_known + (NSPEC - 1) * NW) / SPB < kVarlenRecBlocks);
    int spec_raw[NSPEC];
#pragma unroll
    for (int j = 0; j < NSPEC; ++j) {
        const int bi = min(u_known + j * NW, max_units - 1) / SPB;
        spec_raw[j] = start_known ? (ORDERED ? uniform_load(rec, 4 + bi) : uniform_load(bt, bi)) : -1;
    }
    int q0 = ORDERED ? q0_rec : uniform_load(p.cu_seqlens_q, s);
    int q1 = ORDERED ? q1_rec : uniform_load(p.cu_seqlens_q, s + 1);
    int pos = ORDERED ? pos_rec : uniform_load(p.pos_offsets, s);
    static_assert(NSPEC <= 3, "the barrier below names at most three block ids");
    asm volatile("" ::"s"(q0), "s"(q1), "s"(pos), "s"(spec_raw[0]), "s"(spec_raw[NSPEC > 1 ? 1 : 0]),
                 "s"(spec_raw[NSPEC > 2 ? 2 : 0])
                 : "memory");
    q0 = q0 < 0 ? 0 : (q0 > p.T ? p.T : q0);
    q1 = q1 < q0 ? q0 : (q1 > p.T ? p.T : q1);
    pos = pos < 0 ? 0 : (pos > cap ? cap : pos);
    if (p.N <= 0)
        q1 = q0;  // an empty pool holds no rows
    const int qlen = q1 - q0;

    const uint32_t k_lane = k_lane_offset(r, g4);
    const uint32_t v_lane = v_lane_offset(D, r, g4);
    const int64_t head_off = (int64_t)hk * (BS * D);
    const int64_t block_stride = (int64_t)p.Hkv * (BS * D);

    // Fused step: units nu0 .. nu0 + n_new_units - 1 hold the new rows pos .. pos + qlen - 1.  The wave that computes
    // unit u in every tile group (u % NW: with one pass the range starts at unit 0) copies that unit's new rows to
    // its LDS slot (K [16][D] row-major, then V [D][16]; rows that are not new stay unset and are never read).  Its
    // first kPreChunks 16-byte chunks per lane of K and of V are loaded into registers before any K/V load and
    // written to LDS once the first units' loads are in flight, so that the wait for them covers only these older
    // loads (a wave's loads retire in order: copying through LDS before the first K/V loads held the owner wave's
    // stream back by a round trip, and loading the rows after them made the wait cover the whole first unit).
    // Chunks past those (more new rows in the unit than the registers hold), and the units of a wave that owns more
    // than one, are copied at once, the slow way.
    const int nu0 = pos >> 4;
    const int n_new_units = FUSED && qlen > 0 ? min(kFusedUnits, ((pos + qlen - 1) >> 4) - nu0 + 1) : 0;
    _Float16 *sm_new = reinterpret_cast<_Float16 *>(smem + merge_floats(D, 16, NW));
    constexpr int kPreChunks = 2;
    // new unit k (of n_new_units): its new rows start at unit row row0_of(k); chunk c = row * (D / 8) + piece
    auto row0_of = [&](int k) { return max(pos, 16 * (nu0 + k)) - 16 * (nu0 + k); };
    auto rows_of = [&](int k) { return min(pos + qlen, 16 * (nu0 + k) + 16) - 16 * (nu0 + k) - row0_of(k); };
    auto chunk_src = [&](int k, int c) {  // offset of chunk c of unit k in k_new / v_new
        const int rr = c / (D / 8), piece = c - rr * (D / 8);
        return ((int64_t)(q0 + 16 * (nu0 + k) + row0_of(k) - pos + rr) * p.Hkv + hk) * D + 8 * piece;
    };
    auto chunk_to_lds = [&](int k, int c, const f16x8 &kk, const f16x8 &vv) {
        const int rr = c / (D / 8), piece = c - rr * (D / 8);
        const int row = row0_of(k) + rr;
        _Float16 *slot_k = sm_new + k * 32 * D;
        _Float16 *slot_v = slot_k + 16 * D;
        *reinterpret_cast<f16x8 *>(slot_k + row * D + 8 * piece) = kk;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            slot_v[(8 * piece + e) * 16 + row] = vv[e];
    };
    auto copy_now = [&](int k, int c0) {  // chunks c0, c0 + 64, ... of unit k, lane-strided, waited for at once
        for (int c = c0 + lane; c < rows_of(k) * (D / 8); c += 64)
            chunk_to_lds(k, c, *reinterpret_cast<const f16x8 *>(p.k_new + chunk_src(k, c)),
                         *reinterpret_cast<const f16x8 *>(p.v_new + chunk_src(k, c)));
    };
    const int own = (wave - nu0 % NW + NW) % NW;  // the wave's first unit among the new ones, if < n_new_units
    const bool owner = FUSED && own < n_new_units;  // (wave-uniform)
    f16x8 pre_k[kPreChunks], pre_v[kPreChunks];
    if (owner) {
#pragma unroll
        for (int i = 0; i < kPreChunks; ++i) {
            const int c = lane + 64 * i;
            if (c < rows_of(own) * (D / 8)) {
                pre_k[i] = *reinterpret_cast<const f16x8 *>(p.k_new + chunk_src(own, c));
                pre_v[i] = *reinterpret_cast<const f16x8 *>(p.v_new + chunk_src(own, c));
            }
        }
        copy_now(own, 64 * kPreChunks);
        for (int k = own + NW; k < n_new_units; k += NW)  // fewer waves than new units: the wave's other units
            copy_now(k, 0);
    }
    bool pre_pending = owner;  // the register chunks still wait to be written to LDS (before the owned unit's patch)
    auto flush_pre = [&]() {
        if (pre_pending) {
#pragma unroll
            for (int i = 0; i < kPreChunks; ++i) {
                const int c = lane + 64 * i;
                if (c < rows_of(own) * (D / 8))
                    chunk_to_lds(own, c, pre_k[i], pre_v[i]);
            }
            pre_pending = false;
        }
    };
    auto raw_block = [&](int u) -> int { return uniform_load(bt, min(u, max_units - 1) / SPB); };
    auto resolve = [&](int raw, bool &dead) -> int {
        const int b = __builtin_amdgcn_readfirstlane(raw);
        dead = (unsigned)b >= (unsigned)p.N;
        return dead ? 0 : b;
    };
    auto k_ptr = [&](int blk, int u) {
        return p.k_pool + (int64_t)blk * block_stride + head_off + (u % SPB) * (16 * D);
    };
    auto v_ptr = [&](int blk, int u) {
        return p.v_pool + (int64_t)blk * block_stride + head_off + (u % SPB) * (16 * D);
    };
    float *sm_m = smem;
    float *sm_l = smem + NW * 16;
    float *sm_o = smem + 2 * NW * 16;

    // Tile group g (QT consecutive tiles) of this slot: g = slot, slot + tiles_per_seq, ...
    for (int grp = slot; grp * QT * p.R < qlen; grp += p.tiles_per_seq) {
        // per tile t of the group: rows i0[t] .. i0[t] + nrows[t] - 1 of the sequence's new rows (nrows may be 0)
        int i0[QT], nrows[QT], crow = r / p.G;
        bool col_ok[QT];
        RowLimits lim[QT];
        int last_all = -1;  // the group's last row any column attends
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            i0[t] = (grp * QT + t) * p.R;
            nrows[t] = max(0, min(p.R, qlen - i0[t]));
            col_ok[t] = r < nrows[t] * p.G;  // column r: new row i0 + r / G, query head hk * G + r % G
            lim[t].lo = 0;
            lim[t].first = min(pos + i0[t], cap - 1);
            lim[t].all = min(pos + i0[t] + nrows[t] - 1, cap - 1);
            lim[t].col = col_ok[t] ? min(pos + i0[t] + crow, cap - 1) : -1;
            if (nrows[t] > 0)
                last_all = max(last_all, lim[t].all);
        }
        const int nb = (last_all + 1 + BS - 1) / BS;
        int b0 = 0, b1 = nb;
        if (SPLIT) {
            const int chunk = p.chunk_blocks > 0 ? p.chunk_blocks : (nb + p.num_splits - 1) / p.num_splits;
            b0 = min(split * chunk, nb);
            b1 = min(nb, b0 + chunk);
        }
        const int u_begin = b0 * SPB;
        const int u_end = min(b1 * SPB, (last_all + 1 + 15) >> 4);
        const int u_first = u_begin + wave;
        const int n_units = u_first < u_end ? (u_end - u_first + NW - 1) / NW : 0;

        f16x8 qf[QT][KC];
        f32x4 o[QT][VC];
        float m_run[QT], l_run[QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            const int tok = q0 + i0[t] + (col_ok[t] ? crow : 0);
            const int hq = hk * p.G + (col_ok[t] ? r % p.G : 0);
            const _Float16 *qrow = p.q + ((int64_t)min(tok, p.T - 1) * p.Hq + hq) * D + 8 * g4;
#pragma unroll
            for (int c = 0; c < KC; ++c)
                qf[t][c] = *reinterpret_cast<const f16x8 *>(qrow + 32 * c);
#pragma unroll
            for (int c = 0; c < VC; ++c)
                o[t][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
            m_run[t] = kNegBig;
            l_run[t] = 0.f;
        }

        if (n_units > 0) {
            Frag<D, BS> f[NS];
            bool dead[NS];
            int uu[NS];
            int raw_q[NS];
            int blk_of[NS];  // block of each pipeline slot (the fused step writes its patched units back there)
#pragma unroll
            for (int j = 0; j < NS - 1; ++j) {
                uu[j] = u_first + j * NW;
                const int blk = resolve(start_known ? spec_raw[j] : raw_block(uu[j]), dead[j]);
                blk_of[j] = blk;
                load_unit<D, BS>(f[j], k_ptr(blk, uu[j]), v_ptr(blk, uu[j]), k_lane, v_lane,
                                 j < n_units && !dead[j]);
            }
#pragma unroll
            for (int j = 0; j < NS; ++j)
                raw_q[j] = start_known ? spec_raw[NS - 1 + j]
                                       : raw_block(u_first + min(NS - 1 + j, n_units - 1) * NW);
            if (FUSED)
                flush_pre();
            int k = 0;
            for (;;) {
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const int jn = (j + NS - 1) % NS;
                    uu[jn] = u_first + min(k + NS - 1, n_units - 1) * NW;
                    const int blk = resolve(raw_q[j], dead[jn]);
                    blk_of[jn] = blk;
                    load_unit<D, BS>(f[jn], k_ptr(blk, uu[jn]), v_ptr(blk, uu[jn]), k_lane, v_lane,
                                     k + NS - 1 < n_units && !dead[jn]);
                    raw_q[j] = raw_block(u_first + min(k + 2 * NS - 1, n_units - 1) * NW);
                    if (FUSED) {  // the unit's new rows (if any) patched in and the unit written back, once per load
                        const int kslot = uu[j] - nu0;
                        if (kslot >= 0 && kslot < n_new_units) {  // wave-uniform
                            const int prow = max(pos, 16 * uu[j]) - 16 * uu[j];
                            const int prow_end = min(pos + qlen, 16 * uu[j] + 16) - 16 * uu[j];
                            const _Float16 *sk = sm_new + kslot * 32 * D;
                            patch_unit_rows<D, BS>(f[j], prow, prow_end, sk, sk + 16 * D,
                                                   p.k_dst + (k_ptr(blk_of[j], uu[j]) - p.k_pool),
                                                   p.v_dst + (v_ptr(blk_of[j], uu[j]) - p.v_pool), dead[j], r, g4,
                                                   k_lane, v_lane);
                        }
                    }
                    // Every tile of the group uses this unit's fragments.  Later tiles first: a tile zeroes the V
                    // rows past its own last row, which every earlier tile leaves unused too.
#pragma unroll
                    for (int t = QT - 1; t >= 0; --t) {
                        if (nrows[t] > 0)  // wave-uniform
                            compute_unit<D, BS>(f[j], qf[t], o[t], m_run[t], l_run[t], uu[j], lim[t], dead[j], r, g4,
                                                p.scale_log2, -1, nullptr, nullptr, nullptr, nullptr, k_lane, v_lane);
                    }
                    if (++k >= n_units)
                        goto tile_done;
                }
            }
        tile_done:;
        }

        // cross-wave merge, as in decode_kernel, one tile of the group after the other through the same LDS
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            if (nrows[t] == 0)
                break;  // later tiles of the group are empty too
            const float lt = rows_sum(l_run[t]);
            if (grp != slot || t > 0)
                __syncthreads();  // the previous merge has read the LDS
            if (g4 == 0) {
                sm_m[wave * 16 + r] = m_run[t];
                sm_l[wave * 16 + r] = lt;
            }
            __syncthreads();
            float Mc = kNegBig;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                Mc = fmaxf(Mc, sm_m[w * 16 + r]);
            float den = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                den += exp2_fast(sm_m[w * 16 + r] - Mc) * sm_l[w * 16 + r];
            const int64_t my_row = (int64_t)(q0 + i0[t] + crow) * p.Hq + hk * p.G + r % p.G;  // token * Hq + hq
            {
                const float a = exp2_fast(m_run[t] - Mc);
                const float fs = SPLIT ? a : (den > 0.f ? a / den : 0.f);
                if (col_ok[t]) {  // 16-byte writes: with DP = D + 4 the eight lanes of a pass hit distinct banks
                    float *dst = sm_o + (wave * 16 + r) * DP + 4 * g4;
#pragma unroll
                    for (int c = 0; c < VC; ++c)
                        *reinterpret_cast<f32x4 *>(dst + 16 * c) = o[t][c] * fs;
                }
                if (SPLIT && wave == 0 && g4 == 0 && col_ok[t]) {
                    // a split without rows (b0 >= b1) leaves M = -1e30 and l = 0: weight 0 in the combine
                    p.part_m[my_row * p.num_splits + split] = Mc * kLn2;
                    p.part_l[my_row * p.num_splits + split] = den;
                }
            }
            __syncthreads();
            // four dims per thread, as in decode_kernel
            const int ncols = nrows[t] * p.G;
            for (int idx = threadIdx.x; idx < ncols * (D / 4); idx += NW * 64) {
                const int c = idx / (D / 4);
                const int d = 4 * (idx - c * (D / 4));
                f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    num += *reinterpret_cast<const f32x4 *>(sm_o + (w * 16 + c) * DP + d);
                const int64_t row = (int64_t)(q0 + i0[t] + c / p.G) * p.Hq + hk * p.G + c % p.G;  // token * Hq + hq
                if (!SPLIT) {
                    f16x4 y;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y[e] = (_Float16)num[e];
                    *reinterpret_cast<f16x4 *>(p.out + row * D + d) = y;
                } else {
                    *reinterpret_cast<f32x4 *>(p.part_o + (row * p.num_splits + split) * D + d) = num;
                }
            }
        }
    }
}

// Split-K phase 2: one wavefront per (sequence, query head), lanes over dims.
// out = sum_j e^(m_j - M) O_j / sum_j e^(m_j - M) l_j over the non-empty splits.
// Up to 64 splits (lane j holds m_j, l_j), every load the row needs is issued before its length arrives -- the
// partials of splits past the last non-empty one are read but never used -- so the kernel waits on memory once;
// the weights reach the dim lanes by lane broadcast.  More splits take the general loop.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    constexpr int PER = (D + 63) / 64;
    constexpr int CH = 8;  // splits whose outputs are requested together
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // s * Hq + hq
    if (row >= p.B * p.Hq)
        return;
    const int s = row / p.Hq;
    const int S = p.num_splits;
    const int64_t base = (int64_t)row * S;
    const bool fast = S <= 64;
    float mj = kNegBig, lj = 0.f, o0[CH][PER];
    if (fast) {
        if (lane < S) {
            mj = p.part_m[base + lane];
            lj = p.part_l[base + lane];
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int d = lane + 64 * k;
                o0[c][k] = (c < S && d < D) ? p.part_o[(base + c) * D + d] : 0.f;
            }
        }
    }
    int nvalid = S;  // no lengths: every split was written (varlen phase 1)
    if (p.context_lens != nullptr) {
        int L = p.context_lens[s];
        L = L < 0 ? 0 : (L > p.M * p.BS ? p.M * p.BS : L);
        const int nb = (L + p.BS - 1) / p.BS;
        const int b_lo = ((p.window > 0 && L > p.window) ? L - p.window : 0) / p.BS;
        nvalid = 0;
        if (nb > b_lo) {
            const int n = nb - b_lo;
            const int chunk = p.chunk_blocks > 0 ? p.chunk_blocks : (n + S - 1) / S;
            nvalid = min(S, (n + chunk - 1) / chunk);
        }
    }
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k)
        acc[k] = 0.f;
    float den = 0.f;
    if (fast) {
        float M = lane < nvalid ? mj : kNegBig;
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1)
            M = fmaxf(M, xor_lane(M, mask));
        const float a_lane = lane < nvalid ? expf(mj - M) : 0.f;
        den = lane < nvalid ? a_lane * lj : 0.f;
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1)
            den += xor_lane(den, mask);
        for (int j0 = 0; j0 < nvalid; j0 += CH) {
            float o[CH][PER];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    const int d = lane + 64 * k;
                    o[c][k] = j0 == 0 ? o0[c][k]
                                      : ((j0 + c < S && d < D) ? p.part_o[(base + j0 + c) * D + d] : 0.f);
                }
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int j = j0 + c;
                const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a_lane), j < 64 ? j : 63));
                if (j < nvalid) {
#pragma unroll
                    for (int k = 0; k < PER; ++k)
                        acc[k] += a * o[c][k];
                }
            }
        }
    } else {
        float M = kNegBig;
        for (int j = lane; j < nvalid; j += 64)
            M = fmaxf(M, p.part_m[base + j]);
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1)
            M = fmaxf(M, xor_lane(M, mask));
        for (int j = 0; j < nvalid; ++j) {
            const float a = expf(p.part_m[base + j] - M);
            den += a * p.part_l[base + j];
            const float *oj = p.part_o + (base + j) * D;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int d = lane + 64 * k;
                if (d < D)
                    acc[k] += a * oj[d];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int d = lane + 64 * k;
        if (d < D)
            p.out[(int64_t)row * D + d] = (_Float16)(den > 0.f ? acc[k] / den : 0.f);
    }
}

// The appends' thread order: one thread per (token, kv head, 8-dim piece), in groups of four tokens -- thread
// ((t/4 * Hkv + h) * D/8 + c) * 4 + t%4 -- so that a wavefront reads whole rows of the [T][Hkv][D] input (four
// tokens' rows of one head; a tokens-fastest order read each 128-byte line for one 16-byte piece, 8x the input
// bytes), four neighbouring lanes write a row's 64-byte K run ([D/32][16][32] panel), and the lanes of one piece
// write four consecutive tokens' values side by side in a V quad ([4][D][4]), whole 64-byte runs when the tokens'
// rows are consecutive (a sequence's new rows).
struct AppendThread {
    int i;  // token (>= T for the padding of the last group)
    int h;  // kv head
    int c;  // 8-dim piece
};
__device__ __forceinline__ AppendThread append_thread(int64_t gid, int Hkv, int pieces) {
    AppendThread a;
    const int64_t g = gid >> 2;  // (t/4 * Hkv + h) * pieces + c
    a.c = (int)(g % pieces);
    const int64_t th = g / pieces;
    a.h = (int)(th % Hkv);
    a.i = (int)((th / Hkv) * 4 + (gid & 3));
    return a;
}
__host__ __device__ constexpr int64_t append_threads(int64_t T, int Hkv, int D) {
    return (T + 3) / 4 * 4 * Hkv * (D / 8);
}

// Paged KV append [kapsl-backends 0.1.1, src/gguf_native.rs: launch_kv_write,
// launch_batch_kv_write]: each thread (order above) copies one 8-dim piece of a
// token's K and V rows: one 16-byte K store into the row's 64-byte run of its
// 32-dim group in the panel (a row touches D/32 lines), and 8 two-byte V stores
// 8 bytes apart into the row's quad of the V panel, two 32-byte sectors.
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const int pieces = p.D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= append_threads(p.T, p.Hkv, p.D))
        return;
    const AppendThread a = append_thread(gid, p.Hkv, pieces);
    const int i = a.i, h = a.h, c = a.c;
    if (i >= p.T)
        return;
    const int64_t th = (int64_t)i * p.Hkv + h;  // token * Hkv + head
    const int64_t slot = p.slot_mapping[i];
    if (slot < 0 || slot >= (int64_t)p.N * p.BS)
        return;
    const int64_t blk = slot / p.BS;
    const int off = (int)(slot - blk * p.BS);
    const int64_t src = th * p.D + 8 * c;
    const uint4 kv = *reinterpret_cast<const uint4 *>(p.k + src);
    const uint4 vv = *reinterpret_cast<const uint4 *>(p.v + src);
    // the row's 16-row panel inside the (block, kv head) tile
    const int64_t panel = (blk * p.Hkv + h) * (int64_t)p.BS * p.D + (int64_t)(off / 16) * 16 * p.D;
    const int row = off % 16;
    *reinterpret_cast<uint4 *>(p.k_pool + panel + ((int64_t)(c >> 2) * 16 + row) * 32 + 8 * (c & 3)) = kv;  // [D/32][16][32]
    const uint16_t *vh = reinterpret_cast<const uint16_t *>(&vv);
    uint16_t *vdst = reinterpret_cast<uint16_t *>(p.v_pool + panel + (int64_t)(row >> 2) * 4 * p.D + 32 * c +
                                                  (row & 3));  // V panel [4][D][4]: dims 8c .. 8c+7 of the row
#pragma unroll
    for (int e = 0; e < 8; ++e)
        vdst[e * 4] = vh[e];
}

constexpr int kOrderSeqsPerGroup = 64;  // sequences one order workgroup ranks
// LDS of a ranking workgroup: all B keys rounded up to 4, and four 8-byte partial sums
__host__ __device__ constexpr size_t order_lds_bytes(int B) { return sizeof(int) * ((size_t)(B + 3) / 4 * 4 + 8); }
template <bool VARLEN>
__device__ __forceinline__ void rank_into_records(const int32_t *__restrict__ lens, const int32_t *__restrict__ cu,
                                                  const int32_t *__restrict__ pos,
                                                  const int32_t *__restrict__ block_tables, int B, int M, int cap_rows,
                                                  int window, int32_t *__restrict__ order, int group, int *keys,
                                                  const PieceRule &pieces);

// The decode step's append as its own launch: the new row of sequence s (block bt[s][(L-1)/BS], row (L-1)%BS, as
// the fused step places it) for every kv head.  One workgroup per (sequence, kv head), each thread one 16-byte
// chunk.  In the K panel the row is D/32 runs of 64 bytes (whole 32-byte sectors, half a line each), written as they
// are; in the V panel its values are 2-byte fields spread over the D/16 lines of its quad, and those lines are
// rewritten whole (read, replace the row's fields, write back), so no partial sector is ever written.  Valid only
// because the block holding a sequence's newest row belongs to that sequence alone.
// With p.order set, the workgroups past the T * Hkv appends write the dispatch-order records instead (the ranking
// of launch_order, in the same launch as the append).
__global__ __launch_bounds__(256) void append_newest_kernel(AppendParams p) {
    if (p.order != nullptr && blockIdx.x >= (unsigned)(p.T * p.Hkv)) {
        extern __shared__ int keys[];
        rank_into_records<false>(p.context_lens, nullptr, nullptr, p.block_tables, p.T, p.M, p.order_cap,
                                 p.order_window, p.order, (int)(blockIdx.x - (unsigned)(p.T * p.Hkv)), keys,
                                 p.pieces);
        return;
    }
    const int s = (int)(blockIdx.x / (unsigned)p.Hkv);
    const int h = (int)(blockIdx.x - (unsigned)s * p.Hkv);
    int L = p.context_lens[s];
    L = L > p.M * p.BS ? p.M * p.BS : L;
    if (L <= 0)
        return;
    const int b = p.block_tables[(int64_t)s * p.M + (L - 1) / p.BS];
    if (b < 0 || b >= p.N)
        return;
    const int off = (L - 1) % p.BS;
    const int row = off % 16;
    const int64_t panel = ((int64_t)b * p.Hkv + h) * p.BS * p.D + (int64_t)(off / 16) * 16 * p.D;
    const _Float16 *kn = p.k + ((int64_t)s * p.Hkv + h) * p.D;
    const _Float16 *vn = p.v + ((int64_t)s * p.Hkv + h) * p.D;
    // One 16-byte chunk per thread (head_dim <= 256, so D/8 K chunks and D/2 V chunks fit the 256 threads).
    const int q = (int)threadIdx.x;
    if (q < p.D / 8) {
        // K panel [D/32][16][32]: dims 8q .. 8q+7 of the row, in the 64-byte run of its 32-dim group q / 4
        *reinterpret_cast<f16x8 *>(p.k_pool + panel + ((q >> 2) * 16 + row) * 32 + 8 * (q & 3)) =
            *reinterpret_cast<const f16x8 *>(kn + 8 * q);
    }
    if (q < p.D / 2) {
        // V panel [4][D][4]: the row's quad; chunk q holds dims 2q (its first 8 bytes) and 2q + 1 (its last 8), four
        // rows each, so the row is 16-bit field row % 4 of both halves
        uint64_t *dst = reinterpret_cast<uint64_t *>(p.v_pool + panel + (row >> 2) * 4 * p.D + 8 * q);
        const int sh = 16 * (row & 3);
        const uint64_t keep = ~(0xFFFFull << sh);
        const uint16_t *vbits = reinterpret_cast<const uint16_t *>(vn);
        const uint64_t a = dst[0], b = dst[1];
        dst[0] = (a & keep) | ((uint64_t)vbits[2 * q] << sh);
        dst[1] = (b & keep) | ((uint64_t)vbits[2 * q + 1] << sh);
    }
}

// The varlen step's append as its own launch: token t of sequence s (tokens cu[s] .. cu[s+1]-1) goes to row
// pos[s] + (t - cu[s]) of the sequence, through its block table.  One thread per (token, kv head, 8-dim piece), in
// the order of append_kernel; the token's sequence by binary search of the prefix sums.  Rows past the table's
// capacity and table entries outside the pool are skipped.
__global__ __launch_bounds__(256) void append_varlen_kernel(AppendParams p, const int32_t *cu, const int32_t *pos,
                                                            int num_seqs) {
    const int pieces = p.D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= append_threads(p.T, p.Hkv, p.D))
        return;
    const AppendThread a = append_thread(gid, p.Hkv, pieces);
    const int i = a.i, h = a.h, c = a.c;
    if (i >= p.T)
        return;
    int lo = 0, hi = num_seqs - 1;  // the last s with cu[s] <= i
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= i)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int64_t row = (int64_t)pos[lo] + (i - cu[lo]);
    if (row < 0 || row >= (int64_t)p.M * p.BS || i >= cu[lo + 1])
        return;
    const int32_t blk = p.block_tables[(int64_t)lo * p.M + row / p.BS];
    if (blk < 0 || blk >= p.N)
        return;
    const int off = (int)(row % p.BS);
    const int64_t src = ((int64_t)i * p.Hkv + h) * p.D + 8 * c;
    const uint4 kv = *reinterpret_cast<const uint4 *>(p.k + src);
    const uint4 vv = *reinterpret_cast<const uint4 *>(p.v + src);
    const int64_t panel = ((int64_t)blk * p.Hkv + h) * (int64_t)p.BS * p.D + (int64_t)(off / 16) * 16 * p.D;
    const int prow = off % 16;
    *reinterpret_cast<uint4 *>(p.k_pool + panel + ((int64_t)(c >> 2) * 16 + prow) * 32 + 8 * (c & 3)) = kv;
    const uint16_t *vh = reinterpret_cast<const uint16_t *>(&vv);
    uint16_t *vdst = reinterpret_cast<uint16_t *>(p.v_pool + panel + (int64_t)(prow >> 2) * 4 * p.D + 32 * c +
                                                  (prow & 3));
#pragma unroll
    for (int e = 0; e < 8; ++e)
        vdst[e * 4] = vh[e];
}

// The varlen step's append by panel: workgroup (s, h, j) takes the j-th 16-row unit that sequence s's new rows touch
// (rows pos[s] .. pos[s] + n - 1, n = cu[s+1] - cu[s], clipped to 0 .. M*BS - 1), stages those rows of kv head h in
// LDS and writes their K runs and the V quads that hold them, the quads' old rows as read, so the pools see
// whole-sector and whole-line writes only (as append_newest_kernel; the per-row form above scatters 2-byte V stores;
// rewriting both panels whole moved 5x the new rows' bytes).  Valid only
// because the blocks receiving a sequence's new rows belong to that sequence alone.  units: unit slots per sequence,
// enough for max_q_len rows from any offset in a unit; rows past them are not written.  With p.order set, the
// workgroups past num_seqs * Hkv * units write the varlen dispatch-order records instead (as order_varlen_kernel;
// placed first in the grid, they made the attention launch that follows slower, c4-shaped decode by 13 us).  Head
// dim at most 256 (two 16-byte chunks of each panel per thread).  Dynamic LDS: max(2 * 16 * D halves, the keys).
__global__ __launch_bounds__(256) void append_varlen_panels_kernel(AppendParams p, const int32_t *cu,
                                                                   const int32_t *pos, int num_seqs, int units) {
    extern __shared__ __align__(16) unsigned char panel_lds[];
    const unsigned per_seq = (unsigned)p.Hkv * (unsigned)units;
    const unsigned appends = (unsigned)num_seqs * per_seq;
    if (blockIdx.x >= appends) {
        rank_into_records<true>(nullptr, cu, pos, p.block_tables, num_seqs, p.M, p.order_cap, 0, p.order,
                                (int)(blockIdx.x - appends), reinterpret_cast<int *>(panel_lds), PieceRule{});
        return;
    }
    const int s = (int)(blockIdx.x / per_seq);
    const int rem = (int)(blockIdx.x - (unsigned)s * per_seq);
    const int h = rem / units;
    const int j = rem - h * units;
    const int64_t first = pos[s];
    const int64_t cap = (int64_t)p.M * p.BS;
    const int64_t lo = first < 0 ? 0 : first;
    int64_t hi = first + ((int64_t)cu[s + 1] - cu[s]);
    hi = hi > cap ? cap : hi;
    const int64_t r0 = (lo / 16 + j) * 16;  // this workgroup's unit: rows r0 .. r0 + 15 of the sequence
    if (lo >= hi || r0 >= hi)
        return;
    const int b = p.block_tables[(int64_t)s * p.M + r0 / p.BS];
    if (b < 0 || b >= p.N)
        return;
    const int a = (int)((lo > r0 ? lo : r0) - r0);         // new rows of the unit: a .. e - 1
    const int e = (int)((hi < r0 + 16 ? hi : r0 + 16) - r0);
    const int64_t panel = ((int64_t)b * p.Hkv + h) * p.BS * p.D + (r0 % p.BS) * p.D;
    // Only what holds new rows is written: in the K panel [D/32][16][32] (chunk q: dims 8 * (4 * (q / 64) + q % 4)
    // .. +8 of row (q / 4) % 16) a new row's own 64-byte runs, which need no read; in the V panel [4][D][4] (chunk q:
    // dims 2*(q % (D/2)) and the next of quad q / (D/2), i.e. of rows 4*(q / (D/2)) .. +4) the quads that hold new
    // rows, whole 128-byte lines -- a quad that also holds old rows is read first (before the staging, so both sets
    // of loads are in flight together) and written back with them unchanged.
    const int qpd = p.D / 2;  // V chunks per quad
    f16x8 vc[2] = {};
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int q = (int)threadIdx.x + 256 * it;
        if (q < 2 * p.D) {
            const int vr = 4 * (q / qpd);
            if (vr + 3 >= a && vr < e && (vr < a || vr + 4 > e))
                vc[it] = *reinterpret_cast<const f16x8 *>(p.v_pool + panel + 8 * q);
        }
    }
    const int pieces = p.D / 8;
    f16x8 *kst = reinterpret_cast<f16x8 *>(panel_lds);  // [16][D/8]
    f16x8 *vst = kst + 16 * pieces;                      // [16][D/8]
    const int64_t t0 = (int64_t)cu[s] + (r0 - first);  // token of unit row r (used for a <= r < e only)
    for (int i = threadIdx.x; i < 16 * pieces; i += 256) {
        const int r = i / pieces;
        if (r >= a && r < e && t0 + r < p.T) {  // (t0 + r >= cu[s] >= 0; the bound holds for valid prefix sums)
            const int64_t src = ((t0 + r) * p.Hkv + h) * p.D + 8 * (i - r * pieces);
            kst[i] = *reinterpret_cast<const f16x8 *>(p.k + src);
            vst[i] = *reinterpret_cast<const f16x8 *>(p.v + src);
        }
    }
    __syncthreads();
    const _Float16 *vsh = reinterpret_cast<const _Float16 *>(vst);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int q = (int)threadIdx.x + 256 * it;
        if (q < 2 * p.D) {
            const int kr = (q >> 2) & 15;
            if (kr >= a && kr < e)
                *reinterpret_cast<f16x8 *>(p.k_pool + panel + 8 * q) = kst[kr * pieces + 4 * (q >> 6) + (q & 3)];
            const int vq = q / qpd, d0 = 2 * (q - vq * qpd);
            if (4 * vq + 3 >= a && 4 * vq < e) {
#pragma unroll
                for (int x = 0; x < 8; ++x) {  // element x: dim d0 + x / 4 of row 4 * vq + x % 4
                    const int vr = 4 * vq + (x & 3);
                    if (vr >= a && vr < e)
                        vc[it][x] = vsh[vr * p.D + d0 + (x >> 2)];
                }
                *reinterpret_cast<f16x8 *>(p.v_pool + panel + 8 * q) = vc[it];
            }
        }
    }
}

// Dispatch order for a multi-round decode grid: each sequence is ranked against every other by the rows it attends
// (descending, ties by index), so the ranks are a permutation, and its record is written at its rank.  Every
// workgroup holds all B keys in LDS (padded to a multiple of 4 with -1, which never counts) and ranks 64 sequences,
// four lanes per sequence, each lane scanning a quarter of the keys 16 bytes at a time; the quad sums its counts.
// One workgroup's share (sequences group * 64 ..) of the ranking; keys: LDS for all B keys, rounded up to 4.
// A key (rows) longer than the piece rows C in pieces: ceil(key / C) pieces of equal rows rounded up to 64 (so each
// starts on a block), and the count of those pieces that the key fills: (rows of each but the last, pieces).  Out of
// line: the ranking calls it only for the rare keys past C.
__device__ __noinline__ int2 piece_split(int key, int C) {
    const int64_t n = ((int64_t)key + C - 1) / C;
    const int64_t pr = (((int64_t)key + n - 1) / n + 63) / 64 * 64;
    return make_int2((int)pr, (int)(((int64_t)key + pr - 1) / pr));
}

// Decode (VARLEN false): key = rows attended, min(clamp(L, 0, cap_rows), window) with window > 0; records as
// launch_order describes them (pieces.records > 0 and no window: the longest sequences split into pieces, see
// PieceRule).  Varlen: key = clamp(pos[s] + new rows, 0, cap_rows), the rows its last new row attends; record =
// sequence, cu[s], cu[s + 1], pos[s], then its first kVarlenRecBlocks table entries.
// keys: LDS for all B keys rounded up to 4, plus 8 ints.
template <bool VARLEN>
__device__ __forceinline__ void rank_into_records(const int32_t *__restrict__ lens, const int32_t *__restrict__ cu,
                                                  const int32_t *__restrict__ pos,
                                                  const int32_t *__restrict__ block_tables, int B, int M, int cap_rows,
                                                  int window, int32_t *__restrict__ order, int group, int *keys,
                                                  const PieceRule &pieces) {
    constexpr int kHead = VARLEN ? 4 : kOrderRecHead;
    constexpr int kBlocks = kOrderRecord - kHead;
    const int B4 = (B + 3) / 4;
    int64_t my_sum = 0;  // this thread's share of the rows of all sequences (the piece rule's fair share)
    for (int i = threadIdx.x; i < 4 * B4; i += 256) {
        int key = -1;
        if (i < B) {
            if (VARLEN) {
                const int64_t n = (int64_t)cu[i + 1] - cu[i];
                const int64_t rows = (int64_t)pos[i] + (n > 0 ? n : 0);
                key = rows < 0 ? 0 : (rows > cap_rows ? cap_rows : (int)rows);
            } else {
                int L = lens[i];
                L = L < 0 ? 0 : (L > cap_rows ? cap_rows : L);
                key = window > 0 && L > window ? window : L;
            }
            my_sum += key;
        }
        keys[i] = key;
    }
    const bool split = !VARLEN && pieces.records > 0 && window <= 0;  // (uniform)
    int64_t *sums = reinterpret_cast<int64_t *>(keys + 4 * B4);
    if (split) {
        // the sum of all keys: wave sums, then the four waves' through LDS (8-byte aligned: 4 * B4 ints is even)
        for (int m = 32; m >= 1; m >>= 1)
            my_sum += __shfl_xor(my_sum, m);
        if ((threadIdx.x & 63) == 0)
            sums[threadIdx.x >> 6] = my_sum;
    }
    const int s = group * kOrderSeqsPerGroup + (int)(threadIdx.x >> 2);
    const int part = (int)(threadIdx.x & 3);
    // this lane's share of the record's table entries (i = part, part + 4, ...), requested before the scan
    const int nb = M < kBlocks ? M : kBlocks;
    constexpr int kPer = (kBlocks + 3) / 4;
    int ids[kPer];
    // clamped into the table, so every load is unconditional (entries past nb and rows past B are never stored)
    const int32_t *trow = block_tables + (int64_t)(s < B ? s : B - 1) * M;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = part + 4 * k;
        ids[k] = nb > 0 ? trow[i < nb ? i : nb - 1] : 0;
    }
    __syncthreads();
    if (s >= B)
        return;  // the whole quad of s leaves together
    // piece rows C (a key longer than C is split): INT32_MAX when nothing is split, so that every key compares
    // below it
    int C = INT32_MAX;
    if (split) {
        const int64_t total = sums[0] + sums[1] + sums[2] + sums[3];
        const int64_t fair = (total * pieces.hkv + pieces.cus - 1) / (pieces.cus > 0 ? pieces.cus : 1);
        const int64_t c = (fair + 63) / 64 * 64;
        C = c < kMinPieceRows ? kMinPieceRows : (c > INT32_MAX ? INT32_MAX : (int)c);
    }
    const int ks = keys[s];
    int rank = 0, extra = 0;  // extra: the pieces past the first of the sequences ranked before s
    const int4 *k4 = reinterpret_cast<const int4 *>(keys);
#pragma unroll 4
    for (int j4 = part; j4 < B4; j4 += 4) {
        const int4 kv = k4[j4];
        const int j = 4 * j4;
        const bool bx = kv.x > ks || (kv.x == ks && j < s);
        const bool by = kv.y > ks || (kv.y == ks && j + 1 < s);
        const bool bz = kv.z > ks || (kv.z == ks && j + 2 < s);
        const bool bw = kv.w > ks || (kv.w == ks && j + 3 < s);
        rank += (bx ? 1 : 0) + (by ? 1 : 0) + (bz ? 1 : 0) + (bw ? 1 : 0);
        if (bx && kv.x > C)  // (rare: only keys past a CU's fair share)
            extra += piece_split(kv.x, C).y - 1;
        if (by && kv.y > C)
            extra += piece_split(kv.y, C).y - 1;
        if (bz && kv.z > C)
            extra += piece_split(kv.z, C).y - 1;
        if (bw && kv.w > C)
            extra += piece_split(kv.w, C).y - 1;
    }
    rank += __shfl_xor(rank, 1);
    rank += __shfl_xor(rank, 2);
    extra += __shfl_xor(extra, 1);
    extra += __shfl_xor(extra, 2);
    const int start = rank + extra;
    const int2 split_s = ks > C ? piece_split(ks, C) : make_int2(ks, 1);
    const int pr = split_s.x;
    const int n = split_s.y;
    if (split) {
        // this launch's piece counters start at zero
        for (int h = part; h < pieces.hkv; h += 4)
            pieces.counters[(int64_t)s * pieces.hkv + h] = 0;
        // the last sequence in the order marks the records past the last piece unused
        if (rank == B - 1)
            for (int r = start + n + part; r < pieces.records; r += 4)
                order[(int64_t)r * kOrderRecord] = -1;
    }
    for (int pc = 0; pc < n; ++pc) {
        if (split && start + pc >= pieces.records)
            break;  // (never: the extra records number less than cus / hkv)
        int32_t *rec = order + (int64_t)(start + pc) * kOrderRecord;
        const int u0 = pc * (pr / 16);
        if (part == 0) {
            rec[0] = s;
            if (VARLEN) {
                rec[1] = cu[s];
                rec[2] = cu[s + 1];
                rec[3] = pos[s];
            } else {
                rec[1] = lens[s];
                rec[2] = u0;
                rec[3] = pc + 1 < n ? u0 + pr / 16 : INT32_MAX;
                rec[4] = pc | (n << 16);
                rec[5] = start;
            }
        }
        if (pc == 0) {  // (a later piece's workgroups read their first block ids from the table themselves)
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int i = part + 4 * k;
                if (i < nb)
                    rec[kHead + i] = ids[k];
            }
        }
    }
}

__global__ __launch_bounds__(256) void order_kernel(const int32_t *__restrict__ lens,
                                                    const int32_t *__restrict__ block_tables, int B, int M,
                                                    int cap_rows, int window, int32_t *__restrict__ order,
                                                    PieceRule pieces) {
    extern __shared__ int keys[];
    rank_into_records<false>(lens, nullptr, nullptr, block_tables, B, M, cap_rows, window, order, (int)blockIdx.x,
                             keys, pieces);
}

__global__ __launch_bounds__(256) void order_varlen_kernel(const int32_t *__restrict__ cu,
                                                           const int32_t *__restrict__ pos,
                                                           const int32_t *__restrict__ block_tables, int B, int M,
                                                           int cap_rows, int32_t *__restrict__ order) {
    extern __shared__ int keys[];
    rank_into_records<true>(nullptr, cu, pos, block_tables, B, M, cap_rows, 0, order, (int)blockIdx.x, keys,
                            PieceRule{});
}

// ---------------------------------------------------------------------------
// launchers

template <int D, int BS, int NW>
static hipError_t launch_decode_t(const DecodeParams &p, int num_seqs, bool split, hipStream_t stream) {
    // an ordered single pass has a workgroup per (record, kv head); a record may be a piece of a sequence
    const int64_t rows = p.order != nullptr && !split && p.order_records > 0 ? p.order_records : num_seqs;
    dim3 grid((unsigned)(rows * p.Hkv * (split ? p.num_splits : 1)), 1u, 1u);
    dim3 block(NW * 64);
    const size_t lds = decode_lds_bytes(D, p.G, NW);
    const bool fused = p.k_new != nullptr;
    if (p.qkv != nullptr) {  // the decode step from QKV rows
        if (split)
            hipLaunchKernelGGL((decode_kernel<D, BS, NW, true, true, true>), grid, block, lds, stream, p);
        else
            hipLaunchKernelGGL((decode_kernel<D, BS, NW, false, true, true>), grid, block, lds, stream, p);
    } else if (p.order != nullptr && !fused) {  // a multi-round grid in dispatch order (never the one-launch step)
        if (split)
            hipLaunchKernelGGL((decode_kernel<D, BS, NW, true, false, false, true>), grid, block, lds, stream, p);
        else
            hipLaunchKernelGGL((decode_kernel<D, BS, NW, false, false, false, true>), grid, block, lds, stream, p);
    } else if (split && fused)
        hipLaunchKernelGGL((decode_kernel<D, BS, NW, true, true>), grid, block, lds, stream, p);
    else if (split)
        hipLaunchKernelGGL((decode_kernel<D, BS, NW, true, false>), grid, block, lds, stream, p);
    else if (fused)
        hipLaunchKernelGGL((decode_kernel<D, BS, NW, false, true>), grid, block, lds, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<D, BS, NW, false, false>), grid, block, lds, stream, p);
    return hipGetLastError();
}

template <int D, int BS>
static hipError_t launch_decode_w(const DecodeParams &p, int num_seqs, int waves, bool split, hipStream_t stream) {
    switch (waves) {
    case 1: return launch_decode_t<D, BS, 1>(p, num_seqs, split, stream);
    case 2: return launch_decode_t<D, BS, 2>(p, num_seqs, split, stream);
    case 4: return launch_decode_t<D, BS, 4>(p, num_seqs, split, stream);
    case 8:
        if constexpr (D >= 256)
            return hipErrorInvalidValue;
        else
            return launch_decode_t<D, BS, 8>(p, num_seqs, split, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
static hipError_t launch_decode_d(const DecodeParams &p, int num_seqs, int block_size, int waves, bool split,
                                  hipStream_t stream) {
    switch (block_size) {
    case 16: return launch_decode_w<D, 16>(p, num_seqs, waves, split, stream);
    case 32: return launch_decode_w<D, 32>(p, num_seqs, waves, split, stream);
    case 64: return launch_decode_w<D, 64>(p, num_seqs, waves, split, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeParams &p, int num_seqs, int head_dim, int block_size, int waves, bool split,
                         hipStream_t stream) {
    switch (head_dim) {
    case 64: return launch_decode_d<64>(p, num_seqs, block_size, waves, split, stream);
    case 128: return launch_decode_d<128>(p, num_seqs, block_size, waves, split, stream);
    case 256: return launch_decode_d<256>(p, num_seqs, block_size, waves, split, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int D, int BS, int NW>
static hipError_t launch_varlen_t(const VarlenParams &p, int num_seqs, bool split, hipStream_t stream) {
    dim3 grid((unsigned)((int64_t)num_seqs * p.tiles_per_seq * p.Hkv * (split ? p.num_splits : 1)), 1u, 1u);
    dim3 block(NW * 64);
    const bool fused = p.k_new != nullptr;
    const size_t lds = varlen_lds_bytes(D, NW, fused);
    if (fused && p.QT == 2) {  // the fused step runs as one pass; head dim 256 takes it with one tile per group
        if constexpr (D <= 128)
            hipLaunchKernelGGL((varlen_kernel<D, BS, NW, false, 2, true>), grid, block, lds, stream, p);
        else
            return hipErrorInvalidValue;
    } else if (fused)
        hipLaunchKernelGGL((varlen_kernel<D, BS, NW, false, 1, true>), grid, block, lds, stream, p);
    else if (p.order != nullptr) {  // a multi-round grid in dispatch order
        if (split && p.QT == 2)
            hipLaunchKernelGGL((varlen_kernel<D, BS, NW, true, 2, false, true>), grid, block, lds, stream, p);
        else if (split)
            hipLaunchKernelGGL((varlen_kernel<D, BS, NW, true, 1, false, true>), grid, block, lds, stream, p);
        else if (p.QT == 2)
            hipLaunchKernelGGL((varlen_kernel<D, BS, NW, false, 2, false, true>), grid, block, lds, stream, p);
        else
            hipLaunchKernelGGL((varlen_kernel<D, BS, NW, false, 1, false, true>), grid, block, lds, stream, p);
    }
    else if (split && p.QT == 2)
        hipLaunchKernelGGL((varlen_kernel<D, BS, NW, true, 2>), grid, block, lds, stream, p);
    else if (split)
        hipLaunchKernelGGL((varlen_kernel<D, BS, NW, true, 1>), grid, block, lds, stream, p);
    else if (p.QT == 2)
        hipLaunchKernelGGL((varlen_kernel<D, BS, NW, false, 2>), grid, block, lds, stream, p);
    else
        hipLaunchKernelGGL((varlen_kernel<D, BS, NW, false, 1>), grid, block, lds, stream, p);
    return hipGetLastError();
}
template <int D, int BS>
static hipError_t launch_varlen_w(const VarlenParams &p, int num_seqs, int waves, bool split, hipStream_t stream) {
    switch (waves) {
    case 1: return launch_varlen_t<D, BS, 1>(p, num_seqs, split, stream);
    case 2: return launch_varlen_t<D, BS, 2>(p, num_seqs, split, stream);
    case 4: return launch_varlen_t<D, BS, 4>(p, num_seqs, split, stream);
    case 8:
        if constexpr (D >= 256)
            return hipErrorInvalidValue;
        else
            return launch_varlen_t<D, BS, 8>(p, num_seqs, split, stream);
    default: return hipErrorInvalidValue;
    }
}
template <int D>
static hipError_t launch_varlen_d(const VarlenParams &p, int num_seqs, int block_size, int waves, bool split,
                                  hipStream_t stream) {
    switch (block_size) {
    case 16: return launch_varlen_w<D, 16>(p, num_seqs, waves, split, stream);
    case 32: return launch_varlen_w<D, 32>(p, num_seqs, waves, split, stream);
    case 64: return launch_varlen_w<D, 64>(p, num_seqs, waves, split, stream);
    default: return hipErrorInvalidValue;
    }
}
hipError_t launch_varlen(const VarlenParams &p, int num_seqs, int head_dim, int block_size, int waves, bool split,
                         hipStream_t stream) {
    switch (head_dim) {
    case 64: return launch_varlen_d<64>(p, num_seqs, block_size, waves, split, stream);
    case 128: return launch_varlen_d<128>(p, num_seqs, block_size, waves, split, stream);
    case 256: return launch_varlen_d<256>(p, num_seqs, block_size, waves, split, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine(const CombineParams &p, int head_dim, hipStream_t stream) {
    const int rows = p.B * p.Hq;
    dim3 grid((unsigned)((rows + 3) / 4));
    dim3 block(256);
    switch (head_dim) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, block, 0, stream, p); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_append_newest(const AppendParams &p, hipStream_t stream) {
    if (p.T <= 0)
        return hipSuccess;
    if (p.order != nullptr && p.T > kOrderMaxSeqs)
        return hipErrorInvalidValue;
    const unsigned order_groups = p.order ? (unsigned)((p.T + kOrderSeqsPerGroup - 1) / kOrderSeqsPerGroup) : 0u;
    const size_t lds = p.order ? order_lds_bytes(p.T) : 0;
    hipLaunchKernelGGL(append_newest_kernel, dim3((unsigned)((int64_t)p.T * p.Hkv) + order_groups), dim3(256), lds,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_append_varlen(const AppendParams &p, const int32_t *cu_seqlens_q, const int32_t *pos_offsets,
                                int num_seqs, int max_q_len, hipStream_t stream) {
    if (num_seqs <= 0)
        return hipSuccess;
    if (p.order != nullptr && num_seqs > kOrderMaxSeqs)
        return hipErrorInvalidValue;
    const unsigned order_groups =
        p.order ? (unsigned)((num_seqs + kOrderSeqsPerGroup - 1) / kOrderSeqsPerGroup) : 0u;
    // unit slots for max_q_len rows starting anywhere in a 16-row unit
    const int64_t units = max_q_len > 0 ? ((int64_t)max_q_len + 14) / 16 + 1 : 0;
    const int64_t panels = (int64_t)num_seqs * p.Hkv * units;
    if (units > 0 && p.T > 0 && p.D <= 256 && panels + order_groups <= kMaxGroups) {
        const size_t stage = sizeof(_Float16) * 2 * 16 * (size_t)p.D;
        const size_t keys = p.order ? order_lds_bytes(num_seqs) : 0;
        hipLaunchKernelGGL(append_varlen_panels_kernel, dim3((unsigned)panels + order_groups), dim3(256),
                           stage > keys ? stage : keys, stream, p, cu_seqlens_q, pos_offsets, num_seqs, (int)units);
        return hipGetLastError();
    }
    if (p.T > 0) {
        const int64_t total = append_threads(p.T, p.Hkv, p.D);
        hipLaunchKernelGGL(append_varlen_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p,
                           cu_seqlens_q, pos_offsets, num_seqs);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (p.order == nullptr)
        return hipSuccess;
    return launch_order_varlen(cu_seqlens_q, pos_offsets, p.block_tables, num_seqs, p.M, p.order_cap, p.order,
                               stream);
}

hipError_t launch_order(const int32_t *context_lens, const int32_t *block_tables, int B, int M, int cap_rows,
                        int window, int32_t *order, const PieceRule &pieces, hipStream_t stream) {
    if (B <= 0 || B > kOrderMaxSeqs)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(order_kernel, dim3((unsigned)((B + kOrderSeqsPerGroup - 1) / kOrderSeqsPerGroup)), dim3(256),
                       order_lds_bytes(B), stream, context_lens, block_tables, B, M, cap_rows, window, order, pieces);
    return hipGetLastError();
}

hipError_t launch_order_varlen(const int32_t *cu_seqlens_q, const int32_t *pos_offsets, const int32_t *block_tables,
                               int B, int M, int cap_rows, int32_t *order, hipStream_t stream) {
    if (B <= 0 || B > kOrderMaxSeqs)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(order_varlen_kernel, dim3((unsigned)((B + kOrderSeqsPerGroup - 1) / kOrderSeqsPerGroup)),
                       dim3(256), order_lds_bytes(B), stream, cu_seqlens_q, pos_offsets,
                       block_tables, B, M, cap_rows, order);
    return hipGetLastError();
}

hipError_t launch_append(const AppendParams &p, hipStream_t stream) {
    const int64_t total = append_threads(p.T, p.Hkv, p.D);
    dim3 grid((unsigned)((total + 255) / 256));
    dim3 block(256);
    hipLaunchKernelGGL(append_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
