// pkv_internal.h -- private interface between the host API (pkv_api.hip) and
// the kernels (pkv_kernels.hip, pkv_qkv.hip, pkv_check.hip).  Not installed; callers use include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Arguments of the decode-attention kernel (single pass and split-K phase 1).
// Fields the kernel needs first (before any K/V load) lead, so they arrive in its first kernel-argument loads.
struct DecodeParams {
    const _Float16 *q;            // [B][Hq][D]
    const int32_t *block_tables;  // [B][M]
    const int32_t *context_lens;  // [B]
    // fused decode step: when k_new is non-null, row L-1 of every sequence is first written from
    // k_new / v_new ([B][Hkv][D]) into k_dst / v_dst (the same pools)
    const _Float16 *k_new;
    const _Float16 *v_new;
    // decode step from the QKV projection rows (qkv non-null, fused launch only): q and each sequence's new K/V row
    // come from qkv[B][(Hq + 2*Hkv) * D], the query and key heads RMS-normalised (qk_mode 1) and rotated at
    // position L-1 (see the fields at the end); q_out receives the rotated queries
    const _Float16 *qkv;
    int32_t Hq, Hkv, G, N, M;
    int32_t num_splits;           // grid splits S (1 for a single pass)
    int32_t chunk_blocks;         // > 0 fixed blocks per split, 0 = ceil(blocks in range / S) per sequence
    float scale_log2;             // scale * log2(e)
    int32_t window;               // > 0: attend only the last `window` rows of each sequence; 0 = all rows
    const _Float16 *k_pool;       // [N][Hkv][BS/16][D/32][16][32]
    const _Float16 *v_pool;       // [N][Hkv][BS/16][4][D][4]
    _Float16 *out;                // [B][Hq][D]            (single pass)
    float *part_o;                // [B][Hq][S][D]         (split-K; ordered pieces: [records][Hq][D])
    float *part_m;                // [B][Hq][S]            (ordered pieces: [records][Hq], log2 units)
    float *part_l;                // [B][Hq][S]            (ordered pieces: [records][Hq])
    _Float16 *k_dst;
    _Float16 *v_dst;
    const _Float16 *q_norm_w;     // [D]
    const _Float16 *k_norm_w;     // [D]
    const float *cos_t;           // [P][D/2]
    const float *sin_t;           // [P][D/2]
    int32_t P;
    int32_t qk_mode;
    float eps;
    _Float16 *q_out;              // [B][Hq][D]
    // dispatch order (multi-round grids): workgroup tile t serves the sequence (or piece of one) of record
    // order[t / Hkv] (null: sequence t / Hkv); see kOrderRecord
    const int32_t *order;         // [order_records][kOrderRecord]
    int32_t order_records;        // records in order (a single pass: B plus room for pieces); 0: B
    int32_t *piece_count;         // [B][Hkv] pieces of a split tile done so far (zeroed by the ordering launch)
};

// Arguments of the varlen attention kernel (several new query rows per sequence).
struct VarlenParams {
    const _Float16 *q;            // [T][Hq][D] token-major
    const int32_t *block_tables;  // [B][M]
    const int32_t *cu_seqlens_q;  // [B+1]
    const int32_t *pos_offsets;   // [B]
    int32_t Hq, Hkv, G, N, M, T;
    int32_t R;                    // new rows per tile (16 / G)
    int32_t QT;                   // tiles per workgroup sharing each K/V load (1 or 2)
    int32_t tiles_per_seq;        // tile-group slots per (sequence, kv head) in the grid
    int32_t num_splits;           // 1 = one pass
    int32_t chunk_blocks;         // > 0 fixed blocks per split, 0 = ceil(nb / S) per tile
    float scale_log2;
    const _Float16 *k_pool;
    const _Float16 *v_pool;
    _Float16 *out;                // [T][Hq][D]                (one pass)
    float *part_o;                // [T][Hq][S][D]             (splits)
    float *part_m;                // [T][Hq][S]
    float *part_l;                // [T][Hq][S]
    // fused varlen step (k_new non-null, one pass): token t's K/V rows ([T][Hkv][D]) go to row pos[s] + i of its
    // sequence in k_dst / v_dst (the same pools)
    const _Float16 *k_new;
    const _Float16 *v_new;
    _Float16 *k_dst;
    _Float16 *v_dst;
    // dispatch order (multi-round grids, not with k_new): the sequence of workgroup group t / tiles_per_seq is that
    // of varlen record order[t / tiles_per_seq] (see launch_order_varlen); null: sequence t / tiles_per_seq
    const int32_t *order;
};

struct CombineParams {
    const float *part_o;
    const float *part_m;
    const float *part_l;
    const int32_t *context_lens;  // null: every split of every row was written (varlen)
    _Float16 *out;
    int32_t B, Hq, BS, M;
    int32_t num_splits, chunk_blocks;
    int32_t window;               // as DecodeParams::window (the split ranges start at the window's block)
};

// The pieces of a single-pass decode dispatch order.  A grid of several rounds still ends on its longest tile when
// that tile alone needs more rows than a CU's fair share of the launch (all rows times Hkv over the CUs): its CU
// streams alone at the end.  The ordering launch splits each sequence longer than
// C = max(kMinPieceRows, fair share rounded up to 64 rows) into ceil(rows / C) pieces of equal rows (rounded up to
// 64, so every piece starts on a block), one record each; the attention launch computes each piece as a tile and
// the last piece of a (sequence, kv head) to finish merges them.  The extra records number less than cus / hkv.
struct PieceRule {
    int32_t records;              // records the order array holds (B + ceil(cus / hkv)); 0: one per sequence
    int32_t cus;                  // CUs the launch spreads over
    int32_t hkv;                  // kv heads: tiles per record
    int32_t block_size;
    int32_t *counters;            // [B][hkv]: zeroed by the ordering launch, counted up by the pieces
};
constexpr int kMinPieceRows = 1024;

struct AppendParams {
    const _Float16 *k;            // [T][Hkv][D]
    const _Float16 *v;
    const int32_t *slot_mapping;  // [T]                 (launch_append)
    const int32_t *block_tables;  // [T][M]              (launch_append_newest: token i = sequence i's newest row)
    const int32_t *context_lens;  // [T]                 (launch_append_newest)
    _Float16 *k_pool;
    _Float16 *v_pool;
    int32_t T, Hkv, D, BS, N, M;
    // launch_append_newest and launch_append_varlen: when order is non-null, the launch also writes the
    // dispatch-order records of the sequences (as launch_order / launch_order_varlen, rows capped at order_cap,
    // window order_window for decode)
    int32_t *order;
    int32_t order_cap, order_window;
    PieceRule pieces;             // decode order: the longest sequences' pieces (records == 0: none)
};

// Arguments of the QKV-to-cache kernel (split QKV, q/k RMSNorm, RoPE, paged-cache write).
struct QkvParams {
    const _Float16 *qkv;          // [T][(Hq + 2*Hkv) * D]: query heads, key heads, value heads
    const _Float16 *q_norm_w;     // [D] (qk_mode 1)
    const _Float16 *k_norm_w;     // [D] (qk_mode 1)
    const float *cos_t;           // [P][D/2]
    const float *sin_t;           // [P][D/2]
    const int32_t *cu_seqlens_q;  // [B+1]; null: one sequence of T tokens at rope_base / cache_base
    const int32_t *pos_offsets;   // [B]: first new token's RoPE position and cache row
    const int32_t *block_tables;  // [B][M]
    const int32_t *decode_lens;   // [B] or null: token s is sequence s's new row, at position decode_lens[s] - 1
    int32_t B, T, Hq, Hkv, G, N, M, BS, P;
    int32_t qk_mode;              // 1: RMS-normalise query and key heads first; 0: rotate only
    int32_t rope_base, cache_base;
    int32_t hpp, parts;           // head slots (query heads, K, V) per workgroup, workgroups per (unit, kv head)
    float eps;
    _Float16 *q_out;              // [T][Hq][D]
    _Float16 *k_pool;
    _Float16 *v_pool;
};

// Arguments of the input checks (cold path): block tables with either context lengths (decode) or prefix sums and
// positions (varlen), or a slot mapping alone.
struct CheckParams {
    const int32_t *block_tables;  // [B][M]
    const int32_t *context_lens;  // [B] (decode) or null
    const int32_t *cu_seqlens_q;  // [B+1] (varlen) or null
    const int32_t *pos_offsets;   // [B] (varlen)
    const int32_t *slot_mapping;  // [T] (slot check) or null
    int32_t B, M, N, BS, T;
    int32_t window;               // decode: > 0 reads only the last `window` rows' blocks
    int32_t *report;              // [4]
};

// LDS bytes the decode kernel needs for `waves` wavefronts and group size G.
size_t decode_lds_bytes(int head_dim, int G, int waves);

// Kernel launchers: enqueue on `stream`, return the hipError_t of the launch.
hipError_t launch_decode(const DecodeParams &p, int num_seqs, int head_dim, int block_size, int waves,
                         bool split, hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, int head_dim, hipStream_t stream);
size_t varlen_lds_bytes(int head_dim, int waves, bool fused = false);
// New rows per sequence the one-launch varlen step holds in LDS.
constexpr int kStepFusedRows = 32;
// 16-row units of new rows the fused varlen step's workgroup stages: any kStepFusedRows consecutive rows fit.
constexpr int kFusedUnits = (kStepFusedRows + 2 * 15) / 16;
hipError_t launch_varlen(const VarlenParams &p, int num_seqs, int head_dim, int block_size, int waves, bool split,
                         hipStream_t stream);
hipError_t launch_append(const AppendParams &p, hipStream_t stream);
hipError_t launch_append_newest(const AppendParams &p, hipStream_t stream);
// Sequences that a multi-round decode grid can order longest first.
constexpr int kOrderMaxSeqs = 16384;
// Largest one-dimensional grid of 256-thread workgroups (a launch's threads along x must fit in 32 bits).
constexpr int64_t kMaxGroups = 0xFFFFFFFFll / 256;
// One record per rank of the dispatch order (per piece of a split sequence): the sequence, its length as stored,
// the piece's unit range and place, then the table entries of its first kOrderRecBlocks blocks -- everything a
// decode workgroup reads before its first K/V loads, in one place.
constexpr int kOrderRecord = 32;
constexpr int kOrderRecHead = 6;
constexpr int kOrderRecBlocks = kOrderRecord - kOrderRecHead;
// Records of the sequences sorted by the rows they attend (min(clamp(L, 0, cap_rows), window) with window > 0),
// longest first, ties by index; a sequence split into n pieces (see PieceRule) takes n consecutive records.
// order[r][0] = sequence (-1: an unused record), [1] = context_lens[sequence], [2] = the piece's first 16-row unit,
// [3] = its end unit (INT32_MAX: the sequence's end), [4] = piece index | n << 16, [5] = the record of piece 0,
// [6 + i] = table entry i, i < kOrderRecBlocks (piece 0 and whole sequences only: a later piece's workgroups read
// their first entries from the table).
hipError_t launch_order(const int32_t *context_lens, const int32_t *block_tables, int B, int M, int cap_rows,
                        int window, int32_t *order, const PieceRule &pieces, hipStream_t stream);
// Varlen records: order[rank][0] = sequence, [1] = cu_seqlens_q[s], [2] = cu_seqlens_q[s + 1], [3] = pos_offsets[s],
// [4 + i] = its table entry i (i < min(M, kVarlenRecBlocks)); ranked by min(pos + new rows, cap_rows), longest
// first, ties by index.
constexpr int kVarlenRecBlocks = kOrderRecord - 4;
hipError_t launch_order_varlen(const int32_t *cu_seqlens_q, const int32_t *pos_offsets, const int32_t *block_tables,
                               int B, int M, int cap_rows, int32_t *order, hipStream_t stream);
// The varlen step's new rows (token t of sequence s to row pos[s] + t - cu[s]): whole-panel rewrites, one workgroup
// per (sequence, kv head, 16-row unit the sequence's first max_q_len new rows can touch); a grid past kMaxGroups
// takes the per-row form.  With p.order set (order_cap = M * BS) the same call also writes the varlen dispatch-order
// records (see launch_order_varlen): in extra workgroups of the panel launch, else in an order launch of its own.
hipError_t launch_append_varlen(const AppendParams &p, const int32_t *cu_seqlens_q, const int32_t *pos_offsets,
                                int num_seqs, int max_q_len, hipStream_t stream);
hipError_t launch_qkv_cache(const QkvParams &p, int head_dim, hipStream_t stream);
hipError_t launch_check(const CheckParams &p, hipStream_t stream);

// Geometry support of the compiled kernels.
bool decode_geometry_supported(int head_dim, int block_size);
int max_waves_per_group(int head_dim);  // largest compiled waves per workgroup

}  // namespace pkv
