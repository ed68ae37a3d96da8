// pkv_unit.h -- the per-unit building blocks of the gfx950 decode-attention kernels (pkv_kernels.hip): lane
// reductions, scalar loads of block ids, the panel-layout K/V fragment of one 16-row unit
// and its buffer loads, and the matrix-core step that turns one unit into an online-softmax update.
//
// Decode attention over one unit [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: paged_batched_decode_single_pass;
// kapsl-backends 0.1.1, src/gguf_native.rs: launch_paged_attention]: scores s = scale * q . k for the unit's rows,
// running max m, running sum l = sum 2^(s' - m) and running output o = sum 2^(s' - m) v, with s' the scores in
// log2 units, so that out = o / l over all units.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace pkv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kMaxWaves = 8;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Relaxed agent-scope vector stores and loads: they reach the memory side, coherent across the XCDs' L2 caches,
// without a cache-wide write-back or invalidate.
__device__ __forceinline__ void store_agent(float *p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Reductions over the four 16-lane rows that hold the same MFMA column (lanes r, r+16, r+32, r+48), on the VALU
// (v_permlane16_swap / v_permlane32_swap): no LDS traffic and no wait on the lgkm counter.  Every lane gets the
// same value, summed in the same order.
__device__ __forceinline__ float rows_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Block tables and lengths are read with wave-uniform indices through the constant address space, so they become
// scalar (SMEM) loads: their waits count on the lgkm counter and never hold back the K/V vector loads in flight.
typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr;

__device__ __forceinline__ int uniform_load(const int32_t *p, int64_t i) {
    return ((const_i32_ptr)p)[i];
}

// p[i] and p[i + 1] in one scalar load (i even, p 8-byte aligned).
typedef const __attribute__((address_space(4))) int64_t *const_i64_ptr;
__device__ __forceinline__ void uniform_load_pair(const int32_t *p, int64_t i, int &a, int &b) {
    const int64_t v = ((const_i64_ptr)p)[i / 2];
    a = (int)(uint32_t)v;
    b = (int)(uint32_t)(v >> 32);
}

// Floats of the decode kernel's cross-wave merge area: per wave, the running max and sum of 16 columns, then the
// G heads' D-wide partial outputs (rows padded to D + 4).
__host__ __device__ constexpr int merge_floats(int D, int G, int NW) { return 2 * NW * 16 + NW * G * (D + 4); }

template <int D, int BS>
struct Frag {
    static constexpr int KC = D / 32;  // 16x16x32 steps over the head dim
    static constexpr int VC = D / 16;  // 16-dim output tiles
    f16x8 k[KC];
    f16x4 v[VC];
};

// Loads one 16-row unit with buffer loads.  Every block is stored as panels of 16 rows; a unit is one panel:
//   K panel [D/32][16][32] (each row's dims in 32-wide pieces, piece-major): the A-operand fragment of lane
//     (g4, r) -- row r, dims 32c + 8*g4 .. +8 -- sits at byte 1024*c + 64*r + 16*g4: each wave load is one
//     contiguous 1 KB run of whole cache lines (a row-major tile would touch sixteen half lines per load, which
//     caps one CU at about a third of the rate it reaches on whole lines), and a new row is D/32 runs of 64 bytes
//     (an [D/8][16][8] panel, which loads at the same rate, spreads it over D/8 lines in 16-byte pieces);
//   V panel [4][D][4] (four quads of 4 rows; in a quad each dim's 4 rows are adjacent): lane (g4, r) reads dims
//     16c + r, rows 4*g4 .. +3 -- quad g4 -- at byte 8*(g4*D + r) + 128*c: each wave load is four whole 128-byte
//     lines, one per quad.  A new row then touches D/4 of the panel's 32-byte sectors (4 dims in each), where a
//     dim-major [D][16] panel, equally good to load, would put each of its D values in a sector of its own;
//   k_lane_offset() and v_lane_offset() below give the lane's byte offsets.
// kb / vb are wave-uniform pointers to the panel; each becomes a buffer resource built on the scalar unit, and the
// lane's loop-invariant byte offsets (k_lane, v_lane) are the only VGPR operands, so no per-unit address arithmetic
// lands in vector registers that loads in flight still own.  The resource's record count is the panel's size: an
// offset past it reads 0.
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, no swizzle (gfx9 family)
constexpr int kVGroupBytes = 128;       // V bytes of 16 dims of one quad: the step between a lane's V loads
__host__ __device__ constexpr uint32_t k_lane_offset(int r, int g4) { return (uint32_t)(64 * r + 16 * g4); }
__host__ __device__ constexpr uint32_t v_lane_offset(int D, int r, int g4) { return (uint32_t)(8 * (g4 * D + r)); }
// Cache-policy bits of the streamed K/V loads: nt (non-temporal).  K and V are read once per step, and the hint
// keeps them from displacing lines that are reused (measured on MI355X: 17% faster on the Llama-3-8B-shaped batch,
// 11% on the long-context split; the coherence-scope bits change nothing once it is set).
constexpr int kKvLoadPolicy = 2;

//
// live == false (a pipeline slot past the wave's last unit, or a unit whose block id names no pool block) gives the
// resources a record count of 0: the same instructions issue, so the wait counts stay exact, but every load returns
// zeros without a memory access -- in particular the final prefetches of a wave never hold up its epilogue.
template <int D, int BS>
__device__ __forceinline__ void load_unit(Frag<D, BS> &f, const _Float16 *kb, const _Float16 *vb, uint32_t k_lane,
                                          uint32_t v_lane, bool live) {
    const int nbytes = live ? 32 * D : 0;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16 *>(kb), 0, nbytes,
                                                                        kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16 *>(vb), 0, nbytes,
                                                                        kRsrcWord3);
#pragma unroll
    for (int c = 0; c < Frag<D, BS>::KC; ++c)
        f.k[c] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, k_lane, 1024 * c,
                                                                                 kKvLoadPolicy));
#pragma unroll
    for (int c = 0; c < Frag<D, BS>::VC; ++c)
        f.v[c] = __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(vr, v_lane, kVGroupBytes * c,
                                                                                kKvLoadPolicy));
}

// Rows each score column may attend: lo .. col.  col: this lane's column's last row (per lane); first: the
// smallest last row over the tile's columns; all: the largest (V rows outside lo .. all are never used by any column
// and are zeroed).  A decode tile has one
// limit, L - 1, for every column; a varlen tile gives each (query row, head) column the position of its row.
struct RowLimits {
    int col;
    int first;
    int all;
    int lo;  // first row any column may attend (a sliding window's start; 0 otherwise)
};

// The fused varlen step's pool update for one loaded 16-row unit: rows prow .. prow_end-1 are new -- their K and V
// taken from the workgroup's LDS copy of the unit (sk: [16][D] row-major; sv: [D][16] dim-major, so a lane's four
// rows of one dim are one 8-byte read) -- and the new rows are written to the unit's panels (wb_k, wb_v): their K
// runs (64 bytes per row and 32-dim piece) and the V quads that hold them, whole 128-byte lines whose other rows
// carry the values just loaded.  Nothing else of the panels is rewritten.  A dead unit is patched (its rows are
// masked anyway) but not written.
template <int D, int BS>
__device__ __forceinline__ void patch_unit_rows(Frag<D, BS> &f, int prow, int prow_end, const _Float16 *sk,
                                                const _Float16 *sv, _Float16 *wb_k, _Float16 *wb_v, bool dead, int r,
                                                int g4, uint32_t k_lane, uint32_t v_lane) {
    constexpr int KC = Frag<D, BS>::KC;
    constexpr int VC = Frag<D, BS>::VC;
    if (r >= prow && r < prow_end) {  // K dims 32c + 8*g4 .. +8 of row r
#pragma unroll
        for (int c = 0; c < KC; ++c)
            f.k[c] = *reinterpret_cast<const f16x8 *>(sk + r * D + 32 * c + 8 * g4);
    }
    bool take[4];  // V dims 16c + r of rows 4*g4 + e
#pragma unroll
    for (int e = 0; e < 4; ++e)
        take[e] = 4 * g4 + e >= prow && 4 * g4 + e < prow_end;
#pragma unroll
    for (int c = 0; c < VC; ++c) {  // lanes without new rows read unset LDS and keep their own values
        const f16x4 nv = *reinterpret_cast<const f16x4 *>(sv + (16 * c + r) * 16 + 4 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f.v[c][e] = take[e] ? nv[e] : f.v[c][e];
    }
    if (!dead) {  // the new rows' K runs, and the V quads that hold them (whole lines)
        if (r >= prow && r < prow_end) {
#pragma unroll
            for (int c = 0; c < KC; ++c)
                *reinterpret_cast<f16x8 *>(reinterpret_cast<char *>(wb_k) + k_lane + 1024 * c) = f.k[c];
        }
        if (4 * g4 + 3 >= prow && 4 * g4 < prow_end) {
#pragma unroll
            for (int c = 0; c < VC; ++c)
                *reinterpret_cast<f16x4 *>(reinterpret_cast<char *>(wb_v) + v_lane + kVGroupBytes * c) = f.v[c];
        }
    }
}

// One 16-row unit: scores, online-softmax update, P.V accumulation.  A dead unit (its block id names no pool
// block) is computed with every row masked, so that the loads of every unit are consumed on every path.
//
// prow >= 0 (fused decode step only): row prow of this unit is the token appended by this same launch; its K and V
// come from the workgroup's LDS copy of the new row (pk, pv: D halves each, natural order) instead of the loaded
// fragment.  Row prow is then written to the unit's panels (wb_k, wb_v): its K runs and its V quad -- the quad's
// 128-byte lines whole, its other three rows as loaded -- so no partial sector is written and no row but prow
// changes value.  (Rewriting both panels whole moved 8 KB per unit for 512 bytes of new row: the windowed step
// took 14.8 us against 14.0 with the row alone.)
// A unit whose block id names no pool block (dead) is neither written nor used.
template <int D, int BS>
__device__ __forceinline__ void compute_unit(Frag<D, BS> &f, const f16x8 (&qf)[D / 32], f32x4 (&o)[D / 16],
                                             float &m_run, float &l_run, int u, const RowLimits &lim, bool dead,
                                             int r, int g4,
                                             float scale_log2, int prow, const _Float16 *pk, const _Float16 *pv,
                                             _Float16 *wb_k, _Float16 *wb_v, uint32_t k_lane, uint32_t v_lane) {
    constexpr int KC = Frag<D, BS>::KC;
    constexpr int VC = Frag<D, BS>::VC;
    if (prow >= 0) {  // wave-uniform
        if (r == prow) {  // K dims 32c + 8*g4 .. +8
#pragma unroll
            for (int c = 0; c < KC; ++c)
                f.k[c] = *reinterpret_cast<const f16x8 *>(pk + 32 * c + 8 * g4);
        }
        if (g4 == (prow >> 2)) {  // V dims 16c + r
            const int e = prow & 3;  // selects with constant element indices keep the fragment in registers
#pragma unroll
            for (int c = 0; c < VC; ++c) {
                const _Float16 x = pv[16 * c + r];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    f.v[c][j] = (j == e) ? x : f.v[c][j];
            }
        }
        if (!dead) {  // the pool update, before any row is masked: the row's K runs and its V quad (whole lines)
            if (r == prow) {
#pragma unroll
                for (int c = 0; c < KC; ++c)
                    *reinterpret_cast<f16x8 *>(reinterpret_cast<char *>(wb_k) + k_lane + 1024 * c) = f.k[c];
            }
            if (g4 == (prow >> 2)) {
#pragma unroll
                for (int c = 0; c < VC; ++c)
                    *reinterpret_cast<f16x4 *>(reinterpret_cast<char *>(wb_v) + v_lane + kVGroupBytes * c) = f.v[c];
            }
        }
    }
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.k[c], qf[c], sc, 0, 0, 0);
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        y[e] = sc[e] * scale_log2;
    const int t0 = u * 16 + 4 * g4;  // row of y[0] in the sequence
    if (dead || u * 16 + 15 > lim.first || u * 16 < lim.lo) {  // a unit crossing a limit, or dead (wave-uniform)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in_lo = (t0 + e) >= lim.lo;
            y[e] = (!dead && in_lo && (t0 + e) <= lim.col) ? y[e] : -INFINITY;
            const bool row_ok = !dead && in_lo && (t0 + e) <= lim.all;
#pragma unroll
            for (int c = 0; c < VC; ++c)
                f.v[c][e] = row_ok ? f.v[c][e] : (_Float16)0.0f;  // rows past every column's last may hold anything
        }
    }
    const float bm = rows_max(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = exp2_fast(m_run - m_new);
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        pe[e] = exp2_fast(y[e] - m_new);
    l_run = l_run * alpha + ((pe[0] + pe[1]) + (pe[2] + pe[3]));
    m_run = m_new;
    // The weights enter the f16 matrix-core product rounded once to fp16 (l keeps the f32 sum): a weight moves by up
    // to 2^-11 of itself, the output by at most 2^-11 * max|v| when every weight sits just off a rounding midpoint
    // and V's signs follow the rounding directions, and far less otherwise -- the size of the fp16 output's own
    // rounding.  Carrying the rounding residue as a second fp16 product removed it but cost 0.6% on the
    // Llama-3-8B-shaped step and 4.7% on the two-tile varlen step.
    f16x4 pf;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        pf[e] = (_Float16)pe[e];
#pragma unroll
    for (int c = 0; c < VC; ++c) {
        o[c] *= alpha;
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(f.v[c], pf, o[c], 0, 0, 0);
    }
}

// Units in flight per wave (NS - 1 while one is computed).  Two stages: measured on MI355X, deeper pipelines gain
// nothing once a workgroup keeps its CU's memory path busy, and cost registers.
template <int D, int NW>
constexpr int pipeline_stages() {
    return 2;
}

}  // namespace pkv
