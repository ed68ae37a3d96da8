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
//     lets every lane load a 16-byte piece of a K row straight from HBM; V is
//     stored transposed per tile, so a lane's 4 consecutive rows of one dim are
//     8 contiguous bytes and each V load of the wave is one 512-byte run.
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

namespace pkv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kMaxWaves = 8;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Block id of the wave's i-th unit: lane j of `window` holds the id for unit
// index base + j, refreshed every 64 units.
template <int SPB>
__device__ __forceinline__ int table_window(const int32_t *bt, int u_first, int stride, int i_base, int u_end,
                                            int lane) {
    const int u = u_first + stride * (i_base + lane);
    return (u < u_end) ? bt[u / SPB] : -1;
}

template <int D, int BS>
struct Frag {
    static constexpr int KC = D / 32;  // 16x16x32 steps over the head dim
    static constexpr int VC = D / 16;  // 16-dim output tiles
    f16x8 k[KC];
    f16x4 v[VC];
};

// Loads unit u (16 rows) of physical block `blk` for kv head hk.
template <int D, int BS>
__device__ __forceinline__ void load_unit(Frag<D, BS> &f, const DecodeParams &p, int blk, int hk, int u, int r,
                                          int g4) {
    constexpr int SPB = BS / 16;
    const int sub = u % SPB;
    const int64_t tile = ((int64_t)blk * p.Hkv + hk) * (int64_t)(BS * D);
    const _Float16 *kb = p.k_pool + tile + (int64_t)(sub * 16 + r) * D + 8 * g4;
#pragma unroll
    for (int c = 0; c < Frag<D, BS>::KC; ++c)
        f.k[c] = *reinterpret_cast<const f16x8 *>(kb + 32 * c);
    const _Float16 *vb = p.v_pool + tile + (int64_t)r * BS + sub * 16 + 4 * g4;
#pragma unroll
    for (int c = 0; c < Frag<D, BS>::VC; ++c)
        f.v[c] = *reinterpret_cast<const f16x4 *>(vb + 16 * c * BS);
}

// One 16-row unit: scores, online-softmax update, P.V accumulation.
template <int D, int BS>
__device__ __forceinline__ void compute_unit(Frag<D, BS> &f, const f16x8 (&qf)[D / 32], f32x4 (&o)[D / 16],
                                             float &m_run, float &l_run, int u, int L, int g4, float scale_log2) {
    constexpr int KC = Frag<D, BS>::KC;
    constexpr int VC = Frag<D, BS>::VC;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.k[c], qf[c], sc, 0, 0, 0);
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        y[e] = sc[e] * scale_log2;
    const int t0 = u * 16 + 4 * g4;  // row of y[0] in the sequence
    if (u * 16 + 16 > L) {           // the unit holding row L-1 (wave-uniform branch)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool live = (t0 + e) < L;
            y[e] = live ? y[e] : -INFINITY;
#pragma unroll
            for (int c = 0; c < VC; ++c)
                f.v[c][e] = live ? f.v[c][e] : (_Float16)0.0f;  // rows past L may hold anything
        }
    }
    float bm = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
    bm = fmaxf(bm, xor_lane(bm, 16));
    bm = fmaxf(bm, xor_lane(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = exp2_fast(m_run - m_new);
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        pe[e] = exp2_fast(y[e] - m_new);
    l_run = l_run * alpha + ((pe[0] + pe[1]) + (pe[2] + pe[3]));
    m_run = m_new;
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

template <int D, int BS, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeParams p) {
    constexpr int KC = D / 32;
    constexpr int VC = D / 16;
    constexpr int SPB = BS / 16;
    constexpr int DP = D + 4;  // padded LDS row of one head's output
    extern __shared__ float smem[];

    const int tile = blockIdx.x;
    const int s = tile / p.Hkv;
    const int hk = tile - s * p.Hkv;
    const int split = SPLIT ? (int)blockIdx.y : 0;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int g4 = lane >> 4;

    int L = p.context_lens[s];
    L = L < 0 ? 0 : (L > p.M * BS ? p.M * BS : L);
    const int nb = (L + BS - 1) / BS;
    int b0 = 0, b1 = nb;
    if (SPLIT) {
        const int chunk = p.chunk_blocks > 0 ? p.chunk_blocks : (nb + p.num_splits - 1) / p.num_splits;
        b0 = split * chunk;
        b1 = min(nb, b0 + chunk);
        if (b0 >= b1)
            return;  // empty split: the combine never reads it
    }
    const int u_begin = b0 * SPB;
    const int u_end = min(b1 * SPB, (L + 15) >> 4);
    const int32_t *bt = p.block_tables + (int64_t)s * p.M;

    // Q^T as the B operand: lane (g4, r) holds head r, dims 32c + 8*g4 .. +8.
    f16x8 qf[KC];
    {
        const bool head_ok = r < p.G;
        const _Float16 *qrow = p.q + ((int64_t)s * p.Hq + hk * p.G + (head_ok ? r : 0)) * D + 8 * g4;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            f16x8 x = *reinterpret_cast<const f16x8 *>(qrow + 32 * c);
            qf[c] = head_ok ? x : (f16x8)(_Float16)0.0f;
        }
    }

    f32x4 o[VC];
#pragma unroll
    for (int c = 0; c < VC; ++c)
        o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = kNegBig;
    float l_run = 0.f;

    int u = u_begin + wave;
    if (u < u_end) {
        int window = table_window<SPB>(bt, u_begin + wave, NW, 0, u_end, lane);
        int i = 0;
        Frag<D, BS> fa, fb;
        int blk_a = __builtin_amdgcn_readlane(window, 0);
        bool ok_a = (unsigned)blk_a < (unsigned)p.N;
        if (ok_a)
            load_unit<D, BS>(fa, p, blk_a, hk, u, r, g4);
        for (;;) {
            // prefetch the next unit into fb, then compute fa
            int un = u + NW;
            bool has_b = un < u_end;
            int blk_b = -1;
            if (has_b) {
                ++i;
                if ((i & 63) == 0)
                    window = table_window<SPB>(bt, u_begin + wave, NW, i, u_end, lane);
                blk_b = __builtin_amdgcn_readlane(window, i & 63);
                if ((unsigned)blk_b < (unsigned)p.N)
                    load_unit<D, BS>(fb, p, blk_b, hk, un, r, g4);
            }
            if (ok_a)
                compute_unit<D, BS>(fa, qf, o, m_run, l_run, u, L, g4, p.scale_log2);
            if (!has_b)
                break;
            u = un;
            bool ok_b = (unsigned)blk_b < (unsigned)p.N;
            // prefetch the next unit into fa, then compute fb
            un = u + NW;
            bool has_a = un < u_end;
            if (has_a) {
                ++i;
                if ((i & 63) == 0)
                    window = table_window<SPB>(bt, u_begin + wave, NW, i, u_end, lane);
                blk_a = __builtin_amdgcn_readlane(window, i & 63);
                if ((unsigned)blk_a < (unsigned)p.N)
                    load_unit<D, BS>(fa, p, blk_a, hk, un, r, g4);
            }
            if (ok_b)
                compute_unit<D, BS>(fb, qf, o, m_run, l_run, u, L, g4, p.scale_log2);
            if (!has_a)
                break;
            u = un;
            ok_a = (unsigned)blk_a < (unsigned)p.N;
        }
    }

    // l over the four lane groups that hold the same head
    l_run += xor_lane(l_run, 16);
    l_run += xor_lane(l_run, 32);

    float *sm_m = smem;
    float *sm_l = smem + NW * 16;
    float *sm_o = smem + 2 * NW * 16;
    if (g4 == 0) {
        sm_m[wave * 16 + r] = m_run;
        sm_l[wave * 16 + r] = l_run;
    }
    if (r < p.G) {
        float *dst = sm_o + (wave * p.G + r) * DP + 4 * g4;
#pragma unroll
        for (int c = 0; c < VC; ++c) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[16 * c + e] = o[c][e];
        }
    }
    __syncthreads();

    const int total = p.G * D;
    for (int idx = threadIdx.x; idx < total; idx += NW * 64) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = kNegBig;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            M = fmaxf(M, sm_m[w * 16 + h]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float a = exp2_fast(sm_m[w * 16 + h] - M);
            den += a * sm_l[w * 16 + h];
            num += a * sm_o[(w * p.G + h) * DP + d];
        }
        const int64_t row = (int64_t)s * p.Hq + hk * p.G + h;
        if (!SPLIT) {
            p.out[row * D + d] = (_Float16)(den > 0.f ? num / den : 0.f);
        } else {
            const int64_t base = row * p.num_splits + split;
            p.part_o[base * D + d] = num;
            if (d == 0) {
                p.part_m[base] = M * kLn2;
                p.part_l[base] = den;
            }
        }
    }
}

// Split-K phase 2: one wavefront per (sequence, query head), lanes over dims.
// out = sum_j e^(m_j - M) O_j / sum_j e^(m_j - M) l_j over the non-empty splits.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    constexpr int PER = (D + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // s * Hq + hq
    if (row >= p.B * p.Hq)
        return;
    const int s = row / p.Hq;
    int L = p.context_lens[s];
    L = L < 0 ? 0 : (L > p.M * p.BS ? p.M * p.BS : L);
    const int nb = (L + p.BS - 1) / p.BS;
    int nvalid = 0;
    if (nb > 0) {
        const int chunk = p.chunk_blocks > 0 ? p.chunk_blocks : (nb + p.num_splits - 1) / p.num_splits;
        nvalid = min(p.num_splits, (nb + chunk - 1) / chunk);
    }
    const int64_t base = (int64_t)row * p.num_splits;
    float M = kNegBig;
    for (int j = lane; j < nvalid; j += 64)
        M = fmaxf(M, p.part_m[base + j]);
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1)
        M = fmaxf(M, xor_lane(M, mask));
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k)
        acc[k] = 0.f;
    float den = 0.f;
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
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int d = lane + 64 * k;
        if (d < D)
            p.out[(int64_t)row * D + d] = (_Float16)(den > 0.f ? acc[k] / den : 0.f);
    }
}

// Paged KV append [kapsl-backends 0.1.1, src/gguf_native.rs: launch_kv_write,
// launch_batch_kv_write]: one thread per (token, kv head, 8-dim piece).  The K
// piece is one 16-byte store into its row; the V piece is 8 two-byte stores,
// one per transposed row of the tile.
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const int pieces = p.D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.T * p.Hkv * pieces;
    if (gid >= total)
        return;
    const int c = (int)(gid % pieces);
    const int64_t th = gid / pieces;  // token * Hkv + head
    const int h = (int)(th % p.Hkv);
    const int i = (int)(th / p.Hkv);
    const int64_t slot = p.slot_mapping[i];
    if (slot < 0 || slot >= (int64_t)p.N * p.BS)
        return;
    const int64_t blk = slot / p.BS;
    const int off = (int)(slot - blk * p.BS);
    const int64_t src = th * p.D + 8 * c;
    const uint4 kv = *reinterpret_cast<const uint4 *>(p.k + src);
    const uint4 vv = *reinterpret_cast<const uint4 *>(p.v + src);
    const int64_t tile = (blk * p.Hkv + h) * (int64_t)p.BS * p.D;
    *reinterpret_cast<uint4 *>(p.k_pool + tile + (int64_t)off * p.D + 8 * c) = kv;
    const uint16_t *vh = reinterpret_cast<const uint16_t *>(&vv);
    uint16_t *vdst = reinterpret_cast<uint16_t *>(p.v_pool + tile + (int64_t)(8 * c) * p.BS + off);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        vdst[(int64_t)e * p.BS] = vh[e];
}

// ---------------------------------------------------------------------------
// launchers

size_t decode_lds_bytes(int head_dim, int G, int waves) {
    return sizeof(float) * ((size_t)2 * waves * 16 + (size_t)waves * G * (head_dim + 4));
}

bool decode_geometry_supported(int head_dim, int block_size) {
    return (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
           (block_size == 16 || block_size == 32 || block_size == 64);
}

int max_waves_per_group() { return kMaxWaves; }

template <int D, int BS, int NW>
static hipError_t launch_decode_t(const DecodeParams &p, int num_seqs, bool split, hipStream_t stream) {
    dim3 grid((unsigned)(num_seqs * p.Hkv), split ? (unsigned)p.num_splits : 1u, 1u);
    dim3 block(NW * 64);
    const size_t lds = decode_lds_bytes(D, p.G, NW);
    if (split)
        hipLaunchKernelGGL((decode_kernel<D, BS, NW, true>), grid, block, lds, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<D, BS, NW, false>), grid, block, lds, stream, p);
    return hipGetLastError();
}

template <int D, int BS>
static hipError_t launch_decode_w(const DecodeParams &p, int num_seqs, int waves, bool split, hipStream_t stream) {
    switch (waves) {
    case 1: return launch_decode_t<D, BS, 1>(p, num_seqs, split, stream);
    case 2: return launch_decode_t<D, BS, 2>(p, num_seqs, split, stream);
    case 4: return launch_decode_t<D, BS, 4>(p, num_seqs, split, stream);
    case 8: return launch_decode_t<D, BS, 8>(p, num_seqs, split, stream);
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

hipError_t launch_append(const AppendParams &p, hipStream_t stream) {
    const int64_t total = (int64_t)p.T * p.Hkv * (p.D / 8);
    dim3 grid((unsigned)((total + 255) / 256));
    dim3 block(256);
    hipLaunchKernelGGL(append_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
