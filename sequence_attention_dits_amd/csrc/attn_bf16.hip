// attn_bf16.hip -- blockwise attention forward with LSE on the gfx950 matrix
// cores (bf16 inputs, fp32 accumulation and softmax).
//
// What it computes: for every query row the pair (out, lse) that each Ring
// step hands to the merge ("Add Unified Sequence Parallel attention",
// diffusers PR #12693, review thread; "Context parallelism" docs, "Ring
// Attention": each GPU computes attention against the K/V block it holds),
// with keys masked by global position for the zigzag / stripe / basic ring
// layouts (USP / yunchang summary, "How It Works").
//
// How (CDNA4, wave64):
//  * A workgroup owns 128 query rows of one (batch, head): 4 wavefronts of 32
//    rows.  Each wave keeps its Q rows in registers as matrix-core operands.
//  * K and V are streamed in tiles of 64 keys through LDS, double-buffered:
//    while the waves compute on one LDS stage, the next tile's global loads
//    are in flight in registers and land in the other stage afterwards, so
//    one barrier per tile suffices.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the accumulator layout then gives each lane
//    one query row (lane % 32) and 32 of the tile's 64 keys, so the row
//    maximum and sum need only one cross-lane step (lane ^ 32).
//  * The K rows fed to the score product are permuted inside each group of
//    32 so that a lane's score registers hold 8 consecutive keys per 16-key
//    chunk: those registers, rounded to bf16, are directly the P operand of
//    O^T += V^T P^T, and V is kept in LDS packed 8 keys per 16-byte unit so
//    each V operand is one 16-byte LDS read.  The output accumulator also
//    keeps one query row per lane, so the online-softmax rescale is a plain
//    per-lane multiply.
//  * LDS layouts are XOR-swizzled in 16-byte units so the operand reads and
//    the tile writes are free of bank conflicts.
//  * exp2 with scale * log2(e) folded into one multiply-add; the LSE is
//    converted back to the natural log at the end.  Rows with no allowed key
//    give o = 0, lse = -inf.
#include "attn_common.h"

namespace uaa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;

// float -> bfloat16 bits, round to nearest even (inputs here are finite or
// zero; NaN stays a quiet NaN).
__device__ __forceinline__ unsigned int bf16_rne(float f)
{
    const unsigned int u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ unsigned int pack_bf16(float lo, float hi)
{
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// XOR swizzle of a K row's 16-byte units.  The score product reads, in one
// instruction, rows {0..3, 8..11} (lanes 0-7), {4..7, 12..15} (lanes 8-15)
// and so on of a 32-row group at one unit column; this bit permutation of the
// row's low 4 bits sends those rows to distinct units.
template <int UPR>
__device__ __forceinline__ int k_swz(int row)
{
    return (((row & 3) | (((row >> 3) & 1) << 2) | (((row >> 2) & 1) << 3))) & (UPR - 1);
}

// Key (within a 32-key block) whose K row feeds operand row m of the score
// product: for score register v of lane-half h the key is
// 16 * (v / 8) + 8 * h + v % 8, i.e. 8 consecutive keys per 16-key chunk.
__device__ __forceinline__ int k_perm(int m)
{
    const int a = m >> 3, h = (m >> 2) & 1, b = m & 3;
    return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const AttnArgs a)
{
    constexpr int UPR = D / 8;          // 16-byte units per K row
    constexpr int NKC = D / 16;         // k-chunks of the score product
    constexpr int NDB = D / 32;         // 32-wide feature blocks of the output
    constexpr int NJB = kBN / 32;       // 32-key blocks of the score product
    constexpr int NPC = kBN / 16;       // 16-key chunks of the PV product
    constexpr int KU = kBN * UPR / 128; // K units loaded per K-loading thread
    constexpr int VB = (kBN / 8) * (D / 8); // 8x8 V blocks per tile

    __shared__ u32x4 Ks[2][kBN * UPR];
    __shared__ u32x4 Vs[2][(kBN / 8) * D];

    int64_t qt, hh, b;
    decode_tile(a, qt, hh, b);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hg = lane >> 5;
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const int64_t ld = H * D;           // elements between consecutive tokens
    const int64_t q0 = qt * kBM;
    const int64_t i = q0 + wave * 32 + l32;

    const unsigned short* Q = static_cast<const unsigned short*>(a.q);
    const unsigned short* Kg = static_cast<const unsigned short*>(a.k) + (b * Sk * H + hh) * D;
    const unsigned short* Vg = static_cast<const unsigned short*>(a.v) + (b * Sk * H + hh) * D;

    // Q operands: lane holds row i, features 16*kc + 8*hg .. +7.
    bf16x8 qop[NKC];
    {
        const bool ok = i < Sq;
        const u32x4* qrow = reinterpret_cast<const u32x4*>(Q + ((b * Sq + (ok ? i : 0)) * H + hh) * D);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            u32x4 w = ok ? qrow[2 * kc + hg] : u32x4{0u, 0u, 0u, 0u};
            qop[kc] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // Position ranges for masking: of this workgroup's rows and of this wave's.
    const bool masked = a.masked != 0;
    int64_t wg_qmax = 0, w_qmin = 0, w_qmax = 0, qpos = 0;
    bool wave_live = q0 + wave * 32 < Sq;
    if (masked) {
        int64_t dummy;
        const int64_t wg_hi = q0 + kBM < Sq ? q0 + kBM : Sq;
        pos_range(a.qmap, q0, wg_hi, dummy, wg_qmax);
        if (wave_live) {
            const int64_t w_lo = q0 + wave * 32;
            const int64_t w_hi = w_lo + 32 < Sq ? w_lo + 32 : Sq;
            pos_range(a.qmap, w_lo, w_hi, w_qmin, w_qmax);
        }
        qpos = pos_of(a.qmap, i);
    }

    const int n_tiles = (int)((Sk + kBN - 1) / kBN);
    // A tile is skipped when no row of the workgroup may see any of its keys.
    auto tile_live = [&](int t) -> bool {
        if (!masked) return true;
        const int64_t j0 = (int64_t)t * kBN;
        const int64_t j1 = j0 + kBN < Sk ? j0 + kBN : Sk;
        int64_t kmin, kmax;
        pos_range(a.kmap, j0, j1, kmin, kmax);
        return kmin <= wg_qmax;
    };
    auto next_live = [&](int t) -> int {
        while (t < n_tiles && !tile_live(t)) ++t;
        return t;
    };

    // ---- global -> register -> LDS staging of one K/V tile --------------
    // Threads 0-127 load K: unit u = tid + 128*k is row u / UPR, unit column
    // u % UPR.  Threads 128-255 load V as 8x8 blocks (8 keys x 8 features),
    // transpose them in registers and store 16-byte units of 8 keys.
    u32x4 stage[8];
    auto load_tile = [&](int t) {
        const int64_t j0 = (int64_t)t * kBN;
        if (tid < 128) {
#pragma unroll
            for (int k = 0; k < KU; ++k) {
                const int u = tid + 128 * k;
                const int row = u / UPR, c = u % UPR;
                const int64_t j = j0 + row;
                stage[k] = j < Sk ? *reinterpret_cast<const u32x4*>(Kg + j * ld + 8 * c)
                                  : u32x4{0u, 0u, 0u, 0u};
            }
        } else {
            const int t2 = tid - 128;
            const int jg = t2 & 7, dg = t2 >> 3;
            if (t2 < VB) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int64_t j = j0 + 8 * jg + r;
                    stage[r] = j < Sk ? *reinterpret_cast<const u32x4*>(Vg + j * ld + 8 * dg)
                                      : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };
    auto store_tile = [&](int st) {
        if (tid < 128) {
#pragma unroll
            for (int k = 0; k < KU; ++k) {
                const int u = tid + 128 * k;
                const int row = u / UPR, c = u % UPR;
                Ks[st][row * UPR + (c ^ k_swz<UPR>(row))] = stage[k];
            }
        } else {
            const int t2 = tid - 128;
            const int jg = t2 & 7, dg = t2 >> 3;
            if (t2 < VB) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    // column c of the 8x8 block: keys 8*jg .. +7 of feature 8*dg + c
                    const int e = c >> 1;
                    u32x4 col;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const unsigned int lo = stage[2 * p][e], hi = stage[2 * p + 1][e];
                        col[p] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                         : ((lo & 0xffffu) | (hi << 16));
                    }
                    const int d = 8 * dg + c;
                    Vs[st][jg * D + (d ^ jg)] = col;
                }
            }
        }
    };

    // ---- per-lane softmax state (row i) and output accumulator ----------
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m = -INFINITY;   // running max of scale*log2(e)*score
    float lsum = 0.f;      // this lane's half of the running sum
    const float c2 = a.scale_log2;

    int t = next_live(0);
    int st = 0;
    if (t < n_tiles) {
        load_tile(t);
        store_tile(0);
    }
    __syncthreads();

    while (t < n_tiles) {
        const int tn = next_live(t + 1);
        if (tn < n_tiles) load_tile(tn);

        const int64_t j0 = (int64_t)t * kBN;
        const int64_t j1 = j0 + kBN < Sk ? j0 + kBN : Sk;
        bool any = wave_live, all = true;
        if (masked && wave_live) {
            int64_t kmin, kmax;
            pos_range(a.kmap, j0, j1, kmin, kmax);
            any = kmin <= w_qmax;
            all = kmax <= w_qmin;
        }
        const bool per_elem = !all || j1 - j0 < kBN;

        if (any) {
            // S^T = K Q^T for the tile's two 32-key blocks
            f32x16 sacc[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v) sacc[jb][v] = 0.f;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const int c = 2 * kc + hg;
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {   // independent chains interleave
                    const int row = 32 * jb + k_perm(l32);
                    const bf16x8 kop = __builtin_bit_cast(bf16x8, Ks[st][row * UPR + (c ^ k_swz<UPR>(row))]);
                    sacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kc], sacc[jb], 0, 0, 0);
                }
            }

            // masking (ragged tail, causal by position)
            if (per_elem) {
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t j = j0 + 32 * jb + 16 * (v >> 3) + 8 * hg + (v & 7);
                        bool ok = j < Sk;
                        if (masked && ok) ok = pos_of(a.kmap, j) <= qpos;
                        if (!ok) sacc[jb][v] = -INFINITY;
                    }
            }

            // online softmax for row i
            float mx = -INFINITY;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[jb][v]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m, mx * c2);
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            float psum = 0.f;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sacc[jb][v], c2, -m_use));
                    sacc[jb][v] = p;
                    psum += p;
                }
            lsum = fmaf(lsum, alpha, psum);
            m = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;

            // O^T += V^T P^T, 16 keys per step
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
                const int jb = pc >> 1, v0 = 8 * (pc & 1);
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) pw[e] = pack_bf16(sacc[jb][v0 + 2 * e], sacc[jb][v0 + 2 * e + 1]);
                const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
                const int jg = 2 * pc + hg;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int d = 32 * db + l32;
                    const bf16x8 vop = __builtin_bit_cast(bf16x8, Vs[st][jg * D + (d ^ jg)]);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, oacc[db], 0, 0, 0);
                }
            }
        }

        if (tn < n_tiles) store_tile(st ^ 1);
        __syncthreads();
        st ^= 1;
        t = tn;
    }

    // ---- epilogue: normalise, write O and the natural-log LSE -----------
    const float lt = lsum + __shfl_xor(lsum, 32);
    if (i >= Sq) return;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t orow = ((b * Sq + i) * H + hh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * db + 8 * g + 4 * hg;   // 4 consecutive features
            const float x0 = oacc[db][4 * g] * inv, x1 = oacc[db][4 * g + 1] * inv;
            const float x2 = oacc[db][4 * g + 2] * inv, x3 = oacc[db][4 * g + 3] * inv;
            if (OUT_BF16) {
                u32x2 w{pack_bf16(x0, x1), pack_bf16(x2, x3)};
                *reinterpret_cast<u32x2*>(static_cast<unsigned short*>(a.o) + orow + d0) = w;
            } else {
                u32x4 w{__float_as_uint(x0), __float_as_uint(x1), __float_as_uint(x2), __float_as_uint(x3)};
                *reinterpret_cast<u32x4*>(static_cast<float*>(a.o) + orow + d0) = w;
            }
        }
    if (hg == 0) a.lse[(b * Sq + i) * H + hh] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
}

hipError_t launch_attn_bf16(int D, int o_dtype, const AttnArgs& a, hipStream_t s)
{
    const int64_t blocks = (int64_t)a.n_qtiles * a.H * a.B;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(256);
    const bool ob = o_dtype == UAA_BF16;
    if (D == 128) return ob ? launch_kernel(attn_bf16_kernel<128, true>, grid, block, 0, s, a)
                            : launch_kernel(attn_bf16_kernel<128, false>, grid, block, 0, s, a);
    if (D == 64) return ob ? launch_kernel(attn_bf16_kernel<64, true>, grid, block, 0, s, a)
                           : launch_kernel(attn_bf16_kernel<64, false>, grid, block, 0, s, a);
    return hipErrorInvalidValue;
}

}  // namespace uaa
