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
//  * K and V stream in tiles of 64 keys through LDS, double-buffered: while
//    the waves compute on one LDS stage, the next tile's buffer loads are in
//    flight in registers and land in the other stage afterwards, so one
//    barrier per tile suffices.  Buffer loads return zeros past the end of
//    the key range, which pads the ragged last tile.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the accumulator layout gives each lane one
//    query row (lane % 32) and 32 of the tile's 64 keys, so the row maximum
//    and sum need one cross-half exchange (v_permlane32_swap).
//  * A lane's score registers, rounded to bf16 (v_cvt_pk_bf16_f32), are
//    directly the P operand of O^T += V^T P^T; V is kept in LDS as 16-byte
//    units holding, for one feature, exactly the 8 keys that P operand slot
//    order expects (transposed in registers while staging), so each V operand
//    is one 16-byte LDS read.  O^T keeps one query row per lane too, so the
//    online-softmax rescale is a per-lane multiply.
//  * The running maximum is only raised when it grows by more than 2^8 in
//    exp2 units (a wave-uniform branch, rare after the first tile); between
//    raises the exponentials use the stale maximum, which is exact because
//    O and the sum share it, and stays far from fp32/bf16 overflow.
//  * LDS layouts: K rows padded by 16 bytes (operand reads of 8 or 16
//    consecutive rows hit distinct banks, addresses are base + immediate),
//    V units XOR-swizzled by key group (conflict-free staging writes).
//  * exp2 with scale * log2(e) folded into one multiply-add; the LSE is
//    converted back to the natural log at the end.  Rows with no allowed key
//    give o = 0, lse = -inf.
#include "attn_common.h"

namespace uaa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleThreshold = 8.0f;  // in log2 units of the softmax weights

// two floats -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned int pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(unsigned int, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Key offset (within a 16-key chunk) held in slot s of a lane-half's P
// operand: the S^T accumulator gives lane-half h the keys 4h + {0,1,2,3} and
// 4h + {8,9,10,11} of each 16-key chunk, in that order.
__device__ __forceinline__ int p_slot_key(int s) { return s < 4 ? s : s + 4; }

template <int D, bool MASKED, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const AttnArgs a)
{
    constexpr int UPR = D / 8;            // 16-byte units per K/V row
    constexpr int KST = UPR + 1;          // padded K row stride in units
    constexpr int NKC = D / 16;           // k-chunks of the score product
    constexpr int NDB = D / 32;           // 32-wide feature blocks of the output
    constexpr int NJB = kBN / 32;         // 32-key blocks of the score product
    constexpr int NPC = kBN / 16;         // 16-key chunks of the PV product
    constexpr int KU = kBN * UPR / 128;   // K units staged per K-staging thread
    constexpr int VB = (kBN / 8) * (D / 8);  // 8-key x 8-feature V blocks per tile

    __shared__ u32x4 Ks[2][kBN * KST];
    __shared__ u32x4 Vs[2][(kBN / 8) * D];

    int64_t qt, hh, b;
    decode_tile(a, qt, hh, b);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31, hg = lane >> 5;
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const uint32_t ld2 = (uint32_t)(H * D * 2);   // bytes between consecutive tokens
    const int64_t q0 = qt * kBM;
    const int64_t i = q0 + wave * 32 + l32;       // this lane's query row

    // Buffer resources: Q of this (batch, head), K and V of this (batch, head).
    // Reads past num_records return zero; every offset goes in the VGPR
    // operand, which is the part the range check covers.
    const unsigned char* qbase = static_cast<const unsigned char*>(a.q) + ((b * Sq) * H + hh) * D * 2;
    const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + ((b * Sk) * H + hh) * D * 2;
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + ((b * Sk) * H + hh) * D * 2;
    const uint32_t q_bytes = Sq > 0 ? (uint32_t)((Sq - 1) * ld2 + D * 2) : 0u;
    const uint32_t k_bytes = Sk > 0 ? (uint32_t)((Sk - 1) * ld2 + D * 2) : 0u;
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc((void*)qbase, (short)0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, k_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, k_bytes, 0x00020000);

    // Q operands: lane holds row i, features 16*kc + 8*hg .. +7 (zero past Sq).
    bf16x8 qop[NKC];
    {
        const uint32_t off = (uint32_t)(i < Sq ? i : Sq) * ld2 + hg * 16;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            qop[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, off + kc * 32, 0, 0));
    }

    // Masking: position ranges of the workgroup's rows and of this wave's.
    int64_t wg_qmax = 0, w_qmin = 0, w_qmax = 0, qpos = 0;
    const bool wave_live = q0 + wave * 32 < Sq;
    if (MASKED) {
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
    auto tile_live = [&](int t) -> bool {  // may any row of the workgroup see a key of tile t?
        if (!MASKED) return true;
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

    // ---- staging of one K/V tile: buffer loads -> registers -> LDS -------
    // Waves 0-1 stage K: unit u = tid + 128*k is row u / UPR, unit u % UPR.
    // Waves 2-3 stage V as 8-key x 8-feature blocks: block g holds the keys a
    // P operand slot set expects (16*(g/2) + 4*(g%2) + {0,1,2,3,8,9,10,11}),
    // transposed in registers into 8 units of (8 keys of one feature).
    const bool k_stager = wave < 2;
    const int t2 = tid & 127;
    const int vg = t2 & 7, vdg = t2 >> 3;
    uint32_t stage_goff;   // per-thread byte offset inside a tile
    if (k_stager) {
        stage_goff = (uint32_t)(t2 / UPR) * ld2 + (t2 % UPR) * 16;
    } else {
        stage_goff = (uint32_t)(16 * (vg >> 1) + 4 * (vg & 1)) * ld2 + vdg * 16;
    }
    u32x4 stage[8];
    auto load_tile = [&](int t) {
        const uint32_t tbase = (uint32_t)t * kBN * ld2;
        if (k_stager) {
#pragma unroll
            for (int k = 0; k < KU; ++k)
                stage[k] = __builtin_amdgcn_raw_buffer_load_b128(kr, stage_goff + tbase + (uint32_t)k * (128 / UPR) * ld2, 0, 0);
        } else if (t2 < VB) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                stage[r] = __builtin_amdgcn_raw_buffer_load_b128(vr, stage_goff + tbase + (uint32_t)p_slot_key(r) * ld2, 0, 0);
        }
    };
    auto store_tile = [&](int st) {
        if (k_stager) {
#pragma unroll
            for (int k = 0; k < KU; ++k) {
                const int u = t2 + 128 * k;
                Ks[st][(u / UPR) * KST + (u % UPR)] = stage[k];
            }
        } else if (t2 < VB) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int e = c >> 1;
                const unsigned int sel = (c & 1) ? 0x07060302u : 0x05040100u;
                u32x4 col;
#pragma unroll
                for (int p = 0; p < 4; ++p) col[p] = __builtin_amdgcn_perm(stage[2 * p + 1][e], stage[2 * p][e], sel);
                Vs[st][vg * D + ((8 * vdg + c) ^ vg)] = col;
            }
        }
    };

    // ---- per-lane state ---------------------------------------------------
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m = -INFINITY;   // reference maximum (exp2 units) of row i
    float lsum = 0.f;      // this lane-half's share of the row sum
    const float c2 = a.scale_log2;

    // LDS operand addresses (in 16-byte units): K row l32 of block jb at
    // unit column 2*kc + hg; V unit group g = 2*pc + hg, feature 32*db + l32.
    const int k_unit0 = l32 * KST + hg;
    int v_unit0[NPC];
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
        const int g = 2 * pc + hg;
        v_unit0[pc] = g * D + (l32 ^ g);
    }

    int t = next_live(0);
    if (t < n_tiles) {
        load_tile(t);
        store_tile(0);
    }
    __syncthreads();

    int st = 0;
    while (t < n_tiles) {
        const int tn = next_live(t + 1);
        if (tn < n_tiles) load_tile(tn);

        const int64_t j0 = (int64_t)t * kBN;
        bool any = wave_live, per_elem = j0 + kBN > Sk;
        if (MASKED && wave_live) {
            const int64_t j1 = j0 + kBN < Sk ? j0 + kBN : Sk;
            int64_t kmin, kmax;
            pos_range(a.kmap, j0, j1, kmin, kmax);
            any = kmin <= w_qmax;
            per_elem = per_elem || kmax > w_qmin;
        }

        if (any) {
            const u32x4* K = Ks[st];
            const u32x4* V = Vs[st];
            f32x16 sacc[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v) sacc[jb][v] = 0.f;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    const bf16x8 kop = __builtin_bit_cast(bf16x8, K[k_unit0 + jb * 32 * KST + 2 * kc]);
                    sacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kc], sacc[jb], 0, 0, 0);
                }
            }

            if (per_elem) {
                // register v of block jb holds key 32*jb + 8*(v/4) + 4*hg + v%4
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t j = j0 + 32 * jb + 8 * (v >> 2) + 4 * hg + (v & 3);
                        bool ok = j < Sk;
                        if (MASKED && ok) ok = pos_of(a.kmap, j) <= qpos;
                        if (!ok) sacc[jb][v] = -INFINITY;
                    }
            }

            // online softmax of row i
            float mx = -INFINITY;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) mx = fmaxf(mx, fmaxf(sacc[jb][v], sacc[jb][v + 1]));
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float m_new = fmaxf(m, mx * c2);
            const bool need = m_new > m + kRescaleThreshold;
            if (__any(need)) {
                // lanes that keep their maximum (possibly still -inf) scale by 1
                const float alpha = need ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;   // 0 from -inf
                const float m_upd = need ? m_new : m;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
                m = m_upd;
            }
            const float m_use = m == -INFINITY ? 0.f : m;
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[jb][v], c2, -m_use));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[jb][v + 1], c2, -m_use));
                    sacc[jb][v] = p0;
                    sacc[jb][v + 1] = p1;
                    ps0 += p0;
                    ps1 += p1;
                }
            lsum += ps0 + ps1;

            // O^T += V^T P^T, 16 keys per step
#pragma unroll
            for (int pc = 0; pc < NPC; ++pc) {
                const int jb = pc >> 1, v0 = 8 * (pc & 1);
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) pw[e] = pack_bf16(sacc[jb][v0 + 2 * e], sacc[jb][v0 + 2 * e + 1]);
                const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 vop = __builtin_bit_cast(bf16x8, V[v_unit0[pc] + 32 * db]);
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
    float lt;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
        lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
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

template <int D, bool OB>
static hipError_t launch_d(const AttnArgs& a, dim3 grid, hipStream_t s)
{
    const dim3 block(256);
    if (a.masked) return launch_kernel(attn_bf16_kernel<D, true, OB>, grid, block, 0, s, a);
    return launch_kernel(attn_bf16_kernel<D, false, OB>, grid, block, 0, s, a);
}

hipError_t launch_attn_bf16(int D, int o_dtype, const AttnArgs& a, hipStream_t s)
{
    const int64_t blocks = (int64_t)a.n_qtiles * a.H * a.B;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    const bool ob = o_dtype == UAA_BF16;
    if (D == 128) return ob ? launch_d<128, true>(a, grid, s) : launch_d<128, false>(a, grid, s);
    if (D == 64) return ob ? launch_d<64, true>(a, grid, s) : launch_d<64, false>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace uaa
