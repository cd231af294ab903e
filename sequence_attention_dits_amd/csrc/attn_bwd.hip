// attn_bwd.hip -- attention backward on the gfx950 matrix cores: the
// gradients of one attention call (one Ring key block) from the rows' final
// LSE, bf16 inputs, fp32 accumulation.
//
// What it computes ("Add Unified Sequence Parallel attention", diffusers PR
// #12693, conversation: the Unified / Ring attention is trained through a
// backward of its forward): for the forward (O, LSE) of the attention
// kernels, with P_ij = exp(scale <q_i, k_j> - lse_i) for allowed keys and
//   delta_i = sum_d dO_id O_id - dlse_i          (usp_attn_bwd_delta)
//   dS_ij   = P_ij (dP_ij - delta_i),  dP = dO V^T
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
// lse and O are those over every key block of a Ring pass, so the per-block
// gradients summed over the blocks are the gradient of the merged result.
//
// How (CDNA4, wave64), two kernels with no atomics:
//  * dK/dV kernel: a workgroup owns 128 keys of one (batch, head) and keeps
//    their K and V rows in registers as matrix operands; 8 wavefronts, the
//    key group of 32 being wave % 4 and the half of each 64-query tile
//    wave / 4, so both waves of a SIMD work on the same keys and their dK,
//    dV accumulators are summed once through LDS at the end.  Query tiles of
//    Q, dO, lse and delta stream through three LDS stages by buffer loads
//    that write LDS directly, issued two tiles ahead.  Per tile:
//      S = Q K^T, dP = dO V^T           (16-byte row reads of Q, dO)
//      dV^T += dO^T P, dK^T += Q^T dS   (transposing LDS reads of dO, Q)
//  * dQ kernel: a workgroup owns 256 query rows (32 per wave) with Q and dO
//    in registers; K and V tiles of 64 keys stream through LDS the same way.
//      S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T.
//    S is recomputed here rather than exchanged: the two kernels share no
//    memory but their inputs, and each writes its gradients once.
//  * The transposed operands come from ds_read_b64_tr_b16 on the row-major
//    tiles: within each group of 16 lanes, lane 16g + 4a + c receives the
//    c-th 16-bit element at the addresses of lanes 16g + a + 4e, e = 0..3,
//    so two such reads give a lane 8 rows of one column; the row each source
//    lane addresses is picked to match the row order of the P / dS operand,
//    which comes straight from the score registers (see the forward).
//  * 16-byte units of each row are XOR-swizzled by a row function under which
//    both the row reads (16 consecutive rows, one unit) and the transposing
//    reads (4 rows x 4 units per 16 lanes) hit distinct banks.
//  * Masked keys are removed by global position exactly as in the forward:
//    the allowed set of a row (keys) or of a key (queries) is a union of two
//    index intervals, classified once per workgroup and wave.
#include "attn_common.h"

namespace uaa {

typedef __bf16 bwd_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bwd_bf16x2 __attribute__((ext_vector_type(2)));
typedef float bwd_f32x16 __attribute__((ext_vector_type(16)));
typedef float bwd_f32x4 __attribute__((ext_vector_type(4)));
typedef float bwd_f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int bwd_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int bwd_u32x2 __attribute__((ext_vector_type(2)));
typedef short bwd_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char bwd_lds_u8;
typedef __attribute__((address_space(3))) bwd_u32x4 bwd_lds_u32x4;
typedef __attribute__((address_space(3))) bwd_i16x4 bwd_lds_i16x4;
typedef __attribute__((address_space(3))) bwd_f32x4 bwd_lds_f32x4;

constexpr int kBwdWaves = 8;
constexpr int kBwdT = 64;           // rows of a streamed tile
constexpr int kBwdKeys = 128;       // keys per dK/dV workgroup
constexpr int kBwdRows = 256;       // query rows per dQ workgroup
constexpr float kBwdLog2e = 1.44269504088896340736f;

__device__ __forceinline__ unsigned int bwd_pack(float lo, float hi)
{
    return __builtin_bit_cast(unsigned int, __builtin_convertvector(bwd_f32x2{lo, hi}, bwd_bf16x2));
}
__device__ __forceinline__ float bwd_lo(unsigned int x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bwd_hi(unsigned int x) { return __uint_as_float(x & 0xffff0000u); }

// LDS barrier that leaves global loads and LDS copies in flight.
__device__ __forceinline__ void bwd_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Row swizzle of the 16-byte units of a tile row: physical unit = logical
// unit ^ bwd_swz<D>(row).  D = 128 (16 units): swap the two 2-bit halves of
// row % 16.  D = 64 (8 units, two rows per 256 bytes): rotate (row / 2) % 8.
template <int D>
__device__ __forceinline__ int bwd_swz(int r)
{
    if constexpr (D == 128) {
        return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
        const int x = (r >> 1) & 7;
        return ((x & 1) << 2) | (x >> 1);
    }
}

// Copy instruction i of this wave for a 64-row tile (row r at src + r * ld2,
// bytes from nrec on read as zero) into the swizzled LDS tile dst: the
// instruction writes the 1 KB at (kBwdWaves * i + wave) * 1024, lane s its
// 16-byte slot s.
template <int D>
__device__ __forceinline__ void bwd_copy(const unsigned char* src, uint32_t nrec, uint32_t ld2, bwd_lds_u8* dst,
                                         int wave, int lane, int i)
{
    constexpr int UPR = D / 8, RPD = 1024 / (2 * D);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nrec, 0x00020000);
    const int n = kBwdWaves * i + wave;
    const int row = n * RPD + lane / UPR;
    const uint32_t off = (uint32_t)row * ld2 + (uint32_t)((((lane % UPR) ^ bwd_swz<D>(row))) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + n * 1024, 16, off, 0, 0, 0);
}

// Transposed matrix operand from a row-major swizzled tile: this lane, as
// one of the 64 source lanes (g, e, a) = (lane / 16, lane / 4 % 4, lane % 4),
// addresses rows rb + 4 (g / 2) + e and rb + 8 + 4 (g / 2) + e at features
// 32 db + 16 (g % 2) + 4 a; the result lane (m = feature, half h) then holds
// rows rb + 4h + {0..3, 8..11} of feature 32 db + lane % 32.
// Addressing: logical unit 4 db + w (w < 4) of row r sits at physical unit
// (4 db + w) ^ swz(r) = (4 db) ^ (w ^ swz(r)), so read k of block db is at
// tb.base[k] + ((db << 6) ^ tb.x[k]) (rb a multiple of 16 adds rb * 2D).
struct BwdTr {
    int base[2];
    int x[2];
};

template <int D>
__device__ __forceinline__ BwdTr bwd_tr_setup(int lane)
{
    const int g = lane >> 4, e = (lane >> 2) & 3, a = lane & 3;
    const int w = 2 * (g & 1) + (a >> 1);
    BwdTr t;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = 4 * (g >> 1) + e + 8 * k;
        t.base[k] = r * (2 * D) + 8 * (a & 1);
        t.x[k] = (w ^ bwd_swz<D>(r)) << 4;
    }
    return t;
}

template <int D>
__device__ __forceinline__ bwd_bf16x8 bwd_tr(const bwd_lds_u8* tile, int rb_bytes, const BwdTr& t, int db)
{
    const bwd_i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (bwd_lds_i16x4*)(tile + rb_bytes + t.base[0] + ((db << 6) ^ t.x[0])));
    const bwd_i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (bwd_lds_i16x4*)(tile + rb_bytes + t.base[1] + ((db << 6) ^ t.x[1])));
    return __builtin_bit_cast(bwd_bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row reads: logical unit 2 kc + hg of row r sits at (kc << 5) ^ x with
// x = (hg ^ swz(r)) << 4 bytes into the row.
template <int D>
__device__ __forceinline__ bwd_bf16x8 bwd_row(const bwd_lds_u8* tile, int row_base, int x, int kc)
{
    return __builtin_bit_cast(bwd_bf16x8, *(const bwd_lds_u32x4*)(tile + row_base + ((kc << 5) ^ x)));
}

// Number of leading indices idx < n of the piece base + stride * idx whose
// position is below p (the piece's queries that cannot see a key at p).
__device__ __forceinline__ int64_t bwd_below(int64_t base, int64_t stride, int64_t p, int64_t n)
{
    if (n <= 0 || p <= base) return 0;
    const int64_t c = stride == 1 ? p - base : (p - base + stride - 1) / stride;
    return c < n ? c : n;
}

// ==========================================================================
// dK / dV
// ==========================================================================
template <int D, bool MASKED>
__global__ __launch_bounds__(64 * kBwdWaves, 2) void attn_bwd_dkdv_kernel(const BwdArgs a)
{
    constexpr int ROWB = 2 * D, NKC = D / 16, NDB = D / 32, TB = kBwdT * ROWB;
    constexpr int CPT = TB / 1024 / kBwdWaves;        // copy instructions per wave per tensor per tile
    constexpr int kOps = 2 * CPT;                     // ... for Q and dO (waves 0, 1 add lse / delta)
    constexpr int STAGES = 6 * TB + 6 * 256;          // Q[3], dO[3], lse[3], delta[3]
    constexpr int RED = 4 * 64 * NDB * 16 * 4;        // one accumulator set of the 4 key groups
    constexpr int SMEM = STAGES > 2 * RED ? STAGES : 2 * RED;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];

    const uint32_t unit = xcd_logical(blockIdx.x, gridDim.x);
    const int64_t kt = unit % (uint32_t)a.n_tiles;
    const int64_t rest = unit / (uint32_t)a.n_tiles;
    const int64_t hh = rest % a.H, b = rest / a.H;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hg = lane >> 5;
    const int kg = wave & 3, qh = wave >> 2;
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const uint32_t ld2 = (uint32_t)(H * D * 2);
    const int64_t k0 = kt * kBwdKeys;
    const int64_t kw0 = k0 + 32 * kg;           // first key of this wave
    const int64_t j = kw0 + l32;                 // this lane's key
    const bool wave_keys = kw0 < Sk;

    // K and V rows of this lane's key as the B operands of S = Q K^T and
    // dP = dO V^T: features 16 kc + 8 hg .. +7 (zero past Sk)
    bwd_bf16x8 kop[NKC], vop[NKC];
    {
        const int64_t hoff = ((b * Sk) * H + hh) * D * 2;
        const uint32_t nrec = (uint32_t)((Sk - 1) * ld2 + D * 2);
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const unsigned char*>(a.k) + hoff), (short)0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const unsigned char*>(a.v) + hoff), (short)0, nrec, 0x00020000);
        const uint32_t roff = j < Sk ? (uint32_t)j * ld2 : nrec;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const uint32_t off = roff + (uint32_t)((2 * kc + hg) * 16);
            kop[kc] = __builtin_bit_cast(bwd_bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
            vop[kc] = __builtin_bit_cast(bwd_bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
        }
    }

    // Masking.  Query i may see key j iff qpos(i) >= kpos(j); positions grow
    // within each piece of the query map, so the queries a key position p
    // allows are [s0, segq) u [s1, Sq) with s0, s1 the first indices of the
    // pieces at or above p.  Per lane (this key), per workgroup (its keys'
    // smallest position: the queries some key sees), per wave (smallest and
    // largest: some key / every key).
    const int32_t sq32 = (int32_t)Sq;
    int32_t segq = sq32;
    int32_t qs0 = 0, qs1 = sq32;                         // this key
    int32_t g0 = 0, g1 = sq32, wa0 = 0, wa1 = sq32, wf0 = 0, wf1 = sq32;
    if (MASKED) {
        segq = (int32_t)(a.qmap.seg_len < Sq ? a.qmap.seg_len : Sq);
        const int64_t n1 = Sq - segq;
        auto sets = [&](int64_t p, int32_t& s0, int32_t& s1) {
            s0 = (int32_t)bwd_below(a.qmap.base0, a.qmap.stride, p, segq);
            s1 = segq + (int32_t)bwd_below(a.qmap.base1, a.qmap.stride, p, n1);
        };
        if (j < Sk) {
            sets(pos_of(a.kmap, j), qs0, qs1);
        } else {
            qs0 = segq;
            qs1 = sq32;
        }
        int64_t pmin, pmax;
        pos_range(a.kmap, k0, k0 + kBwdKeys < Sk ? k0 + kBwdKeys : Sk, pmin, pmax);
        sets(pmin, g0, g1);
        if (wave_keys) {
            pos_range(a.kmap, kw0, kw0 + 32 < Sk ? kw0 + 32 : Sk, pmin, pmax);
            sets(pmin, wa0, wa1);
            sets(pmax, wf0, wf1);
        }
    }
    // does [i0, i1) (i1 <= Sq) meet [s0, segq) u [s1, Sq)?
    auto meets = [&](int32_t i0, int32_t i1, int32_t s0, int32_t s1) {
        return (i0 < segq && s0 < segq && s0 < i1) || s1 < i1;
    };
    // is it inside?
    auto inside = [&](int32_t i0, int32_t i1, int32_t s0, int32_t s1) {
        return (i0 >= s0 || i0 >= segq) && ((i0 > segq ? i0 : segq) >= s1 || i1 <= segq);
    };
    const int n_qt = (int)((Sq + kBwdT - 1) / kBwdT);
    // live query tiles of the workgroup: [b0, e0) u [b1, e1)
    const int b0 = g0 / kBwdT, e0 = g0 < segq ? (segq + kBwdT - 1) / kBwdT : 0;
    const int b1 = g1 / kBwdT, e1 = g1 < sq32 ? n_qt : 0;
    auto next_live = [&](int t) -> int {
        if (!MASKED) return t < n_qt ? t : n_qt;
        if (t < e0) return t > b0 ? t : b0;
        t = t > b1 ? t : b1;
        return t < e1 ? t : n_qt;
    };

    // ---- staging -----------------------------------------------------------
    const unsigned char* qbase = static_cast<const unsigned char*>(a.q) + ((b * Sq) * H + hh) * D * 2;
    const unsigned char* obase = static_cast<const unsigned char*>(a.dout) + ((b * Sq) * H + hh) * D * 2;
    auto issue = [&](int t, int st) {
        const int64_t r0 = (int64_t)t * kBwdT;
        const int64_t nv = Sq - r0 < kBwdT ? Sq - r0 : kBwdT;
        const uint32_t nrec = (uint32_t)((nv - 1) * ld2 + D * 2);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            bwd_copy<D>(qbase + r0 * ld2, nrec, ld2, (bwd_lds_u8*)smem + st * TB, wave, lane, i);
            bwd_copy<D>(obase + r0 * ld2, nrec, ld2, (bwd_lds_u8*)smem + (3 + st) * TB, wave, lane, i);
        }
        if (wave < 2) {
            const float* src = (wave == 0 ? a.lse : a.delta) + (b * Sq + r0) * H + hh;
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)src, (short)0, (uint32_t)((nv - 1) * H * 4 + 4), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (bwd_lds_u8*)smem + 6 * TB + (3 * wave + st) * 256, 4,
                                                     (uint32_t)(lane * H * 4), 0, 0, 0);
        }
    };

    // per-lane LDS addressing: row reads of Q / dO (row 32 qh + l32) and
    // the transposing reads
    const int rrow = (32 * qh + l32) * ROWB, rx = (hg ^ bwd_swz<D>(l32)) << 4;
    const BwdTr trs = bwd_tr_setup<D>(lane);

    bwd_f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            dk[db][v] = 0.f;
            dv[db][v] = 0.f;
        }
    const float c2 = a.scale_log2;

    int t = next_live(0);
    int t1 = t < n_qt ? next_live(t + 1) : n_qt;
    int st = 0;
    if (t < n_qt) {
        issue(t, 0);
        if (t1 < n_qt) issue(t1, 1);
    }
    if (t1 < n_qt)
        __builtin_amdgcn_s_waitcnt(0x0F70 | kOps);   // the operands and tile t landed
    else
        __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    while (t < n_qt) {
        const int t2 = t1 < n_qt ? next_live(t1 + 1) : n_qt;
        if (t2 < n_qt) issue(t2, st == 0 ? 2 : st - 1);

        const int32_t i0 = t * kBwdT + 32 * qh;
        const int32_t i1 = i0 + 32 < sq32 ? i0 + 32 : sq32;
        bool any = wave_keys && i0 < sq32, per_elem = false;
        if (MASKED && any) {
            any = meets(i0, i1, wa0, wa1);
            per_elem = !inside(i0, i1, wf0, wf1);
        }
        if (any) {
            const bwd_lds_u8* Ql = (const bwd_lds_u8*)smem + st * TB;
            const bwd_lds_u8* Ol = (const bwd_lds_u8*)smem + (3 + st) * TB;
            const bwd_lds_u8* Ll = (const bwd_lds_u8*)smem + 6 * TB + st * 256;
            const bwd_lds_u8* Dl = (const bwd_lds_u8*)smem + 6 * TB + (3 + st) * 256;
            // S = Q K^T: lane = key, register v = query
            // 32 qh + 8 (v / 4) + 4 hg + v % 4 of the tile
            bwd_f32x16 sc;
#pragma unroll
            for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_row<D>(Ql, rrow, rx, kc), kop[kc], sc, 0, 0, 0);
            // P in bf16, in the operand order of the transposing reads:
            // chunk c, slot s <-> query 16 c + 4 hg + {0..3, 8..11}[s]
            bwd_u32x4 pw[2];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int ql = 32 * qh + 8 * g4 + 4 * hg;   // first of 4 consecutive tile queries
                const bwd_f32x4 lv = *(const bwd_lds_f32x4*)(Ll + ql * 4);
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float sv = sc[4 * g4 + e];
                    if (MASKED && per_elem) {
                        const int32_t iq = t * kBwdT + ql + e;
                        const bool ok = iq < segq ? iq >= qs0 : iq >= qs1;
                        if (!ok) sv = -INFINITY;
                    }
                    // a row with no key at all (lse = -inf) has P = 0
                    const float l2 = lv[e] == -INFINITY ? INFINITY : lv[e] * kBwdLog2e;
                    p[e] = __builtin_amdgcn_exp2f(fmaf(sv, c2, -l2));
                }
                const int c = g4 >> 1, h2 = 2 * (g4 & 1);
                pw[c][h2] = bwd_pack(p[0], p[1]);
                pw[c][h2 + 1] = bwd_pack(p[2], p[3]);
            }
            // dV^T += dO^T P: lane = key, register v = feature
            // 32 db + 8 (v / 4) + 4 hg + v % 4
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bwd_bf16x8 pb = __builtin_bit_cast(bwd_bf16x8, pw[c]);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(Ol, (32 * qh + 16 * c) * ROWB, trs, db),
                                                                     pb, dv[db], 0, 0, 0);
            }
            // dP = dO V^T (same layout as S), dS = P (dP - delta) with the
            // bf16 P of the dV product
            bwd_f32x16 dp;
#pragma unroll
            for (int v = 0; v < 16; ++v) dp[v] = 0.f;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_row<D>(Ol, rrow, rx, kc), vop[kc], dp, 0, 0, 0);
            bwd_u32x4 sw[2];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int ql = 32 * qh + 8 * g4 + 4 * hg;
                const bwd_f32x4 dl = *(const bwd_lds_f32x4*)(Dl + ql * 4);
                const int c = g4 >> 1, h2 = 2 * (g4 & 1);
                const unsigned int p01 = pw[c][h2], p23 = pw[c][h2 + 1];
                sw[c][h2] = bwd_pack(bwd_lo(p01) * (dp[4 * g4] - dl[0]), bwd_hi(p01) * (dp[4 * g4 + 1] - dl[1]));
                sw[c][h2 + 1] = bwd_pack(bwd_lo(p23) * (dp[4 * g4 + 2] - dl[2]), bwd_hi(p23) * (dp[4 * g4 + 3] - dl[3]));
            }
            // dK^T += Q^T dS (scaled at the end)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const bwd_bf16x8 sb = __builtin_bit_cast(bwd_bf16x8, sw[c]);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(Ql, (32 * qh + 16 * c) * ROWB, trs, db),
                                                                     sb, dk[db], 0, 0, 0);
            }
        }

        // the copies of tile t1 must have landed; those of t2 may still run
        if (t2 < n_qt)
            __builtin_amdgcn_s_waitcnt(0x0F70 | kOps);
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        bwd_barrier();
        st = st == 2 ? 0 : st + 1;
        t = t1;
        t1 = t2;
    }

    // ---- epilogue: sum the two query halves, write dK (scaled) and dV -----
    // Waves of half 1 hand their dV to half 0 and half 0 its dK to half 1,
    // through LDS laid out [key group][quad][lane] (16 bytes per lane).
    __builtin_amdgcn_s_waitcnt(0x0F70);
    bwd_barrier();
    bwd_lds_u8* const R0 = (bwd_lds_u8*)smem;         // dV of half 1
    bwd_lds_u8* const R1 = (bwd_lds_u8*)smem + RED;   // dK of half 0
    auto slot = [&](int db, int g4) { return ((kg * NDB * 4 + db * 4 + g4) * 64 + lane) * 16; };
    {
        bwd_lds_u8* W = qh == 1 ? R0 : R1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bwd_f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = qh == 1 ? dv[db][4 * g4 + e] : dk[db][4 * g4 + e];
                *(bwd_lds_f32x4*)(W + slot(db, g4)) = w;
            }
    }
    bwd_barrier();
    if (j >= Sk) return;
    // half 0 writes dV, half 1 writes dK
    const bwd_lds_u8* Rd = qh == 0 ? R0 : R1;
    const float mul = qh == 0 ? 1.f : a.scale;
    void* out = qh == 0 ? a.dv : a.dk;
    const int64_t orow = ((b * Sk + j) * H + hh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const bwd_f32x4 o = *(const bwd_lds_f32x4*)(Rd + slot(db, g4));
            const int f = 32 * db + 8 * g4 + 4 * hg;
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = ((qh == 0 ? dv[db][4 * g4 + e] : dk[db][4 * g4 + e]) + o[e]) * mul;
            if (a.grad_bf16) {
                bwd_u32x2* p = reinterpret_cast<bwd_u32x2*>(static_cast<unsigned short*>(out) + orow + f);
                if (a.accumulate & 2) {
                    const bwd_u32x2 old = *p;
                    r[0] += bwd_lo(old[0]);
                    r[1] += bwd_hi(old[0]);
                    r[2] += bwd_lo(old[1]);
                    r[3] += bwd_hi(old[1]);
                }
                *p = bwd_u32x2{bwd_pack(r[0], r[1]), bwd_pack(r[2], r[3])};
            } else {
                bwd_f32x4* p = reinterpret_cast<bwd_f32x4*>(static_cast<float*>(out) + orow + f);
                bwd_f32x4 w{r[0], r[1], r[2], r[3]};
                if (a.accumulate & 2) w += *p;
                *p = w;
            }
        }
}

// ==========================================================================
// dQ
// ==========================================================================
template <int D, bool MASKED>
__global__ __launch_bounds__(64 * kBwdWaves, 2) void attn_bwd_dq_kernel(const BwdArgs a)
{
    constexpr int ROWB = 2 * D, NKC = D / 16, NDB = D / 32, TB = kBwdT * ROWB;
    constexpr int CPT = TB / 1024 / kBwdWaves;
    constexpr int kOps = 2 * CPT;                    // K and V copies per wave per tile
    __shared__ __attribute__((aligned(1024))) unsigned char smem[6 * TB];   // K[3], V[3]

    const uint32_t unit = xcd_logical(blockIdx.x, gridDim.x);
    int64_t qt = unit % (uint32_t)a.n_tiles;
    const int64_t rest = unit / (uint32_t)a.n_tiles;
    const int64_t hh = rest % a.H, b = rest / a.H;
    if (MASKED) qt = a.n_tiles - 1 - qt;   // later rows see more keys: longest first

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hg = lane >> 5;
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const uint32_t ld2 = (uint32_t)(H * D * 2);
    const int64_t q0 = qt * kBwdRows;
    const int64_t i = q0 + 32 * wave + l32;   // this lane's query row
    const bool wave_live = q0 + 32 * wave < Sq;

    // Q and dO rows of this lane as the B operands of S^T = K Q^T and
    // dP^T = V dO^T (zero past Sq); the row's lse (log2 units, +inf for a
    // row with no key: P = 0) and delta
    bwd_bf16x8 qop[NKC], dop[NKC];
    float l2 = INFINITY, dlt = 0.f;
    {
        const int64_t hoff = ((b * Sq) * H + hh) * D * 2;
        const uint32_t nrec = (uint32_t)((Sq - 1) * ld2 + D * 2);
        const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const unsigned char*>(a.q) + hoff), (short)0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const unsigned char*>(a.dout) + hoff), (short)0, nrec, 0x00020000);
        const uint32_t roff = i < Sq ? (uint32_t)i * ld2 : nrec;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const uint32_t off = roff + (uint32_t)((2 * kc + hg) * 16);
            qop[kc] = __builtin_bit_cast(bwd_bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0));
            dop[kc] = __builtin_bit_cast(bwd_bf16x8, __builtin_amdgcn_raw_buffer_load_b128(orr, off, 0, 0));
        }
        if (i < Sq) {
            const float lv = a.lse[(b * Sq + i) * H + hh];
            l2 = lv == -INFINITY ? INFINITY : lv * kBwdLog2e;
            dlt = a.delta[(b * Sq + i) * H + hh];
        }
    }

    // Masking as in the forward: key j allowed for this row iff j < lim0
    // (first piece of the key map, j < segk) or j < lim1; workgroup / wave
    // key sets as unions of two prefixes of the pieces.
    const int32_t sk32 = (int32_t)Sk;
    int32_t segk = sk32, lim0 = sk32, lim1 = sk32;
    int32_t ln0 = sk32, ln1 = 0, wa0 = sk32, wa1 = 0, wf0 = sk32, wf1 = 0;
    if (MASKED) {
        segk = (int32_t)(a.kmap.seg_len < Sk ? a.kmap.seg_len : Sk);
        const int64_t n1 = Sk - segk;
        const int64_t qp = pos_of(a.qmap, i);
        lim0 = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, qp, segk);
        lim1 = segk + (int32_t)allowed_prefix(a.kmap.base1, a.kmap.stride, qp, n1);
        int64_t pmin, pmax;
        pos_range(a.qmap, q0, q0 + kBwdRows < Sq ? q0 + kBwdRows : Sq, pmin, pmax);
        ln0 = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, pmax, segk);
        ln1 = (int32_t)allowed_prefix(a.kmap.base1, a.kmap.stride, pmax, n1);
        if (wave_live) {
            const int64_t w0 = q0 + 32 * wave;
            pos_range(a.qmap, w0, w0 + 32 < Sq ? w0 + 32 : Sq, pmin, pmax);
            wa0 = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, pmax, segk);
            wa1 = (int32_t)allowed_prefix(a.kmap.base1, a.kmap.stride, pmax, n1);
            wf0 = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, pmin, segk);
            wf1 = (int32_t)allowed_prefix(a.kmap.base1, a.kmap.stride, pmin, n1);
        }
    }
    auto meets = [&](int32_t j0, int32_t j1, int32_t p0, int32_t p1) {
        return j0 < p0 || (j1 > segk && (j0 > segk ? j0 : segk) < segk + p1);
    };
    auto inside = [&](int32_t j0, int32_t j1, int32_t p0, int32_t p1) {
        return (j0 >= segk || (j1 < segk ? j1 : segk) <= p0) && (j1 <= segk || j1 <= segk + p1);
    };
    const int n_kt = (int)((Sk + kBwdT - 1) / kBwdT);
    const int lt0 = (ln0 + kBwdT - 1) / kBwdT;
    const int lt1b = ln1 > 0 ? segk / kBwdT : n_kt, lt1e = ln1 > 0 ? (segk + ln1 + kBwdT - 1) / kBwdT : n_kt;
    auto next_live = [&](int t) -> int {
        if (!MASKED || t < lt0) return t < n_kt ? t : n_kt;
        if (t < lt1b) t = lt1b;
        return t < lt1e && t < n_kt ? t : n_kt;
    };

    const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + ((b * Sk) * H + hh) * D * 2;
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + ((b * Sk) * H + hh) * D * 2;
    auto issue = [&](int t, int st) {
        const int64_t r0 = (int64_t)t * kBwdT;
        const int64_t nv = Sk - r0 < kBwdT ? Sk - r0 : kBwdT;
        const uint32_t nrec = (uint32_t)((nv - 1) * ld2 + D * 2);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            bwd_copy<D>(kbase + r0 * ld2, nrec, ld2, (bwd_lds_u8*)smem + st * TB, wave, lane, c);
            bwd_copy<D>(vbase + r0 * ld2, nrec, ld2, (bwd_lds_u8*)smem + (3 + st) * TB, wave, lane, c);
        }
    };

    const int rrow = l32 * ROWB, rx = (hg ^ bwd_swz<D>(l32)) << 4;
    const BwdTr trs = bwd_tr_setup<D>(lane);

    bwd_f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
    const float c2 = a.scale_log2;

    int t = next_live(0);
    int t1 = t < n_kt ? next_live(t + 1) : n_kt;
    int st = 0;
    if (t < n_kt) {
        issue(t, 0);
        if (t1 < n_kt) issue(t1, 1);
    }
    if (t1 < n_kt)
        __builtin_amdgcn_s_waitcnt(0x0F70 | kOps);
    else
        __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    while (t < n_kt) {
        const int t2 = t1 < n_kt ? next_live(t1 + 1) : n_kt;
        if (t2 < n_kt) issue(t2, st == 0 ? 2 : st - 1);

        const int32_t j0 = t * kBwdT, j1 = j0 + kBwdT < sk32 ? j0 + kBwdT : sk32;
        bool any = wave_live, per_elem = j0 + kBwdT > sk32;
        if (MASKED && wave_live) {
            any = meets(j0, j1, wa0, wa1);
            per_elem = per_elem || !inside(j0, j1, wf0, wf1);
        }
        if (any) {
            const bwd_lds_u8* Kl = (const bwd_lds_u8*)smem + st * TB;
            const bwd_lds_u8* Vl = (const bwd_lds_u8*)smem + (3 + st) * TB;
            // S^T = K Q^T, dP^T = V dO^T: lane = query, register v of block
            // jb = key 32 jb + 8 (v / 4) + 4 hg + v % 4 of the tile
            bwd_f32x16 s[2], dp[2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    s[jb][v] = 0.f;
                    dp[jb][v] = 0.f;
                }
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const int rb = jb * 32 * ROWB + rrow;
                    s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_row<D>(Kl, rb, rx, kc), qop[kc], s[jb], 0, 0, 0);
                    dp[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_row<D>(Vl, rb, rx, kc), dop[kc], dp[jb], 0, 0, 0);
                }
            // dS^T in bf16, 16-key chunk c = slots 4 hg + {0..3, 8..11}
            bwd_u32x4 sw[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int jb = c >> 1, v0 = 8 * (c & 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float d[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const int v = v0 + 2 * e + x;
                        float sv = s[jb][v];
                        if (per_elem) {
                            const int32_t jj = j0 + 32 * jb + 8 * (v >> 2) + 4 * hg + (v & 3);
                            const bool ok = jj < segk ? jj < lim0 : jj < lim1;
                            if (!ok) sv = -INFINITY;
                        }
                        const float p = __builtin_amdgcn_exp2f(fmaf(sv, c2, -l2));
                        d[x] = p * (dp[jb][v] - dlt);
                    }
                    sw[c][e] = bwd_pack(d[0], d[1]);
                }
            }
            // dQ^T += K^T dS^T: lane = query, register v = feature
            // 32 db + 8 (v / 4) + 4 hg + v % 4
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bwd_bf16x8 sb = __builtin_bit_cast(bwd_bf16x8, sw[c]);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(Kl, 16 * c * ROWB, trs, db), sb,
                                                                      acc[db], 0, 0, 0);
            }
        }

        if (t2 < n_kt)
            __builtin_amdgcn_s_waitcnt(0x0F70 | kOps);
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        bwd_barrier();
        st = st == 2 ? 0 : st + 1;
        t = t1;
        t1 = t2;
    }

    if (i >= Sq) return;
    const int64_t orow = ((b * Sq + i) * H + hh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int f = 32 * db + 8 * g4 + 4 * hg;
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = acc[db][4 * g4 + e] * a.scale;
            if (a.grad_bf16) {
                bwd_u32x2* p = reinterpret_cast<bwd_u32x2*>(static_cast<unsigned short*>(a.dq) + orow + f);
                if (a.accumulate & 1) {
                    const bwd_u32x2 old = *p;
                    r[0] += bwd_lo(old[0]);
                    r[1] += bwd_hi(old[0]);
                    r[2] += bwd_lo(old[1]);
                    r[3] += bwd_hi(old[1]);
                }
                *p = bwd_u32x2{bwd_pack(r[0], r[1]), bwd_pack(r[2], r[3])};
            } else {
                bwd_f32x4* p = reinterpret_cast<bwd_f32x4*>(static_cast<float*>(a.dq) + orow + f);
                bwd_f32x4 w{r[0], r[1], r[2], r[3]};
                if (a.accumulate & 1) w += *p;
                *p = w;
            }
        }
}

// ==========================================================================
// delta = rowsum(dout * o) - dlse
// ==========================================================================
// LPR lanes per row, each with 16 bytes of o and dout; rows strided over the grid.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const DeltaArgs a)
{
    constexpr int VE = 16 / (int)sizeof(T);          // elements per lane
    constexpr int LPR = D / VE;                      // lanes per row
    constexpr int RPB = 256 / LPR;                   // rows per block pass
    const int tid = threadIdx.x;
    const int rl = tid / LPR, part = tid % LPR;
    for (int64_t row = (int64_t)blockIdx.x * RPB + rl; row < a.rows; row += (int64_t)gridDim.x * RPB) {
        const bwd_u32x4 ov = *reinterpret_cast<const bwd_u32x4*>(static_cast<const T*>(a.o) + row * D + part * VE);
        const bwd_u32x4 gv = *reinterpret_cast<const bwd_u32x4*>(static_cast<const T*>(a.dout) + row * D + part * VE);
        float sum = 0.f;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sum = fmaf(bwd_lo(ov[e]), bwd_lo(gv[e]), sum);
                sum = fmaf(bwd_hi(ov[e]), bwd_hi(gv[e]), sum);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) sum = fmaf(__uint_as_float(ov[e]), __uint_as_float(gv[e]), sum);
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, LPR);
        if (part == 0) a.delta[row] = a.dlse != nullptr ? sum - a.dlse[row] : sum;
    }
}

// ==========================================================================
// launchers
// ==========================================================================
template <int D, bool M>
static hipError_t launch_bwd_d(const BwdArgs& a0, hipStream_t s)
{
    if (a0.Sk > 0) {
        BwdArgs a = a0;
        a.n_tiles = (int32_t)((a.Sk + kBwdKeys - 1) / kBwdKeys);
        const hipError_t e = launch_kernel(attn_bwd_dkdv_kernel<D, M>, dim3((uint32_t)(a.B * a.H * a.n_tiles)),
                                           dim3(64 * kBwdWaves), 0, s, a);
        if (e != hipSuccess) return e;
    }
    if (a0.Sq == 0) return hipSuccess;
    BwdArgs a = a0;
    a.n_tiles = (int32_t)((a.Sq + kBwdRows - 1) / kBwdRows);
    return launch_kernel(attn_bwd_dq_kernel<D, M>, dim3((uint32_t)(a.B * a.H * a.n_tiles)), dim3(64 * kBwdWaves), 0,
                         s, a);
}

hipError_t launch_attn_bwd_bf16(int D, const BwdArgs& a, hipStream_t s)
{
    if (a.B * a.H == 0 || (a.Sq == 0 && a.Sk == 0)) return hipSuccess;
    // no query: dK = dV = 0 (nothing to add when accumulating into them)
    if (a.Sq == 0 && (a.accumulate & 2)) return hipSuccess;
    if (D == 128) return a.masked ? launch_bwd_d<128, true>(a, s) : launch_bwd_d<128, false>(a, s);
    return a.masked ? launch_bwd_d<64, true>(a, s) : launch_bwd_d<64, false>(a, s);
}

hipError_t launch_bwd_delta(int dtype, int D, const DeltaArgs& a, hipStream_t s)
{
    if (a.rows == 0) return hipSuccess;
    auto grid = [&](int rpb) {
        const int64_t n = (a.rows + rpb - 1) / rpb;
        return dim3((uint32_t)(n < 8192 ? n : 8192));
    };
    if (dtype == UAA_BF16) {
        if (D == 128) return launch_kernel(attn_bwd_delta_kernel<unsigned short, 128>, grid(256 / 16), dim3(256), 0, s, a);
        return launch_kernel(attn_bwd_delta_kernel<unsigned short, 64>, grid(256 / 8), dim3(256), 0, s, a);
    }
    if (D == 128) return launch_kernel(attn_bwd_delta_kernel<float, 128>, grid(256 / 32), dim3(256), 0, s, a);
    return launch_kernel(attn_bwd_delta_kernel<float, 64>, grid(256 / 16), dim3(256), 0, s, a);
}

}  // namespace uaa
