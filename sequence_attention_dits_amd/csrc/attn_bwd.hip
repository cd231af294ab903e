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
//  * dK/dV kernel: a workgroup owns 128 keys of one (batch, head); 8
//    wavefronts, the key group of 32 being wave % 4.  The two waves of a
//    SIMD split the work by role, not by query: wave / 4 = 0 keeps the
//    group's K rows as matrix operands and accumulates dK, wave / 4 = 1
//    keeps the V rows and accumulates dV, and they hand P and dS to each
//    other through LDS, so no accumulator is ever summed across waves.
//    Query tiles of Q, dO, lse and delta stream through LDS stages by buffer
//    loads that write LDS directly, issued two tiles ahead.  Per tile:
//      S = Q K^T, dP = dO V^T           (16-byte row reads of Q, dO)
//      dV^T += dO^T P, dK^T += Q^T dS   (transposing LDS reads of dO, Q)
//  * dQ kernel: a workgroup owns 256 query rows (32 per wave) with Q and dO
//    in registers; K and V tiles of 64 keys stream through LDS the same way.
//      S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T.
//    S is recomputed here rather than exchanged: the two kernels share no
//    memory but their inputs, and each writes its gradients once.
//  * With a dS workspace (bf16 inputs, D = 128, every pair allowed) the
//    dK/dV kernel also stores dS, as the dQ products' B operands, and the
//    dQ kernel is replaced by one that streams them: dQ^T += K^T dS^T with
//    no scores computed a second time (attn_bwd_dqs_kernel).
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
#include <type_traits>

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
typedef __attribute__((address_space(3))) bwd_u32x2 bwd_lds_u32x2;
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

// The same copy issued from inline assembly, for a kernel that runs one
// workgroup per compute unit: the compiler does not count a load it cannot
// see, so it places no vmcnt(0) in front of the LDS reads that follow (it
// does for the builtin, and with no second workgroup to run meanwhile that
// wait would expose each copy's latency); the kernel waits with explicit
// vmcnt counts before the barrier that publishes a tile.  The descriptor
// fields are uniform; readfirstlane keeps them in scalar registers.
typedef unsigned int bwd_rsrc __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ void bwd_copy_asm(const unsigned char* src, uint32_t nrec, uint32_t ld2, bwd_lds_u8* dst,
                                             int wave, int lane, int i)
{
    constexpr int UPR = D / 8, RPD = 1024 / (2 * D);
    const int n = kBwdWaves * i + wave;
    const int row = n * RPD + lane / UPR;
    const uint32_t off = (uint32_t)row * ld2 + (uint32_t)((((lane % UPR) ^ bwd_swz<D>(row))) << 4);
    const uint64_t p = (uint64_t)src;
    const bwd_rsrc r{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu)),
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)nrec), 0x00020000u};
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass has no SGPR operand constraint
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(r),
                   "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(dst + n * 1024)))
                 : "memory", "m0");
#endif
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
// The two waves of a SIMD (w and w + 4) own the same 32 keys in two roles:
//   K side (w < 4): K rows as operands, dK accumulators; S = Q K^T, P
//   V side (w >= 4): V rows as operands, dV accumulators; dP = dO V^T
// and exchange P and dS through LDS.  Step i (query tile t_i), two phases:
//   1. K: S_i, P_i (bf16) -> LDS           V: dP_i - delta
//   2. V: dV += dO_i^T P_i, dS_i -> LDS     K: dK += Q_{i-1}^T dS_{i-1}
// so in each phase one wave's vector work runs beside the other's matrix
// work; dK trails by one step (Q tiles stay for three steps, dS is double
// buffered).  Operand reads run four matrix instructions ahead.
template <int D, bool MASKED>
__global__ __launch_bounds__(64 * kBwdWaves, 2) void attn_bwd_dkdv_kernel(const BwdArgs a)
{
    constexpr int ROWB = 2 * D, NKC = D / 16, NDB = D / 32, TB = kBwdT * ROWB;
    constexpr int CPT = TB / 1024 / kBwdWaves;        // copy instructions per wave per tensor per tile
    // An exchange buffer: key group x chunk x lane x 16 bytes, the two lane
    // halves of a chunk XH bytes apart and chunks XC apart (64 and 128 bytes
    // past a multiple of the 256-byte bank period), so that the transposing
    // reads of the dS workspace blocks, whose source lanes span two chunks and
    // both halves, hit distinct banks; every 16 lanes of a slot access stay
    // contiguous.
    constexpr int XH = 32 * 16 + 64, XC = 2 * XH, XB = 4 * 4 * XC;
    // LDS: Q[3] | dO[2] | lse[2] (log2 units) | delta[2] | P | dS[2]
    constexpr int OFF_Q = 0, OFF_O = 3 * TB, OFF_L = 5 * TB, OFF_D = OFF_L + 512, OFF_P = OFF_D + 512;
    constexpr int OFF_S = OFF_P + XB, SMEM = OFF_S + 2 * XB;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
    bwd_lds_u8* const L = (bwd_lds_u8*)smem;

    const uint32_t unit = xcd_logical(blockIdx.x, gridDim.x);
    const int64_t kt = unit % (uint32_t)a.n_tiles;
    const int64_t rest = unit / (uint32_t)a.n_tiles;
    const int64_t hh = rest % a.H, b = rest / a.H;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hg = lane >> 5;
    const int kg = wave & 3, role = wave >> 2;       // role 0: K side, 1: V side
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const uint32_t ld2 = (uint32_t)(H * D * 2);
    const int64_t k0 = kt * kBwdKeys;
    const int64_t kw0 = k0 + 32 * kg;           // first key of this wave
    const int64_t j = kw0 + l32;                 // this lane's key
    const bool wave_keys = kw0 < Sk;

    // this lane's K (K side) or V (V side) row as the B operand of S = Q K^T
    // or dP = dO V^T: features 16 kc + 8 hg .. +7 (zero past Sk)
    bwd_bf16x8 kvop[NKC];
    {
        const int64_t hoff = ((b * Sk) * H + hh) * D * 2;
        const uint32_t nrec = (uint32_t)((Sk - 1) * ld2 + D * 2);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const unsigned char*>(role == 0 ? a.k : a.v) + hoff), (short)0, nrec, 0x00020000);
        const uint32_t roff = j < Sk ? (uint32_t)j * ld2 : nrec;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            kvop[kc] = __builtin_bit_cast(
                bwd_bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, roff + (uint32_t)((2 * kc + hg) * 16), 0, 0));
    }

    // Masking.  Query i may see key j iff qpos(i) >= kpos(j); positions grow
    // within each piece of the query map, so the queries a key position p
    // allows are [s0, segq) u [s1, Sq) with s0, s1 the first indices of the
    // pieces at or above p.  Per lane (this key), per workgroup (its keys'
    // smallest position: the queries some key sees), per wave (smallest and
    // largest: some key / every key).
    const int32_t sq32 = (int32_t)Sq;
    int32_t segq = sq32;
    int32_t qs0 = 0, qs1 = sq32;
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

    // ---- staging: tile of step i into Q stage qs and dO / lse / delta stage os
    const unsigned char* qbase = static_cast<const unsigned char*>(a.q) + ((b * Sq) * H + hh) * D * 2;
    const unsigned char* obase = static_cast<const unsigned char*>(a.dout) + ((b * Sq) * H + hh) * D * 2;
    auto issue = [&](int t, int qs, int os) {
        const int64_t r0 = (int64_t)t * kBwdT;
        const int64_t nv = Sq - r0 < kBwdT ? Sq - r0 : kBwdT;
        const uint32_t nrec = (uint32_t)((nv - 1) * ld2 + D * 2);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            bwd_copy<D>(qbase + r0 * ld2, nrec, ld2, L + OFF_Q + qs * TB, wave, lane, i);
            bwd_copy<D>(obase + r0 * ld2, nrec, ld2, L + OFF_O + os * TB, wave, lane, i);
        }
        if (wave < 2) {
            const float* src = (wave == 0 ? a.lse : a.delta) + (b * Sq + r0) * H + hh;
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)src, (short)0, (uint32_t)((nv - 1) * H * 4 + 4), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, L + (wave == 0 ? OFF_L : OFF_D) + os * 256, 4,
                                                     (uint32_t)(lane * H * 4), 0, 0, 0);
        }
    };
    // the lse of stage os to log2 units, +inf for a row with no key (P = 0);
    // wave 0 copied it and runs this once its copy has landed
    auto convert_lse = [&](int os) {
        __attribute__((address_space(3))) float* p = (__attribute__((address_space(3))) float*)(L + OFF_L + os * 256) + lane;
        const float x = *p;
        *p = x == -INFINITY ? INFINITY : x * kBwdLog2e;
    };

    const int rrow = l32 * ROWB, rx = (hg ^ bwd_swz<D>(l32)) << 4;
    const BwdTr trs = bwd_tr_setup<D>(lane);
    // exchange slot of chunk c of this key group
    auto xslot = [&](int c) { return (kg * 4 + c) * XC + (lane >> 5) * XH + (lane & 31) * 16; };

    bwd_f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
    const float c2 = a.scale_log2;

    // S = Q K^T or dP = dO V^T for the tile's two 32-row blocks (rows
    // 32 qb + l32), the blocks' instructions alternating so that two
    // accumulations are in flight; operands read four instructions ahead
    int rxl = rx;            // per-step copies, opaque to the compiler so that the
    BwdTr trl = trs;         // derived LDS addresses are formed at use, not kept live
    auto rows_product = [&](const bwd_lds_u8* tile, bwd_f32x16 (&r)[2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int v = 0; v < 16; ++v) r[qb][v] = 0.f;
        constexpr int N = 2 * NKC;
        auto rd = [&](int n) { return bwd_row<D>(tile, (n & 1) * 32 * ROWB + rrow, rxl, n >> 1); };
        bwd_bf16x8 op[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) op[n] = rd(n);
#pragma unroll
        for (int n = 0; n < N; ++n) {
            r[n & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n & 3], kvop[n >> 1], r[n & 1], 0, 0, 0);
            if (n + 4 < N) op[n & 3] = rd(n + 4);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // acc^T += tile^T X over the tile's 64 rows: chunk c of X in x[c]
    auto tr_product = [&](const bwd_lds_u8* tile, const bwd_u32x4 (&x)[4]) {
        constexpr int N = 4 * NDB;
        auto rd = [&](int r) { return bwd_tr<D>(tile, 16 * (r / NDB) * ROWB, trl, r % NDB); };
        bwd_bf16x8 op[2];
        op[0] = rd(0);
        op[1] = rd(1);
#pragma unroll
        for (int r = 0; r < N; ++r) {
            acc[r % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[r & 1], __builtin_bit_cast(bwd_bf16x8, x[r / NDB]),
                                                                  acc[r % NDB], 0, 0, 0);
            if (r + 2 < N) op[r & 1] = rd(r + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    int t = next_live(0);
    int qs = 0, os = 0, dsb = 0;           // stages of the current step
    if (t < n_qt) issue(t, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);    // the operands and tile t landed
    if (wave == 0 && t < n_qt) convert_lse(0);
    __syncthreads();

    bool prev_any = false;                 // this wave's keys met the previous tile
    int qprev = 0;                         // Q stage of the previous tile
    bwd_f32x16 r2[2];                      // S (K side) / dP - delta (V side) of the tile's two blocks
    while (t < n_qt) {
        rxl = rx;
        trl = trs;
        asm volatile("" : "+v"(rxl), "+v"(trl.base[0]), "+v"(trl.base[1]), "+v"(trl.x[0]), "+v"(trl.x[1]));
        const int t1 = next_live(t + 1);
        const int qn = qs == 2 ? 0 : qs + 1;
        if (t1 < n_qt) issue(t1, qn, os ^ 1);

        const int32_t i0 = t * kBwdT, i1 = i0 + kBwdT < sq32 ? i0 + kBwdT : sq32;
        bool any = wave_keys, per_elem = false;
        if (MASKED && any) {
            any = meets(i0, i1, wa0, wa1);
            per_elem = !inside(i0, i1, wf0, wf1);
        }
        const bwd_lds_u8* Ol = L + OFF_O + os * TB;

        // ---- phase 1: S = Q K^T (K side) or dP = dO V^T (V side) --------
        if (any) {
            rows_product(role == 0 ? L + OFF_Q + qs * TB : Ol, r2);
            if (role == 0) {
                // P in bf16, chunk c = 2 qb + g4 / 2, slots 4 hg + {0..3, 8..11}
                const bwd_lds_u8* Ll = L + OFF_L + os * 256;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    bwd_u32x4 pw[2];
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int ql = 32 * qb + 8 * g4 + 4 * hg;   // 4 consecutive tile queries
                        const bwd_f32x4 l2 = *(const bwd_lds_f32x4*)(Ll + ql * 4);
                        float p[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float sv = r2[qb][4 * g4 + e];
                            if (MASKED && per_elem) {
                                const int32_t iq = i0 + ql + e;
                                const bool ok = iq < segq ? iq >= qs0 : iq >= qs1;
                                if (!ok) sv = -INFINITY;
                            }
                            p[e] = __builtin_amdgcn_exp2f(fmaf(sv, c2, -l2[e]));
                        }
                        pw[g4 >> 1][2 * (g4 & 1)] = bwd_pack(p[0], p[1]);
                        pw[g4 >> 1][2 * (g4 & 1) + 1] = bwd_pack(p[2], p[3]);
                    }
#pragma unroll
                    for (int h = 0; h < 2; ++h) *(bwd_lds_u32x4*)(L + OFF_P + xslot(2 * qb + h)) = pw[h];
                }
            } else {
                const bwd_lds_u8* Dl = L + OFF_D + os * 256;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const bwd_f32x4 dl = *(const bwd_lds_f32x4*)(Dl + (32 * qb + 8 * g4 + 4 * hg) * 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) r2[qb][4 * g4 + e] -= dl[e];
                    }
            }
        }
        bwd_barrier();

        // ---- phase 2: dV^T += dO^T P (V side, this tile) or dK^T += Q^T dS
        // (K side, previous tile), then the V side's dS -------------------
        if (role == 0 ? prev_any : any) {
            bwd_u32x4 x[4];
            const int xo = role == 0 ? OFF_S + (dsb ^ 1) * XB : OFF_P;
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = *(const bwd_lds_u32x4*)(L + xo + xslot(c));
            tr_product(role == 0 ? L + OFF_Q + qprev * TB : Ol, x);
            if (role == 1) {
                // dS = P (dP - delta), chunk c = 2 qb + h: dword e holds
                // rows 8 h + 2 e, 8 h + 2 e + 1 of block qb
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int qb = c >> 1, h = c & 1;
                    bwd_u32x4 sw;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sw[e] = bwd_pack(bwd_lo(x[c][e]) * r2[qb][8 * h + 2 * e],
                                         bwd_hi(x[c][e]) * r2[qb][8 * h + 2 * e + 1]);
                    *(bwd_lds_u32x4*)(L + OFF_S + dsb * XB + xslot(c)) = sw;
                }
                if constexpr (!MASKED) {
                    if (a.ds != nullptr) {
                        // dS^T into the workspace as B-operand blocks (16
                        // keys x 32 queries, 1 KB each), read back from this
                        // wave's slots with transposing reads: block (kk, qq)
                        // holds keys 16 kk .. +15 of the group and queries
                        // 32 qq .. +31 of the tile.  Slot (chunk c, lane
                        // 32 hg + key) holds at byte 8 ep + 2 x the pair of
                        // that key with tile row 32 qb + 16 h + 8 ep + 4 hg + x
                        // (c = 2 qb + h); source lane (g, e, a) = (lane / 16,
                        // lane / 4 % 4, lane % 4) addresses key 16 kk +
                        // 4 (g / 2) + e at rows 32 qq + 16 (g % 2) + 8 (a / 2)
                        // + 4 (a % 2) + {0..3}, so result lane 32 e' + n gets
                        // keys 16 kk + 4 e' + {0..3} of query 32 qq + n, and
                        // the same 8 keys on: keys + {8..11}.
                        const int g = lane >> 4, se = (lane >> 2) & 3, sa = lane & 3;
#pragma unroll
                        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                            for (int kk = 0; kk < 2; ++kk) {
                                const int64_t qc = (i0 >> 5) + qq, kc = (kw0 >> 4) + kk;
                                if (qc >= a.ds_nq || kc >= a.ds_nk) continue;
                                const bwd_lds_u8* src = L + OFF_S + dsb * XB + (kg * 4 + 2 * qq + (g & 1)) * XC +
                                                        (sa & 1) * XH + (16 * kk + 4 * (g >> 1) + se) * 16 +
                                                        (sa >> 1) * 8;
                                const bwd_i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_i16x4*)src);
                                const bwd_i16x4 y =
                                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_i16x4*)(src + 8 * 16));
                                *reinterpret_cast<bwd_u32x4*>(static_cast<unsigned char*>(a.ds) +
                                                              (((b * H + hh) * a.ds_nq + qc) * a.ds_nk + kc) * 1024 +
                                                              lane * 16) =
                                    __builtin_bit_cast(bwd_u32x4, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
                            }
                    }
                }
            }
        }

        // the copies of tile t1 landed; wave 0 converts its lse
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if (wave == 0 && t1 < n_qt) convert_lse(os ^ 1);
        bwd_barrier();
        prev_any = any;
        qprev = qs;
        qs = qn;
        os ^= 1;
        dsb ^= 1;
        t = t1;
    }
    // the last tile's dK
    if (role == 0 && prev_any) {
        bwd_u32x4 x[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = *(const bwd_lds_u32x4*)(L + OFF_S + (dsb ^ 1) * XB + xslot(c));
        tr_product(L + OFF_Q + qprev * TB, x);
    }

    // ---- epilogue: the K side writes dK (scaled), the V side dV ----------
    if (j >= Sk) return;
    const float mul = role == 0 ? a.scale : 1.f;
    void* out = role == 0 ? a.dk : a.dv;
    const int64_t orow = ((b * Sk + j) * H + hh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int f = 32 * db + 8 * g4 + 4 * hg;
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = acc[db][4 * g4 + e] * mul;
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
            // One 32-key block at a time: S^T = K Q^T and dP^T = V dO^T
            // (lane = query, register v = key 32 jb + 8 (v / 4) + 4 hg + v % 4),
            // dS^T, then dQ^T += K^T dS^T (lane = query, register v = feature
            // 32 db + 8 (v / 4) + 4 hg + v % 4).  The LDS operands are read
            // four matrix instructions ahead (two for the transposing reads),
            // and scheduling barriers keep that order.
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const int rb = jb * 32 * ROWB + rrow;
                constexpr int NS = 2 * NKC;                 // S and dP instructions, alternating
                auto rd = [&](int r) { return bwd_row<D>((r & 1) ? Vl : Kl, rb, rx, r >> 1); };
                bwd_f32x16 sc, dp;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    sc[v] = 0.f;
                    dp[v] = 0.f;
                }
                bwd_bf16x8 op[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) op[r] = rd(r);
#pragma unroll
                for (int r = 0; r < NS; ++r) {
                    if (r & 1)
                        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[r & 3], dop[r >> 1], dp, 0, 0, 0);
                    else
                        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[r & 3], qop[r >> 1], sc, 0, 0, 0);
                    if (r + 4 < NS) op[r & 3] = rd(r + 4);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // dS^T in bf16: chunk c = 2 jb + h of the tile, slots 4 hg + {0..3, 8..11}
                bwd_u32x4 sw[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float d[2];
#pragma unroll
                        for (int x = 0; x < 2; ++x) {
                            const int v = 8 * h + 2 * e + x;
                            float sv = sc[v];
                            if (per_elem) {
                                const int32_t jj = j0 + 32 * jb + 8 * (v >> 2) + 4 * hg + (v & 3);
                                const bool ok = jj < segk ? jj < lim0 : jj < lim1;
                                if (!ok) sv = -INFINITY;
                            }
                            const float p = __builtin_amdgcn_exp2f(fmaf(sv, c2, -l2));
                            d[x] = p * (dp[v] - dlt);
                        }
                        sw[h][e] = bwd_pack(d[0], d[1]);
                    }
                constexpr int NQ = 2 * NDB;                 // dQ instructions of the block
                auto tr = [&](int r) { return bwd_tr<D>(Kl, (32 * jb + 16 * (r / NDB)) * ROWB, trs, r % NDB); };
                bwd_bf16x8 ta[2];
                ta[0] = tr(0);
                ta[1] = tr(1);
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const int db = r % NDB;
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[r & 1], __builtin_bit_cast(bwd_bf16x8, sw[r / NDB]),
                                                                      acc[db], 0, 0, 0);
                    if (r + 2 < NQ) ta[r & 1] = tr(r + 2);
                    __builtin_amdgcn_sched_barrier(0);
                }
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
// dQ from the dS workspace (D = 128, every key allowed)
// ==========================================================================
// dQ^T += K^T dS^T per 64-key tile with dS^T read back from the workspace
// the dK/dV kernel filled, instead of recomputed: a workgroup owns 256 query
// rows of one (batch, head), 32 per wave.  The workspace holds dS^T as the
// matrix instructions' B operands, so each wave loads its own operands
// straight into registers (one 1 KB load per 16 keys), kDqsPF tiles ahead;
// the K tiles stream through kDqsStages LDS stages (one copy per wave per
// 1 KB, kDqsStages - 1 tiles ahead) and are read transposed as the A
// operands, three instructions ahead.  The work is the dS stream (2 bytes
// per pair) and 2 D FLOP per pair.
constexpr int kDqsStages = 6;
constexpr int kDqsPF = 4;
// s_waitcnt immediate waiting for vmcnt <= n only (vmcnt is split over
// bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima)
constexpr int bwd_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
__global__ __launch_bounds__(64 * kBwdWaves, 1) void attn_bwd_dqs_kernel(const BwdArgs a)
{
    constexpr int D = 128, ROWB = 2 * D, NDB = D / 32, TB = kBwdT * ROWB;
    constexpr int CPT = TB / 1024 / kBwdWaves;       // K copy instructions per wave per tile
    constexpr int NST = kDqsStages, PF = kDqsPF;
    static_assert(CPT * (NST - 2) + 4 * PF <= 63 && (4 + CPT) * (NST - 2) <= 63, "vmcnt counts up to 63");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NST * TB];

    const uint32_t unit = xcd_logical(blockIdx.x, gridDim.x);
    const int64_t qt = unit % (uint32_t)a.n_tiles;
    const int64_t rest = unit / (uint32_t)a.n_tiles;
    const int64_t hh = rest % a.H, b = rest / a.H;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, hg = lane >> 5;
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const uint32_t ld2 = (uint32_t)(H * D * 2);
    const int64_t qc = qt * (kBwdRows / 32) + wave;               // this wave's 32-query block
    const int64_t i = 32 * qc + (lane & 31);                      // this lane's query row
    const int n_kt = (int)((Sk + kBwdT - 1) / kBwdT);

    // K tile t into stage st (zeros past the last tile, so that every wave
    // issues the same number of copies each step)
    const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + ((b * Sk) * H + hh) * D * 2;
    bwd_lds_u8* const L = (bwd_lds_u8*)smem;
    auto issue_k = [&](int t, int st) {
        const int64_t r0 = (int64_t)t * kBwdT;
        const int64_t nv = t < n_kt ? (Sk - r0 < kBwdT ? Sk - r0 : kBwdT) : 0;
        const unsigned char* src = t < n_kt ? kbase + r0 * ld2 : kbase;
#pragma unroll
        for (int c = 0; c < CPT; ++c)
            bwd_copy_asm<D>(src, nv > 0 ? (uint32_t)((nv - 1) * ld2 + ROWB) : 0u, ld2, L + st * TB, wave, lane, c);
    };
    // this wave's dS^T blocks (key groups 0 .. ds_nk - 1, 1 KB each, in
    // order; reads from the end on, and for a wave past the last query
    // block, return zero)
    const bool live = qc < a.ds_nq;
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<unsigned char*>(a.ds) + (live ? (((b * H + hh) * a.ds_nq + qc) * a.ds_nk) * 1024 : 0), (short)0,
        live ? (uint32_t)(a.ds_nk * 1024) : 0u, 0x00020000);
    auto load_s = [&](int t, bwd_bf16x8 (&sd)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            sd[q] = __builtin_bit_cast(bwd_bf16x8,
                                       __builtin_amdgcn_raw_buffer_load_b128(sr, (uint32_t)((4 * t + q) * 1024 + lane * 16),
                                                                             0, 0));
    };
    const BwdTr trs = bwd_tr_setup<D>(lane);

    bwd_f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;

    // prologue: K tiles 0 .. NST - 2, then the dS of tiles 0 .. PF - 1
    for (int t = 0; t < NST - 1; ++t) issue_k(t, t);
    bwd_bf16x8 sd[PF][4];
#pragma unroll
    for (int p = 0; p < PF; ++p) load_s(p, sd[p]);
    asm volatile("" ::: "memory");   // the loads above stay above the wait
    __builtin_amdgcn_s_waitcnt(bwd_vmcnt(CPT * (NST - 2) + 4 * PF));   // K tile 0 has landed
    __syncthreads();

    // Step t: the products of tile t, the dS of tile t + PF into the
    // registers tile t used, the copies of K tile t + NST - 1 into the stage
    // tile t - 1 used.  Before the barrier that ends step t, K tile t + 1
    // must have landed: it was issued last in step t + 2 - NST (or in the
    // prologue), and every step issues 4 loads and CPT copies, so at most
    // (4 + CPT) (NST - 2) loads after it may still run.  The steps run in
    // groups of PF with no exit in between (past the last tile, K and dS
    // read as zero and add nothing), so the compiler's own waits for the dS
    // registers see the PF - 1 steps of loads issued since; it does not see
    // the copies, which only makes those waits stricter.
    auto step = [&](auto slot_tag, int t) {
        constexpr int s = decltype(slot_tag)::value;
        const bwd_lds_u8* Kl = L + (t % NST) * TB;
        auto tr = [&](int r) { return bwd_tr<D>(Kl, 16 * (r / NDB) * ROWB, trs, r % NDB); };
        bwd_bf16x8 ka[4];
        ka[0] = tr(0);
        ka[1] = tr(1);
        ka[2] = tr(2);
#pragma unroll
        for (int r = 0; r < 4 * NDB; ++r) {
            if (r + 3 < 4 * NDB) ka[(r + 3) & 3] = tr(r + 3);
            acc[r % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[r & 3], sd[s][r / NDB], acc[r % NDB], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        load_s(t + PF, sd[s]);
        issue_k(t + NST - 1, (t + NST - 1) % NST);
        asm volatile("" ::: "memory");   // the count below includes these loads
        __builtin_amdgcn_s_waitcnt(bwd_vmcnt((4 + CPT) * (NST - 2)));
        bwd_barrier();
    };
    static_assert(PF == 4, "the step groups below are written out for PF = 4");
    for (int t0 = 0; t0 < n_kt; t0 += PF) {
        step(std::integral_constant<int, 0>{}, t0);
        step(std::integral_constant<int, 1>{}, t0 + 1);
        step(std::integral_constant<int, 2>{}, t0 + 2);
        step(std::integral_constant<int, 3>{}, t0 + 3);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);

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
    if constexpr (D == 128 && !M) {
        if (a.ds != nullptr)
            return launch_kernel(attn_bwd_dqs_kernel, dim3((uint32_t)(a.B * a.H * a.n_tiles)), dim3(64 * kBwdWaves), 0,
                                 s, a);
    }
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
