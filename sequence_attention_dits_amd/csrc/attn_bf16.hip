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
//  * A workgroup owns 256 query rows of one (batch, head): 8 wavefronts of 32
//    rows, two per SIMD, so each K/V tile staged in LDS serves 256 rows.  Q
//    stays in registers.
//  * K and V stream in tiles of 64 keys, issued two tiles ahead of the one
//    being computed.  K is copied by buffer loads that write LDS directly (no
//    registers, no store instructions) into three LDS stages.  V passes
//    through two register sets: each lane loads two keys x 8 features as
//    16-byte loads that cover whole rows, and writes them transposed into one
//    of two LDS stages, which hold 16-byte units of 8 keys of one feature.
//    One barrier per tile; it waits only for the LDS stores and the copies of
//    the next tile, never for the loads still running.  With D = 128 each
//    wave's four global loads per tile sit between its score instructions,
//    so the waves do not all queue on the address unit right after the
//    barrier.  Loads past the end of the keys return zeros.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane owns one query row (lane % 32) and 32
//    of the tile's 64 keys, so the row maximum and sum need one cross-half
//    exchange (v_permlane32_swap).
//  * The score registers, rounded to bf16 (v_cvt_pk_bf16_f32), are directly
//    the P operand of O^T += V^T P^T: a lane half holds keys 4h + {0..3} and
//    4h + {8..11} of each 16-key chunk, and the V unit it reads holds those
//    same 8 keys in that order, so each V operand is one 16-byte LDS read.  O^T
//    keeps one query row per lane, so the softmax rescale is a per-lane
//    multiply.
//  * The running maximum is only raised when it grows by more than 2^8 in
//    exp2 units (a wave-uniform branch, rare after the first tile); between
//    raises the exponentials use the stale maximum, which is exact because O
//    and the sum share it, and stays far from overflow.
//  * K is XOR-swizzled and V padded in 16-byte units so that operand reads
//    and V stores are free of bank conflicts.
//  * exp2 with scale * log2(e) folded into one multiply-add; the LSE is
//    converted back to the natural log at the end.  Rows with no allowed key
//    give o = 0, lse = -inf.
#include "attn_common.h"

#include <stdlib.h>

#include <type_traits>

namespace uaa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kBM = 256;  // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr int kWaves = 8;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kRescaleThreshold = 8.0f;  // in log2 units of the softmax weights

// two floats -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
// the two bf16 halves of a dword as floats
__device__ __forceinline__ float bf16_lo(unsigned int x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ unsigned int pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(unsigned int, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Workgroup barrier for LDS: global loads and LDS copies still in flight
// stay in flight (a plain __syncthreads waits for them); the caller waits for
// the copies it needs with an explicit vmcnt.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS stores are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Maximum of three floats (v_maximum3_f32: no NaN quieting of the inputs).
__device__ __forceinline__ float fmax3(float a, float b, float c)
{
    return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// Key offset, inside a 16-key chunk, of P operand slot s of lane half h:
// 4h + {0,1,2,3,8,9,10,11}[s].
__device__ __forceinline__ int p_slot_key(int s) { return s < 4 ? s : s + 4; }

// Issue load i of this wave's buffer loads that copy rows of the K tile into
// LDS (i < 64 / RPD / kWaves): load i writes the 1 KB at byte (kWaves * i + wave) * 1024 of the tile, lane s its
// 16-byte slot s: tile row (kWaves * i + wave) * RPD + s / UPR, physical unit
// s % UPR, which holds logical unit (s % UPR) ^ (row % 16).  Bytes past nrec
// read as zero.
template <int D>
__device__ __forceinline__ void fill_k(const unsigned char* ksrc, uint32_t nrec, unsigned char* kdst, int wave,
                                       int lane, uint32_t ld2, int i)
{
    constexpr int UPR = D / 8, RPD = 1024 / (D * 2);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)ksrc, (short)0, nrec, 0x00020000);
    lds_u8* kd = (lds_u8*)kdst;
    const int n = kWaves * i + wave;
    const int row = n * RPD + lane / UPR;
    const uint32_t off = (uint32_t)row * ld2 + (uint32_t)(((lane % UPR) ^ (row & (UPR - 1))) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kd + n * 1024, 16, off, 0, 0, 0);
}

// Occupancy target: 2 waves per SIMD (one workgroup per CU) for D = 128;
// for D = 64 4 waves per SIMD, i.e. at most 128 VGPRs, so that two
// workgroups share a CU (72 KB of LDS each) -- one VGPR more halves it.
template <int D, bool MASKED, bool OUT_BF16, bool SPLIT>
__global__ __launch_bounds__(64 * kWaves, D == 64 ? 4 : 2) void attn_bf16_kernel(const AttnArgs a)
{
    constexpr int UPR = D / 8;               // 16-byte units per row
    constexpr int ROWB = D * 2;              // bytes per row
    constexpr int NKC = D / 16;              // k-chunks of the score product
    constexpr int NDB = D / 32;              // 32-wide feature blocks of the output
    constexpr int TB = kBN * ROWB;           // bytes of one K or V tile

    // V layout (D = 128): unit group g (8 keys) holds feature f at byte
    // g * VGS + 16 * f + 16 * (f / 16): one padding unit after every 16
    // features keeps both the 4-byte stores and the 16-byte operand reads
    // free of bank conflicts.  D = 64 uses an unpadded XOR-swizzled layout.
    constexpr int VGS = D == 128 ? (D + D / 16) * 16 : D * 16;   // bytes per unit group
    constexpr int VTB = 8 * VGS;                                  // bytes of one V stage
    constexpr int QB = kWaves * 32 * ROWB;   // Q staging: 32 rows per wave
    // K stages 0..2, V stages 0..1, then the Q staging region (one workgroup
    // runs per CU, so the 146 KB for D = 128 cost no occupancy)
    __shared__ __attribute__((aligned(1024))) unsigned char smem[3 * TB + 2 * VTB + QB];

    int64_t qt, hh, b;
    uint32_t unit = 0;   // with SPLIT: this workgroup runs key piece `piece` of `np` of this unit
    int piece = 0, np = 1;
    if constexpr (SPLIT) {
        // The pieces of the split units come first, so that they are
        // dispatched first and their combine overlaps the whole units' work;
        // then the whole units.  Each range is XCD-grouped on its own.
        const uint32_t L = blockIdx.x, nw = (uint32_t)a.n_whole, npc = gridDim.x - nw;
        if (L < npc) {
            const uint32_t l = xcd_logical(L, npc);
            np = a.split_p;
            unit = nw + l / (uint32_t)np;
            piece = (int)(l % (uint32_t)np);
        } else {
            unit = xcd_logical(L - npc, nw);
        }
        unit_coords(a, unit, qt, hh, b);
    } else if (MASKED && gridDim.x % 8u == 0u && (gridDim.x / 8u) % (uint32_t)a.n_qtiles == 0u) {
        // Masked, every XCD holding whole heads: with every mask kind later
        // rows of a head see at least as many keys, so each XCD's workgroups
        // (blockIdx = 8 j + x on XCD x) take its heads' q tiles last-first
        // with the heads interleaved -- the longest units of the XCD are
        // dispatched first and the short ones fill in at the end.
        const uint32_t nq = (uint32_t)a.n_qtiles, per = gridDim.x / 8u, hpx = per / nq;
        const uint32_t x = blockIdx.x % 8u, j = blockIdx.x / 8u;
        unit_coords(a, x * per + (j % hpx) * nq + (nq - 1u - j / hpx), qt, hh, b);
    } else {
        decode_tile(a, qt, hh, b);
        // masked: q tiles of a head last-first (see above)
        if (MASKED) qt = a.n_qtiles - 1 - qt;
    }
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31, hg = lane >> 5;
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const int64_t RH = a.row_heads, h_in = a.head0 + hh;   // heads per input token; this head's slot
    const uint32_t ld2 = (uint32_t)(RH * D * 2);   // bytes between consecutive tokens of the inputs
    const int64_t q0 = qt * kBM;
    const int64_t i = q0 + 32 * wave + l32;       // this lane's query row

    const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + ((b * Sk) * RH + h_in) * D * 2;
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + ((b * Sk) * RH + h_in) * D * 2;

    // Masking: position ranges of the workgroup's rows and of this wave's,
    // and for this lane's row the allowed keys as index limits: key j is
    // allowed iff j < lim0 (first piece of the key map, j < segk) or j < lim1
    // (second piece).  Each piece of a position map increases, so the allowed
    // keys of a piece are a prefix of it; without a mask only the ragged end
    // of the keys counts.
    int64_t wg_qmax = 0, w_qmin = 0, w_qmax = 0;
    const bool wave_live = q0 + 32 * wave < Sq;
    const int32_t sk32 = (int32_t)Sk;
    int32_t segk = sk32, lim0 = sk32, lim1 = sk32;
    if (MASKED) {
        int64_t dummy;
        const int64_t wg_hi = q0 + kBM < Sq ? q0 + kBM : Sq;
        pos_range(a.qmap, q0, wg_hi, dummy, wg_qmax);
        if (wave_live) {
            const int64_t w_lo = q0 + 32 * wave;
            const int64_t w_hi = w_lo + 32 < Sq ? w_lo + 32 : Sq;
            pos_range(a.qmap, w_lo, w_hi, w_qmin, w_qmax);
        }
        segk = (int32_t)(a.kmap.seg_len < Sk ? a.kmap.seg_len : Sk);
        const int64_t qp = pos_of(a.qmap, i);
        lim0 = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, qp, segk);
        lim1 = segk + (int32_t)allowed_prefix(a.kmap.base1, a.kmap.stride, qp, Sk - segk);
    }
    // key tiles [t_beg, n_tiles) of this workgroup: all of them, or one piece
    const int n_all = (int)((Sk + kBN - 1) / kBN);
    const int t_beg = SPLIT ? (int)((int64_t)piece * n_all / np) : 0;
    const int n_tiles = SPLIT ? (int)((int64_t)(piece + 1) * n_all / np) : n_all;
    // Key index sets as unions of two intervals, one per piece of the key
    // map (positions increase within a piece, so the keys a position q may
    // see are a prefix of each piece), fixed here once so that the tile loop
    // does a few 32-bit compares per tile:
    //   live   [0, ln0) u [segk, segk + ln1): keys the workgroup's last row sees
    //   wave   [0, wa0) u [segk, segk + wa1): keys some row of this wave sees
    //   full   [0, wf0) u [segk, segk + wf1): keys every row of this wave sees
    int32_t ln0 = sk32, ln1 = 0, wa0 = sk32, wa1 = 0, wf0 = sk32, wf1 = 0;
    if (MASKED) {
        const int64_t n1 = Sk - segk;
        ln0 = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, wg_qmax, segk);
        ln1 = (int32_t)allowed_prefix(a.kmap.base1, a.kmap.stride, wg_qmax, n1);
        wa0 = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, w_qmax, segk);
        wa1 = (int32_t)allowed_prefix(a.kmap.base1, a.kmap.stride, w_qmax, n1);
        wf0 = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, w_qmin, segk);
        wf1 = (int32_t)allowed_prefix(a.kmap.base1, a.kmap.stride, w_qmin, n1);
    }
    // does [j0, j1) meet [0, p0) u [segk, segk + p1)?
    auto meets = [&](int32_t j0, int32_t j1, int32_t p0, int32_t p1) {
        return j0 < p0 || (j1 > segk && (j0 > segk ? j0 : segk) < segk + p1);
    };
    // is [j0, j1) inside it?
    auto inside = [&](int32_t j0, int32_t j1, int32_t p0, int32_t p1) {
        return (j0 >= segk || (j1 < segk ? j1 : segk) <= p0) && (j1 <= segk || j1 <= segk + p1);
    };
    // live tiles: [0, lt0) and [lt1b, lt1e)
    const int lt0 = (ln0 + kBN - 1) / kBN;
    const int lt1b = ln1 > 0 ? segk / kBN : n_all, lt1e = ln1 > 0 ? (segk + ln1 + kBN - 1) / kBN : n_all;
    auto next_live = [&](int t) -> int {   // first live tile >= t, or n_tiles
        if (!MASKED || t < lt0) return t < n_tiles ? t : n_tiles;
        if (t < lt1b) t = lt1b;
        return t < lt1e && t < n_tiles ? t : n_tiles;
    };

    // Q: each wave copies its own 32 rows into its own LDS region with
    // whole-row loads (1 KB, RPD rows, per instruction; 16-byte units
    // swizzled as in the K tile; rows past Sq read as zero) and reads its
    // operands back once the prologue's copies have landed -- instead of
    // gathering 16-byte pieces of 32 rows per load instruction.  Gathering
    // from token shards, the rows of one shard are copied per pass (a wave's
    // rows straddle a shard boundary only when a shard's length is not a
    // multiple of 32), with the lanes of other rows masked off.
    lds_u8* const qst = (lds_u8*)(smem + 3 * TB + 2 * VTB) + wave * 32 * ROWB;
    if (next_live(t_beg) < n_tiles) {   // a workgroup without a live key tile needs no Q
        constexpr int UPRQ = D / 8, RPD = 1024 / ROWB;
        const int64_t r0 = q0 + 32 * wave;
        auto copy_rows = [&](const unsigned char* base, uint32_t nrec, int lo, int hi, bool all) {
            // rows [lo, hi) of the wave's 32 (all: every row, the rest reading
            // as zero) from `base` = the row r0 + lo
            const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, 0x00020000);
#pragma unroll
            for (int n = 0; n < 32 * ROWB / 1024; ++n) {
                const int row = n * RPD + lane / UPRQ;
                const uint32_t off = (uint32_t)(row - lo) * ld2 + (uint32_t)(((lane % UPRQ) ^ (row & (UPRQ - 1))) * 16);
                if (all || (row >= lo && row < hi)) __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, qst + n * 1024, 16, off, 0, 0, 0);
            }
        };
        if (a.n_qsh == 0) {
            const unsigned char* qbase = static_cast<const unsigned char*>(a.q) + ((b * Sq) * RH + h_in) * D * 2;
            const uint32_t nrec = Sq > r0 ? (uint32_t)((Sq - 1 - r0) * ld2 + D * 2) : 0u;
            copy_rows(qbase + (Sq > r0 ? r0 : 0) * ld2, nrec, 0, 32, true);
        } else {
            const int64_t r_end = Sq < r0 + 32 ? Sq : r0 + 32;
            if (r_end < r0 + 32) copy_rows(static_cast<const unsigned char*>(a.k), 0u, (int)(r_end > r0 ? r_end - r0 : 0), 32, false);
            int p = 0;
            for (int64_t rs = r0; rs < r_end;) {   // one pass per shard the rows touch
                while (a.q_row0[p + 1] <= rs) ++p;
                const int64_t sp0 = a.q_row0[p], sp = a.q_row0[p + 1] - sp0;
                const int64_t re = a.q_row0[p + 1] < r_end ? a.q_row0[p + 1] : r_end;
                const unsigned char* sbase = static_cast<const unsigned char*>(a.q_sh[p]) +
                                             ((b * sp + (rs - sp0)) * RH + h_in) * D * 2;
                copy_rows(sbase, (uint32_t)((re - rs - 1) * ld2 + D * 2), (int)(rs - r0), (int)(re - r0),
                          rs == r0 && re == r0 + 32);
                rs = re;
            }
        }
    }

    // ---- V staging ---------------------------------------------------------
    // D = 128: wave w stages unit group g = w.  Lane (i, b) = (lane / 16,
    // lane % 16) loads keys p_slot_key(2i) and p_slot_key(2i) + 1 of the group
    // (key 16*(g/2) + 4*(g%2) + p_slot_key(2i)), features 8b .. 8b+7, as two
    // 16-byte loads that cover four whole rows per instruction, and stores
    // for each feature the 2-key dword at byte 4i of its unit.
    // D = 64: lane (g, h, q) = (tid % 8, part, quad) loads KPL = 2 keys x 4
    // features as 8-byte loads and writes KPL keys of each feature.
    constexpr int KPL = D == 128 ? 2 : D / 32;   // keys per lane
    constexpr int VLD = D == 128 ? 4 : 2;        // dwords per V load
    typedef unsigned int vld_t __attribute__((ext_vector_type(VLD)));
    vld_t vst[2][KPL];    // two register sets: tiles t+1 and t+2 are in flight
    uint32_t v_goff, v_soff;   // global byte offset in the tile, LDS byte offset in the stage
    if constexpr (D == 128) {
        const int g = wave, vi = lane >> 4, vb = lane & 15;
        v_goff = (uint32_t)(16 * (g >> 1) + 4 * (g & 1) + p_slot_key(2 * vi)) * ld2 + vb * 16;
        v_soff = (uint32_t)(g * VGS + 128 * vb + 16 * (vb >> 1) + 4 * vi);
    } else {
        constexpr int HPARTS = 8 / KPL;
        const int vg = tid & 7, vh = (tid >> 3) & (HPARTS - 1), vq = tid / (8 * HPARTS);
        v_goff = (uint32_t)(16 * (vg >> 1) + 4 * (vg & 1) + p_slot_key(KPL * vh)) * ld2 + vq * 8;
        v_soff = 0;
    }
    // a descriptor per tile (scalar work only) whose range ends at the last key
    auto v_rsrc = [&](int t) {
        const int64_t j0 = (int64_t)t * kBN;
        const uint32_t nrec = (uint32_t)((Sk - 1 - j0) * ld2 + D * 2);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + j0 * ld2), (short)0, nrec, 0x00020000);
    };
    auto load_v_part = [&](__amdgpu_buffer_rsrc_t tr, auto set_tag, int r) {
        constexpr int set = decltype(set_tag)::value;
        // keys of one lane are consecutive inside each p_slot_key group of 4
        const uint32_t off = v_goff + (uint32_t)(p_slot_key(r) - p_slot_key(0)) * ld2;
        if constexpr (VLD == 4)
            vst[set][r] = __builtin_bit_cast(vld_t, __builtin_amdgcn_raw_buffer_load_b128(tr, off, 0, 0));
        else
            vst[set][r] = __builtin_bit_cast(vld_t, __builtin_amdgcn_raw_buffer_load_b64(tr, off, 0, 0));
    };
    auto load_v = [&](int t, auto set_tag) {
        const __amdgpu_buffer_rsrc_t tr = v_rsrc(t);
#pragma unroll
        for (int r = 0; r < KPL; ++r) load_v_part(tr, set_tag, r);
    };
    auto store_v = [&](auto set_tag) {   // register set s goes to V stage s
        constexpr int set = decltype(set_tag)::value;
        lds_u8* V = (lds_u8*)(smem + 3 * TB + set * VTB) + v_soff;
        if constexpr (D == 128) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // feature 8b + e: half e%2 of dword e/2 of both keys
                const unsigned int sel = (e & 1) ? 0x07060302u : 0x05040100u;
                const unsigned int w = __builtin_amdgcn_perm(vst[set][1][e >> 1], vst[set][0][e >> 1], sel);
                *(__attribute__((address_space(3))) unsigned int*)(V + 16 * e) = w;
            }
        } else {
            lds_u8* Vs = (lds_u8*)(smem + 3 * TB + set * VTB);
            const int vg = tid & 7, vh = (tid >> 3) & 3, vq = tid >> 5;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // feature 4q + c: half c%2 of dword c/2 of each key, in unit (g, (4q + c) ^ g)
                const int e = c >> 1;
                const unsigned int sel = (c & 1) ? 0x07060302u : 0x05040100u;
                *(__attribute__((address_space(3))) unsigned int*)(Vs + (vg * D + ((4 * vq + c) ^ vg)) * 16 + vh * 4) =
                    __builtin_amdgcn_perm(vst[set][1][e], vst[set][0][e], sel);
            }
        }
    };
    auto issue_k = [&](int t, int ks, int i) {
        const int64_t j0 = (int64_t)t * kBN;
        const uint32_t nrec = (uint32_t)((Sk - 1 - j0) * ld2 + D * 2);   // bytes of valid rows from j0
        fill_k<D>(kbase + j0 * ld2, nrec, smem + ks * TB, wave, lane, ld2, i);
    };
    constexpr int kDmaPerWave = (64 / (1024 / (D * 2))) / kWaves;
    auto issue_k_all = [&](int t, int ks) {
#pragma unroll
        for (int i = 0; i < kDmaPerWave; ++i) issue_k(t, ks, i);
    };
    // vector memory operations each wave issues per tile: K copies, V loads
    constexpr int kVmPerTile = kDmaPerWave + KPL;

    // ---- LDS operand offsets (bytes) -------------------------------------
    // K operand of the score product, block jb, chunk kc: row 32*jb + l32,
    // logical unit 2*kc + hg.  V operand, chunk c, feature block db: unit group
    // g = 2c + hg, feature 32*db + l32.
    uint32_t kaddr[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kaddr[kc] = l32 * ROWB + (((2 * kc + hg) ^ (l32 & (UPR - 1))) * 16);
    // V operand, chunk c, feature block db: unit group g = 2c + hg, feature 32*db + l32
    uint32_t vaddr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int g = 2 * c + hg;
        if constexpr (D == 128)
            vaddr[c] = (uint32_t)(g * VGS + 16 * l32 + 16 * (l32 >> 4));
        else
            vaddr[c] = (uint32_t)(g * D + (l32 ^ g)) * 16;
    }
    constexpr int VDB = D == 128 ? 32 * 16 + 2 * 16 : 512;   // byte step between feature blocks

    // ---- per-lane state ---------------------------------------------------
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m = -INFINITY;   // reference maximum (exp2 units) of row i
    float lsum = 0.f;      // this lane half's share of the row sum
    const float c2 = a.scale_log2;

    // Loads run two tiles ahead: K through three LDS stages, V through two
    // register sets and two LDS stages.
    int t = next_live(t_beg);
    int t1 = t < n_tiles ? next_live(t + 1) : n_tiles;
    int ks = 0;   // K stage of tile t
    if (t < n_tiles) {
        issue_k_all(t, 0);
        load_v(t, std::integral_constant<int, 0>{});
        if (t1 < n_tiles) {
            issue_k_all(t1, 1);
            load_v(t1, std::integral_constant<int, 1>{});
        }
        store_v(std::integral_constant<int, 0>{});
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): every copy issued so far landed
    __syncthreads();

    // Q operands: lane holds row i, features 16*kc + 8*hg .. +7 (zero past Sq)
    bf16x8 qop[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        qop[kc] = __builtin_bit_cast(
            bf16x8, *(const lds_u32x4*)(qst + l32 * ROWB + (((2 * kc + hg) ^ (l32 & (UPR - 1))) * 16)));

    // One tile step with the V stage / register set parity P a template
    // constant.  Returns false after the last live tile.
    auto step = [&](auto parity_tag) -> bool {
        constexpr int P = decltype(parity_tag)::value;
        const int t2 = t1 < n_tiles ? next_live(t1 + 1) : n_tiles;
        const int ks2 = ks == 0 ? 2 : ks - 1;   // (ks + 2) % 3
        // Always issue the copies (of tile t when there is no t2; they land
        // in buffers nothing reads) so that every wave has exactly kVmPerTile
        // vector memory operations per step in flight.  They are issued among
        // the score instructions below, spread out so that the waves of the
        // workgroup do not all queue on the address unit at once.
        const int tl = t2 < n_tiles ? t2 : t;

        if constexpr (D != 128) {
            // few matrix instructions per tile: the loads go up front
            issue_k_all(tl, ks2);
            load_v(tl, std::integral_constant<int, P>{});
        }
        const int64_t j0 = (int64_t)t * kBN;
        bool any = wave_live, per_elem = j0 + kBN > Sk;
        if (MASKED && wave_live) {
            const int32_t j0s = t * kBN, j1s = j0s + kBN < sk32 ? j0s + kBN : sk32;
            any = meets(j0s, j1s, wa0, wa1);
            per_elem = per_elem || !inside(j0s, j1s, wf0, wf1);
        }

        // With D = 128 every wave computes every live tile (the global loads
        // sit among its score instructions); smaller D skips tiles none of the
        // wave's rows can see.
        if (D == 128 || any) {
            const lds_u8* Kl = (const lds_u8*)(smem + ks * TB);
            const lds_u8* Vl = (const lds_u8*)(smem + 3 * TB + P * VTB);

            // S^T = K Q^T: block jb, register v holds key 32*jb + 8*(v/4) + 4*hg + v%4.
            f32x16 sacc[2];
            if constexpr (D == 128) {
                // Matrix instruction r of the scores:
                // Matrix instruction r uses k-chunk r/2 of block r%2; its K operand
                // is read four instructions ahead.  The global loads for tile tl
                // are placed between the matrix instructions, one every few, and
                // scheduling barriers keep that order, so that the waves do not
                // all queue on the address unit at the top of the step.
                constexpr int NS = 2 * NKC;
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) sacc[jb][v] = 0.f;
                auto kread = [&](int r) {
                    return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(Kl + kaddr[r >> 1] + (r & 1) * 32 * ROWB));
                };
                const __amdgpu_buffer_rsrc_t vtr = v_rsrc(tl);
                bf16x8 kop[NS];
#pragma unroll
                for (int r = 0; r < 4; ++r) kop[r] = kread(r);
#pragma unroll
                for (int r = 0; r < NS; ++r) {
                    sacc[r & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[r], qop[r >> 1], sacc[r & 1], 0, 0, 0);
                    if (r + 4 < NS) kop[r + 4] = kread(r + 4);
                    constexpr int kGap = NS / kVmPerTile;
                    if (r % kGap == kGap / 2) {
                        const int m = r / kGap;
                        if (m < kDmaPerWave)
                            issue_k(tl, ks2, m);
                        else if (m < kVmPerTile)
                            load_v_part(vtr, std::integral_constant<int, P>{}, m - kDmaPerWave);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }

            } else {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) sacc[jb][v] = 0.f;
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) {
                        const bf16x8 kop =
                            __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(Kl + kaddr[kc] + jb * 32 * ROWB));
                        sacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kc], sacc[jb], 0, 0, 0);
                    }
                // keep 4 operand reads in flight ahead of the matrix instructions
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int r = 0; r < 2 * NKC - 4; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }

            if (per_elem) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int32_t j = (int32_t)j0 + 32 * jb + 8 * (v >> 2) + 4 * hg + (v & 3);
                        const bool ok = j < segk ? j < lim0 : j < lim1;
                        if (!ok) sacc[jb][v] = -INFINITY;
                    }
            }

            // Raised wave priority while this wave runs its softmax and PV
            // products, so that its vector work is issued ahead of the other
            // wave's score instructions on the same SIMD.
            __builtin_amdgcn_s_setprio(1);
            // online softmax of row i
            float mx;
            {
                // three-input maximum tree over the 32 scores: 16 instructions
                float r[11];
#pragma unroll
                for (int u = 0; u < 10; ++u) {
                    const int e0 = 3 * u, e1 = 3 * u + 1, e2 = 3 * u + 2;
                    r[u] = fmax3(sacc[e0 >> 4][e0 & 15], sacc[e1 >> 4][e1 & 15], sacc[e2 >> 4][e2 & 15]);
                }
                r[10] = __builtin_elementwise_maximum(sacc[1][14], sacc[1][15]);
                const float r0 = fmax3(r[0], r[1], r[2]), r1 = fmax3(r[3], r[4], r[5]);
                const float r2 = fmax3(r[6], r[7], r[8]), r3 = __builtin_elementwise_maximum(r[9], r[10]);
                mx = __builtin_elementwise_maximum(fmax3(r0, r1, r2), r3);
            }
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float m_new = __builtin_elementwise_maximum(m, mx * c2);
            const bool need = m_new > m + kRescaleThreshold;
            if (__any(need)) {
                // lanes that keep their maximum (possibly still -inf) scale by 1
                const float alpha = need ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
                m = need ? m_new : m;
            }
            const float m_use = m == -INFINITY ? 0.f : m;
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int jb = c >> 1, v0 = 8 * (c & 1);
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[jb][v0 + 2 * e], c2, -m_use));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[jb][v0 + 2 * e + 1], c2, -m_use));
                    ps0 += p0;
                    ps1 += p1;
                    pw[e] = pack_bf16(p0, p1);
                }
                // O^T += V^T P^T for this 16-key chunk
                const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 vop = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(Vl + vaddr[c] + db * VDB));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, oacc[db], 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            lsum += ps0 + ps1;
        }

        if (t1 < n_tiles) store_v(std::integral_constant<int, P ^ 1>{});
        // the K copy of tile t1 must have landed; the copies of this step may still run
        __builtin_amdgcn_s_waitcnt(0x0F70 | kVmPerTile);
        lds_barrier();
        ks = ks == 2 ? 0 : ks + 1;
        t = t1;
        t1 = t2;
        return t < n_tiles;
    };
    if (t < n_tiles)
        while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
        }
    // the copies the last step issued (into buffers nothing reads) land
    // before the workgroup ends and its LDS can be reused
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // ---- epilogue: normalise, write O and the natural-log LSE -----------
    // (acc, mref, ls): O accumulators, reference maximum, half-row sum
    // With a.acc the call continues a Ring pass: (o, lse) hold on entry the
    // result over the keys seen so far (lse = -inf: none), and this block's
    // result is merged in -- weights e^(lse_n - lse) as in the LSE merge --
    // so that they hold on return the result over all keys seen.
    // (acc, mref, ls): O accumulators, reference maximum, half-row sum
    auto write_out = [&](const f32x16 (&acc)[NDB], float mref, float ls) {
        float lt;
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ls), __float_as_uint(ls), false, false);
            lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        // log2-domain LSE of this block, and with a.acc the weights of the
        // previous result (wp) and of this block (wb) and the merged LSE
        const float lb2 = lt > 0.f ? mref + __log2f(lt) : -INFINITY;
        float wp = 0.f, wb = 1.f, lse_out2 = lb2;
        if (a.acc) {
            const float lp2 = i < Sq ? a.lse[(b * Sq + i) * H + hh] * kLog2e : -INFINITY;
            const float mm = __builtin_elementwise_maximum(lp2, lb2);
            if (mm == -INFINITY) {
                wp = 0.f;
                wb = 0.f;
                lse_out2 = -INFINITY;
            } else {
                const float ep = __builtin_amdgcn_exp2f(lp2 - mm), eb = __builtin_amdgcn_exp2f(lb2 - mm);
                const float sum = ep + eb;
                wp = ep / sum;
                wb = eb / sum;
                lse_out2 = mm + __log2f(sum);
            }
        }
        if constexpr (OUT_BF16) {
            // The wave's 32 x D output tile goes through LDS (free once every
            // wave has left the main loop and the last copies have landed) so
            // that each global store writes whole rows: 4 rows of 256 bytes
            // per instruction for D = 128, instead of 16-byte pieces of 32 rows.
            constexpr int RS = D * 2 + 16;        // LDS row stride (bytes)
            constexpr int WS = 32 * RS + 32 * 8;  // per wave: the tile, then (wp, wb) of each row
            constexpr int UR = D * 2 / 16;        // 16-byte units per row
            constexpr int RPI = 64 / UR;          // rows per store instruction
            lds_barrier();
            lds_u8* R = (lds_u8*)smem + wave * WS;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = 32 * db + 8 * g + 4 * hg;   // 4 consecutive features
                    const u32x2 w{pack_bf16(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                                  pack_bf16(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
                    *(__attribute__((address_space(3))) u32x2*)(R + l32 * RS + d0 * 2) = w;
                }
            if (a.acc && hg == 0) *(__attribute__((address_space(3))) f32x2*)(R + 32 * RS + l32 * 8) = f32x2{wp, wb};
            const int rr = lane / UR, cu = lane % UR;
            constexpr int NK = 32 / RPI;
            auto dst_of = [&](int k) {
                const int64_t row = q0 + 32 * wave + RPI * k + rr;
                return reinterpret_cast<u32x4*>(static_cast<unsigned char*>(a.o) + ((b * Sq + row) * H + hh) * D * 2 +
                                                cu * 16);
            };
            auto row_ok = [&](int k) { return q0 + 32 * wave + RPI * k + rr < Sq; };
            // the previous result's rows, all loaded before any store (stores
            // to o could alias later loads, which would serialise each pair)
            u32x4 pv[NK];
            if (a.acc) {
#pragma unroll
                for (int k = 0; k < NK; ++k) pv[k] = row_ok(k) ? *dst_of(k) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int r = RPI * k + rr;
                u32x4 w = *(const lds_u32x4*)(R + r * RS + cu * 16);
                if (a.acc) {
                    const f32x2 wr = *(const __attribute__((address_space(3))) f32x2*)(R + 32 * RS + r * 8);
                    // a previous result of weight 0 (lse = -inf) is not used
                    const bool use = wr[0] != 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = fmaf(wr[0], use ? bf16_lo(pv[k][e]) : 0.f, wr[1] * bf16_lo(w[e]));
                        const float hi = fmaf(wr[0], use ? bf16_hi(pv[k][e]) : 0.f, wr[1] * bf16_hi(w[e]));
                        w[e] = pack_bf16(lo, hi);
                    }
                }
                // Plain stores: non-temporal ones make this kernel ~1 us faster but
                // the next kernel (the inverse gather) then misses the caches;
                // on the whole step plain stores measured ~0.5 % faster.
                if (row_ok(k)) *dst_of(k) = w;
            }
        } else {
            if (i < Sq) {
                const int64_t orow = ((b * Sq + i) * H + hh) * D;
                const float sb = wb * inv;
                auto dst_of = [&](int db, int g) {
                    return reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + 32 * db + 8 * g + 4 * hg);
                };
                // previous result loaded before any store (see above); weight 0: not read
                f32x4 pv[NDB][4];
                const bool use = a.acc && wp != 0.f;
                if (use) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int g = 0; g < 4; ++g) pv[db][g] = *dst_of(db, g);
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        f32x4 x{acc[db][4 * g] * sb, acc[db][4 * g + 1] * sb, acc[db][4 * g + 2] * sb,
                                acc[db][4 * g + 3] * sb};
                        if (use) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = fmaf(wp, pv[db][g][e], x[e]);
                        }
                        *dst_of(db, g) = x;
                    }
            }
        }
        if (hg == 0 && i < Sq) a.lse[(b * Sq + i) * H + hh] = lse_out2 * kLn2;
    };

    if (SPLIT && np > 1) {
        // Every piece stores its partial state (O accumulators, reference
        // maximum, half-row sum, as the registers hold them) in its slot and
        // counts in; the last piece of the unit to arrive combines all slots
        // in piece order -- the same loads and arithmetic whichever piece it
        // is, so the result does not depend on timing -- resets the counter
        // and writes the output.  Pieces may run on different XCDs, whose L2
        // caches are not coherent with each other for ordinary accesses: the
        // state moves with device-scope loads and stores (cache policy sc1, as
        // relaxed device-scope atomic loads and stores are), coherent across
        // XCDs by themselves, so no cache-wide write-back or invalidate is
        // needed, only the completion of this wave's stores before its count.
        unsigned char* wsb = static_cast<unsigned char*>(a.ws);
        const uint32_t su = unit - (uint32_t)a.n_whole;   // index among the split units
        const int64_t n_split = (int64_t)(gridDim.x - (uint32_t)a.n_whole) / np;
        int32_t* cnt = reinterpret_cast<int32_t*>(wsb + n_split * np * kSplitSlotBytes) + su;
        // The unit's np slots; in slot q, 16-byte quad r of lane tid sits at
        // ((q * kSplitQuads + r) * kSplitLanes + tid) * 16: quads below 4 NDB
        // are the O accumulators, quad 4 NDB holds the maximum and half-row sum.
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            wsb + (int64_t)su * np * kSplitSlotBytes, (short)0, (int)(np * kSplitSlotBytes), 0x00020000);
        constexpr int kDev = 16;   // cache policy sc1: device-scope access
        const int voff = tid * 16;
        auto qoff = [&](int q, int r) { return (q * (int)kSplitQuads + r) * (int)(kSplitLanes * 16); };
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x4 w{__float_as_uint(oacc[db][4 * g]), __float_as_uint(oacc[db][4 * g + 1]),
                              __float_as_uint(oacc[db][4 * g + 2]), __float_as_uint(oacc[db][4 * g + 3])};
                store_slot_b128(w, wr, voff, qoff(piece, 4 * db + g));
            }
        {
            const u32x4 w{__float_as_uint(m), __float_as_uint(lsum), 0u, 0u};
            store_slot_b128(w, wr, voff, qoff(piece, 4 * NDB));
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the stores above are complete
        __syncthreads();
        volatile int* flag = reinterpret_cast<volatile int*>(smem);
        if (tid == 0) *flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (*flag != np - 1) return;   // pieces of this unit are still running; the last one finishes it
        // The combine has registers of its own (the loop's accumulators are
        // dead once stored) and writes the output itself.
        auto ldq = [&](int q, int r) { return __builtin_amdgcn_raw_buffer_load_b128(wr, voff, qoff(q, r), kDev); };
        f32x16 cacc[NDB];
        float cm, cl;
        {
            const u32x4 ml = ldq(0, 4 * NDB);
            cm = __uint_as_float(ml[0]);
            cl = __uint_as_float(ml[1]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x4 w = ldq(0, 4 * db + g);
#pragma unroll
                for (int e = 0; e < 4; ++e) cacc[db][4 * g + e] = __uint_as_float(w[e]);
            }
        for (int q = 1; q < np; ++q) {
            const u32x4 ml = ldq(q, 4 * NDB);
            const float mq = __uint_as_float(ml[0]), lq = __uint_as_float(ml[1]);
            const float mm = __builtin_elementwise_maximum(cm, mq);
            const float w0 = cm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(cm - mm);
            const float w1 = mq == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mq - mm);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x4 w = ldq(q, 4 * db + g);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        cacc[db][4 * g + e] = fmaf(__uint_as_float(w[e]), w1, cacc[db][4 * g + e] * w0);
                }
            cl = fmaf(lq, w1, cl * w0);
            cm = mm;
        }
        if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        write_out(cacc, cm, cl);
        return;
    }
    write_out(oacc, m, lsum);
}


template <int D, bool OB>
static hipError_t launch_d(const AttnArgs& a, dim3 grid, hipStream_t s)
{
    const dim3 block(64 * kWaves);
    if (a.masked) return launch_kernel(attn_bf16_kernel<D, true, OB, false>, grid, block, 0, s, a);
    if (a.split_p > 1) return launch_kernel(attn_bf16_kernel<D, false, OB, true>, grid, block, 0, s, a);
    return launch_kernel(attn_bf16_kernel<D, false, OB, false>, grid, block, 0, s, a);
}

int64_t attn_bf16_units(int64_t B, int64_t H, int64_t Sq) { return ((Sq + kBM - 1) / kBM) * H * B; }

// One workgroup runs on each compute unit at a time, so U units of N key
// tiles on C compute units take ceil(U / C) rounds of N tile times, the last
// one partial when C does not divide U.  The plan keeps f = floor(U / C)
// rounds' worth of units whole and cuts each of the other r = U - f C units
// into p pieces, r p <= C, which run first: f N + N / p + e tile times, with
// e ~ 1.5 tile times for a piece's start-up and combine when the combine
// overlaps whole units' work (f >= 1) and ~ 3 when it does not.  Picks the
// best p <= 8 (pieces of at least 4 tiles), and no split unless it saves at
// least 8 %.
SplitPlan plan_split(int64_t n_units, int64_t n_tiles, int n_cu)
{
    SplitPlan plan;
    if (n_cu <= 0 || n_units <= 0 || n_tiles < 8) return plan;
    const int64_t f = n_units / n_cu, r = n_units - f * n_cu;
    if (r == 0) return plan;
    const double e = f >= 1 ? 1.5 : 3.0;
    const double base = (double)(f + 1) * (double)n_tiles;
    double best = base;
    for (int p = 2; p <= 8 && n_tiles / p >= 4 && r * p <= n_cu; ++p) {
        const double t = (double)f * n_tiles + (double)n_tiles / p + e;
        if (t < best) {
            best = t;
            plan.p = p;
        }
    }
    if (!(best < 0.92 * base)) plan.p = 1;
    plan.n_whole = plan.p > 1 ? f * n_cu : 0;
    return plan;
}

static bool p32_on()
{
    static const bool on = [] {
        const char* e = getenv("UAA_ATTN_P32");
        return !(e && e[0] == '0');
    }();
    return on;
}

static bool p32_takes(int D, const AttnArgs& a)
{
    return D == 128 && attn_p32_fits(a.Sk, a.row_heads) && p32_on();
}

// The arguments with the general kernel's q-tile count set and a key split
// kept only where it applies (a plan made for the pipelined kernel runs
// only there); false when there is no work.
static bool general_args(int D, const AttnArgs& a0, AttnArgs& a)
{
    a = a0;
    a.n_qtiles = (int32_t)((a.Sq + kBM - 1) / kBM);
    const int64_t units = (int64_t)a.n_qtiles * a.H * a.B;
    if (units <= 0) return false;
    if (a.masked || a.ws == nullptr || a.split_p <= 1 || a.n_whole < 0 || a.n_whole >= units ||
        (a.split_p32 != 0 && !p32_takes(D, a))) {
        a.split_p = 1;
        a.n_whole = 0;
        a.split_p32 = 0;
    }
    return true;
}

// 0: the general kernel; 1: the pipelined kernel; 2: its DIAG form (units
// on a mask diagonal); 3: its key split
static int use_p32(int D, const AttnArgs& a)
{
    if (!p32_takes(D, a)) return 0;
    if (a.split_p > 1) return a.split_p32 ? 3 : 0;
    if (attn_p32_mask_ok(a)) return 1;
    return attn_p32_diag_ok(a) ? 2 : 0;
}

int attn_bf16_kernel_choice(int D, const AttnArgs& a0)
{
    AttnArgs a;
    if (!general_args(D, a0, a)) return USP_KERNEL_NONE;
    const int p = use_p32(D, a);
    if (p == 1) return USP_KERNEL_PIPELINED;
    if (p == 2) return USP_KERNEL_PIPELINED_DIAG;
    if (p == 3) return USP_KERNEL_PIPELINED_SPLIT;
    if (a.masked) return USP_KERNEL_GENERAL_MASKED;
    return a.split_p > 1 ? USP_KERNEL_GENERAL_SPLIT : USP_KERNEL_GENERAL;
}

hipError_t launch_attn_bf16(int D, int o_dtype, const AttnArgs& a0, hipStream_t s)
{
    AttnArgs a;
    if (!general_args(D, a0, a)) return hipSuccess;
    const int64_t units = (int64_t)a.n_qtiles * a.H * a.B;
    const int64_t blocks = a.split_p > 1 ? a.n_whole + (units - a.n_whole) * a.split_p : units;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (const int p = use_p32(D, a)) return launch_attn_p32(o_dtype, p, a, s);
    const dim3 grid((unsigned)blocks);
    const bool ob = o_dtype == UAA_BF16;
    if (D == 128) return ob ? launch_d<128, true>(a, grid, s) : launch_d<128, false>(a, grid, s);
    if (D == 64) return ob ? launch_d<64, true>(a, grid, s) : launch_d<64, false>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace uaa
