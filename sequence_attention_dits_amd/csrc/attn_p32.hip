// attn_p32.hip -- blockwise attention forward with LSE, bf16 inputs, D = 128,
// every key allowed, software-pipelined: the variant the library launches
// for that case.
//
// What it computes is what attn_bf16.hip computes for the unmasked case:
// for every query row the pair (out, lse) of one Ring step ("Add Unified
// Sequence Parallel attention", diffusers PR #12693, review thread; "Context
// parallelism" docs, "Ring Attention"), optionally merged into the running
// (out, lse) of the pass.
//
// Layout as in attn_bf16.hip: a workgroup owns 256 query rows of one
// (batch, head), 8 wavefronts of 32 rows, two per SIMD (wavefront w on SIMD
// w % 4).  What differs is the schedule.  A wavefront's tile step is two
// phases: M(t), matrix instructions only -- the scores of tile t+1 and
// O += V_t^T P_t, interleaved, with the step's K/V copies issued among them
// -- and V(t), vector instructions only: the row maximum and softmax of tile
// t+1.  Wavefronts 0..3 run M while 4..7 run V and the other way round, a
// workgroup barrier between half-steps, so on every SIMD one wavefront's
// matrix instructions run beside the other's vector instructions (the
// other pairing, both wavefronts of a SIMD in the same phase, measured 22%
// slower).  What bounds it, measured by timing copies of the kernel with one
// part removed: the M phase.  Each of its matrix instructions consumes a
// 1 KB LDS operand read (a 16 KB K tile and a 16 KB V tile per wavefront
// and tile), and a SIMD with one wavefront issuing such instructions keeps
// its matrix core only ~75-84% busy; without the LDS reads the softmax-free
// kernel takes a quarter less time, without the softmax only an eighth
// less.  An earlier schedule that interleaved both kinds of work inside
// each wavefront ran 1% slower; 64-row wavefronts, a role split of the two
// wavefronts of a SIMD and early operand reads all ran 5-11% slower.
// What the pipelining takes, learnt the hard way:
//  * the matrix instructions are inline assembly with their registers
//    fixed in VGPRs (scores, O and Q; the vector code reads O in place when
//    it rescales); the compiler does not see them as matrix instructions,
//    so vector code touching their results sits behind explicit wait states
//    (fences below);
//  * the loop body is three M/V pairs (one per LDS stage), branch-free
//    inside, with a uniform exit after each pair, so a unit runs exactly its
//    tile count; a branch inside a phase made the compiler keep a second copy
//    of the O accumulators;
//  * the operand addresses pass through an empty asm at the start of each M
//    phase; otherwise the compiler keeps stage-offset variants of them in
//    registers across the loop and spills;
//  * the softmax results are pinned with an empty asm before the branch
//    that follows them; otherwise IR-level sinking moves the softmax below
//    the branch;
//  * K and V tiles are copied global -> LDS by buffer loads that write LDS,
//    issued as inline assembly: as builtins, the compiler would make the next
//    LDS reads wait for every copy in flight (vmcnt(0)), since it cannot tell
//    the stage being read from the stage being filled.  Three stages each,
//    copies two steps ahead, waited for explicitly before a barrier.
// Measured and not kept: a deeper operand prefetch (3, 4, 6 matrix
// instructions ahead: no change) and a row sum over the bf16 P values (the
// LSE then carries the rounding of the weights, beyond its tolerance).
// V is stored row-major with the 16-byte units of a row swizzled, and the PV
// operands are read with ds_read_b64_tr_b16 (two give a lane the 8 keys of
// one feature in the order the score registers hold them).  Row maximum
// raised lazily (2^8 threshold), exp2 with the scale folded in, natural-log
// LSE at the end.
#include "attn_common.h"

#include <algorithm>
#include <type_traits>

namespace uaa {

typedef __bf16 p_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 p_bf16x2 __attribute__((ext_vector_type(2)));
typedef float p_f32x16 __attribute__((ext_vector_type(16)));
typedef float p_f32x4 __attribute__((ext_vector_type(4)));
typedef float p_f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int p_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int p_u32x2 __attribute__((ext_vector_type(2)));
typedef short p_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char p_lds_u8;
typedef __attribute__((address_space(3))) p_u32x4 p_lds_u32x4;
typedef __attribute__((address_space(3))) p_i16x4 p_lds_i16x4;

constexpr int kPWaves = 8;
constexpr int kPBM = kPWaves * 32;    // query rows per workgroup
constexpr int kPBN = 64;              // keys per tile
constexpr int kPD = 128;
constexpr int kPRowB = 2 * kPD;       // bytes per row
constexpr int kPTB = kPBN * kPRowB;   // bytes of one K or V tile
constexpr float kPLn2 = 0.69314718055994530942f;
constexpr float kPLog2e = 1.44269504088896340736f;
constexpr float kPRescale = 8.0f;     // lazy rescale threshold, log2 units

__device__ __forceinline__ unsigned int p_pack(float lo, float hi)
{
    return __builtin_bit_cast(unsigned int, __builtin_convertvector(p_f32x2{lo, hi}, p_bf16x2));
}
__device__ __forceinline__ float p_lo(unsigned int x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float p_hi(unsigned int x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float p_max3(float a, float b, float c)
{
    return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// Physical 16-byte unit of logical unit u of tile row r: u ^ swz(r), swz
// swapping the two 2-bit halves of r % 16.  Row reads (16 consecutive rows,
// one unit) and the transposing reads (4 rows x 4 units per 16 lanes) then
// fall on distinct banks.
__device__ __forceinline__ int p_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Raw buffer descriptor (stride 0) over nrec bytes from base; reads from
// nrec on return zero.
typedef unsigned int p_rsrc __attribute__((ext_vector_type(4)));
// The values are uniform by construction; readfirstlane keeps them in
// scalar registers where the compiler cannot prove it.
__device__ __forceinline__ p_rsrc p_make_rsrc(const void* base, uint32_t nrec)
{
    const uint64_t p = (uint64_t)base;
    return p_rsrc{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu)),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)nrec), 0x00020000u};
}

// One 16-byte-per-lane copy global -> LDS (buffer_load ... lds): lane s
// writes bytes [lds + 16 s, lds + 16 s + 16), reading byte voff of r.
__device__ __forceinline__ void p_dma(const p_rsrc& r, uint32_t voff, uint32_t lds)
{
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass has no SGPR operand constraint
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds))
                 : "memory", "m0");
#endif
}

__device__ __forceinline__ void p_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// S = K x Q [+ S];  O += V x P  (every operand in VGPRs)
__device__ __forceinline__ void p_mma_s0(p_f32x16& d, const p_bf16x8& k, const p_bf16x8& q)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "v"(q));
}
__device__ __forceinline__ void p_mma_s(p_f32x16& d, const p_bf16x8& k, const p_bf16x8& q)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "v"(q));
}
__device__ __forceinline__ void p_mma_o(p_f32x16& d, const p_bf16x8& v, const p_u32x4& p)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(v), "v"(p));
}
// wait states before vector code touches matrix results: 16 for the scores
// (the compiler itself places 12 between a 32x32x16 bf16 matrix instruction
// and a vector read of its result), 32 for the O accumulators
__device__ __forceinline__ void p_fence_s(p_f32x16 (&s)[2])
{
    asm volatile("s_nop 15" : "+v"(s[0]), "+v"(s[1]));
}
__device__ __forceinline__ void p_fence_o(p_f32x16 (&o)[4])
{
    asm volatile("s_nop 15\n\ts_nop 15" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
}
// the O accumulators are complete here (both sides of a branch that
// rescales them leave them in the same registers)
__device__ __forceinline__ void p_pin_o(p_f32x16 (&o)[4])
{
    asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
}
// values complete at this point (keeps them from being sunk past a branch)
__device__ __forceinline__ void p_pin_p(p_u32x4 (&p)[4])
{
    asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]));
}
__device__ __forceinline__ void p_pin_f(float& x) { asm volatile("" : "+v"(x)); }

// DIAG: a masked call whose key map is one increasing piece, so that the
// keys each query row may see are a prefix of the block (causal by
// position: basic and stripe layouts, a zigzag block of one chunk).  Each
// unit then runs only its live key tiles -- those before the last allowed
// key of its last row -- and the rows of a tile on a unit's diagonal are
// masked one by one (each lane's row has its own allowed-key count); units
// run longest first.  Without DIAG every unit runs every key tile (a masked
// call only when each unit sees every key of the block or none).
// Piece form (SPLIT): the keys of some units are cut into pieces, each run
// by its own workgroup (units [0, n_whole) run whole, one workgroup each;
// each of the others in split_p pieces of about equal length).  Piece
// workgroups come first in the grid, piece index major, so they are
// dispatched first and the whole units fill the compute units as they free
// up.  A piece stores its normalised O (bf16) and its LSE in a slot of the
// workspace and counts in; the last piece of a unit to finish combines the
// unit's slots in piece order and writes the result.  The slot of piece k
// of split unit su is su * split_p + k; then one int32 arrival counter per
// split unit.  A slot holds the 256 rows' O as the lanes' registers hold it
// (16-byte quad j of lane tid at (512 j + tid) * 16) and the rows' LSE
// (log2 units) at 64 KiB.
template <bool OUT_BF16, bool DIAG, bool SPLIT>
__global__ __launch_bounds__(64 * kPWaves, 2) void attn_p32_kernel(const AttnArgs a)
{
    // V stages, K stages, Q staging: every operand read is a per-lane
    // register plus an immediate (stage, chunk, block) below 64 KB
    constexpr int OFF_V = 0, OFF_K = 3 * kPTB, OFF_Q = 6 * kPTB;
    constexpr int SMEM = OFF_Q + kPBM * kPRowB;   // 160 KB
    __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
    p_lds_u8* const L = (p_lds_u8*)smem;

    int64_t qt, hh, b;
    const int32_t nt = (int32_t)((a.Sk + kPBN - 1) / kPBN);
    int32_t tb = 0, te = nt;       // this workgroup's key tiles
    int32_t piece = 0, su = -1;    // SPLIT: piece index and split-unit index (-1: a whole unit)
    if constexpr (SPLIT) {
        const uint32_t L = blockIdx.x, nw = (uint32_t)a.n_whole, np = (uint32_t)a.split_p;
        const uint32_t n_split = (uint32_t)a.n_qtiles * (uint32_t)a.H * (uint32_t)a.B - nw;
        const uint32_t npw = n_split * np;   // piece workgroups
        if (L < npw) {
            // piece-major in dispatch order (every XCD gets its share of
            // each piece index); within a piece index, each XCD a run of units
            piece = (int32_t)(L / n_split);
            su = (int32_t)xcd_logical(L - (uint32_t)piece * n_split, n_split);
            unit_coords(a, nw + (uint32_t)su, qt, hh, b);
            tb = (int32_t)((int64_t)piece * nt / np);
            te = (int32_t)((int64_t)(piece + 1) * nt / np);
        } else {
            unit_coords(a, xcd_logical(L - npw, gridDim.x - npw), qt, hh, b);
        }
    } else if (DIAG && gridDim.x % 8u == 0u && (gridDim.x / 8u) % (uint32_t)a.n_qtiles == 0u) {
        // every XCD holds whole heads: each XCD's workgroups (blockIdx =
        // 8 j + x on XCD x) take its heads' q tiles last-first with the heads
        // interleaved -- later rows see at least as many keys under every
        // mask kind, so the longest units are dispatched first
        const uint32_t nq = (uint32_t)a.n_qtiles, per = gridDim.x / 8u, hpx = per / nq;
        const uint32_t x = blockIdx.x % 8u, j = blockIdx.x / 8u;
        unit_coords(a, x * per + (j % hpx) * nq + (nq - 1u - j / hpx), qt, hh, b);
    } else {
        decode_tile(a, qt, hh, b);
        if (DIAG) qt = a.n_qtiles - 1 - qt;
    }
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hg = lane >> 5;
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const int64_t RH = a.row_heads, h_in = a.head0 + hh;
    const uint32_t ld2 = (uint32_t)(RH * kPD * 2);
    const int64_t r0 = qt * kPBM + 32 * wave;     // first row of this wave
    const int64_t i = r0 + l32;                    // this lane's row
    const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + ((b * Sk) * RH + h_in) * kPD * 2;
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + ((b * Sk) * RH + h_in) * kPD * 2;
    // key tiles this unit runs, and with DIAG this lane's row's allowed keys
    // (a prefix of the block; rows past Sq are never stored and see all)
    int n = te - tb;
    int32_t kcnt = (int32_t)Sk;
    if constexpr (DIAG) {
        const int64_t t0 = qt * kPBM, t1 = t0 + kPBM < Sq ? t0 + kPBM : Sq;
        int64_t qlo, qhi;
        pos_range(a.qmap, t0, t1, qlo, qhi);
        const int64_t live = allowed_prefix(a.kmap.base0, a.kmap.stride, qhi, Sk);
        n = (int)((live + kPBN - 1) / kPBN);
        if (i < Sq) kcnt = (int32_t)allowed_prefix(a.kmap.base0, a.kmap.stride, pos_of(a.qmap, i), Sk);
    }

    // One descriptor per tensor over this head's keys (rows from Sk on read
    // as zero; the launcher checks that the range fits 32 bits) and this
    // lane's byte offset for each of the wave's 2 copy instructions per tile
    // (copy c moves tile rows 4 (8 c + wave) .. +3); tile t adds t * 64 rows.
    const uint32_t nrec_k = Sk > 0 ? (uint32_t)((Sk - 1) * ld2 + kPD * 2) : 0u;
    const p_rsrc krs = p_make_rsrc(kbase, nrec_k);
    const p_rsrc vrs = p_make_rsrc(vbase, nrec_k);
    uint32_t coff[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int row = 4 * (kPWaves * c + wave) + (lane >> 4);
        coff[c] = (uint32_t)row * ld2 + (uint32_t)(((lane & 15) ^ p_swz(row)) << 4);
    }
    const uint32_t tile_bytes = (uint32_t)kPBN * ld2;
    auto copy_tile = [&](const p_rsrc& rs, int off, int t, int s, int c) {
        p_dma(rs, coff[c] + (uint32_t)(tb + t) * tile_bytes,
              (uint32_t)(uintptr_t)(L + off + s * kPTB + (kPWaves * c + wave) * 1024));
    };

    // A masked call runs here only when the rows of every unit see either
    // every key of the block or none (the block lies wholly in their past or
    // their future).  A unit that sees none gives O = 0, LSE = -inf, and
    // continuing a Ring pass leaves (o, lse) as they are.
    if (a.masked) {
        const int64_t t0 = qt * kPBM, t1 = t0 + kPBM < Sq ? t0 + kPBM : Sq;
        int64_t qlo, qhi, klo, khi;
        pos_range(a.qmap, t0, t1, qlo, qhi);
        pos_range(a.kmap, 0, Sk, klo, khi);
        if (klo > qhi || (DIAG && n == 0)) {
            if (!a.acc) {
                constexpr int C = (OUT_BF16 ? 2 : 4) * kPD / 16;   // 16-byte pieces per output row
                for (int j = lane; j < 32 * C; j += 64) {
                    const int64_t row = r0 + j / C;
                    if (row < Sq)
                        *reinterpret_cast<p_u32x4*>(static_cast<unsigned char*>(a.o) +
                                                    ((b * Sq + row) * H + hh) * (C * 16) + (j % C) * 16) =
                            p_u32x4{0u, 0u, 0u, 0u};
                }
                if (hg == 0 && i < Sq) a.lse[(b * Sq + i) * H + hh] = -INFINITY;
            }
            return;
        }
    }

    // ---- prologue: Q (this wave's 32 rows), K0..K2, V0..V1 ----------------
    if (n > 0) {
        // rows [lo, hi) of the wave's 32 (all: every row, the rest reading as
        // zero) from base = row r0 + lo, nrec bytes of it valid
        auto copy_q = [&](const unsigned char* base, uint32_t nrec, int lo, int hi, bool all) {
            const p_rsrc qr = p_make_rsrc(base, nrec);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = 4 * j + (lane >> 4);
                if (all || (row >= lo && row < hi))
                    p_dma(qr, (uint32_t)(row - lo) * ld2 + (uint32_t)(((lane & 15) ^ p_swz(row)) << 4),
                          (uint32_t)(uintptr_t)(L + OFF_Q + wave * 32 * kPRowB + j * 1024));
            }
        };
        if (a.n_qsh == 0) {
            const unsigned char* qbase = static_cast<const unsigned char*>(a.q) + ((b * Sq) * RH + h_in) * kPD * 2;
            const uint32_t nrec = Sq > r0 ? (uint32_t)((Sq - 1 - r0) * ld2 + kPD * 2) : 0u;
            copy_q(qbase + (Sq > r0 ? r0 : 0) * ld2, nrec, 0, 32, true);
        } else {
            // queries gathered from the token shards: one pass per shard the
            // wave's rows touch (two only when a shard length is not a
            // multiple of 32), rows past Sq read as zero
            const int64_t r_end = Sq < r0 + 32 ? Sq : r0 + 32;
            if (r_end < r0 + 32)
                copy_q(static_cast<const unsigned char*>(a.k), 0u, (int)(r_end > r0 ? r_end - r0 : 0), 32, false);
            int p = 0;
            for (int64_t rs = r0; rs < r_end;) {
                while (a.q_row0[p + 1] <= rs) ++p;
                const int64_t sp0 = a.q_row0[p], sp = a.q_row0[p + 1] - sp0;
                const int64_t re = a.q_row0[p + 1] < r_end ? a.q_row0[p + 1] : r_end;
                const unsigned char* sbase = static_cast<const unsigned char*>(a.q_sh[p]) +
                                             ((b * sp + (rs - sp0)) * RH + h_in) * kPD * 2;
                copy_q(sbase, (uint32_t)((re - rs - 1) * ld2 + kPD * 2), (int)(rs - r0), (int)(re - r0),
                       rs == r0 && re == r0 + 32);
                rs = re;
            }
        }
        // K0, K1, V0, K2, V1 in that order (2 copies each per wave), so that
        // the first scores wait only for Q and K0 and step 0 only for K1 and
        // V0 (copy completions count in order); stages past the last tile
        // repeat it: the V a fully masked step multiplies by zero must be
        // finite
        const int t1 = n > 1 ? 1 : 0, t2 = n > 2 ? 2 : n - 1;
#pragma unroll
        for (int c = 0; c < 2; ++c) copy_tile(krs, OFF_K, 0, 0, c);
#pragma unroll
        for (int c = 0; c < 2; ++c) copy_tile(krs, OFF_K, t1, 1, c);
#pragma unroll
        for (int c = 0; c < 2; ++c) copy_tile(vrs, OFF_V, 0, 0, c);
#pragma unroll
        for (int c = 0; c < 2; ++c) copy_tile(krs, OFF_K, t2, 2, c);
#pragma unroll
        for (int c = 0; c < 2; ++c) copy_tile(vrs, OFF_V, t1, 1, c);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70 | 8);   // vmcnt(8): Q and K0 have landed (K1, V0, K2, V1 may still run)
    __syncthreads();

    // ---- operand addressing ----------------------------------------------
    // Row read of logical unit 2 kc + hg of row r: byte r * 256 +
    // ((kc << 5) ^ ((hg ^ swz(r)) << 4)); K rows 32 jb + l32 (swz(l32)).
    const int kx = (hg ^ p_swz(l32)) << 4;
    int kaddr[8];   // + ks * tile + jb * 32 rows
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) kaddr[kc] = OFF_K + l32 * kPRowB + ((kc << 5) ^ kx);
    // Transposing V read k (0, 1): this lane as source lane (g, e, ah) =
    // (lane / 16, lane / 4 % 4, lane % 4) addresses keys 16 c + 4 (g / 2) + e
    // + 8 k at features 32 db + 16 (g % 2) + 4 ah; the result lane (feature
    // 32 db + l32, half hg) holds keys 16 c + 4 hg + {0..3, 8..11}.
    int vaddr[2][4];   // + vs * tile + c * 16 rows
    {
        const int g = lane >> 4, e = (lane >> 2) & 3, ah = lane & 3;
        const int w = 2 * (g & 1) + (ah >> 1);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = 4 * (g >> 1) + e + 8 * k;
#pragma unroll
            for (int db = 0; db < 4; ++db)
                vaddr[k][db] = OFF_V + r * kPRowB + 8 * (ah & 1) + ((db << 6) ^ ((w ^ p_swz(r)) << 4));
        }
    }
    auto vread = [&](int vs, int c, int db) {
        const p_i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (p_lds_i16x4*)(L + vaddr[0][db] + (vs * kPTB + c * 16 * kPRowB)));
        const p_i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (p_lds_i16x4*)(L + vaddr[1][db] + (vs * kPTB + c * 16 * kPRowB)));
        return __builtin_bit_cast(p_bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto kread = [&](int ks, int kc, int jb) {
        return __builtin_bit_cast(p_bf16x8, *(const p_lds_u32x4*)(L + kaddr[kc] + (ks * kPTB + jb * 32 * kPRowB)));
    };

    // Q operands: lane holds row l32 of the wave, features 16 kc + 8 hg .. +7
    p_bf16x8 qop[8];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
        qop[kc] = __builtin_bit_cast(
            p_bf16x8, *(const p_lds_u32x4*)(L + OFF_Q + wave * 32 * kPRowB + l32 * kPRowB + ((kc << 5) ^ kx)));

    const float c2 = a.scale_log2;
    p_f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    p_pin_o(oacc);
    float m = -INFINITY;    // reference maximum (exp2 units) of this lane's row
    float lsum = 0.f;       // this lane half's share of the row sum
    p_f32x16 sacc[1][2];    // [0][jb]: scores S^T of a tile; register v of
                            // block jb holds key 32 jb + 8 (v / 4) + 4 hg + v % 4

    // Keys at or past lim of a tile -> -inf (the ragged end, read as zeros;
    // tiles past the end: lim = 0).  Key 32 jb + 8 (v / 4) + 4 hg + v % 4 is
    // dead iff its constant part reaches lim - 4 hg.
    auto mask_keys = [&](p_f32x16 (&s)[2], int lim) {
        p_fence_s(s);
        const int ll = lim - 4 * hg;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (32 * jb + 8 * (v >> 2) + (v & 3) >= ll) s[jb][v] = -INFINITY;
    };
    // keys of tile t this lane's row may see (a prefix of the tile): the
    // ragged end of the block, and with DIAG the row's own allowed count
    auto key_lim = [&](int t) {
        if (SPLIT && t >= n) return 0;   // past the piece
        const int64_t r = (DIAG ? (int64_t)kcnt : Sk) - (int64_t)(tb + t) * kPBN;
        return r <= 0 ? 0 : (r >= kPBN ? kPBN : (int)r);
    };
    // some lane of the wave has a masked key in tile t (uniform)
    auto tile_masked = [&](int lim) {
        if constexpr (DIAG) return __builtin_amdgcn_ballot_w64(lim < kPBN) != 0;
        return lim < kPBN;
    };
    // Row maximum as 16 single instructions: ten three-way maxima of the
    // lane's 32 scores, one two-way, then the tree.
    float rm[11], ra[4], mx = -INFINITY;
    auto max_op = [&](const p_f32x16 (&s)[2], int j) {
        if (j < 10) {
            const int e0 = 3 * j, e1 = 3 * j + 1, e2 = 3 * j + 2;
            rm[j] = p_max3(s[e0 >> 4][e0 & 15], s[e1 >> 4][e1 & 15], s[e2 >> 4][e2 & 15]);
        } else if (j == 10) {
            rm[10] = __builtin_elementwise_maximum(s[1][14], s[1][15]);
        } else if (j < 14) {
            const int u = 3 * (j - 11);
            ra[j - 11] = p_max3(rm[u], rm[u + 1], rm[u + 2]);
        } else if (j == 14) {
            ra[3] = __builtin_elementwise_maximum(rm[9], rm[10]);
        } else {
            mx = __builtin_elementwise_maximum(p_max3(ra[0], ra[1], ra[2]), ra[3]);
        }
    };
    // both halves of the row; the reference maximum is raised (O and the sum
    // rescaled) when the tile's maximum exceeds it by more than the threshold
    auto finish_max = [&]() {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        const float t = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float mn = __builtin_elementwise_maximum(m, t * c2);
        const bool need = mn > m + kPRescale;
        if (__any(need)) {
            p_fence_o(oacc);
            const float alpha = need ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
            m = need ? mn : m;
            p_pin_o(oacc);
        }
    };
    // softmax numerators, two scores per op k (0..15): key block k / 8,
    // registers 2 (k % 8), +1; 16-key chunk c of the P operand is pw[c]
    float ps0 = 0.f, ps1 = 0.f;
    auto soft_op = [&](const p_f32x16 (&s)[2], p_u32x4 (&pw)[4], float mu, int k) {
        const int jb = k >> 3, v = 2 * (k & 7);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[jb][v], c2, -mu));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[jb][v + 1], c2, -mu));
        ps0 += p0;
        ps1 += p1;
        pw[2 * jb + (v >> 3)][(v & 7) >> 1] = p_pack(p0, p1);
    };
    // score instruction r (0..15): k-chunk r / 2, key block r % 2; its K
    // operand is read two instructions ahead
    constexpr int KPF = 2, VPF = 2;   // operands read this many matrix instructions ahead
    auto score_mma = [&](p_f32x16 (&s)[2], p_bf16x8 (&kop)[16], int ks, int r) {
        const int kc = r >> 1, jb = r & 1;
        if (r + KPF < 16) kop[r + KPF] = kread(ks, (r + KPF) >> 1, (r + KPF) & 1);
        if (kc == 0) p_mma_s0(s[jb], kop[r], qop[kc]);
        else p_mma_s(s[jb], kop[r], qop[kc]);
    };
    // PV instruction r (0..15): chunk r / 4, feature block r % 4; its V
    // operand is read two instructions ahead (the first two during [A])
    auto pv_mma = [&](p_bf16x8 (&vop)[16], const p_u32x4 (&pw)[4], int vs, int r) {
        if (r + VPF < 16) vop[r + VPF] = vread(vs, (r + VPF) >> 2, (r + VPF) & 3);
        p_mma_o(oacc[r & 3], vop[r], pw[r >> 2]);
    };

    // ---- main loop: two wave groups in ping-pong -------------------------
    // A step of one wave is two phases: M(t), its matrix instructions only
    // -- the scores of tile t+1 (K stage (t+1) % 3) and O += V_t^T P_t (V
    // stage t % 3) -- and V(t), its vector work only: the row maximum and
    // softmax of tile t+1, which give P_{t+1}.  Waves 0..3 (one per SIMD)
    // run M(t) while waves 4..7 (the other wave of each SIMD) run V(t-1),
    // and the other way round, one workgroup barrier between half-steps: on
    // every SIMD one wave's matrix instructions run beside the other wave's
    // vector instructions.  M(t) also copies K tile t+3 into stage t % 3 and
    // V tile t+2 into stage (t+2) % 3 (both read last in M(t-1), a half-step
    // or more before) and, before its closing barrier, waits for the copies
    // of M(t-1), which M(t+1) reads.  Copies past the end repeat the last
    // tile.  One score buffer serves: V(t) consumes the scores of tile t+1
    // before M(t+1) writes those of tile t+2.
    p_u32x4 pw[4];
    auto softmax = [&]() {
        const float mu = m == -INFINITY ? 0.f : m;
        ps0 = 0.f;
        ps1 = 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) soft_op(sacc[0], pw, mu, k);
        lsum += ps0 + ps1;
        p_pin_f(lsum);
        p_pin_p(pw);
    };
    if (n > 0) {
        p_bf16x8 kop[16];
#pragma unroll
        for (int r = 0; r < KPF; ++r) kop[r] = kread(0, r >> 1, r & 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) score_mma(sacc[0], kop, 0, r);
        if (tile_masked(key_lim(0))) mask_keys(sacc[0], key_lim(0));
        p_fence_s(sacc[0]);
#pragma unroll
        for (int j = 0; j < 16; ++j) max_op(sacc[0], j);
        finish_max();
        softmax();
    }
    // every wave is done with K stage 0 before M(0) copies tile 3 into it,
    // and K1 and V0 have landed (K2 and V1 may still run: M(0) waits for
    // them before its barrier)
    __builtin_amdgcn_s_waitcnt(0x0F70 | 4);   // vmcnt(4)
    p_barrier();
    // Continuing a Ring pass with bf16 output: the previous result's rows of
    // this wave are copied now into its Q staging region (free once Q is in
    // registers), and its LSE loaded, so that the epilogue's merge does not
    // wait for them.  The copies land before the epilogue (its vmcnt wait).
    float lse_prev = -INFINITY;
    if (a.acc && su < 0) {
        if (i < Sq) lse_prev = a.lse[(b * Sq + i) * H + hh];
        if constexpr (OUT_BF16) {
            const uint32_t ldo = (uint32_t)(H * kPD * 2);
            const int64_t rows = Sq > r0 ? (Sq - r0 < 32 ? Sq - r0 : 32) : 0;
            const p_rsrc orr = p_make_rsrc(static_cast<const unsigned char*>(a.o) +
                                               ((b * Sq + (rows > 0 ? r0 : 0)) * H + hh) * kPD * 2,
                                           rows > 0 ? (uint32_t)((rows - 1) * ldo + kPD * 2) : 0u);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                p_dma(orr, (uint32_t)(4 * j + (lane >> 4)) * ldo + (uint32_t)((lane & 15) << 4),
                      (uint32_t)(uintptr_t)(L + OFF_Q + wave * 32 * kPRowB + j * 1024));
        }
    }
    const bool lead = wave < kPWaves / 2;
    // M(t): the scores of tile t+1 interleaved with the PV instructions of
    // tile t (past the last tile the scores are computed and masked)
    auto mphase = [&](auto t3_tag, int t) {
        constexpr int T3 = decltype(t3_tag)::value;
        constexpr int KS = (T3 + 1) % 3, VS = T3;
        const int tk = t + 3 < n ? t + 3 : n - 1, tv = t + 2 < n ? t + 2 : n - 1;
        p_bf16x8 kop[16], vop[16];
        // the operand addresses pass through here each phase: nothing
        // derived from them (stage offsets, which the reads take as
        // immediates) is kept in registers across the loop
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) asm volatile("" : "+v"(kaddr[kc]));
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(vaddr[k][db]));
#pragma unroll
        for (int r = 0; r < KPF; ++r) kop[r] = kread(KS, r >> 1, r & 1);
#pragma unroll
        for (int r = 0; r < VPF; ++r) vop[r] = vread(VS, r >> 2, r & 3);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            score_mma(sacc[0], kop, KS, r);
            pv_mma(vop, pw, VS, r);
            if ((r & 3) == 1) {
                const int c = r >> 2;
                if (c < 2) copy_tile(krs, OFF_K, tk, T3, c);
                else copy_tile(vrs, OFF_V, tv, (T3 + 2) % 3, c - 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        // the copies of M(t-1) have landed (this phase's 4 may still run)
        __builtin_amdgcn_s_waitcnt(0x0F70 | 4);
        p_barrier();
    };
    // V(t): the row maximum and softmax of tile t+1 (past the last tile:
    // every key masked, nothing changes)
    auto vphase = [&](int t) {
        // the last score instructions of M(t) have written their registers
        p_fence_s(sacc[0]);
        const int lim = key_lim(t + 1);
        if (tile_masked(lim)) mask_keys(sacc[0], lim);
#pragma unroll
        for (int j = 0; j < 16; ++j) max_op(sacc[0], j);
        p_pin_f(mx);
        finish_max();
        softmax();
        p_barrier();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (!lead) p_barrier();   // the second group starts a half-step later
    for (int t = 0; n > 0; t += 3) {
        mphase(I0{}, t);
        vphase(t);
        if (t + 1 >= n) break;
        mphase(I1{}, t + 1);
        vphase(t + 1);
        if (t + 2 >= n) break;
        mphase(I2{}, t + 2);
        vphase(t + 2);
        if (t + 3 >= n) break;
    }
    if (lead) p_barrier();    // and ends a half-step later
    // the last copies (into stages nothing reads) have landed and every wave
    // is done with the stages before the LDS is reused; O is final
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    p_fence_o(oacc);

    // ---- epilogue: O = acc / l, LSE = m + log2 l (natural log stored);
    // with a.acc merged into the (o, lse) already there, with the weights of
    // the LSE merge.
    float lt;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
        lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lb2 = lt > 0.f ? m + __log2f(lt) : -INFINITY;
    // The rows' result (o x inv, LSE lb2 in log2 units) written out; with
    // a.acc merged into the (o, lse) already there (lse_prev, and with bf16
    // output the previous rows copied into this wave's Q staging region).
    auto write_out = [&](const p_f32x16 (&o)[4], const float inv, const float lb2) {
    float wp = 0.f, wb = 1.f, lse_out2 = lb2;
    if (a.acc) {
        const float lp2 = lse_prev * kPLog2e;
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
        // the wave's 32 x 128 tile through LDS, stored as whole rows (4 rows
        // of 256 bytes per instruction)
        constexpr int RS = kPRowB + 16;
        constexpr int WS = 32 * RS + 32 * 8;
        p_lds_u8* R = L + wave * WS;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * db + 8 * g + 4 * hg;
                const p_u32x2 w{p_pack(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                p_pack(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
                *(__attribute__((address_space(3))) p_u32x2*)(R + l32 * RS + d0 * 2) = w;
            }
        if (a.acc && hg == 0) *(__attribute__((address_space(3))) p_f32x2*)(R + 32 * RS + l32 * 8) = p_f32x2{wp, wb};
        // this wave's LDS stores are done before its lanes read each other's
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        const int rr = lane >> 4, cu = lane & 15;
        auto dst_of = [&](int k) {
            const int64_t row = r0 + 4 * k + rr;
            return reinterpret_cast<p_u32x4*>(static_cast<unsigned char*>(a.o) + ((b * Sq + row) * H + hh) * kPD * 2 +
                                              cu * 16);
        };
        auto row_ok = [&](int k) { return r0 + 4 * k + rr < Sq; };
        // the previous result's rows, copied into LDS at the start
        p_u32x4 pvv[8];
        if (a.acc) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                pvv[k] = *(const p_lds_u32x4*)(L + OFF_Q + wave * 32 * kPRowB + (4 * k + rr) * kPRowB + cu * 16);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = 4 * k + rr;
            p_u32x4 w = *(const p_lds_u32x4*)(R + r * RS + cu * 16);
            if (a.acc) {
                const p_f32x2 wr = *(const __attribute__((address_space(3))) p_f32x2*)(R + 32 * RS + r * 8);
                const bool use = wr[0] != 0.f;   // a previous result of weight 0 is not read
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = fmaf(wr[0], use ? p_lo(pvv[k][e]) : 0.f, wr[1] * p_lo(w[e]));
                    const float hi = fmaf(wr[0], use ? p_hi(pvv[k][e]) : 0.f, wr[1] * p_hi(w[e]));
                    w[e] = p_pack(lo, hi);
                }
            }
            if (row_ok(k)) *dst_of(k) = w;
        }
    } else {
        if (i < Sq) {
            const int64_t orow = ((b * Sq + i) * H + hh) * kPD;
            const float sb = wb * inv;
            auto dst_of = [&](int db, int g) {
                return reinterpret_cast<p_f32x4*>(static_cast<float*>(a.o) + orow + 32 * db + 8 * g + 4 * hg);
            };
            p_f32x4 pvv[4][4];
            const bool use = a.acc && wp != 0.f;
            if (use) {
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) pvv[db][g] = *dst_of(db, g);
            }
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    p_f32x4 x{o[db][4 * g] * sb, o[db][4 * g + 1] * sb, o[db][4 * g + 2] * sb,
                              o[db][4 * g + 3] * sb};
                    if (use) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = fmaf(wp, pvv[db][g][e], x[e]);
                    }
                    *dst_of(db, g) = x;
                }
        }
    }
    if (hg == 0 && i < Sq) a.lse[(b * Sq + i) * H + hh] = lse_out2 * kPLn2;
    };
    if (!SPLIT || su < 0) {
        write_out(oacc, inv, lb2);
        return;
    }

    // ---- a piece: store, count in; the last piece of the unit combines ---
    // Pieces of a unit run on different XCDs, whose L2 caches are not
    // coherent with each other for ordinary accesses.  Every slot access is
    // a device-scope one (cache policy sc1, as the memory model's relaxed
    // device-scope atomic loads and stores are), which is coherent across
    // XCDs by itself: each wave's slot stores complete before the workgroup
    // counts in, and no cache-wide write-back or invalidate is needed.
    if constexpr (SPLIT) {
        const int np = a.split_p;
        const int64_t n_split = (int64_t)a.n_qtiles * a.H * a.B - a.n_whole;
        unsigned char* const wsb = static_cast<unsigned char*>(a.ws) + (int64_t)su * np * kP32SlotBytes;
        const __amdgpu_buffer_rsrc_t wr =
            __builtin_amdgcn_make_buffer_rsrc(wsb, (short)0, (int)(np * kP32SlotBytes), 0x00020000);
        constexpr int kDev = 16;   // cache policy sc1: device-scope access
        const int row = 32 * wave + l32;
        {
            const int sb = piece * (int)kP32SlotBytes;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int db = j >> 1, v0 = 8 * (j & 1);
                const p_u32x4 w{p_pack(oacc[db][v0] * inv, oacc[db][v0 + 1] * inv),
                                p_pack(oacc[db][v0 + 2] * inv, oacc[db][v0 + 3] * inv),
                                p_pack(oacc[db][v0 + 4] * inv, oacc[db][v0 + 5] * inv),
                                p_pack(oacc[db][v0 + 6] * inv, oacc[db][v0 + 7] * inv)};
                store_slot_b128(w, wr, tid * 16, sb + j * (kPWaves * 64 * 16));
            }
            if (hg == 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lb2), wr, row * 4, sb + 65536, kDev);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are complete
        __syncthreads();
        int32_t* const cnt = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(a.ws) +
                                                        n_split * np * kP32SlotBytes) + su;
        volatile __attribute__((address_space(3))) int* const flag =
            reinterpret_cast<volatile __attribute__((address_space(3))) int*>(L);
        if (tid == 0) *flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int arrived = *flag;
        __syncthreads();   // every wave has read the flag before the LDS is written again
        if (arrived != np - 1) return;
        // the last piece: the unit's slots in piece order (the same loads and
        // arithmetic whichever piece combines them)
        float mx2 = -INFINITY;
        for (int k = 0; k < np; ++k)
            mx2 = __builtin_elementwise_maximum(
                mx2, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wr, row * 4, k * (int)kP32SlotBytes + 65536,
                                                                          kDev)));
        p_f32x16 comb[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) comb[db][v] = 0.f;
        float wsum = 0.f;
        for (int k = 0; k < np; ++k) {
            const int sb = k * (int)kP32SlotBytes;
            const float lk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wr, row * 4, sb + 65536, kDev));
            const float wk = lk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lk - mx2);
            wsum += wk;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const p_u32x4 q = __builtin_bit_cast(
                    p_u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, tid * 16, sb + j * (kPWaves * 64 * 16), kDev));
                const int db = j >> 1, v0 = 8 * (j & 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    comb[db][v0 + 2 * e] = fmaf(wk, p_lo(q[e]), comb[db][v0 + 2 * e]);
                    comb[db][v0 + 2 * e + 1] = fmaf(wk, p_hi(q[e]), comb[db][v0 + 2 * e + 1]);
                }
            }
        }
        if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // continuing a Ring pass: the running result's LSE, and with bf16
        // output its rows in this wave's Q staging region
        if (a.acc) {
            if (i < Sq) lse_prev = a.lse[(b * Sq + i) * H + hh];
            if constexpr (OUT_BF16) {
                const uint32_t ldo = (uint32_t)(H * kPD * 2);
                const int64_t rows = Sq > r0 ? (Sq - r0 < 32 ? Sq - r0 : 32) : 0;
                const p_rsrc orr = p_make_rsrc(static_cast<const unsigned char*>(a.o) +
                                                   ((b * Sq + (rows > 0 ? r0 : 0)) * H + hh) * kPD * 2,
                                               rows > 0 ? (uint32_t)((rows - 1) * ldo + kPD * 2) : 0u);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    p_dma(orr, (uint32_t)(4 * j + (lane >> 4)) * ldo + (uint32_t)((lane & 15) << 4),
                          (uint32_t)(uintptr_t)(L + OFF_Q + wave * 32 * kPRowB + j * 1024));
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the rows have landed
            }
        }
        const bool live = mx2 != -INFINITY && wsum > 0.f;
        write_out(comb, live ? 1.f / wsum : 0.f, live ? mx2 + __log2f(wsum) : -INFINITY);
    }
}

bool attn_p32_fits(int64_t Sk, int64_t row_heads)
{
    // the key range of one head must fit the 32-bit buffer range
    const int64_t n = (Sk + kPBN - 1) / kPBN;
    return n > 0 && Sk * row_heads * kPD * 2 < (int64_t)0xF0000000;
}

bool attn_p32_diag_ok(const AttnArgs& a)
{
    // one increasing piece of keys covers the block (the allowed keys of a
    // row are a prefix), positions fit the kernel's 32-bit counts
    return a.masked && a.Sq > 0 && a.Sk > 0 && a.kmap.seg_len >= a.Sk && a.kmap.stride >= 1;
}

bool attn_p32_mask_ok(const AttnArgs& a)
{
    if (!a.masked) return true;
    if (a.Sq <= 0 || a.Sk <= 0) return false;
    int64_t klo, khi;
    pos_range(a.kmap, 0, a.Sk, klo, khi);
    for (int64_t t0 = 0; t0 < a.Sq; t0 += kPBM) {
        int64_t qlo, qhi;
        pos_range(a.qmap, t0, t0 + kPBM < a.Sq ? t0 + kPBM : a.Sq, qlo, qhi);
        if (!(khi <= qlo || klo > qhi)) return false;   // this unit holds a diagonal
    }
    return true;
}

// Costs of the kernel's fixed parts in tile steps (one tile step: the 256
// rows of a workgroup against 64 keys), measured on the FLUX.1 share's
// chunks: the prologue up to the first step, a whole unit's epilogue, a
// piece's slot store and count, and the combine of a unit's pieces.
constexpr double kPStartSteps = 2.3, kPEpilogueSteps = 1.1, kPStoreSteps = 1.3, kPCombineSteps = 2.6;

SplitPlan plan_p32_split(int64_t n_units, int64_t n_tiles, int n_cu, int64_t Sk, int64_t row_heads)
{
    // Tile-step model of one launch, one workgroup per compute unit (u: a
    // whole unit's fixed cost, o: a piece's, m: the combine):
    //  * plain: ceil(U / C) rounds of N + u;
    //  * U > C: f = floor(U / C) rounds whole and the last partial round's r
    //    units in p equal pieces, run first: ceil(N / p) + o + m + f (N + u);
    //  * U <= C / 2: every unit in p = min(8, C / U) equal pieces, one round
    //    of ceil(N / p) + o + m.
    // A split is taken when it saves at least 5% of the plain launch.  (A
    // launch that leaves fewer than half the compute units idle runs plain:
    // cutting its units so that the idle ones run the short pieces measured
    // slower than the plain launch.)
    SplitPlan plan;
    if (n_cu <= 0 || n_units <= 0 || n_tiles < 8 || !attn_p32_fits(Sk, row_heads)) return plan;
    const double u = kPStartSteps + kPEpilogueSteps, o = kPStartSteps + kPStoreSteps, m = kPCombineSteps;
    const double N = (double)n_tiles;
    const int64_t f = n_units / n_cu, r = n_units - f * n_cu;
    const double plain = (double)(f + (r > 0)) * (N + u);
    double best = plain;
    if (f >= 1) {
        if (r == 0) return plan;
        for (int p = 2; p <= 8 && r * p <= n_cu && n_tiles / p >= 4; ++p) {
            const double T = (double)((n_tiles + p - 1) / p) + o + m + (double)f * (N + u);
            if (T < best) {
                best = T;
                plan.p = p;
                plan.n_whole = f * n_cu;
            }
        }
    } else {
        const int64_t pe = std::min<int64_t>(8, n_cu / n_units);
        if (pe >= 2) {
            const double T = (double)((n_tiles + pe - 1) / pe) + o + m;
            if (T < best) {
                best = T;
                plan.p = (int)pe;
            }
        }
    }
    if (best >= 0.95 * plain) return SplitPlan{};
    plan.p32 = true;
    return plan;
}

hipError_t launch_attn_p32(int o_dtype, int form, const AttnArgs& a0, hipStream_t s)
{
    AttnArgs a = a0;
    a.n_qtiles = (int32_t)((a.Sq + kPBM - 1) / kPBM);
    const int64_t units = (int64_t)a.n_qtiles * a.H * a.B;
    if (units <= 0) return hipSuccess;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 block(64 * kPWaves);
    const bool ob = o_dtype == UAA_BF16;
    if (form == 3) {
        if (a.split_p <= 1 || a.ws == nullptr || a.masked || a.n_whole < 0 || a.n_whole >= units)
            return hipErrorInvalidValue;
        const int64_t blocks = a.n_whole + (units - a.n_whole) * a.split_p;
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        const dim3 grid((unsigned)blocks);
        return ob ? launch_kernel(attn_p32_kernel<true, false, true>, grid, block, 0, s, a)
                  : launch_kernel(attn_p32_kernel<false, false, true>, grid, block, 0, s, a);
    }
    const dim3 grid((unsigned)units);
    if (form == 2)
        return ob ? launch_kernel(attn_p32_kernel<true, true, false>, grid, block, 0, s, a)
                  : launch_kernel(attn_p32_kernel<false, true, false>, grid, block, 0, s, a);
    return ob ? launch_kernel(attn_p32_kernel<true, false, false>, grid, block, 0, s, a)
              : launch_kernel(attn_p32_kernel<false, false, false>, grid, block, 0, s, a);
}

}  // namespace uaa
