// internal.h -- declarations shared by the HIP translation units of libuaa.
// Not part of the public ABI (include/uaa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/uaa.h"

namespace uaa {

// Launch through hipLaunchKernel so the launch status is this launch's own
// (a <<<>>> launch only reports through the sticky hipGetLastError state).
template <typename Arg>
inline hipError_t launch_kernel(void (*kern)(Arg), dim3 grid, dim3 block, size_t lds_bytes,
                                hipStream_t stream, const Arg& arg)
{
    void* params[] = {const_cast<Arg*>(&arg)};
    return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, params, lds_bytes, stream);
}

// --------------------------------------------------------------------------
// Permute: arguments after host validation.  Offsets are in tokens / heads
// (< 2^31); `vec_bytes` is the access width chosen on the host (1, 2, 4, 8
// or 16), and every head slice and pointer is a multiple of it.  The launch
// grid is (row chunks, source rank, batch * tensor); source y contributes
// T_y rows of run_y vectors.
// --------------------------------------------------------------------------
struct FastDiv {  // n / d for 0 <= n < 2^31, d >= 1, via one mul-hi and a shift
    uint32_t mul;
    uint32_t shift;
    uint32_t d;
};
FastDiv make_fastdiv(uint32_t d);

constexpr int kPermMaxSrc = 64;       // tensors * world source pointers
constexpr int kPermMaxTensors = UAA_MAX_PERMUTE_TENSORS;

struct PermuteArgs {
    const unsigned char* src[kPermMaxSrc];   // [tensor * world + y]
    unsigned char* dst[kPermMaxTensors];
    int32_t seq_off[UAA_MAX_WORLD + 1];
    int32_t head_off[UAA_MAX_WORLD + 1];
    // n / run as mul-hi + shift (mul 0: shift only), per tensor and source y
    uint32_t run_mul[kPermMaxTensors][UAA_MAX_WORLD];
    uint8_t run_shift[kPermMaxTensors][UAA_MAX_WORLD];
    int32_t world, rank, n_tensors;
    int32_t head_vecs[kPermMaxTensors];      // vectors per head slice of one token, per tensor
    int32_t vec_bytes[kPermMaxTensors];      // vector width of each tensor: 16, 8, 4, 2 or 1
    int32_t H;
    int32_t max_rows_x_run;                  // max over tensors and y of T_y * run_y, sizes grid x
};

hipError_t launch_permute(int dir, const PermuteArgs& a, int64_t B, hipStream_t s);

// --------------------------------------------------------------------------
// Merge.
// --------------------------------------------------------------------------
struct MergeArgs {
    const void* o_parts[USP_MAX_PARTS];
    const float* lse_parts[USP_MAX_PARTS];
    void* o_out;
    float* lse_out;
    int64_t rows;         // B * S * H
    int32_t D;
    int32_t n_parts;
};

hipError_t launch_merge(int part_dtype, int out_dtype, const MergeArgs& a, hipStream_t s);

// --------------------------------------------------------------------------
// Attention.  Token positions of both sides as two affine segments:
//   pos(idx) = base0 + stride * idx                    for idx <  seg_len
//            = base1 + stride * (idx - seg_len)        for idx >= seg_len
// Every mask kind of usp_mask maps onto this form on the host.
// --------------------------------------------------------------------------
struct PosMap {
    int64_t base0, base1, stride, seg_len;
};

constexpr int kMaxGather = UAA_MAX_GATHER_WORLD;

struct AttnArgs {
    const void* q;        // [B, Sq, row_heads, D]; unused when n_qsh > 0
    const void* k;        // [B, Sk, row_heads, D]
    const void* v;
    void* o;
    float* lse;
    int64_t B, H, Sq, Sk; // H: heads of the output (and of the work grid)
    // Inputs read head head0 + h of tokens of row_heads heads each (the
    // plain call: row_heads = H, head0 = 0).  With n_qsh > 0 the queries are
    // gathered from token shards: query row r is token r of the sequence,
    // held by shard p (q_row0[p] <= r < q_row0[p+1]) at q_sh[p] as
    // [B, q_row0[p+1] - q_row0[p], row_heads, D].
    int64_t row_heads, head0;
    int32_t n_qsh;
    int32_t q_row0[kMaxGather + 1];
    const void* q_sh[kMaxGather];
    float scale;          // softmax scale as given
    float scale_log2;     // scale * log2(e)
    int32_t masked;       // 0: every key allowed; 1: kpos(j) <= qpos(i)
    int32_t acc;          // 1: merge into the (o, lse) already there (a Ring pass continues)
    PosMap qmap, kmap;
    int32_t n_qtiles;     // ceil(Sq / rows per workgroup), set by the launcher
    // Key split (bf16, unmasked): units [0, n_whole) run whole, one
    // workgroup each; the keys of every later unit (those of the last,
    // partial round of workgroups, or every unit when they are few) are cut
    // into split_p pieces of about equal length, each run by its own
    // workgroup, and the last piece of a unit to finish combines the pieces.
    int32_t split_p;      // 1: no split
    int32_t n_whole;      // units run whole, set by the caller with split_p
    int32_t split_p32;    // 1: the pipelined kernel runs the pieces (its slot layout)
    void* ws;             // workspace: piece partials, then arrival counters
};

// Workspace of the key split: one partial slot per piece of a split unit
// (the 512 lanes' O accumulators and each lane's reference maximum and
// half-row sum), then one int32 arrival counter per split unit.
constexpr int64_t kSplitLanes = 512;
constexpr int64_t kSplitQuads = 17;   // 16-byte quads per lane: 16 of O accumulators, 1 of (max, sum)
constexpr int64_t kSplitSlotBytes = kSplitLanes * kSplitQuads * 16;

struct SplitPlan {
    int p = 1;            // pieces per split unit; 1: no split
    int64_t n_whole = 0;  // units run whole
    bool p32 = false;     // the pipelined kernel runs the pieces
};
inline int64_t split_ws_bytes(int64_t n_split, int p) { return n_split * p * kSplitSlotBytes + 4 * n_split; }

// Workspace of the pipelined kernel's key split: one slot per piece of a
// split unit (the piece's normalised O as bf16, 64 KiB, then its 256 rows'
// LSE), then one int32 arrival counter per split unit.
constexpr int64_t kP32SlotBytes = 65536 + 1024;
inline int64_t p32_split_ws_bytes(int64_t n_split, int p) { return n_split * p * kP32SlotBytes + 4 * n_split; }
inline int64_t split_counter_offset(int64_t n_split, int p, bool p32)
{
    return n_split * p * (p32 ? kP32SlotBytes : kSplitSlotBytes);
}

// Split plan for n_units units of n_tiles key tiles on n_cu compute units,
// and the unit count of the bf16 kernel.
SplitPlan plan_split(int64_t n_units, int64_t n_tiles, int n_cu);
// The pipelined kernel's split plan for this problem (bf16, D = 128,
// unmasked calls), p = 1 when the plain launch is as fast.
SplitPlan plan_p32_split(int64_t n_units, int64_t n_tiles, int n_cu, int64_t Sk, int64_t row_heads);
int64_t attn_bf16_units(int64_t B, int64_t H, int64_t Sq);

hipError_t launch_attn_bf16(int D, int o_dtype, const AttnArgs& a, hipStream_t s);
// the USP_KERNEL_* code of the kernel launch_attn_bf16 runs for these arguments
int attn_bf16_kernel_choice(int D, const AttnArgs& a);
// D = 128, no key split: the software-pipelined kernel, where one head's keys fit its 32-bit buffer range
bool attn_p32_fits(int64_t Sk, int64_t row_heads);
// masked calls: the rows of every 256-row unit see every key of the block or none
bool attn_p32_mask_ok(const AttnArgs& a);
// masked calls whose keys are one increasing piece: units on the diagonal
// run their live tiles with rows masked one by one (the kernel's DIAG form)
bool attn_p32_diag_ok(const AttnArgs& a);
// form: 1 plain, 2 DIAG, 3 key split (a.split_p, a.n_whole)
hipError_t launch_attn_p32(int o_dtype, int form, const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_fp32(int D, const AttnArgs& a, hipStream_t s);

// --------------------------------------------------------------------------
// Attention backward.  Tensors as in the forward: q, dout, dq [B, Sq, H, D];
// k, v, dk, dv [B, Sk, H, D]; lse, delta [B, Sq, H] fp32.
// --------------------------------------------------------------------------
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;     // natural log, over every key block of the rows
    const float* delta;   // rowsum(dout * o) - dlse
    void* dq;
    void* dk;
    void* dv;
    int64_t B, H, Sq, Sk;
    float scale;          // softmax scale as given
    float scale_log2;     // scale * log2(e)
    int32_t masked;       // 0: every key allowed; 1: kpos(j) <= qpos(i)
    int32_t accumulate;   // bit 0: add into dq; bit 1: add into dk and dv
    int32_t grad_bf16;    // gradients stored as bf16 (else fp32)
    int32_t n_tiles;      // work tiles per (batch, head) of the launched kernel, set by the launcher
    PosMap qmap, kmap;
    // dS workspace (null: none): dS^T of every (key, query) pair in bf16 as
    // matrix-core B operands.  Block (b, h, query block qc of 32, key group
    // kc of 16) is 1 KB at (((b * H + h) * ds_nq + qc) * ds_nk + kc) * 1024;
    // its lane L = 32 e + n holds, as 8 bf16, the pairs of query 32 qc + n
    // with keys 16 kc + 4 e + {0, 1, 2, 3, 8, 9, 10, 11}.  The dK/dV kernel
    // writes it; the dQ kernel then forms dQ = scale dS K from it instead of
    // recomputing the scores.
    void* ds;
    int64_t ds_nq;        // ceil(Sq / 32)
    int64_t ds_nk;        // ceil(Sk / 16)
};

struct DeltaArgs {
    const void* o;
    const void* dout;
    const float* dlse;    // may be null
    float* delta;
    int64_t rows;         // B * S * H
};

// dK/dV kernel then dQ kernel (bf16 inputs; fp32 inputs)
hipError_t launch_attn_bwd_bf16(int D, const BwdArgs& a, hipStream_t s);
hipError_t launch_attn_bwd_fp32(int D, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_delta(int dtype, int D, const DeltaArgs& a, hipStream_t s);

}  // namespace uaa
