// attn_common.h -- position maps and tile classification shared by the two
// attention kernels (fp32 and bf16).  Internal to libuaa.
//
// Positions: the USP / yunchang summary ("How It Works", "Highlighted
// Details") names zigzag, stripe and basic ring layouts; every one of them
// gives each side of an attention call a map from local row index to global
// token position made of at most two increasing affine pieces (PosMap).  A
// key is allowed for a query iff kpos <= qpos.
#pragma once

#include "internal.h"

namespace uaa {

__host__ __device__ inline int64_t pos_of(const PosMap& m, int64_t idx)
{
    return idx < m.seg_len ? m.base0 + m.stride * idx : m.base1 + m.stride * (idx - m.seg_len);
}

// [min, max] of pos_of over idx in [lo, hi), hi > lo.  Each piece increases.
__host__ __device__ inline void pos_range(const PosMap& m, int64_t lo, int64_t hi, int64_t& pmin,
                                          int64_t& pmax)
{
    if (hi <= m.seg_len || lo >= m.seg_len) {
        pmin = pos_of(m, lo);
        pmax = pos_of(m, hi - 1);
    } else {
        const int64_t a = pos_of(m, lo), b = pos_of(m, m.seg_len);
        const int64_t c = pos_of(m, m.seg_len - 1), d = pos_of(m, hi - 1);
        pmin = a < b ? a : b;
        pmax = c > d ? c : d;
    }
}

// Number of leading indices of the piece base + stride * idx (idx < n,
// stride >= 1) whose position is <= q: the allowed prefix of that piece.
__device__ __forceinline__ int64_t allowed_prefix(int64_t base, int64_t stride, int64_t q, int64_t n)
{
    if (n <= 0 || q < base) return 0;
    const int64_t c = (stride == 1 ? (q - base) : (q - base) / stride) + 1;
    return c < n ? c : n;
}

// 16-byte buffer store at device scope (cache policy sc1) of a piece's
// slot.  A buffer store of more than 8 bytes with a register offset reads
// its data registers after it issues; a vector ALU write to them in the next
// cycle can replace the data of some lanes before the store has read it
// (seen as dword 0 of lanes 12..15 of each 16 taking the next quad's value).
// The data stays live, and unwritten, through two wait states after the
// store.
template <typename V4>
__device__ __forceinline__ void store_slot_b128(V4 w, __amdgpu_buffer_rsrc_t rs, int voff, int soff)
{
    __builtin_amdgcn_raw_buffer_store_b128(w, rs, voff, soff, 16);
    asm volatile("s_nop 1" ::"v"(w));
}

// Workgroup index -> logical work index.  Workgroups are handed to the 8
// XCDs round-robin, and each XCD has its own L2: renumber so that each XCD
// gets one contiguous run of logical indices, i.e. the q tiles of the same
// head share the L2 that holds that head's K and V.
__device__ __forceinline__ uint32_t xcd_logical(uint32_t L, uint32_t n)
{
    const uint32_t per = n / 8u;
    return (L < per * 8u) ? (L % 8u) * per + L / 8u : L;
}

// Logical unit -> (q tile, head, batch).
__device__ __forceinline__ void unit_coords(const AttnArgs& a, uint32_t unit, int64_t& qt, int64_t& h, int64_t& b)
{
    qt = unit % (uint32_t)a.n_qtiles;
    const int64_t rest = unit / (uint32_t)a.n_qtiles;
    h = rest % a.H;
    b = rest / a.H;
}

__device__ __forceinline__ void decode_tile(const AttnArgs& a, int64_t& qt, int64_t& h, int64_t& b)
{
    unit_coords(a, xcd_logical(blockIdx.x, gridDim.x), qt, h, b);
}

}  // namespace uaa
