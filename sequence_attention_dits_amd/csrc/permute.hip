// permute.hip -- local gather of the Ulysses all-to-all for one rank.
//
// "Context parallelism" (diffusers docs), "Ulysses Attention": the first
// all-to-all leaves each GPU every token of a subset of heads, the second
// regroups by token.  "Ulysses Anything Attention": token and head counts per
// rank are arbitrary and nothing is padded, so the owner of a token (or a
// head) is found from prefix sums instead of a division by the degree.
//
// The copy is HBM-bound: every destination row (one token of one batch) is a
// run of contiguous bytes gathered from one source row (SEQ2HEAD) or from one
// slice of each head shard (HEAD2SEQ).  A wavefront owns a few destination
// rows at a time; its lanes stride along each row with the widest access the
// alignment allows (16 bytes for bf16 rows of 128-wide heads), all loads of a
// pass are issued before any store so many bytes are in flight per CU, and
// both sides use non-temporal accesses since nothing is reused.
#include "internal.h"

namespace uaa {

FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f{0u, 0u, d};
    if (d == 0) return f;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;               // l = ceil(log2 d)
    if ((1ull << l) == d) {                    // power of two: a shift
        f.mul = 0;
        f.shift = l;
        return f;
    }
    // d not a power of two, so l >= 2 and 2^(l-1) < d < 2^l.  With
    // m = ceil(2^(31+l) / d) < 2^32, floor(n * m / 2^(31+l)) == n / d for
    // every n < 2^31 (the rounding term stays below 1/d).
    const unsigned __int128 num = (unsigned __int128)1 << (31 + l);
    f.mul = (uint32_t)((num + d - 1) / d);
    f.shift = l - 1;                           // applied after the high 32 bits
    return f;
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f)
{
    return f.mul == 0 ? (n >> f.shift) : (__umulhi(n, f.mul) >> f.shift);
}

// Last index p in [0, world) with off[p] <= x (the rank owning x; with empty
// ranks several share one offset and the last of them owns the range).
__device__ __forceinline__ int owner(const int64_t* off, int world, int64_t x)
{
    int lo = 0, hi = world - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <typename V>
__device__ __forceinline__ V ld_nt(const V* p) { return __builtin_nontemporal_load(p); }
template <typename V>
__device__ __forceinline__ void st_nt(V* p, V x) { __builtin_nontemporal_store(x, p); }

constexpr int kWaves = 4;     // wavefronts per workgroup
constexpr int kRowsUnroll = 2; // destination rows per lane group per pass
constexpr int kVecUnroll = 4;  // vectors per lane per row per pass

template <int DIR, typename V>
__global__ __launch_bounds__(64 * kWaves) void permute_kernel(const PermuteArgs a)
{
    const int lane = threadIdx.x & 63;
    const int lpr_log2 = a.lanes_per_row_log2;
    const int lpr = 1 << lpr_log2;
    const int groups = 64 >> lpr_log2;         // rows side by side in a wave
    const int sub = lane >> lpr_log2;
    const int sublane = lane & (lpr - 1);
    const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t row0 = wave * (int64_t)(groups * kRowsUnroll);

    const V* const* src = reinterpret_cast<const V* const*>(a.src);
    V* dst = reinterpret_cast<V*>(a.dst);
    const int64_t row_vecs = a.row_vecs;

    bool live[kRowsUnroll];
    const V* srow[kRowsUnroll];     // SEQ2HEAD: start of the source run
    int64_t stok[kRowsUnroll];      // HEAD2SEQ: token index inside each head shard
    V* drow[kRowsUnroll];
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
        const int64_t row = row0 + (int64_t)u * groups + sub;
        live[u] = row < a.n_rows;
        const int64_t r = live[u] ? row : 0;
        const uint32_t b = fast_div((uint32_t)r, a.div_tokens);
        const int64_t tok = r - (int64_t)b * a.div_tokens.d;
        drow[u] = dst + r * row_vecs;
        if (DIR == UAA_SEQ2HEAD) {
            // token tok of the global sequence lives in shard p at tok - off[p]
            const int p = owner(a.seq_off, a.world, tok);
            const int64_t Sp = a.seq_off[p + 1] - a.seq_off[p];
            const int64_t srow_idx = ((int64_t)b * Sp + (tok - a.seq_off[p])) * a.H + a.head_off[a.rank];
            srow[u] = src[p] + srow_idx * a.head_vecs;
            stok[u] = 0;
        } else {
            const int64_t S = a.seq_off[a.world];
            stok[u] = (int64_t)b * S + a.seq_off[a.rank] + tok;
            srow[u] = nullptr;
        }
    }

    for (int64_t c0 = 0; c0 < row_vecs; c0 += (int64_t)kVecUnroll * lpr) {
        V tmp[kRowsUnroll][kVecUnroll];
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < kVecUnroll; ++k) {
                const int64_t vi = c0 + (int64_t)k * lpr + sublane;
                if (live[u] && vi < row_vecs) {
                    if (DIR == UAA_SEQ2HEAD) {
                        tmp[u][k] = ld_nt(srow[u] + vi);
                    } else {
                        // head h of the destination row comes from the shard
                        // whose head range contains h
                        const uint32_t h = fast_div((uint32_t)vi, a.div_head);
                        const int64_t e = vi - (int64_t)h * a.head_vecs;
                        const int r = owner(a.head_off, a.world, h);
                        const int64_t Hr = a.head_off[r + 1] - a.head_off[r];
                        const int64_t off = (stok[u] * Hr + ((int64_t)h - a.head_off[r])) * a.head_vecs + e;
                        tmp[u][k] = ld_nt(src[r] + off);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < kVecUnroll; ++k) {
                const int64_t vi = c0 + (int64_t)k * lpr + sublane;
                if (live[u] && vi < row_vecs) st_nt(drow[u] + vi, tmp[u][k]);
            }
        }
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int DIR>
static hipError_t launch_dir(int vec_bytes, const PermuteArgs& a, hipStream_t s)
{
    const int groups = 64 >> a.lanes_per_row_log2;
    const int64_t rows_per_wave = (int64_t)groups * kRowsUnroll;
    const int64_t waves = (a.n_rows + rows_per_wave - 1) / rows_per_wave;
    const int64_t blocks = (waves + kWaves - 1) / kWaves;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(64 * kWaves);
    switch (vec_bytes) {
    case 16: return launch_kernel(permute_kernel<DIR, u32x4>, grid, block, 0, s, a);
    case 8: return launch_kernel(permute_kernel<DIR, u32x2>, grid, block, 0, s, a);
    case 4: return launch_kernel(permute_kernel<DIR, unsigned int>, grid, block, 0, s, a);
    case 2: return launch_kernel(permute_kernel<DIR, unsigned short>, grid, block, 0, s, a);
    case 1: return launch_kernel(permute_kernel<DIR, unsigned char>, grid, block, 0, s, a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_permute(int dir, int vec_bytes, const PermuteArgs& a, hipStream_t s)
{
    return dir == UAA_SEQ2HEAD ? launch_dir<UAA_SEQ2HEAD>(vec_bytes, a, s)
                               : launch_dir<UAA_HEAD2SEQ>(vec_bytes, a, s);
}

}  // namespace uaa
