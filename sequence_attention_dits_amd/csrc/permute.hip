// permute.hip -- local gather of the Ulysses all-to-all for one rank.
//
// "Context parallelism" (diffusers docs), "Ulysses Attention": the first
// all-to-all leaves each GPU every token of a subset of heads, the second
// regroups by token.  "Ulysses Anything Attention": token and head counts per
// rank are arbitrary and nothing is padded, so row ranges come from prefix
// sums instead of a division by the degree.
//
// Both directions are a set of 2-D strided copies, one per source rank y
// (and per tensor and batch when several are moved in one launch):
//   SEQ2HEAD  source = token shard y: its S_y rows, each the run of this
//             rank's H_r heads (a contiguous slice of the source row), land
//             at destination rows seq_off[y] .. seq_off[y+1]-1;
//   HEAD2SEQ  source = head shard y: this rank's S_p rows of it, each a run
//             of H_y heads, land at head columns head_off[y] .. of the
//             destination rows.
// The launch grid is (chunks, source y, batch * tensor), so every base
// pointer, stride and run length is uniform in a workgroup (scalar
// registers); tensors of one launch may differ in row size (e.g. O and its
// LSE), each moving in the widest vector its rows and pointers allow.
// Inside a chunk each lane moves U vectors of the flattened (row, column)
// space, loads issued before stores; a workgroup walks several chunks.  Loads and stores are plain: the
// gathered Q, K, V are read by the attention right after, and leaving them
// in the caches is worth more to the whole step (-1.4 %) than the
// non-temporal stores that make the gather alone faster; non-temporal loads
// were ~20 % slower.  The row of a vector comes from one multiply-high by a
// host-computed reciprocal.
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

constexpr int kThreads = 256;
constexpr int kVecPerThread = 2;   // vectors in flight per lane (4 and 8 measured slower over the step's permutes)
constexpr int kMaxChunkGroups = 2048;

// The copy of one (source y, tensor, batch b) chunk in vectors of type V.
template <int DIR, typename V>
__device__ __forceinline__ void permute_chunk(const PermuteArgs& a, int y, int tensor, int64_t b)
{
    const int64_t hv = a.head_vecs[tensor];
    const int64_t S = a.seq_off[a.world];

    // uniform description of this source's copy
    int64_t T, run, src_stride, src_col0, src_row0, dst_stride, dst_col0, dst_row0;
    if (DIR == UAA_SEQ2HEAD) {
        T = a.seq_off[y + 1] - a.seq_off[y];
        run = (int64_t)(a.head_off[a.rank + 1] - a.head_off[a.rank]) * hv;
        src_stride = a.H * hv;
        src_col0 = a.head_off[a.rank] * hv;
        src_row0 = b * T;
        dst_stride = run;
        dst_col0 = 0;
        dst_row0 = b * S + a.seq_off[y];
    } else {
        T = a.seq_off[a.rank + 1] - a.seq_off[a.rank];
        run = (int64_t)(a.head_off[y + 1] - a.head_off[y]) * hv;
        src_stride = run;
        src_col0 = 0;
        src_row0 = b * S + a.seq_off[a.rank];
        dst_stride = a.H * hv;
        dst_col0 = a.head_off[y] * hv;
        dst_row0 = b * T;
    }
    const uint32_t n = (uint32_t)(T * run);           // < 2^31, checked on the host
    for (uint32_t base = blockIdx.x * (uint32_t)(kThreads * kVecPerThread); base < n;
         base += gridDim.x * (uint32_t)(kThreads * kVecPerThread)) {
    const V* src = reinterpret_cast<const V*>(a.src[tensor * a.world + y]) + src_row0 * src_stride + src_col0;
    V* dst = reinterpret_cast<V*>(a.dst[tensor]) + dst_row0 * dst_stride + dst_col0;
    const uint32_t mul = a.run_mul[tensor][y], shift = a.run_shift[tensor][y];

    V tmp[kVecPerThread];
    uint32_t row[kVecPerThread], col[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const uint32_t f = base + threadIdx.x + u * kThreads;
        row[u] = mul == 0 ? (f >> shift) : (__umulhi(f, mul) >> shift);
        col[u] = f - row[u] * (uint32_t)run;
        if (f < n) tmp[u] = src[(int64_t)row[u] * src_stride + col[u]];
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const uint32_t f = base + threadIdx.x + u * kThreads;
        if (f < n) dst[(int64_t)row[u] * dst_stride + col[u]] = tmp[u];
    }
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Each tensor moves in its own vector width (a uniform branch per
// workgroup), so a launch that carries O and its 4-byte LSE still moves O in
// 16-byte vectors.
template <int DIR>
__global__ __launch_bounds__(kThreads) void permute_kernel(const PermuteArgs a)
{
    const int y = blockIdx.y;
    const int tensor = (int)(blockIdx.z % (uint32_t)a.n_tensors);
    const int64_t b = blockIdx.z / (uint32_t)a.n_tensors;
    switch (a.vec_bytes[tensor]) {
    case 16: permute_chunk<DIR, u32x4>(a, y, tensor, b); break;
    case 8: permute_chunk<DIR, u32x2>(a, y, tensor, b); break;
    case 4: permute_chunk<DIR, unsigned int>(a, y, tensor, b); break;
    case 2: permute_chunk<DIR, unsigned short>(a, y, tensor, b); break;
    default: permute_chunk<DIR, unsigned char>(a, y, tensor, b); break;
    }
}

template <int DIR>
static hipError_t launch_dir(const PermuteArgs& a, int64_t B, hipStream_t s)
{
    const int64_t chunk = kThreads * kVecPerThread;
    // at most kMaxChunkGroups workgroups per (tensor, batch), each walking
    // its chunks at that stride: 3-4 % faster than one workgroup per chunk
    // at the FLUX.1 share's sizes (28 and 85 MB)
    int64_t gx = ((int64_t)a.max_rows_x_run + chunk - 1) / chunk;
    if (gx > kMaxChunkGroups / a.world) gx = kMaxChunkGroups / a.world > 0 ? kMaxChunkGroups / a.world : 1;
    const int64_t gz = B * a.n_tensors;
    if (gx <= 0 || gz <= 0) return hipSuccess;
    if (gx > 0x7fffffff || gz > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)gx, (unsigned)a.world, (unsigned)gz), block(kThreads);
    return launch_kernel(permute_kernel<DIR>, grid, block, 0, s, a);
}

hipError_t launch_permute(int dir, const PermuteArgs& a, int64_t B, hipStream_t s)
{
    return dir == UAA_SEQ2HEAD ? launch_dir<UAA_SEQ2HEAD>(a, B, s) : launch_dir<UAA_HEAD2SEQ>(a, B, s);
}

}  // namespace uaa
