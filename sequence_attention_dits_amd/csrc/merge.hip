// merge.hip -- N-way LSE-rescaled merge of partial attention results.
//
// "Add Unified Sequence Parallel attention" (diffusers PR #12693), review
// thread: each Ring step's (out, lse) is folded into the running pair in
// fp32 with a sigmoid-weighted update of out and a log-sigmoid update of
// lse, and cast back to the query dtype once.  Folding N partials that way
// is the softmax-weighted mean of the partials; this kernel computes it in
// one pass with the maximum shifted out, which keeps rows whose partials are
// -inf (no allowed key) finite instead of NaN:
//   M = max_n lse_n,  lse = M + log(sum_n exp(lse_n - M)),
//   o = sum_n exp(lse_n - lse) * o_n,   (0, -inf) if every lse_n is -inf.
//
// HBM-bound: each row is D contiguous elements per partial.  A row is split
// over D / VEC lanes (VEC elements = 16 bytes each), so a wavefront covers
// several rows with fully coalesced 16-byte accesses.  The few LSE loads of
// a row come first (shared by the row's lanes through the cache); a partial
// whose LSE is -inf had no allowed key in its block and gets weight 0, so
// its O slice is not read at all (in a zigzag Ring pass that is half the
// rows of most key blocks); the other partials' slices are all loaded before
// any arithmetic.
#include "internal.h"

namespace uaa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(unsigned short b)
{
    return __uint_as_float(((unsigned int)b) << 16);
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ unsigned short f32_to_bf16(float f)
{
    const unsigned int u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);
    return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// VEC elements of type T: loaded as raw bits (Raw; zero bits are 0.0) and
// widened to fp32 only where the arithmetic needs them, so the loads of all
// partials in flight hold half the registers for bf16.
template <typename T, int VEC> struct Slice;

template <> struct Slice<unsigned short, 8> {     // bf16, 16 bytes
    typedef u32x4 Raw;
    static __device__ __forceinline__ Raw load(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
    static __device__ __forceinline__ Raw zero() { return u32x4{0u, 0u, 0u, 0u}; }
    static __device__ __forceinline__ void widen(const Raw& w, float* x)
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(void* p, const float* x)
    {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (unsigned int)f32_to_bf16(x[2 * e]) | ((unsigned int)f32_to_bf16(x[2 * e + 1]) << 16);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    }
};

template <> struct Slice<float, 4> {              // fp32, 16 bytes
    typedef u32x4 Raw;
    static __device__ __forceinline__ Raw load(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
    static __device__ __forceinline__ Raw zero() { return u32x4{0u, 0u, 0u, 0u}; }
    static __device__ __forceinline__ void widen(const Raw& w, float* x)
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
    }
    static __device__ __forceinline__ void store(void* p, const float* x)
    {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(x[e]);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    }
};

template <> struct Slice<unsigned short, 1> {     // bf16, any D
    typedef unsigned short Raw;
    static __device__ __forceinline__ Raw load(const void* p) { return *reinterpret_cast<const unsigned short*>(p); }
    static __device__ __forceinline__ Raw zero() { return 0; }
    static __device__ __forceinline__ void widen(const Raw& w, float* x) { x[0] = bf16_to_f32(w); }
    static __device__ __forceinline__ void store(void* p, const float* x)
    {
        *reinterpret_cast<unsigned short*>(p) = f32_to_bf16(x[0]);
    }
};

template <> struct Slice<float, 1> {              // fp32, any D
    typedef float Raw;
    static __device__ __forceinline__ Raw load(const void* p) { return *reinterpret_cast<const float*>(p); }
    static __device__ __forceinline__ Raw zero() { return 0.f; }
    static __device__ __forceinline__ void widen(const Raw& w, float* x) { x[0] = w; }
    static __device__ __forceinline__ void store(void* p, const float* x)
    {
        *reinterpret_cast<float*>(p) = x[0];
    }
};

// A row's D / VEC slices are spread over `lpr` lanes (a power of two, at most
// 64; lanes loop when a row has more slices), so a wavefront covers 64 / lpr
// rows side by side and no lane index needs a division.  Each lane group
// handles RU rows per pass: the LSEs of all partials of its rows are loaded
// first, then the O slices of the partials with a finite LSE (the others
// count as zero: their weight is 0), then the weights and weighted sums.
template <typename TIn, typename TOut, int VEC, int NMAX, int RU>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a, int lpr_log2)
{
    const int lane = threadIdx.x & 63;
    const int lpr = 1 << lpr_log2;
    const int groups = 64 >> lpr_log2;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t row0 = wave * groups * RU + (lane >> lpr_log2);
    const int N = a.n_parts;
    const int slices = a.D / VEC;              // host guarantees divisibility

    float lse[RU][NMAX];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const int64_t row = row0 + (int64_t)u * groups;
#pragma unroll
        for (int n = 0; n < NMAX; ++n) lse[u][n] = (n < N && row < a.rows) ? a.lse_parts[n][row] : -INFINITY;
    }
    for (int seg = lane & (lpr - 1); seg < slices; seg += lpr) {
        typedef Slice<TIn, VEC> In;
        typename In::Raw x[RU][NMAX];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int64_t row = row0 + (int64_t)u * groups;
            const int64_t elem = row * a.D + (int64_t)seg * VEC;
#pragma unroll
            for (int n = 0; n < NMAX; ++n)   // only rows < a.rows and partials n < N have a finite LSE
                x[u][n] = lse[u][n] != -INFINITY ? In::load(reinterpret_cast<const TIn*>(a.o_parts[n]) + elem)
                                                 : In::zero();
        }
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int64_t row = row0 + (int64_t)u * groups;
            if (row >= a.rows) continue;
            float M = -INFINITY;
#pragma unroll
            for (int n = 0; n < NMAX; ++n) M = fmaxf(M, lse[u][n]);
            float acc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
            float L = -INFINITY;
            if (M != -INFINITY) {
                float sum = 0.f;
#pragma unroll
                for (int n = 0; n < NMAX; ++n)
                    if (n < N) sum += __expf(lse[u][n] - M);
                L = M + __logf(sum);
#pragma unroll
                for (int n = 0; n < NMAX; ++n)
                    if (n < N) {
                        const float w = __expf(lse[u][n] - L);
                        float xv[VEC];
                        In::widen(x[u][n], xv);
#pragma unroll
                        for (int e = 0; e < VEC; ++e) acc[e] = fmaf(w, xv[e], acc[e]);
                    }
            }
            const int64_t elem = row * a.D + (int64_t)seg * VEC;
            Slice<TOut, VEC>::store(reinterpret_cast<TOut*>(a.o_out) + elem, acc);
            // lse_out may be one of the partials' LSE arrays: every lane read
            // its row's partial LSEs before the first pass, and the row's
            // lanes are one wavefront, in step
            if ((seg & (lpr - 1)) == 0 && seg + lpr >= slices) a.lse_out[row] = L;
        }
    }
}

template <typename TIn, typename TOut, int VEC>
static hipError_t launch_vec(const MergeArgs& a, hipStream_t s)
{
    constexpr int RU = 1;   // measured: one row per lane group per pass is fastest
    const int slices = a.D / VEC;
    int lpr_log2 = 0;
    while ((1 << lpr_log2) < slices && lpr_log2 < 6) ++lpr_log2;
    const int64_t rows_per_block = 4 * (64 >> lpr_log2) * RU;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(256);
    void* params[] = {const_cast<MergeArgs*>(&a), &lpr_log2};
    const void* fn;
    if (a.n_parts <= 2) fn = reinterpret_cast<const void*>(merge_kernel<TIn, TOut, VEC, 2, RU>);
    else if (a.n_parts <= 4) fn = reinterpret_cast<const void*>(merge_kernel<TIn, TOut, VEC, 4, RU>);
    else if (a.n_parts <= 8) fn = reinterpret_cast<const void*>(merge_kernel<TIn, TOut, VEC, 8, RU>);
    else fn = reinterpret_cast<const void*>(merge_kernel<TIn, TOut, VEC, 16, RU>);
    return hipLaunchKernel(fn, grid, block, params, 0, s);
}

// 16-byte slices need D * size to be a multiple of 16 on both sides and
// 16-byte aligned base pointers; otherwise one element per lane.
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipError_t launch_merge(int part_dtype, int out_dtype, const MergeArgs& a, hipStream_t s)
{
    bool wide = aligned16(a.o_out);
    for (int n = 0; n < a.n_parts; ++n) wide = wide && aligned16(a.o_parts[n]);
    const bool in_bf = part_dtype == UAA_BF16, out_bf = out_dtype == UAA_BF16;
    if (in_bf && out_bf) {
        if (wide && a.D % 8 == 0) return launch_vec<unsigned short, unsigned short, 8>(a, s);
        return launch_vec<unsigned short, unsigned short, 1>(a, s);
    }
    if (!in_bf && !out_bf) {
        if (wide && a.D % 4 == 0) return launch_vec<float, float, 4>(a, s);
        return launch_vec<float, float, 1>(a, s);
    }
    // mixed dtypes: one element per lane keeps both sides simple
    if (in_bf) return launch_vec<unsigned short, float, 1>(a, s);
    return launch_vec<float, unsigned short, 1>(a, s);
}

}  // namespace uaa
