// abi.hip -- the extern "C" entry points of libuaa.so: host-side validation
// of every argument, conversion of the caller's description into kernel
// arguments, and one asynchronous launch on the caller's stream.  Nothing
// here synchronises the device or reads device memory.
#include <math.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "internal.h"

#define UAA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return UAA_OK;
    return fail(UAA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

constexpr int64_t kMaxElems = int64_t(1) << 46;   // far above any HBM, keeps products in int64
constexpr int64_t kMaxIdx32 = int64_t(1) << 31;

// Default head split: the first H mod world ranks take one extra head.
void even_split(int64_t total, int parts, int64_t* off)
{
    const int64_t base = total / parts, extra = total % parts;
    off[0] = 0;
    for (int p = 0; p < parts; ++p) off[p + 1] = off[p] + base + (p < extra ? 1 : 0);
}

}  // namespace

UAA_EXPORT const char* uaa_last_error(void) { return g_err; }

UAA_EXPORT int uaa_abi_version(void) { return 1; }

#ifndef UAA_BUILD_ID
#define UAA_BUILD_ID "unknown"
#endif
UAA_EXPORT const char* uaa_build_id(void) { return UAA_BUILD_ID; }

UAA_EXPORT int uaa_split_offsets(int64_t total, int parts, int64_t* off)
{
    if (parts < 1) return fail(UAA_ERR_INVALID_ARG, "split: parts must be >= 1, got %d", parts);
    if (total < 0) return fail(UAA_ERR_INVALID_ARG, "split: total must be >= 0, got %lld", (long long)total);
    if (off == nullptr) return fail(UAA_ERR_INVALID_ARG, "split: off is NULL");
    even_split(total, parts, off);
    return UAA_OK;
}

namespace {

// Shared by the permute entry points; Ds[t], elems[t]: features and element
// bytes of tensor t.
int permute_impl(int n_tensors, int dir, int rank, int world, const int64_t* seq_off,
                 const int64_t* head_off, int64_t B, int64_t H, const int64_t* Ds, const int* elems,
                 const void* const* src, void* const* dst, void* stream)
{
    if (dir != UAA_SEQ2HEAD && dir != UAA_HEAD2SEQ)
        return fail(UAA_ERR_INVALID_ARG, "permute: dir must be UAA_SEQ2HEAD or UAA_HEAD2SEQ, got %d", dir);
    if (world < 1 || world > UAA_MAX_WORLD)
        return fail(UAA_ERR_INVALID_ARG, "permute: world must be in [1, %d], got %d", UAA_MAX_WORLD, world);
    if (n_tensors < 1 || n_tensors > uaa::kPermMaxTensors || n_tensors * world > uaa::kPermMaxSrc)
        return fail(UAA_ERR_INVALID_ARG, "permute: need 1 <= n_tensors <= %d and n_tensors * world <= %d",
                    uaa::kPermMaxTensors, uaa::kPermMaxSrc);
    if (rank < 0 || rank >= world)
        return fail(UAA_ERR_INVALID_ARG, "permute: rank %d outside [0, %d)", rank, world);
    if (Ds == nullptr || elems == nullptr) return fail(UAA_ERR_INVALID_ARG, "permute: D or elem_bytes array is NULL");
    for (int t = 0; t < n_tensors; ++t) {
        if (B < 0 || H < 1 || Ds[t] < 1)
            return fail(UAA_ERR_INVALID_ARG, "permute: need B >= 0, H >= 1, D >= 1 (got %lld, %lld, %lld)",
                        (long long)B, (long long)H, (long long)Ds[t]);
        if (elems[t] != 1 && elems[t] != 2 && elems[t] != 4 && elems[t] != 8)
            return fail(UAA_ERR_INVALID_ARG, "permute: elem_bytes must be 1, 2, 4 or 8, got %d", elems[t]);
    }
    if (seq_off == nullptr) return fail(UAA_ERR_INVALID_ARG, "permute: seq_off is NULL");
    if (seq_off[0] != 0) return fail(UAA_ERR_INVALID_ARG, "permute: seq_off[0] must be 0");
    for (int p = 0; p < world; ++p)
        if (seq_off[p + 1] < seq_off[p])
            return fail(UAA_ERR_INVALID_ARG, "permute: seq_off decreases at rank %d", p);
    int64_t hoff[UAA_MAX_WORLD + 1];
    if (head_off == nullptr) {
        even_split(H, world, hoff);
    } else {
        for (int p = 0; p <= world; ++p) hoff[p] = head_off[p];
    }
    if (hoff[0] != 0 || hoff[world] != H)
        return fail(UAA_ERR_INVALID_ARG, "permute: head_off must run from 0 to H = %lld", (long long)H);
    for (int p = 0; p < world; ++p)
        if (hoff[p + 1] <= hoff[p])
            return fail(UAA_ERR_INVALID_ARG,
                        "permute: rank %d gets no heads (head_off must strictly increase; world <= H)", p);
    const int64_t S = seq_off[world];
    for (int t = 0; t < n_tensors; ++t)
        if (S >= kMaxIdx32 || H >= kMaxIdx32 || (double)B * S * H * Ds[t] * elems[t] > (double)kMaxElems)
            return fail(UAA_ERR_INVALID_ARG, "permute: tensor too large");
    if (src == nullptr || dst == nullptr) return fail(UAA_ERR_INVALID_ARG, "permute: src or dst array is NULL");

    const int64_t Sp = seq_off[rank + 1] - seq_off[rank];
    const int64_t out_tokens = dir == UAA_SEQ2HEAD ? S : Sp;
    if (B == 0 || out_tokens == 0) return UAA_OK;
    if (B * n_tensors > 65535) return fail(UAA_ERR_UNSUPPORTED, "permute: B * n_tensors above 65535");

    // Sources that hold data must be present; every pointer must be aligned.
    // Each tensor moves in the widest vector that divides its head slice
    // and that all its pointers' alignment allows.
    int vecs[uaa::kPermMaxTensors];
    for (int t = 0; t < n_tensors; ++t) {
        const int elem_bytes = elems[t];
        int vec = 16;
        while (vec > 1 && (Ds[t] * elem_bytes) % vec != 0) vec >>= 1;
        for (int p = 0; p < world; ++p) {
            // SEQ2HEAD reads every non-empty token shard; HEAD2SEQ every head shard
            if (dir == UAA_SEQ2HEAD && seq_off[p + 1] == seq_off[p]) continue;
            const void* sp = src[t * world + p];
            if (sp == nullptr) return fail(UAA_ERR_INVALID_ARG, "permute: src[%d] is NULL", t * world + p);
            if (!aligned(sp, elem_bytes))
                return fail(UAA_ERR_INVALID_ARG, "permute: src[%d] not aligned to %d bytes", t * world + p,
                            elem_bytes);
            while (vec > 1 && !aligned(sp, vec)) vec >>= 1;
        }
        if (dst[t] == nullptr) return fail(UAA_ERR_INVALID_ARG, "permute: dst[%d] is NULL", t);
        if (!aligned(dst[t], elem_bytes))
            return fail(UAA_ERR_INVALID_ARG, "permute: dst[%d] not aligned to %d bytes", t, elem_bytes);
        while (vec > 1 && !aligned(dst[t], vec)) vec >>= 1;
        vecs[t] = vec;
    }

    uaa::PermuteArgs a{};
    for (int i = 0; i < n_tensors * world; ++i) a.src[i] = static_cast<const unsigned char*>(src[i]);
    for (int t = 0; t < n_tensors; ++t) a.dst[t] = static_cast<unsigned char*>(dst[t]);
    for (int p = 0; p <= world; ++p) {
        a.seq_off[p] = (int32_t)seq_off[p];
        a.head_off[p] = (int32_t)hoff[p];
    }
    int64_t max_n = 0;
    for (int t = 0; t < n_tensors; ++t) {
        const int64_t hv = Ds[t] * elems[t] / vecs[t];
        a.head_vecs[t] = (int32_t)hv;
        a.vec_bytes[t] = vecs[t];
        for (int y = 0; y < world; ++y) {
            const int64_t T = dir == UAA_SEQ2HEAD ? seq_off[y + 1] - seq_off[y] : Sp;
            const int64_t run = (dir == UAA_SEQ2HEAD ? hoff[rank + 1] - hoff[rank] : hoff[y + 1] - hoff[y]) * hv;
            if (run >= kMaxIdx32 || T * run >= kMaxIdx32 - 4096)
                return fail(UAA_ERR_UNSUPPORTED, "permute: one shard moves 2^31 or more elements");
            const uaa::FastDiv f = uaa::make_fastdiv((uint32_t)run);
            a.run_mul[t][y] = f.mul;
            a.run_shift[t][y] = (uint8_t)f.shift;
            if (T * run > max_n) max_n = T * run;
        }
    }
    a.world = world;
    a.rank = rank;
    a.n_tensors = n_tensors;
    a.H = (int32_t)H;
    a.max_rows_x_run = (int32_t)max_n;
    return hip_status(uaa::launch_permute(dir, a, B, static_cast<hipStream_t>(stream)), "permute launch");
}

}  // namespace

UAA_EXPORT int uaa_seq2head_permute(int dir, int rank, int world, const int64_t* seq_off,
                                    const int64_t* head_off, int64_t B, int64_t H, int64_t D,
                                    int elem_bytes, const void* const* src, void* dst, void* stream)
{
    void* dsts[1] = {dst};
    return permute_impl(1, dir, rank, world, seq_off, head_off, B, H, &D, &elem_bytes, src, dsts, stream);
}

UAA_EXPORT int uaa_seq2head_permute_multi(int n_tensors, int dir, int rank, int world, const int64_t* seq_off,
                                          const int64_t* head_off, int64_t B, int64_t H, int64_t D,
                                          int elem_bytes, const void* const* src, void* const* dst,
                                          void* stream)
{
    if (n_tensors < 1 || n_tensors > uaa::kPermMaxTensors)
        return fail(UAA_ERR_INVALID_ARG, "permute: need 1 <= n_tensors <= %d and n_tensors * world <= %d",
                    uaa::kPermMaxTensors, uaa::kPermMaxSrc);
    int64_t Ds[uaa::kPermMaxTensors];
    int elems[uaa::kPermMaxTensors];
    for (int t = 0; t < n_tensors; ++t) {
        Ds[t] = D;
        elems[t] = elem_bytes;
    }
    return permute_impl(n_tensors, dir, rank, world, seq_off, head_off, B, H, Ds, elems, src, dst, stream);
}

UAA_EXPORT int uaa_seq2head_permute_multi_ex(int n_tensors, int dir, int rank, int world,
                                             const int64_t* seq_off, const int64_t* head_off, int64_t B,
                                             int64_t H, const int64_t* D, const int* elem_bytes,
                                             const void* const* src, void* const* dst, void* stream)
{
    return permute_impl(n_tensors, dir, rank, world, seq_off, head_off, B, H, D, elem_bytes, src, dst, stream);
}

namespace {

// Map one side of a usp_mask onto the two-piece affine position map.
int side_map(const usp_mask& m, bool q_side, int64_t n, uaa::PosMap& out)
{
    const int64_t big = int64_t(1) << 62;
    out = uaa::PosMap{0, 0, 1, big};
    switch (m.kind) {
    case USP_MASK_CAUSAL: {
        const int64_t off = q_side ? m.q_off : m.k_off;
        if (off < -(int64_t(1) << 60) || off > (int64_t(1) << 60))
            return fail(UAA_ERR_INVALID_ARG, "attn: causal offset out of range");
        out.base0 = off;
        return UAA_OK;
    }
    case USP_MASK_ZIGZAG: {
        const int32_t* ids = q_side ? m.q_chunks : m.k_chunks;
        if (m.chunk < 1 || m.chunk > (int64_t(1) << 40))
            return fail(UAA_ERR_INVALID_ARG, "attn: zigzag chunk length must be >= 1");
        if (ids[0] < 0) return fail(UAA_ERR_INVALID_ARG, "attn: zigzag chunk id must be >= 0");
        const int n_chunks = ids[1] >= 0 ? 2 : 1;
        if (n > n_chunks * m.chunk)
            return fail(UAA_ERR_INVALID_ARG, "attn: %s side has %lld rows but its chunks hold %lld",
                        q_side ? "query" : "key", (long long)n, (long long)(n_chunks * m.chunk));
        out.base0 = (int64_t)ids[0] * m.chunk;
        if (n_chunks == 2) {
            out.base1 = (int64_t)ids[1] * m.chunk;
            out.seg_len = m.chunk;
        }
        return UAA_OK;
    }
    case USP_MASK_STRIPE: {
        const int32_t r = q_side ? m.q_rank : m.k_rank;
        if (m.world < 1 || r < 0 || r >= m.world)
            return fail(UAA_ERR_INVALID_ARG, "attn: stripe needs world >= 1 and 0 <= rank < world");
        out.base0 = r;
        out.stride = m.world;
        return UAA_OK;
    }
    default:
        return fail(UAA_ERR_INVALID_ARG, "attn: unknown mask kind %d", m.kind);
    }
}

}  // namespace

// Compute units of the current device (cached per device).
static int device_cu_count()
{
    static std::atomic<int> cached[64];   // 0: not yet asked
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// [lo, hi] of the positions of rows [0, n), n >= 1, of a map whose pieces
// each increase.
static void host_pos_range(const uaa::PosMap& m, int64_t n, int64_t& lo, int64_t& hi)
{
    auto pos = [&](int64_t i) { return i < m.seg_len ? m.base0 + m.stride * i : m.base1 + m.stride * (i - m.seg_len); };
    if (n <= m.seg_len) {
        lo = pos(0);
        hi = pos(n - 1);
    } else {
        lo = std::min(pos(0), pos(m.seg_len));
        hi = std::max(pos(m.seg_len - 1), pos(n - 1));
    }
}

// No key of the block lies after any query in position: the mask allows
// every pair, and the call is an unmasked one (a Ring step over a block
// wholly in the past of the rank's queries).
static bool all_pairs_allowed(const uaa::PosMap& q, int64_t Sq, const uaa::PosMap& k, int64_t Sk)
{
    if (Sq <= 0 || Sk <= 0) return false;
    int64_t qlo, qhi, klo, khi;
    host_pos_range(q, Sq, qlo, qhi);
    host_pos_range(k, Sk, klo, khi);
    return khi <= qlo;
}

static bool pipelined_on()
{
    static const bool on = [] {
        const char* e = getenv("UAA_ATTN_P32");
        return !(e && e[0] == '0');
    }();
    return on;
}

// The pipelined kernel's key split where it applies (bf16, D = 128,
// unmasked), else the general kernel's.  row_heads: heads per input token
// (the gathering call reads the shards' rows).
static uaa::SplitPlan attn_split_plan(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                      const usp_mask* mask, int64_t row_heads = 0)
{
    uaa::SplitPlan none;
    if (dtype != UAA_BF16 || (D != 64 && D != 128) || B <= 0 || H <= 0 || Sq <= 0 || Sk <= 0) return none;
    if (mask != nullptr && mask->kind != USP_MASK_FULL) return none;
    if ((double)B * (Sq > Sk ? Sq : Sk) * H * D > (double)kMaxElems) return none;
    const int64_t units = uaa::attn_bf16_units(B, H, Sq);
    if (units > kMaxIdx32 / 8) return none;
    const int cus = device_cu_count();
    if (D == 128 && pipelined_on() && uaa::attn_p32_fits(Sk, row_heads > 0 ? row_heads : H))
        return uaa::plan_p32_split(units, (Sk + 63) / 64, cus, Sk,
                                   row_heads > 0 ? row_heads : H);
    return uaa::plan_split(units, (Sk + 63) / 64, cus);
}

static int64_t plan_ws_bytes(const uaa::SplitPlan& plan, int64_t B, int64_t H, int64_t Sq)
{
    if (plan.p <= 1) return 0;
    if (plan.p32) return uaa::p32_split_ws_bytes(uaa::attn_bf16_units(B, H, Sq) - plan.n_whole, plan.p);
    return uaa::split_ws_bytes(uaa::attn_bf16_units(B, H, Sq) - plan.n_whole, plan.p);
}

UAA_EXPORT size_t usp_attn_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                           const usp_mask* mask)
{
    return (size_t)plan_ws_bytes(attn_split_plan(dtype, B, H, Sq, Sk, D, mask), B, H, Sq);
}

// Queries gathered from token shards (usp_attn_fwd_lse_gather): every shard
// holds its tokens with row_heads heads each, of which this rank reads
// head0 .. head0 + H - 1.
struct GatherSrc {
    int world;
    const int64_t* seq_off;   // host, world + 1, validated by the caller
    const void* const* q_shards;
    int64_t row_heads, head0;
};

// Validates the call, builds the kernel arguments and launches.  With
// `kernel` non-null nothing is launched and the pointers are not checked:
// the USP_KERNEL_* code of the kernel the call would run is stored there (a
// workspace counts as given when workspace_bytes > 0).
// With clear_counters the key split's arrival counters in the workspace are
// zeroed on the stream (a small fill kernel) before the attention launch.
static hipError_t clear_split_counters(const uaa::AttnArgs& a, hipStream_t s);

static int attn_impl(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, const void* q,
                     const void* k, const void* v, void* o, int o_dtype, float* lse, float scale,
                     const usp_mask* mask, void* workspace, size_t workspace_bytes, int acc, const GatherSrc* g,
                     void* stream, int* kernel = nullptr, bool clear_counters = false)
{
    if (dtype != UAA_BF16 && dtype != UAA_FP32)
        return fail(UAA_ERR_INVALID_ARG, "attn: dtype must be UAA_BF16 or UAA_FP32, got %d", dtype);
    if (o_dtype != UAA_BF16 && o_dtype != UAA_FP32)
        return fail(UAA_ERR_INVALID_ARG, "attn: o_dtype must be UAA_BF16 or UAA_FP32, got %d", o_dtype);
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || D < 1)
        return fail(UAA_ERR_INVALID_ARG, "attn: negative size");
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(UAA_ERR_INVALID_ARG, "attn: scale must be finite and > 0");
    if (mask != nullptr && (mask->kind < USP_MASK_FULL || mask->kind > USP_MASK_STRIPE))
        return fail(UAA_ERR_INVALID_ARG, "attn: unknown mask kind %d", mask->kind);
    if (D != 64 && D != 128) return fail(UAA_ERR_UNSUPPORTED, "attn: D must be 64 or 128, got %lld", (long long)D);
    if (dtype == UAA_FP32 && o_dtype != UAA_FP32)
        return fail(UAA_ERR_UNSUPPORTED, "attn: fp32 input needs fp32 output");
    const int64_t RH = g != nullptr ? g->row_heads : H;   // heads per input token
    if ((double)B * (Sq > Sk ? Sq : Sk) * RH * D > (double)kMaxElems)
        return fail(UAA_ERR_INVALID_ARG, "attn: tensor too large");
    if (B == 0 || H == 0 || Sq == 0) {
        if (kernel != nullptr) *kernel = USP_KERNEL_NONE;
        return UAA_OK;
    }
    const bool query = kernel != nullptr;   // the plan only looks at sizes, dtypes and the mask
    if (!query && ((g == nullptr && q == nullptr) || o == nullptr || lse == nullptr))
        return fail(UAA_ERR_INVALID_ARG, "attn: q, o and lse must not be NULL");
    if (!query && Sk > 0 && (k == nullptr || v == nullptr))
        return fail(UAA_ERR_INVALID_ARG, "attn: k and v must not be NULL when Sk > 0");
    if (!query &&
        ((g == nullptr && !aligned(q, 16)) || !aligned(o, 16) || (Sk > 0 && (!aligned(k, 16) || !aligned(v, 16)))))
        return fail(UAA_ERR_INVALID_ARG, "attn: q, k, v and o must be 16-byte aligned");
    if (!query && !aligned(lse, 4)) return fail(UAA_ERR_INVALID_ARG, "attn: lse must be 4-byte aligned");
    if (g != nullptr && !query)
        for (int p = 0; p < g->world; ++p) {
            if (g->seq_off[p + 1] == g->seq_off[p]) continue;
            if (g->q_shards[p] == nullptr || !aligned(g->q_shards[p], 16))
                return fail(UAA_ERR_INVALID_ARG, "attn: q shard %d is NULL or not 16-byte aligned", p);
        }

    uaa::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.Sq = Sq;
    a.Sk = Sk;
    a.row_heads = RH;
    a.head0 = g != nullptr ? g->head0 : 0;
    a.n_qsh = 0;
    if (g != nullptr) {
        a.n_qsh = g->world;
        for (int p = 0; p <= g->world; ++p) a.q_row0[p] = (int32_t)g->seq_off[p];
        for (int p = 0; p < g->world; ++p) a.q_sh[p] = g->q_shards[p];
    }
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    a.masked = 0;
    a.acc = acc;
    if (mask != nullptr && mask->kind != USP_MASK_FULL) {
        a.masked = 1;
        int rc = side_map(*mask, true, Sq, a.qmap);
        if (rc != UAA_OK) return rc;
        rc = side_map(*mask, false, Sk, a.kmap);
        if (rc != UAA_OK) return rc;
        if (all_pairs_allowed(a.qmap, Sq, a.kmap, Sk)) a.masked = 0;
    }
    if (dtype == UAA_BF16 && ((double)(Sq > Sk ? Sq : Sk) * RH * D * 2 >= 4294967296.0))
        return fail(UAA_ERR_UNSUPPORTED, "attn: one batch of q or k/v must stay below 4 GiB");
    // the launcher sets the q-tile count for its tile height; bound the grid here
    if (((Sq + 63) / 64) * H * B >= kMaxIdx32) return fail(UAA_ERR_INVALID_ARG, "attn: grid too large");
    a.split_p = 1;
    a.n_whole = 0;
    a.split_p32 = 0;
    if (query ? workspace_bytes > 0 : workspace != nullptr) {
        if (!query && !aligned(workspace, 256))
            return fail(UAA_ERR_INVALID_ARG, "attn: workspace must be 256-byte aligned");
        const uaa::SplitPlan plan = attn_split_plan(dtype, B, H, Sq, Sk, D, mask, RH);
        if (plan.p > 1 && workspace_bytes >= (size_t)plan_ws_bytes(plan, B, H, Sq)) {
            a.split_p = plan.p;
            a.n_whole = plan.n_whole;
            a.split_p32 = plan.p32 ? 1 : 0;
            // a query has no workspace pointer: any non-null value stands in
            // for it, since the plan only checks that there is one
            a.ws = query ? reinterpret_cast<void*>(uintptr_t(256)) : workspace;
        }
    }
    if (query) {
        *kernel = dtype == UAA_BF16 ? uaa::attn_bf16_kernel_choice((int)D, a) : USP_KERNEL_FP32;
        return UAA_OK;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (clear_counters && a.split_p > 1) {
        const int rc = hip_status(clear_split_counters(a, s), "scratch counter clear");
        if (rc != UAA_OK) return rc;
    }
    if (dtype == UAA_BF16) return hip_status(uaa::launch_attn_bf16((int)D, o_dtype, a, s), "attn launch");
    return hip_status(uaa::launch_attn_fp32((int)D, a, s), "attn launch");
}

UAA_EXPORT int usp_attn_fwd_lse(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                const void* q, const void* k, const void* v, void* o, int o_dtype,
                                float* lse, float scale, const usp_mask* mask, void* stream)
{
    return attn_impl(dtype, B, H, Sq, Sk, D, q, k, v, o, o_dtype, lse, scale, mask, nullptr, 0, 0, nullptr, stream);
}

UAA_EXPORT int usp_attn_fwd_lse_ws(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                   const void* q, const void* k, const void* v, void* o, int o_dtype,
                                   float* lse, float scale, const usp_mask* mask, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    return attn_impl(dtype, B, H, Sq, Sk, D, q, k, v, o, o_dtype, lse, scale, mask, workspace, workspace_bytes,
                     0, nullptr, stream);
}

UAA_EXPORT int usp_attn_fwd_lse_acc(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                    const void* q, const void* k, const void* v, void* o, int o_dtype,
                                    float* lse, float scale, const usp_mask* mask, void* workspace,
                                    size_t workspace_bytes, void* stream)
{
    return attn_impl(dtype, B, H, Sq, Sk, D, q, k, v, o, o_dtype, lse, scale, mask, workspace, workspace_bytes,
                     1, nullptr, stream);
}

UAA_EXPORT int usp_attn_kernel(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, int o_dtype,
                               const usp_mask* mask, size_t workspace_bytes)
{
    int k = USP_KERNEL_NONE;
    const int rc = attn_impl(dtype, B, H, Sq, Sk, D, nullptr, nullptr, nullptr, nullptr, o_dtype, nullptr, 1.0f,
                             mask, nullptr, workspace_bytes, 0, nullptr, nullptr, &k);
    return rc != UAA_OK ? rc : k;
}

UAA_EXPORT int usp_attn_fwd_lse_gather(int dtype, int world, int rank, const int64_t* seq_off,
                                       const int64_t* head_off, int64_t B, int64_t H, int64_t D,
                                       const void* const* q_shards, const void* const* k_shards,
                                       const void* const* v_shards, int k_shard, void* o, int o_dtype,
                                       float* lse, float scale, const usp_mask* mask, void* workspace,
                                       size_t workspace_bytes, int accumulate, void* stream)
{
    if (dtype != UAA_BF16)
        return fail(dtype == UAA_FP32 ? UAA_ERR_UNSUPPORTED : UAA_ERR_INVALID_ARG,
                    "attn gather: bf16 input only, got dtype %d", dtype);
    if (world < 1 || world > UAA_MAX_GATHER_WORLD)
        return fail(UAA_ERR_INVALID_ARG, "attn gather: world must be in [1, %d], got %d", UAA_MAX_GATHER_WORLD, world);
    if (rank < 0 || rank >= world) return fail(UAA_ERR_INVALID_ARG, "attn gather: rank %d outside [0, %d)", rank, world);
    if (k_shard < 0 || k_shard >= world)
        return fail(UAA_ERR_INVALID_ARG, "attn gather: k_shard %d outside [0, %d)", k_shard, world);
    if (B < 0 || H < 1) return fail(UAA_ERR_INVALID_ARG, "attn gather: need B >= 0 and H >= 1");
    if (seq_off == nullptr) return fail(UAA_ERR_INVALID_ARG, "attn gather: seq_off is NULL");
    if (seq_off[0] != 0) return fail(UAA_ERR_INVALID_ARG, "attn gather: seq_off[0] must be 0");
    for (int p = 0; p < world; ++p)
        if (seq_off[p + 1] < seq_off[p])
            return fail(UAA_ERR_INVALID_ARG, "attn gather: seq_off decreases at rank %d", p);
    if (seq_off[world] >= kMaxIdx32) return fail(UAA_ERR_INVALID_ARG, "attn gather: sequence too long");
    int64_t hoff[UAA_MAX_WORLD + 1];
    if (head_off == nullptr) {
        even_split(H, world, hoff);
    } else {
        for (int p = 0; p <= world; ++p) hoff[p] = head_off[p];
    }
    if (hoff[0] != 0 || hoff[world] != H)
        return fail(UAA_ERR_INVALID_ARG, "attn gather: head_off must run from 0 to H = %lld", (long long)H);
    for (int p = 0; p < world; ++p)
        if (hoff[p + 1] <= hoff[p])
            return fail(UAA_ERR_INVALID_ARG, "attn gather: rank %d gets no heads (head_off must strictly increase)", p);
    if (q_shards == nullptr || k_shards == nullptr || v_shards == nullptr)
        return fail(UAA_ERR_INVALID_ARG, "attn gather: a shard array is NULL");
    const GatherSrc g{world, seq_off, q_shards, H, hoff[rank]};
    return attn_impl(dtype, B, hoff[rank + 1] - hoff[rank], seq_off[world], seq_off[k_shard + 1] - seq_off[k_shard], D,
                     nullptr, k_shards[k_shard], v_shards[k_shard], o, o_dtype, lse, scale, mask, workspace,
                     workspace_bytes, accumulate ? 1 : 0, &g, stream);
}

UAA_EXPORT int usp_lse_merge(int n_parts, int64_t B, int64_t S, int64_t H, int64_t D,
                             const void* const* o_parts, int part_dtype, const float* const* lse_parts,
                             void* o_out, int out_dtype, float* lse_out, void* stream)
{
    if (n_parts < 1 || n_parts > USP_MAX_PARTS)
        return fail(UAA_ERR_INVALID_ARG, "merge: n_parts must be in [1, %d], got %d", USP_MAX_PARTS, n_parts);
    if (part_dtype != UAA_BF16 && part_dtype != UAA_FP32)
        return fail(UAA_ERR_INVALID_ARG, "merge: part_dtype must be UAA_BF16 or UAA_FP32");
    if (out_dtype != UAA_BF16 && out_dtype != UAA_FP32)
        return fail(UAA_ERR_INVALID_ARG, "merge: out_dtype must be UAA_BF16 or UAA_FP32");
    if (B < 0 || S < 0 || H < 0 || D < 1) return fail(UAA_ERR_INVALID_ARG, "merge: bad sizes");
    if ((double)B * S * H * D > (double)kMaxElems) return fail(UAA_ERR_INVALID_ARG, "merge: tensor too large");
    const int64_t rows = B * S * H;
    if (rows == 0) return UAA_OK;
    if (D > 65536) return fail(UAA_ERR_UNSUPPORTED, "merge: D above 65536");
    if (o_parts == nullptr || lse_parts == nullptr || o_out == nullptr || lse_out == nullptr)
        return fail(UAA_ERR_INVALID_ARG, "merge: NULL pointer");
    const uintptr_t in_sz = part_dtype == UAA_BF16 ? 2 : 4, out_sz = out_dtype == UAA_BF16 ? 2 : 4;
    uaa::MergeArgs a{};
    for (int n = 0; n < n_parts; ++n) {
        if (o_parts[n] == nullptr || lse_parts[n] == nullptr)
            return fail(UAA_ERR_INVALID_ARG, "merge: part %d is NULL", n);
        if (!aligned(o_parts[n], in_sz) || !aligned(lse_parts[n], 4))
            return fail(UAA_ERR_INVALID_ARG, "merge: part %d misaligned", n);
        if (o_parts[n] == o_out && part_dtype != out_dtype)
            return fail(UAA_ERR_INVALID_ARG, "merge: o_out may alias a part only when the dtypes match");
        a.o_parts[n] = o_parts[n];
        a.lse_parts[n] = lse_parts[n];
    }
    if (!aligned(o_out, out_sz) || !aligned(lse_out, 4))
        return fail(UAA_ERR_INVALID_ARG, "merge: output misaligned");
    a.o_out = o_out;
    a.lse_out = lse_out;
    a.rows = rows;
    a.D = (int32_t)D;
    a.n_parts = n_parts;
    return hip_status(uaa::launch_merge(part_dtype, out_dtype, a, static_cast<hipStream_t>(stream)),
                      "merge launch");
}

// --------------------------------------------------------------------------
// Attention backward.
// --------------------------------------------------------------------------
UAA_EXPORT int usp_attn_bwd_delta(int dtype, int64_t B, int64_t S, int64_t H, int64_t D, const void* o,
                                  const void* dout, const float* dlse, float* delta, void* stream)
{
    if (dtype != UAA_BF16 && dtype != UAA_FP32)
        return fail(UAA_ERR_INVALID_ARG, "bwd delta: dtype must be UAA_BF16 or UAA_FP32, got %d", dtype);
    if (B < 0 || S < 0 || H < 0 || D < 1) return fail(UAA_ERR_INVALID_ARG, "bwd delta: bad sizes");
    if (D != 64 && D != 128) return fail(UAA_ERR_UNSUPPORTED, "bwd delta: D must be 64 or 128, got %lld", (long long)D);
    if ((double)B * S * H * D > (double)kMaxElems) return fail(UAA_ERR_INVALID_ARG, "bwd delta: tensor too large");
    const int64_t rows = B * S * H;
    if (rows == 0) return UAA_OK;
    if (o == nullptr || dout == nullptr || delta == nullptr)
        return fail(UAA_ERR_INVALID_ARG, "bwd delta: o, dout and delta must not be NULL");
    if (!aligned(o, 16) || !aligned(dout, 16)) return fail(UAA_ERR_INVALID_ARG, "bwd delta: o and dout must be 16-byte aligned");
    if (!aligned(delta, 4) || (dlse != nullptr && !aligned(dlse, 4)))
        return fail(UAA_ERR_INVALID_ARG, "bwd delta: delta and dlse must be 4-byte aligned");
    uaa::DeltaArgs a{o, dout, dlse, delta, rows};
    return hip_status(uaa::launch_bwd_delta(dtype, (int)D, a, static_cast<hipStream_t>(stream)), "bwd delta launch");
}

// Bytes of the dS workspace of the backward for these sizes: dS^T in bf16,
// 1 KB per 32 queries x 16 keys (0 where the path does not apply: fp32
// inputs, D != 128, a mask that excludes some pair, or no pair at all).
static size_t bwd_ds_bytes(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, bool masked)
{
    if (dtype != UAA_BF16 || D != 128 || masked || B <= 0 || H <= 0 || Sq <= 0 || Sk <= 0) return 0;
    const double n = (double)B * H * ((Sq + 31) / 32) * ((Sk + 15) / 16) * 1024.0;
    if (n >= 9.0e18) return 0;
    return (size_t)B * (size_t)H * (size_t)((Sq + 31) / 32) * (size_t)((Sk + 15) / 16) * 1024u;
}

static int attn_bwd_impl(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, const void* q,
                         const void* k, const void* v, const void* dout, const float* lse, const float* delta,
                         void* dq, void* dk, void* dv, int grad_dtype, float scale, const usp_mask* mask,
                         int accumulate, void* workspace, size_t workspace_bytes, void* stream)
{
    if (dtype != UAA_BF16 && dtype != UAA_FP32)
        return fail(UAA_ERR_INVALID_ARG, "bwd: dtype must be UAA_BF16 or UAA_FP32, got %d", dtype);
    if (grad_dtype != UAA_BF16 && grad_dtype != UAA_FP32)
        return fail(UAA_ERR_INVALID_ARG, "bwd: grad_dtype must be UAA_BF16 or UAA_FP32, got %d", grad_dtype);
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || D < 1) return fail(UAA_ERR_INVALID_ARG, "bwd: negative size");
    if (!(scale > 0.f) || !isfinite(scale)) return fail(UAA_ERR_INVALID_ARG, "bwd: scale must be finite and > 0");
    if (mask != nullptr && (mask->kind < USP_MASK_FULL || mask->kind > USP_MASK_STRIPE))
        return fail(UAA_ERR_INVALID_ARG, "bwd: unknown mask kind %d", mask->kind);
    if (accumulate < 0 || accumulate > 3) return fail(UAA_ERR_INVALID_ARG, "bwd: accumulate must be in [0, 3]");
    if (D != 64 && D != 128) return fail(UAA_ERR_UNSUPPORTED, "bwd: D must be 64 or 128, got %lld", (long long)D);
    if ((double)B * (Sq > Sk ? Sq : Sk) * H * D > (double)kMaxElems) return fail(UAA_ERR_INVALID_ARG, "bwd: tensor too large");
    if (B == 0 || H == 0 || (Sq == 0 && Sk == 0)) return UAA_OK;
    if (Sq > 0 && (q == nullptr || dout == nullptr || lse == nullptr || delta == nullptr || dq == nullptr))
        return fail(UAA_ERR_INVALID_ARG, "bwd: q, dout, lse, delta and dq must not be NULL when Sq > 0");
    if (Sk > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
        return fail(UAA_ERR_INVALID_ARG, "bwd: k, v, dk and dv must not be NULL when Sk > 0");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
        !aligned(dk, 16) || !aligned(dv, 16))
        return fail(UAA_ERR_INVALID_ARG, "bwd: q, k, v, dout, dq, dk and dv must be 16-byte aligned");
    if (!aligned(lse, 4) || !aligned(delta, 4)) return fail(UAA_ERR_INVALID_ARG, "bwd: lse and delta must be 4-byte aligned");
    // 32-bit buffer offsets within one (batch) slab, with room for a tile past the end
    if ((double)((Sq > Sk ? Sq : Sk) + 256) * H * D * 2 >= 4294967296.0)
        return fail(UAA_ERR_UNSUPPORTED, "bwd: one batch of q or k/v must stay below 4 GiB");
    if (((Sk + 63) / 64) * H * B >= kMaxIdx32 || ((Sq + 63) / 64) * H * B >= kMaxIdx32)
        return fail(UAA_ERR_INVALID_ARG, "bwd: grid too large");

    uaa::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.delta = delta;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = B;
    a.H = H;
    a.Sq = Sq;
    a.Sk = Sk;
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    a.masked = 0;
    a.accumulate = accumulate;
    a.grad_bf16 = grad_dtype == UAA_BF16 ? 1 : 0;
    if (mask != nullptr && mask->kind != USP_MASK_FULL) {
        a.masked = 1;
        int rc = side_map(*mask, true, Sq, a.qmap);
        if (rc != UAA_OK) return rc;
        rc = side_map(*mask, false, Sk, a.kmap);
        if (rc != UAA_OK) return rc;
        if (all_pairs_allowed(a.qmap, Sq, a.kmap, Sk)) a.masked = 0;
    }
    const size_t need = bwd_ds_bytes(dtype, B, H, Sq, Sk, D, a.masked != 0);
    if (workspace != nullptr && need > 0 && workspace_bytes >= need) {
        if (!aligned(workspace, 16)) return fail(UAA_ERR_INVALID_ARG, "bwd: workspace must be 16-byte aligned");
        a.ds = workspace;
        a.ds_nq = (Sq + 31) / 32;
        a.ds_nk = (Sk + 15) / 16;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == UAA_BF16) return hip_status(uaa::launch_attn_bwd_bf16((int)D, a, s), "bwd launch");
    return hip_status(uaa::launch_attn_bwd_fp32((int)D, a, s), "bwd launch");
}

UAA_EXPORT int usp_attn_bwd(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, const void* q,
                            const void* k, const void* v, const void* dout, const float* lse, const float* delta,
                            void* dq, void* dk, void* dv, int grad_dtype, float scale, const usp_mask* mask,
                            int accumulate, void* stream)
{
    return attn_bwd_impl(dtype, B, H, Sq, Sk, D, q, k, v, dout, lse, delta, dq, dk, dv, grad_dtype, scale, mask,
                         accumulate, nullptr, 0, stream);
}

UAA_EXPORT size_t usp_attn_bwd_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                               const usp_mask* mask)
{
    bool masked = false;
    if (mask != nullptr && mask->kind != USP_MASK_FULL) {
        uaa::PosMap qm{}, km{};
        if (side_map(*mask, true, Sq, qm) != UAA_OK || side_map(*mask, false, Sk, km) != UAA_OK) return 0;
        masked = !all_pairs_allowed(qm, Sq, km, Sk);
    }
    return bwd_ds_bytes(dtype, B, H, Sq, Sk, D, masked);
}

UAA_EXPORT int usp_attn_bwd_ws(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, const void* q,
                               const void* k, const void* v, const void* dout, const float* lse, const float* delta,
                               void* dq, void* dk, void* dv, int grad_dtype, float scale, const usp_mask* mask,
                               int accumulate, void* workspace, size_t workspace_bytes, void* stream)
{
    return attn_bwd_impl(dtype, B, H, Sq, Sk, D, q, k, v, dout, lse, delta, dq, dk, dv, grad_dtype, scale, mask,
                         accumulate, workspace, workspace_bytes, stream);
}

// --------------------------------------------------------------------------
// Attention without allocation (usp_attn_fwd_lse_static): the key split's
// workspace is this file-scope device array, one copy per GPU, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (there
// it is a host-side stand-in): its device address is taken once per device
// with hipGetSymbolAddress, with that device current, and that pointer is
// what the kernels get.
// --------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[USP_STATIC_SCRATCH_BYTES];

namespace {

// n 32-bit words from p set to zero (a kernel, not a memset, so that a
// captured graph replays it faithfully)
__global__ void zero_words_kernel(uint32_t* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];   // device address of `scratch` per device, once known

int scratch_address(void** out)
{
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "static attn: hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(UAA_ERR_UNSUPPORTED, "static attn: device %d above the 64 this library tracks", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (g != hipSuccess) return hip_status(g, "static attn: hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(UAA_ERR_HIP, "static attn: scratch has no device address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return UAA_OK;
}

}  // namespace

static hipError_t clear_split_counters(const uaa::AttnArgs& a, hipStream_t s)
{
    const int64_t units = uaa::attn_bf16_units(a.B, a.H, a.Sq);   // both kernels' units are 256 rows
    const int64_t n_split = units - a.n_whole;
    if (n_split <= 0) return hipSuccess;
    uint32_t* cnt = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(a.ws) +
                                                uaa::split_counter_offset(n_split, a.split_p, a.split_p32 != 0));
    const unsigned blocks = (unsigned)std::min<int64_t>((n_split + 255) / 256, 64);
    void* params[] = {&cnt, const_cast<int64_t*>(&n_split)};
    return hipLaunchKernel(reinterpret_cast<const void*>(zero_words_kernel), dim3(blocks), dim3(256), params, 0, s);
}

UAA_EXPORT int usp_attn_fwd_lse_static(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                       const void* q, const void* k, const void* v, void* o, int o_dtype,
                                       float* lse, float scale, const usp_mask* mask, void* stream)
{
    // the workspace this problem's plan needs (0: it runs as the plain call)
    int kern = USP_KERNEL_NONE;
    int rc = attn_impl(dtype, B, H, Sq, Sk, D, q, k, v, o, o_dtype, lse, scale, mask, nullptr,
                       (size_t)USP_STATIC_SCRATCH_BYTES, 0, nullptr, stream, &kern);
    if (rc != UAA_OK) return rc;
    const int64_t need = plan_ws_bytes(attn_split_plan(dtype, B, H, Sq, Sk, D, mask), B, H, Sq);
    if (need > (int64_t)USP_STATIC_SCRATCH_BYTES)
        return fail(UAA_ERR_UNSUPPORTED, "static attn: the key split needs %lld bytes of scratch, the library holds %lld",
                    (long long)need, (long long)USP_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != UAA_OK) return rc;
    return attn_impl(dtype, B, H, Sq, Sk, D, q, k, v, o, o_dtype, lse, scale, mask, need > 0 ? ws : nullptr,
                     (size_t)USP_STATIC_SCRATCH_BYTES, 0, nullptr, stream, nullptr, true);
}
