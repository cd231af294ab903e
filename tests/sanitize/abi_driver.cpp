// Host driver of libuaa's C ABI for an AddressSanitizer + UndefinedBehavior-
// Sanitizer build of the library's host code (test infrastructure, run by
// tests/test_host_sanitize.py, with no GPU): every entry point with valid
// and invalid arguments whose host arrays (offsets, pointer tables, mask,
// sizes) are allocated at exactly their documented lengths, so a read past
// an end in the validation or argument building is reported.  Device
// pointers are stand-ins that nothing on the host dereferences; calls that
// pass validation reach the launch, which fails without a GPU
// (UAA_ERR_HIP) -- both that and UAA_OK count as accepted.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "uaa.h"

static int failures = 0;

static void expect(bool ok, const char* what, int rc)
{
    if (!ok) {
        fprintf(stderr, "FAILED %s: rc %d (%s)\n", what, rc, uaa_last_error());
        ++failures;
    }
}
static void accepted(int rc, const char* what) { expect(rc == UAA_OK || rc == UAA_ERR_HIP, what, rc); }
static void rejected(int rc, int code, const char* what) { expect(rc == code, what, rc); }

template <typename T> static T* exact(std::initializer_list<T> v)
{
    T* p = static_cast<T*>(malloc(sizeof(T) * v.size()));
    size_t i = 0;
    for (const T& x : v) p[i++] = x;
    return p;
}

static void* dptr(uintptr_t i) { return reinterpret_cast<void*>(0x10000000u + 256u * i); }

static void permutes()
{
    int64_t* so = exact<int64_t>({0, 100, 100, 161});   // three token shards, one empty
    int64_t* ho = exact<int64_t>({0, 2, 4, 5});         // five heads: 2 / 2 / 1
    const void** src = static_cast<const void**>(malloc(sizeof(void*) * 3));
    for (int i = 0; i < 3; ++i) src[i] = dptr(i);
    for (int r = 0; r < 3; ++r) {
        accepted(uaa_seq2head_permute(UAA_SEQ2HEAD, r, 3, so, ho, 2, 5, 64, 2, src, dptr(9), nullptr), "s2h");
        accepted(uaa_seq2head_permute(UAA_HEAD2SEQ, r, 3, so, ho, 2, 5, 64, 2, src, dptr(9), nullptr), "h2s");
        accepted(uaa_seq2head_permute(UAA_SEQ2HEAD, r, 3, so, nullptr, 2, 5, 1, 4, src, dptr(9), nullptr),
                 "s2h default heads");
    }
    rejected(uaa_seq2head_permute(UAA_SEQ2HEAD, 3, 3, so, ho, 2, 5, 64, 2, src, dptr(9), nullptr),
             UAA_ERR_INVALID_ARG, "rank");
    int64_t* bad = exact<int64_t>({0, 100, 90, 161});
    rejected(uaa_seq2head_permute(UAA_SEQ2HEAD, 0, 3, bad, ho, 2, 5, 64, 2, src, dptr(9), nullptr),
             UAA_ERR_INVALID_ARG, "decreasing");
    int64_t* hbad = exact<int64_t>({0, 2, 4, 6});
    rejected(uaa_seq2head_permute(UAA_SEQ2HEAD, 0, 3, so, hbad, 2, 5, 64, 2, src, dptr(9), nullptr),
             UAA_ERR_INVALID_ARG, "head_off end");
    // multi: 3 tensors x 3 shards, and mixed widths (O and its LSE)
    const void** msrc = static_cast<const void**>(malloc(sizeof(void*) * 9));
    for (int i = 0; i < 9; ++i) msrc[i] = dptr(10 + i);
    void** mdst = static_cast<void**>(malloc(sizeof(void*) * 3));
    for (int i = 0; i < 3; ++i) mdst[i] = dptr(30 + i);
    accepted(uaa_seq2head_permute_multi(3, UAA_SEQ2HEAD, 1, 3, so, ho, 1, 5, 128, 2, msrc, mdst, nullptr), "multi");
    rejected(uaa_seq2head_permute_multi(5, UAA_SEQ2HEAD, 1, 3, so, ho, 1, 5, 128, 2, msrc, mdst, nullptr),
             UAA_ERR_INVALID_ARG, "multi count");
    int64_t* Ds = exact<int64_t>({128, 1});
    int* eb = exact<int>({2, 4});
    accepted(uaa_seq2head_permute_multi_ex(2, UAA_HEAD2SEQ, 0, 3, so, nullptr, 1, 5, Ds, eb, msrc, mdst, nullptr),
             "multi_ex");
    free(so); free(ho); free(src); free(bad); free(hbad); free(msrc); free(mdst); free(Ds); free(eb);
}

static void attention()
{
    usp_mask* m = static_cast<usp_mask*>(malloc(sizeof(usp_mask)));
    memset(m, 0, sizeof(*m));
    const int kinds[4] = {USP_MASK_FULL, USP_MASK_CAUSAL, USP_MASK_ZIGZAG, USP_MASK_STRIPE};
    for (int kk = 0; kk < 4; ++kk) {
        memset(m, 0, sizeof(*m));
        m->kind = kinds[kk];
        m->q_off = 300;
        m->chunk = 512;
        m->q_chunks[0] = 1;
        m->q_chunks[1] = 6;
        m->k_chunks[0] = 1;
        m->k_chunks[1] = -1;
        m->world = 4;
        m->q_rank = 1;
        m->k_rank = 2;
        for (int D : {64, 128})
            for (int dt : {UAA_BF16, UAA_FP32}) {
                accepted(usp_attn_fwd_lse(dt, 2, 3, 1000, 512, D, dptr(1), dptr(2), dptr(3), dptr(4), UAA_FP32,
                                          static_cast<float*>(dptr(5)), 0.1f, m, nullptr), "attn");
                const int kq = usp_attn_kernel(dt, 2, 3, 1000, 512, D, UAA_FP32, m, 0);
                expect(kq >= USP_KERNEL_NONE && kq <= USP_KERNEL_PIPELINED_DIAG, "kernel query", kq);
            }
    }
    m->kind = USP_MASK_FULL;
    rejected(usp_attn_fwd_lse(UAA_BF16, 1, 1, 4, 4, 96, dptr(1), dptr(2), dptr(3), dptr(4), UAA_BF16,
                              static_cast<float*>(dptr(5)), 0.1f, m, nullptr), UAA_ERR_UNSUPPORTED, "D");
    rejected(usp_attn_fwd_lse(UAA_BF16, 1, 1, 4, 4, 128, nullptr, dptr(2), dptr(3), dptr(4), UAA_BF16,
                              static_cast<float*>(dptr(5)), 0.1f, m, nullptr), UAA_ERR_INVALID_ARG, "null q");
    // workspace sizes and the split's plan (no GPU: 0 compute units, no split)
    const size_t wsb = usp_attn_workspace_bytes(UAA_BF16, 1, 24, 3493, 3493, 128, m);
    accepted(usp_attn_fwd_lse_ws(UAA_BF16, 1, 24, 3493, 3493, 128, dptr(1), dptr(2), dptr(3), dptr(4), UAA_BF16,
                                 static_cast<float*>(dptr(5)), 0.1f, m, dptr(6), wsb, nullptr), "ws");
    accepted(usp_attn_fwd_lse_acc(UAA_BF16, 1, 24, 3493, 3493, 128, dptr(1), dptr(2), dptr(3), dptr(4), UAA_BF16,
                                  static_cast<float*>(dptr(5)), 0.1f, m, nullptr, 0, nullptr), "acc");
    accepted(usp_attn_fwd_lse_static(UAA_BF16, 1, 24, 3493, 3493, 128, dptr(1), dptr(2), dptr(3), dptr(4),
                                     UAA_BF16, static_cast<float*>(dptr(5)), 0.1f, m, nullptr), "static");
    // gathering attention: 3 token shards, one empty
    int64_t* so = exact<int64_t>({0, 100, 100, 161});
    const void** qs = static_cast<const void**>(malloc(sizeof(void*) * 3));
    const void** ks = static_cast<const void**>(malloc(sizeof(void*) * 3));
    const void** vs = static_cast<const void**>(malloc(sizeof(void*) * 3));
    for (int i = 0; i < 3; ++i) {
        qs[i] = dptr(40 + i);
        ks[i] = dptr(50 + i);
        vs[i] = dptr(60 + i);
    }
    for (int r = 0; r < 3; ++r)
        for (int s = 0; s < 3; ++s)
            accepted(usp_attn_fwd_lse_gather(UAA_BF16, 3, r, so, nullptr, 1, 5, 128, qs, ks, vs, s, dptr(7), UAA_BF16,
                                             static_cast<float*>(dptr(8)), 0.1f, m, nullptr, 0, s > 0, nullptr),
                     "gather");
    rejected(usp_attn_fwd_lse_gather(UAA_BF16, 3, 0, so, nullptr, 1, 5, 128, qs, ks, vs, 3, dptr(7), UAA_BF16,
                                     static_cast<float*>(dptr(8)), 0.1f, m, nullptr, 0, 0, nullptr),
             UAA_ERR_INVALID_ARG, "gather k_shard");
    free(so); free(qs); free(ks); free(vs); free(m);
}

static void merges_and_backward()
{
    for (int n = 1; n <= USP_MAX_PARTS; ++n) {
        const void** op = static_cast<const void**>(malloc(sizeof(void*) * n));
        const float** lp = static_cast<const float**>(malloc(sizeof(float*) * n));
        for (int i = 0; i < n; ++i) {
            op[i] = dptr(70 + i);
            lp[i] = static_cast<const float*>(dptr(90 + i));
        }
        accepted(usp_lse_merge(n, 1, 37, 3, 130, op, UAA_BF16, lp, dptr(120), UAA_FP32,
                               static_cast<float*>(dptr(121)), nullptr), "merge");
        free(op);
        free(lp);
    }
    rejected(usp_lse_merge(0, 1, 37, 3, 130, nullptr, UAA_BF16, nullptr, dptr(120), UAA_FP32,
                           static_cast<float*>(dptr(121)), nullptr), UAA_ERR_INVALID_ARG, "merge n");
    accepted(usp_attn_bwd_delta(UAA_BF16, 1, 300, 2, 128, dptr(1), dptr(2), nullptr, static_cast<float*>(dptr(3)),
                                nullptr), "delta");
    usp_mask* m = static_cast<usp_mask*>(malloc(sizeof(usp_mask)));
    memset(m, 0, sizeof(*m));
    m->kind = USP_MASK_CAUSAL;
    accepted(usp_attn_bwd(UAA_BF16, 1, 2, 300, 250, 128, dptr(1), dptr(2), dptr(3), dptr(4),
                          static_cast<const float*>(dptr(5)), static_cast<const float*>(dptr(6)), dptr(7), dptr(8),
                          dptr(9), UAA_FP32, 0.1f, m, 3, nullptr), "bwd");
    rejected(usp_attn_bwd(UAA_BF16, 1, 2, 300, 250, 128, dptr(1), dptr(2), dptr(3), dptr(4),
                          static_cast<const float*>(dptr(5)), static_cast<const float*>(dptr(6)), dptr(7), dptr(8),
                          dptr(9), UAA_FP32, 0.1f, m, 4, nullptr), UAA_ERR_INVALID_ARG, "bwd accumulate");
    // the dS workspace: sizes where it applies and 0 where it does not; a
    // workspace call (the plain one without it), and a misaligned one
    {
        const size_t n = usp_attn_bwd_workspace_bytes(UAA_BF16, 1, 2, 300, 250, 128, nullptr);
        expect(n == (size_t)2 * 10 * 16 * 1024, "bwd ws bytes", (int)(n / 1024));
        expect(usp_attn_bwd_workspace_bytes(UAA_BF16, 1, 2, 300, 250, 128, m) == 0, "bwd ws masked", 0);
        expect(usp_attn_bwd_workspace_bytes(UAA_FP32, 1, 2, 300, 250, 128, nullptr) == 0, "bwd ws fp32", 0);
        expect(usp_attn_bwd_workspace_bytes(UAA_BF16, 1, 2, 300, 250, 64, nullptr) == 0, "bwd ws d64", 0);
        accepted(usp_attn_bwd_ws(UAA_BF16, 1, 2, 300, 250, 128, dptr(1), dptr(2), dptr(3), dptr(4),
                                 static_cast<const float*>(dptr(5)), static_cast<const float*>(dptr(6)), dptr(7),
                                 dptr(8), dptr(9), UAA_FP32, 0.1f, nullptr, 1, dptr(10), n, nullptr),
                 "bwd ws");
        rejected(usp_attn_bwd_ws(UAA_BF16, 1, 2, 300, 250, 128, dptr(1), dptr(2), dptr(3), dptr(4),
                                 static_cast<const float*>(dptr(5)), static_cast<const float*>(dptr(6)), dptr(7),
                                 dptr(8), dptr(9), UAA_FP32, 0.1f, nullptr, 1,
                                 static_cast<unsigned char*>(dptr(10)) + 4, n, nullptr),
                 UAA_ERR_INVALID_ARG, "bwd ws misaligned");
    }
    free(m);
    int64_t* off = static_cast<int64_t*>(malloc(sizeof(int64_t) * 8));
    accepted(uaa_split_offsets(4481, 7, off), "split");
    expect(off[7] == 4481 && off[1] == 641, "split values", (int)off[1]);
    free(off);
    expect(strlen(uaa_build_id()) > 0 && uaa_abi_version() == 1, "ids", 0);
}

int main()
{
    permutes();
    attention();
    merges_and_backward();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("abi host checks ok\n");
    return 0;
}
