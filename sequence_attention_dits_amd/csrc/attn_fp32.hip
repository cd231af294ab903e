// attn_fp32.hip -- fp32 attention forward with LSE (the full-precision path).
//
// Computes, for every query row, the (out, lse) pair each Ring step hands to
// the merge ("Add Unified Sequence Parallel attention", diffusers PR #12693,
// review thread; "Context parallelism" docs, "Ring Attention"), in fp32
// throughout: fp32 products and sums, no bf16 or reduced-precision matrix
// shortcut, and the accurate expf/logf, so it stays within 1e-5 of the exact
// result.  It is the correctness path for fp32 inputs, not a throughput path.
//
// A workgroup owns 64 query rows; four lanes share a row, each holding a
// quarter of the row's q and of its fp32 output accumulator, and a quad-lane
// reduction completes every dot product.  K and V tiles of 32 keys are staged
// in LDS; the four lanes of a row read consecutive 16-byte pieces of a key and
// all rows read the same key (broadcast).  The softmax is blockwise (online):
// per group of 8 keys the running maximum is raised once and the accumulator
// rescaled once.
#include "attn_common.h"

namespace uaa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void attn_fp32_kernel(const AttnArgs a)
{
    constexpr int BM = 64, BN = 32, TPR = 4;
    constexpr int NE = D / (4 * TPR);        // float4 pieces per lane
    __shared__ f32x4 Ks[BN][D / 4];
    __shared__ f32x4 Vs[BN][D / 4];

    int64_t qt, hh, b;
    decode_tile(a, qt, hh, b);
    const int tid = threadIdx.x;
    const int part = tid & (TPR - 1);
    const int64_t q0 = qt * BM;
    const int64_t i = q0 + (tid >> 2);
    const bool row_ok = i < a.Sq;
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const float scale = a.scale;

    const float* Q = static_cast<const float*>(a.q);
    const float* K = static_cast<const float*>(a.k);
    const float* V = static_cast<const float*>(a.v);

    // lane holds features 16*e + 4*part .. +3 for e < NE
    f32x4 q[NE], o[NE];
    const f32x4* qrow = reinterpret_cast<const f32x4*>(Q + ((b * Sq + (row_ok ? i : 0)) * H + hh) * D);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        q[e] = row_ok ? qrow[4 * e + part] : f32x4{0.f, 0.f, 0.f, 0.f};
        o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m = -INFINITY, l = 0.f;

    const int64_t q_hi = (q0 + BM < Sq ? q0 + BM : Sq);
    int64_t qmin = 0, qmax = 0;
    if (a.masked) pos_range(a.qmap, q0, q_hi, qmin, qmax);
    const int64_t qpos = a.masked ? pos_of(a.qmap, i) : 0;

    for (int64_t j0 = 0; j0 < Sk; j0 += BN) {
        const int jn = (int)(Sk - j0 < BN ? Sk - j0 : BN);
        if (a.masked) {
            int64_t kmin, kmax;
            pos_range(a.kmap, j0, j0 + jn, kmin, kmax);
            if (kmin > qmax) continue;               // no row of this tile sees these keys
        }
        __syncthreads();                             // previous tile fully read
        for (int e = tid; e < BN * (D / 4); e += 256) {
            const int jj = e / (D / 4), c = e % (D / 4);
            const bool ok = jj < jn;
            const int64_t off = ((b * Sk + j0 + (ok ? jj : 0)) * H + hh) * D;
            Ks[jj][c] = ok ? reinterpret_cast<const f32x4*>(K + off)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
            Vs[jj][c] = ok ? reinterpret_cast<const f32x4*>(V + off)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();

#pragma unroll 1
        for (int c0 = 0; c0 < BN; c0 += 8) {
            float s[8];
            float cmax = -INFINITY;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int jj = c0 + u;
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    const f32x4 k4 = Ks[jj][4 * e + part];
                    dot = fmaf(q[e][0], k4[0], dot);
                    dot = fmaf(q[e][1], k4[1], dot);
                    dot = fmaf(q[e][2], k4[2], dot);
                    dot = fmaf(q[e][3], k4[3], dot);
                }
                dot += __shfl_xor(dot, 1);
                dot += __shfl_xor(dot, 2);
                bool ok = jj < jn;
                if (a.masked && ok) ok = pos_of(a.kmap, j0 + jj) <= qpos;
                s[u] = ok ? dot * scale : -INFINITY;
                cmax = fmaxf(cmax, s[u]);
            }
            const float m_new = fmaxf(m, cmax);
            if (m_new == -INFINITY) continue;        // nothing allowed yet for this row
            const float alpha = expf(m - m_new);     // 0 when m was -inf
            l *= alpha;
#pragma unroll
            for (int e = 0; e < NE; ++e) o[e] *= alpha;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float p = expf(s[u] - m_new);
                l += p;
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    const f32x4 v4 = Vs[c0 + u][4 * e + part];
                    o[e][0] = fmaf(p, v4[0], o[e][0]);
                    o[e][1] = fmaf(p, v4[1], o[e][1]);
                    o[e][2] = fmaf(p, v4[2], o[e][2]);
                    o[e][3] = fmaf(p, v4[3], o[e][3]);
                }
            }
            m = m_new;
        }
    }

    if (!row_ok) return;
    f32x4* O = reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + ((b * Sq + i) * H + hh) * D);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float lse = l > 0.f ? m + logf(l) : -INFINITY;
    if (a.acc) {
        // continue a Ring pass: merge this block into the result already in
        // (o, lse), weights e^(lse_n - lse); a previous weight of 0 is not read
        const float lp = a.lse[(b * Sq + i) * H + hh];
        const float mm = fmaxf(lp, lse);
        float wp = 0.f, wb = 0.f;
        if (mm != -INFINITY) {
            const float ep = expf(lp - mm), eb = expf(lse - mm);
            wp = ep / (ep + eb);
            wb = eb / (ep + eb);
            lse = mm + logf(ep + eb);
        }
        const float sb = wb * inv;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            f32x4 x = o[e] * sb;
            if (wp != 0.f) {
                const f32x4 pv = O[4 * e + part];
                x[0] = fmaf(wp, pv[0], x[0]);
                x[1] = fmaf(wp, pv[1], x[1]);
                x[2] = fmaf(wp, pv[2], x[2]);
                x[3] = fmaf(wp, pv[3], x[3]);
            }
            O[4 * e + part] = x;
        }
    } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) O[4 * e + part] = o[e] * inv;
    }
    if (part == 0) a.lse[(b * Sq + i) * H + hh] = lse;
}

hipError_t launch_attn_fp32(int D, const AttnArgs& a0, hipStream_t s)
{
    AttnArgs a = a0;
    a.n_qtiles = (int32_t)((a.Sq + 63) / 64);
    const int64_t blocks = (int64_t)a.n_qtiles * a.H * a.B;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(256);
    if (D == 64) return launch_kernel(attn_fp32_kernel<64>, grid, block, 0, s, a);
    if (D == 128) return launch_kernel(attn_fp32_kernel<128>, grid, block, 0, s, a);
    return hipErrorInvalidValue;
}

}  // namespace uaa
