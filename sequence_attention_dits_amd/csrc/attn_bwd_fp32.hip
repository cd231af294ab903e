// attn_bwd_fp32.hip -- fp32 attention backward (the full-precision path).
//
// The gradients of one attention call from the rows' final LSE, as the bf16
// kernels compute them ("Add Unified Sequence Parallel attention", diffusers
// PR #12693, conversation: the Unified / Ring attention has a backward of its
// forward), in fp32 throughout with the accurate expf: the correctness path
// for fp32 inputs, not a throughput path.  Per allowed (i, j):
//   P = exp(scale <q_i, k_j> - lse_i),  dS = P (<dO_i, v_j> - delta_i)
//   dq_i += scale dS k_j,  dk_j += scale dS q_i,  dv_j += P dO_i.
//
// Layout as in the fp32 forward: four lanes share a row (a query row in the
// dQ kernel, a key in the dK/dV kernel), each holding a quarter of the row's
// vectors and accumulators, with a quad-lane reduction per dot product; the
// other side streams through LDS in tiles of 32 rows read by every lane group
// at once (broadcast).
#include "attn_common.h"

namespace uaa {

typedef float bf_f32x4 __attribute__((ext_vector_type(4)));

// probability of (row with lse l, score s); 0 for a row with no key
__device__ __forceinline__ float bwd32_prob(float s, float l) { return l == -INFINITY ? 0.f : expf(s - l); }

template <int D>
__device__ __forceinline__ void bwd32_store(void* out, int grad_bf16, int acc_bit, int64_t row_off, int part,
                                            const bf_f32x4 (&x)[D / 16], float mul)
{
    constexpr int NE = D / 16;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        bf_f32x4 w = x[e] * mul;
        const int f = 16 * e + 4 * part;
        if (grad_bf16) {
            unsigned short* p = static_cast<unsigned short*>(out) + row_off + f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float v = w[c];
                if (acc_bit) v += __uint_as_float((unsigned int)p[c] << 16);
                // round to nearest even
                const unsigned int u = __float_as_uint(v);
                p[c] = (unsigned short)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
            }
        } else {
            bf_f32x4* p = reinterpret_cast<bf_f32x4*>(static_cast<float*>(out) + row_off + f);
            if (acc_bit) w += *p;
            *p = w;
        }
    }
}

// ---- dQ: a workgroup owns 64 query rows -----------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_fp32_dq_kernel(const BwdArgs a)
{
    constexpr int BM = 64, BN = 32, TPR = 4, NE = D / 16;
    __shared__ bf_f32x4 Ks[BN][D / 4];
    __shared__ bf_f32x4 Vs[BN][D / 4];

    const uint32_t unit = blockIdx.x;
    const int64_t qt = unit % (uint32_t)a.n_tiles;
    const int64_t rest = unit / (uint32_t)a.n_tiles;
    const int64_t hh = rest % a.H, b = rest / a.H;
    const int tid = threadIdx.x, part = tid & (TPR - 1);
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const int64_t q0 = qt * BM, i = q0 + (tid >> 2);
    const bool row_ok = i < Sq;
    const float* Q = static_cast<const float*>(a.q);
    const float* G = static_cast<const float*>(a.dout);
    const float* K = static_cast<const float*>(a.k);
    const float* V = static_cast<const float*>(a.v);

    // lane holds features 16 e + 4 part .. +3
    bf_f32x4 q[NE], g[NE], dq[NE];
    const int64_t roff = ((b * Sq + (row_ok ? i : 0)) * H + hh) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        q[e] = row_ok ? reinterpret_cast<const bf_f32x4*>(Q + roff)[4 * e + part] : bf_f32x4{0.f, 0.f, 0.f, 0.f};
        g[e] = row_ok ? reinterpret_cast<const bf_f32x4*>(G + roff)[4 * e + part] : bf_f32x4{0.f, 0.f, 0.f, 0.f};
        dq[e] = bf_f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float lse = row_ok ? a.lse[(b * Sq + i) * H + hh] : -INFINITY;
    const float dlt = row_ok ? a.delta[(b * Sq + i) * H + hh] : 0.f;
    const int64_t qpos = a.masked ? pos_of(a.qmap, i) : 0;
    int64_t qmin = 0, qmax = 0;
    if (a.masked) pos_range(a.qmap, q0, q0 + BM < Sq ? q0 + BM : Sq, qmin, qmax);

    for (int64_t j0 = 0; j0 < Sk; j0 += BN) {
        const int jn = (int)(Sk - j0 < BN ? Sk - j0 : BN);
        if (a.masked) {
            int64_t kmin, kmax;
            pos_range(a.kmap, j0, j0 + jn, kmin, kmax);
            if (kmin > qmax) continue;               // no row of this tile sees these keys
        }
        __syncthreads();
        for (int e = tid; e < BN * (D / 4); e += 256) {
            const int jj = e / (D / 4), c = e % (D / 4);
            const bool ok = jj < jn;
            const int64_t off = ((b * Sk + j0 + (ok ? jj : 0)) * H + hh) * D;
            Ks[jj][c] = ok ? reinterpret_cast<const bf_f32x4*>(K + off)[c] : bf_f32x4{0.f, 0.f, 0.f, 0.f};
            Vs[jj][c] = ok ? reinterpret_cast<const bf_f32x4*>(V + off)[c] : bf_f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        for (int jj = 0; jj < jn; ++jj) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const bf_f32x4 k4 = Ks[jj][4 * e + part], v4 = Vs[jj][4 * e + part];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    s = fmaf(q[e][c], k4[c], s);
                    dp = fmaf(g[e][c], v4[c], dp);
                }
            }
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            dp += __shfl_xor(dp, 1);
            dp += __shfl_xor(dp, 2);
            bool ok = true;
            if (a.masked) ok = pos_of(a.kmap, j0 + jj) <= qpos;
            const float p = ok ? bwd32_prob(s * a.scale, lse) : 0.f;
            const float ds = p * (dp - dlt);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const bf_f32x4 k4 = Ks[jj][4 * e + part];
#pragma unroll
                for (int c = 0; c < 4; ++c) dq[e][c] = fmaf(ds, k4[c], dq[e][c]);
            }
        }
    }
    if (!row_ok) return;
    bwd32_store<D>(a.dq, a.grad_bf16, a.accumulate & 1, ((b * Sq + i) * H + hh) * D, part, dq, a.scale);
}

// ---- dK / dV: a workgroup owns 64 keys ------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_fp32_dkdv_kernel(const BwdArgs a)
{
    constexpr int BM = 64, BN = 32, TPR = 4, NE = D / 16;
    __shared__ bf_f32x4 Qs[BN][D / 4];
    __shared__ bf_f32x4 Gs[BN][D / 4];
    __shared__ float Ls[BN], Ds[BN];

    const uint32_t unit = blockIdx.x;
    const int64_t kt = unit % (uint32_t)a.n_tiles;
    const int64_t rest = unit / (uint32_t)a.n_tiles;
    const int64_t hh = rest % a.H, b = rest / a.H;
    const int tid = threadIdx.x, part = tid & (TPR - 1);
    const int64_t H = a.H, Sq = a.Sq, Sk = a.Sk;
    const int64_t k0 = kt * BM, j = k0 + (tid >> 2);
    const bool key_ok = j < Sk;
    const float* Q = static_cast<const float*>(a.q);
    const float* G = static_cast<const float*>(a.dout);
    const float* K = static_cast<const float*>(a.k);
    const float* V = static_cast<const float*>(a.v);

    bf_f32x4 k[NE], v[NE], dk[NE], dv[NE];
    const int64_t koff = ((b * Sk + (key_ok ? j : 0)) * H + hh) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        k[e] = key_ok ? reinterpret_cast<const bf_f32x4*>(K + koff)[4 * e + part] : bf_f32x4{0.f, 0.f, 0.f, 0.f};
        v[e] = key_ok ? reinterpret_cast<const bf_f32x4*>(V + koff)[4 * e + part] : bf_f32x4{0.f, 0.f, 0.f, 0.f};
        dk[e] = bf_f32x4{0.f, 0.f, 0.f, 0.f};
        dv[e] = bf_f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int64_t kpos = a.masked ? pos_of(a.kmap, j) : 0;
    int64_t kmin = 0, kmax = 0;
    if (a.masked) pos_range(a.kmap, k0, k0 + BM < Sk ? k0 + BM : Sk, kmin, kmax);

    for (int64_t i0 = 0; i0 < Sq; i0 += BN) {
        const int in = (int)(Sq - i0 < BN ? Sq - i0 : BN);
        if (a.masked) {
            int64_t qmin, qmax;
            pos_range(a.qmap, i0, i0 + in, qmin, qmax);
            if (kmin > qmax) continue;               // no key of the workgroup is seen by these rows
        }
        __syncthreads();
        for (int e = tid; e < BN * (D / 4); e += 256) {
            const int ii = e / (D / 4), c = e % (D / 4);
            const bool ok = ii < in;
            const int64_t off = ((b * Sq + i0 + (ok ? ii : 0)) * H + hh) * D;
            Qs[ii][c] = ok ? reinterpret_cast<const bf_f32x4*>(Q + off)[c] : bf_f32x4{0.f, 0.f, 0.f, 0.f};
            Gs[ii][c] = ok ? reinterpret_cast<const bf_f32x4*>(G + off)[c] : bf_f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (tid < BN) {
            const bool ok = tid < in;
            const int64_t r = (b * Sq + i0 + (ok ? tid : 0)) * H + hh;
            Ls[tid] = ok ? a.lse[r] : -INFINITY;
            Ds[tid] = ok ? a.delta[r] : 0.f;
        }
        __syncthreads();
        for (int ii = 0; ii < in; ++ii) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const bf_f32x4 q4 = Qs[ii][4 * e + part], g4 = Gs[ii][4 * e + part];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    s = fmaf(q4[c], k[e][c], s);
                    dp = fmaf(g4[c], v[e][c], dp);
                }
            }
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            dp += __shfl_xor(dp, 1);
            dp += __shfl_xor(dp, 2);
            bool ok = true;
            if (a.masked) ok = kpos <= pos_of(a.qmap, i0 + ii);
            const float p = ok ? bwd32_prob(s * a.scale, Ls[ii]) : 0.f;
            const float ds = p * (dp - Ds[ii]);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const bf_f32x4 q4 = Qs[ii][4 * e + part], g4 = Gs[ii][4 * e + part];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    dk[e][c] = fmaf(ds, q4[c], dk[e][c]);
                    dv[e][c] = fmaf(p, g4[c], dv[e][c]);
                }
            }
        }
    }
    if (!key_ok) return;
    const int64_t ooff = ((b * Sk + j) * H + hh) * D;
    bwd32_store<D>(a.dk, a.grad_bf16, a.accumulate & 2, ooff, part, dk, a.scale);
    bwd32_store<D>(a.dv, a.grad_bf16, a.accumulate & 2, ooff, part, dv, 1.f);
}

template <int D>
static hipError_t launch_bwd32_d(const BwdArgs& a0, hipStream_t s)
{
    if (a0.Sk > 0 && !(a0.Sq == 0 && (a0.accumulate & 2))) {
        BwdArgs a = a0;
        a.n_tiles = (int32_t)((a.Sk + 63) / 64);
        const hipError_t e =
            launch_kernel(attn_bwd_fp32_dkdv_kernel<D>, dim3((uint32_t)(a.B * a.H * a.n_tiles)), dim3(256), 0, s, a);
        if (e != hipSuccess) return e;
    }
    if (a0.Sq == 0) return hipSuccess;
    BwdArgs a = a0;
    a.n_tiles = (int32_t)((a.Sq + 63) / 64);
    return launch_kernel(attn_bwd_fp32_dq_kernel<D>, dim3((uint32_t)(a.B * a.H * a.n_tiles)), dim3(256), 0, s, a);
}

hipError_t launch_attn_bwd_fp32(int D, const BwdArgs& a, hipStream_t s)
{
    if (a.B * a.H == 0 || (a.Sq == 0 && a.Sk == 0)) return hipSuccess;
    if (D == 128) return launch_bwd32_d<128>(a, s);
    return launch_bwd32_d<64>(a, s);
}

}  // namespace uaa
