/*
 * oracle.c -- plain fp64 CPU oracle for one rank's share of context-parallel
 * attention (Ulysses, Ulysses Anything, Ring, Unified).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no source, header, table or
 * helper with the HIP library in sequence_attention_dits_amd/csrc, and the
 * HIP library never calls it.
 *
 * Arithmetic: IEEE binary64 throughout, host libm exp()/log(), built with
 * -ffp-contract=off and without -ffast-math, so every product and sum is
 * rounded exactly where the C source says.  Every loop runs in the order the
 * definition is written: feature index d ascending inside a dot product, key
 * index j ascending inside a softmax sum, partial index n ascending inside a
 * merge.  The order does not depend on how heads or tokens are laid out, so
 * the same (row, head) gives the same bits whatever shard it sits in.
 *
 * Pages cited:
 *   [CP]   "Context parallelism" (diffusers documentation), sections
 *          "Ring Attention", "Ulysses Attention", "Unified Attention",
 *          "Ulysses Anything Attention".
 *   [USP]  "Add Unified Sequence Parallel attention" (diffusers pull request
 *          #12693), review thread: the Ring loop's fp32 merge of (out, lse)
 *          pairs and the (B, S, H_LOCAL) LSE layout of the Unified path.
 *   [UAA]  "UAA: Ulysses Anything Attention" (diffusers issue #12706):
 *          arbitrary sequence length with no padding, per-rank seq_len.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD (-1)

/* ------------------------------------------------------------------ */
/* Shard lookup shared by the two permute directions: the shard that    */
/* owns index x is the LAST p with off[p] <= x.  With zero-length       */
/* shards several p share one offset; the last of them is the one whose */
/* range [off[p], off[p+1]) actually contains x.                        */
/* ------------------------------------------------------------------ */
static int owner_of(int64_t x, int world, const int64_t* off)
{
    int p = 0;
    for (int c = 0; c < world; ++c)
        if (off[c] <= x) p = c;
    return p;
}

static int offsets_ok(int world, const int64_t* off)
{
    if (off[0] != 0) return 0;
    for (int p = 0; p < world; ++p)
        if (off[p + 1] < off[p]) return 0;
    return 1;
}

/*
 * Ulysses first all-to-all, seen from head-rank r ([CP] "Ulysses Attention":
 * after the exchange each GPU holds every token for a subset of the heads;
 * [UAA]/[CP] "Ulysses Anything Attention": token counts per rank arbitrary,
 * no padding, so shard p holds tokens [seq_off[p], seq_off[p+1])).
 *
 *   Y_r[b, s, h, d] = X_p[b, s - seq_off[p], head_off[r] + h, d],
 *   p = owner of s,   X_p : [B, S_p, H, D],   Y_r : [B, S, H_r, D].
 *
 * Elements are copied as opaque elem_bytes-wide words.
 */
int orc_seq2head(int rank, int world, const int64_t* seq_off, const int64_t* head_off,
                 int64_t B, int64_t H, int64_t D, int elem_bytes,
                 const void* const* src, void* dst)
{
    if (world < 1 || rank < 0 || rank >= world) return ORC_BAD;
    if (!offsets_ok(world, seq_off) || !offsets_ok(world, head_off)) return ORC_BAD;
    if (head_off[world] != H) return ORC_BAD;
    const int64_t S = seq_off[world];
    const int64_t h0 = head_off[rank];
    const int64_t Hr = head_off[rank + 1] - head_off[rank];
    unsigned char* out = (unsigned char*)dst;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s) {
            const int p = owner_of(s, world, seq_off);
            const int64_t Sp = seq_off[p + 1] - seq_off[p];
            const int64_t t = s - seq_off[p];
            const unsigned char* in = (const unsigned char*)src[p];
            for (int64_t h = 0; h < Hr; ++h)
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t di = ((b * S + s) * Hr + h) * D + d;
                    const int64_t si = ((b * Sp + t) * H + (h0 + h)) * D + d;
                    memcpy(out + di * elem_bytes, in + si * elem_bytes, (size_t)elem_bytes);
                }
        }
    return ORC_OK;
}

/*
 * Ulysses second all-to-all, seen from seq-rank p ([CP] "Ulysses Attention":
 * a second all-to-all regroups the results by token).  Also moves the LSE of
 * the Unified path ([USP]: LSE exchanged as (B, S, H_LOCAL, 1)), as D = 1.
 *
 *   Z_p[b, t, h, d] = Y_r[b, seq_off[p] + t, h - head_off[r], d],
 *   r = owner of h,   Y_r : [B, S, H_r, D],   Z_p : [B, S_p, H, D].
 */
int orc_head2seq(int rank, int world, const int64_t* seq_off, const int64_t* head_off,
                 int64_t B, int64_t H, int64_t D, int elem_bytes,
                 const void* const* src, void* dst)
{
    if (world < 1 || rank < 0 || rank >= world) return ORC_BAD;
    if (!offsets_ok(world, seq_off) || !offsets_ok(world, head_off)) return ORC_BAD;
    if (head_off[world] != H) return ORC_BAD;
    const int64_t S = seq_off[world];
    const int64_t Sp = seq_off[rank + 1] - seq_off[rank];
    unsigned char* out = (unsigned char*)dst;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < Sp; ++t)
            for (int64_t h = 0; h < H; ++h) {
                const int r = owner_of(h, world, head_off);
                const int64_t Hr = head_off[r + 1] - head_off[r];
                const unsigned char* in = (const unsigned char*)src[r];
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t di = ((b * Sp + t) * H + h) * D + d;
                    const int64_t si = ((b * S + seq_off[rank] + t) * Hr + (h - head_off[r])) * D + d;
                    memcpy(out + di * elem_bytes, in + si * elem_bytes, (size_t)elem_bytes);
                }
            }
    return ORC_OK;
}

/*
 * The seq2head index map itself: for every destination element (in the
 * destination's flat order) the source shard and the flat element index
 * inside that shard.  Used to check a device permute on index-coded input.
 */
int orc_seq2head_index(int rank, int world, const int64_t* seq_off, const int64_t* head_off,
                       int64_t B, int64_t H, int64_t D, int64_t* src_shard, int64_t* src_elem)
{
    if (world < 1 || rank < 0 || rank >= world) return ORC_BAD;
    if (!offsets_ok(world, seq_off) || !offsets_ok(world, head_off)) return ORC_BAD;
    const int64_t S = seq_off[world];
    const int64_t h0 = head_off[rank];
    const int64_t Hr = head_off[rank + 1] - head_off[rank];
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s) {
            const int p = owner_of(s, world, seq_off);
            const int64_t Sp = seq_off[p + 1] - seq_off[p];
            const int64_t t = s - seq_off[p];
            for (int64_t h = 0; h < Hr; ++h)
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t di = ((b * S + s) * Hr + h) * D + d;
                    src_shard[di] = p;
                    src_elem[di] = ((b * Sp + t) * H + (h0 + h)) * D + d;
                }
        }
    return ORC_OK;
}

/*
 * Softmax attention with its log-sum-exp, row by row, by definition.
 * This is the (out, lse) pair every per-rank attention call hands to the
 * Ring loop ([USP] review thread; [CP] "Ring Attention": each GPU computes
 * attention against the K/V block it holds).
 *
 * For batch b, head h and query token i, with J the allowed keys
 * (all keys, or the keys with kpos[j] <= qpos[i] when causal != 0):
 *     s_j  = scale * sum_d q[i,d] * k[j,d]
 *     m    = max_{j in J} s_j
 *     l    = sum_{j in J} exp(s_j - m)
 *     O[d] = (sum_{j in J} exp(s_j - m) * v[j,d]) / l
 *     LSE  = m + log(l)            (natural log)
 * and O = 0, LSE = -inf when J is empty.
 *
 * Layouts (contiguous, row-major): q [B,Sq,H,D], k and v [B,Sk,H,D],
 * qpos [Sq], kpos [Sk] (global token positions, same for every batch).
 * rows[0..n_rows) lists flat query tokens b*Sq + i to evaluate; the results
 * go to o [n_rows, H, D] and lse [n_rows, H] in that list order.
 */
int orc_attention(int64_t B, int64_t Sq, int64_t Sk, int64_t H, int64_t D,
                  const double* q, const double* k, const double* v,
                  const int64_t* qpos, const int64_t* kpos, int causal, double scale,
                  const int64_t* rows, int64_t n_rows, double* o, double* lse)
{
    if (B < 0 || Sq < 0 || Sk < 0 || H < 0 || D < 1 || n_rows < 0) return ORC_BAD;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= B * Sq) return ORC_BAD;
    if (causal && (qpos == NULL || kpos == NULL)) return ORC_BAD;

    const int64_t tasks = n_rows * H;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 16)
        for (int64_t task = 0; task < tasks; ++task) {
            const int64_t r = task / H, h = task % H;
            const int64_t b = rows[r] / Sq, i = rows[r] % Sq;
            const double* qi = q + ((b * Sq + i) * H + h) * D;
            double* oi = o + (r * H + h) * D;

            /* scores of the allowed keys, and their maximum */
            int64_t count = 0;
            double m = -INFINITY;
            for (int64_t j = 0; j < Sk; ++j) {
                if (causal && !(kpos[j] <= qpos[i])) continue;
                const double* kj = k + ((b * Sk + j) * H + h) * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += qi[d] * kj[d];
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
                ++count;
            }
            if (count == 0) {
                for (int64_t d = 0; d < D; ++d) oi[d] = 0.0;
                lse[r * H + h] = -INFINITY;
                continue;
            }

            /* normaliser and weighted sum of values, keys ascending */
            double l = 0.0;
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t j = 0; j < Sk; ++j) {
                if (causal && !(kpos[j] <= qpos[i])) continue;
                const double w = exp(s[j] - m);
                const double* vj = v + ((b * Sk + j) * H + h) * D;
                l += w;
                for (int64_t d = 0; d < D; ++d) acc[d] += w * vj[d];
            }
            for (int64_t d = 0; d < D; ++d) oi[d] = acc[d] / l;
            lse[r * H + h] = m + log(l);
        }
        free(acc);
        free(s);
    }
    return ORC_OK;
}

/*
 * Merge of N partial (O, LSE) pairs of the same query rows, each computed
 * over a disjoint set of keys ([USP] review thread: the Ring loop folds each
 * step's (out, lse) into the running pair, in fp32).  Each such pairwise
 * update weights the running output and the new one by the logistic
 * function of their LSE difference, and sets the LSE to the log of the sum
 * of the two exponentials: for finite inputs, the softmax-weighted mean of
 * the partials with lse = log(exp(prev_lse) + exp(lse)).  Written out for N
 * partials, with the
 * maximum shifted out so that -inf partials (rows with no allowed key) add
 * nothing instead of producing NaN:
 *     M   = max_n LSE_n
 *     L   = M + log(sum_n exp(LSE_n - M))
 *     O   = sum_n exp(LSE_n - L) * O_n
 * and (O, L) = (0, -inf) when every LSE_n is -inf.
 *
 * o_parts[n] : [rows, D], lse_parts[n] : [rows]; out arrays alike.
 */
int orc_lse_merge(int n_parts, int64_t rows, int64_t D,
                  const double* const* o_parts, const double* const* lse_parts,
                  double* o_out, double* lse_out)
{
    if (n_parts < 1 || rows < 0 || D < 1) return ORC_BAD;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int n = 0; n < n_parts; ++n)
            if (lse_parts[n][r] > M) M = lse_parts[n][r];
        if (M == -INFINITY) {
            for (int64_t d = 0; d < D; ++d) o_out[r * D + d] = 0.0;
            lse_out[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int n = 0; n < n_parts; ++n) sum += exp(lse_parts[n][r] - M);
        const double L = M + log(sum);
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int n = 0; n < n_parts; ++n)
                acc += exp(lse_parts[n][r] - L) * o_parts[n][r * D + d];
            o_out[r * D + d] = acc;
        }
        lse_out[r] = L;
    }
    return ORC_OK;
}

/* Number of OpenMP threads a parallel region gets (for the CPU baseline). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
#else
int orc_num_threads(void) { return 1; }
#endif
