/* Host driver of the C oracle for an AddressSanitizer + UndefinedBehavior-
 * Sanitizer build (test infrastructure, run by tests/test_host_sanitize.py):
 * every entry point on small cases whose arrays are allocated at exactly
 * the sizes the calls may touch, so an index past an end is reported.
 * Exits non-zero on a failed check. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_seq2head(int rank, int world, const int64_t* seq_off, const int64_t* head_off, int64_t B, int64_t H,
                 int64_t D, int elem_bytes, const void* const* src, void* dst);
int orc_head2seq(int rank, int world, const int64_t* seq_off, const int64_t* head_off, int64_t B, int64_t H,
                 int64_t D, int elem_bytes, const void* const* src, void* dst);
int orc_seq2head_index(int rank, int world, const int64_t* seq_off, const int64_t* head_off, int64_t B,
                       int64_t H, int64_t D, int64_t* src_shard, int64_t* src_elem);
int orc_attention(int64_t B, int64_t Sq, int64_t Sk, int64_t H, int64_t D, const double* q, const double* k,
                  const double* v, const int64_t* qpos, const int64_t* kpos, int causal, double scale,
                  const int64_t* rows, int64_t n_rows, double* o, double* lse);
int orc_lse_merge(int n_parts, int64_t rows, int64_t D, const double* const* o_parts,
                  const double* const* lse_parts, double* o_out, double* lse_out);

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

static double* filled(int64_t n, unsigned seed)
{
    double* x = malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        seed = seed * 1103515245u + 12345u;
        x[i] = ((double)(seed >> 8) / 16777216.0) - 0.5;
    }
    return x;
}

static void permute_round_trip(void)
{
    /* 3 token shards of 4 / 0 / 3 tokens, 5 heads split 2 / 2 / 1, D = 3 */
    const int world = 3;
    const int64_t B = 2, H = 5, D = 3;
    int64_t* seq_off = malloc(sizeof(int64_t) * (world + 1));
    int64_t* head_off = malloc(sizeof(int64_t) * (world + 1));
    const int64_t so[] = {0, 4, 4, 7}, ho[] = {0, 2, 4, 5};
    memcpy(seq_off, so, sizeof(so));
    memcpy(head_off, ho, sizeof(ho));
    const int64_t S = 7;
    float* shard[3];
    for (int p = 0; p < world; ++p) {
        const int64_t n = B * (seq_off[p + 1] - seq_off[p]) * H * D;
        shard[p] = malloc(sizeof(float) * (size_t)(n ? n : 1));
        for (int64_t i = 0; i < n; ++i) shard[p][i] = (float)(1000 * p + i);
    }
    float* heads[3];
    for (int r = 0; r < world; ++r) {
        const int64_t Hr = head_off[r + 1] - head_off[r];
        heads[r] = malloc(sizeof(float) * (size_t)(B * S * Hr * D));
        CHECK(orc_seq2head(r, world, seq_off, head_off, B, H, D, 4, (const void* const*)shard, heads[r]) == 0);
        int64_t* sh = malloc(sizeof(int64_t) * (size_t)(B * S * Hr * D));
        int64_t* el = malloc(sizeof(int64_t) * (size_t)(B * S * Hr * D));
        CHECK(orc_seq2head_index(r, world, seq_off, head_off, B, H, D, sh, el) == 0);
        for (int64_t i = 0; i < B * S * Hr * D; ++i) CHECK(heads[r][i] == shard[sh[i]][el[i]]);
        free(sh);
        free(el);
    }
    for (int p = 0; p < world; ++p) {
        const int64_t n = B * (seq_off[p + 1] - seq_off[p]) * H * D;
        float* back = malloc(sizeof(float) * (size_t)(n ? n : 1));
        CHECK(orc_head2seq(p, world, seq_off, head_off, B, H, D, 4, (const void* const*)heads, back) == 0);
        for (int64_t i = 0; i < n; ++i) CHECK(back[i] == shard[p][i]);
        free(back);
    }
    /* rejected: rank out of range, decreasing offsets */
    CHECK(orc_seq2head(3, world, seq_off, head_off, B, H, D, 4, (const void* const*)shard, heads[0]) != 0);
    seq_off[2] = 1;
    CHECK(orc_seq2head(0, world, seq_off, head_off, B, H, D, 4, (const void* const*)shard, heads[0]) != 0);
    for (int p = 0; p < world; ++p) {
        free(shard[p]);
        free(heads[p]);
    }
    free(seq_off);
    free(head_off);
}

static void attention_and_merge(void)
{
    const int64_t B = 2, Sq = 9, Sk = 11, H = 3, D = 5;
    double* q = filled(B * Sq * H * D, 1);
    double* k = filled(B * Sk * H * D, 2);
    double* v = filled(B * Sk * H * D, 3);
    int64_t* qpos = malloc(sizeof(int64_t) * Sq);
    int64_t* kpos = malloc(sizeof(int64_t) * Sk);
    for (int64_t i = 0; i < Sq; ++i) qpos[i] = 2 * i;        /* rows 0..: positions 0, 2, ... */
    for (int64_t j = 0; j < Sk; ++j) kpos[j] = 3 + j;        /* row 0 sees no key */
    double* o = malloc(sizeof(double) * (size_t)(B * Sq * H * D));
    double* lse = malloc(sizeof(double) * (size_t)(B * Sq * H));
    int64_t* rows = malloc(sizeof(int64_t) * (size_t)(B * Sq));
    for (int64_t r = 0; r < B * Sq; ++r) rows[r] = r;
    CHECK(orc_attention(B, Sq, Sk, H, D, q, k, v, qpos, kpos, 1, 0.3, rows, B * Sq, o, lse) == 0);
    CHECK(isinf(lse[0]) && lse[0] < 0);
    for (int64_t d = 0; d < D; ++d) CHECK(o[d] == 0.0);
    /* the last row of each batch sees every key: finite */
    CHECK(isfinite(lse[(Sq - 1) * H]));
    /* a subset of rows, unmasked, equals the same rows of the full result */
    double* o_all = malloc(sizeof(double) * (size_t)(B * Sq * H * D));
    double* l_all = malloc(sizeof(double) * (size_t)(B * Sq * H));
    CHECK(orc_attention(B, Sq, Sk, H, D, q, k, v, qpos, kpos, 0, 0.3, rows, B * Sq, o_all, l_all) == 0);
    int64_t* some = malloc(sizeof(int64_t) * 2);
    some[0] = B * Sq - 1;
    some[1] = 3;
    double* o2 = malloc(sizeof(double) * (size_t)(2 * H * D));
    double* l2 = malloc(sizeof(double) * (size_t)(2 * H));
    CHECK(orc_attention(B, Sq, Sk, H, D, q, k, v, qpos, kpos, 0, 0.3, some, 2, o2, l2) == 0);
    for (int64_t x = 0; x < H * D; ++x) CHECK(o2[x] == o_all[(B * Sq - 1) * H * D + x]);
    for (int64_t x = 0; x < H * D; ++x) CHECK(o2[H * D + x] == o_all[3 * H * D + x]);
    /* merge: N = 3 with one all -inf part and one row empty in every part */
    const int64_t R = 4, DD = 6;
    const double* op[3];
    const double* lp[3];
    double* obuf[3];
    double* lbuf[3];
    for (int n = 0; n < 3; ++n) {
        obuf[n] = filled(R * DD, 10 + n);
        lbuf[n] = filled(R, 20 + n);
        op[n] = obuf[n];
        lp[n] = lbuf[n];
    }
    for (int64_t r = 0; r < R; ++r) lbuf[2][r] = -INFINITY;
    lbuf[0][1] = lbuf[1][1] = -INFINITY;
    double* mo = malloc(sizeof(double) * (size_t)(R * DD));
    double* ml = malloc(sizeof(double) * (size_t)R);
    CHECK(orc_lse_merge(3, R, DD, op, lp, mo, ml) == 0);
    CHECK(isinf(ml[1]) && ml[1] < 0);
    for (int64_t d = 0; d < DD; ++d) CHECK(mo[DD + d] == 0.0);
    CHECK(isfinite(ml[0]) && isfinite(ml[3]));
    CHECK(orc_lse_merge(0, R, DD, op, lp, mo, ml) != 0);
    for (int n = 0; n < 3; ++n) {
        free(obuf[n]);
        free(lbuf[n]);
    }
    free(mo); free(ml); free(q); free(k); free(v); free(qpos); free(kpos); free(o); free(lse); free(rows);
    free(o_all); free(l_all); free(some); free(o2); free(l2);
}

int main(void)
{
    permute_round_trip();
    attention_and_merge();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle host checks ok\n");
    return 0;
}
