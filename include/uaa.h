/*
 * uaa.h -- C ABI of libuaa.so: one rank's share of context-parallel
 * attention (Ulysses, Ulysses Anything, Ring, Unified) on one AMD Instinct
 * MI355X (gfx950).
 *
 * Pages whose statement of the problem these calls follow:
 *   [CP]  "Context parallelism" (diffusers documentation), sections
 *         "Ring Attention", "Ulysses Attention", "Unified Attention",
 *         "Ulysses Anything Attention", "Ring Anything Attention".
 *   [USP] "Add Unified Sequence Parallel attention" (diffusers pull request
 *         #12693), review thread: each Ring step's attention returns
 *         (out, lse); the running pair is merged in fp32 and cast back to the
 *         query dtype once; the LSE travels as (B, S, H_LOCAL).
 *   [UAA] "UAA: Ulysses Anything Attention" (diffusers issue #12706): any
 *         sequence length, no padding, only per-rank seq_len is exchanged;
 *         forced host/device syncs are what costs time.
 *   [YC]  USP / yunchang project summary (sourcepulse), "How It Works",
 *         "Highlighted Details": zigzag / stripe / basic ring layouts.
 *
 * Conventions shared by every call
 *   - Tensors are dense, row-major, BSHD: [batch, sequence, heads, feature].
 *     "bf16" is IEEE bfloat16 storage; all arithmetic inside is fp32.
 *   - Pointers named "device" are HIP device pointers; host arrays (offsets,
 *     the arrays of device pointers, the mask descriptor) are read during the
 *     call only and never retained.
 *   - The caller owns every buffer.  No call allocates or frees memory.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *     null stream) and the call returns without waiting for it.  No call
 *     synchronises the device or copies device data to the host ([UAA]: such
 *     forced syncs are the cost to avoid).
 *   - Every argument is validated on the host before anything is enqueued.
 *     A failing check returns a negative status and leaves the stream
 *     untouched; uaa_last_error() then describes it.
 *   - Calls on different streams may run concurrently if their outputs do
 *     not overlap each other or any input.
 */
#ifndef UAA_H
#define UAA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define UAA_OK 0
#define UAA_ERR_INVALID_ARG (-1) /* malformed arguments (null, negative, inconsistent) */
#define UAA_ERR_UNSUPPORTED (-2) /* well-formed but outside what the kernels handle */
#define UAA_ERR_HIP (-3)         /* the HIP runtime reported an error on launch */

/* Element types. */
#define UAA_BF16 0
#define UAA_FP32 1

/* Permute directions. */
#define UAA_SEQ2HEAD 0
#define UAA_HEAD2SEQ 1

/* Largest Ulysses degree a permute accepts, largest N a merge accepts,
 * largest tensor count of one multi-tensor permute, largest Ulysses degree
 * of the gathering attention (usp_attn_fwd_lse_gather). */
#define UAA_MAX_WORLD 64
#define USP_MAX_PARTS 16
#define UAA_MAX_PERMUTE_TENSORS 4
#define UAA_MAX_GATHER_WORLD 8

/* Mask kinds ([YC] ring layouts; "basic" contiguous shards are CAUSAL). */
#define USP_MASK_FULL 0
#define USP_MASK_CAUSAL 1
#define USP_MASK_ZIGZAG 2
#define USP_MASK_STRIPE 3

/*
 * Global token positions of the query rows and key columns of one attention
 * call.  Under every kind but FULL, key j is allowed for query i iff
 * kpos(j) <= qpos(i) (causal by global position).
 *   CAUSAL: qpos(i) = q_off + i,  kpos(j) = k_off + j   (contiguous shards)
 *   ZIGZAG: the sequence is cut into chunks of `chunk` tokens; the query rows
 *           are chunk q_chunks[0] followed by chunk q_chunks[1] (or only
 *           q_chunks[0] when q_chunks[1] < 0), so
 *           qpos(i) = q_chunks[i / chunk] * chunk + i % chunk; keys likewise
 *           with k_chunks.  Rank r of an R-rank zigzag ring holds chunks r
 *           and 2R-1-r.
 *   STRIPE: qpos(i) = q_rank + world * i,  kpos(j) = k_rank + world * j.
 * Unused fields are ignored.
 */
typedef struct usp_mask {
    int32_t kind;
    int32_t world;
    int64_t q_off;
    int64_t k_off;
    int64_t chunk;
    int32_t q_chunks[2];
    int32_t k_chunks[2];
    int32_t q_rank;
    int32_t k_rank;
} usp_mask;

/*
 * uaa_split_offsets -- the default split of `total` items (tokens or heads)
 * over `parts` ranks as exclusive prefix sums: off[0] = 0, off[p+1] =
 * off[p] + n_p with n_p = ceil(total / parts) for the first total mod parts
 * ranks and floor(total / parts) for the rest ([UAA] and [CP] "Ulysses
 * Anything Attention": any length is split without padding; the first
 * ranks take the extra token, so 257 -> 129 / 128 and 4481 -> 2241 / 2240).
 * The permute and gathering-attention calls use this split for the heads
 * when they are given head_off = NULL.
 *
 *   off  host array of parts + 1 entries, written (owned by the caller).
 * parts >= 1, total >= 0 (else UAA_ERR_INVALID_ARG, off untouched).  Host
 * only: no device work, callable without a GPU.
 * Returns UAA_OK or UAA_ERR_INVALID_ARG.
 */
int uaa_split_offsets(int64_t total, int parts, int64_t* off);

/*
 * uaa_seq2head_permute -- the local data movement of the Ulysses all-to-all
 * for one rank, run as a gather ([CP] "Ulysses Attention": the first
 * exchange leaves every GPU all tokens of a subset of heads, the second
 * regroups by token; [CP] "Ulysses Anything Attention" / [UAA]: the token
 * and head counts per rank are arbitrary and nothing is padded).
 *
 * seq_off[0..world]  host, exclusive prefix sums of the per-rank token
 *                    counts: rank p holds tokens [seq_off[p], seq_off[p+1]).
 *                    Must start at 0 and never decrease (empty ranks allowed).
 * head_off[0..world] host, the same for heads; must start at 0, strictly
 *                    increase and end at H (so world <= H).  NULL = split H
 *                    with the first H mod world ranks taking one extra head.
 * S = seq_off[world], S_p = seq_off[p+1]-seq_off[p], H_r likewise.
 *
 * dir = UAA_SEQ2HEAD, `rank` = the head rank r being assembled:
 *   src[p] (p < world): device [B, S_p, H, D]   (rank p's token shard)
 *   dst:                device [B, S, H_r, D]
 *   dst[b, s, h, d] = src[p][b, s - seq_off[p], head_off[r] + h, d]
 *   with p the rank whose token range contains s.
 * dir = UAA_HEAD2SEQ, `rank` = the token rank p being assembled:
 *   src[r] (r < world): device [B, S, H_r, D]   (rank r's head shard)
 *   dst:                device [B, S_p, H, D]
 *   dst[b, t, h, d] = src[r][b, seq_off[p] + t, h - head_off[r], d]
 *   with r the rank whose head range contains h.
 * The LSE of the Unified path ([USP], (B, S, H_LOCAL)) moves with D = 1,
 * elem_bytes = 4.
 *
 * elem_bytes: 1, 2, 4 or 8; elements are copied as opaque bit patterns
 * (bit-exact).  Every pointer must be aligned to elem_bytes; the widest
 * access that alignment and the row sizes allow is chosen internally.
 * src and dst must not overlap.  H, D >= 1, B >= 0 (B = 0 or an empty
 * destination: no work, pointers unchecked).  S < 2^31; one source shard
 * may move fewer than 2^31 access-width elements (else
 * UAA_ERR_UNSUPPORTED); B <= 65535.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int uaa_seq2head_permute(int dir, int rank, int world,
                         const int64_t* seq_off, const int64_t* head_off,
                         int64_t B, int64_t H, int64_t D, int elem_bytes,
                         const void* const* src, void* dst, void* stream);

/*
 * uaa_seq2head_permute_multi -- the same layout change for n_tensors tensors
 * of identical shape in one launch (Q, K and V of a layer move together, so
 * one launch replaces three and the fixed per-launch cost is paid once).
 *
 *   src  host array of n_tensors * world device pointers, tensor t's shard
 *        y at src[t * world + y] (shapes as for uaa_seq2head_permute)
 *   dst  host array of n_tensors device pointers
 * Every other argument is shared and means what it means above.  Limits:
 * 1 <= n_tensors <= UAA_MAX_PERMUTE_TENSORS, n_tensors * world <= 64,
 * B * n_tensors <= 65535.  The result equals n_tensors separate calls.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int uaa_seq2head_permute_multi(int n_tensors, int dir, int rank, int world,
                               const int64_t* seq_off, const int64_t* head_off,
                               int64_t B, int64_t H, int64_t D, int elem_bytes,
                               const void* const* src, void* const* dst, void* stream);

/*
 * uaa_seq2head_permute_multi_ex -- as uaa_seq2head_permute_multi, for
 * tensors that share B, H and the token / head split but not the size of a
 * head slice: tensor t has D[t] features of elem_bytes[t] bytes (host arrays
 * of n_tensors entries).  The output O and its LSE (D = 1, 4 bytes) of the
 * Unified path ([USP]) go back to the token layout in one launch this way.
 * Each tensor moves in the widest access its head slice and pointers
 * allow; the result equals n_tensors separate calls.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int uaa_seq2head_permute_multi_ex(int n_tensors, int dir, int rank, int world,
                                  const int64_t* seq_off, const int64_t* head_off,
                                  int64_t B, int64_t H, const int64_t* D, const int* elem_bytes,
                                  const void* const* src, void* const* dst, void* stream);

/*
 * usp_attn_fwd_lse -- softmax attention of one rank's query rows against
 * one block of keys/values, returning both the output and the per-row
 * log-sum-exp: the (out, lse) pair each Ring step produces ([USP]; [CP]
 * "Ring Attention": each GPU computes attention against the K/V block it
 * holds; "Ring Anything Attention": blocks of any length).
 *
 *   q  device [B, Sq, H, D]  dtype
 *   k  device [B, Sk, H, D]  dtype
 *   v  device [B, Sk, H, D]  dtype
 *   o  device [B, Sq, H, D]  o_dtype (bf16 rounded to nearest even)
 *   lse device [B, Sq, H]    fp32, natural log
 * For every (b, i, h), with J the allowed keys of row i (all j < Sk under
 * USP_MASK_FULL or mask == NULL; kpos(j) <= qpos(i) otherwise):
 *   s_j = scale * <q_i, k_j>,  lse = log(sum_{j in J} exp(s_j)),
 *   o   = sum_{j in J} exp(s_j - lse) * v_j,
 * and o = 0, lse = -inf when J is empty (a row with no allowed key, or
 * Sk = 0), so that such a partial drops out of usp_lse_merge.  A mask under
 * which no key lies after any query in position allows every pair; such a
 * call runs as the unmasked one, with the same result bit for bit.
 *
 * dtype: UAA_BF16 (bf16 matrix-core products, fp32 accumulation and
 * softmax) or UAA_FP32 (fp32 throughout).  o_dtype: UAA_BF16 or UAA_FP32 for
 * bf16 input, UAA_FP32 for fp32 input.  D: 64 or 128 (else
 * UAA_ERR_UNSUPPORTED).  scale: finite, > 0.  q, k, v, o: 16-byte aligned;
 * lse: 4-byte aligned.  Outputs must not overlap inputs.  Sq = 0, B = 0 or
 * H = 0: no work.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int usp_attn_fwd_lse(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                     const void* q, const void* k, const void* v,
                     void* o, int o_dtype, float* lse,
                     float scale, const usp_mask* mask, void* stream);

/*
 * usp_attn_fwd_lse_ws -- usp_attn_fwd_lse with a caller-owned device
 * workspace, for shapes whose work does not divide evenly over the compute
 * units.  The plain call runs one workgroup per 256 query rows of one
 * (batch, head) -- a "unit" -- one workgroup per compute unit at a time, so
 * e.g. 336 units on 256 compute units take two full rounds.  With a
 * workspace, bf16 input and USP_MASK_FULL, the kernel instead keeps
 * floor(units / CUs) rounds' worth of units whole and cuts the keys of each
 * remaining unit (of every unit, when they fill at most half the compute
 * units) into p <= 8 pieces of about equal length, each run by its own
 * workgroup ahead of the whole units, where a cost model of the launch says
 * this pays.  The last piece of a unit to finish merges the pieces' results
 * -- the Ring merge of key blocks ([USP]) done inside the kernel -- in piece
 * order, so the result does not depend on timing.  It equals the plain
 * call's up to rounding (a piece's probabilities are taken relative to that
 * piece's maximum; with D = 128 a piece's O is kept in bf16 between the
 * piece and the merge).
 *
 *   workspace  device, 256-byte aligned, at least
 *              usp_attn_workspace_bytes(...) bytes, zero-filled before its
 *              first use; every call leaves it zero-filled again where it
 *              matters (the arrival counters).  NULL, or fewer bytes than
 *              needed: the plain call.
 * Calls that share a workspace must not run concurrently (stream order is
 * enough).  Every other argument is that of usp_attn_fwd_lse.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int usp_attn_fwd_lse_ws(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                        const void* q, const void* k, const void* v, void* o, int o_dtype,
                        float* lse, float scale, const usp_mask* mask, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * usp_attn_fwd_lse_static -- usp_attn_fwd_lse_ws for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc.  It takes no workspace
 * and allocates nothing (no hipMalloc, hipFree or allocating library call):
 * the key split's workspace is a device array inside the library,
 * USP_STATIC_SCRATCH_BYTES per GPU, which every GPU the library runs on
 * holds from the library's loading until the process ends.  Its device
 * address is looked up once per device on the first call there.  The split's
 * arrival counters are cleared by a small kernel on `stream` ahead of each
 * launch that uses them (a kernel, not a memset, so graph replays repeat
 * it).  Every call on one GPU shares that GPU's array and it keeps the last
 * call's contents: calls that may overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.
 *
 * A problem whose key split would need more than USP_STATIC_SCRATCH_BYTES
 * (a device with more than 256 compute units) returns UAA_ERR_UNSUPPORTED
 * and enqueues nothing.  Results equal usp_attn_fwd_lse_ws given a large
 * enough workspace, bit for bit; every argument is that call's.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
#define USP_STATIC_SCRATCH_BYTES (36u << 20)   /* 256 piece slots of 136 KiB and their counters */
int usp_attn_fwd_lse_static(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                            const void* q, const void* k, const void* v, void* o, int o_dtype,
                            float* lse, float scale, const usp_mask* mask, void* stream);

/*
 * usp_attn_fwd_lse_acc -- one step of a Ring pass in one call: the
 * attention of this key/value block merged into the running result ([USP]:
 * each Ring step's (out, lse) is folded into the accumulated one by the LSE
 * merge; [CP] "Ring Attention").  On entry (o, lse) hold the result over the
 * keys seen so far (lse = -inf for a row with none; its o is then not read);
 * on return they hold the result over those keys and this block:
 *   lse' = log(e^lse + e^lse_b),  o' = e^(lse - lse') o + e^(lse_b - lse') o_b
 * with (o_b, lse_b) what usp_attn_fwd_lse would give for this block.  The
 * merge runs in fp32 in the epilogue, o_b rounded to o_dtype first when that
 * is bf16 (as if merged by usp_lse_merge), and saves the separate merge pass
 * when the blocks arrive one at a time.  o and lse are read and written in
 * place; every other argument (workspace included) is that of
 * usp_attn_fwd_lse_ws.  The first block of a pass uses usp_attn_fwd_lse(_ws)
 * (or starts from lse = -inf).
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int usp_attn_fwd_lse_acc(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                         const void* q, const void* k, const void* v, void* o, int o_dtype,
                         float* lse, float scale, const usp_mask* mask, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * usp_attn_fwd_lse_gather -- usp_attn_fwd_lse(_acc) on this rank's Ulysses
 * view of token-sharded Q, K and V, read straight from the shards instead
 * of from a gathered copy: the SEQ2HEAD gather of uaa_seq2head_permute
 * ([CP] "Ulysses Attention", "Ulysses Anything Attention": any token and head
 * counts, no padding) done inside the attention's loads.  For rank `rank` it
 * computes exactly
 *   Yq = SEQ2HEAD(q_shards), Yk = SEQ2HEAD(k_shards), Yv = SEQ2HEAD(v_shards)
 *   usp_attn_fwd_lse(_acc)(Yq, Yk[:, keys of shard k_shard], Yv[...], ...)
 * i.e. the queries are all S = seq_off[world] tokens, the keys the tokens of
 * shard k_shard (a Ring chunk is one rank's token shard in the Unified
 * composition, [USP]; attention over every token is one call per shard,
 * the first plain and the rest with accumulate = 1).
 *
 *   world <= UAA_MAX_GATHER_WORLD, rank, seq_off, head_off (NULL = even):
 *        as for uaa_seq2head_permute; H = total heads
 *   q_shards, k_shards, v_shards: host arrays of `world` device pointers,
 *        shard p is [B, S_p, H, D] bf16 (16-byte aligned; NULL allowed for
 *        an empty shard, and for the k/v shards other than k_shard)
 *   o   device [B, S, H_r, D] o_dtype, lse device [B, S, H_r] fp32, with H_r
 *        this rank's heads; mask positions are indices into these S queries
 *        and the keys of shard k_shard; scale, mask, workspace as for
 *        usp_attn_fwd_lse_ws; accumulate != 0: as usp_attn_fwd_lse_acc.
 * Results are identical, bit for bit, to the gathered-copy calls above.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED (fp32 input, D
 * not 64 or 128) or UAA_ERR_HIP.
 */
int usp_attn_fwd_lse_gather(int dtype, int world, int rank, const int64_t* seq_off, const int64_t* head_off,
                            int64_t B, int64_t H, int64_t D, const void* const* q_shards,
                            const void* const* k_shards, const void* const* v_shards, int k_shard, void* o,
                            int o_dtype, float* lse, float scale, const usp_mask* mask, void* workspace,
                            size_t workspace_bytes, int accumulate, void* stream);

/*
 * usp_attn_kernel -- which forward kernel usp_attn_fwd_lse(_ws, _acc) would
 * run for this problem on the current device, for profiling and for tests
 * that must know the kernel they cover.  Host only: nothing is launched and
 * no pointer is needed; a workspace counts as given when workspace_bytes >
 * 0 (enough bytes: see usp_attn_workspace_bytes).  Returns one of the codes
 * below, or UAA_ERR_INVALID_ARG / UAA_ERR_UNSUPPORTED for arguments the
 * call itself would reject (as usp_attn_fwd_lse, pointers aside).
 */
#define USP_KERNEL_NONE 0            /* no work (B, H or Sq = 0) */
#define USP_KERNEL_FP32 1            /* fp32 input: the fp32 kernel */
#define USP_KERNEL_GENERAL 2         /* bf16, every key allowed: the general kernel */
#define USP_KERNEL_GENERAL_MASKED 3  /* bf16, a mask with units on its diagonal: the general kernel */
#define USP_KERNEL_GENERAL_SPLIT 4   /* bf16, keys of the last round's units split: the general kernel */
#define USP_KERNEL_PIPELINED 5       /* bf16, D = 128: the software-pipelined kernel */
#define USP_KERNEL_PIPELINED_DIAG 6  /* bf16, D = 128, a mask whose keys form one increasing piece:
                                        the pipelined kernel, diagonal units masked row by row */
#define USP_KERNEL_PIPELINED_SPLIT 7 /* bf16, D = 128, every key allowed, with a workspace: the
                                        pipelined kernel with the keys of some units split into
                                        pieces run on otherwise idle CUs */
int usp_attn_kernel(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, int o_dtype,
                    const usp_mask* mask, size_t workspace_bytes);

/*
 * usp_attn_workspace_bytes -- device workspace usp_attn_fwd_lse_ws uses for
 * this problem on the current device: 0 when it would run as the plain call
 * (fp32, a causal-family mask, or no split that saves at least 8 % by a
 * round-count model); otherwise 136 KiB per piece plus 4 bytes per split
 * unit.  Arguments as for usp_attn_fwd_lse; invalid ones give 0.
 */
size_t usp_attn_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                const usp_mask* mask);

/*
 * usp_lse_merge -- merge N partial (O, LSE) pairs of the same query rows,
 * each over a disjoint set of keys, into the pair over their union ([USP]:
 * the Ring loop's fp32 update of the running (out, lse), cast to the output
 * dtype once at the end).  Per row, computed in fp32:
 *   M   = max_n lse_n
 *   lse = M + log(sum_n exp(lse_n - M))
 *   o   = sum_n exp(lse_n - lse) * o_n
 * and (o, lse) = (0, -inf) when every lse_n is -inf.  On finite inputs this
 * is the pages' pairwise sigmoid / log-sigmoid update folded over n; the
 * max-shifted form also accepts -inf partials, which the pairwise form
 * turns into NaN.  A partial whose lse_n is -inf for a row (its block had
 * no allowed key there) has weight 0 and its O row is not read: whatever
 * it holds, the row's result is that of the other partials.
 *
 *   o_parts   host array of n_parts device pointers, each [B, S, H, D]
 *             part_dtype
 *   lse_parts host array of n_parts device pointers, each [B, S, H] fp32
 *   o_out     device [B, S, H, D] out_dtype (bf16 rounded to nearest even)
 *   lse_out   device [B, S, H] fp32
 * n_parts in [1, USP_MAX_PARTS].  D >= 1.  Pointers aligned to their
 * element size.  lse_out may equal lse_parts[n], and o_out may equal
 * o_parts[n] when part_dtype == out_dtype (in-place accumulation); no other
 * overlap.  B, S or H = 0: no work.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG or UAA_ERR_HIP.
 */
int usp_lse_merge(int n_parts, int64_t B, int64_t S, int64_t H, int64_t D,
                  const void* const* o_parts, int part_dtype, const float* const* lse_parts,
                  void* o_out, int out_dtype, float* lse_out, void* stream);

/*
 * usp_attn_bwd_delta -- the per-row statistic of the attention backward
 * ([USP], pull request conversation: the Unified / Ring attention is trained
 * through a backward of its forward; the backward itself is the chain rule
 * through softmax):
 *   delta[b, s, h] = sum_d dout[b, s, h, d] * o[b, s, h, d]  -  dlse[b, s, h]
 * in fp32, with (o, lse) the forward's result over ALL key blocks of the
 * rows (after the Ring merge), dout the gradient of o and dlse the gradient
 * of lse (NULL: zero).
 *
 *   o, dout    device [B, S, H, D] dtype (UAA_BF16 or UAA_FP32)
 *   dlse       device [B, S, H] fp32, or NULL
 *   delta      device [B, S, H] fp32 (output)
 * D: 64 or 128 (else UAA_ERR_UNSUPPORTED).  o, dout 16-byte aligned; dlse,
 * delta 4-byte aligned.  delta must not overlap the inputs.  B, S or H = 0:
 * no work.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int usp_attn_bwd_delta(int dtype, int64_t B, int64_t S, int64_t H, int64_t D, const void* o,
                       const void* dout, const float* dlse, float* delta, void* stream);

/*
 * usp_attn_bwd -- gradients of one attention call (one Ring key block) of
 * usp_attn_fwd_lse ([USP], as above).  With J the allowed keys of row i (as
 * in the forward), lse the rows' LSE over all key blocks and delta from
 * usp_attn_bwd_delta:
 *   P_ij  = exp(scale <q_i, k_j> - lse_i)   (j in J; 0 otherwise, and 0 for
 *                                            every j when lse_i = -inf)
 *   dS_ij = P_ij (<dout_i, v_j> - delta_i)
 *   dq_i  = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
 *   dv_j  = sum_i P_ij dout_i.
 * For a single block (lse, o of this call) this is the gradient of
 * sum(dout * o) + sum(dlse * lse); over the blocks of a Ring pass, dq summed
 * over the blocks and each block's (dk, dv) are the gradients of the merged
 * result.
 *
 *   q, dout    device [B, Sq, H, D] dtype
 *   k, v       device [B, Sk, H, D] dtype
 *   lse, delta device [B, Sq, H] fp32
 *   dq         device [B, Sq, H, D] grad_dtype (output)
 *   dk, dv     device [B, Sk, H, D] grad_dtype (output)
 * accumulate: bit 0 set -- dq is added to what dq holds, else written;
 * bit 1 set -- dk and dv likewise (a Ring backward adds every block into dq,
 * and each block's dk, dv into the buffers that travel with that block).
 * Sums run in fp32 and are rounded once when grad_dtype is bf16.  dtype:
 * UAA_BF16 (bf16 matrix-core products, fp32 accumulation) or UAA_FP32 (fp32
 * throughout).  grad_dtype: UAA_BF16 or UAA_FP32.  D: 64 or 128.
 * scale: finite, > 0.  mask as in usp_attn_fwd_lse.  q, k, v, dout, dq, dk,
 * dv 16-byte aligned; lse, delta 4-byte aligned.  Outputs must not overlap
 * inputs or each other.  B = 0, H = 0 or Sq = Sk = 0: no work; Sq = 0 gives
 * dk = dv = 0 (nothing added with bit 1); Sk = 0 gives dq = 0.  The
 * two kernels (dk/dv, then dq) run in order on `stream`; no workspace.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int usp_attn_bwd(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                 const void* q, const void* k, const void* v, const void* dout,
                 const float* lse, const float* delta, void* dq, void* dk, void* dv, int grad_dtype,
                 float scale, const usp_mask* mask, int accumulate, void* stream);

/*
 * usp_attn_bwd_ws -- usp_attn_bwd with a caller-owned device workspace that
 * holds dS for the dq kernel.  Without it, the dq kernel recomputes the
 * scores and dP of every pair (the dk/dv kernel forms them too, so S and dP
 * are computed twice: 14 D FLOP per pair against the 10 D of the five
 * products above).  With it, for bf16 input, D = 128 and every pair
 * allowed, the dk/dv kernel also writes dS_ij in bf16 (the value its dk
 * product uses) to the workspace and the dq kernel forms dq_i = scale
 * sum_j dS_ij k_j from it: 2 bytes of traffic each way per pair instead of
 * 4 D FLOP.  The result equals usp_attn_bwd's up to rounding (dS is formed
 * from P rounded to bf16, as in dk).
 *
 *   workspace  device, 16-byte aligned, at least
 *              usp_attn_bwd_workspace_bytes(...) bytes, contents ignored
 *              (both kernels of the call use it; calls that share a
 *              workspace must not overlap).  NULL, fewer bytes than needed,
 *              or a call the path does not cover: the plain call.
 * Every other argument is that of usp_attn_bwd.
 * Returns UAA_OK, UAA_ERR_INVALID_ARG, UAA_ERR_UNSUPPORTED or UAA_ERR_HIP.
 */
int usp_attn_bwd_ws(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                    const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, const float* delta, void* dq, void* dk, void* dv, int grad_dtype,
                    float scale, const usp_mask* mask, int accumulate, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * usp_attn_bwd_workspace_bytes -- bytes of the workspace usp_attn_bwd_ws
 * uses for these sizes and mask: B * H * ceil(Sq / 32) * ceil(Sk / 16) *
 * 1024 (dS in bf16, in blocks of 32 queries x 16 keys), or 0 where the path does not
 * apply (fp32 input, D != 128, a mask that excludes some pair, an empty
 * call, or an invalid mask).  Host only; no device work.
 */
size_t usp_attn_bwd_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                    const usp_mask* mask);

/*
 * uaa_last_error -- text describing the last non-zero status returned on
 * the calling thread ("" if none).  The pointer stays valid until the next
 * call on that thread.
 */
const char* uaa_last_error(void);

/* uaa_abi_version -- version of this header's contract (currently 1). */
int uaa_abi_version(void);

/* uaa_build_id -- sha256 (hex) of the sources, headers and flags this
 * library was built from, as the build script computes it ("unknown" when
 * built without it); lets a caller check that a library matches its
 * sources.  Static storage, never freed. */
const char* uaa_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* UAA_H */
