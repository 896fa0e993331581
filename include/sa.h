/* sa.h -- C ABI of libsa.so, DeepSeek-V4.1 sparse latent attention for AMD MI355X (gfx950).
 *
 * The operation is sparse_attn as the attention API docs define it
 * (docs.atlascybernetics.ai/api/spark_model/layers/deepseek_v41_ref/attn/, "sparse_attn" and
 * the precision paragraph) and as Attention.forward calls it
 * (atlas.klimoza.dev/models/deepseek-v4.1/.../attention/output, Attention.forward): for every
 * query and head, gather the latent KV rows that an index list names (negative = skip),
 * score them as q.k * softmax_scale with the same row serving as key and value, take a
 * softmax in f32 whose denominator also holds exp(attn_sink[head]), and return the weighted
 * sum of the rows in bf16.
 *
 * Conventions shared by every entry point:
 *   - Device pointers are caller-owned (for example PyTorch tensors). The library never
 *     allocates, frees or retains them, and holds no state between calls apart from a
 *     per-device cache of the compute-unit count.
 *   - Strides are counted in elements of the pointed-to type.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the null stream)
 *     and runs asynchronously. The return value reports host-side argument validation and
 *     launch errors only; argument checks happen before any HIP call is made.
 *   - bf16 means the 16-bit bfloat16 format; out-of-kernel values are never converted.
 *   - Calls are thread-safe. Two calls that write the same output or workspace race.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 2

/* status codes */
enum {
    SA_OK = 0,
    SA_ERR_INVALID = -1,      /* a null pointer, a negative or zero size, a bad stride ... */
    SA_ERR_UNSUPPORTED = -2,  /* well-formed but outside what the kernels implement */
    SA_ERR_HIP = -3,          /* the HIP runtime reported an error at launch */
    SA_ERR_WORKSPACE = -4,    /* workspace missing or smaller than sa_sparse_attn_workspace */
    SA_ERR_SCRATCH = -5       /* sa_sparse_attn_noalloc: the plan needs more workspace than
                                 SA_NOALLOC_SCRATCH_BYTES */
};

/* KV storage formats */
enum {
    SA_KV_BF16 = 0,           /* kv: bf16 [b][kv_rows][d] */
    SA_KV_FP8_E4M3_B32 = 1    /* kv: e4m3fn bytes [b][kv_rows][d] + kv_scale: e8m0 bytes
                                 [b][kv_rows][d/32]; value = e4m3 * 2^(scale_byte - 127),
                                 the storage form of sa_quant_kv_fp8 */
};

/* flags */
enum {
    SA_FLAG_CHECK_IDX = 1u    /* report errors found on the device in *err_word (bits are
                                 OR-ed in): bit 0 (value 1) an index >= kv_rows, bit 1
                                 (value 2) a position outside [0, max_pos) with the RoPE
                                 epilogue on, bit 2 (value 4) a row sa_kv_write could not
                                 store. Without the flag nothing is reported; the
                                 handling is the same either way */
};

typedef struct sa_attn_args {
    int32_t b;          /* sequences (>= 1) */
    int32_t s;          /* queries per sequence (>= 1) */
    int32_t h;          /* heads (>= 1) */
    int32_t d;          /* latent row width: 64, 128, 256 or 512 */
    int32_t topk;       /* index columns per query (>= 1) */
    int32_t kv_rows;    /* rows of kv per sequence (>= 1) */

    const void *q;          int64_t q_seq_stride;        /* bf16 [b][s][h][d]; each
                                                            sequence's [s][h][d] contiguous */
    const void *kv;         int64_t kv_seq_stride;       /* see kv_format; each sequence's
                                                            [kv_rows][d] contiguous */
    const uint8_t *kv_scale; int64_t kv_scale_seq_stride;/* e8m0 [b][kv_rows][d/32] for
                                                            SA_KV_FP8_E4M3_B32, else NULL */
    int32_t kv_format;                                   /* SA_KV_* */
    const float *sink;                                   /* f32 [h], shared by all sequences;
                                                            a raw logit (not scaled) */
    const int32_t *idx;     int64_t idx_seq_stride;      /* int32 [b][s][topk]; values are rows
                                                            of the query's own sequence; any
                                                            negative value skips the column;
                                                            values >= kv_rows are a caller
                                                            error, skipped like a negative
                                                            value (see SA_FLAG_CHECK_IDX) */
    float scale;                                         /* softmax_scale, e.g. d^-0.5 */
    void *out;              int64_t out_seq_stride;      /* bf16 [b][s][h][d]; must not alias
                                                            q, kv or idx */

    /* optional inverse-RoPE epilogue (Attention.forward applies it to the output):
       rope_dim = 0 disables it; otherwise rope_dim is even and <= d, and the last rope_dim
       elements of every output row, taken as adjacent (real, imag) pairs, are multiplied
       in f32 by the conjugate of (cos, sin) = rope_cos_sin[pos][pair] and rounded to bf16
       again. */
    int32_t rope_dim;
    const float *rope_cos_sin; int32_t max_pos;          /* f32 [max_pos][rope_dim/2][2] */
    const int32_t *pos;     int64_t pos_seq_stride;      /* int32 [b][s] absolute positions,
                                                            each in [0, max_pos); a row at a
                                                            position outside is left
                                                            unrotated (a caller error) */

    /* workspace, sized by sa_sparse_attn_workspace (16-byte aligned; may be NULL when that
       function reports 0 bytes): the f32 partial results of plans that split the index
       columns, and, with fp8 storage whose rows are each named by many (query, column) pairs
       (prefill: at least 16 on average), the cache turned into bf16 rows by one pass before
       the attention kernel (exact, so the result is that of the bf16 rows) */
    void *workspace;        size_t workspace_bytes;

    uint32_t flags;                                      /* SA_FLAG_* */
    int32_t *err_word;                                   /* device int32, with
                                                            SA_FLAG_CHECK_IDX only; the caller
                                                            clears it beforehand */

    /* optional fused window lists: with window > 0 the first `win` columns of every index
       list are the window lists of sa_window_topk_idxs (attention API docs,
       "window_topk_idxs" and the ring-cache paragraph), generated inside the kernel from
       the query's position p = pos[n][t] instead of read from idx (whose first `win`
       columns are then never read; the caller need not fill them):
         SA_WINDOW_RING:  the decode list of a ring of `window` slots at position p, oldest
                          first: (p + 1 + j) mod window when p >= window - 1, else j for
                          j <= p and -1 beyond (a negative p lists nothing); win = window;
         SA_WINDOW_CHUNK: the prefill list into the chunk itself for the query at p: rows
                          max(0, p - window + 1) + j while <= p, then -1;
                          win = min(s, window).
       win <= topk; pos is then required (also without the epilogue). window = 0: off. */
    int32_t window;
    int32_t window_mode;                                 /* SA_WINDOW_RING or SA_WINDOW_CHUNK */
} sa_attn_args;

enum { SA_WINDOW_RING = 1, SA_WINDOW_CHUNK = 2 };

/* sparse_attn: out[n][t][hh][:] for every sequence n, query t and head hh, as described at
 * the top of this file, followed by the optional inverse-RoPE epilogue. Queries whose
 * index list selects nothing produce zeros (the sink takes the whole mass). */
int sa_sparse_attn(const sa_attn_args *a, void *stream);

/* sa_sparse_attn without a caller workspace and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The split partials of plans that need a workspace go
 * to a static device buffer of SA_NOALLOC_SCRATCH_BYTES held by the library on each GPU it
 * runs on until the process ends; a->workspace and a->workspace_bytes are ignored. Plans
 * needing more than that (sa_sparse_attn_workspace reports the bytes) are refused with
 * SA_ERR_SCRATCH before any HIP call. Nothing in the buffer has to start at zero: a call
 * writes every partial it reads. All calls on one GPU share its buffer, so calls that
 * overlap in time on one GPU (other streams, other threads) race; calls ordered on one
 * stream do not. The first call on a device looks up the buffer's device address there
 * (hipGetSymbolAddress, no allocation and no stream operation). Otherwise the same
 * arguments, results and errors as sa_sparse_attn. */
#define SA_NOALLOC_SCRATCH_BYTES (64u << 20)
int sa_sparse_attn_noalloc(const sa_attn_args *a, void *stream);

/* Bytes of workspace sa_sparse_attn needs for these arguments on the current device (only
 * the sizes, kv_format and flags are read; pointers may be NULL). Writes *bytes. */
int sa_sparse_attn_workspace(const sa_attn_args *a, size_t *bytes);

/* Window index lists of the sliding-window ring cache (attention API docs,
 * "window_topk_idxs" and the ring-cache paragraph; the slot of token p is p mod window).
 *   start_pos == NULL: prefill of seqlen tokens from position 0 in each of nseq sequences;
 *       cols = min(seqlen, window); row t lists chunk rows max(0, t-window+1) .. t in
 *       ascending order, then -1 padding.
 *   start_pos != NULL: decode, seqlen must be 1; start_pos is a device int32 [nseq] with each
 *       sequence's position P >= 0; cols = window; the list is the ring's occupied slots
 *       oldest first: (P+1+j) mod window when P >= window-1, else 0..P then -1 padding.
 *       A negative P produces a row of -1.
 *   start_pos != NULL with seqlen > 1 (a chunked prefill) is SA_ERR_UNSUPPORTED.
 * Writes idx[n * idx_seq_stride + t * idx_row_stride + j] for j < cols and *cols (host).
 * idx_row_stride >= cols; the columns from cols on are left untouched, so a caller can
 * append the compressed part of the list in place. */
int sa_window_topk_idxs(int32_t window, int32_t seqlen, int32_t nseq, const int32_t *start_pos,
                        int32_t *idx, int64_t idx_seq_stride, int64_t idx_row_stride,
                        int32_t *cols, void *stream);

/* Block-32 ue8m0 fp8 quantisation of bf16 KV rows (attention API docs, "act_quant_inplace",
 * "FP8_BLOCK" and "pow2_ceil"): for every 32 consecutive elements of a row,
 * s = pow2_ceil(max(amax, 1e-4) / 448), codes = e4m3fn(x / s) with round-to-nearest-even
 * after clamping to +-448. kv: bf16 [rows][d], d a multiple of 32.
 *   e4m3_out (nullable): bytes [rows][d];   e8m0_out (nullable): bytes [rows][d/32] holding
 *   the biased exponent of s;   bf16_out (nullable, may equal kv for in-place): the round
 *   trip codes * s, which is exact in bf16. At least one output must be given. */
int sa_quant_kv_fp8(const void *kv, int64_t rows, int32_t d, uint8_t *e4m3_out,
                    uint8_t *e8m0_out, void *bf16_out, void *stream);

/* The KV write path, the step before sparse_attn on the same cache and formats (attention
 * API docs, module notes: "a single latent KV row per token ... RoPE on the last
 * rope_head_dim ... the KV row quantised to fp8 in place (block 32, ue8m0 scale), a
 * sliding-window ring cache", and the ring-cache paragraph; Attention.forward and
 * apply_rotary_emb on the attention output page). For every row t of sequence n, in order:
 *   1. rotate the last rope_dim elements forward at position p = pos[n][t]: adjacent pairs
 *      times (cos, sin) = rope_cos_sin[p][pair], in f32, back to bf16;
 *   2. quantise to fp8 in blocks of 32 (as sa_quant_kv_fp8) and take the round trip;
 *   3. store it: window > 0: into slot p mod window of sequence n's ring (cache rows
 *      [0, window)), only for the last `window` rows of the call (t >= s - window: a prefill
 *      of s tokens leaves tokens s-window .. s-1, as in the ring-cache paragraph);
 *      window == 0: at cache row row0[n] + t (a linear cache such as the compressed one).
 *      kv_format SA_KV_BF16 stores the bf16 round trip (what the pages' cache holds);
 *      SA_KV_FP8_E4M3_B32 stores the codes and scale bytes (sparse_attn's fp8 form).
 *   rows_out (nullable) receives the bf16 round trip of every row (the chunk's kv rows that
 *   a prefill's sparse_attn reads).
 * The input rows are the normalised latent rows (after wkv and kv_norm). A row whose
 * position is negative, or >= max_pos with rope_dim > 0, is neither stored nor written to
 * rows_out; a linear destination outside [0, cache_rows) is not stored; with
 * SA_FLAG_CHECK_IDX either case ORs bit value 4 into *err_word. b * s >= 2^31 is
 * SA_ERR_UNSUPPORTED. */
typedef struct sa_kv_write_args {
    int32_t b, s, d;        /* sequences, rows per sequence, row width (64, 128, 256, 512) */
    int32_t rope_dim;       /* 0, or even and <= d */
    const void *x;          int64_t x_seq_stride;       /* bf16 [b][s][d]; [s][d] contiguous */
    const float *rope_cos_sin; int32_t max_pos;         /* f32 [max_pos][rope_dim/2][2] */
    const int32_t *pos;     int64_t pos_seq_stride;     /* int32 [b][s] token positions */
    int32_t window;                                     /* ring slots, or 0 for a linear cache */
    const int32_t *row0;                                /* int32 [b] first row (window == 0) */
    int32_t cache_rows;                                 /* rows per sequence (>= window) */
    int32_t kv_format;                                  /* SA_KV_* */
    void *cache;            int64_t cache_seq_stride;   /* bf16 [b][cache_rows][d], or e4m3
                                                           bytes [b][cache_rows][d] */
    uint8_t *cache_scale;   int64_t cache_scale_seq_stride; /* e8m0 [b][cache_rows][d/32],
                                                           fp8 only */
    void *rows_out;         int64_t rows_out_seq_stride; /* bf16 [b][s][d] or NULL */
    uint32_t flags;                                     /* SA_FLAG_CHECK_IDX or 0 */
    int32_t *err_word;                                  /* device int32, with the flag */
} sa_kv_write_args;

int sa_kv_write(const sa_kv_write_args *a, void *stream);

/* The indexer, which produces the compressed half of sparse_attn's index lists (indexer
 * page, open-model-atlas.../source-layer/attention?inspect=indexer, Indexer.forward).
 * For query t of sequence n at absolute position p = pos[n][t], the first
 * (p + 1) / ratio compressed positions are visible (p = t in a prefill from 0, end_pos - 1
 * in decode: the page's (t+1)//ratio and end_pos//ratio). For each visible position u:
 *   score[u] = sum over heads hh of w[n][t][hh] * relu(q[n][t][hh] . k[n][u])
 * in f32 from bf16 q and k (w is the caller's weights_proj output times softmax_scale *
 * h^-0.5). Positions not visible, and with cand != NULL (the second level of the two-level
 * top-k) positions whose cand byte is 0, score -inf. The scores go to `scores` (always
 * written: select_candidate_blocks reads them as its logits). With idx != NULL each query
 * then lists the topk positions with the best finite scores, in ascending position order
 * (equal scores: the lower position first), each plus `offset` (the rows before the
 * compressed ones in sparse_attn's kv), then -1 up to topk columns; the pages' list length
 * is min(index_topk, end_pos // ratio). Output: idx[n * idx_seq_stride + t * idx_row_stride
 * + j] for j < topk (other columns untouched, so the window part of a list can share the
 * row). Supported: h = 16, 32 or 64 (64 with d <= 128), d = 64, 128 or 256, n_pos <= 2^28
 * (<= 32768 when idx != NULL). Pointers are device pointers, caller-owned; q, k 16-byte aligned. */
typedef struct sa_indexer_args {
    int32_t b, s, h, d;     /* sequences, queries per sequence, index heads, index head dim */
    int32_t n_pos;          /* compressed positions of k per sequence */
    int32_t ratio;          /* compress ratio (>= 1) */
    const void *q;          int64_t q_seq_stride;        /* bf16 [b][s][h][d] */
    const void *k;          int64_t k_seq_stride;        /* bf16 [b][n_pos][d] */
    const float *w;         int64_t w_seq_stride;        /* f32 [b][s][h] */
    const int32_t *pos;     int64_t pos_seq_stride;      /* int32 [b][s] */
    const uint8_t *cand;    int64_t cand_seq_stride;     /* uint8 [b][s][n_pos] or NULL */
    float *scores;          int64_t scores_seq_stride;   /* f32 [b][s][n_pos] (output) */
    int32_t topk;           /* columns of each list (>= 1) */
    int32_t offset;         /* added to every listed position */
    int32_t *idx;           int64_t idx_seq_stride, idx_row_stride; /* int32 or NULL */
} sa_indexer_args;

int sa_indexer_topk(const sa_indexer_args *a, void *stream);

/* Level one of the two-level top-k (indexer page, select_candidate_blocks): for query t of
 * sequence n, the logits (sa_indexer_topk's scores, -inf where unreachable) are cut into
 * blocks of block_size positions, the last one padded with -inf; a block scores its
 * maximum, the block of the newest visible position ((len - 1) / block_size with floor
 * division, len = (pos + 1) / ratio as above; none when len = 0) scores +inf; the
 * min(topk_blocks, blocks) best blocks are kept if their score is above -inf (equal
 * scores: the lower block first); mask[n][t][u] = 1 for the positions u of kept blocks,
 * else 0. Supported: n_pos / block_size <= 32768 blocks. */
typedef struct sa_candidate_args {
    int32_t b, s, n_pos, ratio, topk_blocks, block_size;
    const float *logits;    int64_t logits_seq_stride;   /* f32 [b][s][n_pos] */
    const int32_t *pos;     int64_t pos_seq_stride;      /* int32 [b][s] */
    uint8_t *mask;          int64_t mask_seq_stride;     /* uint8 [b][s][n_pos] (output) */
} sa_candidate_args;

int sa_candidate_blocks(const sa_candidate_args *a, void *stream);

/* The grouped output projection, the step after sparse_attn and its inverse RoPE
 * (attention output page, Attention.forward: the output viewed as [tokens][o_groups]
 * [heads/o_groups * head_dim] is multiplied group by group with wo_a viewed as
 * [o_groups][o_lora_rank][heads/o_groups * head_dim], the einsum "bsgd,grd->bsgr"; wo_a is
 * block-diagonal over groups). For token t, group gg and row n < r:
 *   out[t][gg][n] = sum over k < kg of o[t][gg][k] * W[gg][n][k]
 * with f32 accumulation, rounded to bf16 (the attention API docs' precision paragraph: a
 * bf16 GEMM). W is bf16, or (w_format SA_KV_FP8_E4M3_B32) e4m3 codes with e8m0 scale bytes
 * per 32 consecutive k (sa_quant_kv_fp8's form, rows of kg), whose values are exact bf16
 * values: the result is the bf16 product with the decoded weights, at half the weight
 * bytes (the page's note on an fp8 grouped GEMM). Supported: kg a multiple of 64 and r a
 * multiple of 128, or m <= 64 with r a multiple of 32 and kg a multiple of 256, or with r a
 * multiple of 16 and kg a multiple of 512; other shapes return SA_ERR_UNSUPPORTED. Device
 * pointers, caller-owned, 16-byte aligned (w_scale: 4-byte aligned); strides in elements. */
typedef struct sa_grouped_proj_args {
    int32_t m;              /* tokens */
    int32_t g;              /* groups (o_groups) */
    int32_t r;              /* rows of W per group (o_lora_rank) */
    int32_t kg;             /* k per group: heads per group * head_dim */
    const void *o;          int64_t o_stride;            /* bf16 [m][>= g * kg] */
    int32_t w_format;                                    /* SA_KV_BF16 or SA_KV_FP8_E4M3_B32 */
    const void *w;                                       /* bf16 or e4m3 [g][r][kg] */
    const uint8_t *w_scale;                              /* e8m0 [g][r][kg / 32] (fp8 only) */
    void *out;              int64_t out_stride;          /* bf16 [m][>= g * r] */
} sa_grouped_proj_args;

int sa_grouped_proj(const sa_grouped_proj_args *a, void *stream);

/* The (cos, sin) table that the inverse-RoPE epilogue reads (rope_cos_sin above):
 * precompute_freqs_cis of Attention.__init__ (atlas.klimoza.dev/.../attention/output,
 * precompute_freqs_cis; attention API docs, "freqs_cis"), evaluated on the device with the
 * page's f32 roundings. Pair i of the rope tail has frequency f_i = 1 / base^(2i/rope_dim);
 * with original_seq_len > 0 the YaRN correction of the same function blends f_i towards
 * f_i / factor across the pairs between those that complete beta_fast and beta_slow turns
 * over original_seq_len positions (original_seq_len = 0: no YaRN, the ratio-0 layers'
 * form). Entry p of the table is (cos, sin) of the f32 angle p * f_i.
 *   cos_sin: device f32 [max_pos][rope_dim/2][2], caller-owned, 8-byte aligned.
 *   rope_dim even and >= 2, max_pos >= 1, base > 1 and finite; with YaRN also factor > 0
 *   and beta_fast > beta_slow > 0 (the model config's 16, 32 and 1). Errors:
 *   SA_ERR_INVALID for any other argument. */
int sa_rope_table(int32_t rope_dim, int32_t max_pos, int32_t original_seq_len, float base,
                  float factor, float beta_fast, float beta_slow, float *cos_sin, void *stream);

/* A static description of a status code. */
const char *sa_status_string(int status);

/* SA_ABI_VERSION of the built library. */
int sa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SA_H */
