/* Plain CPU oracle for DeepSeek-V4.1 sparse latent attention.
 *
 * TEST INFRASTRUCTURE ONLY. This library exists so that tests, the smoke check and the
 * bench's CPU-baseline leg can compare the GPU library against a slow, obviously correct
 * implementation written from the pages. No product code may include, link or call it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * Sources ("the pages"):
 *   [attn-docs]  docs.atlascybernetics.ai/api/spark_model/layers/deepseek_v41_ref/attn/
 *                (module attn: precision paragraph, ring-cache paragraph, FP8_BLOCK,
 *                act_quant_inplace, apply_rotary, freqs_cis, pow2_ceil, sparse_attn,
 *                window_topk_idxs)
 *   [attn-fwd]   atlas.klimoza.dev/models/deepseek-v4.1/.../attention/output?mode=prefill
 *                (Attention.forward, precompute_freqs_cis, apply_rotary_emb, Attention.__init__)
 *   [indexer]    open-model-atlas.../source-layer/attention?inspect=indexer&mode=prefill
 *                (Indexer.forward: compressed index contract)
 *
 * Every function below names the passage it follows. Where the pages are silent the reading
 * taken is stated next to the function.
 *
 * Parity status: every function here is pinned by a CPU test against something other than
 * itself (worked example, closed form, library routine, brute force). No function is
 * "parity unpinned".
 */
#ifndef SA_ORACLE_H
#define SA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- bf16 <-> f32 ([attn-docs] precision paragraph: bf16 tensors, f32 arithmetic) ---- */
float    orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);                 /* round to nearest, ties to even */
void     orc_f32_to_bf16_array(const float *x, uint16_t *y, int64_t n);
void     orc_bf16_to_f32_array(const uint16_t *x, float *y, int64_t n);

/* ---- pow2_ceil ([attn-docs] pow2_ceil): 2**ceil(log2 v) for positive normal f32 ---- */
float orc_pow2_ceil(float v);

/* ---- e4m3 (OCP e4m3fn: max 448, no infinity) ([attn-docs] act_quant_inplace) ---- */
uint8_t orc_e4m3_encode(float x);                  /* clamp to +-448, then RNE */
float   orc_e4m3_decode(uint8_t c);

/* ---- block-32 ue8m0 fp8 round trip ([attn-docs] act_quant_inplace, FP8_BLOCK) ----
 * x, y: bf16 [rows][d] (y may equal x); codes: e4m3 [rows][d] or NULL;
 * scale_bytes: e8m0 [rows][d/32] or NULL. d must be a multiple of 32. Returns 0, or -1. */
int orc_act_quant_rows(const uint16_t *x, int64_t rows, int32_t d, uint16_t *y,
                       uint8_t *codes, uint8_t *scale_bytes);
/* decode the storage form back to bf16: y = e4m3(code) * 2^(scale_byte - 127) */
int orc_fp8_storage_decode(const uint8_t *codes, const uint8_t *scale_bytes, int64_t rows,
                           int32_t d, uint16_t *y);

/* ---- window index lists ([attn-docs] window_topk_idxs and ring-cache paragraph) ----
 * Writes idx [nseq][seqlen][cols] and *cols. Prefill (start_pos == NULL, every sequence
 * from position 0): cols = min(seqlen, window). Decode (start_pos != NULL, one position
 * P >= 0 per sequence, seqlen == 1): cols = window.
 * Returns 0, -1 on invalid arguments, -2 for a decode call with seqlen > 1 (a chunked
 * prefill, which the pages do not define). */
int orc_window_topk_idxs(int32_t window, int32_t seqlen, const int32_t *start_pos, int32_t nseq,
                         int32_t *idx, int32_t *cols);
/* query the column count only (same rules) */
int orc_window_cols(int32_t window, int32_t seqlen, const int32_t *start_pos, int32_t nseq,
                    int32_t *cols);

/* ---- ring writes of the window cache ([attn-docs] ring-cache paragraph; [attn-fwd]
 * window_kv_cache buffer). ring: [window][row_elems] of any 2-byte type. ---- */
void orc_ring_prefill(uint16_t *ring, int32_t window, int32_t row_elems,
                      const uint16_t *chunk_rows, int32_t seqlen);
void orc_ring_decode(uint16_t *ring, int32_t window, int32_t row_elems,
                     const uint16_t *row, int32_t pos);

/* ---- sparse_attn ([attn-docs] sparse_attn and precision paragraph; call in
 * [attn-fwd] Attention.forward) ---- */
typedef struct {
    int32_t b, s, h, d, topk, kv_rows;
    const uint16_t *q;   int64_t q_seq_stride;    /* bf16 [b][s][h][d] */
    const uint16_t *kv;  int64_t kv_seq_stride;   /* bf16 [b][kv_rows][d] */
    const float *sink;                            /* f32 [h] */
    const int32_t *idx;  int64_t idx_seq_stride;  /* int32 [b][s][topk]; < 0 skips */
    float scale;
} orc_attn_problem;

/* qsel: flattened query ids (seq*s + t) to compute, or NULL for all b*s queries.
 * out: bf16 [nsel][h][d]. nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on invalid arguments / an index >= kv_rows. */
int orc_sparse_attn(const orc_attn_problem *p, const int64_t *qsel, int64_t nsel,
                    uint16_t *out, int32_t nthreads);
/* the same arithmetic in f64, unrounded output f64 [nsel][h][d]; for tests */
int orc_sparse_attn_f64(const orc_attn_problem *p, const int64_t *qsel, int64_t nsel,
                        double *out, int32_t nthreads);
/* the softmax weights of one (query, head), f64, over the topk columns (0 for skipped
 * columns) and the sink's share; for tests of the denominator. */
int orc_sparse_attn_weights_f64(const orc_attn_problem *p, int64_t query, int32_t head,
                                double *w, double *sink_share);

/* ---- rotary table ([attn-fwd] precompute_freqs_cis without YaRN; [attn-docs] freqs_cis)
 * cos_sin: f32 [max_pos][rd/2][2] = (cos, sin) of pos * base^(-2i/rd), computed in f32. */
void orc_freqs_cis(int32_t rd, int32_t max_pos, float base, float *cos_sin);
/* the same with the YaRN correction of precompute_freqs_cis when original_seq_len > 0
 * (factor, beta_fast, beta_slow as the page names them). Returns 0, or -1. */
int orc_freqs_cis_yarn(int32_t rd, int32_t max_pos, int32_t original_seq_len, float base,
                       float factor, float beta_fast, float beta_slow, float *cos_sin);

/* ---- rotary ([attn-fwd] apply_rotary_emb; [attn-docs] apply_rotary) on the last rd
 * elements of every d-wide row of x (bf16 [n][h][d], in place); row i at position pos[i].
 * inverse != 0 multiplies by the conjugate. Returns 0, or -1. */
int orc_apply_rotary(uint16_t *x, int64_t n, int32_t h, int32_t d, int32_t rd,
                     const float *cos_sin, int32_t max_pos, const int32_t *pos, int32_t inverse);

/* ---- KV write path ([attn-docs] module notes and ring-cache paragraph; [attn-fwd]
 * Attention.forward, apply_rotary_emb): x bf16 [b][s][d] normalised latent rows, pos int32
 * [b][s]; each row is rotated forward on its last rd elements at pos, fp8 round-tripped
 * (block 32) and stored: window > 0: slot pos mod window of sequence n's ring, only for
 * t >= s - window; window == 0: row row0[n] + t. Caches are [b][cache_rows][...]: bf16 rows
 * (cache_bf16) and/or e4m3 codes + e8m0 scale bytes; rows_out (nullable) bf16 [b][s][d]
 * gets every processed row. Returns 0, or -1. */
int orc_kv_write(const uint16_t *x, int32_t b, int32_t s, int32_t d, int32_t rd,
                 const float *cos_sin, int32_t max_pos, const int32_t *pos, int32_t window,
                 const int32_t *row0, int32_t cache_rows, uint16_t *cache_bf16,
                 uint8_t *cache_codes, uint8_t *cache_scales, uint16_t *rows_out);

/* ---- indexer ([indexer] Indexer.forward, select_candidate_blocks) ----
 * q bf16 [b][s][h][d] index queries; k bf16 [b][n_pos][d] index keys; w f32 [b][s][h] head
 * weights; pos int32 [b][s] absolute query positions; a query at p sees the first
 * (p+1)/ratio positions. cand (nullable) uint8 [b][s][n_pos]: 1 = candidate.
 * scores f32 [b][s][n_pos]: sum_h w_h relu(q_h . k_t), -inf where not visible / candidate. */
int orc_index_scores(const uint16_t *q, const uint16_t *k, const float *w, const int32_t *pos,
                     const uint8_t *cand, int32_t b, int32_t s, int32_t h, int32_t d,
                     int32_t n_pos, int32_t ratio, float *scores, int32_t nthreads);
/* idx int32 [b][s][topk]: the topk best finite scores (ties: lower position first) in
 * ascending position order, + offset, then -1. */
int orc_index_topk(const float *scores, int32_t b, int32_t s, int32_t n_pos, int32_t topk,
                   int32_t offset, int32_t *idx);
/* mask uint8 [b][s][n_pos] of select_candidate_blocks (ties: lower block first) */
int orc_candidate_blocks(const float *logits, const int32_t *pos, int32_t b, int32_t s,
                         int32_t n_pos, int32_t ratio, int32_t topk_blocks, int32_t block_size,
                         uint8_t *mask);

/* ---- grouped output projection ([attn-fwd] Attention.forward, the wo_a einsum):
 * out bf16 [m][g][r] = per group gg, o[t][gg][:] . w[gg][rr][:] in f32, rounded to bf16.
 * o: bf16 tokens of g * kg elements at stride o_stride; w: bf16 [g][r][kg]. */
int orc_grouped_proj(const uint16_t *o, int64_t o_stride, const uint16_t *w, int32_t m,
                     int32_t g, int32_t r, int32_t kg, uint16_t *out, int32_t nthreads);

/* threads an nthreads <= 0 call uses (the OpenMP default), 1 without OpenMP */
int32_t orc_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
