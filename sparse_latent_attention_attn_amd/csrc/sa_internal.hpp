// Internal interface between the C-ABI entry points (sa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sa.h"

namespace sa {

// Tiling shared by the planner (sa_api.cpp) and the kernels (attn_fwd.hip).
constexpr int kTileKeys = 32;       // index columns per key tile
constexpr int kHeadsPerWave = 16;   // heads in one block (the N of a 16x16 MFMA tile)
constexpr int kMaxWaves = 4;        // waves per workgroup
constexpr int kMaxColsPerSplit = 4096;  // index columns one workgroup stages in LDS
constexpr int kMaxColsCompact = 256;    // the same in the compact layout (two workgroups per CU)
constexpr int kMaxColsFp8Pipe = 3072;   // the same for fp8 storage at d = 512 (its raw slots take the rest)

// Everything one sparse_attn launch needs, passed by value as the kernel argument.
struct KParams {
    int32_t b, s, h, d, topk, kv_rows;
    const uint16_t* q;       int64_t q_seq_stride;          // elements
    const uint8_t* kv;       int64_t kv_seq_stride_bytes;   // bytes
    const uint8_t* kv_scale; int64_t kv_scale_seq_stride;   // bytes
    const float* sink;
    const int32_t* idx;      int64_t idx_seq_stride;        // elements
    float scale_log2;                                      // softmax_scale * log2(e)
    uint16_t* out;           int64_t out_seq_stride;        // elements
    int32_t rope_dim;
    const float* rope_cs;    int32_t max_pos;
    const int32_t* pos;      int64_t pos_seq_stride;
    float* ws_o;                                           // [b*s][splits][h_pad][d]
    float* ws_ml;                                          // [b*s][splits][h_pad][2]
    int32_t splits, cols_per_split, head_blocks, h_pad;
    uint32_t flags;
    int32_t* err_word;
    int32_t window, window_mode, win_cols;                  // fused window lists (0: off)
};

// One sa_kv_write launch (pointers already offset to element 0; strides in elements of the
// pointed-to type).
struct KvWriteParams {
    int32_t b, s, d, rope_dim;
    const uint16_t* x;       int64_t x_seq_stride;
    const float* rope_cs;    int32_t max_pos;
    const int32_t* pos;      int64_t pos_seq_stride;
    int32_t window;
    const int32_t* row0;
    int32_t cache_rows;
    uint16_t* cache_bf16;    int64_t cache_seq_stride;          // bf16 storage
    uint8_t* cache_codes;                                      // fp8 storage (same stride, bytes)
    uint8_t* cache_scales;   int64_t cache_scale_seq_stride;
    uint16_t* rows_out;      int64_t rows_out_seq_stride;
    uint32_t flags;
    int32_t* err_word;
};

// One indexer launch (sa_indexer_topk): scores, then the top-k lists.
struct IdxParams {
    int32_t b, s, h, d, n_pos, ratio;
    const uint16_t* q;       int64_t q_seq_stride;        // elements
    const uint16_t* k;       int64_t k_seq_stride;
    const float* w;          int64_t w_seq_stride;
    const int32_t* pos;      int64_t pos_seq_stride;
    const uint8_t* cand;     int64_t cand_seq_stride;
    float* scores;           int64_t scores_seq_stride;
    int32_t topk, offset;
    int32_t* idx;            int64_t idx_seq_stride, idx_row_stride;
};

// One sa_candidate_blocks launch.
struct CandParams {
    int32_t b, s, n_pos, ratio, topk_blocks, block_size;
    const float* logits;     int64_t logits_seq_stride;
    const int32_t* pos;      int64_t pos_seq_stride;
    uint8_t* mask;           int64_t mask_seq_stride;
};

// One grouped output projection (sa_grouped_proj): out[t][gg][:] = o[t][gg][:] . W[gg]^T.
struct ProjParams {
    int32_t m, g, r, kg;                 // tokens, groups, rows of W per group, K per group
    const uint16_t* o;       int64_t o_stride;       // bf16 tokens, stride in elements
    const uint16_t* w;                              // bf16 [g][r][kg], or null with fp8
    const uint8_t* wq;       const uint8_t* ws;     // e4m3 [g][r][kg] + e8m0 [g][r][kg/32]
    uint16_t* out;           int64_t out_stride;     // bf16 [m][g][r], stride in elements
};

// Split plan shared by sa_sparse_attn and sa_sparse_attn_workspace.
struct Plan {
    int nw;             // waves per workgroup
    int hpw;            // blocks of 16 heads per wave (1, or 2 for wide bf16 d = 512 work)
    int kg;             // key groups: waves that share a query's heads and split its tiles
    int head_blocks;
    int h_pad;
    int splits;
    int cols_per_split; // a multiple of the key tile
    bool compact;       // two-wave workgroups with a two-tile ring, two of them per compute unit
    bool dequant;       // fp8 storage turned into bf16 rows at the start of the workspace first
    size_t dq_bytes;    // bytes of those rows (0 without)
    size_t ws_bytes;    // the whole workspace: dequantised rows, then the split partials
};

// Validation, plan and kernel parameters of a sparse_attn call (sa_api.cpp); returns an SA_*
// status. ws / ws_bytes: the buffer of the split partials.
int prepare_sparse_attn(const sa_attn_args* a, void* ws, size_t ws_bytes, KParams& p, Plan& pl);
hipError_t launch_sparse_attn(const KParams& p, bool fp8, int nw, int hpw, int kg, bool compact, hipStream_t st);
// The kernels of a prepared call: the dequantisation pass when the plan has one, then
// sparse_attn (and its combine kernel).
hipError_t run_sparse_attn(const sa_attn_args* a, const KParams& p, const Plan& pl, hipStream_t st);
// fp8 storage rows (e4m3 codes [b][rows][d] + e8m0 scales [b][rows][d/32], sequence strides
// in bytes) to bf16 rows [b][rows][d], contiguous.
hipError_t launch_dequant_kv(const uint8_t* codes, int64_t codes_seq_stride, const uint8_t* scales,
                             int64_t scales_seq_stride, int b, int rows, int d, uint16_t* out, hipStream_t st);
hipError_t launch_window_idxs(int32_t window, int32_t seqlen, int32_t nseq, const int32_t* start_pos,
                              int32_t* idx, int64_t seq_stride, int64_t row_stride, int32_t cols,
                              hipStream_t st);
hipError_t launch_rope_table(int32_t rope_dim, int32_t max_pos, float base, int32_t yarn, int32_t low,
                             int32_t high, float factor, float* cs, hipStream_t st);
hipError_t launch_index_scores(const IdxParams& p, hipStream_t st);
hipError_t launch_index_topk(const IdxParams& p, hipStream_t st);
hipError_t launch_candidate_blocks(const CandParams& p, hipStream_t st);
hipError_t launch_grouped_proj(const ProjParams& p, hipStream_t st);
hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t st);
hipError_t launch_quant_fp8(const uint16_t* kv, int64_t rows, int32_t d, uint8_t* codes,
                            uint8_t* scales, uint16_t* rt, hipStream_t st);

}  // namespace sa
