// The indexer that produces the compressed half of sparse_attn's index lists (the indexer
// page: Indexer.forward and select_candidate_blocks), on gfx950:
//   * index_scores_kernel: score[t] = sum_h w_h relu(q_h . k_t) per query, on bf16 MFMA with
//     f32 accumulation; positions the query cannot see (and, for the second level, positions
//     outside the candidate mask) are -inf;
//   * index_topk_kernel: per query, the topk best finite scores by a threshold search over
//     keys held in registers (bit by bit with one wave per query; with several, halving a key
//     interval bracketed from a sample), listed in position order (ties: the lower position
//     first), shifted by the offset and padded with -1;
//   * candidate_wave_kernel (blocks of 4, 8 or 16 in rows of whole 16-byte mask pieces) and
//     candidate_blocks_kernel (other shapes): per query, block maxima, the newest visible
//     block pinned, the best blocks kept (the wave kernel by the same threshold search, the
//     other by a radix select in LDS), expanded to a position mask.
#include "lds_dma.hpp"
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

// ------------------------------------------------------------------ scores
// Positions a query at absolute position p can see: the first (p + 1) / ratio ("a block
// becomes visible once the query has passed its last token").
__device__ __forceinline__ int visible_positions(int pos, int ratio, int n_pos) {
    if (pos < 0) return 0;
    const int64_t v = ((int64_t)pos + 1) / ratio;
    return v < n_pos ? (int)v : n_pos;
}

// Row t of sequence n of a [b][s][n_pos] array of `bytes_per`-byte elements as a buffer:
// stores at an offset past its end are dropped and loads there return zero, so lanes that
// have nothing to store or load need no branch (a branch around a memory operation makes
// the compiler's wait counts assume the worst on both paths, which in a pipelined loop
// means waiting for every load in flight). Rows of dead queries (t >= s) get no records.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t score_row(const void* base, int64_t seq_stride, int n, int t,
                                                            int s, int n_pos, int bytes_per) {
    const uint8_t* row = (const uint8_t*)base + ((int64_t)n * seq_stride + (int64_t)min(t, s - 1) * n_pos) * bytes_per;
    return __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, t < s ? n_pos * bytes_per : 0, 0x00020000);
}

__device__ __forceinline__ void store_score(__amdgpu_buffer_rsrc_t row, int pp, bool on, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(f32_bits(v), row, on ? pp * 4 : kBufferPastEnd, 0, 0);
}

// relu(x) as one median of three (x, 0, +inf): fmaxf(x, 0) costs a canonicalising max first
// in IEEE mode. The upper bound goes through an empty asm so that the compiler cannot see it
// is +inf (it would turn the median back into that max). NaN gives 0 (with a NaN operand the
// median of three is their minimum), as fmaxf does.
__device__ __forceinline__ float relu_inf() {
    float v = INFINITY;
    asm("" : "+s"(v));
    return v;
}
__device__ __forceinline__ float relu_f32(float x, float inf) { return __builtin_amdgcn_fmed3f(x, 0.0f, inf); }

// S[head][position] = Q . K^T on v_mfma_f32_16x16x32_bf16: Q is the A operand (rows = 16
// heads, held in registers), K the B operand (columns = 16 positions, loaded straight from
// memory, one 16-byte piece per lane and k-step). In the accumulator each lane holds one
// position and 4 heads, so the weighted head sum is in-lane work plus two exchanges across
// the lane groups. A wave takes QPW queries of one sequence (sharing every K load) and
// kScoreChunk positions, with the keys of kScoreAhead blocks of 16 positions in flight; a
// workgroup is 4 such waves. CAND: positions outside the candidate mask score -inf (its
// bytes are loaded with the keys).
constexpr int kScoreChunk = 256, kScoreAhead = 3;

template <int D, int HB, int QPW, bool CAND>
__global__ __launch_bounds__(256) void index_scores_kernel(const IdxParams p) {
    constexpr int KS = D / 32;
    // the wave index in a scalar register: the buffer resources built from it below must be
    // uniform (a resource in vector registers costs a loop around every access)
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int groups = (p.s + QPW - 1) / QPW;                   // query groups per sequence
    const int64_t wave = (int64_t)blockIdx.x * 4 + wid;
    if (wave >= (int64_t)p.b * groups) return;                  // no barriers in this kernel
    const int n = (int)(wave / groups);
    const int t0 = (int)(wave % groups) * QPW;
    // chunks staggered by sequence: the waves in flight together then read at different
    // offsets of their sequences' keys rather than all at the same one (4 MB apart at 16384
    // positions; 79 -> 75 us on 64 sequences x 16384 positions)
    const int c0 = (int)((blockIdx.y + (uint32_t)n * 7u) % gridDim.y) * kScoreChunk;
    const int cend = min(p.n_pos, c0 + kScoreChunk);

    int vis[QPW];
    int vmax = 0;
    __amdgpu_buffer_rsrc_t srow[QPW], crow[QPW];
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        const bool live = t0 + j < p.s;
        vis[j] = live ? visible_positions(p.pos[(int64_t)n * p.pos_seq_stride + t0 + j], p.ratio, p.n_pos) : 0;
        vmax = max(vmax, vis[j]);
        srow[j] = score_row(p.scores, p.scores_seq_stride, n, t0 + j, p.s, p.n_pos, 4);
        if constexpr (CAND) crow[j] = score_row(p.cand, p.cand_seq_stride, n, t0 + j, p.s, p.n_pos, 1);
    }
    const int vend = min(cend, vmax);                            // blocks with a visible position
    if (vend <= c0) {
        // nothing visible in this chunk: -inf throughout, no keys needed
        for (int pb = c0; pb < cend; pb += 16) {
            const int pp = pb + l16;
#pragma unroll
            for (int j = 0; j < QPW; ++j) store_score(srow[j], pp, g == 0 && pp < cend, -INFINITY);
        }
        return;
    }
    const uint16_t* kseq = p.k + (int64_t)n * p.k_seq_stride;
    // Q of each query: A operand of (head block mb, k-step kk): head 16 mb + l16, d 32 kk + 8 g
    u32x4 qa[QPW][HB][KS];
    float wv[QPW][HB][4];
    const float pinf = relu_inf();
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        const int t = min(t0 + j, p.s - 1);
        const uint16_t* qq = p.q + (int64_t)n * p.q_seq_stride + (int64_t)t * p.h * D;
        const float* ww = p.w + (int64_t)n * p.w_seq_stride + (int64_t)t * p.h;
#pragma unroll
        for (int mb = 0; mb < HB; ++mb) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                qa[j][mb][kk] = *(const u32x4*)(qq + (int64_t)(16 * mb + l16) * D + 32 * kk + 8 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[j][mb][r] = ww[16 * mb + 4 * g + r];
        }
    }
    // Keys (and candidate bytes) of block pb: positions past the last visible one re-read it,
    // so every block issues the same loads.
    const int klast = vend - 1;
    auto load_blk = [&](int pb, u32x4 (&kb)[KS], uint32_t (&cb)[QPW]) {
        const int pp = min(pb + l16, klast);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) kb[kk] = *(const u32x4*)(kseq + (int64_t)pp * D + 32 * kk + 8 * g);
        if constexpr (CAND) {
#pragma unroll
            for (int j = 0; j < QPW; ++j) cb[j] = __builtin_amdgcn_raw_buffer_load_b8(crow[j], pp, 0, 0);
        }
    };
    // one 16-position block: its operands are in (cur, ccur); those of the block kScoreAhead
    // blocks later go to (nxt, cnxt), the buffers the previous block used
    auto step = [&](int pb, const u32x4 (&cur)[KS], const uint32_t (&ccur)[QPW], u32x4 (&nxt)[KS],
                    uint32_t (&cnxt)[QPW]) {
        load_blk(pb + 16 * kScoreAhead, nxt, cnxt);
        const int pp = pb + l16;
        const bool any = pb < vend;                              // wave-uniform
#pragma unroll
        for (int j = 0; j < QPW; ++j) {
            float part = 0.0f;
            if (any) {
                f32x4 acc[HB];
#pragma unroll
                for (int mb = 0; mb < HB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                    for (int mb = 0; mb < HB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, qa[j][mb][kk]), __builtin_bit_cast(bf16x8, cur[kk]), acc[mb], 0, 0, 0);
#pragma unroll
                for (int mb = 0; mb < HB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) part += wv[j][mb][r] * relu_f32(acc[mb][r], pinf);
                part = sum_xor32(sum_xor16(part));
            }
            bool keep = pp < vis[j];
            if constexpr (CAND) keep = keep && ccur[j] != 0;
            store_score(srow[j], pp, g == 0 && pp < cend, keep ? part : -INFINITY);
        }
    };
    // A ring of kScoreAhead + 1 operand buffers over the chunk's blocks, fully unrolled:
    // straight-line code, so the compiler's wait before each block counts exactly the loads
    // issued after it (a loop back edge would make it wait for all of them). Steps past the
    // end of a short last chunk load clamped keys and store nothing.
    constexpr int NBUF = kScoreAhead + 1;
    u32x4 kr[NBUF][KS];
    uint32_t cr[NBUF][QPW];
#pragma unroll
    for (int j = 0; j < kScoreAhead; ++j) load_blk(c0 + 16 * j, kr[j], cr[j]);
#pragma unroll
    for (int u = 0; u < kScoreChunk / 16; ++u)
        step(c0 + 16 * u, kr[u % NBUF], cr[u % NBUF], kr[(u + kScoreAhead) % NBUF], cr[(u + kScoreAhead) % NBUF]);
}

// The same scores for many queries of one sequence (prefill): a workgroup of 4 waves takes
// 8 consecutive queries (2 per wave) and walks their visible positions in tiles of 64 keys,
// staged in LDS by contiguous 16-byte loads (8 cache lines per load instruction instead of
// the 16 rows x 64 bytes of an operand-shaped load) and double-buffered; each wave reads its B
// operands from LDS (rows XOR-swizzled in 16-byte chunks so that the 16 rows of an operand
// read fall in distinct banks). Every staged key then feeds 8 queries x h heads.
constexpr int kLdsQueries = 8, kLdsTile = 64;

template <int D, int HB, bool CAND>
__global__ __launch_bounds__(256) void index_scores_lds_kernel(const IdxParams p) {
    constexpr int KS = D / 32, CH = D / 8;                      // k-steps; 16-byte chunks per row
    constexpr int kTileBytes = kLdsTile * D * 2;
    constexpr int kPer = kTileBytes / 16 / 256;                 // staging loads per thread
    __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kTileBytes];
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int n = blockIdx.y;
    // this wave's two queries; the last query groups go first: in a prefill chunk positions
    // grow along the chunk, so the longest score rows start first and the short ones fill
    // the tail (8192 queries x 2048 positions: 116 -> 99 us against the chunk order)
    const int t0 = (gridDim.x - 1 - blockIdx.x) * kLdsQueries + 2 * wid;
    int vis[2];
    int vmax_w = 0;
    __amdgpu_buffer_rsrc_t srow[2], crow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        vis[j] = t0 + j < p.s ? visible_positions(p.pos[(int64_t)n * p.pos_seq_stride + t0 + j], p.ratio, p.n_pos) : 0;
        vmax_w = max(vmax_w, vis[j]);
        srow[j] = score_row(p.scores, p.scores_seq_stride, n, t0 + j, p.s, p.n_pos, 4);
        if constexpr (CAND) crow[j] = score_row(p.cand, p.cand_seq_stride, n, t0 + j, p.s, p.n_pos, 1);
    }
    // the workgroup's extent: the maximum over its 8 queries (all waves walk the same tiles)
    __shared__ int vmax_s[4];
    if (lane == 0) vmax_s[wid] = vmax_w;
    __syncthreads();
    const int vmax = max(max(vmax_s[0], vmax_s[1]), max(vmax_s[2], vmax_s[3]));
    const uint16_t* kseq = p.k + (int64_t)n * p.k_seq_stride;
    u32x4 qa[2][HB][KS];
    float wv[2][HB][4];
    const float pinf = relu_inf();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = min(t0 + j, p.s - 1);
        const uint16_t* qq = p.q + (int64_t)n * p.q_seq_stride + (int64_t)t * p.h * D;
        const float* ww = p.w + (int64_t)n * p.w_seq_stride + (int64_t)t * p.h;
#pragma unroll
        for (int mb = 0; mb < HB; ++mb) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                qa[j][mb][kk] = *(const u32x4*)(qq + (int64_t)(16 * mb + l16) * D + 32 * kk + 8 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[j][mb][r] = ww[16 * mb + 4 * g + r];
        }
    }
    // staging: load u of thread tid moves chunk (tid + 256 u) of the tile (row = chunk / CH);
    // rows past the last visible position re-read it
    const int klast = max(vmax, 1) - 1;
    u32x4 st[kPer];
    auto fetch = [&](int tb) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int c = tid + 256 * u, row = c / CH;
            const int pp = min(tb + row, klast);
            st[u] = *(const u32x4*)(kseq + (int64_t)pp * D + 8 * (c % CH));
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int c = tid + 256 * u, row = c / CH, ch = c % CH;
            *(SA_LDS u32x4*)((SA_LDS uint8_t*)tiles[buf] + row * (D * 2) + ((ch ^ (row & (CH - 1) & 15)) << 4)) = st[u];
        }
    };
    const int ntiles = (vmax + kLdsTile - 1) / kLdsTile;
    const int nall = (p.n_pos + kLdsTile - 1) / kLdsTile;
    if (ntiles > 0) {
        fetch(0);
        stage(0);
    }
    // Q, the weights and the first tile have landed: no load from before the loop is still
    // counted inside it (the loop's waits then count only its own loads and stores)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // The loop issues the same memory operations on every path: the next tile's loads (the
    // last iteration re-reads its own tile), one buffer store per score (dropped for lanes
    // and positions that store nothing), and the staging of the next tile (the last copy is
    // never read).
    for (int it = 0; it < ntiles; ++it) {
        const int tb = it * kLdsTile;
        uint32_t cb[kLdsTile / 16][2];
        if constexpr (CAND) {
            // this tile's candidate bytes, before the next tile's loads so that waiting for
            // them never waits for those
#pragma unroll
            for (int nb = 0; nb < kLdsTile / 16; ++nb)
#pragma unroll
                for (int j = 0; j < 2; ++j) cb[nb][j] = __builtin_amdgcn_raw_buffer_load_b8(crow[j], tb + 16 * nb + l16, 0, 0);
        }
        fetch(min(tb + kLdsTile, (ntiles - 1) * kLdsTile));
        SA_LDS const uint8_t* tile = (SA_LDS const uint8_t*)tiles[it & 1];
#pragma unroll
        for (int nb = 0; nb < kLdsTile / 16; ++nb) {
            const int row = 16 * nb + l16, pp = tb + row;
            u32x4 kb[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                kb[kk] = *(SA_LDS const u32x4*)(tile + row * (D * 2) + (((4 * kk + g) ^ (row & (CH - 1) & 15)) << 4));
            // both queries' head blocks accumulate side by side (k-step outermost): 2 HB
            // independent accumulators between dependent matrix instructions
            f32x4 acc[2][HB];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int mb = 0; mb < HB; ++mb) acc[j][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int mb = 0; mb < HB; ++mb)
                        acc[j][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, qa[j][mb][kk]), __builtin_bit_cast(bf16x8, kb[kk]), acc[j][mb], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // two partial sums per lane, added at the end
                float part2[2] = {0.0f, 0.0f};
#pragma unroll
                for (int mb = 0; mb < HB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) part2[r & 1] += wv[j][mb][r] * relu_f32(acc[j][mb][r], pinf);
                const float part = sum_xor32(sum_xor16(part2[0] + part2[1]));
                bool keep = pp < vis[j];
                if constexpr (CAND) keep = keep && cb[nb][j] != 0;
                store_score(srow[j], pp, g == 0 && pp < p.n_pos, keep ? part : -INFINITY);
            }
        }
        stage((it + 1) & 1);
        __syncthreads();
    }
    // tiles past every query's visible positions: -inf, no keys needed
    for (int it = ntiles; it < nall; ++it) {
        const int pp = it * kLdsTile + lane;
#pragma unroll
        for (int j = 0; j < 2; ++j) store_score(srow[j], pp, pp < p.n_pos, -INFINITY);
    }
}

// The prefill scores for 32 index heads (the model's indexer shape) on
// v_mfma_f32_32x32x16_bf16: one 32 x 32 tile holds S[head][position] for all heads of a query
// and 32 positions. In that accumulator lane l holds position l % 32 and 16 of the heads (the
// other 16 are in lane l ^ 32), so the weighted head sum is 16 in-lane terms, and a single
// permlane32 swap completes it for both of the wave's queries at once: lanes 0..31 end with
// the first query's 32 scores, lanes 32..63 with the second's, and one store writes both rows.
// Against the 16 x 16 form this halves the non-matrix instructions per score, which bound
// that loop. Workgroups as in index_scores_lds_kernel (8 queries, 4 waves of 2, key tiles of
// 64 rows staged in LDS, double-buffered), with two differences: the staged rows are padded
// by 16 bytes instead of swizzled (the 16 rows of each operand read still fall in distinct
// banks, and every LDS address is a fixed per-lane base plus an immediate), and the keys come
// in through a buffer resource per tile whose rows past the workgroup's last visible position
// read as zero (the scores of those positions are masked like any invisible one's).
template <int D, bool CAND>
__global__ __launch_bounds__(256) void index_scores_h32_kernel(const IdxParams p) {
    static_assert(D == 64 || D == 128, "32-head scores: D is 64 or 128");
    constexpr int KS = D / 16;                                  // k-steps of 16
    constexpr int CH = D / 8;                                   // 16-byte chunks per key row
    constexpr int RB = D * 2 + 16;                              // padded LDS row
    constexpr int kTileBytes = kLdsTile * RB;
    constexpr int kPer = kLdsTile * CH / 256;                   // staging loads per thread
    constexpr int kRowsPer = 256 / CH;                          // rows per staging load
    __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kTileBytes];
    __shared__ int vmax_s[4];
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int n = blockIdx.y;
    // the wave's two queries t0, t0 + 1 (the last query groups first, as above); lane half hi
    // stores row t0 + hi
    const int t0 = (gridDim.x - 1 - blockIdx.x) * kLdsQueries + 2 * wid;
    const int tl = min(t0, p.s - 1);
    const int live = max(0, min(2, p.s - t0));                  // rows of the pair that exist
    const int32_t* posq = p.pos + (int64_t)n * p.pos_seq_stride;
    const int vis0 = live > 0 ? visible_positions(posq[t0], p.ratio, p.n_pos) : 0;
    const int vis1 = live > 1 ? visible_positions(posq[t0 + 1], p.ratio, p.n_pos) : 0;
    const int vis_l = hi ? vis1 : vis0;
    if (lane == 0) vmax_s[wid] = max(vis0, vis1);
    // both score rows (and candidate rows) as one buffer: stores past the live rows are dropped
    const __amdgpu_buffer_rsrc_t srows = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.scores + (int64_t)n * p.scores_seq_stride + (int64_t)tl * p.n_pos), 0,
        __builtin_amdgcn_readfirstlane((int)((uint32_t)live * (uint32_t)p.n_pos * 4u)), 0x00020000);
    __amdgpu_buffer_rsrc_t crows;
    if constexpr (CAND)
        crows = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.cand + (int64_t)n * p.cand_seq_stride + (int64_t)tl * p.n_pos), 0,
            __builtin_amdgcn_readfirstlane((int)((uint32_t)live * (uint32_t)p.n_pos)), 0x00020000);
    const int rowoff = hi * p.n_pos;                            // the lane's row, in elements
    // Q: A operand of k-step kk is head l32, d 16 kk + 8 hi; w of accumulator element r is
    // that of head 8 (r / 4) + 4 hi + r % 4
    u32x4 qa[2][KS];
    float wv[2][16];
    const float pinf = relu_inf();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = min(t0 + j, p.s - 1);
        const uint16_t* qq = p.q + (int64_t)n * p.q_seq_stride + (int64_t)t * 32 * D + l32 * D + 8 * hi;
        const float* ww = p.w + (int64_t)n * p.w_seq_stride + (int64_t)t * 32 + 4 * hi;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) qa[j][kk] = *(const u32x4*)(qq + 16 * kk);
#pragma unroll
        for (int r = 0; r < 16; ++r) wv[j][r] = ww[8 * (r / 4) + r % 4];
    }
    __syncthreads();
    const int vmax = __builtin_amdgcn_readfirstlane(max(max(vmax_s[0], vmax_s[1]), max(vmax_s[2], vmax_s[3])));
    const uint16_t* kseq = p.k + (int64_t)n * p.k_seq_stride;
    // staging: load u of thread tid moves bytes 16 (tid + 256 u) of tile tb's rows, i.e. row
    // tid / CH + kRowsPer u, chunk tid % CH
    u32x4 st[kPer];
    // (the clamps below would otherwise be computed by a vector median instruction, and a
    // buffer resource in vector registers costs a loop around every access)
    auto fetch = [&](int tb) {
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kseq + (int64_t)tb * D), 0, __builtin_amdgcn_readfirstlane(max(0, min(kLdsTile, vmax - tb)) * D * 2),
            0x00020000);
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            st[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, 16 * tid + 4096 * u, 0, 0));
    };
    const int wbase = (tid / CH) * RB + (tid % CH) * 16;
    auto stage = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            *(SA_LDS u32x4*)((SA_LDS uint8_t*)tiles[buf] + wbase + kRowsPer * RB * u) = st[u];
    };
    const int ntiles = (vmax + kLdsTile - 1) / kLdsTile;
    const int nall = (p.n_pos + kLdsTile - 1) / kLdsTile;
    if (ntiles > 0) {
        fetch(0);
        stage(0);
    }
    // Q, w and the first tile have landed: the loop's waits count only its own memory operations
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int rbase = l32 * RB + hi * 16;                       // B operand: row l32, chunk 2 kk + hi
    // Each iteration issues the same memory operations on every path (as in
    // index_scores_lds_kernel): the next tile's loads (the last one re-reads its own tile),
    // one store per 32 positions, the staging of the next tile.
    for (int it = 0; it < ntiles; ++it) {
        const int tb = it * kLdsTile;
        uint32_t cb[kLdsTile / 32];
        if constexpr (CAND) {
#pragma unroll
            for (int nb = 0; nb < kLdsTile / 32; ++nb) {
                const int pp = tb + 32 * nb + l32;
                cb[nb] = __builtin_amdgcn_raw_buffer_load_b8(crows, pp < p.n_pos ? rowoff + pp : kBufferPastEnd, 0, 0);
            }
        }
        fetch(min(tb + kLdsTile, (ntiles - 1) * kLdsTile));
        SA_LDS const uint8_t* tile = (SA_LDS const uint8_t*)tiles[it & 1] + rbase;
#pragma unroll
        for (int nb = 0; nb < kLdsTile / 32; ++nb) {
            f32x16 acc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
            u32x4 kb[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) kb[kk] = *(SA_LDS const u32x4*)(tile + 32 * nb * RB + 32 * kk);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, qa[j][kk]), __builtin_bit_cast(bf16x8, kb[kk]), acc[j], 0, 0, 0);
            }
            // Schedule: the B operands two k-steps ahead of their products (left to itself the
            // compiler reads each just before its use and waits for it); the compiler then also
            // runs this block's products beside the previous block's relu/weight work. 207
            // registers, two waves per SIMD: 73.4 -> 69.4 us on 8192 queries x 2048 positions.
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int i = 0; i < KS - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            float part[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float a[2] = {0.0f, 0.0f};
#pragma unroll
                for (int r = 0; r < 16; ++r) a[r & 1] += wv[j][r] * relu_f32(acc[j][r], pinf);
                part[j] = a[0] + a[1];
            }
            // lanes 32..63 of part[0] trade places with lanes 0..31 of part[1]
            const auto sw = __builtin_amdgcn_permlane32_swap(f32_bits(part[0]), f32_bits(part[1]), false, false);
            const float score = bits_f32(sw[0]) + bits_f32(sw[1]);
            const int pp = tb + 32 * nb + l32;
            bool keep = pp < vis_l;
            if constexpr (CAND) keep = keep && cb[nb] != 0;
            __builtin_amdgcn_raw_buffer_store_b32(f32_bits(keep ? score : -INFINITY), srows,
                                                  pp < p.n_pos ? (rowoff + pp) * 4 : kBufferPastEnd, 0, 0);
        }
        stage((it + 1) & 1);
        __syncthreads();
    }
    // tiles past every query's visible positions: -inf, no keys needed
    for (int it = ntiles; it < nall; ++it) {
#pragma unroll
        for (int nb = 0; nb < kLdsTile / 32; ++nb) {
            const int pp = it * kLdsTile + 32 * nb + l32;
            __builtin_amdgcn_raw_buffer_store_b32(f32_bits(-INFINITY), srows,
                                                  pp < p.n_pos ? (rowoff + pp) * 4 : kBufferPastEnd, 0, 0);
        }
    }
}

// ------------------------------------------------------------------ radix select
// Order-preserving 32-bit key of a score; -inf, NaN (and nothing else) map to 0, so only
// finite scores (and +inf) are ever selected; -0 counts as +0.
__device__ __forceinline__ uint32_t score_key(float v) {
    if (!(v > -INFINITY)) return 0u;
    uint32_t u = f32_bits(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup's threads in thread order, and the total
// (NT threads); `tot` holds NT / 64 words of LDS. One barrier before the totals are read and
// one after, so consecutive calls can reuse `tot`.
template <int NT>
__device__ __forceinline__ int block_excl_sum(int v, SA_LDS int* tot, int& total) {
    constexpr int NWV = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        incl += lane >= o ? u : 0;
    }
    if (lane == 63) tot[wid] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        const int c = tot[w];
        before += w < wid ? c : 0;
        total += c;
    }
    __syncthreads();
    return before + incl - v;
}

// The k-th largest key among keys[0 .. n) in LDS (k >= 1, at most the number of non-zero
// keys) by a 4-pass radix select (8 bits per pass, most significant first), and how many
// keys equal to it are among the k largest (the rest of the k are greater). NT threads;
// hist: 256 words of LDS; misc: 8 words.
template <int NT>
__device__ void radix_threshold(SA_LDS const uint32_t* keys, int n, int k, SA_LDS uint32_t* hist,
                                SA_LDS int* misc, uint32_t& thr, int& ties) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint32_t prefix = 0, mask = 0;
    int rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
        if (shift == 24 && NT <= 256) {
            // the first digit (sign and high exponent bits) takes few values, so same-address
            // atomics would serialise: equal digits of a wave are counted first and added once
            // (measured on the 256-thread lists of the long prefill; the 1024-thread ones of
            // decode ran faster with plain atomics)
            for (int i0 = 0; i0 < n; i0 += NT) {
                const int i = i0 + tid;
                const bool act = i < n;
                const uint32_t dig = act ? keys[i] >> 24 : 0u;
                uint64_t todo = __ballot(act);
                while (todo) {
                    const int leader = __builtin_ctzll(todo);
                    const uint32_t d = __shfl(dig, leader, 64);
                    const uint64_t same = __ballot(act && dig == d);
                    if (lane == leader)
                        __hip_atomic_fetch_add(&hist[d], (uint32_t)__builtin_popcountll(same), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
                    todo &= ~same;
                }
            }
        } else {
            for (int i = tid; i < n; i += NT) {
                const uint32_t u = keys[i];
                if ((u & mask) == prefix)
                    __hip_atomic_fetch_add(&hist[(u >> shift) & 255u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        __syncthreads();
        if (tid < 64) {
            // lane L holds bins 4L .. 4L+3; suffix sums from the top bin down
            uint32_t b4[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) b4[d] = hist[4 * lane + d];
            const int own = (int)(b4[0] + b4[1] + b4[2] + b4[3]);
            int suf = own;                                           // sum over lanes >= L
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_down(suf, o, 64);
                suf += lane + o < 64 ? v : 0;
            }
            const uint64_t reach = __ballot(suf >= rem);
            const int top = 63 - __builtin_clzll(reach);             // highest lane reaching rem
            if (lane == top) {
                int cum = suf - own;                                 // keys in higher bins
                int digit = 0;
#pragma unroll
                for (int d = 3; d >= 0; --d) {
                    if (cum + (int)b4[d] >= rem) { digit = 4 * lane + d; break; }
                    cum += (int)b4[d];
                }
                misc[0] = digit;
                misc[1] = rem - cum;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)misc[0] << shift;
        mask |= 255u << shift;
        rem = misc[1];
        __syncthreads();
    }
    thr = prefix;
    ties = rem;
}

// Number of non-zero keys among keys[0 .. n) (the selectable ones), in every thread.
template <int NT>
__device__ __forceinline__ int count_selectable(SA_LDS const uint32_t* keys, int n, SA_LDS int* tot) {
    int c = 0;
    for (int i = threadIdx.x; i < n; i += NT) c += keys[i] != 0u;
    int total;
    block_excl_sum<NT>(c, tot, total);
    return total;
}

// The ordered selection: wave w owns positions [w * chunk, (w + 1) * chunk), read as rows of
// 64 consecutive keys (lane l takes position base + 64 r + l, so every LDS read is free of
// bank conflicts); the rank of a selected entry among the selected, in position order, counts
// the selected entries of earlier waves (one block scan over the waves' totals), of earlier
// rows of its wave and of lower lanes of its row. Among equal keys at the threshold the
// lowest positions are taken first. Calls take(i, rank) for every selected entry i.
template <int NT, typename Take>
__device__ __forceinline__ void select_in_order(SA_LDS const uint32_t* keys, int n, uint32_t thr, int ties,
                                                SA_LDS int* tot, Take take) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int rows = (n + NT - 1) / NT;
    const int base = wid * rows * 64;
    const uint64_t below = (1ull << lane) - 1;
    // keys equal to the threshold before this wave's chunk
    int eq_w = 0;
    for (int r = 0; r < rows; ++r) {
        const int i = base + 64 * r + lane;
        eq_w += __builtin_popcountll(__ballot(i < n && keys[i] == thr));
    }
    int total;
    const int eq_before = __shfl(block_excl_sum<NT>(lane == 0 ? eq_w : 0, tot, total), 0, 64);
    // whether entry i is selected, given the ties met before its row
    auto sel_row = [&](int r, int& tie_seen) {
        const int i = base + 64 * r + lane;
        const uint32_t u = i < n ? keys[i] : 0u;
        const uint64_t beq = __ballot(i < n && u == thr);
        const bool sel = u > thr || (((beq >> lane) & 1) && tie_seen + __builtin_popcountll(beq & below) < ties);
        tie_seen += __builtin_popcountll(beq);
        return __ballot(sel);
    };
    int sel_w = 0, tie_seen = eq_before;
    for (int r = 0; r < rows; ++r) sel_w += __builtin_popcountll(sel_row(r, tie_seen));
    int rank = __shfl(block_excl_sum<NT>(lane == 0 ? sel_w : 0, tot, total), 0, 64);
    tie_seen = eq_before;
    for (int r = 0; r < rows; ++r) {
        const uint64_t bs = sel_row(r, tie_seen);
        if ((bs >> lane) & 1) take(base + 64 * r + lane, rank + __builtin_popcountll(bs & below));
        rank += __builtin_popcountll(bs);
    }
}

// ------------------------------------------------------------------ top-k lists
// Sum of a wave-uniform value over the W waves that hold one query (the same result in every
// wave), and the part of the waves before this one. `red` holds 2 x W words; consecutive
// calls alternate between its halves (gen), so one barrier per call suffices: a wave writes
// half g only after every wave has passed the barrier of the call before, i.e. has finished
// reading half g two calls back. W = 1: no LDS, no barrier.
template <int W>
__device__ __forceinline__ int query_sum(int v, SA_LDS int* red, int& gen, int& before) {
    before = 0;
    if constexpr (W == 1) {
        return v;
    } else {
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        if (lane == 0) red[gen * W + wid] = v;
        __syncthreads();
        int tot = 0;
#pragma unroll
        for (int u = 0; u < W; ++u) {
            const int c = red[gen * W + u];
            tot += c;
            before += u < wid ? c : 0;
        }
        gen ^= 1;
        return tot;
    }
}

// W waves per query hold its scores as keys in registers: wave w, row j, lane l holds
// position (w * J + j) * 64 + l (positions past n_pos hold key 0, as -inf does). The k-th
// largest key is found with counts, a count being the popcount of one compare ballot per row,
// summed over the query's waves through LDS: one wave builds it from the top bit down; several
// waves (whose counts each end at a barrier) halve an interval of keys that starts between a
// bracket taken from 64 sampled keys (each end checked by its count) or the query's largest
// key. Both end early at a key with exactly k keys at or above it. One ordered pass over the same registers then lists the chosen positions in
// ascending order (which is also the order the page re-sorts them into), shifted by the
// offset; among keys equal to the threshold the lower positions are taken first. W = 1: four
// queries per workgroup, one per wave, with no barriers at all.
template <int W, int J>
__global__ __launch_bounds__(W == 1 ? 256 : W * 64) void index_topk_kernel(const IdxParams p) {
    __shared__ int red[2][W];                       // per-wave partial sums, two generations
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t qi = W == 1 ? (int64_t)blockIdx.x * 4 + wid : (int64_t)blockIdx.x;
    if (W == 1 && qi >= (int64_t)p.b * p.s) return;             // no barriers when W = 1
    const int w = W == 1 ? 0 : wid;                              // wave within the query
    const int n = (int)(qi / p.s), t = (int)(qi % p.s);
    const float* sc = p.scores + (int64_t)n * p.scores_seq_stride + (int64_t)t * p.n_pos;
    const int base = w * J * 64;
    // every load issued before the first use (addresses clamped rather than branched around)
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = sc[min(base + 64 * j + lane, p.n_pos - 1)];
    uint32_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) key[j] = score_key(v[j]) & (base + 64 * j + lane < p.n_pos ? ~0u : 0u);
    int gen = 0;
    auto block_sum = [&](int v, int& before) { return query_sum<W>(v, (SA_LDS int*)&red[0][0], gen, before); };
    // A count: each lane counts its keys, DPP adds the lanes up (row shifts 1, 2, 4, 8 leave
    // each row's total in its last lane, the row broadcasts of lanes 15 and 31 carry them on,
    // lane 63 ends with the wave's sum), and with several waves LDS adds the waves up. Vector
    // work only, where a compare ballot per row would add a scalar popcount and a scalar add
    // after each compare.
    auto count_ge = [&](uint32_t c) {
        int v = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) v += key[j] >= c ? 1 : 0;
        v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
        v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
        v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
        v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
        v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
        v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
        int before;
        return block_sum(__builtin_amdgcn_readlane(v, 63), before);
    };
    // W > 1: the query's largest key and a sample of 64 of its keys (sample m from wave m % W,
    // lane m, row (m + wave) % J), exchanged through LDS ahead of the first count's barrier
    __shared__ uint32_t samp_s[64], kmax_s[W];
    uint32_t mine = 0;
    if constexpr (W > 1) {
        uint32_t kmax = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            kmax = max(kmax, key[j]);
            mine = (lane + w) % J == j ? key[j] : mine;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
        if (lane % W == w) samp_s[lane] = mine;
        if (lane == 0) kmax_s[w] = kmax;
    }
    const int selectable = count_ge(1u);                         // (the barrier for those writes)
    const int k = min(p.topk, selectable);
    // chosen: key > thr, or key == thr among the first `ties` such positions
    uint32_t thr = 0;
    int ties = 0;
    if (k > 0 && k < selectable && W == 1) {
        // One wave per query: a count costs no barrier, and the k-th largest key is built from
        // the top bit down (a bit stays set when at least k keys are at or above the
        // candidate), ending early at a candidate with exactly k keys at or above it.
        uint32_t lo = 0;                                         // count_ge(lo) >= k throughout
        bool exact = false;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = lo | (1u << bit);
            const int cnt = count_ge(c);
            if (cnt >= k) {
                lo = c;
                if (cnt == k) { exact = true; break; }
            }
        }
        if (exact) {
            thr = lo - 1;                                        // the k keys >= lo (lo >= 1)
        } else {
            // lo is the k-th largest key; the keys above it are fewer than k
            thr = lo;
            ties = k - (lo == 0xffffffffu ? 0 : count_ge(lo + 1));
        }
    } else if (k > 0 && k < selectable) {
        // Several waves per query: every count ends at a barrier, so counts are saved by
        // starting from a narrow interval.
        const uint32_t samp = samp_s[lane];
        uint32_t kmax_q = 0;
#pragma unroll
        for (int u = 0; u < W; ++u) kmax_q = max(kmax_q, kmax_s[u]);
        // the r-th largest sample: the largest key with at least r samples at or above it
        auto sample_kth = [&](int r) {
            uint32_t v = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t c = v | (1u << bit);
                if (__builtin_popcountll(__ballot(samp >= c)) >= r) v = c;
            }
            return v;
        };
        // [lo, hi) in key space with count_ge(lo) >= k > count_ge(hi) = c_hi; each count
        // narrows it, and one of exactly k ends the search
        uint32_t lo = 1;                                         // count_ge(1) = selectable > k
        uint64_t hi = (uint64_t)kmax_q + 1;                      // no key above the largest
        int c_hi = 0;
        bool exact = false;
        auto probe = [&](uint32_t c) {
            const int cnt = count_ge(c);
            if (cnt >= k) {
                lo = c;
                exact = cnt == k;
            } else {
                hi = c;
                c_hi = cnt;
            }
        };
        // A bracket from the sample: of the 64 samples, 64 k / N are expected at or above the
        // k-th largest key (N = 64 W J key slots); the ranks 3 standard deviations and one more
        // to either side give a key expected above it and one expected below it. Each is
        // checked by its count, so a poor sample only leaves the interval wider.
        const float q = (float)k / (float)(64 * W * J);
        const float mu = 64.0f * q, sd = __builtin_sqrtf(64.0f * q * (1.0f - q));
        const int r_above = (int)(mu - 3.0f * sd) - 1, r_below = (int)(mu + 3.0f * sd) + 2;
        if (r_above >= 1) {
            const uint32_t c = sample_kth(r_above);
            if (c > lo && c < hi) probe(c);
        }
        if (!exact && r_below <= 64) {
            const uint32_t c = sample_kth(r_below);
            if (c > lo && c < hi) probe(c);
        }
        // then halve the interval (uniform in every wave: the same counts, the same barriers)
        while (!exact && hi - lo > 1) probe(lo + (uint32_t)((hi - lo) >> 1));
        if (exact) {
            thr = lo - 1;                                        // the k keys >= lo (lo >= 1)
        } else {
            // lo is the k-th largest key: count_ge(lo) >= k > count_ge(lo + 1) = c_hi
            thr = lo;
            ties = k - c_hi;
        }
    }
    // ties met before this wave's positions
    int tie_before = 0;
    if (ties > 0) {
        int eq = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) eq += __builtin_popcountll(__ballot(key[j] == thr));
        block_sum(eq, tie_before);
    }
    const uint64_t below = (1ull << lane) - 1;
    auto row_sel = [&](int j, int& tie_seen) {
        if (ties == 0) return (uint64_t)__ballot(key[j] > thr);
        const uint64_t beq = __ballot(key[j] == thr);
        const bool sel = key[j] > thr || (key[j] == thr && tie_seen + __builtin_popcountll(beq & below) < ties);
        tie_seen += __builtin_popcountll(beq);
        return (uint64_t)__ballot(sel);
    };
    int sel_w = 0, tie_seen = tie_before;
#pragma unroll
    for (int j = 0; j < J; ++j) sel_w += __builtin_popcountll(row_sel(j, tie_seen));
    int rank;
    block_sum(sel_w, rank);
    int32_t* out = p.idx + (int64_t)n * p.idx_seq_stride + (int64_t)t * p.idx_row_stride;
    tie_seen = tie_before;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const uint64_t bs = row_sel(j, tie_seen);
        if ((bs >> lane) & 1) out[rank + __builtin_popcountll(bs & below)] = base + 64 * j + lane + p.offset;
        rank += __builtin_popcountll(bs);
    }
    for (int c = k + w * 64 + lane; c < p.topk; c += W * 64) out[c] = -1;
}

// ------------------------------------------------------------------ candidate blocks
// select_candidate_blocks for rows whose blocks fit in lanes: W waves per query, lane l of
// wave w holds the J consecutive positions from (w * 64 + l) * J on, so a block of BS
// positions (a power of two up to J) lies inside one lane and its maximum is in-lane work.
// Block order is (wave, lane, slot). The kept blocks are chosen as in index_topk_kernel
// (bitwise threshold over the block keys, equal keys: the lower block first), or all of
// them when they are at most topk_blocks; each lane writes its J mask bytes as 16-byte
// stores. Rows of whole 16-byte pieces only (n_pos, the mask pointer and its strides
// multiples of 16).
template <int W, int J, int BS>
__global__ __launch_bounds__(W == 1 ? 256 : W * 64) void candidate_wave_kernel(const CandParams p) {
    constexpr int NBL = J / BS;                                  // blocks per lane
    static_assert(J % 16 == 0 && BS >= 1 && J % BS == 0 && (BS & (BS - 1)) == 0, "blocks inside lanes");
    __shared__ int red[2][W];
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t qi = W == 1 ? (int64_t)blockIdx.x * 4 + wid : (int64_t)blockIdx.x;
    if (W == 1 && qi >= (int64_t)p.b * p.s) return;             // no barriers when W = 1
    const int w = W == 1 ? 0 : wid;
    const int n = (int)(qi / p.s), t = (int)(qi % p.s);
    const int u0 = (w * 64 + lane) * J;                          // this lane's first position
    const float* lg = p.logits + (int64_t)n * p.logits_seq_stride + (int64_t)t * p.n_pos;
    const __amdgpu_buffer_rsrc_t lrow = __builtin_amdgcn_make_buffer_rsrc((void*)lg, 0, p.n_pos * 4, 0x00020000);
    u32x4 x[J / 4];
#pragma unroll
    for (int c = 0; c < J / 4; ++c)
        x[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(lrow, (u0 + 4 * c) * 4, 0, 0));
    // block keys: the maximum of the order-preserving keys (-inf padding past n_pos: key 0)
    uint32_t bk[NBL];
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
        uint32_t m = 0;
#pragma unroll
        for (int e = i * BS; e < (i + 1) * BS; ++e)
            m = max(m, score_key(bits_f32(x[e / 4][e % 4])) & (u0 + e < p.n_pos ? ~0u : 0u));
        bk[i] = m;
    }
    const int pos = p.pos[(int64_t)n * p.pos_seq_stride + t];
    const int64_t len = pos < 0 ? 0 : ((int64_t)pos + 1) / p.ratio;
    const int64_t last = len > 0 ? (len - 1) / BS : -1;          // the newest visible block
    const int nblk = (p.n_pos + BS - 1) / BS;
    const int b0 = u0 / BS;                                      // this lane's first block
#pragma unroll
    for (int i = 0; i < NBL; ++i)
        if (last < nblk && b0 + i == last) bk[i] = score_key(INFINITY);
    int gen = 0;
    auto count = [&](auto pred) {
        int c = 0;
#pragma unroll
        for (int i = 0; i < NBL; ++i) c += __builtin_popcountll(__ballot(pred(bk[i])));
        int before;
        return query_sum<W>(c, (SA_LDS int*)&red[0][0], gen, before);
    };
    const int selectable = count([](uint32_t k) { return k != 0u; });
    const int k = min(p.topk_blocks, selectable);
    uint32_t thr = 0;                                            // kept: key > thr, or == thr
    int ties = 0;                                                // among the first `ties`
    if (k > 0 && k < selectable) {
        uint32_t lo = 0;
        bool exact = false;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = lo | (1u << bit);
            const int cnt = count([c](uint32_t kv) { return kv >= c; });
            if (cnt >= k) {
                lo = c;
                if (cnt == k) { exact = true; break; }
            }
        }
        if (exact) {
            thr = lo - 1;
        } else {
            thr = lo;
            ties = k - (lo == 0xffffffffu ? 0 : count([lo](uint32_t kv) { return kv > lo; }));
        }
    }
    uint32_t keep = 0;                                           // bit i: slot i kept
#pragma unroll
    for (int i = 0; i < NBL; ++i) keep |= (uint32_t)(bk[i] > thr) << i;
    if (ties > 0) {
        // rank of each tied block in block order: tied blocks of earlier waves, of lower
        // lanes, of earlier slots of this lane
        const uint64_t below = (1ull << lane) - 1;
        int lower = 0, wave_ties = 0;
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            const uint64_t m = __ballot(bk[i] == thr);
            lower += __builtin_popcountll(m & below);
            wave_ties += __builtin_popcountll(m);
        }
        int before;
        query_sum<W>(wave_ties, (SA_LDS int*)&red[0][0], gen, before);
        int r = before + lower;
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            const bool eq = bk[i] == thr;
            keep |= (uint32_t)(eq && r < ties) << i;
            r += eq;
        }
    }
    uint8_t* mrow = p.mask + (int64_t)n * p.mask_seq_stride + (int64_t)t * p.n_pos;
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc((void*)mrow, 0, p.n_pos, 0x00020000);
#pragma unroll
    for (int c = 0; c < J / 16; ++c) {
        u32x4 word;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t v = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) v |= ((keep >> ((16 * c + 4 * q + e) / BS)) & 1u) << (8 * e);
            word[q] = v;
        }
        __builtin_amdgcn_raw_buffer_store_b128(word, mr, u0 + 16 * c, 0, 0);
    }
}

// select_candidate_blocks for one query per workgroup: block maxima (the last block padded
// with -inf), the block of the newest visible position, (len - 1) / block_size with floor
// division, pinned to +inf, the min(topk_blocks, blocks) best blocks kept when above -inf
// (ties: the lower block first), each block's flag repeated over its positions.
template <int NT>
__global__ __launch_bounds__(NT) void candidate_blocks_kernel(const CandParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    SA_LDS uint32_t* hist = (SA_LDS uint32_t*)smem_raw;
    SA_LDS int* misc = (SA_LDS int*)(hist + 256);
    SA_LDS uint32_t* keys = (SA_LDS uint32_t*)(misc + 16);       // one per block
    SA_LDS uint8_t* keep = (SA_LDS uint8_t*)(keys + ((p.n_pos + p.block_size - 1) / p.block_size));
    const int tid = threadIdx.x;
    const int64_t qi = blockIdx.x;
    const int n = (int)(qi / p.s), t = (int)(qi % p.s);
    const float* lg = p.logits + (int64_t)n * p.logits_seq_stride + (int64_t)t * p.n_pos;
    const int nblk = (p.n_pos + p.block_size - 1) / p.block_size;
    const int pos = p.pos[(int64_t)n * p.pos_seq_stride + t];
    const int64_t len = pos < 0 ? 0 : ((int64_t)pos + 1) / p.ratio;
    const int64_t last = len > 0 ? (len - 1) / p.block_size : -1;
    // block maxima as the maxima of the order-preserving keys (-inf padding is key 0), with
    // 8 logit loads in flight per thread. A block size that is a power of two up to 64 puts
    // each block in consecutive lanes of one wave: their maximum is taken by lane exchanges
    // and stored by the block's first lane; other sizes use LDS atomics.
    const bool lanes = p.block_size <= 64 && (p.block_size & (p.block_size - 1)) == 0;
    for (int j = tid; j < nblk; j += NT) {
        if (!lanes) keys[j] = 0u;
        keep[j] = 0;
    }
    __syncthreads();
    for (int i0 = 0; i0 < p.n_pos; i0 += 8 * NT) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * NT + tid;
            v[u] = i < p.n_pos ? lg[i] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * NT + tid;
            uint32_t key = score_key(v[u]);
            if (lanes) {
                for (int o = 1; o < p.block_size; o <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, o, 64));
                if (i % p.block_size == 0 && i < p.n_pos) keys[i / p.block_size] = key;
            } else if (i < p.n_pos && key != 0u) {
                __hip_atomic_fetch_max(&keys[i / p.block_size], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    __syncthreads();
    if (tid == 0 && last >= 0 && last < nblk) keys[last] = score_key(INFINITY);
    __syncthreads();
    const int selectable = count_selectable<NT>(keys, nblk, misc);
    const int k = min(p.topk_blocks, selectable);
    if (k > 0 && k == selectable) {
        // every block with a visible position is kept: no selection needed
        for (int j = tid; j < nblk; j += NT) keep[j] = keys[j] != 0u;
    } else if (k > 0) {
        uint32_t thr;
        int ties;
        radix_threshold<NT>(keys, nblk, k, hist, misc, thr, ties);
        select_in_order<NT>(keys, nblk, thr, ties, misc, [&](int j, int) { keep[j] = 1; });
    }
    __syncthreads();
    // each block's flag repeated over its positions, 16 bytes per store where the row allows
    uint8_t* mask = p.mask + (int64_t)n * p.mask_seq_stride + (int64_t)t * p.n_pos;
    const int n16 = ((uintptr_t)mask % 16 == 0) ? p.n_pos / 16 : 0;
    for (int c = tid; c < n16; c += NT) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) word |= (uint32_t)keep[(16 * c + 4 * q + b) / p.block_size] << (8 * b);
            w[q] = word;
        }
        *(u32x4*)(mask + 16 * c) = w;
    }
    for (int u = 16 * n16 + tid; u < p.n_pos; u += NT) mask[u] = keep[u / p.block_size];
}

// ------------------------------------------------------------------ launches
template <int D, int HB>
static hipError_t launch_scores_hb(const IdxParams& p, hipStream_t st) {
    if constexpr (HB == 2 && (D == 64 || D == 128)) {
        // 32 heads: one buffer over a wave's two score rows stays far below the offset that
        // stands for "past the end" while n_pos <= 2^26
        if (p.s >= kLdsQueries && p.n_pos <= (1 << 26)) {
            const int64_t gx = (p.s + kLdsQueries - 1) / kLdsQueries;
            if (gx > 0x7fffffff || p.b > 65535) return hipErrorInvalidValue;
            if (p.cand) hipLaunchKernelGGL((index_scores_h32_kernel<D, true>), dim3((unsigned)gx, (unsigned)p.b), dim3(256), 0, st, p);
            else hipLaunchKernelGGL((index_scores_h32_kernel<D, false>), dim3((unsigned)gx, (unsigned)p.b), dim3(256), 0, st, p);
            return hipGetLastError();
        }
    }
    if constexpr (HB * D <= 256) {
        if (p.s >= kLdsQueries) {
            const int64_t gx = (p.s + kLdsQueries - 1) / kLdsQueries;
            if (gx > 0x7fffffff || p.b > 65535) return hipErrorInvalidValue;
            if (p.cand) hipLaunchKernelGGL((index_scores_lds_kernel<D, HB, true>), dim3((unsigned)gx, (unsigned)p.b), dim3(256), 0, st, p);
            else hipLaunchKernelGGL((index_scores_lds_kernel<D, HB, false>), dim3((unsigned)gx, (unsigned)p.b), dim3(256), 0, st, p);
            return hipGetLastError();
        }
    }
    constexpr int QPW = HB * D <= 256 ? 2 : 1;
    const int qpw = p.s > 1 ? QPW : 1;                      // decode: one query per sequence
    const int64_t waves = (int64_t)p.b * ((p.s + qpw - 1) / qpw);
    const int64_t gx = (waves + 3) / 4;
    const int gy = (p.n_pos + kScoreChunk - 1) / kScoreChunk;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    const bool cand = p.cand != nullptr;
    if (qpw == 2 && cand) hipLaunchKernelGGL((index_scores_kernel<D, HB, QPW, true>), grid, dim3(256), 0, st, p);
    else if (qpw == 2) hipLaunchKernelGGL((index_scores_kernel<D, HB, QPW, false>), grid, dim3(256), 0, st, p);
    else if (cand) hipLaunchKernelGGL((index_scores_kernel<D, HB, 1, true>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((index_scores_kernel<D, HB, 1, false>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_scores_d(const IdxParams& p, hipStream_t st) {
    switch (p.h / 16) {
        case 1: return launch_scores_hb<D, 1>(p, st);
        case 2: return launch_scores_hb<D, 2>(p, st);
        case 4:
            if constexpr (D <= 128) return launch_scores_hb<D, 4>(p, st);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_index_scores(const IdxParams& p, hipStream_t st) {
    switch (p.d) {
        case 64: return launch_scores_d<64>(p, st);
        case 128: return launch_scores_d<128>(p, st);
        case 256: return launch_scores_d<256>(p, st);
        default: return hipErrorInvalidValue;
    }
}

template <int W, int J>
static hipError_t launch_topk_wj(const IdxParams& p, hipStream_t st) {
    const int64_t nq = (int64_t)p.b * p.s;
    const int64_t grid = W == 1 ? (nq + 3) / 4 : nq;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((index_topk_kernel<W, J>), dim3((unsigned)grid), dim3(W == 1 ? 256 : W * 64), 0, st, p);
    return hipGetLastError();
}

// keys per query: up to 2048 in one wave, 8192 in four, 32768 in sixteen
hipError_t launch_index_topk(const IdxParams& p, hipStream_t st) {
    const int n = p.n_pos;
    if (n <= 512) return launch_topk_wj<1, 8>(p, st);
    if (n <= 1024) return launch_topk_wj<1, 16>(p, st);
    if (n <= 2048) return launch_topk_wj<1, 32>(p, st);
    if (n <= 4096) return launch_topk_wj<4, 16>(p, st);
    if (n <= 8192) return launch_topk_wj<4, 32>(p, st);
    if (n <= 16384) return launch_topk_wj<16, 16>(p, st);
    if (n <= 32768) return launch_topk_wj<16, 32>(p, st);
    return hipErrorInvalidValue;
}

template <int W, int J, int BS>
static hipError_t launch_cand_wj(const CandParams& p, hipStream_t st) {
    const int64_t nq = (int64_t)p.b * p.s;
    const int64_t grid = W == 1 ? (nq + 3) / 4 : nq;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((candidate_wave_kernel<W, J, BS>), dim3((unsigned)grid), dim3(W == 1 ? 256 : W * 64), 0, st, p);
    return hipGetLastError();
}

template <int BS>
static hipError_t launch_cand_bs(const CandParams& p, hipStream_t st) {
    if (p.n_pos <= 2048) return launch_cand_wj<1, 32, BS>(p, st);
    if (p.n_pos <= 4096) return launch_cand_wj<4, 16, BS>(p, st);
    if (p.n_pos <= 8192) return launch_cand_wj<4, 32, BS>(p, st);
    if (p.n_pos <= 16384) return launch_cand_wj<16, 16, BS>(p, st);
    return launch_cand_wj<16, 32, BS>(p, st);
}

hipError_t launch_candidate_blocks(const CandParams& p, hipStream_t st) {
    // rows of whole 16-byte mask pieces, blocks of 4, 8 or 16 positions: one wave (or 4, or
    // 16) per query, blocks inside lanes
    const bool rows16 = p.n_pos % 16 == 0 && (uintptr_t)p.mask % 16 == 0 && (p.b == 1 || p.mask_seq_stride % 16 == 0);
    if (rows16 && p.n_pos <= 32768) {
        if (p.block_size == 4) return launch_cand_bs<4>(p, st);
        if (p.block_size == 8) return launch_cand_bs<8>(p, st);
        if (p.block_size == 16) return launch_cand_bs<16>(p, st);
    }
    const int nblk = (p.n_pos + p.block_size - 1) / p.block_size;
    const size_t lds = (256 + 16) * 4 + (size_t)nblk * 5;
    const int64_t nq = (int64_t)p.b * p.s;
    if (lds > 160 * 1024 || nq > 0x7fffffff) return hipErrorInvalidValue;
    // long rows get four times the threads (more logit loads in flight per query)
    const bool wide = p.n_pos > 4096;
    const void* k = wide ? (const void*)candidate_blocks_kernel<1024> : (const void*)candidate_blocks_kernel<256>;
    hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (wide) hipLaunchKernelGGL(candidate_blocks_kernel<1024>, dim3((unsigned)nq), dim3(1024), lds, st, p);
    else hipLaunchKernelGGL(candidate_blocks_kernel<256>, dim3((unsigned)nq), dim3(256), lds, st, p);
    return hipGetLastError();
}

}  // namespace sa
