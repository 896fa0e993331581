// The indexer that produces the compressed half of sparse_attn's index lists (the indexer
// page: Indexer.forward and select_candidate_blocks), on gfx950:
//   * index_scores_kernel: score[t] = sum_h w_h relu(q_h . k_t) per query, on bf16 MFMA with
//     f32 accumulation; positions the query cannot see (and, for the second level, positions
//     outside the candidate mask) are -inf;
//   * index_topk_kernel: per query, the topk best finite scores by a radix select on LDS,
//     listed in position order (ties: the lower position first), shifted by the offset and
//     padded with -1;
//   * candidate_blocks_kernel: per query, block maxima, the newest visible block pinned, the
//     best blocks kept by the same radix select, expanded to a position mask.
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

// S[head][position] = Q . K^T on v_mfma_f32_16x16x32_bf16: Q is the A operand (rows = 16
// heads, held in registers), K the B operand (columns = 16 positions, loaded straight from
// memory, one 16-byte piece per lane and k-step). In the accumulator each lane holds one
// position and 4 heads, so the weighted head sum is in-lane work plus two exchanges across
// the lane groups. A wave takes QPW queries of one sequence (sharing every K load) and
// kChunk positions; a workgroup is 4 such waves.
constexpr int kScoreChunk = 256;

template <int D, int HB, int QPW>
__global__ __launch_bounds__(256) void index_scores_kernel(const IdxParams p) {
    constexpr int KS = D / 32;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int groups = (p.s + QPW - 1) / QPW;                   // query groups per sequence
    const int64_t wave = (int64_t)blockIdx.x * 4 + wid;
    if (wave >= (int64_t)p.b * groups) return;                  // no barriers in this kernel
    const int n = (int)(wave / groups);
    const int t0 = (int)(wave % groups) * QPW;
    const int c0 = blockIdx.y * kScoreChunk;
    const int cend = min(p.n_pos, c0 + kScoreChunk);

    int vis[QPW];
    int vmax = 0;
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        const bool live = t0 + j < p.s;
        vis[j] = live ? visible_positions(p.pos[(int64_t)n * p.pos_seq_stride + t0 + j], p.ratio, p.n_pos) : 0;
        vmax = max(vmax, vis[j]);
    }
    const uint16_t* kseq = p.k + (int64_t)n * p.k_seq_stride;
    // Q of each query: A operand of (head block mb, k-step kk): head 16 mb + l16, d 32 kk + 8 g
    u32x4 qa[QPW][HB][KS];
    float wv[QPW][HB][4];
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
    auto load_k = [&](int pb, u32x4 (&kb)[KS]) {
        const int pp = min(pb + l16, p.n_pos - 1);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) kb[kk] = *(const u32x4*)(kseq + (int64_t)pp * D + 32 * kk + 8 * g);
    };
    const int vend = min(cend, vmax);                            // blocks with a visible position
    // one 16-position block: its K operands are in `cur`; the next block's go to `nxt`
    auto step = [&](int pb, const u32x4 (&cur)[KS], u32x4 (&nxt)[KS]) {
        const int pp = pb + l16;
        const bool any = pb < vend;
        if (any && pb + 16 < vend) load_k(pb + 16, nxt);
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
                    for (int r = 0; r < 4; ++r) part += wv[j][mb][r] * fmaxf(acc[mb][r], 0.0f);
                part = sum_xor32(sum_xor16(part));
            }
            const int t = t0 + j;
            if (g == 0 && t < p.s && pp < cend) {
                bool keep = pp < vis[j];
                if (keep && p.cand) keep = p.cand[(int64_t)n * p.cand_seq_stride + (int64_t)t * p.n_pos + pp] != 0;
                p.scores[(int64_t)n * p.scores_seq_stride + (int64_t)t * p.n_pos + pp] = keep ? part : -INFINITY;
            }
        }
    };
    u32x4 ka[KS], kb[KS];
    if (c0 < vend) load_k(c0, ka);
    for (int pb = c0; pb < cend; pb += 32) {
        step(pb, ka, kb);
        if (pb + 16 < cend) step(pb + 16, kb, ka);
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

// Exclusive prefix count of `bit` over the workgroup's threads in thread order, and the
// total; `tot` is 4 words of LDS. Contains one barrier before the totals are read and one
// after, so consecutive calls can reuse `tot`.
__device__ __forceinline__ int block_excl_count(bool bit, SA_LDS int* tot, int& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const uint64_t m = __ballot(bit);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (lane == 0) tot[wid] = __builtin_popcountll(m);
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int c = tot[w];
        before += w < wid ? c : 0;
        total += c;
    }
    __syncthreads();
    return before + below;
}

// The keep flags of the k largest keys among keys[0 .. n) in LDS (k >= 1, at most the number
// of non-zero keys): keys greater than the k-th largest, and as many keys equal to it as are
// still needed, the lowest positions first. Writes the threshold key and that number of ties.
// 256 threads; hist: 256 words of LDS; misc: 8 words.
__device__ void radix_threshold(SA_LDS const uint32_t* keys, int n, int k, SA_LDS uint32_t* hist,
                                SA_LDS int* misc, uint32_t& thr, int& ties) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint32_t prefix = 0, mask = 0;
    int rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += 256) {
            const uint32_t u = keys[i];
            if ((u & mask) == prefix)
                __hip_atomic_fetch_add(&hist[(u >> shift) & 255u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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
__device__ __forceinline__ int count_selectable(SA_LDS const uint32_t* keys, int n, SA_LDS int* tot) {
    int c = 0;
    for (int i = threadIdx.x; i < n; i += 256) c += keys[i] != 0u;
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) tot[threadIdx.x >> 6] = c;
    __syncthreads();
    const int total = tot[0] + tot[1] + tot[2] + tot[3];
    __syncthreads();
    return total;
}

// ------------------------------------------------------------------ top-k lists
// One workgroup per query: the query's scores become keys in LDS; the k-th largest is found
// by a 4-pass radix select; one ordered pass then lists the chosen positions in ascending
// order (which is also the order the page re-sorts them into), shifted by the offset.
__global__ __launch_bounds__(256) void index_topk_kernel(const IdxParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    SA_LDS uint32_t* hist = (SA_LDS uint32_t*)smem_raw;          // 256
    SA_LDS int* misc = (SA_LDS int*)(hist + 256);                // 8
    SA_LDS uint32_t* keys = (SA_LDS uint32_t*)(misc + 8);        // n_pos
    const int tid = threadIdx.x;
    const int64_t qi = blockIdx.x;
    const int n = (int)(qi / p.s), t = (int)(qi % p.s);
    const float* sc = p.scores + (int64_t)n * p.scores_seq_stride + (int64_t)t * p.n_pos;
    for (int i = tid; i < p.n_pos; i += 256) keys[i] = score_key(sc[i]);
    __syncthreads();
    int32_t* out = p.idx + (int64_t)n * p.idx_seq_stride + (int64_t)t * p.idx_row_stride;
    const int k = min(p.topk, count_selectable(keys, p.n_pos, misc));
    int listed = 0;
    if (k > 0) {
        uint32_t thr;
        int ties;
        radix_threshold(keys, p.n_pos, k, hist, misc, thr, ties);
        int tie_base = 0;
        for (int c = 0; c < p.n_pos; c += 256) {
            const int i = c + tid;
            const uint32_t u = i < p.n_pos ? keys[i] : 0u;
            int eq_total, fl_total;
            const int tie_rank = tie_base + block_excl_count(u == thr, misc, eq_total);
            const bool take = u > thr || (u == thr && tie_rank < ties);
            const int slot = listed + block_excl_count(take, misc, fl_total);
            if (take) out[slot] = i + p.offset;
            tie_base += eq_total;
            listed += fl_total;
        }
    }
    for (int j = listed + tid; j < p.topk; j += 256) out[j] = -1;
}

// ------------------------------------------------------------------ candidate blocks
// select_candidate_blocks for one query per workgroup: block maxima (the last block padded
// with -inf), the block of the newest visible position, (len - 1) / block_size with floor
// division, pinned to +inf, the min(topk_blocks, blocks) best blocks kept when above -inf
// (ties: the lower block first), each block's flag repeated over its positions.
__global__ __launch_bounds__(256) void candidate_blocks_kernel(const CandParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    SA_LDS uint32_t* hist = (SA_LDS uint32_t*)smem_raw;
    SA_LDS int* misc = (SA_LDS int*)(hist + 256);
    SA_LDS uint32_t* keys = (SA_LDS uint32_t*)(misc + 8);        // one per block
    const int tid = threadIdx.x;
    const int64_t qi = blockIdx.x;
    const int n = (int)(qi / p.s), t = (int)(qi % p.s);
    const float* lg = p.logits + (int64_t)n * p.logits_seq_stride + (int64_t)t * p.n_pos;
    const int nblk = (p.n_pos + p.block_size - 1) / p.block_size;
    const int pos = p.pos[(int64_t)n * p.pos_seq_stride + t];
    const int64_t len = pos < 0 ? 0 : ((int64_t)pos + 1) / p.ratio;
    const int64_t last = len > 0 ? (len - 1) / p.block_size : -1;
    for (int j = tid; j < nblk; j += 256) {
        float m = -INFINITY;
        const int t0 = j * p.block_size, t1 = min(p.n_pos, t0 + p.block_size);
        for (int u = t0; u < t1; ++u) m = fmaxf(m, lg[u]);
        keys[j] = score_key(j == last ? INFINITY : m);
    }
    __syncthreads();
    const int k = min(p.topk_blocks, count_selectable(keys, nblk, misc));
    uint32_t thr = 0xffffffffu;
    int ties = 0;
    if (k > 0) radix_threshold(keys, nblk, k, hist, misc, thr, ties);
    // the keep flags replace the keys (each thread rewrites only the entries it read)
    int tie_base = 0;
    for (int c = 0; c < nblk; c += 256) {
        const int j = c + tid;
        const uint32_t u = j < nblk ? keys[j] : 0u;
        int eq_total;
        const int tie_rank = tie_base + block_excl_count(k > 0 && u == thr, misc, eq_total);
        const bool keep = k > 0 && (u > thr || (u == thr && tie_rank < ties));
        if (j < nblk) keys[j] = keep ? 1u : 0u;
        tie_base += eq_total;
    }
    __syncthreads();
    uint8_t* mask = p.mask + (int64_t)n * p.mask_seq_stride + (int64_t)t * p.n_pos;
    for (int u = tid; u < p.n_pos; u += 256) mask[u] = (uint8_t)keys[u / p.block_size];
}

// ------------------------------------------------------------------ launches
template <int D, int HB>
static hipError_t launch_scores_hb(const IdxParams& p, hipStream_t st) {
    constexpr int QPW = HB * D <= 256 ? 2 : 1;
    const int qpw = p.s > 1 ? QPW : 1;                      // decode: one query per sequence
    const int64_t waves = (int64_t)p.b * ((p.s + qpw - 1) / qpw);
    const int64_t gx = (waves + 3) / 4;
    const int gy = (p.n_pos + kScoreChunk - 1) / kScoreChunk;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    if (qpw == 2) hipLaunchKernelGGL((index_scores_kernel<D, HB, QPW>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((index_scores_kernel<D, HB, 1>), grid, dim3(256), 0, st, p);
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

hipError_t launch_index_topk(const IdxParams& p, hipStream_t st) {
    const size_t lds = (256 + 8) * 4 + (size_t)p.n_pos * 4;
    const int64_t nq = (int64_t)p.b * p.s;
    if (lds > 160 * 1024 || nq > 0x7fffffff) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void*)index_topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(index_topk_kernel, dim3((unsigned)nq), dim3(256), lds, st, p);
    return hipGetLastError();
}

hipError_t launch_candidate_blocks(const CandParams& p, hipStream_t st) {
    const int nblk = (p.n_pos + p.block_size - 1) / p.block_size;
    const size_t lds = (256 + 8) * 4 + (size_t)nblk * 4;
    const int64_t nq = (int64_t)p.b * p.s;
    if (lds > 160 * 1024 || nq > 0x7fffffff) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void*)candidate_blocks_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(candidate_blocks_kernel, dim3((unsigned)nq), dim3(256), lds, st, p);
    return hipGetLastError();
}

}  // namespace sa
