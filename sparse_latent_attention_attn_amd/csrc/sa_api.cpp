// C-ABI entry points of libsa.so (declared in include/sa.h). Each call validates its
// arguments on the host before making any HIP call, then plans and launches the kernels on
// the caller's stream. Nothing is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/sa.h"
#include "sa_internal.hpp"

#define SA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// compute units of the current device (cached per device)
int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Shape and stride checks of sa_attn_args that need no pointer (shared with the workspace
// query). Returns SA_OK or an error status.
int check_shape(const sa_attn_args* a) {
    if (!a) return SA_ERR_INVALID;
    if (a->b < 1 || a->s < 1 || a->h < 1 || a->topk < 1 || a->kv_rows < 1) return SA_ERR_INVALID;
    if (a->d != 64 && a->d != 128 && a->d != 256 && a->d != 512) return SA_ERR_UNSUPPORTED;
    if (a->kv_format != SA_KV_BF16 && a->kv_format != SA_KV_FP8_E4M3_B32) return SA_ERR_INVALID;
    if ((a->flags & ~(uint32_t)SA_FLAG_CHECK_IDX) != 0) return SA_ERR_INVALID;
    if (a->rope_dim < 0 || a->rope_dim > a->d || (a->rope_dim & 1)) return SA_ERR_INVALID;
    const int64_t shd = (int64_t)a->s * a->h * a->d;
    if (a->b > 1) {
        const int64_t kv_row_elems = a->d;   // elements of the storage type per row
        if (a->q_seq_stride < shd || a->out_seq_stride < shd) return SA_ERR_INVALID;
        if (a->kv_seq_stride < (int64_t)a->kv_rows * kv_row_elems) return SA_ERR_INVALID;
        if (a->idx_seq_stride < (int64_t)a->s * a->topk) return SA_ERR_INVALID;
        if (a->kv_format == SA_KV_FP8_E4M3_B32 &&
            a->kv_scale_seq_stride < (int64_t)a->kv_rows * (a->d / 32))
            return SA_ERR_INVALID;
        if (a->rope_dim > 0 && a->pos_seq_stride < a->s) return SA_ERR_INVALID;
    }
    // 16-byte vector access of q, out and kv rows needs strides in whole 16-byte units
    if (a->q_seq_stride % 8 || a->out_seq_stride % 8) return SA_ERR_INVALID;
    if (a->kv_format == SA_KV_BF16 ? (a->kv_seq_stride % 8) : (a->kv_seq_stride % 16)) return SA_ERR_INVALID;
    if (!std::isfinite(a->scale)) return SA_ERR_INVALID;
    if (a->window < 0) return SA_ERR_INVALID;
    if (a->window > 0) {
        if (a->window_mode != SA_WINDOW_RING && a->window_mode != SA_WINDOW_CHUNK) return SA_ERR_INVALID;
        const int64_t win = a->window_mode == SA_WINDOW_RING ? a->window : std::min<int64_t>(a->s, a->window);
        if (win > a->topk) return SA_ERR_INVALID;
        if (a->b > 1 && a->pos_seq_stride < a->s) return SA_ERR_INVALID;
    }
    // one sequence's kv rows are addressed with 32-bit byte offsets
    const int64_t row_bytes = a->kv_format == SA_KV_BF16 ? 2 * (int64_t)a->d : a->d;
    if ((int64_t)a->kv_rows * row_bytes > INT32_MAX) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

int check_pointers(const sa_attn_args* a) {
    if (!a->q || !a->kv || !a->sink || !a->idx || !a->out) return SA_ERR_INVALID;
    if (!aligned(a->q, 16) || !aligned(a->kv, 16) || !aligned(a->out, 16) || !aligned(a->idx, 4) ||
        !aligned(a->sink, 4))
        return SA_ERR_INVALID;
    if (a->kv_format == SA_KV_FP8_E4M3_B32 && !a->kv_scale) return SA_ERR_INVALID;
    if (a->rope_dim > 0) {
        if (!a->rope_cos_sin || !a->pos || a->max_pos < 1 || !aligned(a->rope_cos_sin, 8)) return SA_ERR_INVALID;
    }
    if ((a->flags & SA_FLAG_CHECK_IDX) && !a->err_word) return SA_ERR_INVALID;
    if (a->window > 0 && (!a->pos || !aligned(a->pos, 4))) return SA_ERR_INVALID;
    return SA_OK;
}

// Work decomposition. A workgroup takes 16*nw heads of one query and a contiguous range
// of its index columns; its waves share every gathered key tile. Prefer the widest head
// block that still gives at least one workgroup per compute unit (fewest re-reads of a
// query's rows); split the columns across workgroups only when even one-wave blocks leave
// compute units idle and each split keeps at least kMinTilesPerSplit tiles, because every
// split writes an f32 partial of 16*nw heads x d (as large as 16*nw/8 key tiles).
constexpr int kMinTilesPerSplit = 8;
// fp8 storage whose rows are each named by at least this many (query, column) pairs on
// average (prefill) is dequantised into bf16 rows once per call, and the bf16 kernels run on
// those: the per-tile conversion in LDS then costs more than one pass over the cache
// (measured on 8192 queries x 128 heads x 2176 rows: 4.41 ms with the in-kernel conversion).
// Decode, where a row is named about once, keeps the conversion inside the kernel.
constexpr int64_t kDequantReuse = 16;

sa::Plan make_plan(const sa_attn_args* a, int cus) {
    using sa::kHeadsPerWave;
    using sa::kTileKeys;
    sa::Plan pl{};
    const int64_t nq = (int64_t)a->b * a->s;
    if (a->kv_format == SA_KV_FP8_E4M3_B32 && nq * a->topk >= kDequantReuse * a->b * (int64_t)a->kv_rows &&
        (int64_t)a->kv_rows * a->d * 2 <= INT32_MAX) {
        pl.dequant = true;
        pl.dq_bytes = ((size_t)a->b * a->kv_rows * a->d * 2 + 255) / 256 * 256;
    }
    // the storage the attention kernel reads
    const bool bf16_rows = a->kv_format == SA_KV_BF16 || pl.dequant;
    auto blocks_for = [&](int nw) { return (a->h + nw * kHeadsPerWave - 1) / (nw * kHeadsPerWave); };
    const int max_nw = std::min<int>(sa::kMaxWaves, (a->h + kHeadsPerWave - 1) / kHeadsPerWave);
    // The widest workgroup the heads allow: one gathered tile then serves the most heads,
    // and a workgroup of several waves keeps more loads in flight than a lone wave (which
    // measured 2-3x slower per byte). When that leaves fewer than half the compute units a
    // workgroup, halve it (down to two waves): more, shorter workgroups start sooner (each
    // loads Q for fewer heads) and run side by side; measured on 32 queries x 64 heads,
    // 4 -> 2 waves took the kernel from 13.9 to 11.0 us. Further occupancy comes from splits.
    pl.nw = max_nw == 3 ? 2 : max_nw;
    while (pl.nw > 2 && nq * blocks_for(pl.nw) < cus / 2) pl.nw /= 2;
    // Two head blocks per wave (one gathered operand feeds two MFMAs) when there are enough
    // workgroups without splitting: bf16 rows of 512, 128 heads or more.
    pl.hpw = 1;
    if (bf16_rows && a->d == 512 && pl.nw == 4 && a->h >= 8 * kHeadsPerWave &&
        nq * blocks_for(8) >= cus)
        pl.hpw = 2;
    pl.kg = 1;
    const int ntiles = (a->topk + kTileKeys - 1) / kTileKeys;
    // Short lists (at most kMaxColsCompact columns) with enough workgroups for two per
    // compute unit: two-wave workgroups with a two-tile ring and a small index stage, so that
    // two of them share a compute unit and one's memory round trips (Q, the first tile, the
    // output) overlap the other's products.
    // (Plans with two head blocks per wave keep them: one workgroup then gathers for 128 heads.)
    if (bf16_rows && a->d == 512 && pl.hpw == 1 && a->topk <= sa::kMaxColsCompact &&
        nq * blocks_for(2) >= 2 * (int64_t)cus) {
        pl.nw = 2;
        pl.hpw = 1;
        pl.compact = true;
    }
    pl.head_blocks = blocks_for(pl.nw * pl.hpw);
    int64_t wgs = nq * pl.head_blocks;
    int splits = 1;
    if (wgs < cus) {
        const int64_t want = (cus + wgs - 1) / wgs;
        splits = (int)std::max<int64_t>(1, std::min<int64_t>(want, ntiles / kMinTilesPerSplit));
    }
    // Key groups instead of splits (rows of 512; fp8 storage: at most two groups): the four
    // waves of a workgroup take the same 16 or 32 heads and share out the query's tiles,
    // merging their partial results in LDS, which saves the f32 partials (one per head and
    // split, as large as 2 KB per head) and the combine kernel. Measured on 64 queries x 128 heads x 640 columns: 41.5 us with
    // two splits, 36.7 us with two key groups. The most key groups that keep one round of
    // workgroups on the GPU and leave no group without tiles.
    if (splits > 1 && a->d == 512 && pl.hpw == 1 && !pl.compact) {
        for (int kg = bf16_rows ? 4 : 2; kg >= 2; kg /= 2) {
            if (nq * blocks_for(4 / kg) <= cus && ntiles >= kg) {
                pl.kg = kg;
                pl.nw = 4;
                pl.head_blocks = blocks_for(4 / kg);
                splits = 1;
                break;
            }
        }
    } else if (wgs < cus && ntiles >= 2 && a->d == 512 && pl.hpw == 1 && !pl.compact && nq * blocks_for(2) <= cus) {
        // A short list that leaves compute units idle: two key groups of two waves on the
        // same heads. Measured on 32 queries x 64 heads x 128 columns: 11.65 us against 12.0
        // with one two-wave group (four key groups: 12.0), and with fp8 storage 12.4 against
        // 15.4 us (four waves convert each tile).
        pl.kg = 2;
        pl.nw = 4;
        pl.head_blocks = blocks_for(2);
    }
    pl.h_pad = pl.head_blocks * pl.nw / pl.kg * pl.hpw * kHeadsPerWave;
    // a workgroup stages at most kMaxColsPerSplit index columns (kMaxColsFp8Pipe for fp8
    // storage at d = 512)
    const int max_cols = pl.compact ? sa::kMaxColsCompact
                         : !bf16_rows && a->d == 512 ? sa::kMaxColsFp8Pipe : sa::kMaxColsPerSplit;
    const int max_tiles = max_cols / kTileKeys;
    splits = std::max(splits, (ntiles + max_tiles - 1) / max_tiles);
    const int tiles_per_split = (ntiles + splits - 1) / splits;
    pl.cols_per_split = tiles_per_split * kTileKeys;
    pl.splits = (a->topk + pl.cols_per_split - 1) / pl.cols_per_split;
    pl.ws_bytes = pl.dq_bytes;
    if (pl.splits > 1) {
        const size_t slots = (size_t)a->b * a->s * pl.splits * pl.h_pad;
        pl.ws_bytes += slots * a->d * sizeof(float) + slots * 2 * sizeof(float);
    }
    return pl;
}

}  // namespace

SA_EXPORT int sa_abi_version(void) { return SA_ABI_VERSION; }

SA_EXPORT const char* sa_status_string(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported argument combination";
        case SA_ERR_HIP: return "HIP runtime error";
        case SA_ERR_WORKSPACE: return "workspace missing or too small";
        case SA_ERR_SCRATCH: return "the plan needs more than the library's static scratch buffer holds";
        default: return "unknown status";
    }
}

SA_EXPORT int sa_sparse_attn_workspace(const sa_attn_args* a, size_t* bytes) {
    if (!bytes) return SA_ERR_INVALID;
    const int rc = check_shape(a);
    if (rc != SA_OK) return rc;
    *bytes = make_plan(a, cu_count()).ws_bytes;
    return SA_OK;
}

namespace sa {

// Validation, plan and kernel parameters of one sparse_attn call, shared by the entry points
// that take a caller workspace and the one that uses the library's static scratch buffer.
// ws / ws_bytes: the split partials' buffer (may be null when the plan needs none).
int prepare_sparse_attn(const sa_attn_args* a, void* ws, size_t ws_bytes, KParams& p, Plan& pl) {
    int rc = check_shape(a);
    if (rc != SA_OK) return rc;
    rc = check_pointers(a);
    if (rc != SA_OK) return rc;
    pl = make_plan(a, cu_count());
    const int64_t blocks = (int64_t)a->b * a->s * pl.head_blocks * pl.splits;
    if (blocks > INT32_MAX) return SA_ERR_UNSUPPORTED;
    // the combine kernel of a split plan indexes its waves, one per (query, head), in int32
    if (pl.splits > 1 && (int64_t)a->b * a->s * a->h > INT32_MAX - 3) return SA_ERR_UNSUPPORTED;
    if (pl.ws_bytes > 0 && (!ws || ws_bytes < pl.ws_bytes || !aligned(ws, 16)))
        return SA_ERR_WORKSPACE;

    p = KParams{};
    p.b = a->b; p.s = a->s; p.h = a->h; p.d = a->d; p.topk = a->topk; p.kv_rows = a->kv_rows;
    p.q = (const uint16_t*)a->q; p.q_seq_stride = a->q_seq_stride;
    if (pl.dequant) {       // the kernels read the bf16 rows the dequantisation pass writes
        p.kv = (const uint8_t*)ws;
        p.kv_seq_stride_bytes = (int64_t)a->kv_rows * a->d * 2;
    } else {
        p.kv = (const uint8_t*)a->kv;
        p.kv_seq_stride_bytes = a->kv_format == SA_KV_BF16 ? a->kv_seq_stride * 2 : a->kv_seq_stride;
        p.kv_scale = a->kv_scale; p.kv_scale_seq_stride = a->kv_scale_seq_stride;
    }
    p.sink = a->sink;
    p.idx = a->idx; p.idx_seq_stride = a->idx_seq_stride;
    p.scale_log2 = a->scale * 1.4426950408889634f;
    p.out = (uint16_t*)a->out; p.out_seq_stride = a->out_seq_stride;
    p.rope_dim = a->rope_dim; p.rope_cs = a->rope_cos_sin; p.max_pos = a->max_pos;
    p.pos = a->pos; p.pos_seq_stride = a->pos_seq_stride;
    p.splits = pl.splits; p.cols_per_split = pl.cols_per_split;
    p.head_blocks = pl.head_blocks; p.h_pad = pl.h_pad;
    if (pl.splits > 1) {
        const size_t slots = (size_t)a->b * a->s * pl.splits * pl.h_pad;
        p.ws_o = (float*)((uint8_t*)ws + pl.dq_bytes);
        p.ws_ml = p.ws_o + slots * a->d;
    }
    p.flags = a->flags; p.err_word = a->err_word;
    if (a->window > 0) {
        p.window = a->window;
        p.window_mode = a->window_mode;
        p.win_cols = a->window_mode == SA_WINDOW_RING ? a->window : std::min(a->s, a->window);
    }
    return SA_OK;
}

hipError_t run_sparse_attn(const sa_attn_args* a, const KParams& p, const Plan& pl, hipStream_t st) {
    if (pl.dequant) {
        const hipError_t e = launch_dequant_kv((const uint8_t*)a->kv, a->kv_seq_stride, a->kv_scale,
                                               a->kv_scale_seq_stride, a->b, a->kv_rows, a->d,
                                               (uint16_t*)p.kv, st);
        if (e != hipSuccess) return e;
    }
    return launch_sparse_attn(p, a->kv_format == SA_KV_FP8_E4M3_B32 && !pl.dequant, pl.nw, pl.hpw, pl.kg, pl.compact, st);
}

}  // namespace sa

SA_EXPORT int sa_sparse_attn(const sa_attn_args* a, void* stream) {
    sa::KParams p;
    sa::Plan pl;
    const int rc = sa::prepare_sparse_attn(a, a ? a->workspace : nullptr, a ? a->workspace_bytes : 0, p, pl);
    if (rc != SA_OK) return rc;
    const hipError_t e = sa::run_sparse_attn(a, p, pl, (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

SA_EXPORT int sa_window_topk_idxs(int32_t window, int32_t seqlen, int32_t nseq, const int32_t* start_pos,
                                  int32_t* idx, int64_t idx_seq_stride, int64_t idx_row_stride,
                                  int32_t* cols, void* stream) {
    if (window < 1 || seqlen < 1 || nseq < 1 || !idx || !cols) return SA_ERR_INVALID;
    if (start_pos && seqlen > 1) return SA_ERR_UNSUPPORTED;
    const int32_t c = start_pos ? window : (seqlen < window ? seqlen : window);
    if (idx_row_stride < c) return SA_ERR_INVALID;
    if (nseq > 1 && idx_seq_stride < (int64_t)(seqlen - 1) * idx_row_stride + c) return SA_ERR_INVALID;
    if (!aligned(idx, 4) || (start_pos && !aligned(start_pos, 4))) return SA_ERR_INVALID;
    *cols = c;
    const hipError_t e = sa::launch_window_idxs(window, seqlen, nseq, start_pos, idx, idx_seq_stride,
                                                idx_row_stride, c, (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

SA_EXPORT int sa_quant_kv_fp8(const void* kv, int64_t rows, int32_t d, uint8_t* e4m3_out,
                              uint8_t* e8m0_out, void* bf16_out, void* stream) {
    if (!kv || rows < 0 || d < 32 || d % 32 != 0) return SA_ERR_INVALID;
    if (!e4m3_out && !e8m0_out && !bf16_out) return SA_ERR_INVALID;
    if (!aligned(kv, 16) || (e4m3_out && !aligned(e4m3_out, 8)) || (bf16_out && !aligned(bf16_out, 16)))
        return SA_ERR_INVALID;
    if (rows == 0) return SA_OK;
    const hipError_t e = sa::launch_quant_fp8((const uint16_t*)kv, rows, d, e4m3_out, e8m0_out,
                                              (uint16_t*)bf16_out, (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : (e == hipErrorInvalidValue ? SA_ERR_UNSUPPORTED : SA_ERR_HIP);
}

SA_EXPORT int sa_rope_table(int32_t rope_dim, int32_t max_pos, int32_t original_seq_len, float base,
                            float factor, float beta_fast, float beta_slow, float* cos_sin, void* stream) {
    if (rope_dim < 2 || (rope_dim & 1) || max_pos < 1 || original_seq_len < 0 || !cos_sin) return SA_ERR_INVALID;
    if (!std::isfinite(base) || !(base > 1.0f) || !aligned(cos_sin, 8)) return SA_ERR_INVALID;
    int32_t low = 0, high = 0;
    const int yarn = original_seq_len > 0;
    if (yarn) {
        if (!std::isfinite(factor) || !(factor > 0.0f) || !std::isfinite(beta_fast) || !std::isfinite(beta_slow) ||
            !(beta_slow > 0.0f) || !(beta_fast > beta_slow))
            return SA_ERR_INVALID;
        // the pair index whose wavelength fits `rotations` times into original_seq_len
        // (precompute_freqs_cis, corrected_dim), in f64 as the page evaluates it
        auto corrected_dim = [&](double rotations) {
            return rope_dim * std::log((double)original_seq_len / (rotations * 2.0 * M_PI)) / (2.0 * std::log((double)base));
        };
        const double lo = std::floor(corrected_dim(beta_fast));
        const double hi = std::ceil(corrected_dim(beta_slow));
        low = lo > 0.0 ? (int32_t)std::min(lo, (double)INT32_MAX / 2) : 0;
        high = hi < (double)(rope_dim - 1) ? (int32_t)std::max(hi, -(double)INT32_MAX / 2) : rope_dim - 1;
    }
    const hipError_t e = sa::launch_rope_table(rope_dim, max_pos, base, yarn, low, high, factor, cos_sin,
                                               (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : (e == hipErrorInvalidValue ? SA_ERR_UNSUPPORTED : SA_ERR_HIP);
}

SA_EXPORT int sa_kv_write(const sa_kv_write_args* a, void* stream) {
    if (!a) return SA_ERR_INVALID;
    if (a->b < 1 || a->s < 1 || a->cache_rows < 1 || a->window < 0) return SA_ERR_INVALID;
    if (a->d != 64 && a->d != 128 && a->d != 256 && a->d != 512) return SA_ERR_UNSUPPORTED;
    if ((int64_t)a->b * a->s > INT32_MAX) return SA_ERR_UNSUPPORTED;      // rows split in 32 bits
    if (a->rope_dim < 0 || a->rope_dim > a->d || (a->rope_dim & 1)) return SA_ERR_INVALID;
    if (a->kv_format != SA_KV_BF16 && a->kv_format != SA_KV_FP8_E4M3_B32) return SA_ERR_INVALID;
    if ((a->flags & ~(uint32_t)SA_FLAG_CHECK_IDX) != 0) return SA_ERR_INVALID;
    if (!a->x || !a->pos || !a->cache) return SA_ERR_INVALID;
    if (a->rope_dim > 0 && (!a->rope_cos_sin || a->max_pos < 1 || !aligned(a->rope_cos_sin, 8))) return SA_ERR_INVALID;
    if (a->window > 0 ? a->cache_rows < a->window : !a->row0) return SA_ERR_INVALID;
    const bool fp8 = a->kv_format == SA_KV_FP8_E4M3_B32;
    if (fp8 && !a->cache_scale) return SA_ERR_INVALID;
    if ((a->flags & SA_FLAG_CHECK_IDX) && !a->err_word) return SA_ERR_INVALID;
    if (!aligned(a->x, 16) || !aligned(a->cache, fp8 ? 8 : 16) || !aligned(a->pos, 4) ||
        (a->rows_out && !aligned(a->rows_out, 16)) || (a->row0 && !aligned(a->row0, 4)))
        return SA_ERR_INVALID;
    const int64_t sd = (int64_t)a->s * a->d, rd_ = (int64_t)a->cache_rows * a->d;
    if (a->x_seq_stride % 8 || a->cache_seq_stride % 8 || (a->rows_out && a->rows_out_seq_stride % 8))
        return SA_ERR_INVALID;
    if (a->b > 1) {
        if (a->x_seq_stride < sd || a->pos_seq_stride < a->s || a->cache_seq_stride < rd_) return SA_ERR_INVALID;
        if (a->rows_out && a->rows_out_seq_stride < sd) return SA_ERR_INVALID;
        if (fp8 && a->cache_scale_seq_stride < (int64_t)a->cache_rows * (a->d / 32)) return SA_ERR_INVALID;
    }
    sa::KvWriteParams p{};
    p.b = a->b; p.s = a->s; p.d = a->d; p.rope_dim = a->rope_dim;
    p.x = (const uint16_t*)a->x; p.x_seq_stride = a->x_seq_stride;
    p.rope_cs = a->rope_cos_sin; p.max_pos = a->max_pos;
    p.pos = a->pos; p.pos_seq_stride = a->pos_seq_stride;
    p.window = a->window; p.row0 = a->row0; p.cache_rows = a->cache_rows;
    if (fp8) {
        p.cache_codes = (uint8_t*)a->cache;
        p.cache_scales = a->cache_scale; p.cache_scale_seq_stride = a->cache_scale_seq_stride;
    } else {
        p.cache_bf16 = (uint16_t*)a->cache;
    }
    p.cache_seq_stride = a->cache_seq_stride;
    p.rows_out = (uint16_t*)a->rows_out; p.rows_out_seq_stride = a->rows_out_seq_stride;
    p.flags = a->flags; p.err_word = a->err_word;
    const hipError_t e = sa::launch_kv_write(p, (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : (e == hipErrorInvalidValue ? SA_ERR_UNSUPPORTED : SA_ERR_HIP);
}

SA_EXPORT int sa_indexer_topk(const sa_indexer_args* a, void* stream) {
    if (!a) return SA_ERR_INVALID;
    if (a->b < 1 || a->s < 1 || a->n_pos < 1 || a->ratio < 1 || a->h < 1) return SA_ERR_INVALID;
    if (a->d != 64 && a->d != 128 && a->d != 256) return SA_ERR_UNSUPPORTED;
    if (a->h != 16 && a->h != 32 && a->h != 64) return SA_ERR_UNSUPPORTED;
    if (a->h == 64 && a->d > 128) return SA_ERR_UNSUPPORTED;
    if (!a->q || !a->k || !a->w || !a->pos || !a->scores) return SA_ERR_INVALID;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->w, 4) || !aligned(a->pos, 4) ||
        !aligned(a->scores, 4) || (a->idx && !aligned(a->idx, 4)))
        return SA_ERR_INVALID;
    if (a->q_seq_stride % 8 || a->k_seq_stride % 8) return SA_ERR_INVALID;
    // a query's score row is addressed as one buffer of n_pos f32 (32-bit byte offsets)
    if (a->n_pos > (1 << 28)) return SA_ERR_UNSUPPORTED;
    const int64_t s_np = (int64_t)a->s * a->n_pos;
    if (a->b > 1) {
        if (a->q_seq_stride < (int64_t)a->s * a->h * a->d || a->k_seq_stride < (int64_t)a->n_pos * a->d ||
            a->w_seq_stride < (int64_t)a->s * a->h || a->pos_seq_stride < a->s || a->scores_seq_stride < s_np ||
            (a->cand && a->cand_seq_stride < s_np))
            return SA_ERR_INVALID;
    }
    if (a->idx) {
        if (a->topk < 1 || a->idx_row_stride < a->topk) return SA_ERR_INVALID;
        if (a->b > 1 && a->idx_seq_stride < (int64_t)(a->s - 1) * a->idx_row_stride + a->topk) return SA_ERR_INVALID;
        if (a->n_pos > 32768) return SA_ERR_UNSUPPORTED;
    }
    sa::IdxParams p{};
    p.b = a->b; p.s = a->s; p.h = a->h; p.d = a->d; p.n_pos = a->n_pos; p.ratio = a->ratio;
    p.q = (const uint16_t*)a->q; p.q_seq_stride = a->q_seq_stride;
    p.k = (const uint16_t*)a->k; p.k_seq_stride = a->k_seq_stride;
    p.w = a->w; p.w_seq_stride = a->w_seq_stride;
    p.pos = a->pos; p.pos_seq_stride = a->pos_seq_stride;
    p.cand = a->cand; p.cand_seq_stride = a->cand_seq_stride;
    p.scores = a->scores; p.scores_seq_stride = a->scores_seq_stride;
    p.topk = a->topk; p.offset = a->offset;
    p.idx = a->idx; p.idx_seq_stride = a->idx_seq_stride; p.idx_row_stride = a->idx_row_stride;
    hipError_t e = sa::launch_index_scores(p, (hipStream_t)stream);
    if (e == hipSuccess && a->idx) e = sa::launch_index_topk(p, (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : (e == hipErrorInvalidValue ? SA_ERR_UNSUPPORTED : SA_ERR_HIP);
}

SA_EXPORT int sa_candidate_blocks(const sa_candidate_args* a, void* stream) {
    if (!a) return SA_ERR_INVALID;
    if (a->b < 1 || a->s < 1 || a->n_pos < 1 || a->ratio < 1 || a->topk_blocks < 1 || a->block_size < 1)
        return SA_ERR_INVALID;
    if (!a->logits || !a->pos || !a->mask || !aligned(a->logits, 4) || !aligned(a->pos, 4)) return SA_ERR_INVALID;
    const int64_t s_np = (int64_t)a->s * a->n_pos;
    if (a->b > 1 && (a->logits_seq_stride < s_np || a->mask_seq_stride < s_np || a->pos_seq_stride < a->s))
        return SA_ERR_INVALID;
    if ((a->n_pos + (int64_t)a->block_size - 1) / a->block_size > 32768) return SA_ERR_UNSUPPORTED;
    sa::CandParams p{};
    p.b = a->b; p.s = a->s; p.n_pos = a->n_pos; p.ratio = a->ratio;
    p.topk_blocks = a->topk_blocks; p.block_size = a->block_size;
    p.logits = a->logits; p.logits_seq_stride = a->logits_seq_stride;
    p.pos = a->pos; p.pos_seq_stride = a->pos_seq_stride;
    p.mask = a->mask; p.mask_seq_stride = a->mask_seq_stride;
    const hipError_t e = sa::launch_candidate_blocks(p, (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : (e == hipErrorInvalidValue ? SA_ERR_UNSUPPORTED : SA_ERR_HIP);
}

SA_EXPORT int sa_grouped_proj(const sa_grouped_proj_args* a, void* stream) {
    if (!a) return SA_ERR_INVALID;
    if (a->m < 1 || a->g < 1 || a->r < 1 || a->kg < 1) return SA_ERR_INVALID;
    if (a->w_format != SA_KV_BF16 && a->w_format != SA_KV_FP8_E4M3_B32) return SA_ERR_INVALID;
    const bool fp8 = a->w_format == SA_KV_FP8_E4M3_B32;
    if (!a->o || !a->w || !a->out || (fp8 && !a->w_scale)) return SA_ERR_INVALID;
    if (!aligned(a->o, 16) || !aligned(a->w, 16) || !aligned(a->out, 16) || (fp8 && !aligned(a->w_scale, 4)))
        return SA_ERR_INVALID;
    if (a->o_stride < (int64_t)a->g * a->kg || a->out_stride < (int64_t)a->g * a->r || a->o_stride % 8 ||
        a->out_stride % 8)
        return SA_ERR_INVALID;
    const bool skinny = a->m <= 64 && ((a->r % 32 == 0 && a->kg % 256 == 0) || (a->r % 16 == 0 && a->kg % 512 == 0));
    if (!skinny && (a->r % 128 != 0 || a->kg % 64 != 0)) return SA_ERR_UNSUPPORTED;
    if ((int64_t)a->g * a->r * a->kg > ((int64_t)1 << 40)) return SA_ERR_UNSUPPORTED;
    sa::ProjParams p{};
    p.m = a->m; p.g = a->g; p.r = a->r; p.kg = a->kg;
    p.o = (const uint16_t*)a->o; p.o_stride = a->o_stride;
    if (fp8) {
        p.wq = (const uint8_t*)a->w;
        p.ws = a->w_scale;
    } else {
        p.w = (const uint16_t*)a->w;
    }
    p.out = (uint16_t*)a->out; p.out_stride = a->out_stride;
    const hipError_t e = sa::launch_grouped_proj(p, (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : (e == hipErrorInvalidValue ? SA_ERR_UNSUPPORTED : SA_ERR_HIP);
}
