// sparse_attn for gfx950: one workgroup per (query, block of heads, split of the index
// columns). The operation follows the attention API docs ("sparse_attn", precision
// paragraph) and the call in Attention.forward: per query and head, a softmax in f32 over
// the gathered latent rows plus the sink (denominator only), bf16 output.
//
// Work inside a workgroup of NW waves (NW = 1, 2 or 4), HPW blocks of 16 heads per wave:
//   * key tiles of 32 index columns are gathered row by row from HBM straight into LDS
//     (buffer_load_dwordx4 ... lds, 16 B per lane) through a ring of 4 buffers, 2 tiles in
//     flight ahead of the two being worked on. All waves of the workgroup read the same
//     tile: one gather serves every head of the query in the workgroup. Rows carry a
//     16-byte-chunk XOR swizzle so that both LDS read patterns below avoid bank conflicts.
//   * scores are computed transposed, S^T[key][head] = K . Q^T, on v_mfma_f32_16x16x32_bf16:
//     K comes from LDS as the A operand (each read feeds the HPW head blocks), Q stays in
//     registers as the B operand. In the accumulator layout each lane holds one head and 4
//     keys per 16-key block, so the softmax needs in-lane work plus two exchanges across
//     the 4 lane groups.
//   * the probabilities are rounded to bf16 in registers and are already the B operand of
//     O^T[d][head] += V^T . P^T (a 32-key step); V^T is read from the same LDS tile with the
//     transposing ds_read_b64_tr_b16, so the tile is stored once and is both K and V.
//   * the key loop is software-pipelined: iteration t scores tile t, then multiplies the
//     probabilities of tile t-1 while tile t's softmax steps run between those matrix
//     instructions.
//   * softmax against a fixed reference per head (taken at the first tile that names a row,
//     from the sink and that tile's scores), with a rare second pass over the keys when a
//     later score exceeds it by too much: O is never rescaled inside the key loop and stays
//     in accumulator registers (4 f32 per lane per 16-wide slice of d and head block).
//   * the sink enters the running sum as exp(sink - reference), in one lane group and in
//     split 0 and key group 0 only, which puts it in the denominator.
//   * key groups (KG > 1): the waves share a query's heads and split its tiles; their
//     partial results are merged in LDS.
//   * fp8 storage: tiles of e4m3 codes and e8m0 scales are gathered into raw slots and
//     converted in LDS to the bf16 tiles above (exact), so the products are the same.
//   * with more than one split, unnormalised partials (O, reference, sum) go to the
//     workspace and a small combine kernel merges them; otherwise the epilogue (divide,
//     bf16, optional inverse RoPE) runs here.
#pragma once

#include "lds_dma.hpp"
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;

// 16-byte chunk swizzle of LDS row r. Both operand reads must hit distinct banks (64 banks
// of 4 bytes; a bank group is a 16-byte chunk index mod 16):
//   V operand: a transposing read serves 32 lanes at a time, covering 8 consecutive rows x
//   2 adjacent chunks (c, c^1) -> swz(r) >> 1 must differ across every 8 aligned rows;
//   K operand: each ds_read_b128 lane group (two octets) reads rows 0-7 at chunk c and rows
//   8-15 at chunk c ^ 2 -> swz must map rows 0-7 and rows 8-15 to complementary sets that
//   the XOR by 2 keeps apart.
// ((r & 7) << 1) | ((r >> 3) & 1) does both (rows 0-7 -> even, rows 8-15 -> odd chunks); it
// only changes the low four bits of a chunk index (for rows narrower than 16 chunks it is
// cut down to the row).
template <int CH>
__device__ __forceinline__ int swz(int r) {
    return (((r & 7) << 1) | ((r >> 3) & 1)) & (CH - 1);
}

template <int D>
struct Geo {
    static constexpr int kRowBytes = D * 2;                 // one bf16 row in LDS
    static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
    static constexpr int kRowsPerInst = 64 / kChunks;       // rows one wave load covers
    static constexpr int kKSteps = D / 32;                  // QK k-steps (32 d each)
    static constexpr int kDBlocks = D / 16;                 // 16-wide slices of d for PV
    static constexpr int kTileBytes = kTileKeys * kRowBytes;
};

// What the index stage in LDS holds per column: with bf16 storage the row's byte offset in
// the KV buffer (row * 2 D, which the host keeps below 2^31) or kBufferPastEnd for a skip,
// so that a gather needs one OR per load; with fp8 storage the row, or -1 for a skip. Either
// way a column names a row exactly when its word is below kBufferPastEnd.
template <bool FP8, int D>
__device__ __forceinline__ int stage_word(int row) {
    if constexpr (FP8) return row;
    else return row < 0 ? kBufferPastEnd : row * (2 * D);
}
__device__ __forceinline__ bool staged_row(int w) { return (uint32_t)w < (uint32_t)kBufferPastEnd; }

// Direct-to-LDS gather of one key tile (bf16 storage). The tile's byte offsets are read
// from the index stage in LDS. Every wave issues exactly kInsts/NW loads per tile, whatever
// the indices, so that waiting for the oldest tile in flight is an exact vmcnt: a skipped
// row is loaded from an offset past the end of the buffer (kBufferPastEnd with the lane's
// chunk ORed into bits it already has set), for which the buffer's range check returns zeros
// without a memory access, so it lands as a zero row (a zero row can never turn a zero
// probability into a NaN).
// Wave wid issues loads wid*kPer .. wid*kPer+kPer-1 of the tile; load j covers rows
// j*kRowsPerInst .. +kRowsPerInst-1. All row indices are read before the first load issues.
template <int D, int NW>
__device__ __forceinline__ void gather_tile_bf16(i32x4 rsrc, SA_LDS const int32_t* tidx,
                                                 SA_LDS uint8_t* buf, int wid, int lane) {
    using G = Geo<D>;
    constexpr int kInsts = kTileKeys / G::kRowsPerInst;
    static_assert(kTileKeys % G::kRowsPerInst == 0 && kInsts % NW == 0, "tile split");
    constexpr int kPer = kInsts / NW;
    const int sub = lane / G::kChunks;          // row within one load
    const int pc = lane % G::kChunks;           // physical chunk this lane fills
    int rows[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) rows[j] = tidx[(wid * kPer + j) * G::kRowsPerInst + sub];   // byte offsets
    const uint32_t base = lds_byte_addr(buf);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int r0 = (wid * kPer + j) * G::kRowsPerInst;
        const int r = r0 + sub;
        const int voff = rows[j] | ((pc ^ swz<G::kChunks>(r)) << 4);
        lds_dma16(rsrc, __builtin_amdgcn_readfirstlane(base + r0 * G::kRowBytes), voff);
    }
}

// fp8 storage: the gather of e4m3 codes (D bytes per row) and the row's D/32 scale bytes
// into a raw staging tile (zeros for skipped rows), converted to the bf16 tile by
// convert_tile_fp8.
template <int D, int NW>
__device__ __forceinline__ void gather_tile_fp8(const uint8_t* kv_seq, const uint8_t* sc_seq,
                                                SA_LDS const int32_t* tidx, SA_LDS uint8_t* raw,
                                                SA_LDS uint8_t* raw_sc, int wid, int lane) {
    constexpr int kCodeChunks = D / 16;                    // 16-byte chunks of codes per row
    constexpr int kRowsPerInst = 64 / kCodeChunks;
    constexpr int kInsts = kTileKeys / kRowsPerInst;
    static_assert(kTileKeys % kRowsPerInst == 0, "tile split");
    const int sub = lane / kCodeChunks;
    const int pc = lane % kCodeChunks;
#pragma unroll
    for (int j = 0; j < (kInsts + NW - 1) / NW; ++j) {
        const int i = wid + j * NW;
        if (i >= kInsts) break;
        const int r0 = i * kRowsPerInst;
        const int r = r0 + sub;
        const int row = tidx[r];
        if (row >= 0) {
            const uint8_t* src = kv_seq + (int64_t)row * D + pc * 16;
            __builtin_amdgcn_global_load_lds((const void*)src, (SA_LDS void*)(raw + r0 * D), 16, 0, 0);
        } else {
            *(SA_LDS u32x4*)(raw + r * D + pc * 16) = u32x4{0, 0, 0, 0};
        }
    }
    constexpr int kSc = D / 32;
    if (wid == 0 && lane < kTileKeys) {
        const int row = tidx[lane];
        for (int j = 0; j < kSc; ++j)
            raw_sc[lane * kSc + j] = row >= 0 ? sc_seq[(int64_t)row * kSc + j] : (uint8_t)0;
    }
}

// e4m3fn code -> f32 (exact): placing the 7 magnitude bits at f32 bits 20..26 gives the
// code's value times 2^-120 for normal and subnormal codes alike.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    return bits_f32(((c & 0x80u) << 24) | ((c & 0x7fu) << 20)) * 0x1p120f;
}

template <int D, int NW>
__device__ __forceinline__ void convert_tile_fp8(SA_LDS const uint8_t* raw, SA_LDS const uint8_t* raw_sc,
                                                 SA_LDS uint8_t* buf, int tid) {
    using G = Geo<D>;
    constexpr int kUnits = kTileKeys * D / 8;              // 8 codes -> one 16-byte bf16 chunk
    for (int u = tid; u < kUnits; u += NW * kWave) {
        const int r = u / (D / 8);
        const int c8 = u % (D / 8);                         // logical 16-byte chunk of the row
        const u32x2 codes = *(SA_LDS const u32x2*)(raw + r * D + c8 * 8);
        const float s = bits_f32((uint32_t)raw_sc[r * (D / 32) + (c8 * 8) / 32] << 23);
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w = codes[k >> 1] >> ((k & 1) * 16);
            // the product of an e4m3 value and a power of two has at most 4 significant
            // bits, so dropping the low half of the f32 is the exact bf16 value
            const uint32_t lo = f32_bits(e4m3_to_f32(w & 0xffu) * s) >> 16;
            const uint32_t hi = f32_bits(e4m3_to_f32((w >> 8) & 0xffu) * s) >> 16;
            o[k] = lo | (hi << 16);
        }
        const int pcn = c8 ^ swz<G::kChunks>(r);
        *(SA_LDS u32x4*)(buf + r * G::kRowBytes + pcn * 16) = o;
    }
}

// fp8 storage at d = 512, pipelined: a raw slot holds a tile's e4m3 codes ([32][D] bytes)
// followed by its e8m0 scale bytes ([32][D/32]).
template <int D>
struct RawSlot {
    static constexpr int kCodes = kTileKeys * D;
    static constexpr int kBytes = kCodes + kTileKeys * (D / 32);
};

// Direct-to-LDS gather of one tile's codes and scale bytes into a raw slot. Codes: 16 B per
// lane, two rows of 512 codes per load, dealt to the waves (kTileKeys * D / 1024 / NW loads
// each); scales: one load per wave, a lane per row (rows wid * 32/NW ..), 16 bytes each.
// Every wave issues the same number of loads, so the waits are exact vmcnt counts; a skipped
// column loads row 0, and the conversion writes zeros for it.
template <int D, int NW>
struct RawGather {
    static_assert(D == 512, "pipelined fp8 path: rows of 512 codes");
    static constexpr int kCodeLoads = RawSlot<D>::kCodes / 1024 / NW;
    static constexpr int kLoads = kCodeLoads + 1;            // loads per wave per tile
    __device__ static void issue(i32x4 codes_rsrc, i32x4 sc_rsrc, SA_LDS const int32_t* tidx,
                                 SA_LDS uint8_t* slot, int wid, int lane) {
        const int sub = lane >> 5, pc = lane & 31;
        int rows[kCodeLoads];
#pragma unroll
        for (int j = 0; j < kCodeLoads; ++j) rows[j] = tidx[2 * (wid * kCodeLoads + j) + sub];
        constexpr int kScRows = kTileKeys / NW;
        const int sc_row = tidx[wid * kScRows + (lane & (kScRows - 1))];
        const uint32_t base = lds_byte_addr(slot);
        // a skipped row (-1) is loaded from past the end of the buffer: zero codes and a zero
        // scale byte, which the conversion turns into a zero row by itself
#pragma unroll
        for (int j = 0; j < kCodeLoads; ++j)
            lds_dma16(codes_rsrc, __builtin_amdgcn_readfirstlane(base + 2 * (wid * kCodeLoads + j) * D),
                  rows[j] < 0 ? kBufferPastEnd : rows[j] * D + 16 * pc);
        if (lane < kScRows)
            lds_dma16(sc_rsrc, __builtin_amdgcn_readfirstlane(base + RawSlot<D>::kCodes + wid * kScRows * (D / 32)),
                  sc_row < 0 ? kBufferPastEnd : sc_row * (D / 32));
    }
};

// Codes of a landed raw slot -> the bf16 tile (same layout and swizzle as a gathered bf16
// tile), on v_cvt_scalef32_pk_bf16_fp8: each code times its block's scale 2^(e - 127), which
// is exact in bf16 (the stored values are bf16 values). A lane converts 8 codes (one 16-byte
// bf16 chunk) per step, a wave one row; skipped columns, gathered as zero codes with a zero
// scale, become zero rows.
template <int D, int NW>
__device__ __forceinline__ void convert_raw_fp8(SA_LDS const uint8_t* slot, SA_LDS const int32_t* tidx,
                                                SA_LDS uint8_t* buf, int wid, int lane) {
    using G = Geo<D>;
    static_assert(G::kChunks == kWave, "one bf16 row per wave and step");
    constexpr int kSteps = kTileKeys / NW;                      // rows per wave
    constexpr int kBatch = kSteps < 4 ? kSteps : 4;
    // The reads of a batch of rows go out before its writes: the compiler cannot tell that a
    // write to the bf16 tile never meets a later read of the raw slot, so row by row it would
    // wait for each read in turn.
#pragma unroll
    for (int j0 = 0; j0 < kSteps; j0 += kBatch) {
        u32x2 codes[kBatch];
        uint32_t sbyte[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int r = (j0 + u) * NW + wid;
            codes[u] = *(SA_LDS const u32x2*)(slot + r * D + 8 * lane);
            sbyte[u] = slot[RawSlot<D>::kCodes + r * (D / 32) + (lane >> 2)];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int r = (j0 + u) * NW + wid;
            const float sc = bits_f32(sbyte[u] << 23);
            u32x4 o;
            o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[u][0], sc, false));
            o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[u][0], sc, true));
            o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[u][1], sc, false));
            o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[u][1], sc, true));
            *(SA_LDS u32x4*)(buf + r * G::kRowBytes + ((lane ^ swz<G::kChunks>(r)) << 4)) = o;
        }
    }
}

// Score product step with the accumulator in VGPRs: acc (+)= A . B on
// v_mfma_f32_16x16x32_bf16. Written as inline assembly because the compiler picks one
// register class for every MFMA accumulator of a kernel: with O in AGPRs (the kernels that
// hold 32 heads per wave need all 256 of them for O) it would give the scores AGPRs too and
// move part of O in and out of VGPRs around every tile. The compiler does not see these as
// matrix instructions, so the hazards it would otherwise handle are handled here:
//   * the A and B operands come from LDS (waits on its counter, which the compiler inserts
//     for the asm inputs) or are Q, held in VGPRs since start-up: no vector instruction
//     writes them just ahead (checked on the compiled code of the kernel that uses this);
//   * back-to-back steps on the same accumulator (same opcode, same registers) need no wait
//     states;
//   * vector instructions read the result only after mfma_v_drain, which waits out the
//     pipeline (an 8-pass matrix instruction needs 11 wait states before a vector read or
//     write of its result; 24 are given) and is tied to every accumulator, so that no read
//     can be scheduled ahead of it.
__device__ __forceinline__ void mfma_vz(f32x4& acc, const u32x4& a, const u32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4& acc, const u32x4& a, const u32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <int N>
__device__ __forceinline__ void mfma_v_drain(f32x4 (&acc)[2][N]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < N; ++n) asm volatile("" : "+v"(acc[m][n]));
}

// Epilogue for 4 consecutive output elements d0..d0+3 of one head: o = acc * inv_l rounded
// to bf16; with `rot`, the inverse rotation of the pairs that fall in the last rope_dim
// elements (apply_rotary_emb with inverse=True: multiply by the conjugate in f32, back to
// bf16). A pair outside the rope tail is rotated by (1, 0), which returns it unchanged.
// `cs` is the position's row of the (cos, sin) table. Returns two packed bf16 pairs.
template <typename CsPtr>
__device__ __forceinline__ u32x2 epilogue4(float a0, float a1, float a2, float a3, float inv_l,
                                           bool rot, int d0, int r0, CsPtr cs) {
    uint32_t w[2] = {pack_bf16x2(a0 * inv_l, a1 * inv_l), pack_bf16x2(a2 * inv_l, a3 * inv_l)};
    if (rot) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int dk = d0 + 2 * k;
            const bool in = dk >= r0;
            const int o = in ? (dk - r0) : 0;
            const float c = in ? cs[o] : 1.0f, sn = in ? cs[o + 1] : 0.0f;
            const float x = bf16_lo(w[k]), y = bf16_hi(w[k]);
            w[k] = pack_bf16x2(x * c + y * sn, y * c - x * sn);
        }
    }
    return u32x2{w[0], w[1]};
}

// Position of query t of sequence seq and its (cos, sin) row, or nullptr when the epilogue
// is off or the position has no row in the table (then no rotation is applied; bit 2 of
// the error word records it when checking is on).
// The position is read with a vector load (through a zero offset held in a vector register,
// which the compiler cannot see through): a scalar load would be waited for together with the
// kernel-argument loads (scalar loads complete out of order, so the compiler can only wait
// for all of them), which would hold back every load issued after that wait by one memory
// round trip.
__device__ __forceinline__ int rope_pos(const KParams& p, int seq, int t) {
    if (p.rope_dim == 0 && p.window == 0) return 0;
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    return p.pos[(int64_t)seq * p.pos_seq_stride + t + zero];
}
__device__ __forceinline__ const float* rope_ptr(const KParams& p, int pos, bool report) {
    if (p.rope_dim == 0) return nullptr;
    if (pos < 0 || pos >= p.max_pos) {
        if (report && (p.flags & 1u)) atomicOr(p.err_word, 2);
        return nullptr;
    }
    return p.rope_cs + (int64_t)pos * p.rope_dim;
}
__device__ __forceinline__ const float* rope_row(const KParams& p, int seq, int t, bool report) {
    return rope_ptr(p, rope_pos(p, seq, t), report);
}

// The fused window list of a query at position pos (the window_topk_idxs lists): ring
// (decode): the slots of a ring of `window` rows oldest first; chunk (prefill from 0): the
// chunk rows max(0, pos - window + 1) .. pos; -1 where the list holds nothing. The one
// division is done once per query (`first`: the slot of the oldest token of a full ring, or
// the chunk's first row); an entry is then an add and a compare.
struct WindowList {
    int pos, window, first;
    bool full;
    __device__ __forceinline__ WindowList(const KParams& p, int pos_) : pos(pos_), window(p.window) {
        const bool ring = p.window_mode == 1;
        full = ring && pos >= window - 1;
        first = ring ? (full ? (pos + 1) % window : 0) : max(0, pos - window + 1);
    }
    // entry j; a negative position lists nothing (first + j > pos)
    __device__ __forceinline__ int operator()(int j) const {
        const int v = first + j;
        return full ? (v >= window ? v - window : v) : (v <= pos ? v : -1);
    }
};

// Work item of block b (items are query-major: item = query * per_q + j). Workgroups are
// dealt to the 8 XCDs round-robin: block b runs on XCD b % 8, as the (b / 8)-th workgroup
// there. The per_q items of one query (its head blocks and splits, which gather the same
// rows) go to one XCD back to back, so they share its L2; queries go round-robin over the
// XCDs, so each XCD gets an equal share of the work even when the work per query grows with
// the query index (causal prefill); each XCD takes its queries in descending order, so the
// longest start first. The last nq % 8 queries keep the identity order.
__device__ __forceinline__ int work_item(int b, int nq, int per_q) {
    const int q8 = nq / 8;
    if (b >= q8 * 8 * per_q) return b;
    const int x = b % 8, k = b / 8;
    const int r = k / per_q, j = k % per_q;
    return (8 * (q8 - 1 - r) + x) * per_q + j;
}

__device__ __forceinline__ float sum4groups(float v) { return sum_xor32(sum_xor16(v)); }
__device__ __forceinline__ float max4groups(float v) { return max_xor32(max_xor16(v)); }

// Pipeline shape of the bf16 path: kBuffers LDS tile buffers, tiles gathered kAhead ahead
// of the one being multiplied. The only vector-memory operations inside the key loop are
// the tile loads (kLoadsPerWave per wave per tile), so when tile t is needed the loads
// issued after it are exactly those of tiles t+1 .. t+kAhead-1: the wait is vmcnt(kWait),
// which must fit the 6-bit counter.
template <int D, int NW>
struct Pipe {
    static constexpr int kLoadsPerWave = kTileKeys / Geo<D>::kRowsPerInst / NW;
    static constexpr int kBuffers = 4;
    static constexpr int kAheadMax = 1 + 63 / kLoadsPerWave;
    static constexpr int kAhead = kBuffers - 1 < kAheadMax ? kBuffers - 1 : kAheadMax;
    static constexpr int kWait = (kAhead - 1) * kLoadsPerWave;
};

// LDS plan of one kernel instance: the index stage, the bf16 tile buffers and, for fp8
// storage, the raw slots of codes and scales.
template <int D, bool FP8, int NW, bool CMP = false>
struct KernelLds {
    static constexpr bool kFp8Pipe = FP8 && D == 512;
    // bf16: the ring of the pipelined loop (compact: two tiles, the next gathered while the
    // current one is worked on); fp8 at d = 512: the tiles being scored, multiplied and
    // converted; other fp8: one tile
    static constexpr int kTileBufs = CMP ? 2 : FP8 ? (kFp8Pipe ? 3 : 1) : Pipe<D, NW>::kBuffers;
    static constexpr int kRawSlots = FP8 ? (kFp8Pipe ? 3 : 2) : 0;
    // the pipelined fp8 path stages fewer index columns so that its slots fit in LDS; the
    // compact layout stages few, so that two workgroups share a compute unit's LDS
    static constexpr int kStageCols = CMP ? kMaxColsCompact : kFp8Pipe ? kMaxColsFp8Pipe : kMaxColsPerSplit;
    static constexpr size_t kTiles = (size_t)kTileBufs * Geo<D>::kTileBytes + (size_t)kRawSlots * RawSlot<D>::kBytes;
};


// KG key groups: the NW waves form NW / KG head groups times KG key groups; the waves of
// one key group take every KG-th tile of the item's index columns, so one query's keys are
// worked on by KG waves side by side, and their partial results are merged in LDS at the
// end (KG = 1: every wave takes every tile, for its own heads).
template <int D, bool FP8, int NW, int HPW, int KG = 1, bool CMP = false>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_kernel(const KParams p) {
    static_assert(KG == 1 || ((!FP8 || D == 512) && NW % KG == 0), "key groups: bf16, or fp8 at d = 512");
    static_assert(!CMP || (KG == 1 && !FP8), "compact layout: bf16 storage, one key group");
    constexpr int HB = NW / KG;                 // head groups of the workgroup
    using G = Geo<D>;
    using PP = Pipe<D, NW>;
    using KL = KernelLds<D, FP8, NW, CMP>;
    constexpr int NB = KL::kTileBufs;
    constexpr bool kFp8Pipe = KL::kFp8Pipe;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    SA_LDS uint8_t* smem = (SA_LDS uint8_t*)smem_raw;
    // LDS: the index stage (KL::kStageCols int32), 64 B of flags, the position's (cos, sin)
    // row (D f32), then NB bf16 tiles; fp8 adds raw slots of codes and scale bytes.
    SA_LDS int32_t* istage = (SA_LDS int32_t*)smem;
    SA_LDS float* cs_lds = (SA_LDS float*)(smem + KL::kStageCols * 4 + 64);
    SA_LDS uint8_t* tiles = smem + KL::kStageCols * 4 + 64 + D * 4;
    auto tile = [&](int i) { return tiles + i * G::kTileBytes; };
    auto raw = [&](int i) { return tiles + NB * G::kTileBytes + i * RawSlot<D>::kBytes; };
    auto raw_sc = [&](int i) { return raw(i) + RawSlot<D>::kCodes; };

    // The kernel arguments that start-up needs, all at once: scalar loads complete out of
    // order, so the compiler can only wait for all of them, and loads placed next to their
    // uses would cost one memory round trip per group before the first vector load issues.
    asm volatile("" ::"s"(p.q), "s"(p.q_seq_stride), "s"(p.idx), "s"(p.idx_seq_stride), "s"(p.pos),
                 "s"(p.pos_seq_stride), "s"(p.sink), "s"(p.kv), "s"(p.kv_seq_stride_bytes), "s"(p.b),
                 "s"(p.s), "s"(p.h), "s"(p.topk), "s"(p.kv_rows), "s"(p.rope_dim), "s"(p.splits),
                 "s"(p.cols_per_split), "s"(p.head_blocks));
    const int tid = threadIdx.x;
    // the wave index in a scalar register: what derives from it (key group, head group, the
    // gather's LDS destinations) is then uniform to the compiler too
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int kg = wid / HB;                    // this wave's key group
    const int hbw = wid % HB;                   // and head group
    const int l16 = lane & 15;                  // this lane's head within a 16-head block
    const int q4 = lane >> 4;                   // lane group 0..3
    // d chunk (8 elements) that lane group q4 takes in each 32-wide step of the QK product:
    // 0, 2, 1, 3. Any order is correct as long as K and Q use the same one; this one keeps the
    // K operand reads free of bank conflicts (ds_read_b128 serves the lanes in four groups of
    // two octets, {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63}, {40-47, 48-55}, and with the
    // row swizzle below these groups then read sixteen distinct 16-byte bank groups).
    const int qc = ((q4 & 1) << 1) | (q4 >> 1);

    // work item: ((query * head_blocks) + head block) * splits + split, in the XCD-aware
    // order of work_item
    int item = work_item(blockIdx.x, p.b * p.s, p.head_blocks * p.splits);
    const int split = item % p.splits;
    item /= p.splits;
    const int hblk = item % p.head_blocks;
    const int qi = item / p.head_blocks;
    const int seq = qi / p.s;
    const int t = qi % p.s;

    // the wave's HPW blocks of 16 heads: head(hb) = head0 + 16*hb + l16
    const int head0 = (hblk * HB + hbw) * HPW * kHeadsPerWave + l16;
    auto head_of = [&](int hb) { return head0 + hb * kHeadsPerWave; };

    const int32_t* idx_row = p.idx + (int64_t)seq * p.idx_seq_stride + (int64_t)t * p.topk;
    const int col_begin = split * p.cols_per_split;
    const int ncols = max(0, min(p.topk, col_begin + p.cols_per_split) - col_begin);

    const uint8_t* kv_seq = p.kv + (int64_t)seq * p.kv_seq_stride_bytes;
    const uint8_t* sc_seq = FP8 ? p.kv_scale + (int64_t)seq * p.kv_scale_seq_stride : nullptr;
    const i32x4 kv_rsrc = make_buffer_rsrc(kv_seq, (uint32_t)p.kv_rows * (uint32_t)(FP8 ? D : 2 * D));

    // ---- start-up, arranged so that its memory latencies overlap: the position and the
    // index loads go out first, then Q and the sink; the index stage is written as soon as
    // the index loads land (Q may still be in flight).
    // Every load here is issued by every lane (addresses clamped instead of per-lane
    // branches), so the compiler's waits for one group never cover the next.
    const int pos = rope_pos(p, seq, t);

    // Stage this split's index columns in LDS, skips and out-of-range rows as -1, padded
    // to whole tiles, and find the last column that names a row (trailing tiles of padding
    // are never gathered). Each thread issues kStageUnroll index loads at a time; columns
    // past the end re-read the last column and are masked afterwards.
    constexpr int kStageUnroll = 16;
    const int ncols_pad = (ncols + kTileKeys - 1) / kTileKeys * kTileKeys;
    const int32_t* cols = idx_row + col_begin;
    int err = 0;
    int last = -1;
    int stage_v[kStageUnroll];
    // with fused window lists, columns below win_cols are generated from the position and
    // idx is read only from there on (its loads are clamped to that range)
    const int gen_end = min(ncols, max(0, p.win_cols - col_begin));      // generated columns
    const bool any_loaded = gen_end < ncols;
    if (any_loaded) {
#pragma unroll
        for (int u = 0; u < kStageUnroll; ++u) stage_v[u] = cols[max(gen_end, min(tid + u * NW * kWave, ncols - 1))];
    } else {
#pragma unroll
        for (int u = 0; u < kStageUnroll; ++u) stage_v[u] = -1;
    }
    // Q as the B operand of the 16x16x32 product: lane holds head l16 of each block,
    // d = 32*kk + 8*qc + 0..7. Padding heads (past h) repeat the last head: they are never
    // stored, and their softmax, identical to that head's, flags nothing new.
    u32x4 qreg[HPW][G::kKSteps];
    float sink_raw[HPW];
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
        const int hq = min(head_of(hb), p.h - 1);
        const uint16_t* qrow = p.q + (int64_t)seq * p.q_seq_stride + ((int64_t)t * p.h + hq) * D;
#pragma unroll
        for (int kk = 0; kk < G::kKSteps; ++kk) qreg[hb][kk] = *(const u32x4*)(qrow + 32 * kk + 8 * qc);
        sink_raw[hb] = p.sink[hq];
    }
    for (int c0 = 0; c0 < ncols_pad; c0 += kStageUnroll * NW * kWave) {
        if (c0 > 0 && any_loaded) {
#pragma unroll
            for (int u = 0; u < kStageUnroll; ++u) stage_v[u] = cols[max(gen_end, min(c0 + tid + u * NW * kWave, ncols - 1))];
        }
#pragma unroll
        for (int u = 0; u < kStageUnroll; ++u) {
            const int c = c0 + tid + u * NW * kWave;
            int row = c < ncols && c >= gen_end ? stage_v[u] : -1;
            if (row >= p.kv_rows) { err = 1; row = -1; }
            row = row < 0 ? -1 : row;
            if (c < ncols_pad && c >= gen_end) istage[c] = stage_word<FP8, D>(row);
            if (row >= 0) last = c;
        }
    }
    if (gen_end > 0) {
        // the fused window columns, generated from the position (a short loop of its own, so
        // that the unrolled staging above stays as compact as without them)
        const WindowList win_list(p, pos);
#pragma unroll 1
        for (int c = tid; c < gen_end; c += NW * kWave) {
            int row = win_list(col_begin + c);
            if (row >= p.kv_rows) { err = 1; row = -1; }
            istage[c] = stage_word<FP8, D>(row);
            if (row >= 0) last = max(last, c);
        }
    }
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, kWave));
    SA_LDS int32_t* lastw = istage + KL::kStageCols;             // one word per wave
    SA_LDS int32_t* redo = lastw + 8;                           // second-pass flag
    if (lane == 0) lastw[wid] = last;
    if (tid == 0) *redo = 0;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) last = max(last, lastw[w]);
    // 0 when nothing is named; the same in every lane, kept in a scalar register
    const int ntiles = __builtin_amdgcn_readfirstlane((last + kTileKeys) / kTileKeys);
    float sink2[HPW];
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) sink2[hb] = sink_raw[hb] * kLog2e;
    // Q and the sink have landed before the first tile load issues: the compiler does not
    // count the tile loads (inline assembly), so its own waits for Q must not meet them.
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    // The position's (cos, sin) row is only needed by the epilogue: its loads go out here,
    // before every tile load, so they never disturb the tile waits (which count only tile
    // loads issued after them), and they land with the first tile at the latest.
    // nullptr: no rotation here (none asked for, or the combine kernel finishes the rows)
    const float* cs_g = p.splits == 1 ? rope_ptr(p, pos, tid == 0) : nullptr;
    constexpr int kCsPer = (D + NW * kWave - 1) / (NW * kWave);
    float cs_v[kCsPer];
    if (cs_g != nullptr) {
#pragma unroll
        for (int u = 0; u < kCsPer; ++u) cs_v[u] = cs_g[min(tid + u * NW * kWave, p.rope_dim - 1)];
    }

    // Softmax reference. Every probability of a pass is exp2(score - m_ref) with one fixed
    // reference per head, so O is never rescaled inside the key loop: m_ref is taken at the
    // first tile that names a row (max of the sink and that tile's scores; O is still zero
    // then), and later scores may exceed it by up to kSlack (probabilities up to 2^kSlack,
    // well inside f32 and bf16 range). A score beyond that flags the workgroup; the whole key
    // loop then runs once more with m_ref = the maximum of every score seen (which no score
    // can exceed), a rare second pass instead of a rescale on every tile.
    constexpr float kSlack = 32.0f;
    const bool sink_lane = q4 == 0 && split == 0 && kg == 0;  // the sink counts once per head
    float m_ref[HPW], m_seen[HPW], l_run[HPW];                 // log2 domain, per head
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
        // finite even for a sink of -inf, so that exp2(score - m_ref) of a skipped key (-inf)
        // is 0 and never NaN before the first tile with a row sets the reference
        m_ref[hb] = fmaxf(sink2[hb], -FLT_MAX);
        m_seen[hb] = -INFINITY;                                // this lane's maximum score
        l_run[hb] = sink_lane ? fast_exp2(sink2[hb] - m_ref[hb]) : 0.0f;
    }
    bool have_ref = false;                                     // same in all lanes of a wave
    bool over = false;                                         // a score passed m_ref + kSlack
    f32x4 o_acc[G::kDBlocks][HPW];
#pragma unroll
    for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) o_acc[b][hb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Per-lane LDS byte offsets of the two operand reads (the swizzle only touches the low
    // four bits of a chunk index, so each read is one of these plus a multiple of 256 B; rows
    // 16 apart share a swizzle, so the second 16-key block is the same plus kHalf):
    //   K operand, block mb, step kk: qk_off[kk % 4] + 256 * (kk / 4) + kHalf * mb
    //   V operand, read ab, d slice db: pv_off[db % 8] + 256 * (db / 8) + kHalf * ab
    constexpr int kHalf = 16 * G::kRowBytes;
    int qk_off[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) qk_off[k] = l16 * G::kRowBytes + 16 * ((4 * k + qc) ^ swz<G::kChunks>(l16));
    int pv_off[8];
    {
        // 16-lane group q4 reads keys 4*q4 + (0..3) (then 16 + ...) of d columns
        // 16*db + (0..15); lane i of the group names row i/4 and columns 4*(i%4)..+3 of that
        // 4 x 16 block and receives column i.
        const int rr = 4 * q4 + (l16 >> 2);
#pragma unroll
        for (int b8 = 0; b8 < 8; ++b8) {
            const int col = 16 * b8 + 4 * (l16 & 3);           // bf16 column within 128
            pv_off[b8] = rr * G::kRowBytes + (col & 7) * 2 + 16 * ((col >> 3) ^ swz<G::kChunks>(rr));
        }
    }

    // ---- the stages of one key tile, shared by the two loop shapes below ----------------
    // QK: S^T = K . Q^T over the tile's two 16-key blocks. K operands are read kPre steps
    // ahead of their multiply; scheduling fences keep the compiler from hoisting every read of
    // the unrolled loop.
    // With two head blocks per wave O takes all 256 AGPRs (that kernel's accumulators live in
    // AGPRs): the score accumulators are then kept in VGPRs by writing the score product in
    // assembly (mfma_v). With one head block every accumulator is a VGPR already.
    constexpr bool kScoresInVgprs = HPW == 2;
    auto qk = [&](SA_LDS const uint8_t* cur, f32x4 (&s_acc)[2][HPW]) {
        constexpr int kPre = G::kKSteps < 3 ? G::kKSteps : 3;
        u32x4 a0[kPre], a1[kPre];
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            a0[k] = *(SA_LDS const u32x4*)(cur + qk_off[k & 3] + 256 * (k >> 2));
            a1[k] = *(SA_LDS const u32x4*)(cur + qk_off[k & 3] + 256 * (k >> 2) + kHalf);
        }
#pragma unroll
        for (int kk = 0; kk < G::kKSteps; ++kk) {
            const u32x4 c0 = a0[kk % kPre], c1 = a1[kk % kPre];
            if (kk + kPre < G::kKSteps) {
                const int nk = kk + kPre;
                a0[kk % kPre] = *(SA_LDS const u32x4*)(cur + qk_off[nk & 3] + 256 * (nk >> 2));
                a1[kk % kPre] = *(SA_LDS const u32x4*)(cur + qk_off[nk & 3] + 256 * (nk >> 2) + kHalf);
            }
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) {
                if constexpr (kScoresInVgprs) {
                    if (kk == 0) {
                        mfma_vz(s_acc[0][hb], c0, qreg[hb][kk]);
                        mfma_vz(s_acc[1][hb], c1, qreg[hb][kk]);
                    } else {
                        mfma_v(s_acc[0][hb], c0, qreg[hb][kk]);
                        mfma_v(s_acc[1][hb], c1, qreg[hb][kk]);
                    }
                } else {
                    // the first step starts from a zero accumulator (an inline constant)
                    const bf16x8 qb = __builtin_bit_cast(bf16x8, qreg[hb][kk]);
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    s_acc[0][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, c0), qb, kk == 0 ? z : s_acc[0][hb], 0, 0, 0);
                    s_acc[1][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, c1), qb, kk == 0 ? z : s_acc[1][hb], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the scores are read by vector instructions next: wait out the matrix pipeline
        if constexpr (kScoresInVgprs) mfma_v_drain(s_acc);
    };

    // Softmax, part 1 (log2 domain; this lane: head l16 of each block, keys 16*mb + 4*q4 + r;
    // a score in log2 units is raw * scale_log2). Skipped keys (rows zeroed in LDS) get a raw
    // score of -inf; a tile whose keys all name a row, the common case, needs no masking.
    // With a positive scale a maximum of scores is the scaled maximum of the raw scores and
    // each probability is exp2(fma(raw, scale, -m_ref)); otherwise the scores are scaled here
    // (skipped keys set to -inf again) and the returned scale is 1. At the first tile that
    // names a row the reference is taken (O is still zero then).
    // (IEEE maximum, v_maximum3_f32: fmaxf in IEEE mode would first canonicalise every score
    // with a max of its own; a NaN score, which only NaN or infinite inputs make, carries over)
    auto lane_max = [&](const f32x4 (&s_acc)[2][HPW], int hb) {
        const auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
        const float t0 = mx(mx(s_acc[0][hb][0], s_acc[0][hb][1]), mx(s_acc[0][hb][2], s_acc[0][hb][3]));
        const float t1 = mx(mx(s_acc[1][hb][0], s_acc[1][hb][1]), mx(s_acc[1][hb][2], s_acc[1][hb][3]));
        return mx(t0, t1);
    };
    auto prepare = [&](f32x4 (&s_acc)[2][HPW], uint32_t valid) {
        if (valid != 0xffffffffu) {
            const uint32_t lm = valid >> (4 * q4);     // bits r and 16 + r: this lane's keys
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = (lm >> (16 * mb + r)) & 1u;
#pragma unroll
                    for (int hb = 0; hb < HPW; ++hb) s_acc[mb][hb][r] = keep ? s_acc[mb][hb][r] : -INFINITY;
                }
        }
        float sc = p.scale_log2;
        if (!(sc > 0.0f)) {
            // skipped keys are -inf by now; they stay -inf (tested on the score rather than on
            // the mask bits, which the compiler would otherwise extract for every tile)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int hb = 0; hb < HPW; ++hb)
                        s_acc[mb][hb][r] = s_acc[mb][hb][r] == -INFINITY ? -INFINITY : s_acc[mb][hb][r] * sc;
            sc = 1.0f;
        }
        if (!have_ref && valid != 0) {
            // first tile with a row (valid != 0, so its maximum is finite)
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) {
                m_ref[hb] = fmaxf(sink2[hb], max4groups(lane_max(s_acc, hb) * sc));
                l_run[hb] = sink_lane ? fast_exp2(sink2[hb] - m_ref[hb]) : 0.0f;
            }
            have_ref = true;
        }
        return sc;
    };
    // Softmax, part 2, in kSoftSteps small steps that can be interleaved with matrix work:
    // steps 0 .. 4*HPW-1 turn two scores into probabilities (packed to bf16 as the PV B
    // operand, summed per lane), then one step per head block tracks the lane's maximum
    // score and flags a score more than kSlack above the reference, and the last step adds
    // the sums to the running denominators.
    constexpr int kSoftSteps = 5 * HPW + 1;
    auto soft_step = [&](int k, const f32x4 (&s_acc)[2][HPW], float sc, u32x4 (&pb)[HPW], float (&psum)[HPW]) {
        if (k < 4 * HPW) {
            const int hb = k >> 2, mb = (k >> 1) & 1, h = k & 1;
            const float nm = -m_ref[hb];
            const float p0 = fast_exp2(fmaf(s_acc[mb][hb][2 * h], sc, nm));
            const float p1 = fast_exp2(fmaf(s_acc[mb][hb][2 * h + 1], sc, nm));
            psum[hb] += p0 + p1;
            pb[hb][2 * mb + h] = pack_bf16x2(p0, p1);
        } else if (k < 5 * HPW) {
            const int hb = k - 4 * HPW;
            const float lm = lane_max(s_acc, hb) * sc;
            m_seen[hb] = __builtin_elementwise_maximum(m_seen[hb], lm);
            over |= lm > m_ref[hb] + kSlack;
        } else if (k == 5 * HPW) {
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) l_run[hb] += psum[hb];
        }
    };
    // PV: O^T += V^T . P^T over the whole 32-key tile, one 16-wide d slice at a time; V
    // operands read kPre slices ahead. hook(j) runs after every second slice (j = db / 2),
    // and the hooks the slices did not reach run at the end.
    auto pv = [&](SA_LDS const uint8_t* cur, const u32x4 (&pb)[HPW], auto hook) {
        constexpr int kPre = 2;
        bf16x4v va[kPre], vb[kPre];
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            va[k] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4v*)(cur + pv_off[k & 7] + 256 * (k >> 3)));
            vb[k] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4v*)(cur + pv_off[k & 7] + 256 * (k >> 3) + kHalf));
        }
#pragma unroll
        for (int db = 0; db < G::kDBlocks; ++db) {
            const bf16x8 a = __builtin_shufflevector(va[db % kPre], vb[db % kPre], 0, 1, 2, 3, 4, 5, 6, 7);
            if (db + kPre < G::kDBlocks) {
                const int nb = db + kPre;
                va[db % kPre] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4v*)(cur + pv_off[nb & 7] + 256 * (nb >> 3)));
                vb[db % kPre] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4v*)(cur + pv_off[nb & 7] + 256 * (nb >> 3) + kHalf));
            }
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb)
                o_acc[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, pb[hb]), o_acc[db][hb], 0, 0, 0);
            if ((db & 1) == 0 && db / 2 < kSoftSteps) hook(db / 2);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = (G::kDBlocks + 1) / 2; j < kSoftSteps; ++j) hook(j);
    };
    // Opaque to the optimiser: addresses derived from the offsets are then formed next to
    // their reads inside the loop instead of being hoisted (and spilled) in bulk.
    auto pin_offsets = [&]() {
#pragma unroll
        for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(qk_off[k]));
#pragma unroll
        for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(pv_off[k]));
    };

    // fp8 storage: the rows' scale bytes
    const i32x4 sc_rsrc = FP8 ? make_buffer_rsrc(sc_seq, (uint32_t)p.kv_rows * (uint32_t)(D / 32)) : kv_rsrc;
    for (int pass = 0;; ++pass) {
    if constexpr (FP8 && !kFp8Pipe) {
        // fp8 storage (d other than 512): one bf16 tile; the codes of the next tile are
        // gathered into a raw staging tile while the current one is converted and multiplied
        if (ntiles > 0) gather_tile_fp8<D, NW>(kv_seq, sc_seq, istage, raw(0), raw_sc(0), wid, lane);
        for (int it = 0; it < ntiles; ++it) {
            SA_LDS const int32_t* tidx = istage + it * kTileKeys;
            // which columns of this tile name a row (one bit per key)
            const uint32_t valid = (uint32_t)__ballot(lane < kTileKeys && staged_row(tidx[lane & 31]));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (it + 1 < ntiles)
                gather_tile_fp8<D, NW>(kv_seq, sc_seq, tidx + kTileKeys, raw((it + 1) & 1), raw_sc((it + 1) & 1), wid, lane);
            convert_tile_fp8<D, NW>(raw(it & 1), raw_sc(it & 1), tile(0), tid);
            __syncthreads();
            if (valid == 0) continue;                          // a tile of skips only
            pin_offsets();
            f32x4 s_acc[2][HPW];
            qk(tile(0), s_acc);
            const float sc = prepare(s_acc, valid);
            u32x4 pb[HPW];
            float psum[HPW];
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) psum[hb] = 0.0f;
#pragma unroll
            for (int k = 0; k < kSoftSteps; ++k) soft_step(k, s_acc, sc, pb, psum);
            __builtin_amdgcn_sched_barrier(0);
            pv(tile(0), pb, [](int) {});
        }
    } else if constexpr (KG > 1 || CMP) {
        // Key groups: the waves of key group g work on tile s*KG + g of super tile s (the
        // compact layout runs this loop with one group: a two-tile ring, the next tile
        // gathered while the current one is worked on).
        //   bf16 storage: the tile ring holds NS super tiles of KG tiles and all waves gather
        //   every tile. With two super tiles in the ring the next one is gathered while the
        //   current one is worked on; with one, after it (a barrier in between).
        //   fp8 storage: the codes and scales of the next super tile are gathered into raw
        //   slots while the current one is worked on; all waves convert a landed super tile
        //   into the bf16 tiles between two barriers.
        constexpr int NS = kFp8Pipe ? 1 : NB / KG;
        static_assert(NS >= 1 && (!kFp8Pipe || KL::kRawSlots >= KG), "tile ring too small for the key groups");
        const int nsuper = (ntiles + KG - 1) / KG;
        auto gather_super = [&](int su) {
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                const int ti = su * KG + g;
                if (ti < ntiles) {
                    if constexpr (kFp8Pipe)
                        RawGather<D, NW>::issue(kv_rsrc, sc_rsrc, istage + ti * kTileKeys, raw(g), wid, lane);
                    else
                        gather_tile_bf16<D, NW>(kv_rsrc, istage + ti * kTileKeys, tile((su % NS) * KG + g), wid, lane);
                }
            }
        };
        if (nsuper > 0) gather_super(0);
        for (int su = 0; su < nsuper; ++su) {
            const int ti = su * KG + kg;
            // the wave's tile's column indices, read before the waits (the valid-key mask is
            // formed after them, so the LDS read's latency hides behind the waits)
            const int tv = ti < ntiles ? istage[ti * kTileKeys + (lane & 31)] : -1;
            vmcnt_wait<0>();
            if constexpr (kFp8Pipe) {
                lds_sync();             // super tile su's codes; every wave done with su-1
#pragma unroll
                for (int g = 0; g < KG; ++g) {
                    const int ti = su * KG + g;
                    if (ti < ntiles) convert_raw_fp8<D, NW>(raw(g), istage + ti * kTileKeys, tile(g), wid, lane);
                }
                lds_sync();             // super tile su converted; its raw slots free
                if (su + 1 < nsuper) gather_super(su + 1);
            } else {
                lds_sync();             // super tile su visible to all
                if (NS > 1 && su + 1 < nsuper) gather_super(su + 1);
            }
            const uint32_t valid = (uint32_t)__ballot(lane < kTileKeys && staged_row(tv));
            if (valid != 0) {
                SA_LDS const uint8_t* cur = tile((su % NS) * KG + kg);
                pin_offsets();
                f32x4 s_acc[2][HPW];
                qk(cur, s_acc);
                const float sc = prepare(s_acc, valid);
                u32x4 pb[HPW];
                float psum[HPW];
#pragma unroll
                for (int hb = 0; hb < HPW; ++hb) psum[hb] = 0.0f;
#pragma unroll
                for (int k = 0; k < kSoftSteps; ++k) soft_step(k, s_acc, sc, pb, psum);
                __builtin_amdgcn_sched_barrier(0);
                pv(cur, pb, [](int) {});
            }
            if (!kFp8Pipe && NS == 1 && su + 1 < nsuper) {
                lds_sync();             // every wave is done with the super tile
                gather_super(su + 1);
            }
        }
    } else {
        // Software-pipelined: iteration `it` scores tile it, then multiplies the probabilities
        // of tile it-1 with its rows while tile it's softmax runs in between the matrix
        // instructions. The only vector-memory operations inside the loop are the tile loads.
        //   bf16 storage: tiles it-1 and it are in use and tiles it+1 and it+2 are in flight
        //   (kBuffers = 4), so tile it has landed once only tile it+1's loads remain.
        //   fp8 storage (d = 512): the codes and scales of tiles it+1 and it+2 sit in raw
        //   slots (it+1 landed, it+2 in flight) and tile it+1 is converted into its bf16
        //   buffer between the two products; tile it+3's loads go out at the top.
        constexpr int kAh = 2;
        static_assert(kFp8Pipe || NB >= kAh + 2, "tile ring too small for the pipeline");
        if constexpr (kFp8Pipe) {
            using RG = RawGather<D, NW>;
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (j < ntiles) RG::issue(kv_rsrc, sc_rsrc, istage + j * kTileKeys, raw(j), wid, lane);
            if (ntiles > 0) {
                if (ntiles >= 3) vmcnt_wait<2 * RG::kLoads>();
                else if (ntiles == 2) vmcnt_wait<RG::kLoads>();
                else vmcnt_wait<0>();
                lds_sync();                 // tile 0's codes from every wave
                convert_raw_fp8<D, NW>(raw(0), istage, tile(0), wid, lane);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kAh; ++j)
                if (j < ntiles) gather_tile_bf16<D, NW>(kv_rsrc, istage + j * kTileKeys, tile(j), wid, lane);
        }
        // One PV instance for every iteration, so that O stays in the same registers
        // throughout: iteration 0 has no previous tile (its softmax runs on its own), and the
        // extra last iteration scores nothing (all its keys are masked, p = 0) while it
        // multiplies the last tile.
        u32x4 pb_prev[HPW];
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) pb_prev[hb] = u32x4{0, 0, 0, 0};
        SA_LDS const uint8_t* prev = tiles;
        for (int it = 0; it <= ntiles; ++it) {
            SA_LDS uint8_t* cur = tile(it % NB);
            uint32_t valid = 0;
            f32x4 s_acc[2][HPW];
            if (it < ntiles) {
                SA_LDS const int32_t* tidx = istage + it * kTileKeys;
                // this tile's column indices are read before the waits and turned into the
                // valid-key mask after them, so the LDS read's latency hides behind the waits
                const int tv = tidx[lane & 31];
                if constexpr (kFp8Pipe) {
                    using RG = RawGather<D, NW>;
                    if (it + 2 < ntiles) vmcnt_wait<RG::kLoads>();
                    else vmcnt_wait<0>();
                    // tile it converted by every wave, tile it+1's codes visible; the slot of
                    // tile it and the buffer of tile it-2 are free
                    lds_sync();
                    if (it + 3 < ntiles)
                        RG::issue(kv_rsrc, sc_rsrc, tidx + 3 * kTileKeys, raw((it + 3) % 3), wid, lane);
                } else {
                    if (it + 1 < ntiles) vmcnt_wait<PP::kLoadsPerWave>();
                    else vmcnt_wait<0>();
                    lds_sync();         // tile it visible to all; buffer of tile it-2 free
                    if (it + kAh < ntiles)
                        gather_tile_bf16<D, NW>(kv_rsrc, tidx + kAh * kTileKeys, tile((it + kAh) % NB), wid, lane);
                }
                valid = (uint32_t)__ballot(lane < kTileKeys && staged_row(tv));
                pin_offsets();
                qk(cur, s_acc);
            } else {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int hb = 0; hb < HPW; ++hb) s_acc[mb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            const float sc = prepare(s_acc, valid);
            if constexpr (kFp8Pipe) {
                if (it + 1 < ntiles)
                    convert_raw_fp8<D, NW>(raw((it + 1) % 3), istage + (it + 1) * kTileKeys, tile((it + 1) % NB), wid, lane);
            }
            u32x4 pb[HPW];
            float psum[HPW];
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) psum[hb] = 0.0f;
            auto hook = [&](int k) { soft_step(k, s_acc, sc, pb, psum); };
            if (it > 0) {
                pin_offsets();
                pv(prev, pb_prev, hook);
            } else {
#pragma unroll
                for (int k = 0; k < kSoftSteps; ++k) hook(k);
            }
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) pb_prev[hb] = pb[hb];
            prev = cur;
        }
    }
    if (cs_g != nullptr) {
#pragma unroll
        for (int u = 0; u < kCsPer; ++u)
            if (tid + u * NW * kWave < p.rope_dim) cs_lds[tid + u * NW * kWave] = cs_v[u];
    }
    // A score ran more than kSlack above its head's reference (rare): run the key loop again
    // against the maximum of all scores, which every wave has tracked for its heads.
    if (__ballot(over) != 0 && lane == 0) *redo = 1;
    __syncthreads();
    const int again = *redo;
    if (pass > 0 || again == 0) break;
    __syncthreads();                                           // every wave has read the flag
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
        // finite also for a key group that saw no row while another one flagged the pass
        m_ref[hb] = fmaxf(fmaxf(sink2[hb], max4groups(m_seen[hb])), -FLT_MAX);
        l_run[hb] = sink_lane ? fast_exp2(sink2[hb] - m_ref[hb]) : 0.0f;
    }
    have_ref = true;
    over = false;
#pragma unroll
    for (int b = 0; b < G::kDBlocks; ++b)
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) o_acc[b][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // a skipped index >= kv_rows is reported once per wave
    if ((p.flags & 1u) && __ballot(err) != 0 && lane == 0) atomicOr(p.err_word, 1);

    // ---- finish: the four lane groups share m_ref; their partial sums add up
    float l_tot[HPW];
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) l_tot[hb] = sum4groups(l_run[hb]);
    // With two key groups each group finishes one half of d (group g: d0 = g * D/2) and all
    // waves share the epilogue; otherwise a wave finishes all of d.
    constexpr bool kHalves = KG == 2;
    constexpr int kEpiD = kHalves ? D / 2 : D;                  // elements of d this wave finishes
    constexpr int kEpiBlocks = kEpiD / 16;
    const int d0 = kHalves ? kg * kEpiD : 0;
    if constexpr (kHalves) {
        // Each wave leaves the half of O it does not finish, with its (m, l), in LDS behind
        // the staging area of the epilogue (the tile buffers are free: a barrier ended the key
        // loop), and adds the other group's part of its own half: m = max(m_0, m_1),
        // O = O_0 2^(m_0 - m) + O_1 2^(m_1 - m), l likewise. Its finished half then sits in
        // o_acc[0 .. kEpiBlocks-1] (group 1 moves its upper half down) for the epilogue.
        constexpr int kSlotO = HPW * kEpiBlocks * kWave * 16;
        constexpr int kSlot = kSlotO + HPW * kWave * 8;
        SA_LDS uint8_t* mrg = tiles + NW * kHeadsPerWave * (2 * kEpiD + 16);
        SA_LDS uint8_t* mine = mrg + wid * kSlot;
        SA_LDS const uint8_t* other = mrg + ((1 - kg) * HB + hbw) * kSlot;
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
#pragma unroll
            for (int db = 0; db < kEpiBlocks; ++db)
                *(SA_LDS f32x4*)(mine + ((hb * kEpiBlocks + db) * kWave + lane) * 16) =
                    kg == 0 ? o_acc[db + kEpiBlocks][hb] : o_acc[db][hb];
            *(SA_LDS f32x2*)(mine + kSlotO + (hb * kWave + lane) * 8) = f32x2{m_ref[hb], l_tot[hb]};
        }
        __syncthreads();
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
            const f32x2 ml = *(SA_LDS const f32x2*)(other + kSlotO + (hb * kWave + lane) * 8);
            const float m = fmaxf(m_ref[hb], ml[0]);
            const float w0 = m_ref[hb] == -INFINITY ? 0.0f : fast_exp2(m_ref[hb] - m);   // no row and no sink
            const float w1 = ml[0] == -INFINITY ? 0.0f : fast_exp2(ml[0] - m);
#pragma unroll
            for (int db = 0; db < kEpiBlocks; ++db) {
                const f32x4 own = kg == 0 ? o_acc[db][hb] : o_acc[db + kEpiBlocks][hb];
                o_acc[db][hb] = own * w0 + *(SA_LDS const f32x4*)(other + ((hb * kEpiBlocks + db) * kWave + lane) * 16) * w1;
            }
            m_ref[hb] = m;
            l_tot[hb] = l_tot[hb] * w0 + ml[1] * w1;
        }
    } else if constexpr (KG > 1) {
        // Merge the key groups into group 0: m = max m_g, O = sum O_g 2^(m_g - m),
        // l = sum l_g 2^(m_g - m). Groups 1.. leave O (accumulator layout, 16 bytes per lane
        // and slice) and (m, l) in LDS behind the epilogue's output staging area; the tile
        // buffers are free (a barrier ended the key loop).
        constexpr int kSlotO = HPW * G::kDBlocks * kWave * 16;
        constexpr int kSlot = kSlotO + HPW * kWave * 8;
        SA_LDS uint8_t* mrg = tiles + HB * kHeadsPerWave * (2 * D + 16);
        if (kg > 0) {
            SA_LDS uint8_t* slot = mrg + ((kg - 1) * HB + hbw) * kSlot;
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) {
#pragma unroll
                for (int db = 0; db < G::kDBlocks; ++db)
                    *(SA_LDS f32x4*)(slot + ((hb * G::kDBlocks + db) * kWave + lane) * 16) = o_acc[db][hb];
                *(SA_LDS f32x2*)(slot + kSlotO + (hb * kWave + lane) * 8) = f32x2{m_ref[hb], l_tot[hb]};
            }
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
            float mg[KG], lg[KG];
            mg[0] = m_ref[hb];
            lg[0] = l_tot[hb];
#pragma unroll
            for (int g = 1; g < KG; ++g) {
                const f32x2 ml = *(SA_LDS const f32x2*)(mrg + ((g - 1) * HB + hbw) * kSlot + kSlotO + (hb * kWave + lane) * 8);
                mg[g] = ml[0];
                lg[g] = ml[1];
            }
            float m = mg[0];
#pragma unroll
            for (int g = 1; g < KG; ++g) m = fmaxf(m, mg[g]);
            float wg[KG], l = 0.0f;
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                wg[g] = mg[g] == -INFINITY ? 0.0f : fast_exp2(mg[g] - m);   // no row and no sink
                l += lg[g] * wg[g];
            }
#pragma unroll
            for (int db = 0; db < G::kDBlocks; ++db) {
                f32x4 o = o_acc[db][hb] * wg[0];
#pragma unroll
                for (int g = 1; g < KG; ++g)
                    o += *(SA_LDS const f32x4*)(mrg + ((g - 1) * HB + hbw) * kSlot + ((hb * G::kDBlocks + db) * kWave + lane) * 16) * wg[g];
                o_acc[db][hb] = o;
            }
            m_ref[hb] = m;
            l_tot[hb] = l;
        }
    }
    // O^T accumulator layout: lane holds head head_of(hb), d = 16*db + 4*q4 + (0..3)
    if (p.splits == 1) {
        // The rows go out through LDS: each lane's 4-element pieces (which lie 16 heads x 4
        // lane groups apart) are written to a per-wave staging block of 16 head rows, read back
        // a whole row per instruction and stored to HBM as full, contiguous rows. The tile
        // buffers are free once the key loop is done (a barrier ends it). Rows carry 16 bytes
        // of padding so that the 8-byte writes, the 16-byte reads and the rotation's 4-byte
        // accesses are free of bank conflicts. The position's (cos, sin) row was staged in LDS
        // at start-up.
        // This code runs once per workgroup, so its instructions are fetched cold: it is kept
        // short and nearly free of branches (the rotation is a small loop over the staged rows
        // rather than a test in every slice of d, and the stores take one uniform branch).
        constexpr int kOutStride = 2 * kEpiD + 16;                  // bytes per staged row
        constexpr int kLanesPerRow = 2 * kEpiD / 16;                // 16-byte pieces per row
        constexpr int kRowsPerRead = kWave / kLanesPerRow;
        constexpr int kReads = kHeadsPerWave / kRowsPerRead;
        SA_LDS uint8_t* ob = tiles + wid * (kHeadsPerWave * kOutStride);
        const int r0 = D - p.rope_dim;
        const int wave_head0 = head0 - l16;                         // first head of block 0
        const int prow = lane / kLanesPerRow, pcol = lane % kLanesPerRow;
        uint16_t* out_q = p.out + (int64_t)seq * p.out_seq_stride + (int64_t)t * p.h * D + d0;
        // inverse RoPE (apply_rotary_emb with inverse=True: the bf16 pair times the conjugate
        // of (cos, sin) in f32, back to bf16). With one head block per wave and rope_dim = 64
        // the rotated elements are the last four slices of d, rotated in registers before
        // staging (by (1, 0), which returns the pair unchanged, when no rotation applies);
        // otherwise they are rotated in the staged rows: lane takes row lane / 4 and its pairs
        // lane % 4, +4, ... (with two head blocks per wave the in-register form measured 1%
        // slower over the whole kernel, the loop 5% faster per workgroup on one block).
        // (Rotated pairs in this wave's part of d, d0 .. d0+kEpiD-1: the in-register form needs
        // the tail of d; the staged form takes pairs rot_lo .. rot_hi-1 of the rotated part.)
        constexpr int kTail = HPW == 1 ? kEpiBlocks - 4 : kEpiBlocks;     // first slice of the tail
        const bool rot_tail = HPW == 1 && cs_g != nullptr && p.rope_dim == 64 && d0 + kEpiD == D;
        SA_LDS uint8_t* rot_row = ob + (lane >> 2) * kOutStride + 2 * (r0 - d0);
        const int rot_lo = max(0, (d0 - r0) / 2);
        const int rot_hi = cs_g != nullptr && !rot_tail ? min(p.rope_dim / 2, (d0 + kEpiD - r0) / 2) : 0;
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
            const float inv_l = l_tot[hb] > 0.0f ? 1.0f / l_tot[hb] : 0.0f;
#pragma unroll
            for (int db = 0; db < kEpiBlocks; ++db) {
                const f32x4 o = o_acc[db][hb] * inv_l;
                uint32_t w[2] = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                if (db >= kTail) {
                    // this lane's pairs are pairs 8 * (db - kTail) + 2 * q4 and the next one
                    const f32x4 cs = *(SA_LDS const f32x4*)(cs_lds + 16 * (db - kTail) + 4 * q4);
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const float c = rot_tail ? cs[2 * k] : 1.0f, sn = rot_tail ? cs[2 * k + 1] : 0.0f;
                        const float x = bf16_lo(w[k]), y = bf16_hi(w[k]);
                        w[k] = pack_bf16x2(x * c + y * sn, y * c - x * sn);
                    }
                }
                *(SA_LDS u32x2*)(ob + l16 * kOutStride + 2 * (16 * db + 4 * q4)) = u32x2{w[0], w[1]};
            }
            // the wave's own LDS accesses complete in order: no barrier between the phases
            for (int i = rot_lo + (lane & 3); i < rot_hi; i += 4) {
                SA_LDS uint32_t* e = (SA_LDS uint32_t*)(rot_row + 4 * i);
                const f32x2 cs = *(SA_LDS const f32x2*)(cs_lds + 2 * i);
                const uint32_t w = *e;
                const float x = bf16_lo(w), y = bf16_hi(w);
                *e = pack_bf16x2(x * cs[0] + y * cs[1], y * cs[0] - x * cs[1]);
            }
            u32x4 v[kReads];
#pragma unroll
            for (int j = 0; j < kReads; ++j)
                v[j] = *(SA_LDS const u32x4*)(ob + (j * kRowsPerRead + prow) * kOutStride + 16 * pcol);
            // the rows are written once and not read again here: non-temporal stores keep
            // them from displacing the gathered kv rows in L2 (measured 0.5% on the long
            // prefill)
            const int hrow0 = wave_head0 + hb * kHeadsPerWave;
            uint16_t* orow = out_q + (int64_t)(hrow0 + prow) * D + 8 * pcol;
            if (hrow0 + kHeadsPerWave <= p.h) {
#pragma unroll
                for (int j = 0; j < kReads; ++j) __builtin_nontemporal_store(v[j], (u32x4*)(orow + (int64_t)j * kRowsPerRead * D));
            } else {
#pragma unroll
                for (int j = 0; j < kReads; ++j)
                    if (hrow0 + j * kRowsPerRead + prow < p.h) __builtin_nontemporal_store(v[j], (u32x4*)(orow + (int64_t)j * kRowsPerRead * D));
            }
        }
    } else {
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
            if (head_of(hb) >= p.h) continue;
            const int64_t slot = ((int64_t)qi * p.splits + split) * p.h_pad + head_of(hb);
            float* wo = p.ws_o + slot * D + d0;
#pragma unroll
            for (int db = 0; db < kEpiBlocks; ++db) *(f32x4*)(wo + 16 * db + 4 * q4) = o_acc[db][hb];
            if (q4 == 0 && d0 == 0) {
                p.ws_ml[slot * 2 + 0] = m_ref[hb];
                p.ws_ml[slot * 2 + 1] = l_tot[hb];
            }
        }
    }
}

template <int D, bool FP8, int NW, int HPW = 1, int KG = 1, bool CMP = false>
inline hipError_t launch_fwd(const KParams& p, int blocks, hipStream_t st) {
    using G = Geo<D>;
    using KL = KernelLds<D, FP8, NW, CMP>;
    // after the tile buffers (and the fp8 raw slots) the region must also hold the
    // epilogue's 16 padded output rows per wave
    constexpr size_t kTiles = KL::kTiles;
    constexpr size_t kOut = (size_t)NW * kHeadsPerWave * (2 * D + 16);
    constexpr size_t lds = (size_t)KL::kStageCols * 4 + 64 + (size_t)D * 4 + (kTiles > kOut ? kTiles : kOut);
    static_assert(lds <= 160 * 1024, "LDS plan exceeds 160 KB");
    // the key-group merge slots sit behind the output staging area
    static_assert(KG != 2 || (size_t)NW * kHeadsPerWave * (D + 16) +
                                 (size_t)NW * (HPW * (G::kDBlocks / 2) * kWave * 16 + HPW * kWave * 8) <= kTiles,
                  "key-group merge does not fit the tile region");
    static_assert(KG <= 2 || (size_t)(NW / KG) * kHeadsPerWave * (2 * D + 16) +
                                 (size_t)(KG - 1) * (NW / KG) * (HPW * G::kDBlocks * kWave * 16 + HPW * kWave * 8) <= kTiles,
                  "key-group merge does not fit the tile region");
    auto k = attn_fwd_kernel<D, FP8, NW, HPW, KG, CMP>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(NW * kWave), lds, st, p);
    return hipGetLastError();
}

}  // namespace sa
