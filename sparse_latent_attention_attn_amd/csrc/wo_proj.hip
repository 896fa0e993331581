// The grouped output projection after sparse_attn (attention output page, Attention.forward:
// wo_a is block-diagonal over the groups, "bsgd,grd->bsgr"): for every token t and group gg,
// out[t][gg][n] = sum_k o[t][gg][k] * W[gg][n][k], f32 accumulation, bf16 result (the attention
// API docs' precision paragraph: a bf16 GEMM). W is bf16, or e4m3 codes with block-32 e8m0
// scales along k whose products are exact bf16 values (the page's note: an fp8 grouped GEMM
// halves the memory), dequantised on the way to the matrix cores.
//
// The kernels compute the transposed product C^T[n][t] = W . O^T on v_mfma_f32_16x16x32_bf16
// (A = rows of W, B = token rows of O), so each lane ends with 4 consecutive outputs of one
// token and stores them as 8 bytes.
//   * proj_wide_kernel (many tokens, bf16 weights): 256 rows of W x 256 tokens per workgroup
//     of 8 waves (two per SIMD), k steps of 64 copied into LDS by direct-to-LDS loads of whole
//     rows, double-buffered.
//   * proj_tiled_kernel (many tokens, fp8 weights or other shapes): 128 rows of W x 256
//     tokens per workgroup, k steps of 64 staged in LDS through registers (double-buffered,
//     16-byte chunks XOR-swizzled by row), 4 waves of 64 x 128.
//   * proj_stream_kernel (decode, at most 64 tokens, r a multiple of 32, kg of 256): the cost
//     is streaming W once; 32 rows of W per workgroup, weights and tokens copied into LDS by
//     direct-to-LDS loads of whole rows, the 4 waves split k and LDS sums the parts.
//   * proj_skinny_kernel (the other decode shapes): the same split with operands loaded
//     straight into registers.
#include "lds_dma.hpp"
#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

// 8 weights of row n (bf16 view) at k .. k+7 as a bf16 MFMA operand.
template <bool FP8>
__device__ __forceinline__ u32x4 load_w8(const ProjParams& p, int64_t row_elem, int k) {
    if constexpr (!FP8) {
        return *(const u32x4*)(p.w + row_elem + k);
    } else {
        const u32x2 c = *(const u32x2*)(p.wq + row_elem + k);
        const float sc = bits_f32((uint32_t)p.ws[(row_elem + k) / 32] << 23);   // 2^(e - 127)
        u32x4 o;
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, false));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, true));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, false));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, true));
        return o;
    }
}

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ skinny (decode)
// Grid (r / (16 NB)) * g workgroups of KW waves; wave w takes k in
// [w kg/KW, (w+1) kg/KW) for NB blocks of 16 rows of W and MB blocks of 16 tokens, and LDS
// sums the KW parts. Each token operand loaded feeds NB matrix instructions (every load
// passes the texture unit at about 64 bytes per clock per CU, and the tokens are re-read
// by every workgroup of their group), and the k range of a wave is short (4 rounds of 4
// k-steps at kg = 8192): the loop is a chain of memory round trips, so more waves with
// shorter chains keep more bytes in flight.
template <bool FP8, int MB, int NB, int KW>
__global__ __launch_bounds__(KW * 64) void proj_skinny_kernel(const ProjParams p) {
    __shared__ f32x4 part[KW - 1][NB][MB][64];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int l16 = lane & 15, gq = lane >> 4;
    // 1-D grid, group fastest: workgroups are dealt to the 8 XCDs round-robin, so with 8
    // groups each XCD takes one group and its L2 keeps that group's tokens, which every
    // workgroup of the group reads in full
    const int gg = blockIdx.x % p.g, n0 = (blockIdx.x / p.g) * 16 * NB, m0 = blockIdx.y * 16 * MB;
    const int kq = p.kg / KW, kbeg = wid * kq;
    int64_t wrow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wrow[nb] = ((int64_t)gg * p.r + n0 + 16 * nb + l16) * p.kg;
    const uint16_t* orow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        orow[mb] = p.o + (int64_t)min(m0 + 16 * mb + l16, p.m - 1) * p.o_stride + (int64_t)gg * p.kg + 8 * gq;
    f32x4 acc[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kbeg; k0 < kbeg + kq; k0 += 128) {           // kq is a multiple of 128
        // fp8: the scale bytes of the round's four 32-blocks, one word per row
        uint32_t sc4[NB];
        if constexpr (FP8) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sc4[nb] = *(const uint32_t*)(p.ws + (wrow[nb] + k0) / 32);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = k0 + 32 * u;
            u32x4 a[NB], b[MB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if constexpr (FP8) {
                    const u32x2 c = *(const u32x2*)(p.wq + wrow[nb] + k + 8 * gq);
                    const float sc = bits_f32(((sc4[nb] >> (8 * u)) & 0xffu) << 23);
                    a[nb][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, false));
                    a[nb][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, true));
                    a[nb][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, false));
                    a[nb][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, true));
                } else {
                    a[nb] = load_w8<false>(p, wrow[nb], k + 8 * gq);
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) b[mb] = *(const u32x4*)(orow[mb] + k);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma16(a[nb], b[mb], acc[nb][mb]);
        }
    }
    if (wid > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) part[wid - 1][nb][mb][lane] = acc[nb][mb];
    }
    __syncthreads();
    if (wid > 0) return;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x4 v = acc[nb][mb];
#pragma unroll
            for (int w = 0; w < KW - 1; ++w) v += part[w][nb][mb][lane];
            const int t = m0 + 16 * mb + l16;
            if (t < p.m)
                *(u32x2*)(p.out + (int64_t)t * p.out_stride + (int64_t)gg * p.r + n0 + 16 * nb + 4 * gq) =
                    u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
}

template <bool FP8, int NB, int KW>
static void launch_skinny_mb(const ProjParams& p, hipStream_t st) {
    const dim3 grid((p.r / (16 * NB)) * p.g, 1, 1), block(KW * 64);
    if (p.m <= 16) hipLaunchKernelGGL((proj_skinny_kernel<FP8, 1, NB, KW>), grid, block, 0, st, p);
    else if (p.m <= 32) hipLaunchKernelGGL((proj_skinny_kernel<FP8, 2, NB, KW>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((proj_skinny_kernel<FP8, 4, NB, KW>), grid, block, 0, st, p);
}

// k split over KW waves: as many as keep a wave's range at 512 or more (a multiple of 128)
template <bool FP8, int NB>
static void launch_skinny_nb(const ProjParams& p, hipStream_t st) {
    if (p.kg % (16 * 512) == 0) launch_skinny_mb<FP8, NB, 16>(p, st);
    else if (p.kg % (8 * 512) == 0) launch_skinny_mb<FP8, NB, 8>(p, st);
    else launch_skinny_mb<FP8, NB, 4>(p, st);
}

// ------------------------------------------------------------------ stream (decode)
// The decode shape streams W once from HBM and re-reads the group's tokens from L2 in every
// workgroup. Loads shaped like MFMA operands touch 16 rows x 64 bytes per instruction, which
// the vector L1 serves at a fraction of its line rate (the operand-load kernel above takes
// 54 us on 64 tokens x 8 groups x 1024 x 8192); here every load instruction instead copies
// whole 16-byte pieces of 2 (bf16) or 4 (fp8) consecutive rows straight into LDS, and the
// operands are read from there (35 us). A workgroup of 4 waves takes 32 rows of W of one
// group (1-D grid, group fastest, so each XCD keeps one group's tokens in L2) and walks k in
// chunks of 256, three chunks in LDS, loads two chunks ahead of the one multiplied; the
// waves split each chunk's 8 k-steps and LDS sums their parts at the end. What bounds it
// now is L2 traffic: every workgroup reads its group's 1 MB of tokens (with the weights
// too served from L2 the kernel still takes 23 us); deeper rings, 8 waves and L2 touches of
// later weight chunks were no faster.

constexpr int kStreamRows = 32, kStreamK = 256, kStreamStages = 3, kStreamWaves = 4;
constexpr int kStreamAhead = kStreamStages - 1;                 // chunks in flight ahead
constexpr int kStreamSteps = kStreamK / 32 / kStreamWaves;      // k-steps per wave and chunk
static_assert(kStreamSteps >= 1 && kStreamK % (32 * kStreamWaves) == 0, "chunk split");

template <bool FP8, int MB>
struct StreamGeo {
    static constexpr int kWRowBytes = FP8 ? kStreamK : 2 * kStreamK;    // one weight row of a chunk
    static constexpr int kWPieces = kWRowBytes / 16;
    static constexpr int kWBytes = kStreamRows * kWRowBytes;
    static constexpr int kScRow = kStreamK / 32;                         // scale bytes per row and chunk
    static constexpr int kScBytes = FP8 ? kStreamWaves * 256 : 0;       // one 256-byte landing area per wave
    static constexpr int kTRowBytes = 2 * kStreamK;
    static constexpr int kTPieces = kTRowBytes / 16;
    static constexpr int kTBytes = MB * 16 * kTRowBytes;
    static constexpr int kStage = kWBytes + kScBytes + kTBytes;
    static constexpr int kWLoads = kWBytes / 1024 / kStreamWaves;       // per wave and chunk
    static constexpr int kTLoads = kTBytes / 1024 / kStreamWaves;
    static constexpr int kLoads = kWLoads + (FP8 ? 1 : 0) + kTLoads;
    static constexpr int kPartBytes = kStreamWaves * 2 * MB * 64 * 16;
    static constexpr size_t kLds = (size_t)kStreamStages * kStage > (size_t)kPartBytes
                                       ? (size_t)kStreamStages * kStage : (size_t)kPartBytes;
    static_assert(kWBytes % (1024 * kStreamWaves) == 0 && kTBytes % (1024 * kStreamWaves) == 0, "load split");
    static_assert(kWPieces >= 8 && kWPieces <= 64 && kTPieces >= 16 && kTPieces <= 64, "row pieces");
    static_assert(!FP8 || kScRow % 4 == 0, "scale words");
};

// Position of 16-byte piece c of LDS row r (a row of `pieces` pieces): XOR-ed so that the
// operand reads of 16 consecutive rows fall in distinct banks. Rows of 16 or more pieces
// (256 bytes and up, a multiple of the 64 banks) take (r & 15): a ds_read_b128 lane group
// (rows 0-7 at piece c, rows 8-15 at piece c+1, or the mirror) then reads 16 distinct bank
// groups, and a ds_read_b64 pass (rows 0-15 at the two halves of one piece) 32 distinct bank
// pairs. Rows of 8 pieces (128 bytes, two rows per bank cycle) take (r >> 1) & 7, which keeps
// that pass on 32 distinct bank pairs.
template <int PIECES>
__device__ __forceinline__ int stream_swz(int r) { return PIECES >= 16 ? (r & 15) : ((r >> 1) & 7); }

template <bool FP8, int MB>
__global__ __launch_bounds__(kStreamWaves * 64) void proj_stream_kernel(const ProjParams p) {
    using G = StreamGeo<FP8, MB>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    SA_LDS uint8_t* smem = (SA_LDS uint8_t*)smem_raw;
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, gq = lane >> 4;
    const int gg = blockIdx.x % p.g, n0 = (blockIdx.x / p.g) * kStreamRows;
    const int64_t row0 = (int64_t)gg * p.r + n0;
    // buffer resources over this workgroup's 32 weight rows, their scale bytes, and the
    // group's token columns (the host keeps each under 2^31 bytes)
    const i32x4 w_rsrc = FP8 ? make_buffer_rsrc(p.wq + row0 * p.kg, (uint32_t)(kStreamRows * p.kg))
                             : make_buffer_rsrc(p.w + row0 * p.kg, (uint32_t)(kStreamRows * p.kg * 2));
    const i32x4 s_rsrc = FP8 ? make_buffer_rsrc(p.ws + row0 * (p.kg / 32), (uint32_t)(kStreamRows * (p.kg / 32))) : w_rsrc;
    const i32x4 t_rsrc = make_buffer_rsrc(p.o + (int64_t)gg * p.kg,
                                          (uint32_t)(((int64_t)(p.m - 1) * p.o_stride + p.kg) * 2));
    const int nc = p.kg / kStreamK;

    // per-lane parts of the load addresses that do not depend on the chunk: a load
    // instruction fills 1 KB of LDS with 64 / pieces whole rows of the chunk, lane i filling
    // piece position i % pieces of row i / pieces from the global piece stored there
    int w_off[G::kWLoads], t_off[G::kTLoads];
#pragma unroll
    for (int j = 0; j < G::kWLoads; ++j) {
        const int r = (wid * G::kWLoads + j) * (64 / G::kWPieces) + lane / G::kWPieces;
        w_off[j] = r * p.kg * (FP8 ? 1 : 2) + 16 * ((lane % G::kWPieces) ^ stream_swz<G::kWPieces>(r));
    }
#pragma unroll
    for (int j = 0; j < G::kTLoads; ++j) {
        const int r = (wid * G::kTLoads + j) * (64 / G::kTPieces) + lane / G::kTPieces;
        const int t = min(r, p.m - 1);               // token rows past m repeat the last one
        t_off[j] = (int)((int64_t)t * p.o_stride * 2) + 16 * ((lane % G::kTPieces) ^ stream_swz<G::kTPieces>(r));
    }
    // fp8 scale bytes: the kScRows rows of wave w land in its area as [row][kScRow bytes]
    constexpr int kScWords = G::kScRow / 4, kScRows = kStreamRows / kStreamWaves;
    static_assert(kScRows * kScWords <= 64 && kScRows * G::kScRow <= 256, "scale landing area");
    const int s_off = lane < kScRows * kScWords
                          ? (kScRows * wid + lane / kScWords) * (p.kg / 32) + 4 * (lane % kScWords) : kBufferPastEnd;

    auto issue = [&](int c) {
        SA_LDS uint8_t* st = smem + (c % kStreamStages) * G::kStage;
        const uint32_t base = lds_byte_addr(st);
#pragma unroll
        for (int j = 0; j < G::kWLoads; ++j)
            lds_dma16(w_rsrc, base + (wid * G::kWLoads + j) * 1024, w_off[j] + c * G::kWRowBytes);
        if constexpr (FP8) lds_dma4(s_rsrc, base + G::kWBytes + wid * 256, s_off == kBufferPastEnd ? s_off : s_off + c * G::kScRow);
#pragma unroll
        for (int j = 0; j < G::kTLoads; ++j)
            lds_dma16(t_rsrc, base + G::kWBytes + G::kScBytes + (wid * G::kTLoads + j) * 1024, t_off[j] + c * G::kTRowBytes);
    };

    f32x4 acc[2][MB];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < kStreamAhead && c < nc; ++c) issue(c);
    for (int c = 0; c < nc; ++c) {
        // chunks c .. c + ahead - 1 are in flight: wait until only the later ones are
        vmcnt_wait_groups<G::kLoads, kStreamAhead - 1>(min(kStreamAhead - 1, nc - 1 - c));
        lds_sync();                                  // chunk c has landed for every wave
        if (c + kStreamAhead < nc) issue(c + kStreamAhead);    // into the stage chunk c-1 used
        SA_LDS const uint8_t* st = smem + (c % kStreamStages) * G::kStage;
        SA_LDS const uint8_t* wt = st;
        SA_LDS const uint8_t* tt = st + G::kWBytes + G::kScBytes;
#pragma unroll
        for (int u = 0; u < kStreamSteps; ++u) {
            const int s = kStreamSteps * wid + u;    // this wave's k-steps of the chunk
            const int pc = 4 * s + gq;               // 16-byte piece (8 k) of a bf16 row
            u32x4 a[2], b[MB];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int r = 16 * nb + l16;
                if constexpr (FP8) {
                    const u32x2 cw = *(SA_LDS const u32x2*)(wt + r * G::kWRowBytes + 8 * (pc ^ (2 * stream_swz<G::kWPieces>(r))));
                    const uint32_t e = st[G::kWBytes + (r / kScRows) * 256 + (r % kScRows) * G::kScRow + s];
                    const float sc = bits_f32(e << 23);
                    a[nb][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[0], sc, false));
                    a[nb][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[0], sc, true));
                    a[nb][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[1], sc, false));
                    a[nb][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[1], sc, true));
                } else {
                    a[nb] = *(SA_LDS const u32x4*)(wt + r * G::kWRowBytes + 16 * (pc ^ stream_swz<G::kWPieces>(r)));
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int r = 16 * mb + l16;
                b[mb] = *(SA_LDS const u32x4*)(tt + r * G::kTRowBytes + 16 * (pc ^ stream_swz<G::kTPieces>(r)));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma16(a[nb], b[mb], acc[nb][mb]);
        }
    }
    // sum the four waves' parts: every wave stores its accumulators, then wave w adds up
    // and stores the (row block, token block) pairs w, w + 4, ...
    __syncthreads();
    SA_LDS f32x4* part = (SA_LDS f32x4*)smem;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) part[((wid * 2 + nb) * MB + mb) * 64 + lane] = acc[nb][mb];
    __syncthreads();
    for (int q = wid; q < 2 * MB; q += kStreamWaves) {
        const int nb = q / MB, mb = q % MB;
        f32x4 v = part[((0 * 2 + nb) * MB + mb) * 64 + lane];
#pragma unroll
        for (int w = 1; w < kStreamWaves; ++w) v += part[((w * 2 + nb) * MB + mb) * 64 + lane];
        const int t = 16 * mb + l16;
        if (t < p.m)
            *(u32x2*)(p.out + (int64_t)t * p.out_stride + (int64_t)gg * p.r + n0 + 16 * nb + 4 * gq) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
}

template <bool FP8, int MB>
static hipError_t launch_stream_mb(const ProjParams& p, hipStream_t st) {
    using G = StreamGeo<FP8, MB>;
    auto k = proj_stream_kernel<FP8, MB>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::kLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((p.r / kStreamRows) * p.g), dim3(kStreamWaves * 64), G::kLds, st, p);
    return hipGetLastError();
}

// The stream kernel's conditions: at most 64 tokens, whole 32-row blocks and 256-wide k
// chunks, and every buffer it addresses under 2^31 bytes.
static bool stream_fits(const ProjParams& p) {
    const int64_t t_bytes = ((int64_t)(p.m - 1) * p.o_stride + p.kg) * 2;
    return p.m <= 64 && p.r % kStreamRows == 0 && p.kg % kStreamK == 0 && (int64_t)kStreamRows * p.kg * 2 < (1ll << 31) &&
           t_bytes < (1ll << 31) - 64 && (int64_t)(p.r / kStreamRows) * p.g <= 0x7fffffff;
}

// ------------------------------------------------------------------ tiled
constexpr int kProjN = 128, kProjM = 256, kProjK = 64;          // workgroup tile
constexpr int kProjRowBytes = kProjK * 2;                       // one LDS row (8 chunks)
constexpr int kProjStage = (kProjN + kProjM) * kProjRowBytes;    // 48 KB

// LDS byte offset of 16-byte chunk c of row r. A ds_read_b128 serves a wave in lane groups
// that each take 8 rows of the A/B operand at one chunk and 8 other rows at the next; with
// the chunk XOR-ed by (r >> 1) & 7, even and odd rows land in different halves of the 64 banks
// and each half sees 8 distinct chunks, so a group reads 16 distinct bank groups.
__device__ __forceinline__ int proj_lds(int r, int c) { return r * kProjRowBytes + ((c ^ ((r >> 1) & 7)) << 4); }

template <bool FP8>
__global__ __launch_bounds__(256) void proj_tiled_kernel(const ProjParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    SA_LDS uint8_t* smem = (SA_LDS uint8_t*)smem_raw;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, gq = lane >> 4;
    const int wn = wid & 1, wm = wid >> 1;                       // wave: 64 rows of W x 128 tokens
    // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, so the row tiles of
    // one (token tile, group) pair go to the same XCD back to back and read that token tile
    // through one L2 (with the row tile fastest in a 3-D grid they went to 8 XCDs and every
    // token byte came from HBM 8 times); pairs past the last one (padding to a multiple of 8)
    // exit at once.
    const int nt = p.r / kProjN, nm = (p.m + kProjM - 1) / kProjM;
    const int xcd = blockIdx.x % 8, q = blockIdx.x / 8;
    const int pair = (q / nt) * 8 + xcd;
    if (pair >= nm * p.g) return;
    const int n_base = (q % nt) * kProjN, m_base = (pair % nm) * kProjM, gg = pair / nm;
    // staging: thread tid fills chunk tid % 8 of rows tid / 8 + 32 i
    const int sc_ = tid & 7, sr = tid >> 3;
    int64_t wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[i] = ((int64_t)gg * p.r + n_base + sr + 32 * i) * p.kg + 8 * sc_;
    const uint16_t* orow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        orow[i] = p.o + (int64_t)min(m_base + sr + 32 * i, p.m - 1) * p.o_stride + (int64_t)gg * p.kg + 8 * sc_;
    u32x4 sw[4], so[8];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sw[i] = load_w8<FP8>(p, wrow[i], k0);
#pragma unroll
        for (int i = 0; i < 8; ++i) so[i] = *(const u32x4*)(orow[i] + k0);
    };
    auto stage = [&](int buf) {
        SA_LDS uint8_t* wt = smem + buf * kProjStage;
        SA_LDS uint8_t* ot = wt + kProjN * kProjRowBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(SA_LDS u32x4*)(wt + proj_lds(sr + 32 * i, sc_)) = sw[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) *(SA_LDS u32x4*)(ot + proj_lds(sr + 32 * i, sc_)) = so[i];
    };
    f32x4 acc[4][8];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nk = p.kg / kProjK;
    fetch(0);
    stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) fetch((kt + 1) * kProjK);
        SA_LDS const uint8_t* wt = smem + (kt & 1) * kProjStage;
        SA_LDS const uint8_t* ot = wt + kProjN * kProjRowBytes;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            u32x4 a[4], b[8];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                a[nb] = *(SA_LDS const u32x4*)(wt + proj_lds(wn * 64 + nb * 16 + l16, 4 * kk + gq));
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
                b[mb] = *(SA_LDS const u32x4*)(ot + proj_lds(wm * 128 + mb * 16 + l16, 4 * kk + gq));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int mb = 0; mb < 8; ++mb) acc[nb][mb] = mfma16(a[nb], b[mb], acc[nb][mb]);
        }
        if (kt + 1 < nk) stage((kt + 1) & 1);
        __syncthreads();
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int t = m_base + wm * 128 + mb * 16 + l16;
        if (t >= p.m) continue;
        uint16_t* orow_out = p.out + (int64_t)t * p.out_stride + (int64_t)gg * p.r + n_base + wn * 64 + 4 * gq;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            *(u32x2*)(orow_out + nb * 16) = u32x2{pack_bf16x2(acc[nb][mb][0], acc[nb][mb][1]),
                                                  pack_bf16x2(acc[nb][mb][2], acc[nb][mb][3])};
    }
}

// ------------------------------------------------------------------ wide tiles (bf16)
// Many tokens, bf16 weights: 256 rows of W x 256 tokens per workgroup of 8 waves (two per
// SIMD, so one wave's memory stalls are covered by the other's matrix work), each wave 64
// rows x 128 tokens. k advances in steps of kWideK: the step's 512 rows are copied straight
// into LDS by direct-to-LDS loads of whole rows, kWideStages steps in LDS, the next ones
// loading while the current one is multiplied.
constexpr int kWideN = 256, kWideM = 256, kWideK = 64, kWideWaves = 8, kWideStages = 2;
constexpr int kWideRowBytes = kWideK * 2;                            // bytes of one staged row
constexpr int kWidePieces = kWideRowBytes / 16;                      // 16-byte pieces per row
constexpr int kWideRowsPerLoad = 64 / kWidePieces;
constexpr int kWideStage = (kWideN + kWideM) * kWideRowBytes;
constexpr int kWideLoads = (kWideN + kWideM) / kWideRowsPerLoad / kWideWaves;   // per wave and step
static_assert(kWidePieces == 4 || kWidePieces == 8, "rows of 64 or 128 bytes");

// Position of piece c of staged row r: with 8 pieces (128-byte rows, two rows per bank
// cycle) XOR (r >> 1) & 7, with 4 pieces (64-byte rows, four per bank cycle) XOR (r >> 2) & 3;
// either way the 16 rows of an operand read (8 at piece c, 8 at the next) hit 16 distinct
// bank groups.
__device__ __forceinline__ int wide_lds(int r, int c) {
    const int x = kWidePieces == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
    return r * kWideRowBytes + ((c ^ x) << 4);
}

__global__ __launch_bounds__(kWideWaves * 64) void proj_wide_kernel(const ProjParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    SA_LDS uint8_t* smem = (SA_LDS uint8_t*)smem_raw;
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, gq = lane >> 4;
    const int wn = wid & 3, wm = wid >> 2;                       // wave: rows 64 wn.., tokens 128 wm..
    // XCD-aware order, as in proj_tiled_kernel: the row tiles of one (token tile, group) pair
    // go to one XCD back to back
    const int nt = p.r / kWideN, nm = (p.m + kWideM - 1) / kWideM;
    const int xcd = blockIdx.x % 8, q = blockIdx.x / 8;
    const int pair = (q / nt) * 8 + xcd;
    if (pair >= nm * p.g) return;
    const int n_base = (q % nt) * kWideN, m_base = (pair % nm) * kWideM, gg = pair / nm;
    const int m_rows = min(kWideM, p.m - m_base);                // token rows that exist
    const i32x4 w_rsrc = make_buffer_rsrc(p.w + ((int64_t)gg * p.r + n_base) * p.kg, (uint32_t)(kWideN * p.kg * 2));
    const i32x4 t_rsrc = make_buffer_rsrc(p.o + (int64_t)m_base * p.o_stride + (int64_t)gg * p.kg,
                                          (uint32_t)(((int64_t)(m_rows - 1) * p.o_stride + p.kg) * 2));
    // load j of this wave fills the kWideRowsPerLoad rows from R = I * kWideRowsPerLoad on
    // (I = wid * kWideLoads + j; stage rows 0 .. 255 are W, 256 .. 511 tokens): lane fills
    // piece position lane % kWidePieces of row R + lane / kWidePieces from the global piece
    // stored there
    int off[kWideLoads];
#pragma unroll
    for (int j = 0; j < kWideLoads; ++j) {
        const int row = kWideRowsPerLoad * (wid * kWideLoads + j) + lane / kWidePieces;
        const int pos = (wide_lds(row, lane % kWidePieces) - row * kWideRowBytes) >> 4;   // = piece stored there
        off[j] = row < kWideN ? row * p.kg * 2 + 16 * pos
                              : min(row - kWideN, m_rows - 1) * (int)(p.o_stride * 2) + 16 * pos;
    }
    auto issue = [&](int kt) {
        const uint32_t base = lds_byte_addr(smem + (kt % kWideStages) * kWideStage);
#pragma unroll
        for (int j = 0; j < kWideLoads; ++j) {
            const int I = wid * kWideLoads + j;                  // uniform: W or token rows
            lds_dma16(I < kWideN / kWideRowsPerLoad ? w_rsrc : t_rsrc, base + I * 1024, off[j] + kt * kWideRowBytes);
        }
    };
    f32x4 acc[4][8];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nk = p.kg / kWideK;
    for (int kt = 0; kt < kWideStages - 1 && kt < nk; ++kt) issue(kt);
    for (int kt = 0; kt < nk; ++kt) {
        // steps kt .. kt + stages - 2 are in flight: wait until only the later ones are
        vmcnt_wait_groups<kWideLoads, kWideStages - 2>(min(kWideStages - 2, nk - 1 - kt));
        lds_sync();                                  // step kt landed; step kt-1 done by all
        if (kt + kWideStages - 1 < nk) issue(kt + kWideStages - 1);
        SA_LDS const uint8_t* wt = smem + (kt % kWideStages) * kWideStage;
        SA_LDS const uint8_t* ot = wt + kWideN * kWideRowBytes;
        static_assert(kWideK == 64, "two 32-wide half-steps per k step");
        u32x4 a[2][4], b[2][8];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                a[kk][nb] = *(SA_LDS const u32x4*)(wt + wide_lds(wn * 64 + nb * 16 + l16, 4 * kk + gq));
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
                b[kk][mb] = *(SA_LDS const u32x4*)(ot + wide_lds(wm * 128 + mb * 16 + l16, 4 * kk + gq));
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int mb = 0; mb < 8; ++mb) acc[nb][mb] = mfma16(a[kk][nb], b[kk][mb], acc[nb][mb]);
        // Schedule: half-step 0's operand reads, then its products with half-step 1's reads
        // spread among them (two matrix instructions, one read), then the rest; left to
        // itself the compiler issues each read just ahead of its first use and waits on it
        // (0.955 -> 0.930 ms for 8192 tokens; 226 registers, still two waves per SIMD).
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 40, 0);
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int t = m_base + wm * 128 + mb * 16 + l16;
        if (t >= p.m) continue;
        uint16_t* orow_out = p.out + (int64_t)t * p.out_stride + (int64_t)gg * p.r + n_base + wn * 64 + 4 * gq;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            *(u32x2*)(orow_out + nb * 16) = u32x2{pack_bf16x2(acc[nb][mb][0], acc[nb][mb][1]),
                                                  pack_bf16x2(acc[nb][mb][2], acc[nb][mb][3])};
    }
}

// The wide kernel's conditions: bf16 weights, whole 256-row tiles and 64-wide k steps, and
// every buffer it addresses under 2^31 bytes.
static bool wide_fits(const ProjParams& p) {
    return p.w != nullptr && p.r % kWideN == 0 && p.kg % kWideK == 0 && (int64_t)kWideN * p.kg * 2 < (1ll << 31) &&
           ((int64_t)(kWideM - 1) * p.o_stride + p.kg) * 2 < (1ll << 31) - 64;
}

// ------------------------------------------------------------------ launch
template <bool FP8>
static hipError_t launch_proj(const ProjParams& p, hipStream_t st) {
    if (stream_fits(p)) {
        if (p.m <= 16) return launch_stream_mb<FP8, 1>(p, st);
        if (p.m <= 32) return launch_stream_mb<FP8, 2>(p, st);
        return launch_stream_mb<FP8, 4>(p, st);
    }
    if (p.m <= 64 && p.r % 16 == 0 && p.kg % 512 == 0) {
        if (p.r % 32 == 0) launch_skinny_nb<FP8, 2>(p, st);
        else launch_skinny_nb<FP8, 1>(p, st);
        return hipGetLastError();
    }
    if (!FP8 && wide_fits(p)) {
        const int64_t pairs = ((p.m + kWideM - 1) / kWideM) * (int64_t)p.g;
        const int64_t blocks = (pairs + 7) / 8 * 8 * (p.r / kWideN);
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        const size_t lds = kWideStages * (size_t)kWideStage;
        hipError_t e = hipFuncSetAttribute((const void*)proj_wide_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(proj_wide_kernel, dim3((unsigned)blocks), dim3(kWideWaves * 64), lds, st, p);
        return hipGetLastError();
    }
    if (p.r % kProjN != 0 || p.kg % kProjK != 0) return hipErrorInvalidValue;
    const int64_t pairs = ((p.m + kProjM - 1) / kProjM) * (int64_t)p.g;
    const int64_t blocks = (pairs + 7) / 8 * 8 * (p.r / kProjN);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = 2 * (size_t)kProjStage;
    auto k = proj_tiled_kernel<FP8>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), lds, st, p);
    return hipGetLastError();
}

hipError_t launch_grouped_proj(const ProjParams& p, hipStream_t st) {
    return p.w ? launch_proj<false>(p, st) : launch_proj<true>(p, st);
}

}  // namespace sa
