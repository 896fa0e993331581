// The grouped output projection after sparse_attn (attention output page, Attention.forward:
// wo_a is block-diagonal over the groups, "bsgd,grd->bsgr"): for every token t and group gg,
// out[t][gg][n] = sum_k o[t][gg][k] * W[gg][n][k], f32 accumulation, bf16 result (the attention
// API docs' precision paragraph: a bf16 GEMM). W is bf16, or e4m3 codes with block-32 e8m0
// scales along k whose products are exact bf16 values (the page's note: an fp8 grouped GEMM
// halves the memory), dequantised on the way to the matrix cores.
//
// Both kernels compute the transposed product C^T[n][t] = W . O^T on v_mfma_f32_16x16x32_bf16
// (A = rows of W, B = token rows of O), so each lane ends with 4 consecutive outputs of one
// token and stores them as 8 bytes.
//   * proj_tiled_kernel (many tokens): 128 rows of W x 256 tokens per workgroup, k steps of
//     64 staged in LDS (double-buffered, 16-byte chunks XOR-swizzled by row), 4 waves of
//     64 x 128.
//   * proj_skinny_kernel (decode, at most 64 tokens): the cost is streaming W once, so each
//     workgroup takes 32 (or 16) rows of W, its 4 to 16 waves split k, and LDS sums the
//     parts.
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
    const int n_base = blockIdx.x * kProjN, m_base = blockIdx.y * kProjM, gg = blockIdx.z;
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

// ------------------------------------------------------------------ launch
template <bool FP8>
static hipError_t launch_proj(const ProjParams& p, hipStream_t st) {
    if (p.m <= 64 && p.r % 16 == 0 && p.kg % 512 == 0) {
        if (p.r % 32 == 0) launch_skinny_nb<FP8, 2>(p, st);
        else launch_skinny_nb<FP8, 1>(p, st);
        return hipGetLastError();
    }
    if (p.r % kProjN != 0 || p.kg % kProjK != 0) return hipErrorInvalidValue;
    const int64_t gy = (p.m + kProjM - 1) / kProjM;
    if (gy > 65535 || p.g > 65535) return hipErrorInvalidValue;
    const size_t lds = 2 * (size_t)kProjStage;
    auto k = proj_tiled_kernel<FP8>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(p.r / kProjN, (unsigned)gy, p.g), dim3(256), lds, st, p);
    return hipGetLastError();
}

hipError_t launch_grouped_proj(const ProjParams& p, hipStream_t st) {
    return p.w ? launch_proj<false>(p, st) : launch_proj<true>(p, st);
}

}  // namespace sa
