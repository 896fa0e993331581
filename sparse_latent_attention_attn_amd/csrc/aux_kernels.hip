// The two helpers around sparse_attn: the ring-cache window index lists and the block-32
// ue8m0 fp8 quantisation of KV rows.
#include <climits>

#include "sa_device.hpp"
#include "sa_internal.hpp"

namespace sa {

// ------------------------------------------------------------------ window index lists
// Attention API docs, "window_topk_idxs" and the ring-cache paragraph: the slot of token p
// is p mod window; prefill lists a causal window into the chunk itself, decode lists the
// whole ring oldest first, -1 marking a slot that holds nothing. One thread per entry.
__global__ void window_idxs_kernel(int32_t window, int32_t seqlen, int32_t nseq,
                                   const int32_t* __restrict__ start_pos, int32_t* __restrict__ idx,
                                   int64_t seq_stride, int64_t row_stride, int32_t cols) {
    // one thread per list entry: blockIdx.y walks the (sequence, query) rows, x the columns
    const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= cols) return;
    for (int32_t rt = blockIdx.y; rt < nseq * seqlen; rt += gridDim.y) {
        const int32_t t = rt % seqlen;
        const int32_t n = rt / seqlen;
        int32_t v;
        if (start_pos == nullptr) {
            // prefill from position 0: chunk rows lo..t, lo = max(0, t - window + 1)
            const int32_t lo = max(0, t - window + 1);
            v = lo + j <= t ? lo + j : -1;
        } else {
            const int32_t P = start_pos[n];
            if (P < 0) v = -1;
            else if (P >= window - 1) {
                // full ring: the oldest token P - window + 1 sits in slot (P + 1) mod window
                const int32_t s = P % window + 1 + j;
                v = s >= window ? s - window : s;
            } else {
                v = j <= P ? j : -1;                              // ring holds slots 0..P
            }
        }
        idx[(int64_t)n * seq_stride + (int64_t)t * row_stride + j] = v;
    }
}

hipError_t launch_window_idxs(int32_t window, int32_t seqlen, int32_t nseq, const int32_t* start_pos,
                              int32_t* idx, int64_t seq_stride, int64_t row_stride, int32_t cols,
                              hipStream_t st) {
    if ((int64_t)nseq * seqlen > INT32_MAX) return hipErrorInvalidValue;
    const int threads = cols >= 256 ? 256 : ((cols + 63) / 64) * 64;
    const int gx = (cols + threads - 1) / threads;
    const int64_t rows = (int64_t)nseq * seqlen;
    const int gy = (int)(rows < 65535 ? rows : 65535);
    hipLaunchKernelGGL(window_idxs_kernel, dim3(gx, gy), dim3(threads), 0, st, window, seqlen, nseq,
                       start_pos, idx, seq_stride, row_stride, cols);
    return hipGetLastError();
}

// ------------------------------------------------------------------ block-32 fp8 quant
// Attention API docs, "act_quant_inplace", "FP8_BLOCK", "pow2_ceil": per 32 consecutive
// elements, s = pow2_ceil(max(amax, 1e-4) / 448); codes = e4m3fn(x / s), round to nearest
// even after clamping to +-448; the round trip codes * s is exact in bf16.

// 2^ceil(log2 v) for a positive normal f32, from its fields: exponent + (mantissa != 0).
__device__ __forceinline__ float pow2_ceil_f32(float v) {
    const uint32_t u = f32_bits(v);
    const uint32_t e = ((u >> 23) & 0xffu) + ((u & 0x7fffffu) != 0u ? 1u : 0u);
    return bits_f32(e << 23);
}

// e4m3fn codes of eight values |y| <= 448 into two words (code k in byte k % 4 of word k / 4):
// v_cvt_pk_fp8_f32 rounds to nearest even, with the format's subnormals (step 2^-9), and
// saturates at 448; its codes equal the exact encode on every bf16 value of magnitude up to
// 448 (checked exhaustively), and the values here are bf16 values times a power of two.
__device__ __forceinline__ u32x2 e4m3_pack8(const float (&y)[8]) {
    u32x2 w;
    w[0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w[0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)w[0], true);
    w[1] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    w[1] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)w[1], true);
    return w;
}

// The bf16 round trip code * s of eight packed codes, s a power of two: exact (at most 4
// significant bits), and a product past the bf16 range is inf, as the f32 product is.
__device__ __forceinline__ u32x4 e4m3_roundtrip8(u32x2 w, float s) {
    u32x4 o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], s, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], s, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], s, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], s, true));
    return o;
}

// One block of 32 elements per 4 lanes (8 elements = 16 bytes each); 16 blocks per wave.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ kv, int64_t nblocks,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                        uint16_t* rt) {
    const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = gtid >> 2;
    const int part = (int)(gtid & 3);
    const bool live = blk < nblocks;
    u32x4 v = live ? *(const u32x4*)(kv + blk * 32 + part * 8) : u32x4{0, 0, 0, 0};
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) { x[2 * k] = bf16_lo(v[k]); x[2 * k + 1] = bf16_hi(v[k]); }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    amax = fmaxf(amax, 1e-4f);
    const float s = pow2_ceil_f32(amax / 448.0f);
    if (!live) return;
    // x / s: s is a power of two whose reciprocal is a normal f32 (2^-120 .. 2^22), so the
    // product with the exact reciprocal rounds exactly as the division would
    const float inv_s = 1.0f / s;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = x[k] * inv_s;
    const u32x2 w = e4m3_pack8(y);
    if (codes) *(u32x2*)(codes + blk * 32 + part * 8) = w;
    if (scales && part == 0) scales[blk] = (uint8_t)((f32_bits(s) >> 23) & 0xffu);
    if (rt) *(u32x4*)(rt + blk * 32 + part * 8) = e4m3_roundtrip8(w, s);
}

hipError_t launch_quant_fp8(const uint16_t* kv, int64_t rows, int32_t d, uint8_t* codes,
                            uint8_t* scales, uint16_t* rt, hipStream_t st) {
    const int64_t nblocks = rows * (d / 32);
    const int64_t threads = nblocks * 4;
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_fp8_kernel, dim3((unsigned)grid), dim3(256), 0, st, kv, nblocks, codes, scales, rt);
    return hipGetLastError();
}

// ------------------------------------------------------------------ rotary table
// precompute_freqs_cis (attention output page; the attention API docs, "freqs_cis"): pair
// i of the rope tail turns at f_i = 1 / base^(2i/rope_dim) per position, optionally with the
// YaRN blend towards f_i / factor between pairs low and high (band limits from the host);
// entry (p, i) = (cos, sin) of the f32 angle p * f_i. Every step is rounded to f32 as the
// page's torch code does, with no contraction into fused multiply-adds; base^e is evaluated
// in f64 and rounded (the correctly rounded f32 power), cos and sin in f64 and rounded.
__global__ __launch_bounds__(256) void rope_table_kernel(int32_t rope_dim, int32_t max_pos, float base, int32_t yarn,
                                                         int32_t low, int32_t high, float factor,
                                                         float* __restrict__ cs) {
#pragma clang fp contract(off)
    const int32_t half = rope_dim / 2;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)max_pos * half) return;
    const int32_t i = (int32_t)(e % half);
    const int32_t pos = (int32_t)(e / half);
    const float expo = (float)(2 * i) / (float)rope_dim;
    const float pw = (float)pow((double)base, (double)expo);
    float f = 1.0f / pw;
    if (yarn) {
        const float span = high - low > 0 ? (float)(high - low) : 1e-3f;
        const float ramp = fminf(fmaxf(((float)i - (float)low) / span, 0.0f), 1.0f);
        const float smooth = 1.0f - ramp;
        const float scaled = f / factor * (1.0f - smooth);
        const float kept = f * smooth;
        f = scaled + kept;
    }
    const float ang = (float)pos * f;
    cs[2 * e + 0] = (float)cos((double)ang);
    cs[2 * e + 1] = (float)sin((double)ang);
}

hipError_t launch_rope_table(int32_t rope_dim, int32_t max_pos, float base, int32_t yarn, int32_t low,
                             int32_t high, float factor, float* cs, hipStream_t st) {
    const int64_t n = (int64_t)max_pos * (rope_dim / 2);
    const int64_t grid = (n + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)grid), dim3(256), 0, st, rope_dim, max_pos, base, yarn,
                       low, high, factor, cs);
    return hipGetLastError();
}

// ------------------------------------------------------------------ KV write path
// The step before sparse_attn on the same cache (attention API docs: module notes and the
// ring-cache paragraph; Attention.forward and apply_rotary_emb): each normalised latent row
// is rotated forward on its last rope_dim elements at its position (pairs times (cos, sin)
// in f32, back to bf16), quantised to fp8 in blocks of 32 (the round trip is stored as bf16,
// or the codes and scale bytes), and stored: into slot pos mod window of its sequence's ring
// (only the last `window` rows of a call, later rows win a shared slot), or at row
// row0[n] + t of a linear cache. One thread per 8 elements (16 bytes) of a row, a 32-element
// block per 4 threads. No contraction into fused multiply-adds, as in the page's f32 steps.
template <int D>
__global__ __launch_bounds__(256) void kv_write_kernel(const KvWriteParams p) {
#pragma clang fp contract(off)
    constexpr int kLanesPerRow = D / 8;
    const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gtid / kLanesPerRow;
    const int part = (int)(gtid % kLanesPerRow);
    const bool live = row < (int64_t)p.b * p.s;
    // b * s < 2^31 (checked on the host): a 32-bit division
    const uint32_t r32 = live ? (uint32_t)row : 0u;
    const int n = (int)(r32 / (uint32_t)p.s);
    const int t = (int)(r32 - (uint32_t)n * (uint32_t)p.s);
    // the row's bytes and its position are loaded side by side (one memory round trip)
    u32x4 v = live ? *(const u32x4*)(p.x + (int64_t)n * p.x_seq_stride + (int64_t)t * D + 8 * part)
                   : u32x4{0, 0, 0, 0};
    const int pos = live ? p.pos[(int64_t)n * p.pos_seq_stride + t] : 0;
    const bool pos_ok = live && pos >= 0 && (p.rope_dim == 0 || pos < p.max_pos);
    if (!pos_ok) v = u32x4{0, 0, 0, 0};
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) { x[2 * k] = bf16_lo(v[k]); x[2 * k + 1] = bf16_hi(v[k]); }
    // forward rotation of the pairs in the rope tail
    const int r0 = D - p.rope_dim;
    if (pos_ok && 8 * part + 8 > r0) {
        const float* cs = p.rope_cs + (int64_t)pos * p.rope_dim;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = 8 * part + 2 * k;
            if (e >= r0) {
                const float c = cs[e - r0], sn = cs[e - r0 + 1];
                const float a = x[2 * k], b = x[2 * k + 1];
                const float re = a * c - b * sn;
                const float im = a * sn + b * c;
                const uint32_t w = pack_bf16x2(re, im);
                x[2 * k] = bf16_lo(w);
                x[2 * k + 1] = bf16_hi(w);
            }
        }
    }
    // block-32 fp8 round trip (the four threads of a block share its maximum)
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    amax = fmaxf(amax, 1e-4f);
    const float sc = pow2_ceil_f32(amax / 448.0f);
    if (!live) return;
    int64_t dst = -1;
    if (pos_ok) {
        if (p.window > 0) dst = t >= p.s - p.window ? pos % p.window : -2;   // -2: a later row wins
        else dst = (int64_t)p.row0[n] + t;
    }
    const bool store = dst >= 0 && dst < p.cache_rows;
    if ((p.flags & 1u) && part == 0 && (!pos_ok || (dst != -2 && !store))) atomicOr(p.err_word, 4);
    if (!pos_ok) return;
    const float inv_sc = 1.0f / sc;                                  // exact (a power of two)
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = x[k] * inv_sc;
    const u32x2 w = e4m3_pack8(y);
    const u32x4 rt = e4m3_roundtrip8(w, sc);
    if (p.rows_out) *(u32x4*)(p.rows_out + (int64_t)n * p.rows_out_seq_stride + (int64_t)t * D + 8 * part) = rt;
    if (!store) return;
    const int64_t off = (int64_t)n * p.cache_seq_stride + dst * D + 8 * part;
    if (p.cache_bf16) {
        *(u32x4*)(p.cache_bf16 + off) = rt;
    } else {
        *(u32x2*)(p.cache_codes + off) = w;
        if ((part & 3) == 0)
            p.cache_scales[(int64_t)n * p.cache_scale_seq_stride + dst * (D / 32) + part / 4] =
                (uint8_t)((f32_bits(sc) >> 23) & 0xffu);
    }
}

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t st) {
    const int64_t threads = (int64_t)p.b * p.s * (p.d / 8);
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid), blk(256);
    switch (p.d) {
        case 64: hipLaunchKernelGGL(kv_write_kernel<64>, g, blk, 0, st, p); break;
        case 128: hipLaunchKernelGGL(kv_write_kernel<128>, g, blk, 0, st, p); break;
        case 256: hipLaunchKernelGGL(kv_write_kernel<256>, g, blk, 0, st, p); break;
        case 512: hipLaunchKernelGGL(kv_write_kernel<512>, g, blk, 0, st, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sa
