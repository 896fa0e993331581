// sparse_attn launches: the key-loop kernel (attn_fwd_kernel.hpp) for every supported
// shape except the wide bf16 one (attn_fwd_wide.hip), the split combine kernel, and the pass
// that turns fp8 storage into bf16 rows for plans that read each row many times.
#include "attn_fwd_kernel.hpp"

namespace sa {

hipError_t launch_fwd_wide(const KParams& p, int blocks, hipStream_t st);

// Merge the split partials of one (query, head): m = max m_i, l = sum l_i 2^(m_i - m),
// o = sum O_i 2^(m_i - m) / l (the sink is in l_0 only). One wave per (query, head); each
// lane owns max(D/64, 4) consecutive elements of d.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const KParams p) {
    const int wave = blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (wave >= p.b * p.s * p.h) return;
    const int head = wave % p.h;
    const int qi = wave / p.h;
    const int seq = qi / p.s, t = qi % p.s;
    constexpr int kPer = D / 64 >= 4 ? D / 64 : 4;             // elements per lane
    constexpr int kLanes = D / kPer;
    float m = -INFINITY;
    for (int i = 0; i < p.splits; ++i)
        m = fmaxf(m, p.ws_ml[(((int64_t)qi * p.splits + i) * p.h_pad + head) * 2]);
    if (m == -INFINITY) m = 0.0f;        // no split saw a row and the sink is -inf: all weights 0
    float l = 0.0f;
    float acc[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] = 0.0f;
    for (int i = 0; i < p.splits; ++i) {
        const int64_t slot = ((int64_t)qi * p.splits + i) * p.h_pad + head;
        const float wgt = fast_exp2(p.ws_ml[slot * 2] - m);
        l += p.ws_ml[slot * 2 + 1] * wgt;
        if (lane < kLanes) {
            const float* src = p.ws_o + slot * D + lane * kPer;
#pragma unroll
            for (int k = 0; k < kPer; k += 4) {
                const f32x4 v = *(const f32x4*)(src + k);
                acc[k] += v[0] * wgt; acc[k + 1] += v[1] * wgt;
                acc[k + 2] += v[2] * wgt; acc[k + 3] += v[3] * wgt;
            }
        }
    }
    if (lane >= kLanes) return;
    const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
    const float* cs = rope_row(p, seq, t, lane == 0);
    const int r0 = D - p.rope_dim;
    uint16_t* orow = p.out + (int64_t)seq * p.out_seq_stride + ((int64_t)t * p.h + head) * D;
#pragma unroll
    for (int k = 0; k < kPer; k += 4) {
        const int d0 = lane * kPer + k;
        *(u32x2*)(orow + d0) = epilogue4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3], inv_l,
                                         cs != nullptr && d0 + 4 > r0, d0, r0, cs);
    }
}

// ------------------------------------------------------------------ launch
template <int D, bool FP8>
static hipError_t launch_fwd_nw(const KParams& p, int nw, int hpw, int kg, bool compact, int blocks, hipStream_t st) {
    if (compact) {
        if constexpr (D == 512 && !FP8)
            if (nw == 2 && hpw == 1 && kg == 1) return launch_fwd<512, false, 2, 1, 1, true>(p, blocks, st);
        return hipErrorInvalidValue;
    }
    if constexpr (D == 512) {
        if constexpr (!FP8)
            if (hpw == 2) return nw == 4 && kg == 1 ? launch_fwd_wide(p, blocks, st) : hipErrorInvalidValue;
        if (kg == 2) return nw == 4 && hpw == 1 ? launch_fwd<D, FP8, 4, 1, 2>(p, blocks, st) : hipErrorInvalidValue;
        if constexpr (!FP8)   // fp8: at most two key groups (its raw slots hold two tiles of a super tile)
            if (kg == 4) return nw == 4 && hpw == 1 ? launch_fwd<D, FP8, 4, 1, 4>(p, blocks, st) : hipErrorInvalidValue;
    }
    if (hpw != 1 || kg != 1) return hipErrorInvalidValue;
    if (nw == 1) return launch_fwd<D, FP8, 1>(p, blocks, st);
    if (nw == 2) return launch_fwd<D, FP8, 2>(p, blocks, st);
    return launch_fwd<D, FP8, 4>(p, blocks, st);
}

template <int D>
static hipError_t launch_all(const KParams& p, bool fp8, int nw, int hpw, int kg, bool compact, int blocks,
                             hipStream_t st) {
    hipError_t e = fp8 ? launch_fwd_nw<D, true>(p, nw, hpw, kg, compact, blocks, st)
                       : launch_fwd_nw<D, false>(p, nw, hpw, kg, compact, blocks, st);
    if (e != hipSuccess || p.splits == 1) return e;
    // one wave per (query, head); the host keeps b * s * h within int32 for split plans
    const int64_t waves = (int64_t)p.b * p.s * p.h;
    hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, p);
    return hipGetLastError();
}

// fp8 storage -> bf16 rows: each thread turns one 16-byte piece of codes (16 elements of one
// 32-element block) into 32 bytes of bf16, code x 2^(e - 127) on v_cvt_scalef32_pk_bf16_fp8
// (exact: the stored values are bf16 values). Streams the cache once (HBM-bound).
__global__ __launch_bounds__(256) void dequant_kv_kernel(const uint8_t* codes, int64_t codes_seq_stride,
                                                         const uint8_t* scales, int64_t scales_seq_stride,
                                                         int b, int rows, int d, uint16_t* out) {
    const int pieces = d / 16;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_seq = (int64_t)rows * pieces;
    if (i >= per_seq * b) return;
    const int64_t n = i / per_seq, rem = i % per_seq;
    const int64_t r = rem / pieces;
    const int pc = (int)(rem % pieces);
    const u32x4 c = *(const u32x4*)(codes + n * codes_seq_stride + r * d + 16 * pc);
    const float sc = bits_f32((uint32_t)scales[n * scales_seq_stride + r * (d / 32) + pc / 2] << 23);
    u32x4 o[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[j / 2][2 * (j % 2)] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], sc, false));
        o[j / 2][2 * (j % 2) + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], sc, true));
    }
    u32x4* dst = (u32x4*)(out + (n * rows + r) * d + 16 * pc);
    dst[0] = o[0];
    dst[1] = o[1];
}

hipError_t launch_dequant_kv(const uint8_t* codes, int64_t codes_seq_stride, const uint8_t* scales,
                             int64_t scales_seq_stride, int b, int rows, int d, uint16_t* out, hipStream_t st) {
    const int64_t threads = (int64_t)b * rows * (d / 16);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dequant_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, codes_seq_stride,
                       scales, scales_seq_stride, b, rows, d, out);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const KParams& p, bool fp8, int nw, int hpw, int kg, bool compact, hipStream_t st) {
    const int blocks = p.b * p.s * p.head_blocks * p.splits;
    switch (p.d) {
        case 64: return launch_all<64>(p, fp8, nw, hpw, kg, compact, blocks, st);
        case 128: return launch_all<128>(p, fp8, nw, hpw, kg, compact, blocks, st);
        case 256: return launch_all<256>(p, fp8, nw, hpw, kg, compact, blocks, st);
        case 512: return launch_all<512>(p, fp8, nw, hpw, kg, compact, blocks, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sa
