// k_pack.hip -- final group quantization of W diag(s) and bit packing (step 5).
//
// Quantizer, fp32 in this exact operation order (bit-exact contract):
//   v = w * s
//   symmetric ("GPTQ and AWQ weight quantisation", "Per-group symmetric int4
//   (RTN)" and the n-bit form under "Output MSE vs bit width"):
//     scale = max(max|v| / L, 1e-8), q = clamp(rne(v / scale), -L-1, L), code = q + 2^(b-1)
//   asymmetric ("AWQ vs GPTQ Quantization Architectures Compared", group_params
//   and rtn under "GPTQ: compensate the error you just made"):
//     lo = min(min v, 0), hi = max(max v, 0), scale = max((hi - lo) / maxq, 1e-8),
//     zero = rne(-lo / scale), code = clamp(rne(v / scale) + zero, 0, maxq)
// With clipping ratios r (one per row and group, from the clipping-range
// search) the group's range is scaled first -- symmetric [-r max|v|, r max|v|],
// asymmetric [r lo, r hi] -- v is clamped into it, and the scale (and zero)
// are those of the scaled range; r = 1 gives the unclipped quantizer exactly.
// Every quotient is the correctly rounded one (an IEEE division per group for
// the reciprocal, two fma residual steps per weight), the library is built
// with -ffp-contract=off and rintf is v_rndne_f32.
//
// Layout: one lane owns 32 consecutive columns of one row. 32 codes of b bits
// fill exactly b 32-bit words, so a lane writes whole words of the row's
// little-endian bit stream with no neighbour; a group of G columns spans G/32
// adjacent lanes, whose max/min are combined with xor shuffles. A wave takes
// 2048 consecutive columns of one row and four waves take four rows of the
// same columns, whose scale factors are read from HBM once per block. Loads
// and stores of a wave are contiguous. HBM bound: read W (2 or 4 B per
// weight), write b/8 B per weight plus 5 B per group.
#include "awq_internal.h"

#include <float.h>
#include <math.h>

#include <type_traits>

namespace awq {

// fp32(w * s) for the low (H = 0) or high (H = 1) fp16 of a packed pair in
// one v_fma_mix_f32: the fp16 source is widened exactly and w * s + (-0) is
// rounded once, which is the product itself, signed zeros included.
template <int H>
__device__ __forceinline__ float mul_f16_exact(uint32_t pair, float s)
{
    float r;
    const float nz = -0.0f;
    if (H == 0)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(s), "v"(nz));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r)
            : "v"(pair), "v"(s), "v"(nz));
    return r;
}

// a / b rounded to nearest even, for finite b >= 1e-8 and y = a correctly
// rounded 1/b (an IEEE division, once per group). q0 = a*y is within 2 ulp of
// a/b; one residual step (the residual a - b*q is exact or nearly so in an
// fma) makes it faithful, and a second one, with a faithful q and a correctly
// rounded y, gives the correctly rounded quotient (Markstein's theorem).
// Quotients small enough for the residual to underflow lie far below 0.5 and
// round to the same integer either way.
__device__ __forceinline__ float div_rn(float a, float b, float y)
{
    float q = a * y;
    q = fmaf(fmaf(-b, q, a), y, q);
    return fmaf(fmaf(-b, q, a), y, q);
}

// codes of one lane's 32 values: clamp(rne(v / scale) + zero, lo, hi) for
// asymmetric, clamp(rne(v / scale), lo, hi) + zero for symmetric. FAST uses
// div_rn (finite scale), otherwise the IEEE division (infinite scale, where
// the residual steps would turn 0 * inf into NaN). With a finite scale and
// finite values only the asymmetric upper bound can bind: |v| / scale <=
// L (1 + 2^-23) < L + 1/2 for symmetric groups, and rne(v / scale) >=
// rne(lo / scale) = -zero for asymmetric ones (rne is odd and monotone), so
// FAST drops the other clamps. (Codes of groups with NaN values are
// unspecified.)
//
// FAST first rounds u = v * y (y = RN(1/scale)): u lies within
// 1.5 * 2^-23 |v / scale| <= 1.5 * 2^(BITS-23) of the correctly rounded
// quotient (|v / scale| <= 2^BITS here), so rne(u) is rne of that quotient
// unless u lies within that distance of a half-integer (a tie included). A
// wave in which some u lies within 2^(BITS-21) of one computes all its
// quotients correctly rounded instead (rare: about 2^(BITS-20) of the
// weights are that close).
template <int BITS, bool ASYM, bool FAST>
__device__ __forceinline__ void codes(const float (&v)[32], float scale, float lo, float hi, float zero,
                                      uint32_t (&word)[BITS])
{
    const float y = FAST ? 1.0f / scale : 0.0f;
    float qs[32];
    if (FAST) {
        float dmax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float u = v[i] * y;
            qs[i] = rintf(u);
            dmax = fmaxf(dmax, fabsf(u - qs[i]));
        }
        const float thr = 0.5f - (float)(1 << BITS) * 0x1p-21f;
        if (__builtin_amdgcn_ballot_w64(dmax >= thr) != 0) {
#pragma unroll
            for (int i = 0; i < 32; ++i)
                qs[i] = rintf(div_rn(v[i], scale, y));
        }
    }
#pragma unroll
    for (int k = 0; k < BITS; ++k)
        word[k] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        float q = FAST ? qs[i] : rintf(v[i] / scale);
        uint32_t code;
        if (ASYM) {
            q = FAST ? fminf(q + zero, hi) : fminf(fmaxf(q + zero, lo), hi);
            code = (uint32_t)(int)q;
        } else {
            if (!FAST)
                q = fminf(fmaxf(q, lo), hi);
            code = (uint32_t)((int)q + (int)zero);
        }
        // code i at bits [i*BITS, (i+1)*BITS) of the lane's BITS words
        const int bit = i * BITS, wi = bit >> 5, sh = bit & 31;
        word[wi] |= code << sh;
        if (sh + BITS > 32)
            word[wi + 1] |= code >> (32 - sh);
    }
}

// Block: kPackRows rows (one wave each) x kPackChunks 32-column chunks (2048
// columns, a multiple of every group); the tile's 2048 scale factors are
// staged once in LDS and shared by its rows.
constexpr int kPackRows = 4;
constexpr int kPackChunks = 64;

template <typename T, int BITS, bool CLIP>
__global__ __launch_bounds__(kPackRows * 64) void k_quantize_pack(const T *__restrict__ W, int64_t out,
                                                                  int64_t in, const float *__restrict__ s,
                                                                  const float *__restrict__ clip,
                                                                  int lanes_per_group, int mode,
                                                                  uint32_t *__restrict__ qweight,
                                                                  float *__restrict__ scales,
                                                                  uint8_t *__restrict__ zeros)
{
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    // sl[i][l] = s[c0 + 32 l + 4 i .. + 3]: lane l's 32 factors as eight
    // 16-byte reads at consecutive addresses across the lanes
    __shared__ f32x4v sl[8][kPackChunks];
    const int64_t chunks = in / 32;
    const int64_t tiles = (chunks + kPackChunks - 1) / kPackChunks;
    const int64_t rblk = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row_raw = rblk * kPackRows + wave, ch_raw = tile * kPackChunks + lane;
    const bool active = row_raw < out && ch_raw < chunks;
    const int64_t row = active ? row_raw : 0;
    const int64_t ch = active ? ch_raw : 0;
    // the lane's 32 weights, loaded before the scale factors' staging and
    // barrier so that the two memory round trips overlap
    typename Vec8<T>::type wl[4];
    {
        const T *wp = W + row * in + ch * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            wl[q] = load8(wp + q * 8);
    }
    {
        const int l = threadIdx.x >> 2, part = threadIdx.x & 3;   // 8 factors each
        const int64_t col = (tile * kPackChunks + l) * 32 + part * 8;
        f32x8 s8 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (col < in)                              // in % 32 == 0: all 8 are in range
            s8 = *reinterpret_cast<const f32x8 *>(s + col);
        sl[2 * part][l] = f32x4v{s8[0], s8[1], s8[2], s8[3]};
        sl[2 * part + 1][l] = f32x4v{s8[4], s8[5], s8[6], s8[7]};
    }
    __syncthreads();

    float v[32];
    if (active) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4v s_lo = sl[2 * q][lane], s_hi = sl[2 * q + 1][lane];
            const f32x8 s8 = {s_lo[0], s_lo[1], s_lo[2], s_lo[3], s_hi[0], s_hi[1], s_hi[2], s_hi[3]};
            if constexpr (std::is_same<T, f16>::value) {
                typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 pr = __builtin_bit_cast(u32x4, wl[q]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[q * 8 + 2 * e] = mul_f16_exact<0>(pr[e], s8[2 * e]);
                    v[q * 8 + 2 * e + 1] = mul_f16_exact<1>(pr[e], s8[2 * e + 1]);
                }
            } else {
                float w8[8];
                widen8<T>(wl[q], w8);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[q * 8 + i] = w8[i] * s8[i];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            v[i] = 0.f;
    }

    // Clamping into the clipped range keeps |x| / scale (and x / scale above
    // lo / scale) within the bounds the FAST code path relies on.
    const float ratio = CLIP ? clip[row * (chunks / lanes_per_group) + ch / lanes_per_group] : 1.0f;
    uint32_t word[BITS];
    float scale, zero;
    if (mode == AWQ_SYM) {
        const float levels = (float)((1 << (BITS - 1)) - 1);
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 32; i += 2)
            m = fmaxf(fmaxf(m, fabsf(v[i])), fabsf(v[i + 1]));
        for (int off = 1; off < lanes_per_group; off <<= 1)
            m = fmaxf(m, __shfl_xor(m, off));
        if (CLIP) {
            m = ratio * m;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                v[i] = fminf(fmaxf(v[i], -m), m);
        }
        scale = fmaxf(m / levels, 1e-8f);
        zero = (float)(1 << (BITS - 1));
        if (scale <= FLT_MAX)
            codes<BITS, false, true>(v, scale, -levels - 1.0f, levels, zero, word);
        else
            codes<BITS, false, false>(v, scale, -levels - 1.0f, levels, zero, word);
    } else {
        const float maxq = (float)((1 << BITS) - 1);
        float lo = 0.f, hi = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            lo = fminf(lo, v[i]);
            hi = fmaxf(hi, v[i]);
        }
        for (int off = 1; off < lanes_per_group; off <<= 1) {
            lo = fminf(lo, __shfl_xor(lo, off));
            hi = fmaxf(hi, __shfl_xor(hi, off));
        }
        if (CLIP) {
            lo = ratio * lo;
            hi = ratio * hi;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                v[i] = fminf(fmaxf(v[i], lo), hi);
        }
        scale = fmaxf((hi - lo) / maxq, 1e-8f);
        zero = rintf(-lo / scale);
        if (scale <= FLT_MAX)
            codes<BITS, true, true>(v, scale, 0.0f, maxq, zero, word);
        else
            codes<BITS, true, false>(v, scale, 0.0f, maxq, zero, word);
    }
    if (!active)
        return;

    uint32_t *dst = qweight + row * (chunks * BITS) + ch * BITS;
#pragma unroll
    for (int k = 0; k < BITS; ++k)
        dst[k] = word[k];
    if (ch % lanes_per_group == 0) {
        const int64_t gi = row * (in / (32 * lanes_per_group)) + ch / lanes_per_group;
        scales[gi] = scale;
        zeros[gi] = (uint8_t)(int)zero;
    }
}

template <typename T, bool CLIP>
static void pack_typed(const T *W, int64_t out, int64_t in, const float *s, const float *clip,
                       int bits, int lpg, int mode, uint32_t *qweight, float *scales,
                       uint8_t *zeros, hipStream_t st)
{
    const int64_t tiles = (in / 32 + kPackChunks - 1) / kPackChunks;
    dim3 grid((unsigned)(((out + kPackRows - 1) / kPackRows) * tiles));
#define AWQ_PACK_LAUNCH(B)                                                                               \
    hipLaunchKernelGGL((k_quantize_pack<T, B, CLIP>), grid, dim3(kPackRows * 64), 0, st, W, out, in, s, \
                       clip, lpg, mode, qweight, scales, zeros)
    switch (bits) {
    case 2: AWQ_PACK_LAUNCH(2); break;
    case 3: AWQ_PACK_LAUNCH(3); break;
    case 4: AWQ_PACK_LAUNCH(4); break;
    case 5: AWQ_PACK_LAUNCH(5); break;
    case 6: AWQ_PACK_LAUNCH(6); break;
    case 7: AWQ_PACK_LAUNCH(7); break;
    default: AWQ_PACK_LAUNCH(8); break;
    }
#undef AWQ_PACK_LAUNCH
}

template <typename T>
static void pack_clip_or_not(const T *W, int64_t out, int64_t in, const float *s, const float *clip,
                             int bits, int lpg, int mode, uint32_t *qweight, float *scales,
                             uint8_t *zeros, hipStream_t st)
{
    if (clip)
        pack_typed<T, true>(W, out, in, s, clip, bits, lpg, mode, qweight, scales, zeros, st);
    else
        pack_typed<T, false>(W, out, in, s, clip, bits, lpg, mode, qweight, scales, zeros, st);
}

hipError_t launch_pack(const void *W, int dtype, int64_t out, int64_t in, const float *s,
                       const float *clip, int bits, int group, int mode, uint32_t *qweight,
                       float *scales, uint8_t *zeros, hipStream_t st)
{
    const int lpg = group / 32;
    switch (dtype) {
    case AWQ_F32:
        pack_clip_or_not((const float *)W, out, in, s, clip, bits, lpg, mode, qweight, scales, zeros, st);
        break;
    case AWQ_F16:
        pack_clip_or_not((const f16 *)W, out, in, s, clip, bits, lpg, mode, qweight, scales, zeros, st);
        break;
    default:
        pack_clip_or_not((const bf16 *)W, out, in, s, clip, bits, lpg, mode, qweight, scales, zeros, st);
        break;
    }
    return hipGetLastError();
}

}  // namespace awq
