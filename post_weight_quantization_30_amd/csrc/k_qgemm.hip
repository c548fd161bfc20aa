// k_qgemm.hip -- the deployment product over the packed layout.
//
// Y[m][n] = sum_k X[m][k] * Wd[n][k],  Wd[n][k] = scale[n][g] * (code[n][k] - zero[n][g]),
// g = k / group: the serving-side consumer of the quantized weights ("AWQ vs
// GPTQ Quantization Architectures Compared", "What lands on disk" and "From
// checkpoint to kernel": at decode batch sizes the layer is memory-bound and
// the speed-up comes from reading a quarter of the bytes).
//
// Exactness: code - zero is a small integer, exact in fp16 and bf16, so the
// MFMA multiplies X by exact integer-valued weights; each group's fp32 sum is
// multiplied once by its scale (one fma into the fp32 total). No weight is
// ever rounded to 16 bits.
//
// Layout: one block = (16 NT) output rows x (16 MT) tokens, 8 waves; wave w
// takes groups w, w + 8, w + 16, ... (split-K inside the block, so a 4096-row
// layer at decode still fills 256 blocks), and the 8 partial tiles are added
// in wave order through LDS. The packed rows go through LDS so that the HBM
// reads are whole cache lines (see QStage). In an MFMA k-step the four 8-wide k-slots of lane
// group c hold columns c * G/4 + 8 s + e of the group (s = step, e = element),
// for the X operand and for the codes alike, so a lane reads G/4 consecutive
// codes of its row (whole 32-bit words) and G/4 consecutive activations.
#include "awq_internal.h"

#include <type_traits>

namespace awq {

constexpr int kQWaves = 8;

template <typename TX> struct QOp;
template <> struct QOp<f16> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x4 mfma(const vec &a, const vec &b, const f32x4 &c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct QOp<bf16> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x4 mfma(const vec &a, const vec &b, const f32x4 &c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// Per-block staging of the packed rows. A round covers 8 consecutive groups
// (one per wave) of the block's R = 16 NT rows: RB = 8 G BITS / 8 bytes per
// row, loaded with contiguous 16-byte chunks per lane (whole cache lines, a
// wave covering one or more rows end to end), together with the round's
// scales and zeros, and stored to LDS rows padded by 16 bytes (the 16 rows a
// 16-byte LDS read touches then fall on distinct banks).
template <int BITS, int G, int NT>
struct QStage {
    static constexpr int R = 16 * NT;
    static constexpr int GB = G * BITS / 8;          // bytes of one group of one row
    static constexpr int RB = 8 * GB;                // bytes of a round of one row
    static constexpr int RBP = RB + 16;              // padded LDS row stride
    static constexpr int CHUNKS = R * RB / 16;       // 16-byte chunks per round
    static constexpr int PER_THREAD = (CHUNKS + kQWaves * 64 - 1) / (kQWaves * 64);
    static constexpr int BUF = R * RBP + R * 8 * 4 + R * 8;   // codes, scales, zeros
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int BITS, int G, int NT>
struct QRound {
    typedef QStage<BITS, G, NT> S;
    u32x4 chunk[S::PER_THREAD];
    float scale;
    uint8_t zero;
};

// Global -> registers for round q (every access in bounds: rows past `out`
// are clamped, groups past ng are not loaded).
template <int BITS, int G, int NT>
__device__ __forceinline__ void q_fetch(QRound<BITS, G, NT> &rd, const uint8_t *qbytes, const float *scales,
                                        const uint8_t *zeros, int64_t n0, int64_t out, int64_t ng,
                                        int64_t row_bytes, int64_t q)
{
    typedef QStage<BITS, G, NT> S;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < S::PER_THREAD; ++k) {
        const int ch = tid + k * kQWaves * 64;
        if (ch < S::CHUNKS) {
            const int row = ch / (S::RB / 16), off = (ch % (S::RB / 16)) * 16;
            int64_t n = n0 + row;
            n = n < out ? n : out - 1;
            const int64_t byte = q * S::RB + off;
            if (byte < row_bytes)
                rd.chunk[k] = *reinterpret_cast<const u32x4 *>(qbytes + n * row_bytes + byte);
        }
    }
    if (tid < S::R * 8) {
        const int row = tid / 8, j = tid % 8;
        int64_t n = n0 + row;
        n = n < out ? n : out - 1;
        const int64_t g = q * 8 + j;
        if (g < ng) {
            rd.scale = scales[n * ng + g];
            rd.zero = zeros[n * ng + g];
        }
    }
}

template <int BITS, int G, int NT>
__device__ __forceinline__ void q_stash(const QRound<BITS, G, NT> &rd, uint8_t *buf)
{
    typedef QStage<BITS, G, NT> S;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < S::PER_THREAD; ++k) {
        const int ch = tid + k * kQWaves * 64;
        if (ch < S::CHUNKS) {
            const int row = ch / (S::RB / 16), off = (ch % (S::RB / 16)) * 16;
            *reinterpret_cast<u32x4 *>(buf + row * S::RBP + off) = rd.chunk[k];
        }
    }
    if (tid < S::R * 8) {
        reinterpret_cast<float *>(buf + S::R * S::RBP)[tid] = rd.scale;
        (buf + S::R * S::RBP + S::R * 8 * 4)[tid] = rd.zero;
    }
}

// X fragments of one group for one lane (MT token tiles). Token rows past M
// load the last row instead: their products only reach accumulator rows that
// are never stored. (A zero fill on a per-lane branch would make the compiler
// wait for the load at the join.)
template <typename TX, int G, int MT>
__device__ __forceinline__ void q_fetch_x(typename QOp<TX>::vec (&x)[MT][G / 32], const TX *X, int64_t M,
                                          int64_t in, int64_t g, int64_t m0, int r, int c)
{
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int64_t m = m0 + t * 16 + r;
        m = m < M ? m : M - 1;
        const TX *xp = X + m * in + g * G + c * (G / 4);
#pragma unroll
        for (int s = 0; s < G / 32; ++s)
            x[t][s] = load8(xp + 8 * s);
    }
}

// (a & m) | o in one v_and_or_b32. The compiler splits it in two when m and
// o are literals (a VOP3 instruction on this target takes no literal), so the
// constants are passed in registers.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
    return r;
}

// fp16 operands: the eight codes of a k-step become (code - zero) two at a
// time without leaving 16 bits. 0x6400 | c is the fp16 value 1024 + c
// (c < 1024), so one mask-and-or makes a pair from two codes that sit 16 bits
// apart in the code words, and one packed fp16 subtraction of 1024 + zero
// leaves the exact small integers. The pairs come out in the order PERM
// (4-bit: codes 0,4,1,5,2,6,3,7 of a word; 8-bit: 0,2,1,3 of each word), and
// the X fragment is permuted the same way: the contraction over k does not
// depend on the order in which both operands present it.
template <int BITS> struct F16Pairs;
template <> struct F16Pairs<4> {
    static constexpr int PERM[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    static constexpr uint32_t kMask = 0x000F000Fu;
    static __device__ __forceinline__ void make(const uint32_t *w, uint32_t (&u)[4], uint32_t mask,
                                                uint32_t magic)
    {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            u[p] = and_or(w[0] >> (4 * p), mask, magic);
    }
};
template <> struct F16Pairs<8> {
    static constexpr int PERM[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    static constexpr uint32_t kMask = 0x00FF00FFu;
    static __device__ __forceinline__ void make(const uint32_t *w, uint32_t (&u)[4], uint32_t mask,
                                                uint32_t magic)
    {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            u[2 * q] = and_or(w[q], mask, magic);
            u[2 * q + 1] = and_or(w[q] >> 8, mask, magic);
        }
    }
};

// One group for one wave: B fragments of its NT row tiles from the staged
// round, X fragments from registers; each row tile's fp32 group sums are
// scaled into the totals.
template <typename TX, int BITS, int G, int MT, int NT>
__device__ __forceinline__ void q_group(const uint8_t *buf, int w, const typename QOp<TX>::vec (&x)[MT][G / 32],
                                        f32x4 (&acc)[MT][NT], int r, int c)
{
    typedef QStage<BITS, G, NT> S;
    typedef typename QOp<TX>::vec vec;
    constexpr int STEPS = G / 32;
    constexpr int WPL = G * BITS / 128;              // code words per lane
    constexpr uint32_t cmask = (1u << BITS) - 1u;
    constexpr bool kPairs = std::is_same<TX, f16>::value;
    vec xs[MT][STEPS];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            if constexpr (kPairs) {
                constexpr const int *P = F16Pairs<BITS>::PERM;
                xs[t][s] = __builtin_shufflevector(x[t][s], x[t][s], P[0], P[1], P[2], P[3], P[4], P[5],
                                                   P[6], P[7]);
            } else {
                xs[t][s] = x[t][s];
            }
        }
    const float *sbuf = reinterpret_cast<const float *>(buf + S::R * S::RBP);
    const uint8_t *zbuf = buf + S::R * S::RBP + S::R * 8 * 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int row = nt * 16 + r;
        uint32_t wv[WPL];
        const uint8_t *src = buf + row * S::RBP + w * S::GB + c * (S::GB / 4);
        if constexpr (WPL % 4 == 0) {
#pragma unroll
            for (int q = 0; q < WPL / 4; ++q) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 16 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    wv[4 * q + e] = v[e];
            }
        } else if constexpr (WPL == 2) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = *reinterpret_cast<const u32x2 *>(src);
            wv[0] = v[0];
            wv[1] = v[1];
        } else {
            wv[0] = *reinterpret_cast<const uint32_t *>(src);
        }
        const float scale = sbuf[row * 8 + w];
        const int zero = zbuf[row * 8 + w];
        vec b[STEPS];
        if constexpr (kPairs) {
            const f16 zb = static_cast<f16>(1024 + zero);           // exact: at most 1279
            const f16x2 z2 = {zb, zb};
            const uint32_t mask = F16Pairs<BITS>::kMask, magic = 0x64006400u;
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                uint32_t u[4];
                F16Pairs<BITS>::make(&wv[s * BITS / 4], u, mask, magic);    // the step's BITS/4 words
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const f16x2 d = __builtin_bit_cast(f16x2, u[p]) - z2;   // exact
                    b[s][2 * p] = d[0];
                    b[s][2 * p + 1] = d[1];
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 8 * s + e;                // code j of the lane's G/4 codes
                    const int code = (int)((wv[(j * BITS) / 32] >> ((j * BITS) % 32)) & cmask);
                    b[s][e] = static_cast<TX>(static_cast<float>(code - zero));   // exact
                }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
                part = QOp<TX>::mfma(xs[t][s], b[s], part);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][nt][i] = fmaf(scale, part[i], acc[t][nt][i]);
        }
    }
}

// Block: (16 NT) output rows x (16 MT) tokens, 8 waves; round q stages groups
// 8q .. 8q+7 and wave w computes group 8q + w. Round q + 1 is fetched from
// HBM (codes, scales, zeros, and each wave's X fragments) while round q is
// computed; one barrier per round.
template <typename TX, int BITS, int G, int MT, int NT, bool YF32>
__global__ __launch_bounds__(kQWaves * 64) void k_qgemm(const TX *__restrict__ X, int64_t M, int64_t in,
                                                        const uint32_t *__restrict__ qweight,
                                                        const float *__restrict__ scales,
                                                        const uint8_t *__restrict__ zeros, int64_t out,
                                                        void *__restrict__ Y)
{
    typedef QStage<BITS, G, NT> S;
    typedef typename QOp<TX>::vec vec;
    constexpr int RED = kQWaves * MT * NT * 64 * 16;
    constexpr int LDS = 2 * S::BUF > RED ? 2 * S::BUF : RED;
    __shared__ __align__(16) uint8_t lds[LDS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, c = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * S::R;
    const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
    const int64_t ng = in / G;
    const int64_t row_bytes = in * BITS / 8;
    const int64_t rounds = (ng + 7) / 8;
    const uint8_t *qbytes = reinterpret_cast<const uint8_t *>(qweight);

    f32x4 acc[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    QRound<BITS, G, NT> rd = {};
    vec xcur[MT][G / 32], xnext[MT][G / 32];
    q_fetch(rd, qbytes, scales, zeros, n0, out, ng, row_bytes, 0);
    if (wave < ng)
        q_fetch_x<TX, G, MT>(xcur, X, M, in, wave, m0, r, c);
    q_stash(rd, lds);
    __syncthreads();
    for (int64_t q = 0; q < rounds; ++q) {
        const bool more = q + 1 < rounds;
        const int64_t g = q * 8 + wave, gn = g + 8;
        if (more) {
            q_fetch(rd, qbytes, scales, zeros, n0, out, ng, row_bytes, q + 1);
            if (gn < ng)
                q_fetch_x<TX, G, MT>(xnext, X, M, in, gn, m0, r, c);
        }
        if (g < ng)
            q_group<TX, BITS, G, MT, NT>(lds + (q & 1) * S::BUF, wave, xcur, acc, r, c);
        if (more) {
            q_stash(rd, lds + ((q + 1) & 1) * S::BUF);
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int s = 0; s < G / 32; ++s)
                    xcur[t][s] = xnext[t][s];
        }
        __syncthreads();
    }

    // fixed-order reduction over the waves (the staging buffers are free now)
    f32x4 *red = reinterpret_cast<f32x4 *>(lds);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            red[((wave * MT + t) * NT + nt) * 64 + lane] = acc[t][nt];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * NT * 64; idx += blockDim.x) {
        const int t = idx / (NT * 64), nt = (idx / 64) % NT, l = idx & 63;
        f32x4 sum = red[(t * NT + nt) * 64 + l];
#pragma unroll
        for (int w = 1; w < kQWaves; ++w)
            sum += red[((w * MT + t) * NT + nt) * 64 + l];
        const int64_t nn = n0 + nt * 16 + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + t * 16 + 4 * (l >> 4) + i;
            if (m < M && nn < out) {
                if (YF32)
                    static_cast<float *>(Y)[m * out + nn] = sum[i];
                else
                    static_cast<TX *>(Y)[m * out + nn] = static_cast<TX>(sum[i]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode, up to 4 tokens: a persistent grid (as many blocks as fit on the
// chip at once), each block of 8 waves walking row tiles of 16 NT rows. A
// row's codes are cut into batches of GPB consecutive groups (KB columns);
// in each tile wave w takes batches w, w + 8, ... The block first copies the
// M tokens of X into LDS, in the operand order of the code pairs; the MFMA
// fragments are read from there (the lanes of tokens past M read token
// M - 1: their products reach only accumulator rows that are never stored).
// A wave's work is the list of (tile, batch) items; item i + 1 is loaded
// into the other of two register sets while item i is computed, across tile
// boundaries, so the codes of the next tile are in flight during the
// reduction of the current one. Loads are whole-wave vector loads:
//  * codes straight into registers: lane (r, c) takes quarter c of each group
//    of row r (the k-slot order of the kernel above), so one instruction
//    reads 16 rows x GB contiguous bytes and an item is 4 KB per row tile;
//  * the row's GPB scales as one load and its GPB zeros as one (the layer
//    has a whole number of batches per row, ng % GPB == 0, and the scale and
//    zero arrays are aligned to GPB entries).
// A tile ends with the waves' partial tiles added in wave order through LDS
// (double-buffered: one barrier per tile).
// ---------------------------------------------------------------------------
template <int BITS, int G>
struct DecBatch {
    static constexpr int GB = G * BITS / 8;                     // bytes of one group of one row
    static constexpr int QB = GB / 4;                           // bytes of a lane's quarter
    static constexpr int WPL = QB / 4;                          // code words per lane per group
    static constexpr int GPB = 4 * GB <= 256 ? 4 : 256 / GB;    // groups per batch
};
constexpr int kDecM = 4;                    // tokens
constexpr int kDecXBytes = 64 * 1024;       // LDS for X: M (2 in + 16) bytes at most

// The codes of one group of one lane as (code - zero) operands; the zero is
// byte j of zw. fp16: a mask-and-or turns two codes 16 bits apart into the
// fp16 pair 1024 + c (bits 0-3 of each half) or 1024 + 16 c (bits 4-7); one
// packed fp16 subtraction of 1024 + zero, or fma with 1/16 and -(64 +
// zero), leaves the exact small integers (every intermediate is exact).
// Pairs come out in the order F16Pairs::PERM. With 4-bit codes (zero < 16)
// both constants are bit patterns: 1024 + z is 0x6400 | z and -(64 + z) is
// 0xD400 | z << 4, built from the zero byte copied into both halves.
template <typename TX, int BITS, int G>
__device__ __forceinline__ void dec_operands(const uint32_t *wv, uint32_t zw, int j,
                                             typename QOp<TX>::vec (&b)[G / 32])
{
    constexpr int STEPS = G / 32;
    constexpr uint32_t cmask = (1u << BITS) - 1u;
    const int zero = (int)((zw >> (8 * j)) & 0xFFu);
    if constexpr (std::is_same<TX, f16>::value && BITS == 4) {
        // byte j of zw into bytes 0 and 2, zeros elsewhere (selector 0x0C)
        const uint32_t zrep = __builtin_amdgcn_perm(zw, 0u, 0x0C000C00u | (uint32_t)(4 + j) << 16 | (uint32_t)(4 + j));
        const f16x2 z1 = __builtin_bit_cast(f16x2, zrep | 0x64006400u);
        const f16x2 z16 = __builtin_bit_cast(f16x2, (zrep << 4) | 0xD400D400u);
        const f16x2 sixteenth = {static_cast<f16>(0.0625f), static_cast<f16>(0.0625f)};
        const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = 0x64006400u;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const uint32_t w = wv[s], w8 = w >> 8;
            const f16x2 d0 = __builtin_bit_cast(f16x2, and_or(w, m_lo, magic)) - z1;
            const f16x2 d1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, and_or(w, m_hi, magic)),
                                                       sixteenth, z16);
            const f16x2 d2 = __builtin_bit_cast(f16x2, and_or(w8, m_lo, magic)) - z1;
            const f16x2 d3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, and_or(w8, m_hi, magic)),
                                                       sixteenth, z16);
            b[s][0] = d0[0]; b[s][1] = d0[1];
            b[s][2] = d1[0]; b[s][3] = d1[1];
            b[s][4] = d2[0]; b[s][5] = d2[1];
            b[s][6] = d3[0]; b[s][7] = d3[1];
        }
    } else if constexpr (std::is_same<TX, f16>::value) {
        const f16 zb = static_cast<f16>(1024 + zero);                  // exact: at most 1279
        const f16x2 z2 = {zb, zb};
        const uint32_t mask = F16Pairs<BITS>::kMask, magic = 0x64006400u;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            uint32_t u[4];
            F16Pairs<BITS>::make(&wv[s * BITS / 4], u, mask, magic);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f16x2 d = __builtin_bit_cast(f16x2, u[p]) - z2;   // exact
                b[s][2 * p] = d[0];
                b[s][2 * p + 1] = d[1];
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = 8 * s + e;
                const int code = (int)((wv[(k * BITS) / 32] >> ((k * BITS) % 32)) & cmask);
                b[s][e] = static_cast<TX>(static_cast<float>(code - zero));   // exact
            }
    }
}

template <int BITS, int G>
struct DecRegs {
    typedef DecBatch<BITS, G> D;
    typedef float scv __attribute__((ext_vector_type(D::GPB)));
    uint32_t wv[D::GPB][D::WPL];
    scv sc;
    uint32_t zw;                                                // GPB zero bytes
};

template <int BITS, int G>
bool qgemv_applies(int64_t M, int64_t in, const float *scales, const uint8_t *zeros)
{
    typedef DecBatch<BITS, G> D;
    return M <= kDecM && M * (2 * in + 16) <= kDecXBytes && (in / G) % D::GPB == 0 &&
           ((uintptr_t)scales % (4 * D::GPB)) == 0 && ((uintptr_t)zeros % D::GPB) == 0;
}

template <typename TX, int BITS, int G, bool YF32>
__global__ __launch_bounds__(kQWaves * 64) void k_qgemv(const TX *__restrict__ X, int64_t M, int64_t in,
                                                        const uint32_t *__restrict__ qweight,
                                                        const float *__restrict__ scales,
                                                        const uint8_t *__restrict__ zeros, int64_t out,
                                                        void *__restrict__ Y)
{
    typedef DecBatch<BITS, G> D;
    typedef typename QOp<TX>::vec vec;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef DecRegs<BITS, G> R;
    constexpr int STEPS = G / 32, GPB = D::GPB, WPL = D::WPL;
    constexpr bool kPairs = std::is_same<TX, f16>::value;
    extern __shared__ __align__(16) uint8_t dyn_lds[];          // X: M rows of 2 in + 16 bytes
    __shared__ __align__(16) f32x4 red[2][kQWaves][16];

    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index as a scalar: the item bookkeeping and its branches are
    // then uniform (scalar registers, no exec-masked paths)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, c = lane >> 4;
    const int64_t ng = in / G, nb = ng / GPB;
    const int64_t row_bytes = in * BITS / 8;
    const int64_t ntiles = (out + 15) / 16;
    const int64_t xrow = 2 * in + 16;
    const uint8_t *qb = reinterpret_cast<const uint8_t *>(qweight);

    // a wave's items: (tile, batch) for its tiles blockIdx.x + i gridDim.x
    // and its batches wave + 8 j; the next item is the next batch of the
    // tile or the first batch of the next tile
    const int nw = nb < kQWaves ? (int)nb : kQWaves;            // waves with batches
    auto advance = [&](int64_t &tile, int64_t &b) {
        b += kQWaves;
        if (b >= nb) {
            b = wave;
            tile += gridDim.x;
        }
    };

    // Tile t covers rows base(t) .. base(t) + 15 with base(t) = 16 t, the last
    // tile moved back to end at row out - 1 (it stores only rows past 16 t,
    // the earlier ones belong to the tile before). A lane's offsets from the
    // tile's first row are then the same in every tile: the per-item
    // addresses are a scalar base plus these.
    const int64_t last_base = out > 16 ? out - 16 : 0;
    const int reff = out >= 16 ? r : (r < out ? r : (int)out - 1);
    const uint32_t q_off = (uint32_t)(reff * row_bytes + c * D::QB);
    const uint32_t s_off = (uint32_t)(reff * ng);
    auto row_base = [&](int64_t tile) { return tile * 16 < last_base ? tile * 16 : last_base; };

    auto fetch = [&](R &rg, int64_t tile, int64_t b) {
        const int64_t g0 = b * GPB, n0 = row_base(tile);
        const uint8_t *qrow = qb + n0 * row_bytes + g0 * D::GB + q_off;
#pragma unroll
        for (int j = 0; j < GPB; ++j) {
            const uint8_t *src = qrow + j * D::GB;
            if constexpr (WPL % 4 == 0) {
#pragma unroll
                for (int q = 0; q < WPL / 4; ++q) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 16 * q);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        rg.wv[j][4 * q + e] = v[e];
                }
            } else if constexpr (WPL == 2) {
                const u32x2 v = *reinterpret_cast<const u32x2 *>(src);
                rg.wv[j][0] = v[0];
                rg.wv[j][1] = v[1];
            } else {
                rg.wv[j][0] = *reinterpret_cast<const uint32_t *>(src);
            }
        }
        rg.sc = *reinterpret_cast<const typename R::scv *>(scales + n0 * ng + g0 + s_off);
        if constexpr (GPB == 4)
            rg.zw = *reinterpret_cast<const uint32_t *>(zeros + n0 * ng + g0 + s_off);
        else
            rg.zw = *reinterpret_cast<const uint16_t *>(zeros + n0 * ng + g0 + s_off);
    };

    const int mr = r < M ? r : (int)M - 1;
    const uint8_t *xlane = dyn_lds + mr * xrow + c * (G / 4) * 2;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const R &cur, int64_t b) {
        const uint8_t *xw = xlane + b * GPB * G * 2;
#pragma unroll
        for (int j = 0; j < GPB; ++j) {
            vec xs[STEPS];
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
                xs[s] = *reinterpret_cast<const vec *>(xw + (j * G + 8 * s) * 2);
            vec bop[STEPS];
            dec_operands<TX, BITS, G>(cur.wv[j], cur.zw, j, bop);
            f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
                part = QOp<TX>::mfma(xs[s], bop[s], part);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = fmaf(cur.sc[j], part[i], acc[i]);
        }
    };
    // The end of a tile: the partial tiles to LDS, one barrier, wave 0 adds
    // them in wave order and stores. Lane l, register i holds token
    // 4 (l / 16) + i of row l % 16, so with at most 4 tokens only lanes 0-15
    // hold results.
    int par = 0;
    auto tile_done = [&](int64_t tile) {
        if (wave < nw && lane < 16)
            red[par][wave][lane] = acc;
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
        if (wave == 0 && lane < 16) {
            f32x4 sum = red[par][0][lane];
            for (int w = 1; w < nw; ++w)
                sum += red[par][w][lane];
            const int64_t nn = row_base(tile) + r;
#pragma unroll
            for (int i = 0; i < kDecM; ++i) {
                if (i < M && nn < out && nn >= tile * 16) {
                    if (YF32)
                        static_cast<float *>(Y)[i * out + nn] = sum[i];
                    else
                        static_cast<TX *>(Y)[i * out + nn] = static_cast<TX>(sum[i]);
                }
            }
        }
        par ^= 1;
    };

    R ra, rb;
    const bool busy = wave < nb;
    if (busy)
        fetch(ra, blockIdx.x, wave);                            // in flight while X is staged
    // X into LDS: 16-byte pieces, permuted into the code pairs' order
    for (int64_t p = tid; p < M * in / 8; p += kQWaves * 64) {
        const int64_t m = p / (in / 8), k8 = p % (in / 8);
        u32x4 v = *reinterpret_cast<const u32x4 *>(X + m * in + 8 * k8);
        if constexpr (kPairs) {
            constexpr const int *P = F16Pairs<BITS>::PERM;
            const vec a = __builtin_bit_cast(vec, v);
            v = __builtin_bit_cast(u32x4, __builtin_shufflevector(a, a, P[0], P[1], P[2], P[3], P[4], P[5], P[6],
                                                                  P[7]));
        }
        *reinterpret_cast<u32x4 *>(dyn_lds + m * xrow + 16 * k8) = v;
    }
    __syncthreads();
    if (!busy) {
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x)
            tile_done(tile);
        return;
    }
    // The next item is loaded into the other register set while this one is
    // computed. No copies between the sets (a copy would wait for the loads
    // in flight), and the computation is repeated on the paths with and
    // without a load behind it, so that each waits for its own item's loads
    // only; the empty asm statements differ so that the compiler does not
    // merge the two paths' last instructions after the join.
    int64_t tile = blockIdx.x, b = wave;
    int64_t ntile = tile, nbt = b;
    advance(ntile, nbt);
    while (true) {
        if (ntile < ntiles) {
            fetch(rb, ntile, nbt);
            __builtin_amdgcn_sched_barrier(0);      // the loads go out before the computation
            consume(ra, b);
            asm volatile("; item a, next in flight" : "+v"(acc));
        } else {
            consume(ra, b);
            asm volatile("; item a, last" : "+v"(acc));
        }
        if (ntile != tile)
            tile_done(tile);
        if (ntile >= ntiles)
            break;
        tile = ntile, b = nbt;
        advance(ntile, nbt);
        if (ntile < ntiles) {
            fetch(ra, ntile, nbt);
            __builtin_amdgcn_sched_barrier(0);      // the loads go out before the computation
            consume(rb, b);
            asm volatile("; item b, next in flight" : "+v"(acc));
        } else {
            consume(rb, b);
            asm volatile("; item b, last" : "+v"(acc));
        }
        if (ntile != tile)
            tile_done(tile);
        if (ntile >= ntiles)
            break;
        tile = ntile, b = nbt;
        advance(ntile, nbt);
    }
}

// Blocks of the persistent decode grid: as many as fit on the device at once.
template <typename K>
static unsigned qgemv_grid(K kernel, size_t lds, int64_t ntiles)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kQWaves * 64, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1, cus = cus > 0 ? cus : 256;
    // (measured: fewer blocks with an equal number of tiles each are slower
    // than all that fit; the extra loads in flight outweigh the uneven tail)
    const int64_t fit = (int64_t)cus * per_cu;
    return (unsigned)(ntiles < fit ? ntiles : fit);
}

// ---------------------------------------------------------------------------
// Prefill (many tokens): one block = 64 tokens x 128 output rows over all of
// K, wave w taking rows 16 w .. +15 for all four 16-token tiles. K runs in
// chunks of 128 columns: X (64 x 128) and the packed codes of the 128 rows
// (plus their scales and zeros) are loaded into registers one chunk ahead and
// staged through LDS (double-buffered, one barrier per chunk; fp16 X is
// stored already in the operand order of the code pairs); each wave builds
// the (code - zero) operands of its row tile from the staged codes exactly as
// the decode kernel does and multiplies them with the X fragments of the four
// token tiles, one group at a time, each group's fp32 sums scaled once into
// the totals. Every staged X value serves 128 rows and every built operand 64
// tokens.
// ---------------------------------------------------------------------------
constexpr int kPfM = 64, kPfN = 128, kPfK = 128;

template <int BITS>
struct PfStage {
    static constexpr int XROW = kPfK * 2 + 16;                  // LDS bytes per token row (padded)
    static constexpr int XB = kPfM * XROW;
    static constexpr int CRB = kPfK * BITS / 8;                 // code bytes of one row in a chunk
    static constexpr int CROW = CRB + 16;
    static constexpr int CB = kPfN * CROW;
    static constexpr int NGMAX = kPfK / 32;                     // groups per chunk at most
    static constexpr int BUF = XB + CB + kPfN * NGMAX * 4 + kPfN * NGMAX;
    static constexpr int XCH = kPfM * kPfK * 2 / 16 / (kQWaves * 64);   // 16-byte X chunks per thread (2)
    static constexpr int CCH = kPfN * CRB / 16 / (kQWaves * 64);        // 16-byte code chunks per thread
};

template <typename TX, int BITS, int G, bool YF32>
__global__ __launch_bounds__(kQWaves * 64) void k_qgemm_pf(const TX *__restrict__ X, int64_t M, int64_t in,
                                                           const uint32_t *__restrict__ qweight,
                                                           const float *__restrict__ scales,
                                                           const uint8_t *__restrict__ zeros, int64_t out,
                                                           void *__restrict__ Y)
{
    typedef PfStage<BITS> S;
    typedef typename QOp<TX>::vec vec;
    constexpr int GPC = kPfK / G;               // groups per chunk
    constexpr int STEPS = G / 32;
    constexpr int GB = G * BITS / 8;            // code bytes of one group of one row
    constexpr int WPL = G * BITS / 128;         // code words per lane per group
    constexpr uint32_t cmask = (1u << BITS) - 1u;
    constexpr bool kPairs = std::is_same<TX, f16>::value;
    __shared__ __align__(16) uint8_t lds[2 * S::BUF];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, c = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * kPfM, n0 = (int64_t)blockIdx.x * kPfN;
    const int64_t ng = in / G, row_bytes = in * BITS / 8;
    const int64_t chunks = in / kPfK;
    const uint8_t *qbytes = reinterpret_cast<const uint8_t *>(qweight);

    // registers of the chunk in flight (rows and tokens past the end load the
    // last row/token; their results are never stored)
    u32x4 xr[S::XCH], cr[S::CCH];
    float sr = 0.f;
    uint8_t zr = 0;
    auto fetch = [&](int64_t kc) {
#pragma unroll
        for (int i = 0; i < S::XCH; ++i) {
            const int ch = tid + i * kQWaves * 64;
            int64_t m = m0 + ch / (kPfK * 2 / 16);
            m = m < M ? m : M - 1;
            xr[i] = *reinterpret_cast<const u32x4 *>(X + m * in + kc * kPfK + (ch % (kPfK * 2 / 16)) * 8);
        }
#pragma unroll
        for (int i = 0; i < S::CCH; ++i) {
            const int ch = tid + i * kQWaves * 64;
            int64_t n = n0 + ch / (S::CRB / 16);
            n = n < out ? n : out - 1;
            cr[i] = *reinterpret_cast<const u32x4 *>(qbytes + n * row_bytes + kc * S::CRB + (ch % (S::CRB / 16)) * 16);
        }
        if (tid < kPfN * GPC) {
            int64_t n = n0 + tid / GPC;
            n = n < out ? n : out - 1;
            sr = scales[n * ng + kc * GPC + tid % GPC];
            zr = zeros[n * ng + kc * GPC + tid % GPC];
        }
    };
    auto stash = [&](uint8_t *buf) {
#pragma unroll
        for (int i = 0; i < S::XCH; ++i) {
            const int ch = tid + i * kQWaves * 64;
            u32x4 v = xr[i];
            if constexpr (kPairs) {
                // a 16-byte chunk is one operand's 8 columns: store them in
                // the order the code pairs come out in
                constexpr const int *P = F16Pairs<BITS>::PERM;
                const vec a = __builtin_bit_cast(vec, v);
                v = __builtin_bit_cast(u32x4, __builtin_shufflevector(a, a, P[0], P[1], P[2], P[3], P[4], P[5],
                                                                      P[6], P[7]));
            }
            *reinterpret_cast<u32x4 *>(buf + (ch / (kPfK * 2 / 16)) * S::XROW + (ch % (kPfK * 2 / 16)) * 16) = v;
        }
#pragma unroll
        for (int i = 0; i < S::CCH; ++i) {
            const int ch = tid + i * kQWaves * 64;
            *reinterpret_cast<u32x4 *>(buf + S::XB + (ch / (S::CRB / 16)) * S::CROW + (ch % (S::CRB / 16)) * 16) = cr[i];
        }
        if (tid < kPfN * GPC) {
            reinterpret_cast<float *>(buf + S::XB + S::CB)[tid] = sr;
            (buf + S::XB + S::CB + kPfN * S::NGMAX * 4)[tid] = zr;
        }
    };

    f32x4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    fetch(0);
    stash(lds);
    __syncthreads();
    for (int64_t kc = 0; kc < chunks; ++kc) {
        const uint8_t *buf = lds + (kc & 1) * S::BUF;
        if (kc + 1 < chunks)
            fetch(kc + 1);
        const float *sbuf = reinterpret_cast<const float *>(buf + S::XB + S::CB);
        const uint8_t *zbuf = buf + S::XB + S::CB + kPfN * S::NGMAX * 4;
        const int row = wave * 16 + r;
#pragma unroll
        for (int gq = 0; gq < GPC; ++gq) {
            // B operands of this wave's row tile for group gq of the chunk
            uint32_t wv[WPL];
            const uint8_t *src = buf + S::XB + row * S::CROW + gq * GB + c * (GB / 4);
            if constexpr (WPL % 4 == 0) {
#pragma unroll
                for (int q = 0; q < WPL / 4; ++q) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 16 * q);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        wv[4 * q + e] = v[e];
                }
            } else if constexpr (WPL == 2) {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 v = *reinterpret_cast<const u32x2 *>(src);
                wv[0] = v[0];
                wv[1] = v[1];
            } else {
                wv[0] = *reinterpret_cast<const uint32_t *>(src);
            }
            const float scale = sbuf[row * GPC + gq];
            const int zero = zbuf[row * GPC + gq];
            vec b[STEPS];
            if constexpr (kPairs) {
                const f16 zb = static_cast<f16>(1024 + zero);           // exact: at most 1279
                const f16x2 z2 = {zb, zb};
                const uint32_t mask = F16Pairs<BITS>::kMask, magic = 0x64006400u;
#pragma unroll
                for (int st = 0; st < STEPS; ++st) {
                    uint32_t u[4];
                    F16Pairs<BITS>::make(&wv[st * BITS / 4], u, mask, magic);
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const f16x2 d = __builtin_bit_cast(f16x2, u[p]) - z2;   // exact
                        b[st][2 * p] = d[0];
                        b[st][2 * p + 1] = d[1];
                    }
                }
            } else {
#pragma unroll
                for (int st = 0; st < STEPS; ++st)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = 8 * st + e;
                        const int code = (int)((wv[(j * BITS) / 32] >> ((j * BITS) % 32)) & cmask);
                        b[st][e] = static_cast<TX>(static_cast<float>(code - zero));   // exact
                    }
            }
            // the four token tiles: X fragments from LDS (the same k-slot order)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int tok = mt * 16 + r;
                const uint8_t *xp = buf + tok * S::XROW + (gq * G + c * (G / 4)) * 2;
                f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < STEPS; ++st)
                    part = QOp<TX>::mfma(*reinterpret_cast<const vec *>(xp + 16 * st), b[st], part);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[mt][i] = fmaf(scale, part[i], acc[mt][i]);
            }
        }
        if (kc + 1 < chunks)
            stash(lds + ((kc + 1) & 1) * S::BUF);
        __syncthreads();
    }
    const int64_t nn = n0 + wave * 16 + r;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + mt * 16 + 4 * c + i;
            if (m < M && nn < out) {
                if (YF32)
                    static_cast<float *>(Y)[m * out + nn] = acc[mt][i];
                else
                    static_cast<TX *>(Y)[m * out + nn] = static_cast<TX>(acc[mt][i]);
            }
        }
}

// ---------------------------------------------------------------------------
// Prefill with 32 x 32 x 16 MFMAs: one block = 64 tokens x 256 output rows
// over all of K, wave w taking rows 32 w .. +31 for both 32-token tiles, so
// every staged X fragment serves 32 rows (half the LDS reads per product of
// the 16 x 16 tile above). A = X (lane l: token l % 32), B = the (code -
// zero) operands (lane l: row l % 32), so a lane's 16 results all belong to
// one output row and take one group scale. MFMA step s of a group covers
// its 16 columns 16 s .. 16 s + 15, lanes 0-31 the first eight, lanes 32-63
// the last eight: a step never straddles a group. The codes of each row and
// group are staged with the 8-code units of the two lane halves made
// contiguous (even units first, then odd ones).
// ---------------------------------------------------------------------------
constexpr int kP2M = 64, kP2N = 256, kP2K = 128;
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename TX> struct QOp32;
template <> struct QOp32<f16> {
    static __device__ __forceinline__ f32x16 mfma(const f16x8 &a, const f16x8 &b, const f32x16 &c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct QOp32<bf16> {
    static __device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <int BITS, int RT>
struct P2Stage {
    static constexpr int N = kP2N * RT;                         // rows per block
    static constexpr int XROW = kP2K * 2 + 16;                  // LDS bytes per token row (padded)
    static constexpr int XB = kP2M * XROW;
    static constexpr int CRB = kP2K * BITS / 8;                 // code bytes of one row in a chunk
    static constexpr int CROW = CRB + 16;
    static constexpr int CB = N * CROW;
    static constexpr int NGMAX = kP2K / 32;
    static constexpr int BUF = XB + CB + N * NGMAX * 4 + N * NGMAX;
    static constexpr int XCH = kP2M * kP2K * 2 / 16 / (kQWaves * 64);   // 16-byte X chunks per thread (2)
    static constexpr int CCH = N * CRB / 16 / (kQWaves * 64);           // 16-byte code chunks per thread
    static constexpr int SZ = (N * NGMAX + kQWaves * 64 - 1) / (kQWaves * 64);   // scales per thread
};

// RT: 32-row tiles per wave (the block has 256 RT rows); with RT = 2 each
// X fragment read from LDS serves 64 rows.
template <typename TX, int BITS, int G, bool YF32, int RT>
__global__ __launch_bounds__(kQWaves * 64) void k_qgemm_pf32(const TX *__restrict__ X, int64_t M, int64_t in,
                                                             const uint32_t *__restrict__ qweight,
                                                             const float *__restrict__ scales,
                                                             const uint8_t *__restrict__ zeros, int64_t out,
                                                             void *__restrict__ Y)
{
    typedef P2Stage<BITS, RT> S;
    typedef typename QOp<TX>::vec vec;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int GPC = kP2K / G;               // groups per chunk
    constexpr int STEPS = G / 16;               // 16-column MFMA steps per group
    constexpr int GB = G * BITS / 8;            // code bytes of one group of one row
    constexpr int UB = BITS;                    // bytes of one 8-code unit
    constexpr int UPG = G / 8;                  // units per group
    constexpr uint32_t cmask = (1u << BITS) - 1u;
    constexpr bool kPairs = std::is_same<TX, f16>::value;
    __shared__ __align__(16) uint8_t lds[2 * S::BUF];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, kh = lane >> 5;
    const int64_t m0 = (int64_t)blockIdx.y * kP2M, n0 = (int64_t)blockIdx.x * S::N;
    const int64_t ng = in / G, row_bytes = in * BITS / 8;
    const int64_t chunks = in / kP2K;
    const uint8_t *qbytes = reinterpret_cast<const uint8_t *>(qweight);

    u32x4 xr[S::XCH], cr[S::CCH];
    float sr[S::SZ];
    uint8_t zr[S::SZ];
    auto fetch = [&](int64_t kc) {
#pragma unroll
        for (int i = 0; i < S::XCH; ++i) {
            const int ch = tid + i * kQWaves * 64;
            int64_t m = m0 + ch / (kP2K * 2 / 16);
            m = m < M ? m : M - 1;
            xr[i] = *reinterpret_cast<const u32x4 *>(X + m * in + kc * kP2K + (ch % (kP2K * 2 / 16)) * 8);
        }
#pragma unroll
        for (int i = 0; i < S::CCH; ++i) {
            const int ch = tid + i * kQWaves * 64;
            int64_t n = n0 + ch / (S::CRB / 16);
            n = n < out ? n : out - 1;
            cr[i] = *reinterpret_cast<const u32x4 *>(qbytes + n * row_bytes + kc * S::CRB + (ch % (S::CRB / 16)) * 16);
        }
#pragma unroll
        for (int i = 0; i < S::SZ; ++i) {
            const int e = tid + i * kQWaves * 64;
            if (e < S::N * GPC) {
                int64_t n = n0 + e / GPC;
                n = n < out ? n : out - 1;
                sr[i] = scales[n * ng + kc * GPC + e % GPC];
                zr[i] = zeros[n * ng + kc * GPC + e % GPC];
            }
        }
    };
    auto stash = [&](uint8_t *buf) {
#pragma unroll
        for (int i = 0; i < S::XCH; ++i) {
            const int ch = tid + i * kQWaves * 64;
            u32x4 v = xr[i];
            if constexpr (kPairs) {
                constexpr const int *P = F16Pairs<BITS>::PERM;
                const vec a = __builtin_bit_cast(vec, v);
                v = __builtin_bit_cast(u32x4, __builtin_shufflevector(a, a, P[0], P[1], P[2], P[3], P[4], P[5],
                                                                      P[6], P[7]));
            }
            *reinterpret_cast<u32x4 *>(buf + (ch / (kP2K * 2 / 16)) * S::XROW + (ch % (kP2K * 2 / 16)) * 16) = v;
        }
        // a 16-byte piece holds 16 / UB units starting at an even unit: the
        // even ones go to the group's first half, the odd ones to its second
#pragma unroll
        for (int i = 0; i < S::CCH; ++i) {
            const int ch = tid + i * kQWaves * 64;
            const int row = ch / (S::CRB / 16);
            const int u0 = (ch % (S::CRB / 16)) * (16 / UB);       // first unit of the piece in the chunk row
            const int gq = u0 / UPG, ug = u0 % UPG;
            uint8_t *dst = buf + S::XB + row * S::CROW + gq * GB;
            const u32x4 v = cr[i];
            if constexpr (UB == 4) {
                *reinterpret_cast<u32x2 *>(dst + (ug >> 1) * UB) = u32x2{v[0], v[2]};
                *reinterpret_cast<u32x2 *>(dst + GB / 2 + (ug >> 1) * UB) = u32x2{v[1], v[3]};
            } else {
                *reinterpret_cast<u32x2 *>(dst + (ug >> 1) * UB) = u32x2{v[0], v[1]};
                *reinterpret_cast<u32x2 *>(dst + GB / 2 + (ug >> 1) * UB) = u32x2{v[2], v[3]};
            }
        }
#pragma unroll
        for (int i = 0; i < S::SZ; ++i) {
            const int e = tid + i * kQWaves * 64;
            if (e < S::N * GPC) {
                reinterpret_cast<float *>(buf + S::XB + S::CB)[e] = sr[i];
                (buf + S::XB + S::CB + S::N * S::NGMAX * 4)[e] = zr[i];
            }
        }
    };

    f32x16 acc[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc[rt][tt][i] = 0.f;
    fetch(0);
    stash(lds);
    __syncthreads();
    for (int64_t kc = 0; kc < chunks; ++kc) {
        const uint8_t *buf = lds + (kc & 1) * S::BUF;
        if (kc + 1 < chunks)
            fetch(kc + 1);
        const float *sbuf = reinterpret_cast<const float *>(buf + S::XB + S::CB);
        const uint8_t *zbuf = buf + S::XB + S::CB + S::N * S::NGMAX * 4;
#pragma unroll
        for (int gq = 0; gq < GPC; ++gq) {
            vec b[RT][STEPS];
            float scale[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int row = (wave * RT + rt) * 32 + l32;
                // this lane half's units of the group: STEPS units of UB bytes
                uint32_t wv[STEPS * UB / 4];
                const uint8_t *src = buf + S::XB + row * S::CROW + gq * GB + kh * (GB / 2);
                if constexpr ((STEPS * UB) % 16 == 0) {
#pragma unroll
                    for (int q = 0; q < STEPS * UB / 16; ++q) {
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 16 * q);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            wv[4 * q + e] = v[e];
                    }
                } else {
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(src);
                    wv[0] = v[0];
                    wv[1] = v[1];
                }
                scale[rt] = sbuf[row * GPC + gq];
                const int zero = zbuf[row * GPC + gq];
                if constexpr (kPairs) {
                    const f16 zb = static_cast<f16>(1024 + zero);           // exact: at most 1279
                    const f16x2 z2 = {zb, zb};
                    const uint32_t mask = F16Pairs<BITS>::kMask, magic = 0x64006400u;
#pragma unroll
                    for (int st = 0; st < STEPS; ++st) {
                        uint32_t u[4];
                        F16Pairs<BITS>::make(&wv[st * UB / 4], u, mask, magic);
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const f16x2 d = __builtin_bit_cast(f16x2, u[p]) - z2;   // exact
                            b[rt][st][2 * p] = d[0];
                            b[rt][st][2 * p + 1] = d[1];
                        }
                    }
                } else {
#pragma unroll
                    for (int st = 0; st < STEPS; ++st)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 8 * st + e;               // code j of the lane's STEPS units
                            const int code = (int)((wv[(j * BITS) / 32] >> ((j * BITS) % 32)) & cmask);
                            b[rt][st][e] = static_cast<TX>(static_cast<float>(code - zero));   // exact
                        }
                }
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                // X of token 32 tt + l32, columns 16 st + 8 kh .. + 7 of the group: one read for RT row tiles
                const uint8_t *xp = buf + (tt * 32 + l32) * S::XROW + (gq * G + 8 * kh) * 2;
                f32x16 part[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        part[rt][i] = 0.f;
#pragma unroll
                for (int st = 0; st < STEPS; ++st) {
                    const vec xa = *reinterpret_cast<const vec *>(xp + 32 * st);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        part[rt] = QOp32<TX>::mfma(xa, b[rt][st], part[rt]);
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[rt][tt][i] = fmaf(scale[rt], part[rt][i], acc[rt][tt][i]);
            }
        }
        if (kc + 1 < chunks)
            stash(lds + ((kc + 1) & 1) * S::BUF);
        __syncthreads();
    }
    // lane l, register i: token 8 (i / 4) + 4 (l / 32) + i % 4 of the tile, row l % 32
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int64_t nn = n0 + (wave * RT + rt) * 32 + l32;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t m = m0 + tt * 32 + 8 * (i / 4) + 4 * kh + (i % 4);
                if (m < M && nn < out) {
                    if (YF32)
                        static_cast<float *>(Y)[m * out + nn] = acc[rt][tt][i];
                    else
                        static_cast<TX *>(Y)[m * out + nn] = static_cast<TX>(acc[rt][tt][i]);
                }
            }
    }
}

template <typename TX, int BITS, int G>
static hipError_t qgemm_mt(const void *X, int64_t M, int64_t in, const uint32_t *qweight,
                           const float *scales, const uint8_t *zeros, int64_t out, void *Y, bool yf32,
                           hipStream_t st)
{
    const dim3 block(kQWaves * 64);
    // two 32-row tiles per wave in the 32 x 32 prefill tile: 4-bit codes in
    // groups of 128 only (other widths and groups exceed the LDS or spill)
    constexpr bool kPf32x2 = BITS == 4 && G == 128;
    const bool pf32x2 = kPf32x2;
    // decode up to 4 tokens (whole batches per row, aligned scales and
    // zeros): direct loads, 16 rows per block, or 32 on layers with at least
    // 8192 rows. Otherwise up to 16 tokens: 16 tokens and 16 rows per block,
    // or 32 rows on layers with at least 8192 rows (twice the bytes staged per
    // round; enough blocks remain to fill the chip). Beyond 64 tokens, with in a multiple of 128,
    // the first prefill tile that gives at least one block per compute unit:
    // 32 x 32 MFMAs with 64 tokens x 512 rows (4-bit codes in groups of 128),
    // then 64 x 256, then the 16 x 16 tile with 64 x 128. Otherwise split
    // over K inside the block, 16 tokens x 32 rows up to 32 tokens, 16 x 64
    // up to 64 and 32 x 64 beyond (measured: the smaller tiles win while
    // their extra blocks still fit the chip at once).
#define AWQ_QGEMM(MT, NT, YF)                                                                        \
    hipLaunchKernelGGL((k_qgemm<TX, BITS, G, MT, NT, YF>),                                            \
                       dim3((unsigned)((out + 16 * NT - 1) / (16 * NT)),                             \
                            (unsigned)((M + 16 * MT - 1) / (16 * MT))),                              \
                       block, 0, st, (const TX *)X, M, in, qweight, scales, zeros, out, Y)
#define AWQ_QGEMV(YF)                                                                                \
    do {                                                                                             \
        const size_t lds = (size_t)(M * (2 * in + 16));                                              \
        auto k = k_qgemv<TX, BITS, G, YF>;                                                           \
        hipLaunchKernelGGL(k, dim3(qgemv_grid(k, lds, (out + 15) / 16)), block, lds, st, (const TX *)X, M, in, \
                           qweight, scales, zeros, out, Y);                                          \
    } while (0)
    const bool gemv = qgemv_applies<BITS, G>(M, in, scales, zeros);
    if (gemv) {
        if (yf32) AWQ_QGEMV(true); else AWQ_QGEMV(false);
    } else if (M <= 16 && out < 8192) {
        if (yf32) AWQ_QGEMM(1, 1, true); else AWQ_QGEMM(1, 1, false);
    } else if (M <= 16) {
        if (yf32) AWQ_QGEMM(1, 2, true); else AWQ_QGEMM(1, 2, false);
    } else if (M <= 32) {
        if (yf32) AWQ_QGEMM(1, 2, true); else AWQ_QGEMM(1, 2, false);
    } else if (M <= 64) {
        if (yf32) AWQ_QGEMM(1, 4, true); else AWQ_QGEMM(1, 4, false);
    } else if (pf32x2 && in % kP2K == 0 && ((out + 2 * kP2N - 1) / (2 * kP2N)) * ((M + kP2M - 1) / kP2M) >= 256) {
        if constexpr (kPf32x2) {
            const dim3 grid((unsigned)((out + 2 * kP2N - 1) / (2 * kP2N)), (unsigned)((M + kP2M - 1) / kP2M));
            if (yf32)
                hipLaunchKernelGGL((k_qgemm_pf32<TX, BITS, G, true, 2>), grid, block, 0, st, (const TX *)X, M, in,
                                   qweight, scales, zeros, out, Y);
            else
                hipLaunchKernelGGL((k_qgemm_pf32<TX, BITS, G, false, 2>), grid, block, 0, st, (const TX *)X, M,
                                   in, qweight, scales, zeros, out, Y);
        }
    } else if (in % kP2K == 0 && ((out + kP2N - 1) / kP2N) * ((M + kP2M - 1) / kP2M) >= 256) {
        const dim3 grid((unsigned)((out + kP2N - 1) / kP2N), (unsigned)((M + kP2M - 1) / kP2M));
        if (yf32)
            hipLaunchKernelGGL((k_qgemm_pf32<TX, BITS, G, true, 1>), grid, block, 0, st, (const TX *)X, M, in,
                               qweight, scales, zeros, out, Y);
        else
            hipLaunchKernelGGL((k_qgemm_pf32<TX, BITS, G, false, 1>), grid, block, 0, st, (const TX *)X, M, in,
                               qweight, scales, zeros, out, Y);
    } else if (in % kPfK != 0 || ((out + kPfN - 1) / kPfN) * ((M + kPfM - 1) / kPfM) < 256) {
        if (yf32) AWQ_QGEMM(2, 4, true); else AWQ_QGEMM(2, 4, false);
    } else {
        const dim3 grid((unsigned)((out + kPfN - 1) / kPfN), (unsigned)((M + kPfM - 1) / kPfM));
        if (yf32)
            hipLaunchKernelGGL((k_qgemm_pf<TX, BITS, G, true>), grid, block, 0, st, (const TX *)X, M, in, qweight,
                               scales, zeros, out, Y);
        else
            hipLaunchKernelGGL((k_qgemm_pf<TX, BITS, G, false>), grid, block, 0, st, (const TX *)X, M, in, qweight,
                               scales, zeros, out, Y);
    }
#undef AWQ_QGEMM
#undef AWQ_QGEMV
    return hipGetLastError();
}

template <typename TX, int BITS>
static hipError_t qgemm_g(const void *X, int64_t M, int64_t in, const uint32_t *qweight,
                          const float *scales, const uint8_t *zeros, int64_t out, int group, void *Y,
                          bool yf32, hipStream_t st)
{
    switch (group) {
    case 32: return qgemm_mt<TX, BITS, 32>(X, M, in, qweight, scales, zeros, out, Y, yf32, st);
    case 64: return qgemm_mt<TX, BITS, 64>(X, M, in, qweight, scales, zeros, out, Y, yf32, st);
    default: return qgemm_mt<TX, BITS, 128>(X, M, in, qweight, scales, zeros, out, Y, yf32, st);
    }
}

hipError_t launch_qgemm(const void *X, int dtype, int64_t M, int64_t in, const uint32_t *qweight,
                        const float *scales, const uint8_t *zeros, int64_t out, int bits, int group,
                        void *Y, bool yf32, hipStream_t st)
{
    if (dtype == AWQ_F16)
        return bits == 4 ? qgemm_g<f16, 4>(X, M, in, qweight, scales, zeros, out, group, Y, yf32, st)
                         : qgemm_g<f16, 8>(X, M, in, qweight, scales, zeros, out, group, Y, yf32, st);
    return bits == 4 ? qgemm_g<bf16, 4>(X, M, in, qweight, scales, zeros, out, group, Y, yf32, st)
                     : qgemm_g<bf16, 8>(X, M, in, qweight, scales, zeros, out, group, Y, yf32, st);
}

}  // namespace awq
