// HIP kernels for gfx950 (MI355X): the e4m3 latent-row quantizer, the split-T
// partial attention kernel and the log-sum-exp merge.
//
// Method sources (page, passage):
//   colibri PR #300 "KV8 long-context CUDA: fp8 device shadow, split-T kernels,
//   DSA-aware gather" -- first commit ("KV8 base"), c/kv_fp8.h bullet: RNE
//   e4m3 encoder saturating at +/-448, signed zero kept, NaN stored as 0, per-row
//   quantizer (scale amax/448) with a subnormal-amax guard; attention_rows
//   bullet: the latent is both key and value and the row scale is hoisted out of
//   the dot.  Second commit ("KV8 long-context CUDA"): split-T blocks emitting
//   online-softmax partials (cl[K], m, z), a log-sum-exp merge kernel, and the
//   DSA gather over absolute row indices.
//
// gfx950 design (what differs from the page's CUDA kernels is deliberate):
//   * One workgroup owns a chunk of rows and 32 query-heads, so every row is
//     read from HBM once for all its heads; workgroups sharing a chunk are
//     placed on the same XCD so the second head group hits that XCD's L2.
//   * Rows are staged through LDS in 64-row tiles.  e4m3 bytes are widened to
//     fp16 in registers with v_cvt_scalef32_pk_f16_fp8 (exact: every e4m3 value
//     is an fp16 normal), then fed to v_mfma_f32_16x16x32_f16.
//   * Scores S^T[row][head] = X . Q^T: each wave takes 16 rows x 32 heads; q is
//     resident in registers as an fp16 hi/lo pair (two MFMA passes), scaled by
//     a power of two per head so it sits in fp16's range.
//   * Context O[head][col] += W . X: each wave owns a 128-column slice, reading
//     an 8x8 byte block per lane and transposing it with v_perm_b32 so the row
//     (contraction) index becomes the per-lane MFMA K index.
//   * The row scale is hoisted: scores are (q . code) * scale_t, and the PV
//     weight of row t is exp2(u_t + log2 scale_t - mo) with its own running max
//     mo, so fp16 weights never overflow or lose significant rows.
//   * Online softmax with a lazy running max: the max is only moved when a
//     tile beats it by more than 2^8, which keeps rescaling of the register
//     accumulators off the common path.
#include "mla8_internal.h"

#include <math.h>

namespace mla8 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// e4m3 encoder on the f32 bit pattern.  Round-to-nearest-even onto 3 mantissa
// bits, saturation at 448, sign of zero kept, NaN -> 0x00.
__device__ __forceinline__ uint32_t enc_e4m3(float y)
{
    const uint32_t b = __float_as_uint(y);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return 0u;                  // NaN of either sign: inert zero
    if (a >= 0x43E00000u)
        return sign | 0x7Eu;        // |y| >= 448, infinity included
    uint32_t code;
    if (a >= 0x3C800000u) {         // |y| >= 2^-6: e4m3 normal range
        // Drop 20 mantissa bits with round-half-even; a carry out of the kept
        // mantissa moves into the exponent field by itself.
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);  // re-bias the exponent 127 -> 7
    } else {
        // e4m3 subnormals are the multiples of 2^-9 below 2^-6; the product is
        // exact and v_rndne_f32 rounds half to even.  8 -> 0x08 = 2^-6.
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return sign | code;
}

// One wave per row, four rows per workgroup.
__global__ __launch_bounds__(256) void k_quantize_rows(const float* __restrict__ x,
                                                       int64_t n_rows, int32_t d,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n_rows)
        return;
    const float4* xr = reinterpret_cast<const float4*>(x + row * d);
    const int nv = d >> 2;
    float amax = 0.0f;
    for (int i = lane; i < nv; i += 64) {
        const float4 v = xr[i];
        const float e[4] = {fabsf(v.x), fabsf(v.y), fabsf(v.z), fabsf(v.w)};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (e[k] <= 3.402823466e38f)  // finite only: false for NaN and inf
                amax = fmaxf(amax, e[k]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off));
    // IEEE f32 quotients (the library is built with correctly rounded f32
    // division).  The guard: when 448/amax is not finite the row encodes as
    // signed zeros.
    const float scale = amax / 448.0f;
    float inv = 448.0f / amax;
    if (!(inv <= 3.402823466e38f))
        inv = 0.0f;
    uint32_t* cr = reinterpret_cast<uint32_t*>(codes + row * d);
    for (int i = lane; i < nv; i += 64) {
        const float4 v = xr[i];
        cr[i] = enc_e4m3(v.x * inv) | (enc_e4m3(v.y * inv) << 8) | (enc_e4m3(v.z * inv) << 16) |
                (enc_e4m3(v.w * inv) << 24);
    }
    if (lane == 0)
        scales[row] = scale;
}

__global__ __launch_bounds__(256) void k_test_encode(const float* __restrict__ x, int64_t n,
                                                     uint8_t* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = (uint8_t)enc_e4m3(x[i]);
}

// ---------------------------------------------------------------------------
// 8 e4m3 bytes (two dwords, byte 0 first) -> 8 fp16 values, exactly.
// HI selects bytes 2,3 of the dword instead of bytes 0,1.
template <bool HI>
__device__ __forceinline__ f16x2 cvt2(uint32_t v)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, HI);
}

__device__ __forceinline__ f16x8 cvt8(uint32_t lo, uint32_t hi)
{
    const f16x2 a = cvt2<false>(lo), b = cvt2<true>(lo), c = cvt2<false>(hi),
                e = cvt2<true>(hi);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D += A x (B * 2^(sb - 127)), A and B 16x128 / 128x16 OCP e4m3 operands
// (32 bytes per lane), E8M0 scale 127 = 1.0 for A.
__device__ __forceinline__ f32x4 mfma_fp8_scaled(v8i a, v8i b, f32x4 c, int32_t sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kTau = 8.0f;  // lazy-max slack, log2 units: weights stay <= 2^8

// ---------------------------------------------------------------------------
// Split-T partial.  Grid: n_chunks * n_groups workgroups of 256 threads.
// NKB = number of 64-wide blocks of the padded row width (d <= 64 * NKB).
template <int NKB>
__global__ __launch_bounds__(kThreads, 1) void k_split_partial(AttnArgs a)
{
    constexpr int TR = kTileRows;
    constexpr int HG = kHeadsPerGroup;
    constexpr int DP = 64 * NKB;      // padded row width in LDS (>= d, >= roundup(lc, 128))
    constexpr int XS = DP + 16;       // LDS row stride (bytes)
    constexpr int WSS = TR + 8;       // LDS stride of the weight tile (halves)
    constexpr int NKB2 = (NKB + 1) / 2;  // 128-wide blocks for the fp8 pass

    __shared__ __attribute__((aligned(16))) uint8_t xs[2][TR * XS];
    __shared__ float s_scale[2][TR];
    __shared__ float s_lscale[2][TR];
    __shared__ int32_t s_row[2][TR];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[HG * WSS];
    __shared__ float s_red[4][2][HG];
    __shared__ float s_z[4][HG];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;

    // Workgroup -> (chunk, head group).  Dispatch is round-robin over the 8
    // XCDs; keep the head groups of one chunk on one XCD, launched back to back.
    int chunk, grp;
    {
        const int b = blockIdx.x;
        if ((a.n_chunks & 7) == 0) {
            const int x = b & 7, r = b >> 3;
            chunk = (r / a.n_groups) * 8 + x;
            grp = r % a.n_groups;
        } else {
            chunk = b / a.n_groups;
            grp = b % a.n_groups;
        }
    }
    const int qh0 = grp * HG;
    const int c0 = chunk * a.chunk_rows;
    const int c1 = min(a.n_list, c0 + a.chunk_rows);
    const int ntiles = c1 > c0 ? (c1 - c0 + TR - 1) / TR : 0;

    // ---- query registers.  Lane (n, g) holds, for heads qh0 + n + 16*ht, the
    // elements d = 64j + 16g + e (e < 16).  The same assignment of the
    // contraction index to (lane group, operand slot) is used for the row
    // operand, so the MFMA sums the right products whatever its K labels are.
    //   qhi: fp16(q * 2^k)             two f16x8 per (j, ht)   -> fp16 MFMA
    //   qlo: e4m3((q*2^k - qhi) * 2^k') 32 bytes per (j pair, ht) -> fp8 MFMA
    //        with the E8M0 operand scale 2^-k' undoing k' inside the MFMA.
    f16x8 qhi[NKB][2][2];
    v8i qlo[NKB2][2];
    int32_t qlo_scale[2];
    float hfac[2];
    int32_t tlim[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        const int qh = qh0 + 16 * ht + n;
        const bool hv = qh < a.n_qh;
        auto qsrc = [&](int j) -> const float* {
            const int d0 = 64 * j + 16 * g;
            if (hv && d0 < a.lc)
                return a.q_lat + (size_t)qh * a.lc + d0;
            if (hv && d0 < a.d)
                return a.q_rope + (size_t)qh * a.rc + (d0 - a.lc);
            return nullptr;
        };
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            const float* src = qsrc(j);
            if (src) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float4 v = reinterpret_cast<const float4*>(src)[k];
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)),
                                             fmaxf(fabsf(v.z), fabsf(v.w))));
                }
            }
        }
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        int ex = 0;
        if (amax > 0.0f)
            (void)frexpf(amax, &ex);
        // amax * 2^k2 in [2^13, 2^14); clamped so 2^k2 and 2^-k2 stay normal
        const int k2 = min(max(14 - ex, -126), 126);
        const float mult = ldexpf(1.0f, k2);
        hfac[ht] = a.sm_log2 * ldexpf(1.0f, -k2);
        tlim[ht] = (a.mode == kCausal) ? a.pos0 + (hv ? qh / a.n_heads : 0) + 1 : 0x7FFFFFFF;
        // pass 1: fp16 high part; remember the largest residual
        float lmax = 0.0f;
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            const float* src = qsrc(j);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                f16x8 hi;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const float4 v = src ? reinterpret_cast<const float4*>(src)[2 * hh + k]
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
                    const float e4[4] = {v.x * mult, v.y * mult, v.z * mult, v.w * mult};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const _Float16 h = (_Float16)e4[q];
                        hi[4 * k + q] = h;
                        lmax = fmaxf(lmax, fabsf(e4[q] - (float)h));
                    }
                }
                qhi[j][ht][hh] = hi;
            }
        }
        lmax = fmaxf(lmax, __shfl_xor(lmax, 16));
        lmax = fmaxf(lmax, __shfl_xor(lmax, 32));
        int exl = 0;
        if (lmax > 0.0f)
            (void)frexpf(lmax, &exl);
        // lmax * 2^kl in [128, 256), inside e4m3's range; E8M0 needs |kl| <= 126
        const int kl = min(max(8 - exl, -126), 126);
        const float lmult = ldexpf(1.0f, kl);
        qlo_scale[ht] = 127 - kl;  // E8M0 exponent of 2^-kl
        // pass 2: e4m3 low part, packed four codes per dword
#pragma unroll
        for (int i = 0; i < NKB2; ++i) {
            v8i pk;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int j = 2 * i + half;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t word = 0u;
                    if (j < NKB) {
                        const float* src = qsrc(j);
                        const float4 v = src ? reinterpret_cast<const float4*>(src)[k]
                                             : make_float4(0.f, 0.f, 0.f, 0.f);
                        const float e4[4] = {v.x * mult, v.y * mult, v.z * mult, v.w * mult};
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float r = e4[q] - (float)(_Float16)e4[q];
                            word |= enc_e4m3(r * lmult) << (8 * q);
                        }
                    }
                    pk[4 * half + k] = (int)word;
                }
            }
            qlo[i][ht] = pk;
        }
    }

    // ---- LDS init: zero both row buffers (pads stay zero for the whole run).
    for (int i = tid; i < 2 * TR * XS / 16; i += kThreads)
        reinterpret_cast<uint4*>(&xs[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);

    // ---- tile loader: global -> registers, registers -> LDS.
    const int cpr = a.d >> 4;  // 16-byte chunks per row
    const int tot = TR * cpr;
    uint4 pre[NKB];
    float pre_scale = 0.0f;
    int32_t pre_row = -1;

    auto row_of = [&](int pos) -> int32_t {
        if (pos >= c1)
            return -1;
        if (a.mode == kSelect) {
            const int32_t r = a.sel[pos];
            return (r >= 0 && r < a.t_rows) ? r : -1;
        }
        return pos;
    };
    auto load_tile = [&](int p0) {
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const int id = tid + kThreads * i;
            pre[i] = make_uint4(0u, 0u, 0u, 0u);
            if (id < tot) {
                const int r = id / cpr, c = id - r * cpr;
                const int32_t row = row_of(p0 + r);
                if (row >= 0)
                    pre[i] = *reinterpret_cast<const uint4*>(a.codes + (size_t)row * a.d + c * 16);
            }
        }
        if (tid < TR) {
            pre_row = row_of(p0 + tid);
            pre_scale = pre_row >= 0 ? a.scales[pre_row] : 0.0f;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const int id = tid + kThreads * i;
            if (id < tot) {
                const int r = id / cpr, c = id - r * cpr;
                *reinterpret_cast<uint4*>(&xs[buf][r * XS + c * 16]) = pre[i];
            }
        }
        if (tid < TR) {
            s_scale[buf][tid] = pre_scale;
            s_lscale[buf][tid] = log2f(pre_scale);  // -inf for a zero scale
            s_row[buf][tid] = pre_row;
        }
    };

    float mrun[2] = {-INFINITY, -INFINITY};   // running max of u (z side)
    float morun[2] = {-INFINITY, -INFINITY};  // running max of u + log2 scale (O side)
    float zacc[2] = {0.0f, 0.0f};
    f32x4 O[2][8];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int jm = 0; jm < 8; ++jm)
            O[ht][jm] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int cb = 128 * w;  // this wave's context column block
    const bool pv_active = cb < a.lc;

    __syncthreads();  // zero fill done before the first tile lands
    if (ntiles > 0) {
        load_tile(c0);
        store_tile(0);
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        if (it + 1 < ntiles)
            load_tile(c0 + (it + 1) * TR);

        // ---- scores: S^T[16 rows of this wave][32 heads]
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        const uint8_t* xrow = &xs[buf][(16 * w + n) * XS + 16 * g];
#pragma unroll
        for (int i = 0; i < NKB2; ++i) {
            const uint4 x0 = *reinterpret_cast<const uint4*>(xrow + 128 * i);
            const uint4 x1 = (2 * i + 1 < NKB)
                                 ? *reinterpret_cast<const uint4*>(xrow + 128 * i + 64)
                                 : make_uint4(0u, 0u, 0u, 0u);
            {
                const f16x8 a0 = cvt8(x0.x, x0.y), a1 = cvt8(x0.z, x0.w);
#pragma unroll
                for (int ht = 0; ht < 2; ++ht) {
                    acc[ht] = mfma16(a0, qhi[2 * i][ht][0], acc[ht]);
                    acc[ht] = mfma16(a1, qhi[2 * i][ht][1], acc[ht]);
                }
            }
            if (2 * i + 1 < NKB) {
                const f16x8 a0 = cvt8(x1.x, x1.y), a1 = cvt8(x1.z, x1.w);
#pragma unroll
                for (int ht = 0; ht < 2; ++ht) {
                    acc[ht] = mfma16(a0, qhi[2 * i + 1][ht][0], acc[ht]);
                    acc[ht] = mfma16(a1, qhi[2 * i + 1][ht][1], acc[ht]);
                }
            }
            const v8i x8 = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                               (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
                acc[ht] = mfma_fp8_scaled(x8, qlo[i][ht], acc[ht], qlo_scale[ht]);
        }

        // ---- log2-domain scores u and O-side logits uo; per-wave maxima
        float u[2][4], uo[2][4], tm[2], tmo[2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            tm[ht] = -INFINITY;
            tmo[ht] = -INFINITY;
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * w + 4 * g + v;
            const float sc = s_scale[buf][r], ls = s_lscale[buf][r];
            const int32_t row = s_row[buf][r];
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) {
                const bool valid = row >= 0 && row < tlim[ht];
                const float uu = valid ? (acc[ht][v] * hfac[ht]) * sc : -INFINITY;
                u[ht][v] = uu;
                uo[ht][v] = valid ? uu + ls : -INFINITY;
                tm[ht] = fmaxf(tm[ht], u[ht][v]);
                tmo[ht] = fmaxf(tmo[ht], uo[ht][v]);
            }
        }
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            tm[ht] = fmaxf(tm[ht], __shfl_xor(tm[ht], 16));
            tm[ht] = fmaxf(tm[ht], __shfl_xor(tm[ht], 32));
            tmo[ht] = fmaxf(tmo[ht], __shfl_xor(tmo[ht], 16));
            tmo[ht] = fmaxf(tmo[ht], __shfl_xor(tmo[ht], 32));
            if (g == 0) {
                s_red[w][0][16 * ht + n] = tm[ht];
                s_red[w][1][16 * ht + n] = tmo[ht];
            }
        }
        __syncthreads();

        // ---- running maxima (identical in every wave), weights, z
        float alo[2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int h = 16 * ht + n;
            const float T = fmaxf(fmaxf(s_red[0][0][h], s_red[1][0][h]),
                                  fmaxf(s_red[2][0][h], s_red[3][0][h]));
            const float TO = fmaxf(fmaxf(s_red[0][1][h], s_red[1][1][h]),
                                   fmaxf(s_red[2][1][h], s_red[3][1][h]));
            const float mnew = (T > mrun[ht] + kTau) ? T : mrun[ht];
            const float alz = (mnew == mrun[ht]) ? 1.0f : fast_exp2(mrun[ht] - mnew);
            mrun[ht] = mnew;
            const float monew = (TO > morun[ht] + kTau) ? TO : morun[ht];
            alo[ht] = (monew == morun[ht]) ? 1.0f : fast_exp2(morun[ht] - monew);
            morun[ht] = monew;
            const float mu = (mrun[ht] == -INFINITY) ? 0.0f : mrun[ht];
            const float muo = (morun[ht] == -INFINITY) ? 0.0f : morun[ht];
            float ps = 0.0f;
            f16x4 wv;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                ps += fast_exp2(u[ht][v] - mu);
                wv[v] = (_Float16)fast_exp2(uo[ht][v] - muo);
            }
            zacc[ht] = zacc[ht] * alz + ps;
            *reinterpret_cast<f16x4*>(&s_w[h * WSS + 16 * w + 4 * g]) = wv;
        }
        // Rescale the context accumulators when a running max moved.  O holds
        // heads 16*ht + 4*g + v; their factors live in lanes 4*g + v.
        if (__any((alo[0] != 1.0f) || (alo[1] != 1.0f))) {
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float f = __shfl(alo[ht], 4 * g + v);
#pragma unroll
                    for (int jm = 0; jm < 8; ++jm)
                        O[ht][jm][v] *= f;
                }
        }
        __syncthreads();  // weight tile complete

        // ---- context: O[32 heads][128 cols of this wave] += W . X
        if (pv_active) {
#pragma unroll
            for (int ks = 0; ks < TR / 32; ++ks) {
                f16x8 wa[2];
#pragma unroll
                for (int ht = 0; ht < 2; ++ht)
                    wa[ht] = *reinterpret_cast<const f16x8*>(
                        &s_w[(16 * ht + n) * WSS + 32 * ks + 8 * g]);
                uint2 xr[8];
#pragma unroll
                for (int v = 0; v < 8; ++v)
                    xr[v] = *reinterpret_cast<const uint2*>(
                        &xs[buf][(32 * ks + 8 * g + v) * XS + cb + 8 * n]);
#pragma unroll
                for (int jp = 0; jp < 4; ++jp) {
                    // columns 2jp and 2jp+1 of this lane's 8-byte block
                    const int jj = (2 * jp) & 3;
                    const uint32_t selb = (uint32_t)jj | ((uint32_t)(jj + 4) << 8) |
                                          ((uint32_t)(jj + 1) << 16) |
                                          ((uint32_t)(jj + 5) << 24);
                    f16x8 bA, bB;
#pragma unroll
                    for (int uu = 0; uu < 4; ++uu) {
                        const uint32_t r0 = jp < 2 ? xr[2 * uu].x : xr[2 * uu].y;
                        const uint32_t r1 = jp < 2 ? xr[2 * uu + 1].x : xr[2 * uu + 1].y;
                        // bytes: [r0.jj, r1.jj, r0.jj+1, r1.jj+1]
                        const uint32_t pk = __builtin_amdgcn_perm(r1, r0, selb);
                        const f16x2 lo = cvt2<false>(pk), hi = cvt2<true>(pk);
                        bA[2 * uu] = lo[0];
                        bA[2 * uu + 1] = lo[1];
                        bB[2 * uu] = hi[0];
                        bB[2 * uu + 1] = hi[1];
                    }
#pragma unroll
                    for (int ht = 0; ht < 2; ++ht) {
                        O[ht][2 * jp] = mfma16(wa[ht], bA, O[ht][2 * jp]);
                        O[ht][2 * jp + 1] = mfma16(wa[ht], bB, O[ht][2 * jp + 1]);
                    }
                }
            }
        }

        if (it + 1 < ntiles)
            store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: z over lane groups and waves; partial (m, z, cl)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        float zz = zacc[ht];
        zz += __shfl_xor(zz, 16);
        zz += __shfl_xor(zz, 32);
        if (g == 0)
            s_z[w][16 * ht + n] = zz;
    }
    __syncthreads();
    const size_t pbase = (size_t)chunk * a.n_qh;
    if (w == 0 && g == 0) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int h = 16 * ht + n, qh = qh0 + h;
            if (qh < a.n_qh) {
                a.ws_m[pbase + qh] = mrun[ht];
                a.ws_z[pbase + qh] = (s_z[0][h] + s_z[1][h]) + (s_z[2][h] + s_z[3][h]);
            }
        }
    }
    if (pv_active) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const float fown = (mrun[ht] == -INFINITY || morun[ht] == -INFINITY)
                                   ? 0.0f
                                   : fast_exp2(morun[ht] - mrun[ht]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float f = __shfl(fown, 4 * g + v);
                const int qh = qh0 + 16 * ht + 4 * g + v;
                const int col = cb + 8 * n;
                if (qh < a.n_qh && col < a.lc) {
                    float4* dst = reinterpret_cast<float4*>(a.ws_cl + (pbase + qh) * a.lc + col);
                    dst[0] = make_float4(O[ht][0][v] * f, O[ht][1][v] * f, O[ht][2][v] * f,
                                         O[ht][3][v] * f);
                    dst[1] = make_float4(O[ht][4][v] * f, O[ht][5][v] * f, O[ht][6][v] * f,
                                         O[ht][7][v] * f);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the n_chunks partials of every query-head.
// Grid (n_qh, ceil(lc / 64)), one wave per block, one column per lane.
__global__ __launch_bounds__(64) void k_merge(const float* __restrict__ ws_m,
                                              const float* __restrict__ ws_z,
                                              const float* __restrict__ ws_cl, int32_t n_chunks,
                                              int32_t n_qh, int32_t lc, float* __restrict__ out,
                                              float* __restrict__ lse)
{
    const int qh = blockIdx.x;
    const int col = blockIdx.y * 64 + threadIdx.x;
    float M = -INFINITY;
    for (int p = 0; p < n_chunks; ++p)
        M = fmaxf(M, ws_m[(size_t)p * n_qh + qh]);
    float Z = 0.0f, acc = 0.0f;
    if (M != -INFINITY) {
        for (int p = 0; p < n_chunks; ++p) {
            const float mp = ws_m[(size_t)p * n_qh + qh];
            if (mp == -INFINITY)
                continue;
            const float wgt = exp2f(mp - M);
            Z += wgt * ws_z[(size_t)p * n_qh + qh];
            if (col < lc)
                acc += wgt * ws_cl[((size_t)p * n_qh + qh) * lc + col];
        }
    }
    if (col < lc)
        out[(size_t)qh * lc + col] = (M == -INFINITY) ? 0.0f : acc / Z;
    if (lse != nullptr && blockIdx.y == 0 && threadIdx.x == 0)
        lse[qh] = (M == -INFINITY) ? -INFINITY : (M + log2f(Z)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
hipError_t launch_quantize(const float* x, int64_t n_rows, int32_t d, uint8_t* codes,
                           float* scales, hipStream_t stream)
{
    if (n_rows == 0)
        return hipSuccess;
    const int64_t blocks = (n_rows + 3) / 4;
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_rows,
                       d, codes, scales);
    return hipGetLastError();
}

hipError_t launch_test_encode(const float* x, int64_t n, uint8_t* codes, hipStream_t stream)
{
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(k_test_encode, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, codes);
    return hipGetLastError();
}

template <int NKB>
static void launch_partial(const AttnArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(k_split_partial<NKB>, dim3((unsigned)(a.n_chunks * a.n_groups)),
                       dim3(kThreads), 0, stream, a);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream, hipEvent_t ev_before,
                            hipEvent_t ev_after)
{
    // The padded LDS row must cover both the score width d and the context
    // columns the 128-wide column blocks read (up to roundup(lc, 128)).
    const int nkb = max((a.d + 63) / 64, 2 * ((a.lc + 127) / 128));
    if (nkb < 1 || nkb > 10)
        return hipErrorInvalidValue;
    if (ev_before != nullptr) {
        const hipError_t e = hipEventRecord(ev_before, stream);
        if (e != hipSuccess)
            return e;
    }
    switch (nkb) {
    case 1: launch_partial<1>(a, stream); break;
    case 2: launch_partial<2>(a, stream); break;
    case 3: launch_partial<3>(a, stream); break;
    case 4: launch_partial<4>(a, stream); break;
    case 5: launch_partial<5>(a, stream); break;
    case 6: launch_partial<6>(a, stream); break;
    case 7: launch_partial<7>(a, stream); break;
    case 8: launch_partial<8>(a, stream); break;
    case 9: launch_partial<9>(a, stream); break;
    case 10: launch_partial<10>(a, stream); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (ev_after != nullptr) {
        e = hipEventRecord(ev_after, stream);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(k_merge, dim3((unsigned)a.n_qh, (unsigned)((a.lc + 63) / 64)), dim3(64), 0,
                       stream, a.ws_m, a.ws_z, a.ws_cl, a.n_chunks, a.n_qh, a.lc, a.out, a.lse);
    return hipGetLastError();
}

}  // namespace mla8
