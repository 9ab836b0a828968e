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
//   * Rows stream HBM -> LDS in 64-row tiles through a 3-stage ring of direct
//     global_load_lds_dwordx4 loads (two tiles in flight, no register
//     staging).  e4m3 bytes are widened to fp16 in registers with
//     v_cvt_scalef32_pk_f16_fp8 (exact: every e4m3 value is an fp16 normal),
//     then fed to v_mfma_f32_16x16x32_f16.
//   * 8 waves per workgroup (two per SIMD).  Scores S^T[row][head] = X . Q^T:
//     each wave takes 16 rows x 16 heads; q is split into an fp16 high part
//     held in registers (fp16 MFMA) and an e4m3 low part held in LDS (scaled
//     fp8 MFMA straight on the row bytes), with a power of two per head so it
//     sits in fp16's range.
//   * Context O[head][col] += W . X: each wave owns a 64-column slice for all
//     32 heads, reading a 4x8 byte block per lane and transposing it with
//     v_perm_b32 so the row (contraction) index becomes the MFMA K index.
//   * The row scale is hoisted: scores are (q . code) * scale_t, and the PV
//     weight of row t is exp2((u_t - m) + log2 scale_t - d) with d a running
//     max kept relative to the score max m, so fp16 weights never overflow or
//     lose significant rows, and large scores never swallow log2 scale_t.
//   * Online softmax with a lazy running max: the max is only moved when a
//     tile beats it by more than 2^8, which keeps rescaling of the register
//     accumulators off the common path.
#include "mla8_internal.h"

#include <math.h>

#include <type_traits>

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

// Source of the 16 query elements d = 64j + 16g .. +16 of query-head qh, and
// whether they exist (false past the row width or past the last head; the
// pointer then still addresses valid memory, the first q_lat row, so that every
// load can be issued unconditionally and many can be in flight at once).
struct QSrc {
    const float* p;
    bool ok;
};

__device__ __forceinline__ QSrc q_src(const AttnArgs& a, int qh, bool hv, int j, int g)
{
    const int d0 = 64 * j + 16 * g;
    if (hv && d0 < a.lc)
        return {a.q_lat + (size_t)qh * a.lc + d0, true};
    if (hv && d0 < a.d)
        return {a.q_rope + (size_t)qh * a.rc + (d0 - a.lc), true};
    return {a.q_lat, false};
}

__device__ __forceinline__ float4 ld4(const QSrc& s, int k)
{
    const float4 v = reinterpret_cast<const float4*>(s.p)[k];
    return s.ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Query operands for 16 heads.  Lane (n, g) holds, for head qh_base + n, the
// elements d = 64j + 16g + e (e < 16).  The same assignment of the contraction
// index to (lane group, operand slot) is used for the row operand, so the MFMA
// sums the right products whatever its K labels are.
//   qhi: fp16(q * 2^k)                 two f16x8 per j      -> fp16 MFMA,
//        kept in registers;
//   qlo: e4m3((q*2^k - qhi) * 2^6)     32 bytes per j pair  -> fp8 MFMA, whose
//        E8M0 operand scale 2^-6 undoes the 2^6 inside the instruction; written
//        lane-linear to LDS (qlo_lds[i][lane], 32 bytes) when write_lo is set.
// k puts the head's largest |q| in [2^13, 2^14), where the fp16 spacing is 8,
// so every residual is at most 4 and 2^6 * 4 = 256 sits inside e4m3's range.
// Every index is a compile-time constant so qhi stays in registers.
constexpr int kQloShift = 6;

template <int NKB>
__device__ __forceinline__ void load_query(const AttnArgs& a, int qh_base, int n, int g, int lane,
                                           f16x8 (&qhi)[NKB][2], v8i* qlo_lds, bool write_lo,
                                           float& hfac, int32_t& tlim)
{
    const int qh = qh_base + n;
    const bool hv = qh < a.n_qh;
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
        const QSrc src = q_src(a, qh, hv, j, g);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 v = ld4(src, k);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
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
    const float lmult = (float)(1 << kQloShift);
    hfac = a.sm_log2 * ldexpf(1.0f, -k2);
    tlim = (a.mode == kCausal) ? a.pos0 + (hv ? qh / a.n_heads : 0) + 1 : 0x7FFFFFFF;
    int lo[8];
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
        const QSrc src = q_src(a, qh, hv, j, g);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float4 v0 = ld4(src, 2 * hh), v1 = ld4(src, 2 * hh + 1);
            const float e[8] = {v0.x * mult, v0.y * mult, v0.z * mult, v0.w * mult,
                                v1.x * mult, v1.y * mult, v1.z * mult, v1.w * mult};
            f16x8 hi;
            float r[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                hi[q] = (_Float16)e[q];
                r[q] = (e[q] - (float)hi[q]) * lmult;  // exact: |r| <= 256
            }
            qhi[j][hh] = hi;
            // v_cvt_pk_fp8_f32 rounds to nearest even onto OCP e4m3
            int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], w0, true);
            int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[4], r[5], 0, false);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[6], r[7], w1, true);
            lo[4 * (j & 1) + 2 * hh] = w0;
            lo[4 * (j & 1) + 2 * hh + 1] = w1;
        }
        if ((j & 1) || j == NKB - 1) {
            if (!(j & 1))
#pragma unroll
                for (int k = 4; k < 8; ++k)
                    lo[k] = 0;
            if (write_lo)
                qlo_lds[(j >> 1) * 64 + lane] =
                    v8i{lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]};
        }
    }
}

constexpr float kTau = 8.0f;  // lazy-max slack, log2 units: weights stay <= 2^8

// ---------------------------------------------------------------------------
// LDS barrier without a memory fence: wait for this wave's LDS operations,
// then s_barrier.  A fenced __syncthreads would also wait for every
// outstanding global->LDS row load (vmcnt 0) and empty the load pipeline.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
    asm volatile("" ::: "memory");
}

#define MLA8_LDS __attribute__((address_space(3)))

// Direct global -> LDS loads, lane i writing LDS bytes [base + 16i, +16)
// (dwordx4) or [base + 4i, +4) (dword).  Issued through asm so that the
// compiler's wait insertion does not track them: every wait on them is the
// explicit wait_vmcnt<> of the tile pipeline (a tracked load would be waited
// with vmcnt(0) wherever its LDS object is read, draining the pipeline).
// These are the kernel's only users of m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_b128(const void* src, const void* lds_dst)
{
    const uint32_t off = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(MLA8_LDS const void*)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(off), "v"(src)
                 : "memory", "m0");
}

__device__ __forceinline__ void dma_b32(const void* src, const void* lds_dst)
{
    const uint32_t off = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(MLA8_LDS const void*)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(off), "v"(src)
                 : "memory", "m0");
}
// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
__device__ __forceinline__ void dma_b128_s(const void* base, uint32_t voff, const void* lds_dst)
{
    const uint32_t off = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(MLA8_LDS const void*)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(off), "v"(voff), "s"(base)
                 : "memory", "m0");
}

__device__ __forceinline__ void dma_b32_s(const void* base, uint32_t voff, const void* lds_dst)
{
    const uint32_t off = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(MLA8_LDS const void*)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(off), "v"(voff), "s"(base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Split-T partial.  Grid: n_chunks * n_groups workgroups of 512 threads (8
// waves, two per SIMD).  NKB = number of 64-wide blocks of the padded row.
//   loads  : 64-row tiles stream HBM -> LDS through a 3-stage ring of direct
//            global_load_lds_dwordx4 (no register staging), two tiles in
//            flight while a third is consumed;
//   scores : wave w takes rows 16*(w>>1) .. +16 of the tile and heads
//            16*(w&1) .. +16 of the group (fp16 high part of q in registers,
//            e4m3 low part in LDS);
//   context: wave w owns context columns 64*w .. +64 for all 32 heads.
template <int NKB, bool GATHER>
__global__ __launch_bounds__(kThreads, 1) void k_split_partial(AttnArgs a)
{
    constexpr int TR = kTileRows;
    constexpr int HG = kHeadsPerGroup;
    constexpr int NW = kThreads / 64;    // waves
    constexpr int DP = 64 * NKB;         // padded row width in LDS (>= d, >= roundup(lc, 128))
    constexpr int XS = DP + 16;          // LDS row stride: DP bytes + one 16-B pad slot
    constexpr int SPR = XS / 16;         // 16-byte slots per LDS row
    constexpr int NINS = SPR;            // 1-KB DMA instructions per tile (64 rows x SPR slots)
    constexpr int KW = (NINS + NW - 1) / NW;  // row DMA instructions per wave per tile
    constexpr int NVM = KW + 1;          // + one scale DMA: vector-memory ops per wave per tile
    constexpr int NST = 3;               // ring stages
    constexpr int WSS = TR + 8;          // LDS stride of the weight tile (halves)
    constexpr int NKB2 = (NKB + 1) / 2;  // 128-wide blocks for the fp8 pass
    static_assert(TR * XS == NINS * 1024, "a stage is a whole number of 1-KB DMA blocks");
    static_assert(NVM < 64, "vmcnt range");

    // One object per ring stage: the compiler tracks memory per object.
    __shared__ __attribute__((aligned(1024))) uint8_t xs0[TR * XS];
    __shared__ __attribute__((aligned(1024))) uint8_t xs1[TR * XS];
    __shared__ __attribute__((aligned(1024))) uint8_t xs2[TR * XS];
    __shared__ __attribute__((aligned(16))) float sc0[NW][TR];  // per-wave copies of the scales
    __shared__ __attribute__((aligned(16))) float sc1[NW][TR];
    __shared__ __attribute__((aligned(16))) float sc2[NW][TR];
    __shared__ int32_t s_row[NST][TR];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[HG * WSS];
    __shared__ __attribute__((aligned(32))) v8i s_qlo[2][NKB2 * 64];  // [head half][block][lane]
    __shared__ float s_red[4][2][HG];
    __shared__ float s_z[4][HG];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
    const int hh = w & 1;   // head half of the group this wave scores
    const int rq = w >> 1;  // row quarter of the tile this wave scores

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

    // ---- query operands for heads qh0 + 16*hh + n (the low part is written
    // to LDS by the row-quarter-0 wave of each head half)
    f16x8 qhi[NKB][2];
    float hfac;
    int32_t tlim;
    load_query<NKB>(a, qh0 + 16 * hh, n, g, lane, qhi, &s_qlo[hh][0], rq == 0, hfac, tlim);
    const v8i* qlo = &s_qlo[hh][0];

    // ---- tile issue: every wave issues exactly NVM vector-memory operations
    // per tile (so a fixed vmcnt marks a tile complete).  Row DMA instruction k
    // fills LDS bytes [1024k, 1024k + 1024) of the stage: slot 64k + lane is
    // (row r, 16-byte chunk c) with r = slot / SPR, c = slot % SPR.  Slots past
    // the row's data (zero-pad columns, the pad slot) and rows outside the
    // list load chunk 0 / the tile's first row instead: finite bytes that are
    // multiplied by a zero query element, masked out of the softmax, or never
    // read.  Spare instruction slots (k >= NINS) repeat instruction k % NINS
    // (the same bytes to the same place).
    const int cpr = a.d >> 4;  // 16-byte data chunks per row
    auto xs_of = [&](auto S_) __attribute__((always_inline)) -> uint8_t* {
        constexpr int S = decltype(S_)::value;
        if constexpr (S == 0)
            return xs0;
        else if constexpr (S == 1)
            return xs1;
        else
            return xs2;
    };
    auto sc_of = [&](auto S_) __attribute__((always_inline)) -> float* {
        constexpr int S = decltype(S_)::value;
        if constexpr (S == 0)
            return &sc0[0][0];
        else if constexpr (S == 1)
            return &sc1[0][0];
        else
            return &sc2[0][0];
    };
    auto row_of = [&](int pos) __attribute__((always_inline)) -> int32_t {
        if (pos >= c1)
            return -1;
        const int32_t r = a.sel[pos];
        return (r >= 0 && r < a.t_rows) ? r : -1;
    };
    // Per row DMA i of this wave: r << 16 | (r * d + chunk offset), the same
    // for every tile, so it is packed once.
    int dpk[KW];
#pragma unroll
    for (int i = 0; i < KW; ++i) {
        const int k = (w + NW * i) % NINS;
        const int slot = 64 * k + lane;
        const int r = slot / SPR, c = slot - (slot / SPR) * SPR;
        dpk[i] = (r << 16) | (r * a.d + (c < cpr ? 16 * c : 0));
    }
    auto issue = [&](int t, auto S_) __attribute__((always_inline)) {
        constexpr int st = decltype(S_)::value;
        uint8_t* xst = xs_of(S_);
        float* sct = sc_of(S_) + TR * w;
        const int p0 = c0 + t * TR;
        if constexpr (!GATHER) {
            // Contiguous rows p0 .. p0 + nv - 1: SGPR base + 32-bit offsets.
            // Rows past the list reload the tile's first row.
            const int nv = c1 - p0;
            const uint8_t* tb = a.codes + (size_t)p0 * a.d;
#pragma unroll
            for (int i = 0; i < KW; ++i) {
                const int k = (w + NW * i) % NINS;
                const int r = dpk[i] >> 16;
                const uint32_t off = (uint32_t)((dpk[i] & 0xFFFF) - (r < nv ? 0 : r * a.d));
                dma_b128_s(tb, off, xst + 1024 * k);
            }
            dma_b32_s(a.scales + p0, (uint32_t)(4 * (lane < nv ? lane : 0)), sct);
            if (w == 0)
                s_row[st][lane] = lane < nv ? p0 + lane : -1;
        } else {
            // Gather: absolute row indices; entries outside [0, t_rows) and
            // positions past the list reload row 0.
#pragma unroll
            for (int i = 0; i < KW; ++i) {
                const int k = (w + NW * i) % NINS;
                const int r = dpk[i] >> 16;
                const int cc = (dpk[i] & 0xFFFF) - r * a.d;
                const int32_t row = row_of(p0 + r);
                dma_b128(a.codes + (size_t)(row >= 0 ? row : 0) * a.d + cc, xst + 1024 * k);
            }
            const int32_t srow = row_of(p0 + lane);
            dma_b32(a.scales + (srow >= 0 ? srow : 0), sct);
            if (w == 0)
                s_row[st][lane] = srow;
        }
    };

    // Running softmax state, replicated in every wave for heads n and 16 + n
    // of the group: m = lazy max of u (z side), d = lazy max of
    // (u - m) + log2 scale (context side, relative to m).
    float mrun[2] = {-INFINITY, -INFINITY};
    float drun[2] = {-INFINITY, -INFINITY};
    float zacc = 0.0f;  // z partial over this lane's rows, head 16*hh + n
    f32x4 O[2][4];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int jm = 0; jm < 4; ++jm)
            O[ht][jm] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int cb = 64 * w;  // this wave's context columns
    const bool pv_active = cb < a.lc;

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    if (ntiles > 0)
        issue(0, S0{});
    if (ntiles > 1)
        issue(1, S1{});

    // One tile: wait for its loads, refill the stage freed two tiles ago,
    // score, update the softmax state, accumulate the context.  Barrier (A)
    // also publishes the q low part written before the first tile.
    auto tile = [&](int it, auto S_) __attribute__((always_inline)) {
        constexpr int st = decltype(S_)::value;
        const uint8_t* xst = xs_of(S_);
        const float* scs = sc_of(S_) + TR * w;
        // Tile it is complete once only tile it+1's operations may remain.
        if (it + 1 < ntiles)
            wait_vmcnt<NVM>();
        else
            wait_vmcnt<0>();
        lds_barrier();  // (A) tile it visible to all waves; stage (it+2)%3 free
        if (it + 2 < ntiles)
            issue(it + 2, std::integral_constant<int, (st + 2) % NST>{});

        // ---- scores: S^T[16 rows][16 heads]
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint8_t* xrow = xst + (16 * rq + n) * XS + 16 * g;
#pragma unroll
        for (int i = 0; i < NKB2; ++i) {
            const uint4 x0 = *reinterpret_cast<const uint4*>(xrow + 128 * i);
            const uint4 x1 = (2 * i + 1 < NKB)
                                 ? *reinterpret_cast<const uint4*>(xrow + 128 * i + 64)
                                 : make_uint4(0u, 0u, 0u, 0u);
            acc = mfma16(cvt8(x0.x, x0.y), qhi[2 * i][0], acc);
            acc = mfma16(cvt8(x0.z, x0.w), qhi[2 * i][1], acc);
            if (2 * i + 1 < NKB) {
                acc = mfma16(cvt8(x1.x, x1.y), qhi[2 * i + 1][0], acc);
                acc = mfma16(cvt8(x1.z, x1.w), qhi[2 * i + 1][1], acc);
            }
            const v8i x8 = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                               (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            acc = mfma_fp8_scaled(x8, qlo[i * 64 + lane], acc, 127 - kQloShift);
        }

        // ---- log2-domain scores u (rows 16rq + 4g + v, head 16hh + n); per
        // wave: the tile max Tw of u and Cw = max_t (u_t - Tw) + log2 scale_t.
        // Everything after this stays relative to a running max, so a large
        // |u| never swallows log2 scale.
        float u[4], lsv[4];
        float tw = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * rq + 4 * g + v;
            const float sc = scs[r];
            lsv[v] = log2f(sc);  // -inf for a zero scale
            const int32_t row = s_row[st][r];
            const bool valid = row >= 0 && row < tlim;
            u[v] = valid ? (acc[v] * hfac) * sc : -INFINITY;
            tw = fmaxf(tw, u[v]);
        }
        tw = fmaxf(tw, __shfl_xor(tw, 16));
        tw = fmaxf(tw, __shfl_xor(tw, 32));
        float cw = -INFINITY;
        if (tw != -INFINITY) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                cw = fmaxf(cw, (u[v] - tw) + lsv[v]);
        }
        cw = fmaxf(cw, __shfl_xor(cw, 16));
        cw = fmaxf(cw, __shfl_xor(cw, 32));
        if (g == 0) {
            s_red[rq][0][16 * hh + n] = tw;
            s_red[rq][1][16 * hh + n] = cw;
        }
        lds_barrier();  // (B) per-wave maxima exchanged

        // ---- running state for heads n, 16 + n (every wave computes both)
        float alz[2], alo[2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int h = 16 * ht + n;
            float T = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                T = fmaxf(T, s_red[k][0][h]);
            const float mold = mrun[ht];
            const float mnew = (T > mold + kTau) ? T : mold;
            alz[ht] = (mnew == mold) ? 1.0f : fast_exp2(mold - mnew);
            const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
            float tb = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float Tk = s_red[k][0][h];
                if (Tk != -INFINITY)
                    tb = fmaxf(tb, s_red[k][1][h] + (Tk - mu));
            }
            const float dshift = (mnew == mold) ? drun[ht] : drun[ht] + (mold - mnew);
            const float dnew = (tb > dshift + kTau) ? tb : dshift;
            alo[ht] = (dnew == dshift) ? 1.0f : fast_exp2(dshift - dnew);
            mrun[ht] = mnew;
            drun[ht] = dnew;
        }
        // ---- this wave's rows: p = 2^(u - m) into z, w = 2^((u - m) + ls - d)
        {
            const float mu = hh ? mrun[1] : mrun[0];
            const float dd = hh ? drun[1] : drun[0];
            const float mz = (mu == -INFINITY) ? 0.0f : mu;
            const float dn = (dd == -INFINITY) ? 0.0f : dd;
            float ps = 0.0f;
            f16x4 wv;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float av = u[v] - mz;
                ps += fast_exp2(av);
                wv[v] = (_Float16)fast_exp2((av + lsv[v]) - dn);
            }
            zacc = zacc * (hh ? alz[1] : alz[0]) + ps;
            *reinterpret_cast<f16x4*>(&s_w[(16 * hh + n) * WSS + 16 * rq + 4 * g]) = wv;
        }
        // Rescale the context accumulators when a context offset moved.  O
        // holds heads 16*ht + 4*g + v; their factors live in lanes 4*g + v.
        if (__any((alo[0] != 1.0f) || (alo[1] != 1.0f))) {
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float f = __shfl(alo[ht], 4 * g + v);
#pragma unroll
                    for (int jm = 0; jm < 4; ++jm)
                        O[ht][jm][v] *= f;
                }
        }
        lds_barrier();  // (C) weight tile complete; s_red free

        // ---- context: O[32 heads][64 cols of this wave] += W . X.  Lane (n, g)
        // reads rows 32ks + 8g + 0..7, columns cb + 4n .. +4, and byte-transposes
        // them so the row index becomes the MFMA K index; MFMA jm covers the
        // columns cb + 4n' + jm over the 16 lanes n'.
        if (pv_active) {
#pragma unroll
            for (int ks = 0; ks < TR / 32; ++ks) {
                f16x8 wa[2];
#pragma unroll
                for (int ht = 0; ht < 2; ++ht)
                    wa[ht] = *reinterpret_cast<const f16x8*>(
                        &s_w[(16 * ht + n) * WSS + 32 * ks + 8 * g]);
                uint32_t xr[8];
#pragma unroll
                for (int v = 0; v < 8; ++v)
                    xr[v] = *reinterpret_cast<const uint32_t*>(
                        xst + (32 * ks + 8 * g + v) * XS + cb + 4 * n);
#pragma unroll
                for (int jp = 0; jp < 2; ++jp) {
                    // columns 2jp and 2jp+1: bytes [r0.c, r1.c, r0.c+1, r1.c+1]
                    const uint32_t jj = 2 * jp;
                    const uint32_t selb = jj | ((jj + 4) << 8) | ((jj + 1) << 16) | ((jj + 5) << 24);
                    f16x8 bA, bB;
#pragma unroll
                    for (int uu = 0; uu < 4; ++uu) {
                        const uint32_t pk = __builtin_amdgcn_perm(xr[2 * uu + 1], xr[2 * uu], selb);
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
    };

    for (int it = 0; it < ntiles; it += NST) {
        tile(it, S0{});
        if (it + 1 < ntiles)
            tile(it + 1, S1{});
        if (it + 2 < ntiles)
            tile(it + 2, S2{});
    }

    // ---- epilogue: z over lane groups and row quarters; partial (m, z, cl)
    {
        float zz = zacc;
        zz += __shfl_xor(zz, 16);
        zz += __shfl_xor(zz, 32);
        if (g == 0)
            s_z[rq][16 * hh + n] = zz;
    }
    __syncthreads();
    const size_t pbase = (size_t)chunk * a.n_qh;
    if (rq == 0 && g == 0) {
        const int h = 16 * hh + n, qh = qh0 + h;
        if (qh < a.n_qh) {
            a.ws_m[pbase + qh] = hh ? mrun[1] : mrun[0];
            a.ws_z[pbase + qh] = (s_z[0][h] + s_z[1][h]) + (s_z[2][h] + s_z[3][h]);
        }
    }
    if (pv_active) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            // cl = sum_t p_t scale_t x_t = 2^d * O
            const float fown =
                (mrun[ht] == -INFINITY || drun[ht] == -INFINITY) ? 0.0f : fast_exp2(drun[ht]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float f = __shfl(fown, 4 * g + v);
                const int qh = qh0 + 16 * ht + 4 * g + v;
                const int col = cb + 4 * n;
                if (qh < a.n_qh && col < a.lc)
                    *reinterpret_cast<float4*>(a.ws_cl + (pbase + qh) * a.lc + col) =
                        make_float4(O[ht][0][v] * f, O[ht][1][v] * f, O[ht][2][v] * f,
                                    O[ht][3][v] * f);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the n_chunks partials of every query-head.
// Grid (n_qh, ceil(lc / 64)), 256 threads: lane = context column, the four
// waves split the partials (p = wave, wave + 4, ...) with independent,
// unrolled loads, then combine through LDS.
//   M = max_p m_p;  w_p = 2^(m_p - M);  out = sum_p w_p cl_p / sum_p w_p z_p;
//   lse = (M + log2 sum_p w_p z_p) * ln 2.
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ ws_m,
                                               const float* __restrict__ ws_z,
                                               const float* __restrict__ ws_cl, int32_t n_chunks,
                                               int32_t n_qh, int32_t lc, float* __restrict__ out,
                                               float* __restrict__ lse)
{
    __shared__ float s_part[4][64];
    __shared__ float s_zp[4];
    __shared__ float s_m[4];
    const int qh = blockIdx.x;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int col = blockIdx.y * 64 + lane;
    // M over all partials
    float M = -INFINITY;
    for (int p = threadIdx.x; p < n_chunks; p += 256)
        M = fmaxf(M, ws_m[(size_t)p * n_qh + qh]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0)
        s_m[wv] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float Z = 0.0f, acc = 0.0f;
    if (M != -INFINITY) {
        const bool cv = col < lc;
        int p = wv;
        for (; p + 12 < n_chunks; p += 16) {
            float mp[4], zp[4], cp[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const size_t i = (size_t)(p + 4 * k) * n_qh + qh;
                mp[k] = ws_m[i];
                zp[k] = ws_z[i];
                cp[k] = cv ? ws_cl[i * lc + col] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float wgt = (mp[k] == -INFINITY) ? 0.0f : exp2f(mp[k] - M);
                Z += wgt * zp[k];
                acc += wgt * cp[k];
            }
        }
        for (; p < n_chunks; p += 4) {
            const size_t i = (size_t)p * n_qh + qh;
            const float mp = ws_m[i];
            const float wgt = (mp == -INFINITY) ? 0.0f : exp2f(mp - M);
            Z += wgt * ws_z[i];
            if (cv)
                acc += wgt * ws_cl[i * lc + col];
        }
    }
    s_part[wv][lane] = acc;
    if (lane == 0)
        s_zp[wv] = Z;
    __syncthreads();
    if (wv == 0) {
        const float A = (s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane]);
        const float ZZ = (s_zp[0] + s_zp[1]) + (s_zp[2] + s_zp[3]);
        if (col < lc)
            out[(size_t)qh * lc + col] = (M == -INFINITY) ? 0.0f : A / ZZ;
        if (lse != nullptr && blockIdx.y == 0 && lane == 0)
            lse[qh] = (M == -INFINITY) ? -INFINITY : (M + log2f(ZZ)) * 0.69314718055994531f;
    }
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
    if (a.mode == kSelect)
        hipLaunchKernelGGL((k_split_partial<NKB, true>), dim3((unsigned)(a.n_chunks * a.n_groups)),
                           dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_split_partial<NKB, false>),
                           dim3((unsigned)(a.n_chunks * a.n_groups)), dim3(kThreads), 0, stream, a);
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
    hipLaunchKernelGGL(k_merge, dim3((unsigned)a.n_qh, (unsigned)((a.lc + 63) / 64)), dim3(256), 0,
                       stream, a.ws_m, a.ws_z, a.ws_cl, a.n_chunks, a.n_qh, a.lc, a.out, a.lse);
    return hipGetLastError();
}

}  // namespace mla8
