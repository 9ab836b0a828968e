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
//   * Rows stream HBM -> LDS in 64-row tiles through a ring of direct
//     global_load_lds_dwordx4 loads (4 stages with two tiles in flight, or 3
//     with one when 4 do not fit), laid out for the readers; no register
//     staging.
//   * 8 waves per workgroup (two per SIMD) in two roles, one of each per
//     SIMD.  Score waves: S^T[row][head] = X . Q^T for 32 rows x 16 heads on
//     v_mfma_f32_16x16x32_f16, the row bytes widened to fp16 exactly and the
//     query split into fp16 hi + lo held in registers (the fp8 MFMAs cut their
//     products in groups of 8, too coarse for the scores; see the query
//     operands below); then the softmax weights.  Context waves: O[head][col]
//     += W . X for a 128-column slice and all 32 heads; ds_read_b64_tr_b8
//     reads the row bytes transposed so the row (contraction) index becomes
//     the MFMA K index, and v_cvt_scalef32_pk_f16_fp8 widens them to fp16
//     exactly (every e4m3 value is an fp16 value) for v_mfma_f32_16x16x32_f16
//     with fp16 weights.  The context waves also issue every row load.
//   * The row scale is hoisted: scores are (q . code) * scale_t, and the PV
//     weight of row t is exp2((u_t - m) + log2 scale_t - d) with d a running
//     max kept relative to the score max m, so fp16 weights never overflow or
//     lose significant rows, and large scores never swallow log2 scale_t.
//   * Online softmax with a lazy running max: the max is only moved when a
//     tile beats it by more than 2^8, which keeps rescaling of the register
//     accumulators off the common path.
#include "mla8_device.h"
#include "mla8_internal.h"
#include "mla8_pipe.h"

#include <math.h>

#include <type_traits>

namespace mla8 {

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
    quantize_row_wave(x + row * d, d, codes + row * d, scales + row, lane);
}

// Mixed rows, one wave per row: the noPE part through the row quantizer (its
// own amax and scale), the RoPE part to bf16.
__global__ __launch_bounds__(256) void k_quantize_rows_mx(const float* __restrict__ x,
                                                          int64_t n_rows, int32_t lc, int32_t rc,
                                                          uint8_t* __restrict__ rows,
                                                          float* __restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n_rows)
        return;
    quantize_row_mx_wave(x + row * (lc + rc), lc, rc, rows + row * (lc + 2 * rc), scales + row,
                         lane);
}

__global__ __launch_bounds__(256) void k_test_encode(const float* __restrict__ x, int64_t n,
                                                     uint8_t* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = (uint8_t)enc_e4m3(x[i]);
}

// The packed hardware encoder of the e4m3 lo query term, four values per
// thread (n4 groups of four).
__global__ __launch_bounds__(256) void k_test_encode_pk(const float4* __restrict__ x, int64_t n4,
                                                        uint32_t* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 v = x[i];
        out[i] = enc_e4m3_pk4(v.x, v.y, v.z, v.w);
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Query operands: fp16 hi + lo per element, on the fp16 MFMA.
//
// The fp8 MFMAs (the scaled 16x16x128 one and the plain 16x16x32 one) add
// their products in aligned groups of 8 K indices: inside a group each product
// is cut toward zero at 2^-13 of the largest operand-exponent sum of the group,
// and only the group sums are added in f32.  On random rows that leaves about
// 2^-19 of sum_i |e_i k_i| in every score, however many query terms carry e,
// and a row with a 50x scale whose score is a near-tie reached through
// cancellation turns that into an output error above 2e-3 of the largest
// output.  The fp16 MFMA adds like f32.  So the scores run on
// v_mfma_f32_16x16x32_f16: the row bytes are widened to fp16 exactly (every
// e4m3 value is an fp16 value), and each query head's vector
// e = (q_lat | q_rope) * sm_scale * log2(e), scaled by a power of two 2^k that
// puts its largest |element| in [2^14, 2^15), is split as
//     hi = fp16(e 2^k),  lo = fp16(e 2^k - hi)
// (the subtraction is exact in f32; both conversions round to nearest even):
// about 22 significant bits.  The f32 accumulators hold 2^k times the
// log2-domain score in code units.
//
// K order.  Lane (n, g) reads its row's elements 128 j + 32 g .. +31 of a full
// 128-element block j (two 16-byte chunks of the LDS tile layout); MFMA step s
// (0..3) of the block takes bytes 8 s .. 8 s + 7 of them, so the MFMA's K
// index 8 g + i of step s is element 128 j + 32 g + 8 s + i.  A trailing half
// block (64 elements) is read as one 16-byte chunk per lane, elements
// 128 j + 16 g .. +15, in two steps.  The query operands follow the same
// assignment.
//
// The operands are built once per workgroup into an LDS staging area laid out
// as the waves consume them: qt[head half][slot][lane][16 bytes], slot
// 8 j + 2 s + term for a full block, 8 NFULL + 2 s + term for the half block
// (term 0 = hi, 1 = lo), lane n + 16 g holding head 16 hh + n; zero past the
// row width.
template <int NFULL_, bool HALF_>
struct QueryF16 {
    static constexpr int NFULL = NFULL_;                   // full 128-element blocks
    static constexpr bool HALF = HALF_;                    // a trailing 64-element block
    static constexpr int NB = NFULL + (HALF ? 1 : 0);      // 128-wide K blocks
    static constexpr int NSLOT = 8 * NFULL + (HALF ? 4 : 0);
    static constexpr int BYTES = 2 * NSLOT * 64 * 16;
};
template <int NKB>
using QueryTerms = QueryF16<NKB / 2, (NKB & 1) != 0>;

// The hi / lo operands of elements 4 gi .. 4 gi + 3 (values r, already
// scaled by 2^k) of head 16 hh + n into the staging area; elements past the
// padded row have no slot.
template <class QF>
__device__ __forceinline__ void put_query_f16(uint8_t* qt, int hh, int n, int gi,
                                              const float (&r)[4])
{
    const int j = gi >> 5;
    int slot, g;
    if (j < QF::NFULL) {
        g = (gi >> 3) & 3;
        slot = 8 * j + 2 * ((gi >> 1) & 3);
    } else if (QF::HALF && j == QF::NFULL && (gi & 31) < 16) {
        g = (gi >> 2) & 3;
        slot = 8 * QF::NFULL + 2 * ((gi >> 1) & 1);
    } else {
        return;
    }
    f16x4 hi, lo;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        hi[c] = (_Float16)r[c];
        lo[c] = (_Float16)(r[c] - (float)hi[c]);
    }
    uint8_t* p = qt + ((size_t)(hh * QF::NSLOT + slot) * 64 + n + 16 * g) * 16 + 8 * (gi & 1);
    *reinterpret_cast<f16x4*>(p) = hi;
    *reinterpret_cast<f16x4*>(p + 64 * 16) = lo;  // slot + 1
}


// Query loads of build_query_terms: work item t (0 .. 511) handles head
// h = t / 16 (16 items per head, one 16-lane row of a wave) and the 4-element
// groups gi = t % 16 + 16 s of that head.  Every load is issued before any is
// used.
template <int NKB>
__device__ __forceinline__ void load_query(const AttnArgs& a, int qh0, int t,
                                           float4 (&v)[2 * QueryTerms<NKB>::NB])
{
    constexpr int PER = 2 * QueryTerms<NKB>::NB;  // NB blocks x 32 groups / 16 threads
    const int h = t >> 4, i = t & 15;
    const int qh = qh0 + h;
    const bool hv = qh < a.n_qh;
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        const int d = 4 * (i + 16 * s);
        const float* p = a.q_lat;  // always a valid address
        bool ok = false;
        if (hv && d < a.lc) {
            p = a.q_lat + (size_t)qh * a.lc + d;
            ok = true;
        } else if (hv && d < a.d) {
            p = a.q_rope + (size_t)qh * a.rc + (d - a.lc);
            ok = true;
        }
        const float4 x = *reinterpret_cast<const float4*>(p);
        v[s] = ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int NKB>
__device__ __forceinline__ void build_query_terms(const AttnArgs& a, int t,
                                                  const float4 (&v)[2 * QueryTerms<NKB>::NB],
                                                  uint8_t* qt, int* s_k)
{
    using Q = QueryTerms<NKB>;
    constexpr int PER = 2 * Q::NB;
    const int h = t >> 4, i = t & 15;
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < PER; ++s)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[s].x), fabsf(v[s].y)),
                                 fmaxf(fabsf(v[s].z), fabsf(v[s].w))));
    amax = row16_max(amax);
    // e = q * sm log2(e); k from the largest |e| (computed in f32 like e)
    const float es = a.sm_log2;
    const int k = query_exp(amax * es);
    if (i == 0)
        s_k[h] = k;
    const float mult = ldexpf(es, k);  // e 2^k = q * mult up to one rounding
#pragma unroll
    for (int s = 0; s < PER; ++s) {
        // one rounded f32 value per entry, opaque to the compiler, so that hi
        // and lo are split from the same r (hi is otherwise free to become the
        // fp16 rounding of the exact product, off by an fp16 step at ties)
        float r[4] = {v[s].x * mult, v[s].y * mult, v[s].z * mult, v[s].w * mult};
        asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
        put_query_f16<Q>(qt, h >> 4, h & 15, i + 16 * s, r);
    }
}

// ---------------------------------------------------------------------------
// Mixed rows ("B1 Mixed FP8/BF16 FMHA first pass" storage format, the 448 / 64
// shape): a stored row is the 448 noPE values as e4m3 bytes (scale: the
// noPE part's amax/448) followed by the 64 RoPE values as bf16, 576 bytes.
// The noPE part takes the fp16 hi + lo operands above: three full blocks and
// a half block, the first half of LDS block 3 (whose second half holds RoPE
// bytes).  The RoPE part is scored on the bf16 MFMA: e_rope = q_rope * sm *
// log2(e) splits into two bf16 terms hi + lo (about 16 significant bits),
// scaled by neither 2^k nor the row scale, in two K steps of 32.
// Staging after both head halves' fp16 slots: qr[hh][slot 2m + term][lane][16
// bytes], lane n + 16 g holding head 16 hh + n, RoPE elements 32 m + 8 g ..
// 32 m + 8 g + 7 (the row operand reads the same elements: 16-byte chunk
// 28 + 4 m + g of the row).
struct QueryTermsMx {
    static constexpr int LC = 448, RC = 64;
    using NP = QueryF16<3, true>;                   // the noPE operands
    static constexpr int NSLOT = NP::NSLOT;         // fp16 operand slots
    static constexpr int NRS = 2 * (RC / 32);       // bf16 operand slots
    static constexpr int RBASE = NP::BYTES;
    static constexpr int BYTES = RBASE + 2 * NRS * 64 * 16;
    static constexpr int NG = LC / 4 / 16;          // noPE float4 groups per thread
};

// Query loads for mixed rows: work item t takes head t / 16; noPE groups
// gi = t % 16 + 16 s (s < NG) and RoPE group t % 16.
__device__ __forceinline__ void load_query_mx(const AttnArgs& a, int qh0, int t,
                                              float4 (&v)[QueryTermsMx::NG + 1])
{
    using Q = QueryTermsMx;
    const int h = t >> 4, i = t & 15;
    const int qh = qh0 + h;
    const bool hv = qh < a.n_qh;
#pragma unroll
    for (int s = 0; s < Q::NG; ++s) {
        const float4 x = *reinterpret_cast<const float4*>(
            a.q_lat + (size_t)(hv ? qh : 0) * Q::LC + 4 * (i + 16 * s));
        v[s] = hv ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float4 x = *reinterpret_cast<const float4*>(a.q_rope + (size_t)(hv ? qh : 0) * Q::RC +
                                                      4 * i);
    v[Q::NG] = hv ? x : make_float4(0.f, 0.f, 0.f, 0.f);
}

__device__ __forceinline__ void build_query_terms_mx(const AttnArgs& a, int t,
                                                     const float4 (&v)[QueryTermsMx::NG + 1],
                                                     uint8_t* qt, int* s_k)
{
    using Q = QueryTermsMx;
    const int h = t >> 4, i = t & 15;
    const int hh = h >> 4, n = h & 15;
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < Q::NG; ++s)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[s].x), fabsf(v[s].y)),
                                 fmaxf(fabsf(v[s].z), fabsf(v[s].w))));
    amax = row16_max(amax);
    const float es = a.sm_log2;
    const int k = query_exp(amax * es);
    if (i == 0)
        s_k[h] = k;
    const float mult = ldexpf(es, k);
#pragma unroll
    for (int s = 0; s < Q::NG; ++s) {
        float r[4] = {v[s].x * mult, v[s].y * mult, v[s].z * mult, v[s].w * mult};
        asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));  // as above
        put_query_f16<Q::NP>(qt, hh, n, i + 16 * s, r);
    }
    // RoPE elements 4 i .. 4 i + 3: K step m = i / 8, lane group (i / 2) % 4,
    // bf16 positions 4 (i % 2) .. + 3
    const float4 e4 = v[Q::NG];
    const float e[4] = {e4.x * es, e4.y * es, e4.z * es, e4.w * es};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        hi[c] = bf16_rne_bits(e[c]);
        lo[c] = bf16_rne_bits(e[c] - __uint_as_float(hi[c] << 16));
    }
    const int m = i >> 3, gl = (i >> 1) & 3, pos = 4 * (i & 1);
    uint8_t* rb = qt + Q::RBASE;
    auto put2 = [&](int slot, const uint32_t (&w)[4]) __attribute__((always_inline)) {
        *reinterpret_cast<uint2*>(rb + (((hh * Q::NRS + slot) * 64 + n + 16 * gl) * 16 +
                                        2 * pos)) =
            make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
    };
    put2(2 * m, hi);
    put2(2 * m + 1, lo);
}

// Byte offsets of the split-T partial kernel's LDS objects (one array, so the
// query-term staging area can reuse ring stages 1-3 before they fill).
//
// A ring stage holds one 64-row tile, laid out for the readers rather than
// row by row: row quarter rq (rows 16 rq .. +16) is a block of NKB KB; inside
// it, for every 128-byte column block j and half h, the 16-byte chunks
// (row 16 rq + n, chunk 8 j + 2 g + h) sit at slot n + 16 g of a 1-KB group
// (a 512-byte group of slots n + 16 g, g < 2, for a trailing half block).  A
// score read (lane n + 16 g, block j, half h) is then one linear 1-KB read and
// a transposed context read (8 rows x 16 bytes per 16 lanes) one linear
// 128-byte read: no LDS bank conflicts.  The direct loads choose, lane by
// lane, which 16 bytes of HBM land in each slot.
template <int NKB, bool MXL = false>
struct PartialLds {
    static constexpr int TR = kTileRows;
    static constexpr int NW = kThreads / 64;
    static constexpr int HG = kHeadsPerGroup;
    static constexpr int NB = (NKB + 1) / 2;   // 128-wide K blocks of the scores
    static constexpr int NFULL = NKB / 2;      // full 128-byte blocks
    static constexpr int ROWB = 64 * NKB;      // padded row bytes
    static constexpr int RQB = 16 * ROWB;      // one row quarter (NKB KB)
    static constexpr int STAGE = TR * ROWB;    // one ring stage
    static constexpr int WSS = TR + 8;         // weight-tile stride (halves)
    static constexpr int FIXED = 2 * HG * WSS * 2 + 2 * HG * 4 * 4 + HG * 4 * 8 +
                                 4 * HG * 4 + HG * 4;
    static constexpr int LIMIT = 160 * 1024;
    // Ring stages: 4 (loads issued two tiles ahead) when they fit, else 3
    // (one tile ahead).  A stage is read in two phases (scores, then context).
    static constexpr int NST = (4 * (STAGE + 2 * TR * 4) + FIXED <= LIMIT) ? 4 : 3;
    static constexpr int DIST = NST - 2;  // tiles issued ahead
    static constexpr int SC = NST * STAGE;                 // f32 [NST][TR] row scales
    static constexpr int ROW = SC + NST * TR * 4;          // i32 [NST][TR] (gathered rows)
    static constexpr int W = ROW + NST * TR * 4;           // f16 [2][HG][WSS] weights
    static constexpr int MX = W + 2 * HG * WSS * 2;        // f32 [2][HG][4] tile check sums
    static constexpr int CR = MX + 2 * HG * 4 * 4;         // float2 [HG][4] exact tile maxima
    static constexpr int Z = CR + HG * 4 * 8;              // f32 [4][HG]
    static constexpr int HK = Z + 4 * HG * 4;              // i32 [HG] query exponent k
    static constexpr int END = HK + HG * 4;
    // query terms, both head halves
    static constexpr int QT_BYTES = MXL ? QueryTermsMx::BYTES : QueryTerms<NKB>::BYTES;
    // The staging area reuses the stages that are not filled before the
    // terms are built (tiles 0 .. DIST-1 are already in flight then).
    static constexpr int QT = (DIST * STAGE + QT_BYTES <= SC) ? DIST * STAGE : END;
    static constexpr int TOTAL = (QT + QT_BYTES > END) ? QT + QT_BYTES : END;
    static_assert(STAGE % 1024 == 0, "stages are whole DMA blocks");
    static_assert(TOTAL <= LIMIT, "LDS budget");
};

// Value of quad lane V broadcast to the four lanes of every quad.
template <int V>
__device__ __forceinline__ float quad_bcast(float x)
{
    return __int_as_float(
        __builtin_amdgcn_mov_dpp(__float_as_int(x), V * 0x55, 0xF, 0xF, false));
}

typedef int v2i __attribute__((ext_vector_type(2)));

// Split-T partial.  Grid: n_chunks * n_groups workgroups of 512 threads (8
// waves, two per SIMD).  NKB = number of 64-byte blocks of the padded row.
// The waves take two roles, one of each per SIMD, so that the MFMA-heavy score
// work of one overlaps the conversion and softmax work of the other:
//   score waves (0-3): rows 32*(w>>1) .. +32 of each tile against heads
//            16*(w&1) .. +16 of the group: the fp16 hi + lo query operands in
//            registers x the row bytes widened to fp16, on the fp16 MFMA;
//            then the weights and the check sums;
//   context waves (4-7): context columns 128*(w-4) .. +128 for all 32 heads;
//            the row bytes are read transposed (ds_read_b64_tr_b8) so the row
//            index lands on the MFMA K index, widened to fp16 exactly; they
//            also issue every direct load of the row stream.
//   loads  : 64-row tiles stream HBM -> LDS through a ring of direct
//            global_load_lds_dwordx4 (no register staging).
// One barrier per tile: in phase p the score waves score tile p and write its
// weights with the softmax state as it stands, while the context waves
// accumulate tile p-1; both first vote on tile p-1's maxima against that
// state.
template <int NKB, bool GATHER, bool MXL = false>
__global__ __launch_bounds__(kThreads, 1) void k_split_partial(AttnArgs a)
{
    using L = PartialLds<NKB, MXL>;
    using Q = QueryTerms<NKB>;
    using QM = QueryTermsMx;
    static_assert(!MXL || NKB == 9, "mixed rows: the 448 / 64 shape");
    constexpr int NSL = MXL ? QM::NSLOT : Q::NSLOT;  // fp16 query operand slots
    constexpr int TR = L::TR, NW = L::NW, HG = L::HG, NB = L::NB, NFULL = L::NFULL;
    constexpr int RQB = L::RQB, WSS = L::WSS, NST = L::NST, DIST = L::DIST;
    constexpr int NINS = L::STAGE / 1024;     // 1-KB DMA instructions per tile
    constexpr int NWI = NW / 2;               // waves that issue the direct loads
    constexpr int KW = (NINS + NWI - 1) / NWI;  // row DMA instructions per issuing wave per tile
    static_assert(KW + 1 < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[L::TOTAL];
    float* const s_sc = reinterpret_cast<float*>(lds + L::SC);
    int32_t* const s_row = reinterpret_cast<int32_t*>(lds + L::ROW);
    _Float16* const s_w = reinterpret_cast<_Float16*>(lds + L::W);
    float* const s_mx = reinterpret_cast<float*>(lds + L::MX);
    float* const s_cr = reinterpret_cast<float*>(lds + L::CR);
    float* const s_z = reinterpret_cast<float*>(lds + L::Z);
    int* const s_k = reinterpret_cast<int*>(lds + L::HK);
    // LDS byte address of the array (wave-uniform; the direct loads take it in m0)
    const uint32_t lds_u32 = (uint32_t)(uintptr_t)(MLA8_LDS uint8_t*)lds;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
    const int hh = w & 1;  // head half of the group a score wave scores

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

    // ---- tile issue.  The context waves (w >= NWI) issue every direct load:
    // KW row DMAs per tile each and the first of them one more for the row
    // scales, so a fixed per-wave vmcnt marks a tile complete.  The score
    // waves issue none (their phase is the longer one; sharing the loads
    // between both roles measured slower).  Row DMA instruction k fills stage
    // slots [64k, 64k + 64) (16 bytes each, layout above).  Slots past the
    // row's data (zero-pad columns) and rows outside the list load chunk 0 /
    // the tile's first row instead: finite bytes that are multiplied by a zero
    // query element, masked out of the softmax, or never read.  Spare
    // instruction slots (k >= NINS) repeat instruction k % NINS (the same
    // bytes to the same place).
    const int cpr = a.d >> 4;  // 16-byte data chunks per row
    const int wi = (w >= NWI) ? w - NWI : 0;  // issuer index
    const bool dma_lead = w == NWI;           // issues the scale loads too
    auto row_of = [&](int pos) __attribute__((always_inline)) -> int32_t {
        if (pos >= c1)
            return -1;
        const int32_t r = a.sel[pos];
        return (r >= 0 && r < a.t_rows) ? r : -1;
    };
    // Per row DMA i of this wave: r << 16 | (r * d + chunk offset), the same
    // for every tile, so it is packed once.
    int dpk[KW];
    // LDS byte offset of this wave's row DMA i within a stage (wave-uniform,
    // kept in scalar registers)
    uint32_t kofs[KW];
#pragma unroll
    for (int i = 0; i < KW; ++i)
        kofs[i] = __builtin_amdgcn_readfirstlane((uint32_t)(1024 * ((wi + NWI * i) % NINS)));
#pragma unroll
    for (int i = 0; i < KW; ++i) {
        const int k = (wi + NWI * i) % NINS;
        const int sl = 64 * k + lane;
        const int q4 = sl / (64 * NKB), s1 = sl - q4 * (64 * NKB);
        int j, h, ln;
        if (s1 < NFULL * 128) {
            j = s1 >> 7;
            h = (s1 >> 6) & 1;
            ln = s1 & 63;
        } else {
            j = NFULL;
            h = (s1 - NFULL * 128) >> 5;
            ln = s1 & 31;
        }
        const int r = 16 * q4 + (ln & 15), c16 = 8 * j + 2 * (ln >> 4) + h;
        dpk[i] = (r << 16) | (r * a.d + (c16 < cpr ? 16 * c16 : 0));
    }
    // Direct loads [I0, I1) of tile t into stage st (the last part also
    // carries the scale load and, for a gather, the row indices).  A tile's
    // loads are spread over its issuing phase so that the eight waves do not
    // all queue on the load path at once.
    auto issue = [&](int t, int st, auto I0_, auto I1_) __attribute__((always_inline)) {
        constexpr int I0 = decltype(I0_)::value, I1 = decltype(I1_)::value;
        constexpr bool LAST = I1 == KW;
        const uint32_t xst = lds_u32 + (uint32_t)(st * L::STAGE);
        const uint32_t sct = lds_u32 + (uint32_t)(L::SC + st * TR * 4);
        const int p0 = c0 + t * TR;
        if constexpr (!GATHER) {
            // Contiguous rows p0 .. p0 + nv - 1: SGPR base + 32-bit offsets.
            // Rows past the list reload the tile's first row.
            const int nv = c1 - p0;
            const uint8_t* tb = a.codes + (size_t)p0 * a.d;
            if (nv >= TR) {
#pragma unroll
                for (int i = I0; i < I1; ++i)
                    dma_b128_s(tb, (uint32_t)(dpk[i] & 0xFFFF), xst + kofs[i]);
                if (LAST && dma_lead)
                    dma_b32_s(a.scales + p0, (uint32_t)(4 * lane), sct);
            } else {
#pragma unroll
                for (int i = I0; i < I1; ++i) {
                    const int r = dpk[i] >> 16;
                    const uint32_t off =
                        (uint32_t)((dpk[i] & 0xFFFF) - (r < nv ? 0 : r * a.d));
                    dma_b128_s(tb, off, xst + kofs[i]);
                }
                if (LAST && dma_lead)
                    dma_b32_s(a.scales + p0, (uint32_t)(4 * (lane < nv ? lane : 0)), sct);
            }
        } else {
            // Gather: absolute row indices; entries outside [0, t_rows) and
            // positions past the list reload row 0.  The indices are all
            // loaded before the first direct load of the part is issued.
            int32_t rows[(I1 > I0) ? I1 - I0 : 1];
#pragma unroll
            for (int i = I0; i < I1; ++i)
                rows[i - I0] = row_of(p0 + (dpk[i] >> 16));
            int32_t srow = 0;
            if (LAST && dma_lead)
                srow = row_of(p0 + lane);
#pragma unroll
            for (int i = I0; i < I1; ++i) {
                const int r = dpk[i] >> 16;
                const int cc = (dpk[i] & 0xFFFF) - r * a.d;
                const int32_t row = rows[i - I0];
                dma_b128(a.codes + (size_t)(row >= 0 ? row : 0) * a.d + cc, xst + kofs[i]);
            }
            if (LAST && dma_lead) {
                dma_b32(a.scales + (srow >= 0 ? srow : 0), sct);
                s_row[st * TR + lane] = srow;
            }
        }
    };
    using IC0 = std::integral_constant<int, 0>;
    using ICA = std::integral_constant<int, (KW + 2) / 3>;
    using ICB = std::integral_constant<int, (2 * KW + 2) / 3>;
    using ICK = std::integral_constant<int, KW>;
    auto issue_all = [&](int t, int st) __attribute__((always_inline)) {
        issue(t, st, IC0{}, ICK{});
    };
    // Tile t is complete once at most tile t+1's operations remain in flight
    // (two tiles ahead) or none (one tile ahead).
    auto wait_tile = [&](bool next_in_flight) __attribute__((always_inline)) {
        if (DIST == 2 && next_in_flight) {
            if (dma_lead)
                wait_vmcnt<KW + 1>();
            else
                wait_vmcnt<KW>();
        } else {
            wait_vmcnt<0>();
        }
    };

    // ---- fused append: fresh rows [f0, f1) inside this chunk are quantized
    // into the shadow by this workgroup (every head group of the chunk writes
    // the same bytes) before any wave streams them.  Vector memory operations
    // of a wave complete in issue order, so stores issued before the first
    // tile's loads are complete once phase 1 has waited for its tile, and the
    // phase barrier orders them before any wave's later loads: a chunk whose
    // fresh rows start at tile DIST + 1 or later has them quantized after the
    // prologue by the context waves, which wait for their loads every phase
    // (the stall on the fresh row's load then overlaps the first tiles'
    // loads).  Otherwise every wave quantizes, and waits, before the first
    // load is issued.
    int f0 = 0, f1 = 0;
    if (a.n_new > 0) {
        f0 = max(c0, a.new0);
        f1 = min(c1, a.new0 + a.n_new);
    }
    const bool fresh_late = f0 < f1 && (f0 - c0) / TR >= DIST + 1;
    // (mixed rows: an input row is lc + rc f32 values, a stored row a.d bytes)
    auto quantize_fresh = [&](int first, int stride) __attribute__((always_inline)) {
        for (int r = f0 + first; r < f1; r += stride) {
            if constexpr (MXL)
                quantize_row_mx_wave(a.x_new + (size_t)(r - a.new0) * (a.lc + a.rc), a.lc, a.rc,
                                     a.new_codes + (size_t)r * a.d, a.new_scales + r, lane);
            else
                quantize_row_wave(a.x_new + (size_t)(r - a.new0) * a.d, a.d,
                                  a.new_codes + (size_t)r * a.d, a.new_scales + r, lane);
        }
    };
    if (f0 < f1 && !fresh_late) {
        quantize_fresh(w, NW);
        wait_vmcnt<0>();
        __syncthreads();
    }

    // ---- prologue: every wave builds the query operands of one head half
    // (work items tid: score waves head half 0, context waves head half 1)
    // into an LDS staging area over the ring stages not yet in flight; the
    // context waves send their query loads first, then issue the first tiles'
    // direct loads, then build.  The score waves keep their head half's
    // operands in registers after the barrier.  (Measured: the score waves
    // building both halves kept the context waves idle at the barrier for
    // about 6,800 cycles; sharing the build shortens the prologue by about
    // 1 us.)
    if (w >= NWI) {
        if constexpr (MXL) {
            float4 qin[QM::NG + 1];
            load_query_mx(a, qh0, tid, qin);
            if (ntiles > 0)
                issue_all(0, 0);
            if (DIST == 2 && ntiles > 1)
                issue_all(1, 1);
            build_query_terms_mx(a, tid, qin, lds + L::QT, s_k);
        } else {
            float4 qin[2 * NB];
            load_query<NKB>(a, qh0, tid, qin);
            if (ntiles > 0)
                issue_all(0, 0);
            if (DIST == 2 && ntiles > 1)
                issue_all(1, 1);
            build_query_terms<NKB>(a, tid, qin, lds + L::QT, s_k);
        }
    } else if constexpr (MXL) {
        float4 qin[QM::NG + 1];
        load_query_mx(a, qh0, tid, qin);
        build_query_terms_mx(a, tid, qin, lds + L::QT, s_k);
    } else {
        float4 qin[2 * NB];
        load_query<NKB>(a, qh0, tid, qin);
        build_query_terms<NKB>(a, tid, qin, lds + L::QT, s_k);
    }
    lds_barrier();

    // Softmax state, identical in every wave, for heads n and 16 + n of the
    // group: m = lazy max of u (z side), d = lazy max of (u - m) + log2 scale
    // (context side, relative to m).  The weights of tile p are computed with
    // the state as it stands, in the linear domain:
    //     p_t = 2^(u_t - m),  w_t = p_t * (scale_t * 2^-d),
    // and the tile's sums of p + w per (head, row quarter) are checked one
    // phase later.  Only when a sum leaves [0, 2^kTau] (a new maximum by more
    // than kTau, the first tile, or an intermediate that left f32's range) is
    // the state recomputed exactly in the log domain, the context rescaled and
    // the tile's weights rewritten (as 2^((u - m) + log2 scale - d)).
    // (separate scalars, never an array: a lane-dependent pick from an array
    // would put it in scratch memory)
    float mrun0 = -INFINITY, mrun1 = -INFINITY, drun0 = -INFINITY, drun1 = -INFINITY;
    float fown = 1.0f;  // 2^-d of head 16 hh + n (2^0 while d = -inf); score waves
    // A head whose m is still -inf has not met a valid row, and the linear
    // weights of a first valid row may underflow to a zero sum: while any head
    // of the group is in that state every check takes the exact path
    // (uniform: every wave holds the same state).
    bool uninit = true;
    constexpr float kCheck = 256.0f;  // 2^kTau
    static_assert(kTau == 8.0f, "check threshold");
    float2* const s_cr2 = reinterpret_cast<float2*>(s_cr);

    // Vote on tile p-1 (weight buffer bufp): every wave reads the same sums
    // and holds the same state, so the result is uniform across the
    // workgroup and the barriers of the exact path are reached by all waves
    // or none.
    auto vote_read = [&](int bufp, float4 (&S4)[2]) __attribute__((always_inline)) {
        const float* mxp = s_mx + bufp * HG * 4;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
            S4[ht] = *reinterpret_cast<const float4*>(mxp + (16 * ht + n) * 4);
    };
    auto vote = [&](const float4 (&S4)[2]) __attribute__((always_inline)) -> bool {
        bool moved = false;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)  // false for NaN: a non-finite intermediate also recomputes
            moved |= !(fmaxf(fmaxf(S4[ht].x, S4[ht].y), fmaxf(S4[ht].z, S4[ht].w)) <= kCheck);
        return uninit || __any(moved);
    };
    // Exact state move from the tile maxima (T, C) per (head, row quarter) in
    // s_cr; alz / alo receive the factors for z and for the context
    // accumulators of heads n, 16 + n.
    auto state_move = [&](float (&alz)[2], float (&alo)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int h = 16 * ht + n;
            const float4 r01 = *reinterpret_cast<const float4*>(&s_cr2[h * 4]);
            const float4 r23 = *reinterpret_cast<const float4*>(&s_cr2[h * 4 + 2]);
            const float Tk[4] = {r01.x, r01.z, r23.x, r23.z};
            const float Ck[4] = {r01.y, r01.w, r23.y, r23.w};
            const float T = fmaxf(fmaxf(Tk[0], Tk[1]), fmaxf(Tk[2], Tk[3]));
            float& mr = ht ? mrun1 : mrun0;
            float& dr = ht ? drun1 : drun0;
            const float mold = mr;
            const float mnew = (T > mold + kTau) ? T : mold;
            alz[ht] = (mnew == mold) ? 1.0f : fast_exp2(mold - mnew);
            const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
            float tb = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (Tk[k] != -INFINITY)
                    tb = fmaxf(tb, Ck[k] + (Tk[k] - mu));
            const float dshift = (mnew == mold) ? dr : dr + (mold - mnew);
            const float dnew = (tb > dshift + kTau) ? tb : dshift;
            alo[ht] = (dnew == dshift) ? 1.0f : fast_exp2(dshift - dnew);
            mr = mnew;
            dr = dnew;
        }
        const float dd = hh ? drun1 : drun0;
        fown = (dd == -INFINITY) ? 1.0f : fast_exp2(-dd);
        uninit = __any(mrun0 == -INFINITY || mrun1 == -INFINITY);
    };
    const size_t pbase = (size_t)chunk * a.n_qh;

    // Phase p (one barrier): the score waves score tile p (ring stage p % NST)
    // and write its weights into buffer p & 1; the context waves accumulate
    // tile p-1 from the previous buffer.  Both vote on tile p-1 first.  One
    // extra phase finishes the last tile.
    if (w < NW / 2) {
        // ======== score waves: rows 32 rh .. +32 (row quarters 2 rh, 2 rh + 1),
        // heads 16 hh .. +16
        const int rh = w >> 1;
        f16x8 qv[NSL];
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
            qv[sl] = *reinterpret_cast<const f16x8*>(
                lds + L::QT + ((hh * NSL + sl) * 64 + lane) * 16);
        // mixed rows: the RoPE query terms (bf16), two per K step
        bf16x8 qr[MXL ? QM::NRS : 1];
        if constexpr (MXL) {
#pragma unroll
            for (int sl = 0; sl < QM::NRS; ++sl)
                qr[sl] = *reinterpret_cast<const bf16x8*>(
                    lds + L::QT + QM::RBASE + ((hh * QM::NRS + sl) * 64 + lane) * 16);
        }
        // 2^-k of this lane's head: the accumulators hold 2^k times its scores
        const float pk = ldexpf(1.0f, -s_k[16 * hh + n]);
        const int qh_own = qh0 + 16 * hh + n;
        const int32_t tlim = (a.mode == kCausal)
                                 ? a.pos0 + (qh_own < a.n_qh ? qh_own / a.n_heads : 0) + 1
                                 : 0x7FFFFFFF;
        lds_barrier();  // staging area free for the ring

        float zacc = 0.0f;   // z partial over this lane's rows, head 16 hh + n
        float zsave = 0.0f;  // zacc before the last scored tile
        float u[8], scv[8];  // scores / row scales of the last scored tile, [quarter][v]
        // weights of rows 32 rh + 16 r + 4 g + v, head 16 hh + n
        _Float16* const s_w_own = s_w + (16 * hh + n) * WSS + 32 * rh + 4 * g;

        // Weights of this lane's rows (linear form) into buffer buf; chk[r]
        // receives this lane's sum of p + w in row quarter 2 rh + r.
        auto weights_linear = [&](int buf, float (&chk)[2]) __attribute__((always_inline)) {
            const float mu = hh ? mrun1 : mrun0;
            const float mz = (mu == -INFINITY) ? 0.0f : mu;
            float ps = 0.0f;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                f16x4 wv;
                chk[r] = 0.0f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float pv = fast_exp2(u[4 * r + v] - mz);
                    const float wt = pv * (scv[4 * r + v] * fown);
                    ps += pv;
                    chk[r] += pv + wt;
                    wv[v] = (_Float16)wt;
                }
                *reinterpret_cast<f16x4*>(s_w_own + buf * HG * WSS + 16 * r) = wv;
            }
            zacc = zsave + ps;
        };
        // Same in the log domain (exact for any scale), used after a state move.
        auto weights_log = [&](int buf) __attribute__((always_inline)) {
            const float mu = hh ? mrun1 : mrun0;
            const float dd = hh ? drun1 : drun0;
            const float mz = (mu == -INFINITY) ? 0.0f : mu;
            const float dn = (dd == -INFINITY) ? 0.0f : dd;
            float ps = 0.0f;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                f16x4 wv;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float av = u[4 * r + v] - mz;
                    ps += fast_exp2(av);
                    wv[v] = (_Float16)fast_exp2((av + log2f(scv[4 * r + v])) - dn);
                }
                *reinterpret_cast<f16x4*>(s_w_own + buf * HG * WSS + 16 * r) = wv;
            }
            zacc = zsave + ps;
        };

        // Scores of tile p (stage st): S^T[16 rows][16 heads] per row quarter,
        // 2^k times the log2-domain score in code units; the hi and lo
        // operands accumulate apart and the two quarters' MFMAs alternate, so
        // consecutive MFMAs never wait on each other.  Lane (n, g) of full
        // block j reads slot n + 16 g of groups (j, 0) and (j, 1) of its row
        // quarter (elements 128 j + 32 g .. +31); of the half block, chunk g:
        // slot n + 16 (g >> 1) of group (j, g & 1).  Mixed rows: the noPE half
        // block is the first half of LDS block 3 (a full 1-KB group pair);
        // RoPE K step m reads 16-byte chunk 28 + 4m + g of row 16 rq + n, in
        // LDS block 3 (m = 0, lane groups 2-3) or in the trailing half block 4
        // (m = 1, lane groups 0-1).
        constexpr int QNF = MXL ? QM::NP::NFULL : Q::NFULL;
        constexpr bool QHALF = MXL ? QM::NP::HALF : Q::HALF;
        constexpr int HGS = MXL ? 1024 : 512;  // group size of the half block's LDS block
        const int qa = 2 * rh * RQB + 16 * lane;
        const int qa_h = 2 * rh * RQB + QNF * 2048 + (g & 1) * HGS + 16 * (n + 16 * (g >> 1));
        const int ro0 = 2 * rh * RQB + 3 * 2048 + (g & 1) * 1024 + 16 * (n + 16 * (2 + (g >> 1)));
        const int ro1 = 2 * rh * RQB + 4 * 2048 + (g & 1) * 512 + 16 * (n + 16 * (g >> 1));
        f32x4 acc0[2], acc1[2], accr[2];
        auto step = [&](const f16x8 (&xa)[2], int sl) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
                acc0[r] = mfma16(xa[r], qv[sl], acc0[r]);
#pragma unroll
            for (int r = 0; r < 2; ++r)
                acc1[r] = mfma16(xa[r], qv[sl + 1], acc1[r]);
        };
        auto scores = [&](int st) __attribute__((always_inline)) {
            const uint8_t* xst = lds + st * L::STAGE;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                acc0[r] = f32x4{0.f, 0.f, 0.f, 0.f};
                acc1[r] = acc0[r];
                accr[r] = acc0[r];
            }
#pragma unroll
            for (int j = 0; j < QNF; ++j) {
                uint4 x0[2], x1[2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const uint8_t* xp = xst + qa + 2048 * j + r * RQB;
                    x0[r] = *reinterpret_cast<const uint4*>(xp);
                    x1[r] = *reinterpret_cast<const uint4*>(xp + 1024);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    f16x8 xa[2];
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const uint4 x = (s < 2) ? x0[r] : x1[r];
                        xa[r] = (s & 1) ? cvt8(x.z, x.w) : cvt8(x.x, x.y);
                    }
                    step(xa, 8 * j + 2 * s);
                }
            }
            if constexpr (QHALF) {
                uint4 xh[2];
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    xh[r] = *reinterpret_cast<const uint4*>(xst + qa_h + r * RQB);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    f16x8 xa[2];
#pragma unroll
                    for (int r = 0; r < 2; ++r)
                        xa[r] = s ? cvt8(xh[r].z, xh[r].w) : cvt8(xh[r].x, xh[r].y);
                    step(xa, 8 * QNF + 2 * s);
                }
            }
            if constexpr (MXL) {
#pragma unroll
                for (int m = 0; m < QM::NRS / 2; ++m) {
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const bf16x8 xr =
                            *reinterpret_cast<const bf16x8*>(xst + (m ? ro1 : ro0) + r * RQB);
                        accr[r] = mfma_bf16(xr, qr[2 * m], accr[r]);
                        accr[r] = mfma_bf16(xr, qr[2 * m + 1], accr[r]);
                    }
                }
            }
        };
        // Log2-domain scores u of tile p (rows 32 rh + 16 r + 4 g + v, head
        // 16 hh + n) from the accumulators; masking: rows past the list,
        // invalid gathered rows, causal limit.
        auto scores_to_u = [&](const float4 (&scl)[2], int st, int p0, bool mask)
                               __attribute__((always_inline)) {
            zsave = zacc;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float4 sc4 = scl[r];
                scv[4 * r + 0] = sc4.x;
                scv[4 * r + 1] = sc4.y;
                scv[4 * r + 2] = sc4.z;
                scv[4 * r + 3] = sc4.w;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    u[4 * r + v] = MXL ? ((acc0[r][v] + acc1[r][v]) * pk) * scv[4 * r + v] + accr[r][v]
                                       : ((acc0[r][v] + acc1[r][v]) * pk) * scv[4 * r + v];
            }
            if (mask) {
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int row = 32 * rh + 16 * r + 4 * g + v;
                        bool valid;
                        if constexpr (GATHER) {
                            valid = s_row[st * TR + row] >= 0;
                        } else {
                            valid = p0 + row < c1 && p0 + row < tlim;
                        }
                        u[4 * r + v] = valid ? u[4 * r + v] : -INFINITY;
                    }
            }
        };

        for (int p = 0, st = 0; p <= ntiles; ++p, st = (st == NST - 1) ? 0 : st + 1) {
            const int buf = p & 1, bufp = buf ^ 1;
            lds_barrier();  // (A) tile p visible; weights and sums of tile p-1
                            //     complete; stage (p + DIST) % NST (tile p + DIST
                            //     - NST) and buffer p & 1 free
            // the sums of tile p-1 and the scales of tile p are read ahead of
            // the score operands, so they do not queue behind them
            float4 S4[2];
            if (p >= 1)
                vote_read(bufp, S4);
            const bool scored = p < ntiles;
            float4 scl[2];
            if (scored) {
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    scl[r] = *reinterpret_cast<const float4*>(s_sc + st * TR + 32 * rh + 16 * r + 4 * g);
                scores(st);
            }
            if (p >= 1 && vote(S4)) {
                // Keep this path's arithmetic inside the branch: the empty asm
                // makes u and the scales opaque here, so none of it is hoisted
                // into the common path.
                asm volatile("" : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3]), "+v"(u[4]),
                             "+v"(u[5]), "+v"(u[6]), "+v"(u[7]), "+v"(scv[0]), "+v"(scv[1]),
                             "+v"(scv[2]), "+v"(scv[3]), "+v"(scv[4]), "+v"(scv[5]),
                             "+v"(scv[6]), "+v"(scv[7]));
                // exact maxima of tile p-1 per row quarter: T = max u, C =
                // max (u - T) + log2 scale, relative so that a large |u| never
                // swallows log2 scale
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    float tw = fmaxf(fmaxf(u[4 * r], u[4 * r + 1]), fmaxf(u[4 * r + 2], u[4 * r + 3]));
                    tw = max_xor32(max_xor16(tw));
                    float cw = -INFINITY;
                    if (tw != -INFINITY) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            cw = fmaxf(cw, (u[4 * r + v] - tw) + log2f(scv[4 * r + v]));
                    }
                    cw = max_xor32(max_xor16(cw));
                    if (g == 0)
                        s_cr2[(16 * hh + n) * 4 + 2 * rh + r] = make_float2(tw, cw);
                }
                lds_barrier();  // (R1)
                float alz[2], alo[2];
                state_move(alz, alo);
                zsave *= hh ? alz[1] : alz[0];
                weights_log(bufp);  // tile p-1 under the new state
                lds_barrier();      // (R2) rewritten weights visible; s_cr free
            }
            float chk[2] = {0.0f, 0.0f};
            if (scored) {
                const int p0 = c0 + p * TR;
                const bool full = !GATHER && a.mode != kCausal && p0 + TR <= c1;
                scores_to_u(scl, st, p0, !full);
                weights_linear(buf, chk);
            }
            if (p == ntiles)
                break;
            // sums of p + w over the 16 rows of each row quarter (lane groups g)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                float cs = chk[r];
                const auto r1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(cs),
                                                                 __float_as_uint(cs), false, false);
                cs = __uint_as_float(r1[0]) + __uint_as_float(r1[1]);
                const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(cs),
                                                                 __float_as_uint(cs), false, false);
                cs = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
                if (g == 0)
                    s_mx[(buf * HG + 16 * hh + n) * 4 + 2 * rh + r] = cs;
            }
        }
        // z over lane groups
        float zz = zacc;
        zz += __shfl_xor(zz, 16);
        zz += __shfl_xor(zz, 32);
        if (g == 0)
            s_z[rh * HG + 16 * hh + n] = zz;
    } else {
        // ======== context waves: O[32 heads][128 columns 128 c ..] += W . X of
        // tile p-1.  Column tile jm (16 columns) is chunk 8 c + jm: LDS block
        // c, lane group jm / 2, half jm % 2.  MFMA (ht, jm) covers heads
        // 16 ht .. +16.
        const int c = w - NW / 2;
        const int nct = min(8, max(0, (a.lc >> 4) - 8 * c));  // 16-column tiles of this wave
        const bool ctx_half = c >= NFULL;  // the wave's block is a trailing half block
        // Context operand: source lane 2k + h' of 16-lane group g' addresses
        // row 8 g' + k (row quarter g' / 2, slot n = 8 (g' & 1) + k), bytes
        // 8 h' .. of the column chunk; the transposed read hands lane (n, g')
        // column n of rows 8 g' .. 8 g' + 7.
        const int trl = (g >> 1) * RQB + 16 * (8 * (g & 1) + ((lane & 15) >> 1)) + 8 * (lane & 1);
        const int trw = ctx_half ? NFULL * 2048 : c * 2048;
        lds_barrier();  // staging area free for the ring
        if (fresh_late)
            quantize_fresh(wi, NWI);
        f32x4 O[2][8];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int jm = 0; jm < 8; ++jm)
                O[ht][jm] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Operands of one tile: the weights (A, heads x rows) and the row
        // bytes read transposed (B, rows x columns).  The reads of tile p-1
        // go out together with the vote on it; only a state move (which
        // rewrites the tile's weights) makes the weights be read again.
        constexpr int KS = TR / 32;
        f16x8 wa[KS][2];
        v2i xb[KS][8];
        auto read_weights = [&](int buf) __attribute__((always_inline)) {
            const _Float16* sw = s_w + buf * HG * WSS;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int ht = 0; ht < 2; ++ht)
                    wa[ks][ht] =
                        *reinterpret_cast<const f16x8*>(&sw[(16 * ht + n) * WSS + 32 * ks + 8 * g]);
        };
        auto read_rows = [&](int st, auto GUARD_, auto HALF_) __attribute__((always_inline)) {
            constexpr bool GUARD = decltype(GUARD_)::value, HALFC = decltype(HALF_)::value;
            const uint8_t* xst = lds + st * L::STAGE + trw + trl;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int jm = 0; jm < 8; ++jm) {
                    if (GUARD && jm >= nct)
                        break;
                    const int off = 2 * ks * RQB + (jm & 1) * (HALFC ? 512 : 1024) + (jm >> 1) * 256;
                    xb[ks][jm] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (MLA8_LDS v2i*)(MLA8_LDS uint8_t*)(xst + off));
                }
        };
        auto accumulate = [&](auto GUARD_) __attribute__((always_inline)) {
            constexpr bool GUARD = decltype(GUARD_)::value;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int jm = 0; jm < 8; ++jm) {
                    if (GUARD && jm >= nct)
                        break;
                    const f16x8 bx = cvt8((uint32_t)xb[ks][jm][0], (uint32_t)xb[ks][jm][1]);
                    O[0][jm] = mfma16(wa[ks][0], bx, O[0][jm]);
                    O[1][jm] = mfma16(wa[ks][1], bx, O[1][jm]);
                }
        };

        for (int p = 0, st = 0, stp = NST - 1; p <= ntiles;
             ++p, stp = st, st = (st == NST - 1) ? 0 : st + 1) {
            // st = p % NST, stp = (p - 1) % NST
            const int bufp = (p & 1) ^ 1;
            if (p < ntiles)
                wait_tile(p + 1 < ntiles);
            lds_barrier();  // (A)
            const bool more = p + DIST < ntiles;
            const int sti = (st + DIST) % NST;
            const bool ctx = p >= 1 && nct > 0;
            float4 S4[2];
            if (p >= 1)
                vote_read(bufp, S4);
            if (ctx) {
                read_weights(bufp);
                if (ctx_half)
                    read_rows(stp, std::true_type{}, std::true_type{});
                else if (nct < 8)
                    read_rows(stp, std::true_type{}, std::false_type{});
                else
                    read_rows(stp, std::false_type{}, std::false_type{});
            }
            if (more)
                issue(p + DIST, sti, IC0{}, ICA{});
            if (p >= 1 && vote(S4)) {
                lds_barrier();  // (R1) the score waves' tile maxima are in s_cr
                float alz[2], alo[2];
                state_move(alz, alo);
                // O holds tiles < p-1 in units of the old state; its heads
                // 16*ht + 4*g + v take their factors from lanes 4*g + v.
#pragma unroll
                for (int ht = 0; ht < 2; ++ht)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float f = __shfl(alo[ht], 4 * g + v);
#pragma unroll
                        for (int jm = 0; jm < 8; ++jm)
                            O[ht][jm][v] *= f;
                    }
                lds_barrier();  // (R2) the rewritten weights of tile p-1 are visible
                if (ctx)
                    read_weights(bufp);
            }
            if (more)
                issue(p + DIST, sti, ICA{}, ICB{});
            if (ctx) {
                if (nct < 8)
                    accumulate(std::true_type{});
                else
                    accumulate(std::false_type{});
            }
            if (more)
                issue(p + DIST, sti, ICB{}, ICK{});
            if (p == ntiles)
                break;
        }
        // partial cl = sum_t p_t scale_t x_t = 2^d * O
        if (nct > 0) {
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) {
                const float mh = ht ? mrun1 : mrun0, dh = ht ? drun1 : drun0;
                const float fo = (mh == -INFINITY || dh == -INFINITY) ? 0.0f : fast_exp2(dh);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float f = __shfl(fo, 4 * g + v);
                    const int qh = qh0 + 16 * ht + 4 * g + v;
                    if (qh < a.n_qh) {
                        // streaming stores: the merge reads them once, from beyond L2
                        float* dst = a.ws_cl + (pbase + qh) * a.lc + 128 * c + n;
#pragma unroll
                        for (int jm = 0; jm < 8; ++jm)
                            if (jm < nct)
                                __builtin_nontemporal_store(O[ht][jm][v] * f, dst + 16 * jm);
                    }
                }
            }
        }
    }

    // ---- partial m and z (z summed over the two row halves)
    __syncthreads();
    if (w < 2 && g == 0) {
        const int h = 16 * hh + n, qh = qh0 + h;
        if (qh < a.n_qh) {
            a.ws_m[pbase + qh] = hh ? mrun1 : mrun0;
            a.ws_z[pbase + qh] = s_z[h] + s_z[HG + h];
        }
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the n_chunks partials of every query-head.
// NW waves per workgroup; lane = CPL adjacent context columns (one 8- or
// 16-byte load per partial; lc is a multiple of 16).  The waves split into
// slabs of W = min(NW, n_chunks rounded up to a power of two) waves: a slab
// covers 64 CPL columns and its waves fold partials p = c, c + W, ... (c =
// the wave's rank in the slab) with an online maximum, NB partials per batch
// whose loads are all issued before any is used; each slab's waves then
// combine through LDS.  Grid (n_qh, ceil(lc / (64 CPL NW / W))).  A few
// partials (the causal batch's 2 chunks) thus fill the waves with columns
// instead of leaving them idle.  CPL = 4 where that grid still has a
// workgroup for each of the 256 CUs, else 2: against 2 throughout, the
// DeepSeek-V3 shape (128 query-heads) 17.53 against 17.70 us per
// layer-token and the causal batch 5.71 against 5.73, while the gathered
// decode (64 query-heads, 128 workgroups with 4) and the long-context shape
// were no faster with 4.
//   M = max_p m_p;  w_p = 2^(m_p - M);  out = sum_p w_p cl_p / sum_p w_p z_p;
//   lse = (M + log2 sum_p w_p z_p) * ln 2.
// (NW, NB) = (8, 16) for more than 32 partials per query-head, (4, 8) for 5
// to 32, (4, 1) for at most 4, so that up to 128 partials each wave folds its
// own in one batch.  Measured in pairs, alternating on one box: (4, 16)
// against (8, 16): gathered decode (32 partials) -0.26 us per call,
// DeepSeek-V3 shape (32) -0.69 us, causal batch (2) -1.0%, long context
// (128) +1.1 us (and (16, 16) slower at every shape); (4, 8) against
// (4, 16): -0.26 us, -0.32 us, -2.4%; (4, 4) against (4, 8): +0.56 us,
// +0.5 us; (4, 1) against (4, 8) on the causal batch: -0.9%.  Against one
// column per lane and four waves (two batches of 16 per wave): 1.3 us less
// per decode call at the long-context shape.
__host__ __device__ __forceinline__ int merge_waves(int n_chunks)
{
    return n_chunks > 32 ? 8 : 4;
}

__host__ __device__ __forceinline__ int merge_slab_waves(int n_chunks, int nw)
{
    int w = 1;
    while (w < n_chunks && w < nw)
        w <<= 1;
    return w;
}

template <int NW, int NB, int CPL>
__global__ __launch_bounds__(64 * NW) void k_merge(const float* __restrict__ ws_m,
                                                   const float* __restrict__ ws_z,
                                                   const float* __restrict__ ws_cl,
                                                   int32_t n_chunks, int32_t n_qh, int32_t lc,
                                                   float* __restrict__ out,
                                                   float* __restrict__ lse)
{
    typedef float fv __attribute__((ext_vector_type(CPL)));
    __shared__ fv s_a[NW][64];
    __shared__ float s_zw[NW];
    __shared__ float s_mw[NW];
    const int qh = blockIdx.x;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int W = merge_slab_waves(n_chunks, NW);
    const int slab = wv / W, wc = wv - slab * W;
    const int col = (blockIdx.y * (NW / W) + slab) * (64 * CPL) + CPL * lane;
    const bool cv = col < lc;  // lc a multiple of 16: all CPL columns or none
    float mw = -INFINITY, zw = 0.0f;
    fv aw = fv(0.0f);
    for (int base = wc; base < n_chunks; base += W * NB) {
        float mp[NB], zp[NB];
        fv cp[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int pp = base + W * k;
            const bool ok = pp < n_chunks;
            const size_t i = (size_t)(ok ? pp : 0) * n_qh + qh;
            mp[k] = ok ? ws_m[i] : -INFINITY;
            zp[k] = ok ? ws_z[i] : 0.0f;
            cp[k] = (ok && cv) ? *reinterpret_cast<const fv*>(ws_cl + i * lc + col) : fv(0.0f);
        }
        float bm = -INFINITY;
#pragma unroll
        for (int k = 0; k < NB; ++k)
            bm = fmaxf(bm, mp[k]);
        if (bm == -INFINITY)
            continue;
        if (bm > mw) {
            const float f = (mw == -INFINITY) ? 0.0f : exp2f(mw - bm);
            zw *= f;
            aw *= f;
            mw = bm;
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const float wgt = (mp[k] == -INFINITY) ? 0.0f : exp2f(mp[k] - mw);
            zw += wgt * zp[k];
            aw += wgt * cp[k];
        }
    }
    s_a[wv][lane] = aw;
    if (lane == 0) {
        s_zw[wv] = zw;
        s_mw[wv] = mw;
    }
    __syncthreads();
    if (wc == 0) {
        const int w0 = slab * W;
        float M = s_mw[w0];
        for (int k = 1; k < W; ++k)
            M = fmaxf(M, s_mw[w0 + k]);
        fv A = fv(0.0f);
        float Z = 0.0f;
        if (M != -INFINITY) {
            for (int k = 0; k < W; ++k) {
                const float wk = (s_mw[w0 + k] == -INFINITY) ? 0.0f : exp2f(s_mw[w0 + k] - M);
                A += wk * s_a[w0 + k][lane];
                Z += wk * s_zw[w0 + k];
            }
        }
        if (cv) {
            // a streaming store: the kernel's end then has no dirty L2 lines
            // to write back (0.1 us less per gathered decode call)
            const fv o = (M == -INFINITY) ? fv(0.0f) : A / Z;
            __builtin_nontemporal_store(o, reinterpret_cast<fv*>(out + (size_t)qh * lc + col));
        }
        if (lse != nullptr && blockIdx.y == 0 && slab == 0 && lane == 0)
            lse[qh] = (M == -INFINITY) ? -INFINITY : (M + log2f(Z)) * 0.69314718055994531f;
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

hipError_t launch_quantize_mx(const float* x, int64_t n_rows, int32_t lc, int32_t rc,
                              uint8_t* rows, float* scales, hipStream_t stream)
{
    const int64_t blocks = (n_rows + 3) / 4;
    hipLaunchKernelGGL(k_quantize_rows_mx, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       n_rows, lc, rc, rows, scales);
    return hipGetLastError();
}

// Read-bandwidth reference, a measurement aid outside the attention path:
// every 16-byte word of the buffer is loaded once (coalesced, grid-stride,
// eight loads in flight per thread; of the shapes measured, 8 loads x 8192
// workgroups read fastest) and XOR-folded.  Wave v of workgroup b stores its
// fold to out[4 b + v] (plain stores, one word per wave, so no two waves meet
// on an address) and every wave stores, so the XOR of all kStreamWords words
// is the XOR of the buffer's 32-bit words (the grid is kStreamWords / 4
// workgroups of 4 waves).
constexpr int kStreamBlocks = kStreamWords / 4;

__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t x = 0;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        uint4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = p[i + k * stride];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x ^= (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0)
        out[4 * blockIdx.x + (threadIdx.x >> 6)] = x;
}

hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* out, hipStream_t stream)
{
    hipLaunchKernelGGL(k_stream_read, dim3(kStreamBlocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(p), bytes / 16, out);
    return hipGetLastError();
}

hipError_t launch_test_encode_pk(const float* x, int64_t n, uint8_t* codes, hipStream_t stream)
{
    const int64_t n4 = n / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(k_test_encode_pk, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(x), n4, reinterpret_cast<uint32_t*>(codes));
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
    if constexpr (NKB == 9) {
        if (a.layout == kMixed) {
            if (a.mode == kSelect)
                hipLaunchKernelGGL((k_split_partial<9, true, true>),
                                   dim3((unsigned)(a.n_chunks * a.n_groups)), dim3(kThreads), 0,
                                   stream, a);
            else
                hipLaunchKernelGGL((k_split_partial<9, false, true>),
                                   dim3((unsigned)(a.n_chunks * a.n_groups)), dim3(kThreads), 0,
                                   stream, a);
            return;
        }
    }
    if (a.mode == kSelect)
        hipLaunchKernelGGL((k_split_partial<NKB, true>), dim3((unsigned)(a.n_chunks * a.n_groups)),
                           dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_split_partial<NKB, false>),
                           dim3((unsigned)(a.n_chunks * a.n_groups)), dim3(kThreads), 0, stream, a);
}

template <int CPL>
static void launch_merge(const AttnArgs& a, int nw, dim3 grid, hipStream_t stream)
{
    if (nw == 8)
        hipLaunchKernelGGL((k_merge<8, 16, CPL>), grid, dim3(64 * 8), 0, stream, a.ws_m, a.ws_z,
                           a.ws_cl, a.n_chunks, a.n_qh, a.lc, a.out, a.lse);
    else if (a.n_chunks > 4)
        hipLaunchKernelGGL((k_merge<4, 8, CPL>), grid, dim3(64 * 4), 0, stream, a.ws_m, a.ws_z,
                           a.ws_cl, a.n_chunks, a.n_qh, a.lc, a.out, a.lse);
    else
        hipLaunchKernelGGL((k_merge<4, 1, CPL>), grid, dim3(64 * 4), 0, stream, a.ws_m, a.ws_z,
                           a.ws_cl, a.n_chunks, a.n_qh, a.lc, a.out, a.lse);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream, hipEvent_t ev_before,
                            hipEvent_t ev_after)
{
    // The padded LDS row covers the row width d in 64-byte blocks (the
    // context columns each wave reads, 64 * w .. +64 for 64 * w < lc, lie
    // inside it since lc <= d).
    const int nkb = (a.d + 63) / 64;
    if (nkb < 1 || nkb > 10)
        return hipErrorInvalidValue;
    if (ev_before != nullptr) {
        const hipError_t e = hipEventRecord(ev_before, stream);
        if (e != hipSuccess)
            return e;
    }
    if (partial32_applies(a)) {
        launch_partial32(a, stream);
    } else {
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
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (ev_after != nullptr) {
        e = hipEventRecord(ev_after, stream);
        if (e != hipSuccess)
            return e;
    }
    const int nw = merge_waves(a.n_chunks);
    // four columns per lane where the grid still gives every CU a workgroup
    const int slabs = nw / merge_slab_waves(a.n_chunks, nw);
    const int cpl = (long)a.n_qh * ((a.lc + 256 * slabs - 1) / (256 * slabs)) >= 256 ? 4 : 2;
    const int cols = 64 * cpl * slabs;  // columns per workgroup
    const dim3 grid((unsigned)a.n_qh, (unsigned)((a.lc + cols - 1) / cols));
    if (cpl == 4)
        launch_merge<4>(a, nw, grid, stream);
    else
        launch_merge<2>(a, nw, grid, stream);
    return hipGetLastError();
}

}  // namespace mla8
