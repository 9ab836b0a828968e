// Split-T partial kernel on the 32x32x16 fp16 MFMA, for the DeepSeek-V3 row
// shape (Lc = 512, Rc = 64: 576 e4m3 bytes per row): dense rows with the
// optional fused append of fresh rows, and the causal batch when each group of
// 32 query-heads belongs to one query position (its rows end at that
// position, inclusive).  Same result contract as
// k_split_partial: per (row chunk, query-head) the online-softmax partial
// (m in log2 units, z, cl = sum_t p_t scale_t x_t), merged by k_merge.
//
// Method source: colibri PR #300 "KV8 long-context CUDA: fp8 device shadow,
// split-T kernels, DSA-aware gather", second commit ("KV8 long-context
// CUDA"): split-T blocks emitting online-softmax partials (cl[K], m, z) and a
// log-sum-exp merge, and the batch/prefill kernel over (query, head) pairs
// with a causal limit; first commit ("KV8 base"): the latent row is both key
// and value, the row scale is hoisted out of the dot, the producer quantizes
// the fresh row.
//
// gfx950 design.  One workgroup = one row chunk x 32 query-heads, 512 threads,
// one workgroup per CU; waves 0-3 score, waves 4-7 accumulate the context, so
// each SIMD runs one wave of each role.  Measured on MI355X: the kernel is
// bound by each SIMD's VALU issue (an e4m3 -> fp16 widening instruction
// holds it about 6.5 cycles, other VALU instructions 4, a 32x32x16 MFMA a
// few), next to the matrix pipe (32 cycles per 32x32x16 MFMA); the memory
// stream is not the limit (the same kernel with its row loads removed takes
// the same cycles per tile).  Hence:
//   * every row byte is widened once for the scores and once for the
//     context.  A score wave takes 32 rows x half of K (18 K steps of 16)
//     for all 32 heads: columns = heads of one 32x32x16 MFMA, and each
//     widened A operand feeds two MFMAs, the fp16 hi and lo query terms,
//     into one accumulator.  The two K halves of a row half are added
//     through LDS one phase later, each wave taking half of the values;
//   * the context O[32 heads][32 columns] += W . X runs on the same MFMA with
//     the transposed row bytes (ds_read_b64_tr_b8) widened to fp16;
//   * a 64-row tile is stored as 16-row x 64-byte blocks of 16-byte slots
//     (slot r + 16 c of a block holds row r, bytes 16 c ..): one direct load
//     (global_load_lds_dwordx4) fills a block, a score read is four linear
//     256-byte runs and a transposed context read eight consecutive slots, so
//     neither reader meets a bank conflict;
//   * the scores' and the context's readers of a tile both read it in the
//     phase it is scored (the context keeps the bytes in registers for two
//     phases), so a three-stage ring keeps two tiles in flight;
//   * the lazy-max check is a per-wave flag (any weight or probability above
//     2^8, or not finite) instead of cross-lane check sums.
#include "mla8_device.h"
#include "mla8_internal.h"
#include "mla8_pipe.h"

namespace mla8 {

namespace p32 {
constexpr int TR = kTileRows;            // 64 rows per tile
constexpr int HG = kHeadsPerGroup;       // 32 query-heads per workgroup
constexpr int LC = 512, RC = 64, D = LC + RC;
constexpr int NCB = D / 64;              // 9 column blocks of 64 bytes
constexpr int STAGE = TR * D;            // 36,864 bytes per tile
constexpr int NST = 3;                   // ring stages
constexpr int DIST = 2;                  // tiles issued ahead
constexpr int NKS = D / 16;              // 36 score K steps of 16
constexpr int KH = NKS / 2;              // 18 K steps per score wave
constexpr int WSTR = TR + 8;             // weight row stride (halves)
constexpr int NINS = STAGE / 1024;       // 36 row DMA instructions per tile
constexpr int KW = NINS / 4;             // 9 per context wave
// LDS map (bytes)
constexpr int NSC = 4;                   // row-scale slots: tile t in slot t % 4
constexpr int SC = NST * STAGE;          // f32 [NSC][TR] row scales
constexpr int W = SC + NSC * TR * 4;     // f16 [2][HG][WSTR] weights
constexpr int XC = W + 2 * HG * WSTR * 2;  // f32x4 [2][2 rh][2 kh][2][64] partial scores
constexpr int FL = XC + 2 * 2 * 2 * 2 * 64 * 16;  // u32 [2][4] overflow flags
constexpr int CR = FL + 2 * 4 * 4;       // float2 [HG][4] exact tile maxima (head, row quarter)
constexpr int Z = CR + HG * 4 * 8;       // f32 [4][HG] z per score wave
constexpr int HK = Z + 4 * HG * 4;       // i32 [2][HG] query scaling exponents k (and j, LO8)
constexpr int UV = HK + 2 * HG * 4;      // f32x4 [4 waves][4][64]: u, scale of the weighed tile
constexpr int AL = UV + 4 * 4 * 64 * 16; // f32 [4 context waves][HG] accumulator factors
constexpr int VM = AL + 4 * HG * 4;      // gather: u64 [NSC] row-validity masks (bit = tile row)
constexpr int END = VM + NSC * 8;
// query operand staging (one term at a time): stage 2, first filled in phase 0
constexpr int QT = 2 * STAGE;
static_assert(NKS * 64 * 16 <= STAGE, "one query term fits a stage");
static_assert(END <= 160 * 1024, "LDS budget");
static_assert(NINS % 4 == 0, "row DMAs split evenly over the context waves");
}  // namespace p32

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v8i32 __attribute__((ext_vector_type(8)));

// sched_barrier mask: VALU, SALU, transcendental, VMEM and LDS writes may be
// scheduled across; LDS reads and MFMAs stay on their side
constexpr int kNoDsReadCross = 0x2 | 0x4 | 0x10 | 0x20 | 0x40 | 0x200 | 0x400;

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// bf16 x bf16 (the RoPE part of a mixed row against the RoPE query terms)
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// e4m3 x e4m3, K = 64, A unscaled, B (the query's lo term) scaled by the
// E8M0 exponent sb (value 2^(sb - 127)) of each lane's column
__device__ __forceinline__ f32x16 mfma32_f8(v8i32 a, v8i32 b, f32x16 c, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

template <bool LO8, bool GATHER, bool MXL>
__global__ __launch_bounds__(kThreads, 1) void k_partial32(AttnArgs a)
{
    using namespace p32;
    // Mixed rows (MXL): 448 noPE e4m3 bytes (column blocks 0-6) then 64 RoPE
    // bf16 values (blocks 7-8), the same 576 bytes; the output and the
    // context cover the 448 noPE columns.  Only with LO8.
    static_assert(!MXL || LO8, "mixed rows take the e4m3 lo term");
    constexpr int LCO = MXL ? 448 : LC;     // q_lat width, output width
    constexpr int NCN = MXL ? 7 : NCB;      // e4m3 column blocks
    constexpr int NQF = MXL ? 8 : 9;        // query float4 per work item
    __shared__ __attribute__((aligned(1024))) uint8_t lds[END];
    float* const s_sc = reinterpret_cast<float*>(lds + SC);
    _Float16* const s_w = reinterpret_cast<_Float16*>(lds + W);
    uint32_t* const s_fl = reinterpret_cast<uint32_t*>(lds + FL);
    float2* const s_cr2 = reinterpret_cast<float2*>(lds + CR);
    float* const s_z = reinterpret_cast<float*>(lds + Z);
    int* const s_k = reinterpret_cast<int*>(lds + HK);
    const uint32_t lds_u32 = (uint32_t)(uintptr_t)(MLA8_LDS uint8_t*)lds;

    const int tid = threadIdx.x;
    // w through readfirstlane: the compiler then knows the role branches are
    // uniform and keeps the two roles' register live ranges apart
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 15;

    // Workgroup -> (chunk, head group), the two head groups of a chunk on one
    // XCD back to back (dispatch is round-robin over the 8 XCDs).
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
    // causal batch: the group's 32 query-heads belong to one query position
    // (n_heads is a multiple of 32), whose rows end at pos0 + s + 1
    int c1 = min(a.n_list, c0 + a.chunk_rows);
    if (a.mode == kCausal)
        c1 = min(c1, a.pos0 + qh0 / a.n_heads + 1);
    const int ntiles = c1 > c0 ? (c1 - c0 + TR - 1) / TR : 0;

    // ---- row stream: the context waves (4-7) issue every direct load, KW row
    // DMAs per tile each (instruction k = wi + 4 i fills block k = 9 rb + cb:
    // lane r + 16 c loads row 16 rb + r, bytes 64 cb + 16 c ..), and wave 4
    // one more for the 64 row scales, so a fixed per-wave vmcnt marks a tile
    // complete.  A ragged last tile (nv < 64 rows left) loads the list's last
    // 64 rows instead (the list holds at least 64): its first 64 - nv rows,
    // already attended as part of the previous tile or chunk, get no weight.
    const bool ctx_wave = w >= 4;
    const int wi = ctx_wave ? w - 4 : 0;
    const bool dma_lead = w == 4;
    // lane r + 16 c of instruction i: row r of the block, bytes 16 c ..; the
    // block's own offset in the tile (wave-uniform) goes to the scalar base
    const uint32_t lane_off = (uint32_t)((lane & 15) * D + 16 * (lane >> 4));
    auto blk_k = [&](int i) __attribute__((always_inline)) { return wi + 4 * i; };
    auto blk_ofs = [&](int k) __attribute__((always_inline)) {  // 16 rb rows + 64 cb bytes
        return (uint32_t)(64 * (k + 135 * (k / NCB)));
    };
    int32_t g_row[GATHER ? 4 : 1];  // gather: rows of the tile being issued, per row block
    int32_t g_sc = 0;               // gather, wave 4: list entry p0 + lane (its row scale)
    // gather: list entries p0 .. p0 + 63 of tile t are absolute row indices;
    // one outside [0, t_rows) loads row 0 and gets no weight
    auto load_rows = [&](int t, int32_t (&g)[GATHER ? 4 : 1], int32_t& gs)
                         __attribute__((always_inline)) {
        const int p0 = min(c0 + t * TR, c1 - TR);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            g[rb] = a.sel[p0 + 16 * rb + (lane & 15)];
        gs = a.sel[p0 + lane];  // used by wave 4 only; unconditional, no branch
    };
    // have_rows: the tile's list entries are already in g_row and g_sc
    auto issue = [&](int t, int st, auto I0_, auto I1_, bool have_rows = false)
                     __attribute__((always_inline)) {
        constexpr int I0 = decltype(I0_)::value, I1 = decltype(I1_)::value;
        const uint32_t xst = lds_u32 + (uint32_t)(st * STAGE);
        // tile t's scales are read until phase t + 1 (its weights), past the
        // loads of tile t + 3 into its ring stage: a ring of their own
        const uint32_t sct = lds_u32 + (uint32_t)(SC + (t & (NSC - 1)) * TR * 4);
        const int p0 = min(c0 + t * TR, c1 - TR);
        if constexpr (!GATHER) {
            const uint8_t* tb = a.codes + (size_t)p0 * D;
#pragma unroll
            for (int i = I0; i < I1; ++i) {
                const int k = blk_k(i);
                dma_b128_s(tb + blk_ofs(k), lane_off, xst + (uint32_t)(1024 * k));
            }
            if (I1 == KW && dma_lead)
                dma_b32_s(a.scales + p0, (uint32_t)(4 * lane), sct);
        } else {
            // the list entries are loaded with the first part
            if constexpr (I0 == 0) {
                if (!have_rows)
                    load_rows(t, g_row, g_sc);
            }
#pragma unroll
            for (int i = I0; i < I1; ++i) {
                const int k = blk_k(i);
                const int rb = k / NCB, cb = k - NCB * rb;
                const int32_t r = g_row[rb];
                const int32_t row = (r >= 0 && r < a.t_rows) ? r : 0;
                dma_b128(a.codes + (size_t)row * D + 64 * cb + 16 * (lane >> 4),
                         xst + (uint32_t)(1024 * k));
            }
            if (I1 == KW && dma_lead) {
                const int32_t r = g_sc;
                const bool ok = r >= 0 && r < a.t_rows;
                dma_b32(a.scales + (ok ? r : 0), sct);
                const uint64_t valid = __ballot(ok);
                if (lane == 0)
                    reinterpret_cast<uint64_t*>(lds + VM)[t & (NSC - 1)] = valid;
            }
        }
    };
    using IC0 = std::integral_constant<int, 0>;
    using ICA = std::integral_constant<int, 3>;
    using ICB = std::integral_constant<int, 6>;
    using ICK = std::integral_constant<int, KW>;
    static_assert(KW == 9, "three issue points of three loads");
    auto wait_tile = [&](bool next_in_flight) __attribute__((always_inline)) {
        if (next_in_flight) {
            if (dma_lead)
                wait_vmcnt<KW + 1>();
            else
                wait_vmcnt<KW>();
        } else {
            wait_vmcnt<0>();
        }
    };

    // ---- fused append: fresh rows [f0, f1) of this chunk are quantized into
    // the shadow by this workgroup before any wave streams them.  A wave's
    // vector memory operations complete in issue order: fresh rows that start
    // at tile DIST + 1 or later are quantized by the context waves after the
    // prologue (their per-tile waits then cover the stores before the phase
    // barrier that precedes those tiles' loads); otherwise every wave
    // quantizes, and waits, before the first load.
    // A ragged last tile also loads rows before the chunk, which may be fresh
    // rows of the previous chunk: those are quantized here too (the same
    // bytes as the other workgroup writes), so that no loaded byte is stale.
    int f0 = 0, f1 = 0;
    if (a.n_new > 0 && ntiles > 0) {
        f0 = max(min(c0, c1 - TR), a.new0);
        f1 = min(c1, a.new0 + a.n_new);
    }
    const bool fresh_late = f0 < f1 && f0 - c0 >= (DIST + 1) * TR;
    auto quantize_fresh = [&](int first, int stride) __attribute__((always_inline)) {
        for (int r = f0 + first; r < f1; r += stride)
            if constexpr (MXL)
                quantize_row_mx_wave(a.x_new + (size_t)(r - a.new0) * (LCO + RC), LCO, RC,
                                     a.new_codes + (size_t)r * D, a.new_scales + r, lane);
            else
                quantize_row_wave(a.x_new + (size_t)(r - a.new0) * D, D, a.new_codes + (size_t)r * D,
                                  a.new_scales + r, lane);
    };
    if (f0 < f1 && !fresh_late) {
        quantize_fresh(w, 8);
        wait_vmcnt<0>();
        __syncthreads();
    }

    // ---- prologue: query operands, built by the score waves while the
    // context waves issue the first DIST tiles' loads (a wave with those in
    // flight could not wait for query loads of its own without waiting for
    // them too).  The score waves' query loads go out first: a barrier holds
    // the row loads back until they are issued, so that they do not queue
    // behind the 73 KB of row loads in the CU's memory path.  Work item t
    // (two per score-wave thread: t = tid and tid + 256) loads the nine
    // float4 of head t / 16 at elements 4 (t % 16 + 16 s), s < 9; the head's
    // e = q * sm_scale * log2(e) is scaled by 2^k
    // (largest |e| in [2^14, 2^15)) and split into fp16 hi + lo (the
    // subtraction is exact in f32).  hi is staged in the score waves' B
    // operand layout (K step ks = 4 cb + 2 s' + t' covers elements 64 cb +
    // 32 s' + 16 h + 8 t' + (0..7) for lane half h; lane = head + 32 h).
    // LO8: the lo term is quantized to e4m3 with a per-head power-of-2 scale
    // 2^j (largest |lo| 2^j in [128, 256)) for the e4m3 MFMA, which takes the
    // row bytes as they are, and staged at the same time in the weight and
    // exchange buffers (unused until phase 0) as [cb][lane] 32 bytes (byte b
    // < 16: element 64 cb + 16 h + b, b >= 16: 64 cb + 32 + 16 h + b - 16,
    // the row bytes' order in the A operand); score wave kh then holds
    // column blocks 5 kh .. (5 or 4 of them) and the hi term's K steps 20 kh
    // ...  Without LO8 the fp16 lo term is staged where hi was, once hi has
    // been read, and score wave kh holds K steps 18 kh .. + 18 of both.
    const int kh = w & 1;
    constexpr int NQH = LO8 ? 20 : KH;  // hi K steps held by a score wave (at most)
    f16x8 qhi[NQH], qlo[LO8 ? 1 : KH];
    v8i32 ql8[LO8 ? 5 : 1];
    bf16x8 qr[MXL ? 8 : 1];  // mixed rows, kh = 1: RoPE terms [K step m][hi, lo]
    constexpr int QL8 = W;  // LO8: staging of the e4m3 lo term
    static_assert(QL8 + NCB * 64 * 32 <= FL, "the lo term fits the weight and exchange buffers");
    f16x4 lo4[LO8 ? 1 : 2][9];  // without LO8: the lo term until its staging round
    float4 vq[2][NQF];
    // A head beyond n_qh (a partial last group) takes the last head's query:
    // its results are never stored, and the loads stay unconditional.
    auto load_q = [&](auto NIT_) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < decltype(NIT_)::value; ++it) {
            const int t = tid + 256 * it, h = t >> 4, i = t & 15;
            const size_t qh = (size_t)min(qh0 + h, a.n_qh - 1);
            const float* const ql = a.q_lat + qh * LCO + 4 * i;
            const float* const qr = a.q_rope + qh * RC + 4 * i;
#pragma unroll
            for (int s = 0; s < NQF; ++s) {
                // elements 4 (i + 16 s): q_lat, then q_rope (s = 8; mixed
                // rows: s = 7, RoPE elements 4 i ..)
                const float* p = (s < NQF - 1) ? ql + 64 * s : qr;
                vq[it][s] = *reinterpret_cast<const float4*>(p);
            }
        }
    };
    // The split, per element: r = f32(e 2^k); hi = fp16(r); lo = fp16(r -
    // hi).  The largest |lo| of a head is the fp16 rounding of the largest
    // |r - hi| (the rounding is monotonic), so it is taken before lo is
    // rounded; lo 2^j is formed from the fp16 lo, as the encoder's input.
    auto build_q = [&](auto NIT_) __attribute__((always_inline)) {
        constexpr int NN = NQF - (MXL ? 1 : 0);  // float4 of the 2^k-scaled part
#pragma unroll
        for (int it = 0; it < decltype(NIT_)::value; ++it) {
            const int t = tid + 256 * it, h = t >> 4, i = t & 15;
            float amax = 0.0f;
#pragma unroll
            for (int s = 0; s < NN; ++s) {
                amax = max3_abs(amax, vq[it][s].x, vq[it][s].y);
                amax = max3_abs(amax, vq[it][s].z, vq[it][s].w);
            }
            amax = row16_max(amax);
            const float es = a.sm_log2;
            const int k = query_exp(amax * es);
            if (i == 0)
                s_k[h] = k;
            const float mult = ldexpf(es, k);
            uint2 lot[9];  // fp16 lo, two per dword
            float lmax = 0.0f;
#pragma unroll
            for (int s = 0; s < NN; ++s) {
                // r = f32(q 2^k es), rounded once and opaque to the compiler:
                // both terms are split from this one f32 value (otherwise hi
                // may be recomputed as the fp16 rounding of the exact product,
                // which differs where r sits on an fp16 rounding tie)
                float r[4] = {vq[it][s].x * mult, vq[it][s].y * mult, vq[it][s].z * mult,
                              vq[it][s].w * mult};
                asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
                const uint2 hi = make_uint2(pk_f16(r[0], r[1]), pk_f16(r[2], r[3]));
                // r - hi, exact in f32
                const float d0 = sub_f16<0>(r[0], hi.x), d1 = sub_f16<1>(r[1], hi.x);
                const float d2 = sub_f16<0>(r[2], hi.y), d3 = sub_f16<1>(r[3], hi.y);
                lmax = max3_abs(lmax, d0, d1);
                lmax = max3_abs(lmax, d2, d3);
                lot[s] = make_uint2(pk_f16(d0, d1), pk_f16(d2, d3));
                const int e = 4 * (i + 16 * s);
                const int cb = e >> 6, s2 = (e >> 5) & 1, hf = (e >> 4) & 1, t2 = (e >> 3) & 1;
                const int ks = 4 * cb + 2 * s2 + t2;
                *reinterpret_cast<uint2*>(lds + QT + ((size_t)ks * 64 + h + 32 * hf) * 16 +
                                          2 * (e & 7)) = hi;
            }
            if constexpr (MXL) {
                // RoPE elements 4 i .. + 3: e = q_rope es split into bf16 hi
                // + lo (no 2^k, no row scale), staged after the 28 noPE hi K
                // steps as [K step m][term][lane] 16 bytes, m = i / 4, lane =
                // head + 32 ((i / 2) % 2), bf16 positions 4 (i % 2) ..
                const float4 q4 = vq[it][NQF - 1];
                const float e[4] = {q4.x * es, q4.y * es, q4.z * es, q4.w * es};
                uint32_t hb[4], lb[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    hb[c] = bf16_rne_bits(e[c]);
                    lb[c] = bf16_rne_bits(e[c] - __uint_as_float(hb[c] << 16));
                }
                const int m = i >> 2, hr = (i >> 1) & 1;
                uint8_t* rq = lds + QT + 28 * 1024 + ((2 * m) * 64 + h + 32 * hr) * 16 + 8 * (i & 1);
                *reinterpret_cast<uint2*>(rq) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                *reinterpret_cast<uint2*>(rq + 64 * 16) =
                    make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
            }
            if constexpr (LO8) {
                const float lm = (float)(_Float16)row16_max(lmax);  // largest |lo|
                int ex = 0;
                if (lm > 0.0f)
                    (void)frexpf(lm, &ex);
                const int j = (lm > 0.0f) ? max(-100, min(100, 8 - ex)) : 0;
                if (i == 0)
                    s_k[HG + h] = j;
                const float tj = ldexpf(1.0f, j);
#pragma unroll
                for (int s = 0; s < NN; ++s) {
                    const int e = 4 * (i + 16 * s);
                    const int cb = e >> 6, off = e & 63, hf = (off >> 4) & 1;
                    const int b = 16 * (off >> 5) + (off & 15);
                    // |lo 2^j| < 256 and exact: the packed hardware encoder
                    // rounds it as the library's encoder does
                    *reinterpret_cast<uint32_t*>(lds + QL8 + ((size_t)(cb * 64 + h + 32 * hf)) * 32 +
                                                 b) =
                        enc_e4m3_pk4(mul_f16<0>(lot[s].x, tj), mul_f16<1>(lot[s].x, tj),
                                     mul_f16<0>(lot[s].y, tj), mul_f16<1>(lot[s].y, tj));
                }
            } else {
#pragma unroll
                for (int s = 0; s < 9; ++s)
                    lo4[it][s] = __builtin_bit_cast(f16x4, lot[s]);
            }
        }
    };
    // Gather: the context waves load the first two tiles' list entries
    // meanwhile and have them before any row load is in flight (a wait for
    // them behind row loads would wait for those too); a tile past the
    // chunk's last has its entries in the list too (p0 is clamped), so those
    // loads need no branch.  Each role runs its own copy up to the build
    // (with its own barrier), so that no path joins another while query loads
    // are in flight: at a join the compiler would wait for them, and thereby
    // for the row loads, wherever it reuses their registers.  (Every wave
    // building one item on short chunks, the context waves theirs before
    // their row loads, measured the same: 14.53 against 14.53 us per
    // layer-token on the gather, 18.93 against 18.84 on the DeepSeek-V3 shape.)
    using IT2 = std::integral_constant<int, 2>;
    if (!ctx_wave) {
        load_q(IT2{});
        // the score waves' query loads are ahead of the row loads; no build
        // instruction moves before the barrier (it would wait for the query
        // there)
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        build_q(IT2{});
        // distinct ends keep the compiler from merging the roles' tails
        asm volatile("; score-wave query build");
    } else {
        int32_t gp[2][GATHER ? 4 : 1], gsp[2];
        if constexpr (GATHER) {
            load_rows(0, gp[0], gsp[0]);
            load_rows(1, gp[1], gsp[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (GATHER) {
            // every list load has arrived before a row load goes out
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    asm volatile("" : "+v"(gp[u][rb]));
            asm volatile("" : "+v"(gsp[0]), "+v"(gsp[1]));
        }
        if (ntiles > 0) {
            if constexpr (GATHER) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    g_row[rb] = gp[0][rb];
                g_sc = gsp[0];
            }
            issue(0, 0, IC0{}, ICK{}, GATHER);
        }
        if (ntiles > 1) {
            if constexpr (GATHER) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    g_row[rb] = gp[1][rb];
                g_sc = gsp[1];
            }
            issue(1, 1, IC0{}, ICK{}, GATHER);
        }
        asm volatile("; context-wave row issue");
    }
    lds_barrier();
    if (!ctx_wave) {
        // LO8: wave kh holds column blocks CB0 kh .. (dense rows 5 and 4,
        // mixed rows 4 and 3 noPE blocks, then the RoPE part on kh = 1)
        constexpr int CB0 = MXL ? 4 : 5;
        const int ks0 = LO8 ? 4 * CB0 * kh : KH * kh;
        const int nks = LO8 ? 4 * (CB0 - kh) : KH;
#pragma unroll
        for (int m = 0; m < NQH; ++m)
            if (m < nks)
                qhi[m] = *reinterpret_cast<const f16x8*>(lds + QT + ((ks0 + m) * 64 + lane) * 16);
        if constexpr (LO8) {
#pragma unroll
            for (int c = 0; c < 5; ++c)
                if (c < CB0 - kh)
                    ql8[c] = *reinterpret_cast<const v8i32*>(lds + QL8 + ((CB0 * kh + c) * 64 + lane) * 32);
        }
        if constexpr (MXL) {
            if (kh == 1) {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    qr[m] = *reinterpret_cast<const bf16x8*>(lds + QT + 28 * 1024 + (m * 64 + lane) * 16);
            }
        }
    }
    lds_barrier();  // LO8: staging areas free for the ring and the weights
    if constexpr (!LO8) {
        if (!ctx_wave) {
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int t = tid + 256 * it, h = t >> 4, i = t & 15;
#pragma unroll
                for (int s = 0; s < 9; ++s) {
                    const int e = 4 * (i + 16 * s);
                    const int cb = e >> 6, s2 = (e >> 5) & 1, hf = (e >> 4) & 1, t2 = (e >> 3) & 1;
                    const int ks = 4 * cb + 2 * s2 + t2;
                    *reinterpret_cast<f16x4*>(lds + QT + ((size_t)ks * 64 + h + 32 * hf) * 16 +
                                              2 * (e & 7)) = lo4[it][s];
                }
            }
        }
        lds_barrier();
        if (!ctx_wave) {
#pragma unroll
            for (int m = 0; m < KH; ++m)
                qlo[m] = *reinterpret_cast<const f16x8*>(lds + QT + ((KH * kh + m) * 64 + lane) * 16);
        }
        lds_barrier();  // staging area free for the ring
    }

    // Softmax state, identical in every wave, for heads n and 16 + n of the
    // group (lane n = lane % 16): m = lazy max of u (z side), d = lazy max of
    // (u - m) + log2 scale (context side, relative to m).  Tile p's weights
    // are written with the state as it stands, in the linear domain,
    //     p_t = 2^(u_t - m),  w_t = p_t * (scale_t * 2^-d),
    // and every score wave publishes a flag when any of its p or w leaves
    // [0, 2^kTau] (a new maximum by more than kTau, or a value that left f32's
    // range; NaN is caught through the sums).  One phase later every wave
    // reads the four flags: when one is set, or a head of the group has not
    // met a valid row yet, every wave takes the exact path together: the
    // score waves publish exact maxima per (head, row quarter), the state
    // moves by the lazy rule, the context waves rescale their accumulators and
    // the score waves rewrite the tile's weights in the log domain.  Separate
    // scalars, never an array (a lane-dependent pick would go to scratch).
    float mrun0 = -INFINITY, mrun1 = -INFINITY, drun0 = -INFINITY, drun1 = -INFINITY;
    float fown = 1.0f;
    bool uninit = true;
    constexpr float kCheck = 256.0f;
    static_assert(kTau == 8.0f, "check threshold 2^kTau");

    auto vote = [&](uint4 fl) __attribute__((always_inline)) -> bool {
        return uninit || ((fl.x | fl.y | fl.z | fl.w) != 0u);
    };
    auto state_move = [&](float (&alz)[2], float (&alo)[2], int own_hh)
                          __attribute__((always_inline)) {
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
        const float dd = own_hh ? drun1 : drun0;
        fown = (dd == -INFINITY) ? 1.0f : fast_exp2(-dd);
        uninit = __any(mrun0 == -INFINITY || mrun1 == -INFINITY);
    };
    const size_t pbase = (size_t)chunk * a.n_qh;

    if (!ctx_wave) {
        // ======== score waves: rows 32 rh .. +32 of each tile, K steps 18 kh
        // .. +18, all 32 heads as the MFMA's columns.
        auto score_role = [&](auto KHc_) __attribute__((always_inline)) {
            constexpr int KHC = decltype(KHc_)::value;  // = kh
            const int rh = w >> 1;
            const int hf = lane >> 5;              // lane half: K elements 8 hf ..
            const int hd = lane & 31;              // the lane's head (score column)
            const int hsel = hd >> 4;              // state of head n (0) or 16 + n (1)
            const float pk = ldexpf(1.0f, -s_k[hd]);  // the accumulators hold 2^k scores
            // u as weighed: 2^k times the score (dense rows), or the score
            // itself (mixed rows: the RoPE part carries neither 2^k nor the
            // row scale, so each wave's part is scaled before the exchange)
            const float upk = MXL ? 1.0f : pk;
            const int sb_lo = 127 - s_k[HG + hd];         // LO8: E8M0 scale 2^-j of the lo term
            // After the exchange the lane holds head hd, rows rb0 + (0..3) and
            // rb0 + 8 + (0..3) of the wave's 32 (values 8 kh .. +8 of the
            // 32x32 result; row quarter 2 rh + kh).
            const int rb0 = 16 * KHC + 4 * hf;
            float zacc = 0.0f, zsave = 0.0f;
            float accp[8];        // this wave's half of tile p-1's partial scores
            // the lane's u (2^k-scaled score x row scale) and row scales of the
            // last weighed tile, kept for the exact path
            float4* const s_uv = reinterpret_cast<float4*>(lds + UV) + w * 4 * 64 + lane;
            _Float16* const s_w_own = s_w + hd * WSTR + 32 * rh + rb0;
            // A operand: row l % 32 of the half, 16 bytes of half column block
            // hb (slot hf + 2 (hb & 1) of column block hb / 2) at + 512 hb.
            const int rowq = 32 * rh + (lane & 31);
            const int a_off = (rowq >> 4) * (NCB * 1024) + ((rowq & 15) + 16 * hf) * 16 +
                              (LO8 ? 1024 * (MXL ? 4 : 5) * KHC : 512 * (KH / 2) * KHC);
            // exchange: value 8 kh' + 4 j + c of wave (rh, kh) goes to wave
            // (rh, kh') as float4 j at [parity][rh][kh'][j][lane]
            auto xc_ptr = [&](int par, int dst) __attribute__((always_inline)) -> float4* {
                return reinterpret_cast<float4*>(lds + XC) + ((par * 2 + rh) * 2 + dst) * 2 * 64 + lane;
            };
            f32x16 acc;

            // Weights of tile t (= p - 1: own half in accp, the partner's in
            // the exchange buffer; row scales in slot t % NSC) for this lane's
            // rows, linear form, into buffer buf; true when all of them and
            // their p are in [0, 2^kTau].  Only the last tile can be ragged,
            // and it is weighed after the last stream (RAGGED); inside a
            // stream the weighing has no branch, so that the scheduler can
            // spread it among the MFMAs.
            auto weigh = [&](int t, int buf, auto RAGGED_) __attribute__((always_inline)) -> bool {
                const float* scp = s_sc + (t & (NSC - 1)) * TR + 32 * rh + rb0;
                const float4 s0 = *reinterpret_cast<const float4*>(scp);
                const float4 s1 = *reinterpret_cast<const float4*>(scp + 8);
                const float4* xq = xc_ptr(t & 1, KHC);
                const float4 y0 = xq[0], y1 = xq[64];
                zsave = zacc;
                const float scv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
                float u[8];
#pragma unroll
                for (int v = 0; v < 8; ++v)
                    u[v] = MXL ? accp[v] + yv[v] : (accp[v] + yv[v]) * scv[v];
                if constexpr (GATHER) {
                    // -inf for list entries outside [0, t_rows): bit row of
                    // the tile's validity mask
                    const uint64_t mk = reinterpret_cast<const uint64_t*>(lds + VM)[t & (NSC - 1)];
                    const uint32_t bits = (uint32_t)(mk >> (32 * rh + rb0));
#pragma unroll
                    for (int r = 0; r < 2; ++r)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (((bits >> (8 * r + v)) & 1u) == 0u)
                                u[4 * r + v] = -INFINITY;
                }
                if constexpr (decltype(RAGGED_)::value) {
                    const int lead = c0 + (t + 1) * TR - c1;  // rows before the tile's own
#pragma unroll
                    for (int r = 0; r < 2; ++r)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (32 * rh + rb0 + 8 * r + v < lead)
                                u[4 * r + v] = -INFINITY;
                }
                s_uv[0] = make_float4(u[0], u[1], u[2], u[3]);
                s_uv[64] = make_float4(u[4], u[5], u[6], u[7]);
                s_uv[128] = s0;
                s_uv[192] = s1;
                const float mu = hsel ? mrun1 : mrun0;
                const float nmz = (mu == -INFINITY) ? 0.0f : -mu;
                float ps = 0.0f, ws = 0.0f, mx = 0.0f;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    f16x4 wv;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float pv = fast_exp2(fmaf(u[4 * r + v], upk, nmz));
                        const float wt = pv * (scv[4 * r + v] * fown);
                        ps += pv;
                        ws += wt;
                        mx = fmaxf(mx, fmaxf(pv, wt));
                        wv[v] = (_Float16)wt;
                    }
                    *reinterpret_cast<f16x4*>(s_w_own + buf * HG * WSTR + 8 * r) = wv;
                }
                zacc = zsave + ps;
                // fmaxf drops NaN; the sums keep it (every term is >= 0)
                return (mx <= kCheck) && (ps + ws <= 4096.0f);
            };
            // Same in the log domain (exact for any scale), after a state move,
            // from the unscaled scores u.
            auto weights_log = [&](int buf, const float (&u)[8], const float (&scv)[8])
                                   __attribute__((always_inline)) {
                const float mu = hsel ? mrun1 : mrun0;
                const float dd = hsel ? drun1 : drun0;
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
                    *reinterpret_cast<f16x4*>(s_w_own + buf * HG * WSTR + 8 * r) = wv;
                }
                zacc = zsave + ps;
            };
            // The score MFMAs of tile p (ring stage st) into acc: each half
            // column block widened once, then its two K steps times the hi and
            // lo query terms; with WW, the weights of tile p-1 are computed
            // among them (independent work that fills the MFMA shadow).
            auto stream = [&](int st, int ts, auto WW_, int t, int buf)
                              __attribute__((always_inline)) -> bool {
                constexpr bool WW = decltype(WW_)::value;
                bool ok = true;
                const uint8_t* xs = lds + st * STAGE + a_off;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[v] = 0.0f;
                if constexpr (LO8) {
                    // column block c of the wave: both halves (32 row bytes
                    // per lane) feed the e4m3 MFMA as they are and, widened,
                    // the four hi K steps
                    constexpr int NC = MXL ? (KHC ? 3 : 4) : (KHC ? 4 : 5);
                    // the lo products in an accumulator of their own, added
                    // to the hi sum once at the end
                    f32x16 acc_lo;
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc_lo[v] = 0.0f;
                    uint4 xa[2], xb2[2];
                    xa[0] = *reinterpret_cast<const uint4*>(xs);
                    xb2[0] = *reinterpret_cast<const uint4*>(xs + 512);
                    __builtin_amdgcn_sched_barrier(kNoDsReadCross);
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        if (c + 1 < NC) {
                            xa[(c + 1) & 1] = *reinterpret_cast<const uint4*>(xs + 1024 * (c + 1));
                            xb2[(c + 1) & 1] = *reinterpret_cast<const uint4*>(xs + 1024 * (c + 1) + 512);
                        }
                        __builtin_amdgcn_sched_barrier(kNoDsReadCross);
                        const uint4 x0 = xa[c & 1], x1 = xb2[c & 1];
                        acc = mfma32(cvt8(x0.x, x0.y), qhi[4 * c + 0], acc);
                        acc = mfma32(cvt8(x0.z, x0.w), qhi[4 * c + 1], acc);
                        acc = mfma32(cvt8(x1.x, x1.y), qhi[4 * c + 2], acc);
                        acc = mfma32(cvt8(x1.z, x1.w), qhi[4 * c + 3], acc);
                        const v8i32 araw = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                            (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                        acc_lo = mfma32_f8(araw, ql8[c], acc_lo, sb_lo);
                        if constexpr (WW) {
                            if (c == 1)
                                ok = weigh(t, buf, std::false_type{});
                        }
                    }
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[v] += acc_lo[v];
                    if constexpr (MXL) {
                        // this wave's part of the score of value v (row 8 (v /
                        // 4) + 4 hf + v % 4 of the wave's 32): 2^-k scale acc,
                        // with tile ts's row scales
                        const float* scp = s_sc + (ts & (NSC - 1)) * TR + 32 * rh + 4 * hf;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 sq = *reinterpret_cast<const float4*>(scp + 8 * q);
                            const float sv[4] = {sq.x, sq.y, sq.z, sq.w};
#pragma unroll
                            for (int c = 0; c < 4; ++c)
                                acc[4 * q + c] = (acc[4 * q + c] * pk) * sv[c];
                        }
                    }
                    if constexpr (MXL && KHC == 1) {
                        // + the RoPE part (in score units already): blocks 7
                        // and 8 (the wave's blocks 3 and 4), two 16-element K
                        // steps each, bf16 as stored, hi and lo terms
#pragma unroll
                        for (int bb = 0; bb < 2; ++bb) {
                            const bf16x8 r0 = *reinterpret_cast<const bf16x8*>(xs + 1024 * (3 + bb));
                            const bf16x8 r1 = *reinterpret_cast<const bf16x8*>(xs + 1024 * (3 + bb) + 512);
                            acc = mfma32_bf16(r0, qr[4 * bb + 0], acc);
                            acc = mfma32_bf16(r0, qr[4 * bb + 1], acc);
                            acc = mfma32_bf16(r1, qr[4 * bb + 2], acc);
                            acc = mfma32_bf16(r1, qr[4 * bb + 3], acc);
                        }
                    }
                } else {
                    constexpr int NH = KH / 2;  // 9 half column blocks
                    constexpr int PF = 2;
                    uint4 xr[PF + 1];
#pragma unroll
                    for (int j = 0; j < PF; ++j)
                        xr[j] = *reinterpret_cast<const uint4*>(xs + 512 * j);
                    // the row reads stay PF half blocks ahead: no LDS read may
                    // sink below these points (nor MFMAs rise above them)
                    __builtin_amdgcn_sched_barrier(kNoDsReadCross);
#pragma unroll
                    for (int j = 0; j < NH; ++j) {
                        if (j + PF < NH)
                            xr[(j + PF) % (PF + 1)] =
                                *reinterpret_cast<const uint4*>(xs + 512 * (j + PF));
                        __builtin_amdgcn_sched_barrier(kNoDsReadCross);
                        const uint4 x = xr[j % (PF + 1)];
                        const f16x8 a0 = cvt8(x.x, x.y), a1 = cvt8(x.z, x.w);
                        acc = mfma32(a0, qhi[2 * j], acc);
                        acc = mfma32(a0, qlo[2 * j], acc);
                        acc = mfma32(a1, qhi[2 * j + 1], acc);
                        acc = mfma32(a1, qlo[2 * j + 1], acc);
                        if constexpr (WW) {
                            if (j == 1)
                                ok = weigh(t, buf, std::false_type{});
                        }
                    }
                }
                return ok;
            };

            // Phase p (one barrier): the score MFMAs of tile p, the weights of
            // tile p-1 and their flag; first the vote on tile p-2 (the context
            // waves accumulate tile p-2 in this phase).  Two extra phases
            // finish the pipeline.
            for (int p = 0, st = 0; p <= ntiles + 1; ++p, st = (st == NST - 1) ? 0 : st + 1) {
                const int bw = (p + 1) & 1;   // weight / flag buffer of tile p-1
                lds_barrier();  // (A) tile p visible; tile p-1's partner half, the
                                //     weights and flags of tile p-2 complete;
                                //     buffer (p-1) & 1 free
                uint4 fl = make_uint4(0u, 0u, 0u, 0u);
                if (p >= 2)
                    fl = *reinterpret_cast<const uint4*>(s_fl + 4 * (p & 1));
                if (p >= 2 && vote(fl)) {
                    // u and row scales of tile p-2 (stored by its weigh);
                    // unscaled scores: pk is a power of 2
                    const float4 u0 = s_uv[0], u1 = s_uv[64], sc0 = s_uv[128], sc1 = s_uv[192];
                    const float u[8] = {u0.x * upk, u0.y * upk, u0.z * upk, u0.w * upk,
                                        u1.x * upk, u1.y * upk, u1.z * upk, u1.w * upk};
                    const float scv[8] = {sc0.x, sc0.y, sc0.z, sc0.w, sc1.x, sc1.y, sc1.z, sc1.w};
                    // exact maxima of tile p-2 (u, scv) for this lane's row
                    // quarter: T = max u, C = max (u - T) + log2 scale
                    // (relative, so that a large |u| never swallows log2
                    // scale); lanes l and l ^ 32 hold the quarter's 16 rows
                    float tw = -INFINITY;
#pragma unroll
                    for (int v = 0; v < 8; ++v)
                        tw = fmaxf(tw, u[v]);
                    tw = max_xor32(tw);
                    float cw = -INFINITY;
                    if (tw != -INFINITY) {
#pragma unroll
                        for (int v = 0; v < 8; ++v)
                            cw = fmaxf(cw, (u[v] - tw) + log2f(scv[v]));
                    }
                    cw = max_xor32(cw);
                    if (hf == 0)
                        s_cr2[hd * 4 + 2 * rh + KHC] = make_float2(tw, cw);
                    lds_barrier();  // (R1)
                    float alz[2], alo[2];
                    state_move(alz, alo, hsel);
                    zsave *= hsel ? alz[1] : alz[0];
                    weights_log(p & 1, u, scv);  // tile p-2 under the new state
                    lds_barrier();       // (R2) rewritten weights visible; s_cr free
                }
                const bool scored = p < ntiles, weighed = p >= 1 && p <= ntiles;
                bool ok = true;
                if (scored && weighed)
                    ok = stream(st, p, std::true_type{}, p - 1, bw);
                else if (scored)
                    stream(st, p, std::false_type{}, 0, 0);
                else if (weighed)
                    ok = weigh(p - 1, bw, std::true_type{});
                if (weighed) {
                    const bool flag = __any(!ok);
                    if (lane == 0)
                        s_fl[4 * bw + w] = flag ? 1u : 0u;
                }
                if (scored) {
                    // the partner's half of tile p to LDS, this wave's half kept
                    float4* xo = xc_ptr(p & 1, 1 - KHC);
                    constexpr int PO = 8 * (1 - KHC), OW = 8 * KHC;
                    xo[0] = make_float4(acc[PO + 0], acc[PO + 1], acc[PO + 2], acc[PO + 3]);
                    xo[64] = make_float4(acc[PO + 4], acc[PO + 5], acc[PO + 6], acc[PO + 7]);
#pragma unroll
                    for (int v = 0; v < 8; ++v)
                        accp[v] = acc[OW + v];
                }
            }
            // z of head hd over the lane's rows, then lanes l and l ^ 32
            float zz = zacc;
            zz += __shfl_xor(zz, 32);
            if (lane < 32)
                s_z[w * HG + lane] = zz;
        };
        if (kh == 0)
            score_role(std::integral_constant<int, 0>{});
        else
            score_role(std::integral_constant<int, 1>{});
    } else {
        // ======== context waves: O[32 heads][128 columns 128 c ..] += W . X
        // of tile p-2; column block jb = 32 columns, K step ks = 16 rows.
        const int c = wi;
        const int g = lane >> 4;
        // 32-column blocks of this wave (mixed rows: 448 columns, so the last
        // wave has 2)
        const int njb = (MXL && c == 3) ? 2 : 4;
        if (fresh_late)
            quantize_fresh(wi, 4);
        f32x16 O[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                O[jb][v] = 0.0f;
        // Transposed read: 16-lane group g covers columns 16 (g & 1) .. of
        // the 32-column block and rows 8 (g >> 1) .. of the K step; lanes
        // 2 k, 2 k + 1 address row 8 (g >> 1) + k, bytes 8 (lane & 1) of the
        // 16-byte slot.
        const int tr_row = 8 * (g >> 1) + ((lane & 15) >> 1);
        const int tr_off = (tr_row + 16 * (g & 1)) * 16 + 8 * (lane & 1);
        // weight operand: head lane % 32, rows 16 ks + 8 (lane / 32) ..
        const int w_off = (lane & 31) * WSTR + 8 * (lane >> 5);
        f16x8 wa[4];
        auto read_weights = [&](int buf) __attribute__((always_inline)) {
            const _Float16* sw = s_w + buf * HG * WSTR + w_off;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                wa[ks] = *reinterpret_cast<const f16x8*>(sw + 16 * ks);
        };
        auto read_rows = [&](int st, v2i32 (&xb)[4][4]) __attribute__((always_inline)) {
            const uint8_t* xst = lds + st * STAGE + tr_off;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    if (jb >= njb)
                        continue;
                    const int cb = 2 * c + (jb >> 1);
                    const int off = (ks * NCB + cb) * 1024 + 32 * (jb & 1) * 16;
                    xb[ks][jb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (MLA8_LDS v2i32*)(MLA8_LDS uint8_t*)(xst + off));
                }
        };
        auto accumulate = [&](const v2i32 (&xb)[4][4]) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
                    if (jb < njb)
                        O[jb] = mfma32(wa[ks], cvt8((uint32_t)xb[ks][jb][0], (uint32_t)xb[ks][jb][1]),
                                       O[jb]);
        };

        // Phase p: the context of tile p-2 (its weights from buffer p & 1,
        // its rows read into registers xb in phase p-2), after the vote on
        // it; then the rows of tile p into the same registers, for phase p+2.
        // Tile p-1's ring stage is free once this phase's barrier has passed
        // (both readers read it in phase p-1), so the loads of tile p + DIST
        // go there.
        auto phase = [&](int p, int st, v2i32 (&xb)[4][4]) __attribute__((always_inline)) {
            const int bw = p & 1;  // weight / flag buffer of tile p-2
            if (p < ntiles)
                wait_tile(p + 1 < ntiles);
            lds_barrier();  // (A)
            const bool more = p + DIST < ntiles;
            const int sti = (st + DIST) % NST;
            const bool ctx = p >= 2;
            uint4 fl = make_uint4(0u, 0u, 0u, 0u);
            if (ctx) {
                fl = *reinterpret_cast<const uint4*>(s_fl + 4 * bw);
                read_weights(bw);
            }
            if (more)
                issue(p + DIST, sti, IC0{}, ICA{});
            if (ctx && vote(fl)) {
                lds_barrier();  // (R1) the score waves' tile maxima are in s_cr
                float alz[2], alo[2];
                state_move(alz, alo, 0);
                // O holds tiles < p-2 in units of the old state; its head
                // 8 (v / 4) + 4 (lane / 32) + v % 4 takes that head's factor,
                // through a per-wave table in LDS (a wave's LDS accesses
                // complete in order)
                float* const al = reinterpret_cast<float*>(lds + AL) + HG * wi;
                if (lane < 16) {
                    al[lane] = alo[0];
                    al[16 + lane] = alo[1];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 f = reinterpret_cast<const float4*>(al)[2 * q + (lane >> 5)];
                    const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int jb = 0; jb < 4; ++jb)
                            O[jb][4 * q + r] *= fv[r];
                }
                lds_barrier();  // (R2) the rewritten weights of tile p-2 are visible
                read_weights(bw);
            }
            if (more)
                issue(p + DIST, sti, ICA{}, ICB{});
            if (ctx)
                accumulate(xb);
            if (more)
                issue(p + DIST, sti, ICB{}, ICK{});
            if (p < ntiles)
                read_rows(st, xb);
        };
        v2i32 xb0[4][4], xb1[4][4];
        for (int p = 0, st = 0; p <= ntiles + 1; p += 2) {
            phase(p, st, xb0);
            st = (st == NST - 1) ? 0 : st + 1;
            if (p + 1 <= ntiles + 1)
                phase(p + 1, st, xb1);
            st = (st == NST - 1) ? 0 : st + 1;
        }
        // partial cl = sum_t p_t scale_t x_t = 2^d * O
        const float fo0 = (mrun0 == -INFINITY || drun0 == -INFINITY) ? 0.0f : fast_exp2(drun0);
        const float fo1 = (mrun1 == -INFINITY || drun1 == -INFINITY) ? 0.0f : fast_exp2(drun1);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int hd = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const float fa = __shfl(fo0, hd & 15), fb = __shfl(fo1, hd & 15);
            const float f = (hd >> 4) ? fb : fa;
            const int qh = qh0 + hd;
            if (qh < a.n_qh) {
                // streaming stores: the merge reads the partials once, from
                // beyond L2 (another XCD's workgroups wrote most of them)
                float* dst = a.ws_cl + (pbase + qh) * LCO + 128 * c + (lane & 31);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
                    if (jb < njb)
                        __builtin_nontemporal_store(O[jb][v] * f, dst + 32 * jb);
            }
        }
    }

    // ---- partial m and z (z summed over the four score waves' row quarters),
    // streaming stores like cl's: no dirty L2 lines left for the kernel's end
    __syncthreads();
    if (w < 2 && lane < 16) {
        const int h = 16 * (w & 1) + n, qh = qh0 + h;
        if (qh < a.n_qh) {
            __builtin_nontemporal_store((w & 1) ? mrun1 : mrun0, a.ws_m + pbase + qh);
            __builtin_nontemporal_store((s_z[h] + s_z[HG + h]) + (s_z[2 * HG + h] + s_z[3 * HG + h]),
                                        a.ws_z + pbase + qh);
        }
    }
}

bool partial32_applies(const AttnArgs& a)
{
    const bool e4 = a.layout == kE4m3 && a.lc == p32::LC && a.rc == p32::RC;
    // mixed rows (448 e4m3 + 64 bf16) only with the e4m3 lo term; their
    // f32-grade path is the general kernel's
    const bool mx = a.layout == kMixed && a.lc == 448 && a.rc == p32::RC && a.lo8;
    if (!(e4 || mx) || a.n_list < p32::TR)
        return false;
    if (a.mode == kDense || a.mode == kSelect)
        return true;
    // causal batch: every group within one query position, and every query's
    // rows (at least pos0 + 1) fill a tile, which the ragged last tile needs
    return a.mode == kCausal && a.n_heads % kHeadsPerGroup == 0 && a.pos0 + 1 >= p32::TR;
}

template <bool LO8, bool GATHER, bool MXL>
static void launch32(const AttnArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.n_chunks * a.n_groups));
    hipLaunchKernelGGL((k_partial32<LO8, GATHER, MXL>), grid, dim3(kThreads), 0, stream, a);
}

void launch_partial32(const AttnArgs& a, hipStream_t stream)
{
    const bool g = a.mode == kSelect;
    if (a.layout == kMixed) {
        if (g)
            launch32<true, true, true>(a, stream);
        else
            launch32<true, false, true>(a, stream);
    } else if (a.lo8) {
        if (g)
            launch32<true, true, false>(a, stream);
        else
            launch32<true, false, false>(a, stream);
    } else {
        if (g)
            launch32<false, true, false>(a, stream);
        else
            launch32<false, false, false>(a, stream);
    }
}

}  // namespace mla8
