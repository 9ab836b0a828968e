// HIP kernels for gfx950 (MI355X): the fp8 indexer score and the top-k
// selection that produces the rows the selected-row decode attends.
//
// Method source: "B1 Mixed FP8/BF16 FMHA first pass" site, commit message of
// the B2 fp8 indexer score + top-k kernel: the indexer query (64 heads x 128)
// is quantized to fp8, the keys are read as e4m3, each head's dot product is
// dequantized by q_scale * k_scale and passed through ReLU, the heads are
// summed with per-head weights, and the top-k rows are kept.  The row format
// of the keys is the latent shadow's (colibri PR #300, "KV8 base" commit,
// c/kv_fp8.h bullet): e4m3 bytes with one f32 amax/448 scale per row.
//
//     I_t = sum_j w_j * max(0, (acc_jt * q_scale_j) * k_scale_t),
//     acc_jt = sum_d q8_jd * k8_td   (one 16x16x128 fp8 MFMA per 16 heads x 16 rows)
//
// gfx950 design:
//   * k_index_score: 512 rows per workgroup, 4 waves; every workgroup
//     quantizes the query into LDS with the shadow's row arithmetic, then each
//     wave streams 16-row blocks of keys straight from HBM into the B operand
//     of v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales; ihd = 128 is exactly
//     one MFMA K), n_ih / 16 MFMAs per block.  The result lane (n, g) holds
//     heads 4g..4g+3 of each 16-head tile for key row n, so the head sum is
//     in-lane plus two cross-lane adds.  Scores become order-preserving u32
//     keys; a per-workgroup LDS histogram of the keys' top 12 bits is added
//     to a global one.
//     The histogram has one copy per XCD (workgroups are dispatched
//     round-robin over the 8 XCDs), so fewer workgroups add to each bin; the
//     largest key goes by atomic max to one word per copy likewise.
//   * k_index_cand: the first radix digit b1 of the k-th largest key comes
//     from the summed histogram, read in windows from the largest key's bin
//     down until k keys are counted; every workgroup compacts the keys of its
//     4096-row slice whose digit is >= b1 into the slice's part of a
//     candidate buffer, in row order, as (key << 32 | row).
//   * k_index_final (one workgroup): the candidates, packed in row order into
//     LDS, give the k-th largest key tau by a radix select in LDS histograms;
//     the rows with a larger key and the first rows (in row order) with key
//     tau make the selection, written in ascending order by one ordered
//     compaction.  When the candidates do not fit in LDS (many equal scores)
//     it selects over 64-bit (key, ~row) values in global memory and sorts the
//     k rows in LDS instead.
#include "mla8_device.h"
#include "mla8_internal.h"

namespace mla8 {

namespace {

constexpr int kScoreThreads = 512;
constexpr int kScoreRowsPerGroup = 512;  // 32 blocks of 16 rows
constexpr int kScoreBlocksPerWave = kScoreRowsPerGroup / 16 / (kScoreThreads / 64);
constexpr int kSelectThreads = 512;
constexpr int kSelectKeysPerThread = 8;  // contiguous rows per thread
constexpr int kSelectSlice = kSelectThreads * kSelectKeysPerThread;
constexpr int kRadixBits = 11;
constexpr int kLdsCand = 12288;          // candidates resolved in LDS (96 KB)
static_assert(kLdsCand < (1 << 16), "packed 16-bit counts in the ordered output");
static_assert(kIndexMaxRows / kSelectSlice <= kIndexHistBins, "per-slice tables fit in LDS");

__device__ __forceinline__ f32x4 mfma_fp8(v8i a, v8i b, f32x4 c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Order-preserving map of a score to u32: a larger score gives a larger key,
// +0 and -0 give the same key, and NaN gives 0, below every other score.
__device__ __forceinline__ uint32_t order_key(float s)
{
    s = s + 0.0f;  // -0 + 0 = +0 under round-to-nearest
    const uint32_t b = __float_as_uint(s);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u)
        return 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

}  // namespace

// One workgroup per histogram copy and largest-key word.
__global__ __launch_bounds__(kThreads) void k_index_clear(uint32_t* __restrict__ hist,
                                                          uint32_t* __restrict__ top)
{
    uint32_t* h = hist + (size_t)blockIdx.x * kIndexHistBins;
    for (int i = threadIdx.x; i < kIndexHistBins; i += blockDim.x)
        h[i] = 0u;
    if (threadIdx.x == 0)
        top[16 * blockIdx.x] = 0u;
}

// ---------------------------------------------------------------------------
// Scores, keys and the first-digit histogram.  NT = n_ih / 16 head tiles.
template <int NT>
__global__ __launch_bounds__(kScoreThreads) void k_index_score(IndexArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kIndexMaxHeads * kIndexDim];
    __shared__ float s_qs[kIndexMaxHeads];
    __shared__ float s_w[kIndexMaxHeads];
    __shared__ uint32_t s_hist[kIndexHistBins];
    __shared__ uint32_t s_top;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
    constexpr int NW = kScoreThreads / 64;

    // ---- query loads first, then the wave's key blocks w, w + 8, w + 16,
    // w + 24, so the query quantization waits only for the query.  Lane group
    // g of wave w quantizes heads 8w + 4i + g (i = 0, 1), lane n their values
    // 8n .. 8n + 7; whether a head exists is uniform over the wave.
    float4 v[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (8 * w + 4 * i < 16 * NT) {
            const float4* src = reinterpret_cast<const float4*>(
                a.q + (size_t)(8 * w + 4 * i + g) * kIndexDim + 8 * n);
            v[i][0] = src[0];
            v[i][1] = src[1];
        }
    }
    // Lane (n, g) loads row n of a key block, K bytes 16g .. 16g + 15 and
    // 64 + 16g .. 64 + 16g + 15 (the MFMA operand split).
    const int r0 = blockIdx.x * kScoreRowsPerGroup;
    uint4 k0[kScoreBlocksPerWave], k1[kScoreBlocksPerWave];
    float ks[kScoreBlocksPerWave];
    int rows[kScoreBlocksPerWave];
#pragma unroll
    for (int j = 0; j < kScoreBlocksPerWave; ++j) {
        rows[j] = r0 + 16 * (w + NW * j) + n;
        const int rc = min(rows[j], a.t_rows - 1);  // rows past the end reload the last
        const uint8_t* kp = a.k_codes + (size_t)rc * kIndexDim + 16 * g;
        k0[j] = *reinterpret_cast<const uint4*>(kp);
        k1[j] = *reinterpret_cast<const uint4*>(kp + 64);
        ks[j] = a.k_scales[rc];
    }

    for (int i = tid; i < kIndexHistBins; i += kScoreThreads)
        s_hist[i] = 0u;
    if (tid == 0)
        s_top = 0u;
    if (tid < 16 * NT)
        s_w[tid] = a.w[tid];

    // ---- query quantization with the shadow's per-row arithmetic
    {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (8 * w + 4 * i >= 16 * NT)
                continue;
            const int h = 8 * w + 4 * i + g;
            const float e[8] = {v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w,
                                v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w};
            float amax = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c)
                if (fabsf(e[c]) <= 3.402823466e38f)  // finite only
                    amax = fmaxf(amax, fabsf(e[c]));
            amax = row16_max(amax);
            float scale, inv;
            row_scale_inv(amax, scale, inv);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                lo |= enc_e4m3(e[c] * inv) << (8 * c);
                hi |= enc_e4m3(e[4 + c] * inv) << (8 * c);
            }
            *reinterpret_cast<uint2*>(s_q + h * kIndexDim + 8 * n) = make_uint2(lo, hi);
            if (n == 0)
                s_qs[h] = scale;
        }
    }
    __syncthreads();

    // A operand of head tile ht: head 16 ht + n, the same K split as the keys.
    v8i qa[NT];
    float fq[NT][4], fw[NT][4];
#pragma unroll
    for (int ht = 0; ht < NT; ++ht) {
        const uint8_t* qp = s_q + (16 * ht + n) * kIndexDim + 16 * g;
        const uint4 x0 = *reinterpret_cast<const uint4*>(qp);
        const uint4 x1 = *reinterpret_cast<const uint4*>(qp + 64);
        qa[ht] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            fq[ht][v] = s_qs[16 * ht + 4 * g + v];
            fw[ht][v] = s_w[16 * ht + 4 * g + v];
        }
    }

    // ---- scores: lane (n, g) gets heads 16 ht + 4g + v of key row n
    uint32_t kmax = 0u;  // largest key this lane wrote
#pragma unroll
    for (int j = 0; j < kScoreBlocksPerWave; ++j) {
        const v8i kb = v8i{(int)k0[j].x, (int)k0[j].y, (int)k0[j].z, (int)k0[j].w,
                           (int)k1[j].x, (int)k1[j].y, (int)k1[j].z, (int)k1[j].w};
        float r = 0.0f;
#pragma unroll
        for (int ht = 0; ht < NT; ++ht) {
            const f32x4 acc = mfma_fp8(qa[ht], kb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int v = 0; v < 4; ++v)
                r += fw[ht][v] * fmaxf((acc[v] * fq[ht][v]) * ks[j], 0.0f);
        }
        r += __shfl_xor(r, 16);
        r += __shfl_xor(r, 32);
        if (g == 0 && rows[j] < a.t_rows) {
            const uint32_t key = order_key(r);
            a.keys[rows[j]] = key;
            if (a.scores)
                a.scores[rows[j]] = r;
            atomicAdd(&s_hist[key >> 20], 1u);
            kmax = max(kmax, key);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    if (lane == 0)
        atomicMax(&s_top, kmax);
    __syncthreads();
    if (tid == 0)
        atomicMax(&a.top[16 * (blockIdx.x % kIndexHistCopies)], s_top);
    // into the histogram copy of this workgroup's XCD (dispatch is
    // round-robin over the 8 XCDs)
    uint32_t* const hist = a.hist + (size_t)(blockIdx.x % kIndexHistCopies) * kIndexHistBins;
    for (int i = tid; i < kIndexHistBins; i += kScoreThreads) {
        const uint32_t c = s_hist[i];
        if (c)
            atomicAdd(&hist[i], c);
    }
}

// ---------------------------------------------------------------------------
// Workgroup scans for the selection kernel (kSelectThreads threads).
namespace {

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o)
            x += y;
    }
    return x;
}

// Exclusive prefix sum of x over the threads of the workgroup; *total gets the
// sum.  s_tmp holds one entry per wave.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* s_tmp, uint32_t* total)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    constexpr int NWV = kSelectThreads / 64;
    const uint32_t inc = wave_incl_scan(x, lane);
    __syncthreads();
    if (lane == 63)
        s_tmp[wv] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
        const uint32_t t = s_tmp[i];
        before += (i < wv) ? t : 0u;
        all += t;
    }
    *total = all;
    return before + inc - x;
}

// Over histogram bins h[0 .. nb) counted from the top bin down, find the bin
// holding the rem-th largest element (rem >= 1, at most the histogram total):
// writes the bin and the element's rank inside it to s_out[0], s_out[1].
__device__ __forceinline__ void find_bin_from_top(const uint32_t* h, int nb, uint32_t rem,
                                                  uint32_t* s_tmp, uint32_t* s_out)
{
    const int tid = threadIdx.x;
    const int per = (nb + kSelectThreads - 1) / kSelectThreads;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j) {
        const int b = nb - 1 - (tid * per + j);
        if (b >= 0)
            local += h[b];
    }
    uint32_t total;
    const uint32_t excl = block_excl_scan(local, s_tmp, &total);
    if (excl < rem && rem <= excl + local) {
        uint32_t r = rem - excl;
        for (int j = 0; j < per; ++j) {
            const int b = nb - 1 - (tid * per + j);
            const uint32_t c = h[b];
            if (r <= c) {
                s_out[0] = (uint32_t)b;
                s_out[1] = r;
                break;
            }
            r -= c;
        }
    }
    __syncthreads();
}

// Radix select over n values of `bits` significant bits read by get(i):
// the value of rank rem (1 = largest) and, in *rem_out, its rank among the
// values equal to it.  s_h must hold 2^kRadixBits counters.
template <typename Get>
__device__ __forceinline__ uint64_t radix_select(Get get, uint32_t n, int bits, uint32_t rem,
                                                 uint32_t* s_h, uint32_t* s_tmp, uint32_t* s_out,
                                                 uint32_t* rem_out)
{
    const int tid = threadIdx.x;
    uint64_t prefix = 0;
    int done = 0;
    while (done < bits) {
        const int width = min(kRadixBits, bits - done);
        const int shift = bits - done - width;
        const uint32_t nb = 1u << width;
        for (uint32_t i = tid; i < nb; i += kSelectThreads)
            s_h[i] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < n; i += kSelectThreads) {
            bool in;
            const uint64_t v = get(i, in);
            if (in && (done == 0 || (v >> (bits - done)) == prefix))
                atomicAdd(&s_h[(uint32_t)(v >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        find_bin_from_top(s_h, (int)nb, rem, s_tmp, s_out);
        prefix = (prefix << width) | s_out[0];
        rem = s_out[1];
        done += width;
        __syncthreads();
    }
    *rem_out = rem;
    return prefix;
}

}  // namespace

// ---------------------------------------------------------------------------
// Candidates.  Slice i (rows 4096 i ..) is workgroup i's: its keys whose first
// digit is at least that of the k-th largest key go to cand[4096 i ..] in row
// order as (key << 32 | row), their count to wg_cnt[i].
__global__ __launch_bounds__(kSelectThreads) void k_index_cand(IndexArgs a)
{
    __shared__ uint32_t s_tmp[kSelectThreads / 64];
    __shared__ uint32_t s_out[2];

    const int tid = threadIdx.x;
    // thread tid owns rows tb .. tb + 7; its keys load first
    const int tb = blockIdx.x * kSelectSlice + kSelectKeysPerThread * tid;
    uint32_t key[kSelectKeysPerThread];
    if (tb + kSelectKeysPerThread <= a.t_rows) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(a.keys + tb);
        const uint4 x1 = *reinterpret_cast<const uint4*>(a.keys + tb + 4);
        key[0] = x0.x; key[1] = x0.y; key[2] = x0.z; key[3] = x0.w;
        key[4] = x1.x; key[5] = x1.y; key[6] = x1.z; key[7] = x1.w;
    } else {
#pragma unroll
        for (int j = 0; j < kSelectKeysPerThread; ++j)
            key[j] = (tb + j < a.t_rows) ? a.keys[tb + j] : 0u;
    }
    // the bin b1 of the k-th largest key: windows of kSelectThreads bins of
    // the summed histogram copies, from the bin of the largest key down,
    // until the keys counted reach k (every key is counted, and k < t_rows,
    // so the search ends by bin 0)
    const uint32_t k = (uint32_t)a.top_k;
    uint32_t above = 0;  // keys in the bins above the window
    uint32_t tmax = 0u;
#pragma unroll
    for (int r = 0; r < kIndexHistCopies; ++r)
        tmax = max(tmax, a.top[16 * r]);
    for (int wtop = (int)(tmax >> 20);; wtop -= kSelectThreads) {
        const int b = wtop - tid;
        uint32_t c = 0;
        if (b >= 0) {
#pragma unroll
            for (int r = 0; r < kIndexHistCopies; ++r)
                c += a.hist[(size_t)r * kIndexHistBins + b];
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(c, s_tmp, &tot);  // keys in bins b+1 .. wtop
        if (above + ex < k && k <= above + ex + c) {
            s_out[0] = (uint32_t)b;
            s_out[1] = above + ex;  // keys in the bins above b
        }
        if (above + tot >= k || wtop - kSelectThreads < 0)
            break;
        above += tot;
    }
    __syncthreads();
    const uint32_t b1 = s_out[0];
    if (blockIdx.x == 0 && tid == 0) {  // for the final selection
        a.top[1] = b1;
        a.top[2] = s_out[1];
    }

    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kSelectKeysPerThread; ++j)
        cnt += (tb + j < a.t_rows && (key[j] >> 20) >= b1) ? 1u : 0u;
    uint32_t total;
    uint32_t pos = block_excl_scan(cnt, s_tmp, &total);
    uint64_t* const dst = a.cand + (size_t)blockIdx.x * kSelectSlice;
#pragma unroll
    for (int j = 0; j < kSelectKeysPerThread; ++j)
        if (tb + j < a.t_rows && (key[j] >> 20) >= b1)
            dst[pos++] = ((uint64_t)key[j] << 32) | (uint32_t)(tb + j);
    if (tid == 0)
        a.wg_cnt[blockIdx.x] = total;
}

// Final selection, one workgroup: the k-th largest candidate and the rows at
// or above it, in ascending row order.  n_slices = ceil(t_rows / 4096).
__global__ __launch_bounds__(kSelectThreads) void k_index_final(IndexArgs a, int32_t n_slices)
{
    __shared__ uint32_t s_h[kIndexHistBins];   // per-slice counts, then histograms
    __shared__ uint32_t s_pre[kIndexHistBins]; // per-slice start in the packed order
    __shared__ uint32_t s_tmp[kSelectThreads / 64];
    __shared__ uint32_t s_out[2];
    __shared__ uint64_t s_c[kLdsCand];

    const int tid = threadIdx.x;
    const uint32_t k = (uint32_t)a.top_k;
    const uint32_t ns = (uint32_t)n_slices;
    // the candidate pass's first-digit bin and the keys above it, loaded
    // with the counts (not after a barrier, one memory round trip later)
    const uint32_t b1 = a.top[1], above = a.top[2];

    // ---- per-slice counts and their exclusive prefix
    const uint32_t per = (ns + kSelectThreads - 1) / kSelectThreads;
    uint32_t loc = 0;
    for (uint32_t j = 0; j < per; ++j) {
        const uint32_t i = tid * per + j;
        const uint32_t c = (i < ns) ? a.wg_cnt[i] : 0u;
        if (i < ns)
            s_h[i] = c;
        loc += c;
    }
    uint32_t n_cand;
    uint32_t run = block_excl_scan(loc, s_tmp, &n_cand);
    for (uint32_t j = 0; j < per; ++j) {
        const uint32_t i = tid * per + j;
        if (i < ns) {
            s_pre[i] = run;
            run += s_h[i];
        }
    }
    __syncthreads();

    if (n_cand <= (uint32_t)kLdsCand) {
        // ---- candidates into LDS in row order: packed position p lies in
        // the last slice whose start is <= p
        for (uint32_t p0 = 0; p0 < n_cand; p0 += kSelectThreads * 8) {
            uint64_t v[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const uint32_t p = p0 + b * kSelectThreads + tid;
                v[b] = 0;
                if (p < n_cand) {
                    uint32_t lo = 0, hi = ns - 1;
                    while (lo < hi) {
                        const uint32_t mid = (lo + hi + 1) >> 1;
                        if (s_pre[mid] <= p)
                            lo = mid;
                        else
                            hi = mid - 1;
                    }
                    v[b] = a.cand[(size_t)lo * kSelectSlice + (p - s_pre[lo])];
                }
            }
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const uint32_t p = p0 + b * kSelectThreads + tid;
                if (p < n_cand)
                    s_c[p] = v[b];
            }
        }
        __syncthreads();

        // ---- the k-th largest key tau; the rows taken are those with a
        // larger key and the first `rem` (in row order) with key tau.  Its top
        // 12 bits are the candidate pass's bin b1, with `above` keys in higher
        // bins, so only the low 20 bits of the keys in bin b1 are selected on.
        uint32_t rem;
        const uint32_t tau = (b1 << 20) | (uint32_t)radix_select(
            [&](uint32_t i, bool& in) -> uint64_t {
                const uint32_t kk = (uint32_t)(s_c[i] >> 32);
                in = (kk >> 20) == b1;
                return kk & 0xFFFFFu;
            },
            n_cand, 20, k - above, s_h, s_tmp, s_out, &rem);

        // ---- ordered output: thread tid takes a contiguous run of the
        // packed candidates.  One scan of (keys above tau, keys equal to tau)
        // per thread, packed 16 + 16 bits (counts below 2^14), gives both the
        // tie rank of the thread's first tie and its first output position:
        // the ties are taken in row order, so min(tie0, rem) of them precede.
        const uint32_t ch = (n_cand + kSelectThreads - 1) / kSelectThreads;
        const uint32_t c0 = min(n_cand, tid * ch), c1 = min(n_cand, c0 + ch);
        uint32_t ngt = 0, nt = 0;
        for (uint32_t i = c0; i < c1; ++i) {
            const uint32_t kk = (uint32_t)(s_c[i] >> 32);
            ngt += (kk > tau) ? 1u : 0u;
            nt += (kk == tau) ? 1u : 0u;
        }
        uint32_t all;
        const uint32_t ex = block_excl_scan((nt << 16) | ngt, s_tmp, &all);
        const uint32_t tie0 = ex >> 16;
        uint32_t out = (ex & 0xFFFFu) + min(tie0, rem);
        uint32_t tie = tie0;
        for (uint32_t i = c0; i < c1; ++i) {
            const uint32_t kk = (uint32_t)(s_c[i] >> 32);
            if (kk > tau || (kk == tau && tie++ < rem)) {
                if (out < k)
                    a.sel[out] = (int32_t)(uint32_t)s_c[i];
                ++out;
            }
        }
        return;
    }

    // ---- many candidates (many equal scores): select in global memory over
    // 64-bit (key, ~row) values, unique and ordered by score then row, then
    // sort the k rows.  Slot j of the candidate buffer is valid when its
    // offset in slice j / 4096 is below that slice's count.
    uint32_t rem;
    const uint32_t nslot = ns * kSelectSlice;
    const uint64_t tau = radix_select(
        [&](uint32_t j, bool& in) -> uint64_t {
            in = (j & (kSelectSlice - 1)) < s_h[j / kSelectSlice];
            if (!in)
                return 0;
            const uint64_t v = a.cand[j];
            return (v & 0xFFFFFFFF00000000ull) | (uint64_t)(~(uint32_t)v);
        },
        nslot, 64, k, s_pre /* the counts stay in s_h */, s_tmp, s_out, &rem);
    uint32_t* const s_rows = reinterpret_cast<uint32_t*>(s_c);
    if (tid == 0)
        s_out[0] = 0u;
    __syncthreads();
    for (uint32_t j = tid; j < nslot; j += kSelectThreads) {
        if ((j & (kSelectSlice - 1)) >= s_h[j / kSelectSlice])
            continue;
        const uint64_t v = a.cand[j];
        const uint64_t cv = (v & 0xFFFFFFFF00000000ull) | (uint64_t)(~(uint32_t)v);
        if (cv >= tau) {
            const uint32_t p = atomicAdd(&s_out[0], 1u);
            if (p < k)
                s_rows[p] = (uint32_t)v;
        }
    }
    __syncthreads();
    uint32_t np2 = 1;
    while (np2 < k)
        np2 <<= 1;
    for (uint32_t i = k + tid; i < np2; i += kSelectThreads)
        s_rows[i] = 0xFFFFFFFFu;
    __syncthreads();
    for (uint32_t size = 2; size <= np2; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (uint32_t i = tid; i < np2 / 2; i += kSelectThreads) {
                const uint32_t lo = 2 * stride * (i / stride) + (i % stride);
                const uint32_t hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint32_t x = s_rows[lo], y = s_rows[hi];
                if ((x > y) == up) {
                    s_rows[lo] = y;
                    s_rows[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    for (uint32_t i = tid; i < k; i += kSelectThreads)
        a.sel[i] = (int32_t)s_rows[i];
}

// Every row selected (t_rows <= top_k).
__global__ __launch_bounds__(256) void k_index_all(int32_t* __restrict__ sel, int32_t t_rows)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < t_rows)
        sel[i] = i;
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t stream, hipEvent_t ev_before,
                             hipEvent_t ev_after)
{
    hipLaunchKernelGGL(k_index_clear, dim3(kIndexHistCopies), dim3(kThreads), 0, stream, a.hist,
                       a.top);
    const unsigned gs = (unsigned)((a.t_rows + kScoreRowsPerGroup - 1) / kScoreRowsPerGroup);
    if (ev_before != nullptr) {
        const hipError_t e = hipEventRecord(ev_before, stream);
        if (e != hipSuccess)
            return e;
    }
    switch (a.n_ih / 16) {
    case 1: hipLaunchKernelGGL(k_index_score<1>, dim3(gs), dim3(kScoreThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(k_index_score<2>, dim3(gs), dim3(kScoreThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(k_index_score<3>, dim3(gs), dim3(kScoreThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(k_index_score<4>, dim3(gs), dim3(kScoreThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    if (ev_after != nullptr) {
        const hipError_t e = hipEventRecord(ev_after, stream);
        if (e != hipSuccess)
            return e;
    }
    if (a.t_rows <= a.top_k) {
        hipLaunchKernelGGL(k_index_all, dim3((unsigned)((a.t_rows + 255) / 256)), dim3(256), 0,
                           stream, a.sel, a.t_rows);
    } else {
        const unsigned gsel = (unsigned)((a.t_rows + kSelectSlice - 1) / kSelectSlice);
        hipLaunchKernelGGL(k_index_cand, dim3(gsel), dim3(kSelectThreads), 0, stream, a);
        hipLaunchKernelGGL(k_index_final, dim3(1), dim3(kSelectThreads), 0, stream, a,
                           (int32_t)gsel);
    }
    return hipGetLastError();
}

}  // namespace mla8
