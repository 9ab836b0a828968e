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
//   * k_index_select: the first radix digit b1 of the k-th largest key comes
//     from the global histogram; every workgroup compacts the keys of its
//     slice whose digit is >= b1 into a candidate list of 64-bit (key, ~row)
//     values (unique, and larger for a larger score or, on a tie, a smaller
//     row).  The last workgroup to finish (device-scope release/acquire on a
//     counter) finds the k-th largest candidate exactly by a radix select over
//     the 64 bits in LDS histograms, gathers the k rows at or above it and
//     sorts them ascending in LDS (bitonic).
#include "mla8_device.h"
#include "mla8_internal.h"

namespace mla8 {

namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreRowsPerGroup = 512;   // 32 blocks of 16 rows, 8 per wave
constexpr int kScoreBatch = 4;            // blocks whose loads are in flight together
constexpr int kSelectThreads = 512;
constexpr int kSelectKeysPerThread = 8;
constexpr int kSelectSlice = kSelectThreads * kSelectKeysPerThread;
constexpr int kRadixBits = 11;
constexpr int kRadixBins = 1 << kRadixBits;

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

__global__ __launch_bounds__(kThreads) void k_index_clear(uint32_t* __restrict__ hist,
                                                          uint32_t* __restrict__ counters)
{
    for (int i = threadIdx.x; i < kIndexHistBins; i += blockDim.x)
        hist[i] = 0u;
    if (threadIdx.x < 2)
        counters[threadIdx.x] = 0u;
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

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
    for (int i = tid; i < kIndexHistBins; i += kScoreThreads)
        s_hist[i] = 0u;
    if (tid < 16 * NT)
        s_w[tid] = a.w[tid];

    // ---- query quantization, the shadow's per-row arithmetic: lane group g
    // of wave w takes heads 16w + 4i + g, lane n their values 8n .. 8n + 7
    if (w < NT) {
        float4 v[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4* src = reinterpret_cast<const float4*>(
                a.q + (size_t)(16 * w + 4 * i + g) * kIndexDim + 8 * n);
            v[i][0] = src[0];
            v[i][1] = src[1];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 16 * w + 4 * i + g;
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

    // A operand of head tile ht: head 16 ht + n, K bytes 16g .. 16g + 15 and
    // 64 + 16g .. 64 + 16g + 15 (the same K split as the key operand).
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

    // ---- key blocks: wave w takes blocks w, w + 4, ... of the group's rows
    const int r0 = blockIdx.x * kScoreRowsPerGroup;
    constexpr int kBlocksPerWave = kScoreRowsPerGroup / 16 / 4;
    for (int b0 = 0; b0 < kBlocksPerWave; b0 += kScoreBatch) {
        uint4 k0[kScoreBatch], k1[kScoreBatch];
        float ks[kScoreBatch];
        int rows[kScoreBatch];
#pragma unroll
        for (int j = 0; j < kScoreBatch; ++j) {
            rows[j] = r0 + 16 * (w + 4 * (b0 + j)) + n;
            const int rc = min(rows[j], a.t_rows - 1);  // rows past the end reload the last
            const uint8_t* kp = a.k_codes + (size_t)rc * kIndexDim + 16 * g;
            k0[j] = *reinterpret_cast<const uint4*>(kp);
            k1[j] = *reinterpret_cast<const uint4*>(kp + 64);
            ks[j] = a.k_scales[rc];
        }
#pragma unroll
        for (int j = 0; j < kScoreBatch; ++j) {
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
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < kIndexHistBins; i += kScoreThreads) {
        const uint32_t c = s_hist[i];
        if (c)
            atomicAdd(&a.hist[i], c);
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

}  // namespace

__global__ __launch_bounds__(kSelectThreads) void k_index_select(IndexArgs a)
{
    __shared__ uint32_t s_h[kIndexHistBins];
    __shared__ uint32_t s_tmp[kSelectThreads / 64];
    __shared__ uint32_t s_out[2];
    __shared__ uint32_t s_base;
    __shared__ uint32_t s_last;
    __shared__ uint32_t s_rows[kIndexMaxTopK];

    const int tid = threadIdx.x;
    const uint32_t k = (uint32_t)a.top_k;

    // ---- first digit of the k-th largest key, from the global histogram
    for (int i = tid; i < kIndexHistBins; i += kSelectThreads)
        s_h[i] = a.hist[i];
    __syncthreads();
    find_bin_from_top(s_h, kIndexHistBins, k, s_tmp, s_out);
    const uint32_t b1 = s_out[0];

    // ---- candidates of this slice: keys whose first digit is >= b1
    const int t0 = blockIdx.x * kSelectSlice;
    // (a candidate is never 0: its low word ~row is nonzero)
    uint64_t c[kSelectKeysPerThread];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kSelectKeysPerThread; ++j) {
        const int t = t0 + j * kSelectThreads + tid;
        c[j] = 0;
        if (t < a.t_rows) {
            const uint32_t key = a.keys[t];
            if ((key >> 20) >= b1) {
                c[j] = ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)t);
                ++cnt;
            }
        }
    }
    uint32_t total;
    const uint32_t off = block_excl_scan(cnt, s_tmp, &total);
    if (tid == 0)
        s_base = total ? atomicAdd(&a.counters[0], total) : 0u;
    __syncthreads();
    uint32_t pos = s_base + off;
#pragma unroll
    for (int j = 0; j < kSelectKeysPerThread; ++j)
        if (c[j] != 0)
            a.cand[pos++] = c[j];
    // publish this workgroup's candidates; the last workgroup selects
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(&a.counters[1], 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (done == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();
    const uint32_t n_cand = __hip_atomic_load(&a.counters[0], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);

    // ---- radix select of the k-th largest candidate, 11 bits at a time from
    // the top (the last digit has 9)
    uint64_t prefix = 0;
    int done_bits = 0;
    uint32_t rem = k;
    while (done_bits < 64) {
        const int width = min(kRadixBits, 64 - done_bits);
        const int shift = 64 - done_bits - width;
        const uint32_t nb = 1u << width;
        for (uint32_t i = tid; i < nb; i += kSelectThreads)
            s_h[i] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < n_cand; i += kSelectThreads) {
            const uint64_t v = a.cand[i];
            if (done_bits == 0 || (v >> (64 - done_bits)) == prefix)
                atomicAdd(&s_h[(uint32_t)(v >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        find_bin_from_top(s_h, (int)nb, rem, s_tmp, s_out);
        prefix = (prefix << width) | s_out[0];
        rem = s_out[1];
        done_bits += width;
        __syncthreads();
    }
    const uint64_t tau = prefix;  // the k-th largest candidate

    // ---- the k rows at or above tau, sorted ascending
    if (tid == 0)
        s_base = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n_cand; i += kSelectThreads) {
        const uint64_t v = a.cand[i];
        if (v >= tau) {
            const uint32_t p = atomicAdd(&s_base, 1u);
            if (p < k)
                s_rows[p] = ~(uint32_t)v;
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

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(k_index_clear, dim3(1), dim3(kThreads), 0, stream, a.hist, a.counters);
    const unsigned gs = (unsigned)((a.t_rows + kScoreRowsPerGroup - 1) / kScoreRowsPerGroup);
    switch (a.n_ih / 16) {
    case 1: hipLaunchKernelGGL(k_index_score<1>, dim3(gs), dim3(kScoreThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(k_index_score<2>, dim3(gs), dim3(kScoreThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(k_index_score<3>, dim3(gs), dim3(kScoreThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(k_index_score<4>, dim3(gs), dim3(kScoreThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    if (a.t_rows <= a.top_k) {
        hipLaunchKernelGGL(k_index_all, dim3((unsigned)((a.t_rows + 255) / 256)), dim3(256), 0,
                           stream, a.sel, a.t_rows);
    } else {
        const unsigned gsel = (unsigned)((a.t_rows + kSelectSlice - 1) / kSelectSlice);
        hipLaunchKernelGGL(k_index_select, dim3(gsel), dim3(kSelectThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace mla8
