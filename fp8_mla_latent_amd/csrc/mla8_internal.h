// Internal interface between the C-ABI layer (mla8_api.hip) and the kernels
// (mla8_kernels.hip).  Not installed; the public interface is include/mla8.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla8 {

// Rows per tile streamed through LDS, query-heads per workgroup, threads per
// workgroup of the split-T partial kernel.
constexpr int kTileRows = 64;
constexpr int kHeadsPerGroup = 32;
constexpr int kThreads = 512;
// Workgroups the automatic split plan aims for: one per compute unit of an
// MI355X (256 CUs in 8 XCDs).
constexpr int kTargetGroups = 256;

enum RowMode : int32_t { kDense = 0, kSelect = 1, kCausal = 2 };
// Stored row layouts: all e4m3 (codes of Lc + Rc values), or mixed (Lc = 448
// noPE values as e4m3, then Rc = 64 RoPE values as bf16).
enum RowLayout : int32_t { kE4m3 = 0, kMixed = 1 };

// One launch of the split-T attention (partial kernel + merge kernel).
struct AttnArgs {
    const uint8_t* codes;   // shadow codes [t_rows][d]
    const float* scales;    // shadow scales [t_rows]
    int32_t t_rows;         // rows present in the shadow
    const int32_t* sel;     // kSelect: absolute row indices [n_list]
    int32_t n_list;         // length of the attended row list
    const float* q_lat;     // [n_qh][lc]
    const float* q_rope;    // [n_qh][rc]
    int32_t lc, rc, d;      // d: bytes of a stored row (lc + rc, or lc + 2 rc mixed)
    int32_t layout;         // RowLayout
    int32_t n_qh;           // query-heads: n_heads, or n_q * n_heads for kCausal
    int32_t n_heads;        // heads per query position (kCausal)
    int32_t pos0;           // kCausal: position of query 0
    int32_t mode;           // RowMode
    float sm_log2;          // sm_scale * log2(e)
    int32_t n_chunks;       // row chunks (split-T partials)
    int32_t chunk_rows;     // rows per chunk, a multiple of kTileRows
    int32_t n_groups;       // head groups of kHeadsPerGroup
    float* ws_m;            // [n_chunks][n_qh]  running max, log2 units
    float* ws_z;            // [n_chunks][n_qh]  softmax normaliser
    float* ws_cl;           // [n_chunks][n_qh][lc] unnormalised context
    float* out;             // [n_qh][lc]
    float* lse;             // [n_qh] or nullptr
    // Fused append (kDense only): rows [new0, new0 + n_new) of the shadow are
    // quantized from x_new[n_new][d] by the workgroups whose chunk holds them,
    // before they stream it.  n_new = 0: nothing to append.
    const float* x_new;
    uint8_t* new_codes;     // the shadow codes, writable
    float* new_scales;      // the shadow scales, writable
    int32_t new0;
    int32_t n_new;
    // 1: the dense 512/64 partial kernel runs its lo query term on the e4m3
    // MFMA (the default; 0 with mla8_opts.f32_scores); ignored elsewhere
    int32_t lo8;
};

// Largest n_new the fused append takes (rows quantized inside the attention
// launch; larger appends use the quantize kernel).
constexpr int kMaxFusedRows = 64;

// One indexer score + top-k call (fp8 indexer keys of kIndexDim bytes per row).
constexpr int kIndexDim = 128;       // indexer head dimension: one K=128 fp8 MFMA
constexpr int kIndexMaxHeads = 64;   // indexer heads, a multiple of 16
constexpr int kIndexMaxTopK = 4096;  // the selection is sorted in LDS
constexpr int kIndexHistBins = 4096; // first radix digit: the key's top 12 bits
constexpr int kIndexHistCopies = 8;  // one histogram per XCD's workgroups (less contention)
constexpr int64_t kIndexMaxRows = int64_t(4096) * 4096;  // selection slices fit LDS tables
struct IndexArgs {
    const uint8_t* k_codes;  // [t_rows][kIndexDim] e4m3
    const float* k_scales;   // [t_rows]
    int32_t t_rows;
    const float* q;          // [n_ih][kIndexDim] f32
    const float* w;          // [n_ih] f32
    int32_t n_ih;
    int32_t top_k;           // < t_rows (t_rows <= top_k selects every row)
    int32_t* sel;            // [min(top_k, t_rows)] ascending row indices
    float* scores;           // [t_rows] or nullptr
    uint32_t* keys;          // workspace [t_rows]: order keys of the scores
    uint64_t* cand;          // workspace [t_rows]: (key, ~row) candidates
    uint32_t* hist;          // workspace [kIndexHistCopies][kIndexHistBins]
    uint32_t* wg_cnt;        // workspace [ceil(t_rows / 4096)]: candidates per slice
    uint32_t* top;           // workspace [kIndexHistCopies][16]: the largest order key of the
                             // scores, one word per copy (64 bytes apart); words 1 and 2: the
                             // k-th key's first-digit bin and the keys in higher bins
};

// ev_before / ev_after (may be null) are recorded around the score kernel.
hipError_t launch_index_topk(const IndexArgs& a, hipStream_t stream, hipEvent_t ev_before,
                             hipEvent_t ev_after);

hipError_t launch_quantize(const float* x, int64_t n_rows, int32_t d, uint8_t* codes,
                           float* scales, hipStream_t stream);
// Mixed rows: lc noPE values -> e4m3 codes + scale, rc RoPE values -> bf16;
// rows[n][lc + 2 rc] bytes.
hipError_t launch_quantize_mx(const float* x, int64_t n_rows, int32_t lc, int32_t rc,
                              uint8_t* rows, float* scales, hipStream_t stream);
hipError_t launch_test_encode(const float* x, int64_t n, uint8_t* codes, hipStream_t stream);
// n a multiple of 4, x 16-byte and codes 4-byte aligned
hipError_t launch_test_encode_pk(const float* x, int64_t n, uint8_t* codes, hipStream_t stream);
constexpr int kStreamWords = 32768;  // output words of the stream-read reference
hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* out, hipStream_t stream);
// The 32x32x16-MFMA partial kernel (mla8_partial32.hip): dense e4m3 rows of
// the Lc = 512, Rc = 64 shape, with or without the fused append.
bool partial32_applies(const AttnArgs& a);
void launch_partial32(const AttnArgs& a, hipStream_t stream);

// ev_before / ev_after (may be null) are recorded around the partial kernel.
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream, hipEvent_t ev_before,
                            hipEvent_t ev_after);

}  // namespace mla8
