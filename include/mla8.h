/*
 * mla8 -- absorbed MLA decode attention over an fp8-e4m3 latent KV cache, for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Sources, cited by page and passage:
 *   [KV8-base]  colibri PR #300 "KV8 long-context CUDA: fp8 device shadow,
 *               split-T kernels, DSA-aware gather", first commit message
 *               ("KV8 base"): the c/kv_fp8.h bullet (RNE encoder saturating at
 *               +/-448, signed zero kept, NaN stored as 0; per-row quantizer
 *               with a subnormal-amax guard) and the attention_rows bullet
 *               (the producer quantizes the fresh row; the latent row is both
 *               key and value; the row scale is hoisted out of the dot).
 *   [KV8-long]  same page, second commit message ("KV8 long-context CUDA") and
 *               the PR description: the kv_dev_sync8 device shadow that only
 *               receives new rows, split-T partial blocks (cl[K], m, z) with a
 *               log-sum-exp merge kernel, the batch path, and the DSA gather
 *               kernel over absolute row indices.
 *   [B1-FMHA]   "B1 Mixed FP8/BF16 FMHA first pass" (nvfp4-megamoe-kernel
 *               docs): a C-ABI launcher under a thin Python bridge that refuses
 *               unsupported shapes loudly instead of falling back.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host].  `stream` is a
 *     hipStream_t passed as void* (NULL = the default stream).
 *   - Calls only enqueue work on `stream` and return; nothing synchronizes.
 *     Buffers must stay alive until the stream work has finished.
 *   - The caller owns every buffer.  The library never allocates device memory:
 *     scratch space comes in through `workspace` (size from
 *     mla8_workspace_bytes).
 *   - All scalar arguments are checked on the host before any HIP call; a
 *     failed check returns a negative status and enqueues nothing.  Device
 *     contents are not inspected.
 *   - Shadow layout ("latent row"): codes[row][Lc + Rc] uint8 e4m3 bytes, the
 *     Lc kv_lora part first, then the Rc rope part; scales[row] float32, one per
 *     row, equal to amax/448 of the f32 row it came from.
 *   - Supported shapes: 16 <= Lc <= 512, 0 <= Rc <= 128, both multiples of 16,
 *     Lc + Rc <= 640.  Other shapes return MLA8_E_UNSUPPORTED.
 *   - Row counts and indices are below 2^31.
 *   - Pointers must be 16-byte aligned (torch allocations are).
 */
#ifndef MLA8_H
#define MLA8_H

#include <stddef.h>
#include <stdint.h>

/* Exported symbols are marked explicitly; the library is built with
 * -fvisibility=hidden. */
#define MLA8_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MLA8_OK = 0,
    MLA8_E_INVAL = -1,       /* NULL pointer, non-positive size, misalignment */
    MLA8_E_RANGE = -2,       /* a row range outside the shadow (batch, decode) */
    MLA8_E_CAPACITY = -3,    /* append beyond cap_rows; *t_rows left unchanged */
    MLA8_E_WORKSPACE = -4,   /* workspace smaller than mla8_workspace_bytes() */
    MLA8_E_UNSUPPORTED = -5, /* shape outside the supported set (see above) */
    MLA8_E_HIP = -6,         /* a HIP launch, copy or device query failed */
    MLA8_E_IO = -7,          /* shadow file: I/O failed or no valid header */
    MLA8_E_SCRATCH = -8      /* beyond the static scratch of mla8_append_decode_noalloc */
};

/* Operation codes for mla8_workspace_bytes. */
enum { MLA8_OP_DECODE = 0, MLA8_OP_DECODE_SEL = 1, MLA8_OP_BATCH = 2, MLA8_OP_INDEX = 3 };

/*
 * Per-call options, the last argument of every attention call, of
 * mla8_index_topk, mla8_workspace_bytes and mla8_plan_splits.  NULL means
 * the defaults (the automatic split plan, no events).  The library keeps no
 * state between calls, so calls on different streams (or threads) with
 * different options never affect each other.
 *   n_splits   0: automatic split plan; > 0: this many row chunks (split-T
 *              partials), clamped to what the row count allows.  The
 *              workspace must then be sized with the same options.
 *   ev_before, ev_after: hipEvent_t (as void*) recorded on the call's stream
 *              just before and just after the split-T partial kernel (the
 *              indexer's score kernel for mla8_index_topk), so that
 *              hipEventElapsedTime(ev_before, ev_after) is that kernel's
 *              duration; NULL to skip.  Caller-owned.
 *   f32_scores 0 (default): for e4m3 rows with lc = 512, rc = 64 (dense
 *              mla8_decode, mla8_append_decode, mla8_append_decode_noalloc
 *              over at least 64 rows; mla8_decode_sel over at least 64 list
 *              entries; mla8_batch with n_heads a multiple of 32 and pos0 >=
 *              63) the scores use the e4m3 MFMA for the
 *              query's lo term [B1-FMHA first pass, intentional limits: the
 *              noPE QK product on the fp8 tensor cores]: per head, e = q *
 *              sm_scale * log2(e) is scaled by 2^k (largest |e| in [2^14,
 *              2^15)), split into its fp16 rounding hi and the rest lo
 *              (rounded to fp16), and lo is quantized to e4m3 with a
 *              power-of-2 scale 2^j (largest |lo| 2^j in [128, 256)); the
 *              result is attention with the query (hi + e4m3(lo 2^j) 2^-j)
 *              2^-k / (sm_scale log2(e)) in place of q, which differs from q
 *              by about 2^-16 of its largest entry per head.  Mixed rows
 *              (lc = 448, rc = 64; the *_mx calls under the same conditions):
 *              the same for the noPE part, its 2^k and 2^j taken over the noPE
 *              part alone; the RoPE part as the two bf16 terms hi =
 *              bf16(q_rope sm_scale log2(e)), lo = bf16(that - hi), i.e. the
 *              query (hi + lo) / (sm_scale log2(e)) in place of q_rope.  Every
 *              other call attends with q as given, scores of f32 grade.  1:
 *              scores of f32 grade for those calls too (fp16 hi + lo terms on
 *              the fp16 MFMA, slower).
 */
typedef struct mla8_opts {
    int32_t n_splits;
    void* ev_before;
    void* ev_after;
    int32_t f32_scores;
} mla8_opts;

/*
 * Quantize n_rows f32 rows x[n_rows][lc + rc] into e4m3 codes[n_rows][lc + rc]
 * and f32 scales[n_rows]  [KV8-base, c/kv_fp8.h bullet]:
 *   amax  = max |x_i| over the row's finite entries (NaN and +/-inf excluded);
 *   scale = f32(amax / 448)            -- stored;
 *   inv   = f32(448 / amax), or 0 when that is not finite (the guard: amax = 0
 *           or so small that 448/amax overflows);
 *   code_i = enc(f32(x_i * inv)), enc = round-to-nearest-even onto OCP e4m3
 *           (E4M3FN), saturating to +/-448 (0x7E/0xFE), sign of zero kept,
 *           NaN -> 0x00.
 * Bytes and scales are bit-exact with that definition.  n_rows == 0 is a no-op.
 * Errors: E_INVAL (NULL pointer, n_rows < 0), E_UNSUPPORTED (shape), E_HIP.
 */
MLA8_API int mla8_quantize_rows(const float* x, int64_t n_rows, int32_t lc, int32_t rc, uint8_t* codes,
                       float* scales, void* stream);

/*
 * Quantize n_rows fresh f32 rows into the device-resident shadow at rows
 * [*t_rows, *t_rows + n_rows), then advance *t_rows by n_rows
 * [KV8-base, attention_rows bullet: the producer quantizes the fresh row;
 *  KV8-long, kv_dev_sync8 bullet: the shadow only receives the new rows].
 * kv_codes[cap_rows][lc + rc] and kv_scales[cap_rows] are caller-owned.
 * t_rows is a [host] pointer.  Same arithmetic as mla8_quantize_rows.
 * Errors: E_INVAL, E_UNSUPPORTED, E_CAPACITY (*t_rows + n_rows > cap_rows;
 * nothing enqueued, *t_rows unchanged), E_HIP (*t_rows unchanged).
 */
MLA8_API int mla8_append(uint8_t* kv_codes, float* kv_scales, int64_t cap_rows, int64_t* t_rows,
                const float* x, int64_t n_rows, int32_t lc, int32_t rc, void* stream);

/*
 * Dense absorbed decode of n_heads query heads over shadow rows [0, t_rows)
 * [KV8-long, split-T bullet; KV8-base, attention_rows bullet].  Per head h with
 * q = q_lat[h] || q_rope[h] and k_t = dec(codes[t]) * scales[t]:
 *   s_t = sm_scale * (q . k_t);  p = softmax_t(s)  (natural exponential);
 *   out[h][k] = sum_t p_t k_t[k]  for k < lc;  lse[h] = ln sum_t e^{s_t}.
 * Computed split-T: row chunks yield (m, z, cl[lc]) partials in `workspace`,
 * then a log-sum-exp merge writes out.  With lc = 512, rc = 64 and t_rows >=
 * 64, q is the e4m3-lo-term query that mla8_opts.f32_scores describes unless
 * that option is set.
 *   q_lat[n_heads][lc], q_rope[n_heads][rc]: f32.  out[n_heads][lc]: f32.
 *   lse[n_heads]: f32, or NULL to skip.
 * Errors: E_INVAL (NULL, t_rows <= 0, n_heads <= 0, non-finite sm_scale),
 * E_UNSUPPORTED, E_WORKSPACE (ws_bytes < mla8_workspace_bytes(MLA8_OP_DECODE,
 * t_rows, n_heads, 1, lc)), E_HIP.
 */
MLA8_API int mla8_decode(const uint8_t* kv_codes, const float* kv_scales, int64_t t_rows, int32_t lc,
                int32_t rc, const float* q_lat, const float* q_rope, int32_t n_heads,
                float sm_scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                void* stream, const mla8_opts* opts);

/*
 * Append then decode in one launch: the same result as mla8_append(x_new,
 * n_new rows) followed by mla8_decode over the new *t_rows rows, with the
 * fresh rows quantized inside the attention launch by the workgroups whose
 * row chunk holds them [KV8-base, attention_rows bullet: the producer
 * quantizes the fresh row; KV8-long, kv_dev_sync8 and split-T bullets].
 * kv_codes[cap_rows][lc + rc] and kv_scales[cap_rows] receive rows
 * [*t_rows, *t_rows + n_new) exactly as mla8_append writes them; t_rows is a
 * [host] pointer advanced by n_new on success.  1 <= n_new <= 64.
 * Errors: E_INVAL (NULL, n_new <= 0, *t_rows outside [0, cap_rows], and the
 * mla8_decode checks on the new row count), E_RANGE (n_new > 64),
 * E_CAPACITY (*t_rows + n_new > cap_rows), E_UNSUPPORTED, E_WORKSPACE
 * (workspace from mla8_workspace_bytes(MLA8_OP_DECODE, *t_rows + n_new,
 * n_heads, 1, lc)), E_HIP.  On any error nothing is enqueued and *t_rows is
 * unchanged.
 */
MLA8_API int mla8_append_decode(uint8_t* kv_codes, float* kv_scales, int64_t cap_rows,
                       int64_t* t_rows, const float* x_new, int64_t n_new, int32_t lc,
                       int32_t rc, const float* q_lat, const float* q_rope, int32_t n_heads,
                       float sm_scale, float* out, float* lse, void* workspace,
                       size_t ws_bytes, void* stream, const mla8_opts* opts);

/*
 * mla8_append_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, result and *t_rows update as
 * mla8_append_decode, without `workspace`: the split-T partials live in the
 * library's own static device array of MLA8_SCRATCH_BYTES, one copy per GPU,
 * held until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine); it uses the scratch of the current device, so
 * `stream` must belong to that device.  The automatic plan fits for any
 * head count up to 8192 with lc <= 512 (its partials take at most about
 * 16.8 MB); a call needing more (mla8_workspace_bytes(MLA8_OP_DECODE, *t_rows + n_new,
 * n_heads, 1, lc, opts) > MLA8_SCRATCH_BYTES, e.g. with many forced splits)
 * returns MLA8_E_SCRATCH before any HIP call.  Calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (two streams, two threads)
 * race; the scratch needs no clearing between calls.
 * Errors: those of mla8_append_decode except E_WORKSPACE, plus E_SCRATCH.
 */
#define MLA8_SCRATCH_BYTES (20u << 20)
MLA8_API int mla8_append_decode_noalloc(uint8_t* kv_codes, float* kv_scales, int64_t cap_rows,
                                        int64_t* t_rows, const float* x_new, int64_t n_new,
                                        int32_t lc, int32_t rc, const float* q_lat,
                                        const float* q_rope, int32_t n_heads, float sm_scale,
                                        float* out, float* lse, void* stream,
                                        const mla8_opts* opts);

/*
 * Selected-row (DSA gather) decode [KV8-long, DSA bullet]: as mla8_decode, but
 * each head attends only the rows listed in sel[0..ns), absolute indices into
 * the shadow read straight from it.  sel is a multiset (repeats count as often
 * as they appear); entries outside [0, t_rows) are skipped.  If no entry is in
 * range, out is all zeros and lse is -inf.  No cap on ns beyond 2^31.  For
 * lc = 512, rc = 64 and ns >= 64, q is the e4m3-lo-term query that
 * mla8_opts.f32_scores describes unless that option is set.
 * Errors: as mla8_decode, plus E_INVAL for ns <= 0; workspace from
 * mla8_workspace_bytes(MLA8_OP_DECODE_SEL, ns, n_heads, 1, lc).
 */
MLA8_API int mla8_decode_sel(const uint8_t* kv_codes, const float* kv_scales, int64_t t_rows, int32_t lc,
                    int32_t rc, const int32_t* sel, int64_t ns, const float* q_lat,
                    const float* q_rope, int32_t n_heads, float sm_scale, float* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream, const mla8_opts* opts);

/*
 * Batched causal attention [KV8-long: the batch/prefill path over the cached
 * rows, one (query, head) pair per work unit]: query s in [0, n_q) sits at
 * absolute position pos0 + s and attends rows [0, pos0 + s] (its own row
 * included), with the same per-head arithmetic as mla8_decode (for lc = 512,
 * rc = 64, n_heads a multiple of 32 and pos0 >= 63, q is the e4m3-lo-term
 * query that mla8_opts.f32_scores describes unless that option is set).
 *   q_lat[n_q][n_heads][lc], q_rope[n_q][n_heads][rc]: f32.
 *   out[n_q][n_heads][lc]: f32.  lse[n_q][n_heads] or NULL.
 * Errors: E_INVAL (NULL, n_q <= 0, pos0 < 0, ...), E_RANGE (pos0 + n_q >
 * t_rows), E_UNSUPPORTED, E_WORKSPACE (see mla8_workspace_bytes(MLA8_OP_BATCH,
 * pos0 + n_q, n_heads, n_q, lc)), E_HIP.
 */
MLA8_API int mla8_batch(const uint8_t* kv_codes, const float* kv_scales, int64_t t_rows, int32_t lc,
               int32_t rc, const float* q_lat, const float* q_rope, int32_t n_q, int64_t pos0,
               int32_t n_heads, float sm_scale, float* out, float* lse, void* workspace,
               size_t ws_bytes, void* stream, const mla8_opts* opts);

/*
 * Mixed row layout  [B1-FMHA, the storage-format list: noPE KV as e4m3 bytes
 * with a per-row f32 scale, RoPE KV kept in bf16; the decode kernel is for the
 * 512 / 448 / 64 shape].  A stored row holds the lc = 448 noPE values as e4m3
 * codes (quantized exactly as mla8_quantize_rows does, over the noPE part
 * alone: scale = its amax/448) followed by the rc = 64 RoPE values as
 * little-endian bf16 (round to nearest even; a NaN becomes 0x7FC0 with its
 * sign): rows[row][lc + 2 rc] bytes, scales[row] f32.  In attention the key is
 * the dequantized noPE part followed by the bf16 RoPE values (the row scale
 * does not apply to them) and the value is the dequantized noPE part, so out is
 * [H][lc].  Only lc = 448, rc = 64 is supported (E_UNSUPPORTED otherwise).
 */
MLA8_API int mla8_quantize_rows_mx(const float* x, int64_t n_rows, int32_t lc, int32_t rc,
                                   uint8_t* rows, float* scales, void* stream);
/* As mla8_append, for mixed rows (kv_rows [cap_rows][lc + 2 rc]). */
MLA8_API int mla8_append_mx(uint8_t* kv_rows, float* kv_scales, int64_t cap_rows, int64_t* t_rows,
                            const float* x, int64_t n_rows, int32_t lc, int32_t rc, void* stream);
/* As mla8_decode, over mixed rows; workspace from
 * mla8_workspace_bytes(MLA8_OP_DECODE, t_rows, n_heads, 1, lc). */
MLA8_API int mla8_decode_mx(const uint8_t* kv_rows, const float* kv_scales, int64_t t_rows,
                            int32_t lc, int32_t rc, const float* q_lat, const float* q_rope,
                            int32_t n_heads, float sm_scale, float* out, float* lse,
                            void* workspace, size_t ws_bytes, void* stream, const mla8_opts* opts);
/* As mla8_decode_sel (absolute row indices, a multiset, entries outside
 * [0, t_rows) skipped), over mixed rows; workspace from
 * mla8_workspace_bytes(MLA8_OP_DECODE_SEL, ns, n_heads, 1, lc). */
MLA8_API int mla8_decode_sel_mx(const uint8_t* kv_rows, const float* kv_scales, int64_t t_rows,
                                int32_t lc, int32_t rc, const int32_t* sel, int64_t ns,
                                const float* q_lat, const float* q_rope, int32_t n_heads,
                                float sm_scale, float* out, float* lse, void* workspace,
                                size_t ws_bytes, void* stream, const mla8_opts* opts);
/* As mla8_append_decode over mixed rows: the n_new (1..64) fresh f32 rows x_new
 * [n_new][lc + rc] (16-byte aligned) are stored at rows [*t_rows, *t_rows +
 * n_new) in the mla8_quantize_rows_mx format by the same launch that attends
 * the t_rows + n_new rows; *t_rows advances on success only.  Workspace from
 * mla8_workspace_bytes(MLA8_OP_DECODE, *t_rows + n_new, n_heads, 1, lc).
 * Errors as mla8_append_decode (E_RANGE for n_new > 64, E_CAPACITY beyond
 * cap_rows), E_UNSUPPORTED for a shape other than 448 / 64. */
MLA8_API int mla8_append_decode_mx(uint8_t* kv_rows, float* kv_scales, int64_t cap_rows,
                                   int64_t* t_rows, const float* x_new, int64_t n_new, int32_t lc,
                                   int32_t rc, const float* q_lat, const float* q_rope,
                                   int32_t n_heads, float sm_scale, float* out, float* lse,
                                   void* workspace, size_t ws_bytes, void* stream, const mla8_opts* opts);
/* As mla8_batch (query s at position pos0 + s attends rows 0 .. pos0 + s;
 * q_lat [n_q][n_heads][lc], q_rope [n_q][n_heads][rc]; out [n_q][n_heads][lc],
 * lse [n_q][n_heads]) over mixed rows; workspace from
 * mla8_workspace_bytes(MLA8_OP_BATCH, pos0 + n_q, n_heads, n_q, lc). */
MLA8_API int mla8_batch_mx(const uint8_t* kv_rows, const float* kv_scales, int64_t t_rows,
                           int32_t lc, int32_t rc, const float* q_lat, const float* q_rope,
                           int32_t n_q, int64_t pos0, int32_t n_heads, float sm_scale, float* out,
                           float* lse, void* workspace, size_t ws_bytes, void* stream, const mla8_opts* opts);

/*
 * fp8 indexer score + top-k: the selection that mla8_decode_sel attends.
 * Source: "B1 Mixed FP8/BF16 FMHA first pass" site, commit message of the B2
 * fp8 indexer score + top-k kernel: the indexer query is quantized to fp8, the
 * keys are read as e4m3, each head's dot product is dequantized by
 * q_scale * k_scale and passed through ReLU, the heads are summed with per-head
 * weights and the top-k rows are kept.  For one query token:
 *     I_t = sum_j w[j] * max(0, q_scale_j * k_scales[t] * sum_d q8[j][d] k_codes[t][d])
 * where q8[j] / q_scale_j is row j of q quantized with the shadow's row
 * quantizer (the same arithmetic as mla8_quantize_rows).
 *   k_codes  [t_rows][ihd] e4m3 keys, k_scales [t_rows] f32: rows of the shadow
 *            format with lc = ihd, rc = 0 (mla8_quantize_rows(x, n, ihd, 0, ...)).
 *   q        [n_ih][ihd] f32 indexer query (16-byte aligned); w [n_ih] f32 weights.
 *   sel      [min(top_k, t_rows)] int32 out: the rows with the top_k largest
 *            I_t, a tie going to the smaller row, a NaN score below all others
 *            and -0 equal to +0; written in ascending row order.  t_rows <= top_k
 *            selects every row.
 *   scores   [t_rows] f32 out (I_t in f32), or NULL.
 * Supported: ihd = 128, n_ih in {16, 32, 48, 64}, 1 <= top_k <= 4096,
 * t_rows <= 2^24.
 * workspace: mla8_workspace_bytes(MLA8_OP_INDEX, t_rows, n_ih, 1, ihd) bytes,
 * 16-byte aligned; its contents on entry do not matter.
 * Errors: E_INVAL (NULL pointer, t_rows or top_k < 1, misalignment),
 * E_UNSUPPORTED (ihd, n_ih or top_k outside the supported set), E_WORKSPACE,
 * E_HIP.  Calls that overlap on one workspace race.
 */
MLA8_API int mla8_index_topk(const uint8_t* k_codes, const float* k_scales, int64_t t_rows,
                             int32_t ihd, const float* q, const float* w, int32_t n_ih,
                             int32_t top_k, int32_t* sel, float* scores, void* workspace,
                             size_t ws_bytes, void* stream, const mla8_opts* opts);

/*
 * Workspace bytes the given call needs.  `rows` is the number of rows the
 * call attends: t_rows for MLA8_OP_DECODE, ns for MLA8_OP_DECODE_SEL,
 * pos0 + n_q for MLA8_OP_BATCH, t_rows for MLA8_OP_INDEX (whose n_heads is
 * n_ih and lc is ihd).  n_q is ignored except for MLA8_OP_BATCH.  opts: the
 * options the call will be made with (NULL = defaults); the split count
 * changes the size.  Returns 0 for invalid arguments.
 */
MLA8_API size_t mla8_workspace_bytes(int32_t op, int64_t rows, int32_t n_heads, int32_t n_q, int32_t lc, const mla8_opts* opts);

/* Number of row chunks (split-T partials) the plan for a call uses: the
 * automatic plan, or opts->n_splits clamped to what the row count allows.
 * Arguments as mla8_workspace_bytes; returns 0 for invalid arguments. */
MLA8_API int32_t mla8_plan_splits(int32_t op, int64_t rows, int32_t n_heads, int32_t n_q,
                                  const mla8_opts* opts);

/*
 * Persistent shadow files  [KV8-base, the .coli_kv v2 bullet: a versioned file
 * whose header names the row type, appended through a persistent handle and a
 * staging buffer, holding fp8 rows plus scales; files of the previous version
 * hold f32 rows, are quantized when a session resumes and stay untouched on
 * disk until the first append rewrites them in the new version].
 * These calls do host file I/O and SYNCHRONIZE `stream` (the one exception to
 * the enqueue-only rule); they are not for the decode loop's critical path.
 *
 * Format (little-endian): two 64-byte header slots, then the body from byte
 * 128, token-major.  Slot: "MLA8KV\0\0", u32 version (1 = f32 rows, 2 = e4m3
 * rows + f32 scale), u32 n_layers, u32 lc, u32 rc, u64 n_tokens (committed),
 * u64 seq, u32 FNV-1a of the 40 bytes before it, zero padding.  The valid
 * slot with the larger seq is the committed state.  Version-2 token t, at
 * 128 + t * n_layers * (D + 4): per layer, D = lc + rc code bytes then the
 * scale.  Version-1 token: per layer, D f32 values.
 * Crash safety: an append writes and flushes the new tokens past the committed
 * end, then writes and flushes the other header slot; a crash leaves the
 * previous commit readable.
 *
 * kv_codes / kv_scales are [host] arrays of n_layers pointers to each layer's
 * shadow (codes[cap][lc + rc], scales[cap]); the shadows are device memory
 * when on_device != 0, host memory otherwise.
 */

/* A new empty version-2 file (truncates an existing one).
 * Errors: E_INVAL (NULL path, n_layers < 1), E_UNSUPPORTED (shape), E_IO. */
MLA8_API int mla8_kvfile_create(const char* path, int32_t n_layers, int32_t lc, int32_t rc);

/* [host] outputs: the committed header.  Errors: E_INVAL, E_IO. */
MLA8_API int mla8_kvfile_info(const char* path, int32_t* version, int32_t* n_layers, int32_t* lc,
                              int32_t* rc, int64_t* n_tokens);

/* Append shadow rows [t0, t0 + n_tok) of every layer as tokens t0 .. of the
 * file; t0 must equal the file's committed n_tokens.  A version-1 file is
 * first rewritten as version 2 from shadow rows [0, t0 + n_tok) (the shadows
 * hold its rows quantized by mla8_kvfile_load) into `path`.v2tmp, which then
 * replaces `path`.  n_tok = 0 is a no-op.
 * Errors: E_INVAL (NULL pointer, negative t0 / n_tok, a file of another
 * n_layers / lc / rc), E_UNSUPPORTED (shape), E_RANGE (t0 != committed
 * n_tokens), E_HIP (device copy), E_IO. */
MLA8_API int mla8_kvfile_append(const char* path, int32_t n_layers, const uint8_t* const* kv_codes,
                                const float* const* kv_scales, int64_t t0, int64_t n_tok,
                                int32_t lc, int32_t rc, int32_t on_device, void* stream);

/* Load the committed tokens into shadow rows [0, n_tokens) of every layer and
 * set *t_rows [host] = n_tokens.  Version-2 rows are copied as they are.
 * Version-1 (f32) rows are quantized on the device exactly as
 * mla8_quantize_rows does, through `workspace` (device, 16-byte aligned, at
 * least (lc + rc) * 4 bytes; more bytes convert more rows per round trip);
 * the file itself is not changed.  Errors: E_INVAL (NULL pointer, cap_rows < 1,
 * a file of another n_layers / lc / rc), E_UNSUPPORTED (shape; a version-1
 * file into host shadows), E_CAPACITY (n_tokens > cap_rows, nothing loaded),
 * E_WORKSPACE (version 1 without a large enough workspace), E_HIP, E_IO (no
 * usable header slot, or a version-2 row that the quantizer cannot have
 * written: a NaN code 0x7F / 0xFF, or a negative or non-finite scale; the
 * rows before it may then already be in the shadows, *t_rows is unchanged).
 * A header slot is usable when its check matches, its token count is below
 * 2^31 and the body holds all of its tokens; of two usable slots the larger
 * seq wins. */
MLA8_API int mla8_kvfile_load(const char* path, int32_t n_layers, uint8_t* const* kv_codes,
                              float* const* kv_scales, int64_t cap_rows, int64_t* t_rows,
                              int32_t lc, int32_t rc, int32_t on_device, void* workspace,
                              size_t ws_bytes, void* stream);

/* Human-readable text for a status code (static storage). */
MLA8_API const char* mla8_status_string(int status);

/* Library version string (static storage). */
MLA8_API const char* mla8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA8_H */
