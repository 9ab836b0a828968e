// C-ABI entry points of libmla8 (declared in include/mla8.h): argument checks,
// split planning, workspace carving and kernel launches.  Every check runs on
// the host before any HIP call, so the error paths work without a GPU.
#include "mla8.h"
#include "mla8_aux.h"
#include "mla8_internal.h"

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

// Scratch of mla8_append_decode_noalloc, for callers that cannot allocate: the
// split-T partials go to this file-scope device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): its device address comes from
// hipGetSymbolAddress, once per device.
static constexpr size_t kScratchBytes = size_t(20) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

using namespace mla8;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int32_t lc, int32_t rc)
{
    if (lc < 16 || lc > 512 || (lc % 16) != 0)
        return MLA8_E_UNSUPPORTED;
    if (rc < 0 || rc > 128 || (rc % 16) != 0)
        return MLA8_E_UNSUPPORTED;
    if (lc + rc > 640)
        return MLA8_E_UNSUPPORTED;
    return MLA8_OK;
}

struct Plan {
    int32_t n_chunks;
    int32_t chunk_rows;
    int32_t n_groups;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t forced_splits(const mla8_opts* o) { return (o != nullptr && o->n_splits > 0) ? o->n_splits : 0; }
hipEvent_t ev_before(const mla8_opts* o) { return o ? static_cast<hipEvent_t>(o->ev_before) : nullptr; }
hipEvent_t ev_after(const mla8_opts* o) { return o ? static_cast<hipEvent_t>(o->ev_after) : nullptr; }
int32_t lo8_scores(const mla8_opts* o) { return (o != nullptr && o->f32_scores != 0) ? 0 : 1; }

// Row chunks for a call that attends `rows` rows with `n_qh` query-heads.
// Aim for one workgroup per CU; prefer a multiple of 8 chunks (one per XCD
// round); keep chunks at least 128 rows (64 for a gather), so that the partial
// (m, z, cl) traffic stays small next to the rows it summarises (measured at
// T = 4096 with 128 heads: 2 tiles per chunk 20.8 us per layer-token, 4
// tiles 22.1, 1 tile 22.4).
// forced > 0: that many chunks (clamped below), the caller's per-call option.
Plan make_plan(int32_t op, int64_t rows, int32_t n_qh, int32_t forced)
{
    Plan p;
    p.n_groups = (int32_t)cdiv(n_qh, kHeadsPerGroup);
    int64_t P;
    if (forced > 0) {
        P = forced;
    } else {
        P = kTargetGroups / p.n_groups;
        if (P < 1)
            P = 1;
        if (P >= 8)
            P &= ~int64_t(7);
        const int64_t min_rows = (op == MLA8_OP_DECODE_SEL) ? kTileRows : 2 * kTileRows;
        const int64_t cap = cdiv(rows, min_rows);
        if (P > cap)
            P = cap;
    }
    const int64_t max_p = cdiv(rows, kTileRows);
    if (P > max_p)
        P = max_p;
    if (P < 1)
        P = 1;
    int64_t chunk = cdiv(cdiv(rows, P), kTileRows) * kTileRows;
    p.chunk_rows = (int32_t)chunk;
    p.n_chunks = (int32_t)cdiv(rows, chunk);
    return p;
}

size_t ws_bytes_for(const Plan& p, int32_t n_qh, int32_t lc)
{
    // m, z and cl, each section rounded up to 256 bytes
    auto r256 = [](size_t b) { return (b + 255) & ~size_t(255); };
    const size_t mz = (size_t)p.n_chunks * (size_t)n_qh * sizeof(float);
    const size_t cl = mz * (size_t)lc;
    return 2 * r256(mz) + r256(cl);
}

int run_attention(int32_t op, const uint8_t* codes, const float* scales, int64_t t_rows,
                  int32_t lc, int32_t rc, const int32_t* sel, int64_t n_list, const float* q_lat,
                  const float* q_rope, int32_t n_qh, int32_t n_heads, int64_t pos0,
                  float sm_scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                  void* stream, const mla8_opts* opts, const float* x_new = nullptr,
                  uint8_t* new_codes = nullptr, float* new_scales = nullptr, int64_t new0 = 0,
                  int64_t n_new = 0, int32_t layout = kE4m3)
{
    const Plan p = make_plan(op, n_list, n_qh, forced_splits(opts));
    const size_t need = ws_bytes_for(p, n_qh, lc);
    if (workspace == nullptr || ws_bytes < need)
        return MLA8_E_WORKSPACE;
    if (!aligned16(workspace))
        return MLA8_E_INVAL;
    auto r256 = [](size_t b) { return (b + 255) & ~size_t(255); };
    const size_t mz = (size_t)p.n_chunks * (size_t)n_qh * sizeof(float);
    char* ws = static_cast<char*>(workspace);

    AttnArgs a;
    a.codes = codes;
    a.scales = scales;
    a.t_rows = (int32_t)t_rows;
    a.sel = sel;
    a.n_list = (int32_t)n_list;
    a.q_lat = q_lat;
    a.q_rope = q_rope;
    a.lc = lc;
    a.rc = rc;
    a.d = (layout == kMixed) ? lc + 2 * rc : lc + rc;
    a.layout = layout;
    a.n_qh = n_qh;
    a.n_heads = n_heads;
    a.pos0 = (int32_t)pos0;
    a.mode = op == MLA8_OP_DECODE_SEL ? kSelect : (op == MLA8_OP_BATCH ? kCausal : kDense);
    a.sm_log2 = sm_scale * 1.4426950408889634f;
    a.n_chunks = p.n_chunks;
    a.chunk_rows = p.chunk_rows;
    a.n_groups = p.n_groups;
    a.ws_m = reinterpret_cast<float*>(ws);
    a.ws_z = reinterpret_cast<float*>(ws + r256(mz));
    a.ws_cl = reinterpret_cast<float*>(ws + 2 * r256(mz));
    a.out = out;
    a.lse = lse;
    a.x_new = x_new;
    a.new_codes = new_codes;
    a.new_scales = new_scales;
    a.new0 = (int32_t)new0;
    a.n_new = (int32_t)n_new;
    a.lo8 = lo8_scores(opts);
    return launch_attention(a, static_cast<hipStream_t>(stream), ev_before(opts), ev_after(opts)) ==
                   hipSuccess
               ? MLA8_OK
               : MLA8_E_HIP;
}

constexpr int64_t kMaxRows = 0x7FFFFFFF;

// Indexer workspace: keys u32 [t], candidates u64 [t], the first-digit
// histogram copies, the per-slice candidate counts and the largest-key words,
// each section 256-byte aligned.
size_t r256(size_t b) { return (b + 255) & ~size_t(255); }
size_t index_ws_bytes(int64_t t)
{
    return r256((size_t)t * 4) + r256((size_t)t * 8) + r256(kIndexHistCopies * kIndexHistBins * 4) +
           r256((size_t)((t + 4095) / 4096) * 4) + r256(kIndexHistCopies * 64);
}

}  // namespace

extern "C" {

int mla8_quantize_rows(const float* x, int64_t n_rows, int32_t lc, int32_t rc, uint8_t* codes,
                       float* scales, void* stream)
{
    int st = check_shape(lc, rc);
    if (st != MLA8_OK)
        return st;
    if (n_rows < 0 || n_rows > kMaxRows)
        return MLA8_E_INVAL;
    if (n_rows == 0)
        return MLA8_OK;
    if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes) ||
        (reinterpret_cast<uintptr_t>(scales) & 3u))
        return MLA8_E_INVAL;
    return launch_quantize(x, n_rows, lc + rc, codes, scales, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? MLA8_OK
               : MLA8_E_HIP;
}

int mla8_append(uint8_t* kv_codes, float* kv_scales, int64_t cap_rows, int64_t* t_rows,
                const float* x, int64_t n_rows, int32_t lc, int32_t rc, void* stream)
{
    int st = check_shape(lc, rc);
    if (st != MLA8_OK)
        return st;
    if (!kv_codes || !kv_scales || !t_rows || !x)
        return MLA8_E_INVAL;
    if (cap_rows <= 0 || cap_rows > kMaxRows || n_rows < 0 || *t_rows < 0 || *t_rows > cap_rows)
        return MLA8_E_INVAL;
    if (!aligned16(kv_codes) || !aligned16(x) || (reinterpret_cast<uintptr_t>(kv_scales) & 3u))
        return MLA8_E_INVAL;
    if (n_rows > cap_rows - *t_rows)
        return MLA8_E_CAPACITY;
    if (n_rows == 0)
        return MLA8_OK;
    const int64_t d = lc + rc;
    const hipError_t e = launch_quantize(x, n_rows, (int32_t)d, kv_codes + *t_rows * d,
                                         kv_scales + *t_rows, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return MLA8_E_HIP;
    *t_rows += n_rows;
    return MLA8_OK;
}

static int check_decode_common(const uint8_t* codes, const float* scales, int64_t t_rows,
                               int32_t lc, int32_t rc, const float* q_lat, const float* q_rope,
                               int32_t n_heads, float sm_scale, const float* out)
{
    int st = check_shape(lc, rc);
    if (st != MLA8_OK)
        return st;
    if (!codes || !scales || !q_lat || !out || (rc > 0 && !q_rope))
        return MLA8_E_INVAL;
    if (t_rows <= 0 || t_rows > kMaxRows || n_heads <= 0 || !isfinite(sm_scale))
        return MLA8_E_INVAL;
    if (!aligned16(codes) || !aligned16(q_lat) || (rc > 0 && !aligned16(q_rope)) ||
        !aligned16(out) || (reinterpret_cast<uintptr_t>(scales) & 3u))
        return MLA8_E_INVAL;
    return MLA8_OK;
}

int mla8_decode(const uint8_t* kv_codes, const float* kv_scales, int64_t t_rows, int32_t lc,
                int32_t rc, const float* q_lat, const float* q_rope, int32_t n_heads,
                float sm_scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                void* stream, const mla8_opts* opts)
{
    int st = check_decode_common(kv_codes, kv_scales, t_rows, lc, rc, q_lat, q_rope, n_heads,
                                 sm_scale, out);
    if (st != MLA8_OK)
        return st;
    return run_attention(MLA8_OP_DECODE, kv_codes, kv_scales, t_rows, lc, rc, nullptr, t_rows,
                         q_lat, q_rope, n_heads, n_heads, 0, sm_scale, out, lse, workspace,
                         ws_bytes, stream, opts);
}

// Mixed rows: the 448 / 64 shape only.
int check_shape_mx(int32_t lc, int32_t rc)
{
    return (lc == 448 && rc == 64) ? MLA8_OK : MLA8_E_UNSUPPORTED;
}

int mla8_quantize_rows_mx(const float* x, int64_t n_rows, int32_t lc, int32_t rc, uint8_t* rows,
                          float* scales, void* stream)
{
    int st = check_shape_mx(lc, rc);
    if (st != MLA8_OK)
        return st;
    if (n_rows < 0 || n_rows > kMaxRows)
        return MLA8_E_INVAL;
    if (n_rows == 0)
        return MLA8_OK;
    if (!x || !rows || !scales || !aligned16(x) || !aligned16(rows) ||
        (reinterpret_cast<uintptr_t>(scales) & 3u))
        return MLA8_E_INVAL;
    return launch_quantize_mx(x, n_rows, lc, rc, rows, scales, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? MLA8_OK
               : MLA8_E_HIP;
}

int mla8_append_mx(uint8_t* kv_rows, float* kv_scales, int64_t cap_rows, int64_t* t_rows,
                   const float* x, int64_t n_rows, int32_t lc, int32_t rc, void* stream)
{
    int st = check_shape_mx(lc, rc);
    if (st != MLA8_OK)
        return st;
    if (!kv_rows || !kv_scales || !t_rows || !x)
        return MLA8_E_INVAL;
    if (cap_rows <= 0 || cap_rows > kMaxRows || n_rows < 0 || *t_rows < 0 || *t_rows > cap_rows)
        return MLA8_E_INVAL;
    if (!aligned16(kv_rows) || !aligned16(x) || (reinterpret_cast<uintptr_t>(kv_scales) & 3u))
        return MLA8_E_INVAL;
    if (n_rows > cap_rows - *t_rows)
        return MLA8_E_CAPACITY;
    if (n_rows == 0)
        return MLA8_OK;
    const int64_t rb = lc + 2 * (int64_t)rc;
    const hipError_t e = launch_quantize_mx(x, n_rows, lc, rc, kv_rows + *t_rows * rb,
                                            kv_scales + *t_rows, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return MLA8_E_HIP;
    *t_rows += n_rows;
    return MLA8_OK;
}

int mla8_decode_mx(const uint8_t* kv_rows, const float* kv_scales, int64_t t_rows, int32_t lc,
                   int32_t rc, const float* q_lat, const float* q_rope, int32_t n_heads,
                   float sm_scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                   void* stream, const mla8_opts* opts)
{
    int st = check_shape_mx(lc, rc);
    if (st != MLA8_OK)
        return st;
    st = check_decode_common(kv_rows, kv_scales, t_rows, lc, rc, q_lat, q_rope, n_heads, sm_scale,
                             out);
    if (st != MLA8_OK)
        return st;
    return run_attention(MLA8_OP_DECODE, kv_rows, kv_scales, t_rows, lc, rc, nullptr, t_rows,
                         q_lat, q_rope, n_heads, n_heads, 0, sm_scale, out, lse, workspace,
                         ws_bytes, stream, opts, nullptr, nullptr, nullptr, 0, 0, kMixed);
}

int mla8_decode_sel_mx(const uint8_t* kv_rows, const float* kv_scales, int64_t t_rows,
                       int32_t lc, int32_t rc, const int32_t* sel, int64_t ns,
                       const float* q_lat, const float* q_rope, int32_t n_heads, float sm_scale,
                       float* out, float* lse, void* workspace, size_t ws_bytes, void* stream,
                       const mla8_opts* opts)
{
    int st = check_shape_mx(lc, rc);
    if (st != MLA8_OK)
        return st;
    st = check_decode_common(kv_rows, kv_scales, t_rows, lc, rc, q_lat, q_rope, n_heads, sm_scale,
                             out);
    if (st != MLA8_OK)
        return st;
    if (!sel || ns <= 0 || ns > kMaxRows || (reinterpret_cast<uintptr_t>(sel) & 3u))
        return MLA8_E_INVAL;
    return run_attention(MLA8_OP_DECODE_SEL, kv_rows, kv_scales, t_rows, lc, rc, sel, ns, q_lat,
                         q_rope, n_heads, n_heads, 0, sm_scale, out, lse, workspace, ws_bytes,
                         stream, opts, nullptr, nullptr, nullptr, 0, 0, kMixed);
}

// The fused step and the causal batch over mixed rows: the e4m3 entry
// points' checks with the mixed shape; the kernels are the mixed instances.
// Host checks of the fused append + decode step (no HIP call).
static int append_decode_check(const uint8_t* kv, const float* kv_scales, int64_t cap_rows,
                               const int64_t* t_rows, const float* x_new, int64_t n_new,
                               int32_t lc, int32_t rc, const float* q_lat, const float* q_rope,
                               int32_t n_heads, float sm_scale, const float* out)
{
    if (!kv || !kv_scales || !t_rows || !x_new)
        return MLA8_E_INVAL;
    if (cap_rows <= 0 || cap_rows > kMaxRows || n_new <= 0 || *t_rows < 0 || *t_rows > cap_rows)
        return MLA8_E_INVAL;
    if (!aligned16(x_new))
        return MLA8_E_INVAL;
    if (n_new > kMaxFusedRows)
        return MLA8_E_RANGE;
    if (n_new > cap_rows - *t_rows)
        return MLA8_E_CAPACITY;
    return check_decode_common(kv, kv_scales, *t_rows + n_new, lc, rc, q_lat, q_rope, n_heads,
                               sm_scale, out);
}

static int append_decode_layout(uint8_t* kv, float* kv_scales, int64_t cap_rows, int64_t* t_rows,
                                const float* x_new, int64_t n_new, int32_t lc, int32_t rc,
                                const float* q_lat, const float* q_rope, int32_t n_heads,
                                float sm_scale, float* out, float* lse, void* workspace,
                                size_t ws_bytes, void* stream, const mla8_opts* opts,
                                int32_t layout)
{
    int st = append_decode_check(kv, kv_scales, cap_rows, t_rows, x_new, n_new, lc, rc, q_lat,
                                 q_rope, n_heads, sm_scale, out);
    if (st != MLA8_OK)
        return st;
    const int64_t t_new = *t_rows + n_new;
    st = run_attention(MLA8_OP_DECODE, kv, kv_scales, t_new, lc, rc, nullptr, t_new, q_lat,
                       q_rope, n_heads, n_heads, 0, sm_scale, out, lse, workspace, ws_bytes,
                       stream, opts, x_new, kv, kv_scales, *t_rows, n_new, layout);
    if (st == MLA8_OK)
        *t_rows = t_new;
    return st;
}

static int batch_layout(const uint8_t* kv, const float* kv_scales, int64_t t_rows, int32_t lc,
                        int32_t rc, const float* q_lat, const float* q_rope, int32_t n_q,
                        int64_t pos0, int32_t n_heads, float sm_scale, float* out, float* lse,
                        void* workspace, size_t ws_bytes, void* stream, const mla8_opts* opts,
                        int32_t layout)
{
    int st = check_decode_common(kv, kv_scales, t_rows, lc, rc, q_lat, q_rope, n_heads, sm_scale,
                                 out);
    if (st != MLA8_OK)
        return st;
    if (n_q <= 0 || pos0 < 0)
        return MLA8_E_INVAL;
    if ((int64_t)n_q * (int64_t)n_heads > kMaxRows / 1024)
        return MLA8_E_UNSUPPORTED;
    if (pos0 + n_q > t_rows)
        return MLA8_E_RANGE;
    return run_attention(MLA8_OP_BATCH, kv, kv_scales, t_rows, lc, rc, nullptr, pos0 + n_q, q_lat,
                         q_rope, n_q * n_heads, n_heads, pos0, sm_scale, out, lse, workspace,
                         ws_bytes, stream, opts, nullptr, nullptr, nullptr, 0, 0, layout);
}

int mla8_append_decode_mx(uint8_t* kv_rows, float* kv_scales, int64_t cap_rows, int64_t* t_rows,
                          const float* x_new, int64_t n_new, int32_t lc, int32_t rc,
                          const float* q_lat, const float* q_rope, int32_t n_heads,
                          float sm_scale, float* out, float* lse, void* workspace,
                          size_t ws_bytes, void* stream, const mla8_opts* opts)
{
    const int st = check_shape_mx(lc, rc);
    if (st != MLA8_OK)
        return st;
    return append_decode_layout(kv_rows, kv_scales, cap_rows, t_rows, x_new, n_new, lc, rc,
                                q_lat, q_rope, n_heads, sm_scale, out, lse, workspace, ws_bytes,
                                stream, opts, kMixed);
}

int mla8_batch_mx(const uint8_t* kv_rows, const float* kv_scales, int64_t t_rows, int32_t lc,
                  int32_t rc, const float* q_lat, const float* q_rope, int32_t n_q, int64_t pos0,
                  int32_t n_heads, float sm_scale, float* out, float* lse, void* workspace,
                  size_t ws_bytes, void* stream, const mla8_opts* opts)
{
    const int st = check_shape_mx(lc, rc);
    if (st != MLA8_OK)
        return st;
    return batch_layout(kv_rows, kv_scales, t_rows, lc, rc, q_lat, q_rope, n_q, pos0, n_heads,
                        sm_scale, out, lse, workspace, ws_bytes, stream, opts, kMixed);
}

int mla8_append_decode(uint8_t* kv_codes, float* kv_scales, int64_t cap_rows, int64_t* t_rows,
                       const float* x_new, int64_t n_new, int32_t lc, int32_t rc,
                       const float* q_lat, const float* q_rope, int32_t n_heads, float sm_scale,
                       float* out, float* lse, void* workspace, size_t ws_bytes, void* stream,
                       const mla8_opts* opts)
{
    const int st = check_shape(lc, rc);
    if (st != MLA8_OK)
        return st;
    return append_decode_layout(kv_codes, kv_scales, cap_rows, t_rows, x_new, n_new, lc, rc,
                                q_lat, q_rope, n_heads, sm_scale, out, lse, workspace, ws_bytes,
                                stream, opts, kE4m3);
}

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

static int scratch_address(void** addr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MLA8_E_HIP;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return MLA8_E_HIP;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *addr = p;
    return MLA8_OK;
}

int mla8_append_decode_noalloc(uint8_t* kv_codes, float* kv_scales, int64_t cap_rows,
                               int64_t* t_rows, const float* x_new, int64_t n_new, int32_t lc,
                               int32_t rc, const float* q_lat, const float* q_rope,
                               int32_t n_heads, float sm_scale, float* out, float* lse,
                               void* stream, const mla8_opts* opts)
{
    int st = check_shape(lc, rc);
    if (st != MLA8_OK)
        return st;
    st = append_decode_check(kv_codes, kv_scales, cap_rows, t_rows, x_new, n_new, lc, rc, q_lat,
                             q_rope, n_heads, sm_scale, out);
    if (st != MLA8_OK)
        return st;
    const Plan p = make_plan(MLA8_OP_DECODE, *t_rows + n_new, n_heads, forced_splits(opts));
    if (ws_bytes_for(p, n_heads, lc) > kScratchBytes)
        return MLA8_E_SCRATCH;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != MLA8_OK)
        return st;
    return append_decode_layout(kv_codes, kv_scales, cap_rows, t_rows, x_new, n_new, lc, rc,
                                q_lat, q_rope, n_heads, sm_scale, out, lse, ws, kScratchBytes,
                                stream, opts, kE4m3);
}

int mla8_decode_sel(const uint8_t* kv_codes, const float* kv_scales, int64_t t_rows, int32_t lc,
                    int32_t rc, const int32_t* sel, int64_t ns, const float* q_lat,
                    const float* q_rope, int32_t n_heads, float sm_scale, float* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream, const mla8_opts* opts)
{
    int st = check_decode_common(kv_codes, kv_scales, t_rows, lc, rc, q_lat, q_rope, n_heads,
                                 sm_scale, out);
    if (st != MLA8_OK)
        return st;
    if (!sel || ns <= 0 || ns > kMaxRows || (reinterpret_cast<uintptr_t>(sel) & 3u))
        return MLA8_E_INVAL;
    return run_attention(MLA8_OP_DECODE_SEL, kv_codes, kv_scales, t_rows, lc, rc, sel, ns, q_lat,
                         q_rope, n_heads, n_heads, 0, sm_scale, out, lse, workspace, ws_bytes,
                         stream, opts);
}

int mla8_batch(const uint8_t* kv_codes, const float* kv_scales, int64_t t_rows, int32_t lc,
               int32_t rc, const float* q_lat, const float* q_rope, int32_t n_q, int64_t pos0,
               int32_t n_heads, float sm_scale, float* out, float* lse, void* workspace,
               size_t ws_bytes, void* stream, const mla8_opts* opts)
{
    return batch_layout(kv_codes, kv_scales, t_rows, lc, rc, q_lat, q_rope, n_q, pos0, n_heads,
                        sm_scale, out, lse, workspace, ws_bytes, stream, opts, kE4m3);
}

int mla8_index_topk(const uint8_t* k_codes, const float* k_scales, int64_t t_rows, int32_t ihd,
                    const float* q, const float* w, int32_t n_ih, int32_t top_k, int32_t* sel,
                    float* scores, void* workspace, size_t ws_bytes, void* stream,
                    const mla8_opts* opts)
{
    if (!k_codes || !k_scales || !q || !w || !sel)
        return MLA8_E_INVAL;
    if (t_rows <= 0 || t_rows > kMaxRows || top_k <= 0 || n_ih <= 0 || ihd <= 0)
        return MLA8_E_INVAL;
    if (ihd != kIndexDim || (n_ih % 16) != 0 || n_ih > kIndexMaxHeads || top_k > kIndexMaxTopK ||
        t_rows > kIndexMaxRows)
        return MLA8_E_UNSUPPORTED;
    if (!aligned16(k_codes) || !aligned16(q) || (reinterpret_cast<uintptr_t>(k_scales) & 3u) ||
        (reinterpret_cast<uintptr_t>(w) & 3u) || (reinterpret_cast<uintptr_t>(sel) & 3u) ||
        (reinterpret_cast<uintptr_t>(scores) & 3u))
        return MLA8_E_INVAL;
    if (workspace == nullptr || ws_bytes < index_ws_bytes(t_rows))
        return MLA8_E_WORKSPACE;
    if (!aligned16(workspace))
        return MLA8_E_INVAL;
    char* ws = static_cast<char*>(workspace);
    IndexArgs a;
    a.k_codes = k_codes;
    a.k_scales = k_scales;
    a.t_rows = (int32_t)t_rows;
    a.q = q;
    a.w = w;
    a.n_ih = n_ih;
    a.top_k = top_k;
    a.sel = sel;
    a.scores = scores;
    a.keys = reinterpret_cast<uint32_t*>(ws);
    ws += r256((size_t)t_rows * 4);
    a.cand = reinterpret_cast<uint64_t*>(ws);
    ws += r256((size_t)t_rows * 8);
    a.hist = reinterpret_cast<uint32_t*>(ws);
    ws += r256(kIndexHistCopies * kIndexHistBins * 4);
    a.wg_cnt = reinterpret_cast<uint32_t*>(ws);
    ws += r256((size_t)((t_rows + 4095) / 4096) * 4);
    a.top = reinterpret_cast<uint32_t*>(ws);
    return launch_index_topk(a, static_cast<hipStream_t>(stream), ev_before(opts), ev_after(opts)) ==
                   hipSuccess
               ? MLA8_OK
               : MLA8_E_HIP;
}

size_t mla8_workspace_bytes(int32_t op, int64_t rows, int32_t n_heads, int32_t n_q, int32_t lc,
                            const mla8_opts* opts)
{
    if (op < MLA8_OP_DECODE || op > MLA8_OP_INDEX || rows <= 0 || rows > kMaxRows ||
        n_heads <= 0 || lc <= 0)
        return 0;
    if (op == MLA8_OP_INDEX)
        return index_ws_bytes(rows);
    int64_t n_qh = n_heads;
    if (op == MLA8_OP_BATCH) {
        if (n_q <= 0)
            return 0;
        n_qh = (int64_t)n_q * n_heads;
        if (n_qh > kMaxRows / 1024)
            return 0;
    }
    return ws_bytes_for(make_plan(op, rows, (int32_t)n_qh, forced_splits(opts)), (int32_t)n_qh, lc);
}

int32_t mla8_plan_splits(int32_t op, int64_t rows, int32_t n_heads, int32_t n_q,
                         const mla8_opts* opts)
{
    if (rows <= 0 || n_heads <= 0)
        return 0;
    const int64_t n_qh = op == MLA8_OP_BATCH ? (int64_t)n_q * n_heads : n_heads;
    if (n_qh <= 0 || n_qh > kMaxRows / 1024)
        return 0;
    return make_plan(op, rows, (int32_t)n_qh, forced_splits(opts)).n_chunks;
}

const char* mla8_status_string(int status)
{
    switch (status) {
    case MLA8_OK: return "ok";
    case MLA8_E_INVAL: return "invalid argument (NULL pointer, bad size or misaligned buffer)";
    case MLA8_E_RANGE:
        return "row range outside the shadow (pos0 + n_q > t_rows, or an append that does not "
               "start at the file's committed end)";
    case MLA8_E_CAPACITY: return "append would exceed cap_rows";
    case MLA8_E_WORKSPACE: return "workspace smaller than mla8_workspace_bytes()";
    case MLA8_E_UNSUPPORTED:
        return "unsupported shape or mode: need 16<=lc<=512, 0<=rc<=128, both multiples of 16, "
               "lc+rc<=640 (indexer: ihd 128, n_ih a multiple of 16 up to 64, top_k <= 4096)";
    case MLA8_E_HIP: return "HIP launch or copy failed";
    case MLA8_E_IO: return "file I/O failed, or no valid header in the file";
    case MLA8_E_SCRATCH:
        return "the call needs more than the library's static scratch (MLA8_SCRATCH_BYTES) of "
               "mla8_append_decode_noalloc: fewer heads, rows or forced splits, or "
               "mla8_append_decode with a workspace";
    default: return "unknown status";
    }
}

const char* mla8_version(void) { return "mla8 0.1.0 gfx950"; }

static_assert(kStreamWords == MLA8_STREAM_WORDS, "stream-read output words");
static_assert(kScratchBytes == MLA8_SCRATCH_BYTES, "scratch size in the header");

int mla8_stream_read(const void* p, int64_t bytes, uint32_t* out, void* stream)
{
    if (!p || !out || bytes < 0 || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(p) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 15) != 0)
        return MLA8_E_INVAL;
    return launch_stream_read(p, bytes, out, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MLA8_OK
               : MLA8_E_HIP;
}

int mla8_test_encode(const float* x, int64_t n, uint8_t* codes, void* stream)
{
    if (!x || !codes || n < 0)
        return MLA8_E_INVAL;
    if (n == 0)
        return MLA8_OK;
    return launch_test_encode(x, n, codes, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MLA8_OK
               : MLA8_E_HIP;
}

int mla8_test_encode_pk(const float* x, int64_t n, uint8_t* codes, void* stream)
{
    if (!x || !codes || n < 0 || (n & 3) != 0 || (reinterpret_cast<uintptr_t>(x) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(codes) & 3) != 0)
        return MLA8_E_INVAL;
    if (n == 0)
        return MLA8_OK;
    return launch_test_encode_pk(x, n, codes, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MLA8_OK
               : MLA8_E_HIP;
}

}  // extern "C"
