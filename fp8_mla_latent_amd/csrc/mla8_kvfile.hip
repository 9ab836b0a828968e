// Persistent shadow files: the fp8 latent rows of every layer, saved token by
// token so that a session resumes without re-quantizing.
//
// Method source: colibri PR #300 "KV8 long-context CUDA: fp8 device shadow,
// split-T kernels, DSA-aware gather", first commit ("KV8 base"), the .coli_kv
// v2 bullet: a versioned file whose header names the row type, appended
// through a persistent handle and a staging buffer, holding fp8 rows plus
// their scales; files of the previous version (f32 rows) are quantized when a
// session resumes and stay untouched on disk until the first append rewrites
// them in the new version, so a crash before that append loses nothing.
//
// The format is this library's own (not the page's):
//
//   [0, 64)     header slot A        [64, 128)  header slot B
//   [128, ...)  body, token-major: token t at 128 + t * stride
//
//   header slot, little-endian:
//     0  char magic[8] = "MLA8KV\0\0"
//     8  u32  version   1 = f32 rows, 2 = e4m3 rows with an f32 scale
//     12 u32  n_layers
//     16 u32  lc
//     20 u32  rc
//     24 u64  n_tokens  tokens committed
//     32 u64  seq       commit number
//     40 u32  check     FNV-1a (32-bit) of bytes [0, 40)
//     44 ..63 zero
//   version 2 token: for each layer, D = lc + rc code bytes then the f32
//   scale (stride n_layers * (D + 4)); version 1 token: for each layer, D f32
//   values (stride n_layers * D * 4).
//
// Commit protocol: an append writes the new tokens' bytes past the committed
// end, flushes them, then writes the header slot that the current commit does
// not occupy with seq + 1 and the new token count, and flushes it.  A reader
// takes the valid slot (magic, version, check) with the larger seq; bytes past
// its token count are ignored.  A crash at any point leaves the previous
// commit readable.  The first append to a version-1 file writes a complete
// version-2 file next to it (rows from the shadows, which hold the quantized
// version-1 rows after a resume) and renames it over the original.
#include "mla8.h"
#include "mla8_internal.h"

#include <fcntl.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <string>
#include <vector>

namespace {

constexpr char kMagic[8] = {'M', 'L', 'A', '8', 'K', 'V', 0, 0};
constexpr size_t kSlot = 64;
constexpr size_t kBody = 2 * kSlot;
constexpr int64_t kChunkTokens = 1024;  // tokens per staging round trip

struct Header {
    uint32_t version = 0;
    uint32_t n_layers = 0;
    uint32_t lc = 0;
    uint32_t rc = 0;
    uint64_t n_tokens = 0;
    uint64_t seq = 0;
};

uint32_t fnv1a(const uint8_t* p, size_t n)
{
    uint32_t h = 2166136261u;
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 16777619u;
    }
    return h;
}

void put32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
void put64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }
uint32_t get32(const uint8_t* p)
{
    uint32_t v;
    memcpy(&v, p, 4);
    return v;
}
uint64_t get64(const uint8_t* p)
{
    uint64_t v;
    memcpy(&v, p, 8);
    return v;
}

void encode_slot(const Header& h, uint8_t* s)
{
    memset(s, 0, kSlot);
    memcpy(s, kMagic, 8);
    put32(s + 8, h.version);
    put32(s + 12, h.n_layers);
    put32(s + 16, h.lc);
    put32(s + 20, h.rc);
    put64(s + 24, h.n_tokens);
    put64(s + 32, h.seq);
    put32(s + 40, fnv1a(s, 40));
}

bool decode_slot(const uint8_t* s, Header& h)
{
    if (memcmp(s, kMagic, 8) != 0 || get32(s + 40) != fnv1a(s, 40))
        return false;
    h.version = get32(s + 8);
    h.n_layers = get32(s + 12);
    h.lc = get32(s + 16);
    h.rc = get32(s + 20);
    h.n_tokens = get64(s + 24);
    h.seq = get64(s + 32);
    return (h.version == 1 || h.version == 2) && h.n_layers > 0;
}

int64_t row_bytes(const Header& h)
{
    const int64_t d = (int64_t)h.lc + h.rc;
    return h.version == 2 ? d + 4 : d * 4;
}
int64_t stride(const Header& h) { return (int64_t)h.n_layers * row_bytes(h); }

bool pwrite_all(int fd, const void* buf, size_t n, int64_t off)
{
    const uint8_t* p = static_cast<const uint8_t*>(buf);
    while (n > 0) {
        const ssize_t w = pwrite(fd, p, n, (off_t)off);
        if (w <= 0)
            return false;
        p += w;
        n -= (size_t)w;
        off += w;
    }
    return true;
}

bool pread_all(int fd, void* buf, size_t n, int64_t off)
{
    uint8_t* p = static_cast<uint8_t*>(buf);
    while (n > 0) {
        const ssize_t r = pread(fd, p, n, (off_t)off);
        if (r <= 0)
            return false;
        p += r;
        n -= (size_t)r;
        off += r;
    }
    return true;
}

// A slot whose check matches can still describe a file that cannot be read:
// a corrupted or foreign header, or a body cut short after its commit.  Such a
// slot is not used: the layer count and row width must be ones this library
// writes, the token count below 2^31 (row counts are int32 on the device), and
// the body must hold every committed token.
bool slot_usable(const Header& h, int64_t file_bytes)
{
    if (h.n_layers > 65536 || h.lc + (uint64_t)h.rc > 640 || h.n_tokens > 0x7FFFFFFFull)
        return false;
    const int64_t sb = stride(h);
    return sb > 0 && (int64_t)h.n_tokens <= (file_bytes - (int64_t)kBody) / sb;
}

// The committed header (the usable slot with the larger seq) and which slot
// it is in.
int read_header(int fd, Header& h, int& slot)
{
    uint8_t s[kBody];
    struct stat sbuf;
    if (fstat(fd, &sbuf) != 0 || !pread_all(fd, s, kBody, 0))
        return MLA8_E_IO;
    const int64_t file_bytes = (int64_t)sbuf.st_size;
    Header a, b;
    const bool va = decode_slot(s, a) && slot_usable(a, file_bytes);
    const bool vb = decode_slot(s + kSlot, b) && slot_usable(b, file_bytes);
    if (!va && !vb)
        return MLA8_E_IO;
    if (va && (!vb || a.seq >= b.seq)) {
        h = a;
        slot = 0;
    } else {
        h = b;
        slot = 1;
    }
    return MLA8_OK;
}

bool shape_ok(int32_t n_layers, int32_t lc, int32_t rc)
{
    return n_layers > 0 && lc >= 16 && lc <= 512 && lc % 16 == 0 && rc >= 0 && rc <= 128 &&
           rc % 16 == 0 && lc + rc <= 640;
}

// Copies between the shadows (device or host) and host staging.
bool copy_out(void* dst, const void* src, size_t n, bool dev, hipStream_t st)
{
    if (!dev) {
        memcpy(dst, src, n);
        return true;
    }
    return hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToHost, st) == hipSuccess &&
           hipStreamSynchronize(st) == hipSuccess;
}
bool copy_in(void* dst, const void* src, size_t n, bool dev, hipStream_t st)
{
    if (!dev) {
        memcpy(dst, src, n);
        return true;
    }
    return hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, st) == hipSuccess &&
           hipStreamSynchronize(st) == hipSuccess;
}

// Version-2 bytes of tokens [t0, t1) from the shadows, written at their body
// offsets.
int write_rows(int fd, const Header& h, const uint8_t* const* codes, const float* const* scales,
               int64_t t0, int64_t t1, bool dev, hipStream_t st)
{
    const int64_t d = (int64_t)h.lc + h.rc, sb = stride(h), rb = row_bytes(h);
    std::vector<uint8_t> body, rows;
    std::vector<float> sc;
    for (int64_t c0 = t0; c0 < t1; c0 += kChunkTokens) {
        const int64_t n = (t1 - c0 < kChunkTokens) ? t1 - c0 : kChunkTokens;
        body.assign((size_t)(n * sb), 0);
        rows.resize((size_t)(n * d));
        sc.resize((size_t)n);
        for (uint32_t l = 0; l < h.n_layers; ++l) {
            if (!copy_out(rows.data(), codes[l] + c0 * d, (size_t)(n * d), dev, st) ||
                !copy_out(sc.data(), scales[l] + c0, (size_t)n * 4, dev, st))
                return MLA8_E_HIP;
            for (int64_t t = 0; t < n; ++t) {
                uint8_t* dst = body.data() + t * sb + l * rb;
                memcpy(dst, rows.data() + t * d, (size_t)d);
                memcpy(dst + d, &sc[(size_t)t], 4);
            }
        }
        if (!pwrite_all(fd, body.data(), body.size(), (int64_t)kBody + c0 * sb))
            return MLA8_E_IO;
    }
    return MLA8_OK;
}

int commit(int fd, Header h, int cur_slot, uint64_t n_tokens)
{
    if (fdatasync(fd) != 0)
        return MLA8_E_IO;
    h.n_tokens = n_tokens;
    h.seq += 1;
    uint8_t s[kSlot];
    encode_slot(h, s);
    if (!pwrite_all(fd, s, kSlot, (int64_t)((1 - cur_slot) * kSlot)) || fdatasync(fd) != 0)
        return MLA8_E_IO;
    return MLA8_OK;
}

// A complete version-2 file with tokens [0, n) at `tmp`, renamed over `path`.
int rewrite_v2(const char* path, const Header& old, const uint8_t* const* codes,
               const float* const* scales, int64_t n, bool dev, hipStream_t st)
{
    const std::string tmp = std::string(path) + ".v2tmp";
    const int fd = open(tmp.c_str(), O_RDWR | O_CREAT | O_TRUNC, 0644);
    if (fd < 0)
        return MLA8_E_IO;
    Header h = old;
    h.version = 2;
    h.n_tokens = 0;
    h.seq = 0;
    uint8_t s[kBody];
    memset(s, 0, kBody);
    encode_slot(h, s);
    int st_ = pwrite_all(fd, s, kBody, 0) ? MLA8_OK : MLA8_E_IO;
    if (st_ == MLA8_OK)
        st_ = write_rows(fd, h, codes, scales, 0, n, dev, st);
    if (st_ == MLA8_OK)
        st_ = commit(fd, h, 0, (uint64_t)n);
    close(fd);
    if (st_ != MLA8_OK) {
        unlink(tmp.c_str());
        return st_;
    }
    if (rename(tmp.c_str(), path) != 0) {
        unlink(tmp.c_str());
        return MLA8_E_IO;
    }
    // make the rename itself durable
    std::string dir(path);
    const size_t cut = dir.find_last_of('/');
    dir = (cut == std::string::npos) ? std::string(".") : dir.substr(0, cut ? cut : 1);
    const int dfd = open(dir.c_str(), O_RDONLY);
    if (dfd >= 0) {
        fsync(dfd);
        close(dfd);
    }
    return MLA8_OK;
}

}  // namespace

extern "C" {

int mla8_kvfile_create(const char* path, int32_t n_layers, int32_t lc, int32_t rc)
{
    if (!path)
        return MLA8_E_INVAL;
    if (!shape_ok(n_layers, lc, rc))
        return n_layers <= 0 ? MLA8_E_INVAL : MLA8_E_UNSUPPORTED;
    const int fd = open(path, O_RDWR | O_CREAT | O_TRUNC, 0644);
    if (fd < 0)
        return MLA8_E_IO;
    Header h;
    h.version = 2;
    h.n_layers = (uint32_t)n_layers;
    h.lc = (uint32_t)lc;
    h.rc = (uint32_t)rc;
    uint8_t s[kBody];
    memset(s, 0, kBody);
    encode_slot(h, s);
    const bool ok = pwrite_all(fd, s, kBody, 0) && fdatasync(fd) == 0;
    close(fd);
    return ok ? MLA8_OK : MLA8_E_IO;
}

int mla8_kvfile_info(const char* path, int32_t* version, int32_t* n_layers, int32_t* lc,
                     int32_t* rc, int64_t* n_tokens)
{
    if (!path || !version || !n_layers || !lc || !rc || !n_tokens)
        return MLA8_E_INVAL;
    const int fd = open(path, O_RDONLY);
    if (fd < 0)
        return MLA8_E_IO;
    Header h;
    int slot;
    const int st = read_header(fd, h, slot);
    close(fd);
    if (st != MLA8_OK)
        return st;
    *version = (int32_t)h.version;
    *n_layers = (int32_t)h.n_layers;
    *lc = (int32_t)h.lc;
    *rc = (int32_t)h.rc;
    *n_tokens = (int64_t)h.n_tokens;
    return MLA8_OK;
}

int mla8_kvfile_append(const char* path, int32_t n_layers, const uint8_t* const* kv_codes,
                       const float* const* kv_scales, int64_t t0, int64_t n_tok, int32_t lc,
                       int32_t rc, int32_t on_device, void* stream)
{
    if (!path || !kv_codes || !kv_scales || t0 < 0 || n_tok < 0 || t0 + n_tok > 0x7FFFFFFF)
        return MLA8_E_INVAL;
    if (!shape_ok(n_layers, lc, rc))
        return n_layers <= 0 ? MLA8_E_INVAL : MLA8_E_UNSUPPORTED;
    for (int32_t l = 0; l < n_layers; ++l)
        if (!kv_codes[l] || !kv_scales[l])
            return MLA8_E_INVAL;
    const int fd = open(path, O_RDWR);
    if (fd < 0)
        return MLA8_E_IO;
    Header h;
    int slot;
    int st = read_header(fd, h, slot);
    if (st == MLA8_OK && (h.n_layers != (uint32_t)n_layers || h.lc != (uint32_t)lc ||
                          h.rc != (uint32_t)rc))
        st = MLA8_E_INVAL;
    if (st == MLA8_OK && (uint64_t)t0 != h.n_tokens)
        st = MLA8_E_RANGE;
    if (st != MLA8_OK || n_tok == 0) {
        close(fd);
        return st;
    }
    const bool dev = on_device != 0;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (h.version == 1) {
        // first append after a resume from f32 rows: the whole file moves to
        // version 2, built from the shadows, and replaces the original
        close(fd);
        return rewrite_v2(path, h, kv_codes, kv_scales, t0 + n_tok, dev, hs);
    }
    st = write_rows(fd, h, kv_codes, kv_scales, t0, t0 + n_tok, dev, hs);
    if (st == MLA8_OK)
        st = commit(fd, h, slot, (uint64_t)(t0 + n_tok));
    close(fd);
    return st;
}

int mla8_kvfile_load(const char* path, int32_t n_layers, uint8_t* const* kv_codes,
                     float* const* kv_scales, int64_t cap_rows, int64_t* t_rows, int32_t lc,
                     int32_t rc, int32_t on_device, void* workspace, size_t ws_bytes,
                     void* stream)
{
    if (!path || !kv_codes || !kv_scales || !t_rows || cap_rows <= 0 || cap_rows > 0x7FFFFFFF)
        return MLA8_E_INVAL;
    if (!shape_ok(n_layers, lc, rc))
        return n_layers <= 0 ? MLA8_E_INVAL : MLA8_E_UNSUPPORTED;
    for (int32_t l = 0; l < n_layers; ++l)
        if (!kv_codes[l] || !kv_scales[l])
            return MLA8_E_INVAL;
    const int fd = open(path, O_RDONLY);
    if (fd < 0)
        return MLA8_E_IO;
    Header h;
    int slot;
    int st = read_header(fd, h, slot);
    if (st == MLA8_OK && (h.n_layers != (uint32_t)n_layers || h.lc != (uint32_t)lc ||
                          h.rc != (uint32_t)rc))
        st = MLA8_E_INVAL;
    if (st == MLA8_OK && (int64_t)h.n_tokens > cap_rows)
        st = MLA8_E_CAPACITY;
    const bool dev = on_device != 0;
    const int64_t d = lc + rc;
    if (st == MLA8_OK && h.version == 1) {
        // f32 rows are quantized on the device, a chunk of rows at a time
        // through the workspace
        if (!dev)
            st = MLA8_E_UNSUPPORTED;
        else if (!workspace || ws_bytes < (size_t)(d * 4) ||
                 (reinterpret_cast<uintptr_t>(workspace) & 15u))
            st = MLA8_E_WORKSPACE;
    }
    if (st != MLA8_OK) {
        close(fd);
        return st;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int64_t n_all = (int64_t)h.n_tokens, sb = stride(h), rb = row_bytes(h);
    int64_t chunk = kChunkTokens;
    if (h.version == 1 && (int64_t)(ws_bytes / (size_t)(d * 4)) < chunk)
        chunk = (int64_t)(ws_bytes / (size_t)(d * 4));
    std::vector<uint8_t> body, rows;
    std::vector<float> sc;
    for (int64_t c0 = 0; c0 < n_all && st == MLA8_OK; c0 += chunk) {
        const int64_t n = (n_all - c0 < chunk) ? n_all - c0 : chunk;
        body.resize((size_t)(n * sb));
        if (!pread_all(fd, body.data(), body.size(), (int64_t)kBody + c0 * sb)) {
            st = MLA8_E_IO;
            break;
        }
        for (int32_t l = 0; l < n_layers && st == MLA8_OK; ++l) {
            rows.resize((size_t)(n * rb));
            for (int64_t t = 0; t < n; ++t)
                memcpy(rows.data() + t * rb, body.data() + t * sb + l * rb, (size_t)rb);
            if (h.version == 2) {
                std::vector<uint8_t> cd((size_t)(n * d));
                sc.resize((size_t)n);
                for (int64_t t = 0; t < n; ++t) {
                    memcpy(cd.data() + t * d, rows.data() + t * rb, (size_t)d);
                    memcpy(&sc[(size_t)t], rows.data() + t * rb + d, 4);
                }
                // The row quantizer never writes a NaN code (0x7F / 0xFF) nor
                // a negative or non-finite scale: a body holding one is corrupt
                // and is not loaded (this chunk is refused before its copy).
                bool body_ok = true;
                for (size_t i = 0; i < cd.size() && body_ok; ++i)
                    body_ok = (cd[i] & 0x7F) != 0x7F;
                for (int64_t t = 0; t < n && body_ok; ++t)
                    body_ok = sc[(size_t)t] >= 0.0f && sc[(size_t)t] <= 3.402823466e38f;
                if (!body_ok) {
                    st = MLA8_E_IO;
                    break;
                }
                if (!copy_in(kv_codes[l] + c0 * d, cd.data(), cd.size(), dev, hs) ||
                    !copy_in(kv_scales[l] + c0, sc.data(), (size_t)n * 4, dev, hs))
                    st = MLA8_E_HIP;
            } else {
                float* x = static_cast<float*>(workspace);
                if (!copy_in(x, rows.data(), rows.size(), true, hs) ||
                    mla8::launch_quantize(x, n, (int32_t)d, kv_codes[l] + c0 * d,
                                          kv_scales[l] + c0, hs) != hipSuccess ||
                    hipStreamSynchronize(hs) != hipSuccess)
                    st = MLA8_E_HIP;
            }
        }
    }
    close(fd);
    if (st == MLA8_OK)
        *t_rows = n_all;
    return st;
}

}  // extern "C"
