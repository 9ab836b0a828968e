"""Persistent shadow files (mla8_kvfile_*), host shadows, no GPU.

The file format is pinned by an independent reader and writer written here
from the format's definition (two 64-byte header slots with an FNV-1a check,
a token-major body from byte 128), not by calling the library twice.  The
crash-safety cases cut the commit protocol at each step: body bytes written
without a header, a torn newest header slot, both slots torn.
The page passage is the .coli_kv v2 bullet of colibri PR #300's "KV8 base"
commit: a versioned file holding fp8 rows plus scales, appended through a
persistent handle, with files of the previous version (f32 rows) quantized on
resume and left intact until the first append rewrites them.
"""
from __future__ import annotations

import struct

import numpy as np
import pytest

from fp8_mla_latent_amd import mla8 as m

MAGIC = b"MLA8KV\0\0"


def fnv1a(b: bytes) -> int:
    h = 2166136261
    for x in b:
        h = ((h ^ x) * 16777619) & 0xFFFFFFFF
    return h


def slot_bytes(version, n_layers, lc, rc, n_tokens, seq) -> bytes:
    head = MAGIC + struct.pack("<IIIIQQ", version, n_layers, lc, rc, n_tokens, seq)
    return head + struct.pack("<I", fnv1a(head)) + b"\0" * 20


def read_file(path):
    raw = open(path, "rb").read()
    best = None
    for i in range(2):
        s = raw[64 * i:64 * i + 64]
        if s[:8] != MAGIC or struct.unpack("<I", s[40:44])[0] != fnv1a(s[:40]):
            continue
        v, nl, lc, rc, nt, seq = struct.unpack("<IIIIQQ", s[8:40])
        if best is None or seq > best[5]:
            best = (v, nl, lc, rc, nt, seq)
    assert best is not None
    v, nl, lc, rc, nt, seq = best
    d = lc + rc
    rb = d + 4 if v == 2 else 4 * d
    body = np.frombuffer(raw[128:128 + nt * nl * rb], np.uint8).reshape(nt, nl, rb)
    if v == 2:
        codes = [np.ascontiguousarray(body[:, l, :d]) for l in range(nl)]
        scales = [np.ascontiguousarray(body[:, l, d:]).view(np.float32).reshape(nt)
                  for l in range(nl)]
        return best, codes, scales
    rows = [np.ascontiguousarray(body[:, l, :]).view(np.float32).reshape(nt, d)
            for l in range(nl)]
    return best, rows, None


def write_file(path, version, layers, lc, rc, seq=0):
    """layers: version 2 -> list of (codes [T, D] u8, scales [T] f32); version 1
    -> list of f32 rows [T, D]."""
    nt = layers[0][0].shape[0] if version == 2 else layers[0].shape[0]
    out = bytearray(slot_bytes(version, len(layers), lc, rc, nt, seq) + b"\0" * 64)
    for t in range(nt):
        for lay in layers:
            if version == 2:
                out += lay[0][t].tobytes() + lay[1][t:t + 1].astype(np.float32).tobytes()
            else:
                out += lay[t].astype(np.float32).tobytes()
    open(path, "wb").write(bytes(out))


def shadows(n_layers, cap, d):
    return ([np.zeros((cap, d), np.uint8) for _ in range(n_layers)],
            [np.zeros((cap,), np.float32) for _ in range(n_layers)])


def random_rows(g, n_layers, t, d):
    """Random shadow rows as the quantizer writes them: any e4m3 byte but the
    two NaN codes 0x7F / 0xFF, and finite positive scales."""
    def codes():
        c = g.integers(0, 256, (t, d), dtype=np.uint8)
        return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)
    return ([codes() for _ in range(n_layers)],
            [g.random(t, dtype=np.float32) + 0.01 for _ in range(n_layers)])


LC, RC, D = 64, 16, 80


def test_create_info_and_layout(tmp_path):
    p = str(tmp_path / "a.mla8kv")
    m.mla8_kvfile_create(p, 3, LC, RC)
    assert m.mla8_kvfile_info(p) == {"version": 2, "n_layers": 3, "lc": LC, "rc": RC,
                                     "n_tokens": 0}
    raw = open(p, "rb").read()
    assert len(raw) == 128 and raw[:64] == slot_bytes(2, 3, LC, RC, 0, 0)


def test_appends_roundtrip_and_independent_reader(tmp_path):
    g = np.random.Generator(np.random.PCG64(5))
    p = str(tmp_path / "b.mla8kv")
    nl, t = 2, 2500  # more tokens than one staging chunk
    codes, scales = random_rows(g, nl, t, D)
    m.mla8_kvfile_create(p, nl, LC, RC)
    t0 = 0
    for n in (1, 7, 1200, t - 1208):
        m.mla8_kvfile_append(p, codes, scales, t0, n, LC, RC)
        t0 += n
        assert m.mla8_kvfile_info(p)["n_tokens"] == t0
    hdr, fc, fs = read_file(p)
    assert hdr[0] == 2 and hdr[4] == t and hdr[5] == 4  # four commits
    for l in range(nl):
        np.testing.assert_array_equal(fc[l], codes[l])
        np.testing.assert_array_equal(fs[l].view(np.uint32), scales[l].view(np.uint32))
    c2, s2 = shadows(nl, t + 10, D)
    assert m.mla8_kvfile_load(p, c2, s2, LC, RC) == t
    for l in range(nl):
        np.testing.assert_array_equal(c2[l][:t], codes[l])
        np.testing.assert_array_equal(s2[l][:t], scales[l])
        assert not c2[l][t:].any()


def test_load_of_an_independently_written_file(tmp_path):
    g = np.random.Generator(np.random.PCG64(6))
    p = str(tmp_path / "c.mla8kv")
    codes, scales = random_rows(g, 3, 40, D)
    write_file(p, 2, list(zip(codes, scales)), LC, RC, seq=7)
    c2, s2 = shadows(3, 40, D)
    assert m.mla8_kvfile_load(p, c2, s2, LC, RC) == 40
    for l in range(3):
        np.testing.assert_array_equal(c2[l], codes[l])
        np.testing.assert_array_equal(s2[l], scales[l])


def test_refusals(tmp_path):
    g = np.random.Generator(np.random.PCG64(7))
    p = str(tmp_path / "d.mla8kv")
    codes, scales = random_rows(g, 2, 10, D)
    m.mla8_kvfile_create(p, 2, LC, RC)
    m.mla8_kvfile_append(p, codes, scales, 0, 5, LC, RC)
    cases = [
        (lambda: m.mla8_kvfile_append(p, codes, scales, 4, 1, LC, RC), m.MLA8_E_RANGE),
        (lambda: m.mla8_kvfile_append(p, codes, scales, 6, 1, LC, RC), m.MLA8_E_RANGE),
        # shadows as wide as the call's lc + rc, so that the library sees the call
        (lambda: m.mla8_kvfile_append(p, *shadows(2, 10, LC + 32), 5, 1, LC, 32),
         m.MLA8_E_INVAL),
        (lambda: m.mla8_kvfile_append(p, codes[:1], scales[:1], 5, 1, LC, RC), m.MLA8_E_INVAL),
        (lambda: m.mla8_kvfile_append(p, *shadows(2, 10, 72 + RC), 5, 1, 72, RC),
         m.MLA8_E_UNSUPPORTED),
        (lambda: m.mla8_kvfile_load(p, *shadows(2, 4, D), LC, RC), m.MLA8_E_CAPACITY),
        (lambda: m.mla8_kvfile_load(str(tmp_path / "missing"), *shadows(2, 9, D), LC, RC),
         m.MLA8_E_IO),
        (lambda: m.mla8_kvfile_create(str(tmp_path / "e"), 0, LC, RC), m.MLA8_E_INVAL),
    ]
    for call, want in cases:
        with pytest.raises(m.Mla8Error) as e:
            call()
        assert e.value.status == want
    # buffers narrower than the call's rows never reach the library
    with pytest.raises(ValueError, match="shape"):
        m.mla8_kvfile_append(p, codes, scales, 5, 1, LC, 32)
    with pytest.raises(ValueError, match="outside"):
        m.mla8_kvfile_append(p, codes, scales, 5, 6, LC, RC)
    assert m.mla8_kvfile_info(p)["n_tokens"] == 5
    # a capacity refusal leaves the shadows untouched
    c2, s2 = shadows(2, 4, D)
    with pytest.raises(m.Mla8Error):
        m.mla8_kvfile_load(p, c2, s2, LC, RC)
    assert not any(c.any() for c in c2)


def test_crash_between_body_and_header(tmp_path):
    # an append that wrote its tokens but crashed before the header commit
    g = np.random.Generator(np.random.PCG64(8))
    p = str(tmp_path / "f.mla8kv")
    codes, scales = random_rows(g, 2, 30, D)
    m.mla8_kvfile_create(p, 2, LC, RC)
    m.mla8_kvfile_append(p, codes, scales, 0, 20, LC, RC)
    with open(p, "ab") as f:
        f.write(g.integers(0, 256, 2 * (D + 4) * 5, dtype=np.uint8).tobytes())
    c2, s2 = shadows(2, 30, D)
    assert m.mla8_kvfile_load(p, c2, s2, LC, RC) == 20
    np.testing.assert_array_equal(c2[1][:20], codes[1][:20])
    # appending again from the committed end overwrites the torn bytes
    m.mla8_kvfile_append(p, codes, scales, 20, 10, LC, RC)
    hdr, fc, fs = read_file(p)
    assert hdr[4] == 30
    np.testing.assert_array_equal(fc[0], codes[0])


def test_torn_header_falls_back_to_the_previous_commit(tmp_path):
    g = np.random.Generator(np.random.PCG64(9))
    p = str(tmp_path / "g.mla8kv")
    codes, scales = random_rows(g, 1, 12, D)
    m.mla8_kvfile_create(p, 1, LC, RC)
    m.mla8_kvfile_append(p, codes, scales, 0, 8, LC, RC)   # seq 1, slot B
    m.mla8_kvfile_append(p, codes, scales, 8, 4, LC, RC)   # seq 2, slot A
    raw = bytearray(open(p, "rb").read())
    assert struct.unpack("<Q", raw[32:40])[0] == 2
    raw[30] ^= 0xFF  # tear the newest slot (A)
    open(p, "wb").write(bytes(raw))
    assert m.mla8_kvfile_info(p)["n_tokens"] == 8
    c2, s2 = shadows(1, 12, D)
    assert m.mla8_kvfile_load(p, c2, s2, LC, RC) == 8
    np.testing.assert_array_equal(c2[0][:8], codes[0][:8])
    raw[64 + 5] ^= 0x01  # and the other one
    open(p, "wb").write(bytes(raw))
    with pytest.raises(m.Mla8Error) as e:
        m.mla8_kvfile_info(p)
    assert e.value.status == m.MLA8_E_IO


def test_version1_file_needs_device_shadows(tmp_path):
    g = np.random.Generator(np.random.PCG64(10))
    p = str(tmp_path / "h.mla8kv")
    rows = [g.standard_normal((6, D)).astype(np.float32)]
    write_file(p, 1, rows, LC, RC)
    assert m.mla8_kvfile_info(p)["version"] == 1
    with pytest.raises(m.Mla8Error) as e:
        m.mla8_kvfile_load(p, *shadows(1, 6, D), LC, RC)
    assert e.value.status == m.MLA8_E_UNSUPPORTED
    hdr, r, _ = read_file(p)
    np.testing.assert_array_equal(r[0], rows[0])


def test_symbols_exported():
    for name in ("mla8_kvfile_create", "mla8_kvfile_info", "mla8_kvfile_append",
                 "mla8_kvfile_load"):
        assert hasattr(m.lib, name)
    assert m.lib.mla8_status_string(m.MLA8_E_IO)


def test_unusable_headers_are_refused(tmp_path):
    """A slot whose check matches but whose token count is absurd (2^63, which
    an int64 cast would make negative) or larger than the body holds is not
    used; an older slot that the body does hold is used instead."""
    g = np.random.Generator(np.random.PCG64(11))
    codes, scales = random_rows(g, 1, 6, D)
    p = str(tmp_path / "h.mla8kv")
    write_file(p, 2, list(zip(codes, scales)), LC, RC)
    raw = bytearray(open(p, "rb").read())
    for bad_n in (1 << 63, (1 << 64) - 1, 1 << 31, 7):
        raw[:64] = slot_bytes(2, 1, LC, RC, bad_n, 5)
        raw[64:128] = b"\0" * 64
        open(p, "wb").write(bytes(raw))
        with pytest.raises(m.Mla8Error) as e:
            m.mla8_kvfile_info(p)
        assert e.value.status == m.MLA8_E_IO, bad_n
        c2, s2 = shadows(1, 8, D)
        t = None
        with pytest.raises(m.Mla8Error) as e:
            t = m.mla8_kvfile_load(p, c2, s2, LC, RC)
        assert e.value.status == m.MLA8_E_IO and t is None
    # newest slot claims more tokens than the body holds; the older one fits
    raw[:64] = slot_bytes(2, 1, LC, RC, 9, 5)
    raw[64:128] = slot_bytes(2, 1, LC, RC, 4, 4)
    open(p, "wb").write(bytes(raw))
    assert m.mla8_kvfile_info(p)["n_tokens"] == 4
    c2, s2 = shadows(1, 8, D)
    assert m.mla8_kvfile_load(p, c2, s2, LC, RC) == 4
    np.testing.assert_array_equal(c2[0][:4], codes[0][:4])


@pytest.mark.parametrize("what", ["nan_code_pos", "nan_code_neg", "nan_scale", "neg_scale",
                                  "inf_scale"])
def test_corrupt_body_is_not_loaded(tmp_path, what):
    g = np.random.Generator(np.random.PCG64(12))
    codes, scales = random_rows(g, 2, 6, D)
    p = str(tmp_path / "i.mla8kv")
    if what == "nan_code_pos":
        codes[1][3, 17] = 0x7F
    elif what == "nan_code_neg":
        codes[0][5, 0] = 0xFF
    elif what == "nan_scale":
        scales[1][2] = np.float32("nan")
    elif what == "neg_scale":
        scales[0][1] = np.float32(-0.5)
    else:
        scales[1][4] = np.float32("inf")
    write_file(p, 2, list(zip(codes, scales)), LC, RC)
    c2, s2 = shadows(2, 8, D)
    with pytest.raises(m.Mla8Error) as e:
        m.mla8_kvfile_load(p, c2, s2, LC, RC)
    assert e.value.status == m.MLA8_E_IO
    assert m.mla8_kvfile_info(p)["n_tokens"] == 6  # the header itself is fine
