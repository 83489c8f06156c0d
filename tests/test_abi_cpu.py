"""CPU tests of the HIP library's host side: it loads, exports every symbol
the header declares, validates arguments before any launch, and its
tables and host-compiled bin search agree with the printed tables and the
oracle. No compute call is made (there is no GPU here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import kv_cache_quantization_tq_amd as tq
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

pytestmark = pytest.mark.skipif(not os.path.exists(tq.LIB_PATH), reason="libtq.so not built")

FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(tq.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", tq.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)", out))
    for n in names:
        assert n in exported, n
        getattr(tq.lib(), n)


def test_packed_dim():
    for d in (64, 128, 256, 512):
        for b in (2, 3, 4, 5, 8):
            assert tq.packed_dim(d, b) == O.packed_dim(d, b) == d * b // 8
    assert tq.lib().tq_packed_dim(3, 3) == -tq.TQ_E_ALIGN
    assert tq.lib().tq_packed_dim(7, 5) == -tq.TQ_E_ALIGN
    assert tq.lib().tq_packed_dim(64, 9) == -tq.TQ_E_BITS
    assert tq.lib().tq_packed_dim(0, 4) == -tq.TQ_E_BITS


def test_status_strings():
    for s in range(10):
        assert isinstance(tq.status_string(s), str) and tq.status_string(s)
        assert tq.status_string(s) != "unknown status"
    assert tq.status_string(99) == "unknown status"


def test_time_next_call_needs_a_stop_event_with_a_start_event():
    L = tq.lib()
    assert L.tq_time_next_call(FAKE, None) == tq.TQ_E_NULL
    assert L.tq_time_next_call(None, FAKE) == tq.TQ_OK
    assert L.tq_time_next_call(None, None) == tq.TQ_OK
    # arming stores the handles only; a call failing validation disarms
    # without touching them
    assert L.tq_time_next_call(FAKE, FAKE + 64) == tq.TQ_OK
    assert _enc(cfg=(100, 4, 4, 0)) == tq.TQ_E_HEAD_DIM
    assert L.tq_time_next_call(None, None) == tq.TQ_OK


def _enc(k=FAKE, v=FAKE, dtype=tq.TQ_BF16, tokens=16, heads=2, cfg=(128, 4, 4, 0), planes=None):
    planes = planes if planes is not None else [FAKE] * 5
    c = tq.TQConfig(*cfg) if cfg is not None else None
    p = tq.TQPackedKV(*planes)
    return tq.lib().tq_encode_kv(k, v, dtype, tokens, heads, ctypes.byref(c) if c else None, ctypes.byref(p), None)


def _dec(kout=FAKE, vout=FAKE, dtype=tq.TQ_BF16, tokens=16, heads=2, cfg=(128, 4, 4, 0), planes=None, flags=0):
    planes = planes if planes is not None else [FAKE] * 5
    c = tq.TQConfig(*cfg)
    p = tq.TQPackedKV(*planes)
    return tq.lib().tq_decode_kv(ctypes.byref(p), tokens, heads, ctypes.byref(c), kout, vout, dtype, flags, None)


def test_encode_argument_validation():
    assert _enc(cfg=None) == tq.TQ_E_NULL
    assert _enc(k=None, v=None) == tq.TQ_E_NULL
    for d in (0, 32, 96, 100, 1024):
        assert _enc(cfg=(d, 4, 4, 0)) == tq.TQ_E_HEAD_DIM
    for b in (0, 1, 6, 7, 9, 16):
        assert _enc(cfg=(128, b, 4, 0)) == tq.TQ_E_BITS
        assert _enc(cfg=(128, 4, b, 0)) == tq.TQ_E_BITS
    assert _enc(cfg=(128, 4, 4, 1)) == tq.TQ_E_BITS          # signed keys need 8 bits
    assert _enc(cfg=(128, 8, 4, 2)) == tq.TQ_E_BITS
    assert _enc(dtype=2) == tq.TQ_E_DTYPE
    assert _enc(tokens=-1) == tq.TQ_E_SHAPE
    assert _enc(heads=0) == tq.TQ_E_SHAPE
    assert _enc(planes=[None, FAKE, FAKE, FAKE, FAKE]) == tq.TQ_E_NULL
    assert _enc(planes=[FAKE, FAKE, FAKE, None, FAKE]) == tq.TQ_E_NULL
    assert _enc(k=FAKE + 8) == tq.TQ_E_ALIGN
    assert _enc(planes=[FAKE + 8, FAKE, FAKE, FAKE, FAKE]) == tq.TQ_E_ALIGN  # 4-bit codes need 16 B
    assert _enc(planes=[FAKE, FAKE + 1, FAKE, FAKE, FAKE]) == tq.TQ_E_ALIGN
    # the value side's bits and planes are not checked when only keys are encoded
    # (tokens=0 keeps the call from launching)
    assert _enc(v=None, cfg=(128, 4, 7, 0), planes=[FAKE, FAKE, FAKE, None, None], tokens=0) == tq.TQ_OK
    # zero tokens is a no-op that launches nothing and reads no pointer
    assert _enc(tokens=0) == tq.TQ_OK
    assert _enc(k=None, v=None, tokens=0, planes=[None] * 5) == tq.TQ_OK


def test_decode_argument_validation():
    assert _dec(kout=None, vout=None) == tq.TQ_E_NULL
    assert _dec(cfg=(48, 4, 4, 0)) == tq.TQ_E_HEAD_DIM
    assert _dec(cfg=(128, 4, 6, 0)) == tq.TQ_E_BITS
    assert _dec(cfg=(128, 4, 4, 1)) == tq.TQ_E_BITS
    assert _dec(dtype=7) == tq.TQ_E_DTYPE
    assert _dec(flags=4) == tq.TQ_E_SHAPE
    assert _dec(tokens=-5) == tq.TQ_E_SHAPE
    assert _dec(vout=FAKE + 4) == tq.TQ_E_ALIGN
    assert _dec(planes=[FAKE, FAKE, FAKE, None, FAKE]) == tq.TQ_E_NULL
    assert _dec(tokens=0) == tq.TQ_OK
    assert _dec(kout=None, vout=None, tokens=0, planes=[None] * 5) == tq.TQ_OK


def test_unrotate_argument_validation():
    L = tq.lib()
    assert L.tq_unrotate_values(None, FAKE, 0, 4, 128, None) == tq.TQ_E_NULL
    assert L.tq_unrotate_values(None, None, 0, 0, 128, None) == tq.TQ_OK
    assert L.tq_unrotate_values(FAKE, FAKE, 0, 4, 100, None) == tq.TQ_E_HEAD_DIM
    assert L.tq_unrotate_values(FAKE, FAKE, 3, 4, 128, None) == tq.TQ_E_DTYPE
    assert L.tq_unrotate_values(FAKE, FAKE, 0, -1, 128, None) == tq.TQ_E_SHAPE
    assert L.tq_unrotate_values(FAKE + 4, FAKE, 0, 4, 128, None) == tq.TQ_E_ALIGN
    assert L.tq_unrotate_values(FAKE, FAKE, 0, 0, 128, None) == tq.TQ_OK


def test_library_tables_match_printed_text():
    lm = {}
    for ln in open(os.path.join(GOLDEN, "lloyd_max.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        head, v = ln.split(":")
        b, kind = head.split()
        lm.setdefault(int(b), {})[kind] = np.array([np.float32(float(x)) for x in v.split()])
    for b, t in lm.items():
        c, bd = tq.lloyd_max_table(b)
        np.testing.assert_array_equal(c, t["centroids"])
        np.testing.assert_array_equal(bd, t["boundaries"])
    for ln in open(os.path.join(GOLDEN, "sign_vectors.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        d, v = ln.split(":")
        np.testing.assert_array_equal(tq.sign_vector(int(d)), np.array([float(x) for x in v.split()], np.float32))
    with pytest.raises(tq.TQError):
        tq.lloyd_max_table(6)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_kernel_bin_search_equals_oracle_count(bits):
    """The kernels' grid-table bin search (host build of the same code) gives
    exactly the oracle's count of boundaries below z, on a dense grid, at
    every boundary and its neighbouring floats, and at extremes."""
    c, bd = O.lloyd_max(bits)
    rng = np.random.default_rng(bits)
    z = [np.linspace(-7, 7, 200001, dtype=np.float32), bd,
         np.nextafter(bd, np.float32(np.inf)), np.nextafter(bd, np.float32(-np.inf)),
         np.nextafter(np.nextafter(bd, np.float32(np.inf)), np.float32(np.inf)),
         rng.standard_normal(100000).astype(np.float32) * np.float32(1.5),
         np.array([0.0, -0.0, 1e-40, -1e-40, 1e30, -1e30, np.inf, -np.inf, 3.4e38, -3.4e38], np.float32)]
    # every float in a window around each boundary
    for b in bd:
        u = np.float32(b).view(np.int32)
        z.append(np.arange(u - 300, u + 300, dtype=np.int32).view(np.float32))
    z = np.concatenate(z)
    z = z[~np.isnan(z)]
    np.testing.assert_array_equal(tq.value_bin_host(bits, z), O.bin_index(z, bits))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_kernel_bin_search_stays_in_its_table_for_nan(bits):
    """NaN inputs are outside the method (their bins are unspecified), but
    the bin search is the encoder's only data-dependent address (a table
    lookup): for NaN of either sign and any payload it must still give an
    index inside the table. The kernels run this general search for every
    group whose sum of squares is not finite, which any NaN or infinity in
    the group makes it."""
    payloads = np.array([0x7FC00000, 0x7F800001, 0x7FFFFFFF, 0xFFC00000, 0xFF800001, 0xFFFFFFFF, 0x7FA5A5A5],
                        np.uint32)
    z = payloads.view(np.float32)
    assert np.isnan(z).all()
    idx = tq.value_bin_host(bits, z)
    assert idx.dtype == np.uint8 and (idx.astype(np.int64) <= (1 << bits) - 1).all()


def test_kernel_quotient_equals_ieee_division():
    """The quotient the kernels take for key scales, zero points and codes
    (host build of the same code) equals IEEE binary32 division bit for bit,
    the sign of zero included, over the range where the kernels use it
    (divisor in [1e-8, 1e30), |a * RN(1/b)| < 1e30, quotient not subnormal):
    random operands over wide exponents, the constant divisors of the key
    scales, divisors one ulp around powers of two, and signed zeros."""
    rng = np.random.default_rng(77)
    n = 400000

    def wide(k, lo, hi):
        m = rng.uniform(1.0, 2.0, k)
        e = rng.integers(lo, hi, k)
        return (np.ldexp(m, e) * rng.choice([-1.0, 1.0], k)).astype(np.float32)

    a = [wide(n, -60, 60), np.zeros(1000, np.float32), -np.zeros(1000, np.float32)]
    b = [np.abs(wide(n, -26, 99)), np.abs(wide(2000, -20, 20))]
    a = np.concatenate(a)
    b = np.concatenate([np.resize(np.concatenate(b), a.size)])
    # constant divisors of the key scales and divisors next to powers of two
    consts = np.array([3, 7, 15, 31, 255, 254], np.float32)
    p2 = np.ldexp(np.ones(80), np.arange(-26, 54)).astype(np.float32)
    near = np.concatenate([p2, np.nextafter(p2, np.float32(0)), np.nextafter(p2, np.float32(np.inf))])
    hard_b = np.concatenate([consts, near])
    hard_a = wide(hard_b.size * 64, -20, 20)
    a = np.concatenate([a, hard_a, np.nextafter(hard_a, np.float32(0))])
    b = np.concatenate([b, np.repeat(hard_b, 64), np.repeat(hard_b, 64)])
    r = (np.float32(1.0) / b).astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        want = (a / b).astype(np.float32)
        ar = np.abs(a.astype(np.float64) * r.astype(np.float64))
    keep = (b >= np.float32(1e-8)) & (b < np.float32(1e30)) & (ar < 1e30) & \
        ((np.abs(want) >= np.float32(2.0 ** -126)) | (a == 0))
    a, b, want = a[keep], b[keep], want[keep]
    assert a.size > 300000
    got = tq.quotient_host(a, b)
    bad = got.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), (int(bad.sum()), a[bad][:3], b[bad][:3])
    assert np.signbit(got[a == 0]).sum() == np.signbit(a[a == 0]).sum() > 0


def _pk(vals):
    return tq.TQPackedKV(*vals)


def test_batching_argument_validation():
    L = tq.lib()
    cfg = tq.TQConfig(128, 4, 4, 0)
    dst = _pk([FAKE] * 5)
    srcs = (tq.TQPackedKV * 2)(_pk([FAKE] * 5), _pk([FAKE] * 5))
    lens = (ctypes.c_int64 * 2)(3, 5)
    by = ctypes.byref
    # merge
    assert L.tq_merge_rows(srcs, lens, 2, 4, 2, by(cfg), by(dst), None, None) == tq.TQ_E_SHAPE   # width < len
    assert L.tq_merge_rows(srcs, lens, -1, 5, 2, by(cfg), by(dst), None, None) == tq.TQ_E_SHAPE
    assert L.tq_merge_rows(srcs, lens, 0, 5, 2, by(cfg), by(dst), None, None) == tq.TQ_OK       # nothing to do
    assert L.tq_merge_rows(srcs, lens, 2, 5, 0, by(cfg), by(dst), None, None) == tq.TQ_E_SHAPE   # heads
    assert L.tq_merge_rows(srcs, lens, 2, 5, 2, by(tq.TQConfig(96, 4, 4, 0)), by(dst), None, None) == tq.TQ_E_HEAD_DIM
    assert L.tq_merge_rows(srcs, lens, 2, 5, 2, by(tq.TQConfig(128, 6, 4, 0)), by(dst), None, None) == tq.TQ_E_BITS
    # values only: the key bits are not checked
    vdst = _pk([None, None, None, FAKE, FAKE])
    assert L.tq_merge_rows(srcs, lens, 0, 5, 2, by(tq.TQConfig(128, 6, 4, 0)), by(vdst), None, None) == tq.TQ_OK
    assert L.tq_merge_rows(srcs, lens, 2, 5, 2, by(cfg), by(_pk([None] * 5)), None, None) == tq.TQ_E_NULL
    nsrcs = (tq.TQPackedKV * 2)(_pk([FAKE] * 5), _pk([FAKE, FAKE, None, FAKE, FAKE]))
    assert L.tq_merge_rows(nsrcs, lens, 2, 5, 2, by(cfg), by(dst), None, None) == tq.TQ_E_NULL
    # extend
    row = _pk([FAKE] * 5)
    pin = (ctypes.c_int64 * 2)(0, 2)
    pout = (ctypes.c_int64 * 3)()
    assert L.tq_extend_rows(by(dst), 2, 5, pin, by(row), 7, 6, 2, by(cfg), by(dst), pout, None) == tq.TQ_E_SHAPE
    assert L.tq_extend_rows(by(dst), 2, 5, None, by(row), 3, 5, 2, by(cfg), by(dst), pout, None) == tq.TQ_E_NULL
    assert L.tq_extend_rows(by(dst), -1, 5, pin, by(row), 3, 5, 2, by(cfg), by(dst), pout, None) == tq.TQ_E_SHAPE
    # extract
    assert L.tq_extract_row(by(dst), 2, 5, 2, 0, 2, by(cfg), by(dst), None) == tq.TQ_E_SHAPE    # i >= b
    assert L.tq_extract_row(by(dst), 2, 5, 0, 6, 2, by(cfg), by(dst), None) == tq.TQ_E_SHAPE    # pad > width
    assert L.tq_extract_row(by(dst), 0, 5, 0, 0, 2, by(cfg), by(dst), None) == tq.TQ_E_SHAPE
    # filter
    keep = (ctypes.c_int32 * 2)(0, 2)
    assert L.tq_filter_rows(by(dst), 2, 5, keep, 2, 2, by(cfg), by(dst), None) == tq.TQ_E_SHAPE  # keep[1] >= b
    assert L.tq_filter_rows(by(dst), 2, 5, None, 2, 2, by(cfg), by(dst), None) == tq.TQ_E_NULL
    assert L.tq_filter_rows(by(dst), 2, 5, None, 0, 2, by(cfg), by(dst), None) == tq.TQ_OK


def test_batching_segments_stay_inside_their_planes():
    """Every copy segment a batching call builds is checked against the
    extents of its source and destination planes (in tokens, from the call's
    arguments) before anything is launched: one outside returns TQ_E_SHAPE.
    Without a GPU the launch itself fails (TQ_E_HIP), so reaching it means
    every segment of the call passed. Driven here with the merge of 32
    caches that the bench times (three launches of segments), and extend,
    extract and filter shapes around it; plane pointers are never
    dereferenced on the host."""
    import numpy as np
    from kv_cache_quantization_tq_amd import workloads as W
    L = tq.lib()
    by = ctypes.byref
    m = W.MERGE
    lens = W.merge_lengths()
    n, width, H = len(lens), max(lens), m["heads"]
    cfg = tq.TQConfig(m["head_dim"], m["k_bits"], m["v_bits"], 0)
    srcs = (tq.TQPackedKV * n)(*[_pk([FAKE + 4096 * i] * 5) for i in range(n)])
    lens_a = np.asarray(lens, dtype=np.int64)
    dst = _pk([FAKE] * 5)
    pads = np.zeros(n, dtype=np.int64)
    assert L.tq_merge_rows(srcs, lens_a.ctypes.data, n, width, H, by(cfg), by(dst), pads.ctypes.data,
                           None) == tq.TQ_E_HIP
    # ragged shapes: empty, full and one-token sequences; values-only planes
    for ls in ([0, 1, 7], [5, 5, 5], [1], [0, 0, 3]):
        la = np.asarray(ls, dtype=np.int64)
        ss = (tq.TQPackedKV * len(ls))(*[_pk([FAKE] * 5) for _ in ls])
        for d in (dst, _pk([None, None, None, FAKE, FAKE])):
            assert L.tq_merge_rows(ss, la.ctypes.data, len(ls), max(ls), 2, by(cfg), by(d), None,
                                   None) == tq.TQ_E_HIP, ls
    pin = (ctypes.c_int64 * 3)(0, 2, 5)
    pout = (ctypes.c_int64 * 4)()
    row = _pk([FAKE] * 5)
    for b, w, rl, nw in ((3, 5, 5, 5), (3, 5, 2, 9), (0, 0, 4, 4), (3, 5, 0, 6)):
        assert L.tq_extend_rows(by(dst), b, w, pin, by(row), rl, nw, 2, by(cfg), by(dst), pout,
                                None) == tq.TQ_E_HIP, (b, w, rl, nw)
    for i, pad in ((0, 0), (2, 4), (1, 3)):
        assert L.tq_extract_row(by(dst), 3, 5, i, pad, 2, by(cfg), by(dst), None) == tq.TQ_E_HIP
    keep = (ctypes.c_int32 * 4)(2, 0, 2, 1)
    assert L.tq_filter_rows(by(dst), 3, 5, keep, 4, 2, by(cfg), by(dst), None) == tq.TQ_E_HIP


def test_lloyd_fit_argument_validation():
    import numpy as np
    L = tq.lib()
    ws = int(L.tq_lloyd_max_workspace_bytes(10))
    assert L.tq_lloyd_max_workspace_bytes(0) == -tq.TQ_E_SHAPE
    assert L.tq_lloyd_max_workspace_bytes(1 << 31) == -tq.TQ_E_SHAPE
    # the sorted keys (two buffers) and the prefix sums: at least 16 bytes a sample
    assert L.tq_lloyd_max_workspace_bytes(1 << 20) >= 16 << 20
    assert L.tq_lloyd_max_workspace_bytes(1 << 24) > L.tq_lloyd_max_workspace_bytes(1 << 20)
    assert ws > 256 * 8 * 4
    init = np.linspace(-1, 1, 4)
    c = np.zeros(4)
    b = np.zeros(3)
    ip, cp, bp = init.ctypes.data, c.ctypes.data, b.ctypes.data
    assert L.tq_lloyd_max_fit(FAKE, 10, 1, ip, 5, cp, bp, FAKE, ws, None) == tq.TQ_E_BITS
    assert L.tq_lloyd_max_fit(FAKE, 10, 257, ip, 5, cp, bp, FAKE, ws, None) == tq.TQ_E_BITS
    assert L.tq_lloyd_max_fit(FAKE, 0, 4, ip, 5, cp, bp, FAKE, ws, None) == tq.TQ_E_SHAPE
    assert L.tq_lloyd_max_fit(FAKE, 10, 4, ip, -1, cp, bp, FAKE, ws, None) == tq.TQ_E_SHAPE
    assert L.tq_lloyd_max_fit(None, 10, 4, ip, 5, cp, bp, FAKE, ws, None) == tq.TQ_E_NULL
    assert L.tq_lloyd_max_fit(FAKE, 10, 4, None, 5, cp, bp, FAKE, ws, None) == tq.TQ_E_NULL
    assert L.tq_lloyd_max_fit(FAKE, 10, 4, ip, 5, cp, bp, None, ws, None) == tq.TQ_E_NULL
    assert L.tq_lloyd_max_fit(FAKE, 10, 4, ip, 5, cp, bp, FAKE, ws - 1, None) == tq.TQ_E_SHAPE
    assert L.tq_lloyd_max_fit(FAKE + 2, 10, 4, ip, 5, cp, bp, FAKE, ws, None) == tq.TQ_E_ALIGN
    assert L.tq_lloyd_max_fit(FAKE, 10, 4, ip, 5, cp, bp, FAKE + 4, ws, None) == tq.TQ_E_ALIGN
    bad = np.array([-1.0, 0.0, 0.0, 1.0])   # not strictly ascending
    assert L.tq_lloyd_max_fit(FAKE, 10, 4, bad.ctypes.data, 5, cp, bp, FAKE, ws, None) == tq.TQ_E_SHAPE


def test_attention_argument_validation():
    L = tq.lib()
    cfg = tq.TQConfig(128, 4, 4, 0)
    pk = _pk([FAKE] * 5)
    by = ctypes.byref
    ws = int(L.tq_attention_workspace_bytes(2, 2, 8, 128, 1000))
    # 1000 tokens, 2 x 2 (sequence, KV head) pairs: at most ceil(1000 / 128) = 8 splits
    assert ws == 2 * 8 * 8 * (128 + 4) * 4  # 8 splits of (d + 4) floats per output row
    assert L.tq_attention_workspace_bytes(2, 2, 8, 100, 1000) < 0
    assert L.tq_attention_workspace_bytes(2, 2, 8, 128, 0) == 0

    def call(q=FAKE, qd=tq.TQ_F32, batch=2, width=1000, hkv=2, hq=8, c=cfg, scale=0.1, out=FAKE, od=tq.TQ_F32,
             w=FAKE, wb=ws):
        return L.tq_attention_decode(q, qd, by(pk), batch, width, None, hkv, hq, by(c), scale, out, od, w, wb, None)

    assert call(c=tq.TQConfig(96, 4, 4, 0)) == tq.TQ_E_HEAD_DIM
    assert call(c=tq.TQConfig(128, 4, 6, 0)) == tq.TQ_E_BITS
    assert call(qd=5) == tq.TQ_E_DTYPE
    assert call(od=5) == tq.TQ_E_DTYPE
    assert call(hq=7) == tq.TQ_E_SHAPE            # not a multiple of kv heads
    assert call(hq=6, hkv=2) == tq.TQ_E_SHAPE     # 3 query heads per KV head
    assert call(hq=32, hkv=2) == tq.TQ_E_SHAPE    # 16 per KV head
    assert call(scale=float("nan")) == tq.TQ_E_SHAPE
    assert call(batch=-1) == tq.TQ_E_SHAPE
    assert call(batch=0) == tq.TQ_OK
    assert call(q=None) == tq.TQ_E_NULL
    assert call(w=None) == tq.TQ_E_NULL
    assert call(wb=ws - 1) == tq.TQ_E_SHAPE
    assert call(q=FAKE + 4) == tq.TQ_E_ALIGN
    assert call(out=FAKE + 8) == tq.TQ_E_ALIGN
    assert L.tq_attention_decode(FAKE, 0, by(_pk([FAKE, FAKE, None, FAKE, FAKE])), 2, 1000, None, 2, 8, by(cfg),
                                 0.1, FAKE, 0, FAKE, ws, None) == tq.TQ_E_NULL


def test_static_attention_rejects_calls_beyond_its_buffer():
    """tq_attention_decode_static refuses, before any launch or pointer use,
    a call whose split partials would not fit its 64 MiB static buffer, and
    reports argument errors as tq_attention_decode does."""
    L = tq.lib()
    cfg = tq.TQConfig(512, 4, 4, 0)
    need = L.tq_attention_workspace_bytes(4096, 8, 64, 512, 64)
    assert need > 64 << 20
    st = L.tq_attention_decode_static(None, tq.TQ_BF16, None, 4096, 64, None, 8, 64, ctypes.byref(cfg), 0.1,
                                      None, tq.TQ_F32, None)
    assert st == tq.TQ_E_SCRATCH
    assert L.tq_attention_decode_static(None, tq.TQ_BF16, None, 1, 64, None, 8, 64, None, 0.1, None, tq.TQ_F32,
                                        None) == tq.TQ_E_NULL
    bad = tq.TQConfig(96, 4, 4, 0)
    assert L.tq_attention_decode_static(None, tq.TQ_BF16, None, 1, 64, None, 8, 64, ctypes.byref(bad), 0.1, None,
                                        tq.TQ_F32, None) == tq.TQ_E_HEAD_DIM
    # a fitting call with a missing pointer fails its argument check
    assert L.tq_attention_decode_static(None, tq.TQ_BF16, None, 1, 64, None, 8, 64, ctypes.byref(cfg), 0.1, None,
                                        tq.TQ_F32, None) == tq.TQ_E_NULL
