"""GPU parity: the HIP codec (called through the C ABI) against the CPU oracle
on the same seeded inputs. Expected values come from the oracle only; the
decode checks feed the GPU the oracle's planes, so both sides decode the
same bytes."""
import numpy as np
import pytest

import oracle as O
from kv_cache_quantization_tq_amd import workloads as W
from tests import parity as P

torch = pytest.importorskip("torch")
import kv_cache_quantization_tq_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu

KMODES = [(2, False), (3, False), (4, False), (5, False), (8, False), (8, True)]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def special_rows(rows: int, d: int, seed: int) -> np.ndarray:
    """[rows, 1, d] float32 N(0,1) rows with edge cases planted in the first ones."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, 1, d)).astype(np.float32)
    if rows > 10:
        x[0] = 0.5                                   # constant: fp16 zero point overflows
        x[1] = 0.0                                   # zero row
        x[2] *= np.float32(1e4)                      # large values
        x[3] = 0.0
        x[3, 0, 5] = 1.0                             # one-hot
        x[4, 0, ::2] = -0.0                          # signed zeros mixed in
        x[4, 0, :32] = np.where(np.arange(32) % 3 == 0, -0.0, 0.0)
        x[5] = np.float32(1e25)                      # constant huge block: IEEE-division path for keys
        x[5, 0, 40:] += np.float32(1e18) * rng.standard_normal(d - 40).astype(np.float32)
        x[6] *= np.float32(1e31)                     # squares overflow: value scale = inf
        x[7] *= np.float32(1e-41)                    # subnormal inputs
        x[8] = np.round(x[8] * 4) / 4                # values on a coarse grid (ties)
        x[9] *= np.float32(3e-5)
    return x


def run_encode(k, v, d, vb, kb, ks):
    planes = tq.encode_kv(k, v, v_bits=vb, k_bits=kb, k_signed=ks)
    torch.cuda.synchronize()
    return P.host_planes(planes)


def check_case(dev, x_k, x_v, d, vb, kb, ks, dtype, tag):
    """Encode on GPU and oracle, compare; decode the oracle planes on GPU in
    bf16, f32 and rotated modes and compare with the oracle's decode."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    k = torch.from_numpy(x_k).to(dev, tdt)
    v = torch.from_numpy(x_v).to(dev, tdt)
    kn, vn = W.to_oracle(k), W.to_oracle(v)
    rows = kn.shape[0] * kn.shape[1]
    say(f"[case] {tag} encode rows={rows}")
    got = run_encode(k, v, d, vb, kb, ks)
    want = O.encode_kv(kn, vn, head_dim=d, k_bits=kb, v_bits=vb, k_signed=ks)
    P.assert_key_planes_equal(got, want, tag)
    P.assert_value_planes_match(got, want, P.rows_as_f32(vn), d, vb, tag)
    dp = P.device_planes(want, dev)
    for out_dt, odt in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        for rot in (False, True):
            say(f"[case] {tag} decode {odt} rotated={rot}")
            ko, vo = tq.decode_kv(dp, tokens=kn.shape[0], heads=kn.shape[1], head_dim=d, v_bits=vb, k_bits=kb,
                                  k_signed=ks, out_dtype=out_dt, rotated_v=rot)
            torch.cuda.synchronize()
            wk, wv = O.decode_kv(want, rows=rows, head_dim=d, k_bits=kb, v_bits=vb, k_signed=ks,
                                 out_dtype=odt, rotated_v=rot)
            P.assert_decoded_close(P.decoded_to_f32(ko), P.oracle_decoded_f32(wk), f"{tag} K {odt}")
            P.assert_decoded_close(P.decoded_to_f32(vo), P.oracle_decoded_f32(wv), f"{tag} V {odt} rot={rot}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("vb", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_all_configurations_small(dev, d, vb, dtype):
    """Every head_dim x value bits x key mode x dtype, on 37 tokens x 3 heads
    (ragged against every rows-per-wavefront) plus planted edge rows."""
    for i, (kb, ks) in enumerate(KMODES):
        xk = special_rows(111, d, seed=1000 * d + 10 * vb + i).reshape(37, 3, d)
        xv = special_rows(111, d, seed=7 + 1000 * d + 10 * vb + i).reshape(37, 3, d)
        check_case(dev, xk, xv, d, vb, kb, ks, dtype, f"d={d} vb={vb} kb={kb} ks={ks} {dtype}")


@pytest.mark.parametrize("rows", [1, 2, 15, 16, 17, 63, 64, 65, 257])
def test_ragged_row_counts(dev, rows):
    for d in (64, 512):
        x = special_rows(rows, d, seed=rows).reshape(rows, 1, d)
        check_case(dev, x, x[::-1].copy(), d, 4, 4, False, "bf16", f"rows={rows} d={d}")


def test_empty_is_a_noop(dev):
    k = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=dev)
    planes = tq.encode_kv(k, k, v_bits=4, k_bits=4)
    ko, vo = tq.decode_kv(planes, tokens=0, heads=2, head_dim=128, v_bits=4, k_bits=4)
    torch.cuda.synchronize()
    assert ko.numel() == 0 and vo.numel() == 0


def test_one_side_only(dev):
    x = special_rows(40, 128, seed=3).reshape(20, 2, 128)
    k = torch.from_numpy(x).to(dev, torch.bfloat16)
    want = O.encode_kv(W.to_oracle(k), W.to_oracle(k), head_dim=128, k_bits=5, v_bits=3)
    pk = P.host_planes(tq.encode_kv(k, None, v_bits=3, k_bits=5))
    pv = P.host_planes(tq.encode_kv(None, k, v_bits=3, k_bits=5))
    torch.cuda.synchronize()
    assert set(pk) == {"k_codes", "k_scale", "k_zero"} and set(pv) == {"v_codes", "v_scale"}
    P.assert_key_planes_equal(pk, want, "K only")
    P.assert_value_planes_match(pv, want, P.rows_as_f32(W.to_oracle(k)), 128, 3, "V only")
    dp = P.device_planes(want, dev)
    ko, vo = tq.decode_kv(dp, tokens=20, heads=2, head_dim=128, v_bits=3, k_bits=5, values=False)
    assert vo is None
    wk, _ = O.decode_kv(want, rows=40, head_dim=128, k_bits=5, v_bits=3, values=False)
    P.assert_decoded_close(P.decoded_to_f32(ko), P.oracle_decoded_f32(wk), "K only decode")


def test_append_at_token_offset(dev):
    """Encoding tokens [t0, t1) into planes advanced by t0 rows writes the same
    bytes as encoding the whole tensor (groups never cross a row)."""
    w = W.scaled(W.WORKLOADS["long_decode"], 96)
    k, v = W.make_kv(w, dev)
    full = tq.encode_kv(k, v, v_bits=5, k_bits=4)
    part = tq.empty_planes(96 * 8, 256, 4, 5, dev)
    for t0, t1 in ((0, 50), (50, 51), (51, 96)):
        view = {n: p[t0 * 8:t1 * 8] for n, p in part.items()}
        tq.encode_kv(k[t0:t1], v[t0:t1], v_bits=5, k_bits=4, out=view)
    torch.cuda.synchronize()
    for n in full:
        assert torch.equal(full[n], part[n]), n


def test_deterministic(dev):
    w = W.scaled(W.WORKLOADS["prefill"], 2048)
    k, v = W.make_kv(w, dev)
    a = P.host_planes(tq.encode_kv(k, v, v_bits=4, k_bits=4))
    b = P.host_planes(tq.encode_kv(k, v, v_bits=4, k_bits=4))
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    dp = P.device_planes(a, dev)
    ko1, vo1 = tq.decode_kv(dp, tokens=2048, heads=8, head_dim=128, v_bits=4, k_bits=4)
    ko2, vo2 = tq.decode_kv(dp, tokens=2048, heads=8, head_dim=128, v_bits=4, k_bits=4)
    assert torch.equal(ko1.view(torch.int16), ko2.view(torch.int16))
    assert torch.equal(vo1.view(torch.int16), vo2.view(torch.int16))


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unrotate_values(dev, d, dtype):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((333, d)).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    xt = torch.from_numpy(x).to(dev, tdt)
    out = tq.unrotate_values(xt)
    torch.cuda.synchronize()
    want = O.unrotate(W.to_oracle(xt), d)
    P.assert_decoded_close(P.decoded_to_f32(out), P.oracle_decoded_f32(want), f"unrotate d={d} {dtype}")


def test_deferred_v_linearity(dev):
    """Attention is linear in V: un-rotating a weighted sum of rotated-domain
    values equals the weighted sum of fully decoded values (up to rounding)."""
    d, vb = 256, 3
    x = special_rows(512, d, seed=5)[16:].reshape(124, 4, d)
    v = torch.from_numpy(x).to(dev, torch.float32)
    planes = tq.encode_kv(None, v, v_bits=vb, k_bits=8)
    _, rot = tq.decode_kv(planes, tokens=124, heads=4, head_dim=d, v_bits=vb, k_bits=8, keys=False,
                          rotated_v=True, out_dtype=torch.float32)
    _, full = tq.decode_kv(planes, tokens=124, heads=4, head_dim=d, v_bits=vb, k_bits=8, keys=False,
                           out_dtype=torch.float32)
    wts = torch.softmax(torch.randn(7, 124, generator=torch.Generator().manual_seed(0)), dim=-1).to(dev)
    att_rot = (wts @ rot.reshape(124, -1)).reshape(7, 4, d).contiguous()
    att_full = (wts @ full.reshape(124, -1)).reshape(7, 4, d)
    un = tq.unrotate_values(att_rot)
    torch.cuda.synchronize()
    scale = float(att_full.abs().max())
    assert float((un - att_full).abs().max()) <= 1e-5 * max(scale, 1.0)


# ------------------------------------------------------------ workloads

def encode_full_and_check(dev, w, sample_rows=None):
    """GPU encode of the whole workload; oracle parity on all rows or on a
    seeded sample. Returns GPU planes (device), inputs and checked row ids."""
    say(f"[workload] {w.name} generate")
    k, v = W.make_kv(w, dev)
    R, d = w.rows, w.head_dim
    say(f"[workload] {w.name} gpu encode rows={R}")
    planes = tq.encode_kv(k, v, v_bits=w.v_bits, k_bits=w.k_bits, k_signed=w.k_signed)
    torch.cuda.synchronize()
    if sample_rows is None:
        idx = np.arange(R)
    else:
        rng = np.random.default_rng(w.seed + 99)
        idx = np.unique(np.concatenate([rng.choice(R, sample_rows, replace=False), [0, R - 1]]))
        if w.kind == "gauss_zero_rows":
            z = torch.nonzero((k.view(R, d) == 0).all(dim=1)).flatten()[:256].cpu().numpy()
            idx = np.unique(np.concatenate([idx, z]))
    it = torch.from_numpy(idx).to(dev)
    kn = W.to_oracle(k.view(R, d)[it])
    vn = W.to_oracle(v.view(R, d)[it])
    got = {n: P.host_planes({n: p[it]})[n] for n, p in planes.items()}
    say(f"[workload] {w.name} oracle encode rows={idx.size}")
    want = O.encode_kv(kn, vn, head_dim=d, k_bits=w.k_bits, v_bits=w.v_bits, k_signed=w.k_signed)
    P.assert_key_planes_equal(got, want, w.name)
    P.assert_value_planes_match(got, want, P.rows_as_f32(vn), d, w.v_bits, w.name)
    return k, v, planes, idx, want


def decode_full_and_check(dev, w, planes, idx, want, tokens=None):
    """Overwrite the checked rows with the oracle's planes, decode the whole
    cache in one launch, compare those rows with the oracle's decode."""
    d = w.head_dim
    tokens = w.kv_tokens if tokens is None else tokens
    it = torch.from_numpy(idx).to(dev)
    for n, a in P.device_planes(want, dev).items():
        planes[n][it] = a
    say(f"[workload] {w.name} gpu decode tokens={tokens}")
    ko, vo = tq.decode_kv(planes, tokens=tokens, heads=w.heads, head_dim=d, v_bits=w.v_bits, k_bits=w.k_bits,
                          k_signed=w.k_signed)
    torch.cuda.synchronize()
    R = tokens * w.heads
    gk = P.decoded_to_f32(ko.view(R, d)[it])
    gv = P.decoded_to_f32(vo.view(R, d)[it])
    say(f"[workload] {w.name} oracle decode rows={idx.size}")
    wk, wv = O.decode_kv(want, rows=idx.size, head_dim=d, k_bits=w.k_bits, v_bits=w.v_bits, k_signed=w.k_signed)
    P.assert_decoded_close(gk, P.oracle_decoded_f32(wk), f"{w.name} K")
    P.assert_decoded_close(gv, P.oracle_decoded_f32(wv), f"{w.name} V")
    return ko, vo


def test_workload_tiny(dev):
    w = W.WORKLOADS["tiny"]
    k, v, planes, idx, want = encode_full_and_check(dev, w)
    assert (want["k_zero"][7] == 0x7C00).all()
    ko, vo = decode_full_and_check(dev, w, planes, idx, want)
    assert torch.isnan(ko[7].float()).all()


def test_workload_prefill_full(dev):
    w = W.WORKLOADS["prefill"]
    k, v, planes, idx, want = encode_full_and_check(dev, w)
    decode_full_and_check(dev, w, planes, idx, want)


def test_workload_small_head_full(dev):
    w = W.WORKLOADS["small_head"]
    k, v, planes, idx, want = encode_full_and_check(dev, w)
    decode_full_and_check(dev, w, planes, idx, want)


def test_workload_long_decode_append(dev):
    w = W.WORKLOADS["long_decode"]
    T, H, d = w.tokens, w.heads, w.head_dim
    k, v, planes0, idx, want = encode_full_and_check(dev, w, sample_rows=8192)
    steps = 2
    planes = tq.empty_planes((T + steps) * H, d, w.k_bits, w.v_bits, dev)
    for n in planes:
        planes[n][: T * H] = planes0[n]
    del planes0
    for s in range(steps):
        nk, nv = W.append_token(w, s, dev)
        view = {n: p[(T + s) * H:(T + s + 1) * H] for n, p in planes.items()}
        say(f"[workload] long_decode append step {s}")
        tq.encode_kv(nk, nv, v_bits=w.v_bits, k_bits=w.k_bits, out=view)
        torch.cuda.synchronize()
        wa = O.encode_kv(W.to_oracle(nk), W.to_oracle(nv), head_dim=d, k_bits=w.k_bits, v_bits=w.v_bits)
        ga = P.host_planes(view)
        P.assert_key_planes_equal(ga, wa, f"append {s}")
        P.assert_value_planes_match(ga, wa, P.rows_as_f32(W.to_oracle(nv)), d, w.v_bits, f"append {s}")
        rows_new = np.arange((T + s) * H, (T + s + 1) * H)
        idx = np.concatenate([idx, rows_new])
        want = {n: np.concatenate([want[n], wa[n]]) for n in want}
        decode_full_and_check(dev, w, planes, idx, want, tokens=T + s + 1)


def test_workload_joint_large(dev):
    w = W.WORKLOADS["joint_large"]
    k, v, planes, idx, want = encode_full_and_check(dev, w, sample_rows=4096)
    R, d = w.rows, w.head_dim
    nz = int((k.view(R, d) == 0).all(dim=1).sum())
    assert nz == int(round(0.01 * R))
    del k, v
    decode_full_and_check(dev, w, planes, idx, want)
