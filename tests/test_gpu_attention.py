"""GPU parity of attention over the packed cache (tq_attention_decode
through the C ABI) against the binary64 attention oracle on the codec
oracle's decoded rows. The cache planes come from the codec oracle's
encoder; q from seeded numpy.

Tolerance: decoding is exact (both sides use the same bf16 rows). The two
contractions run on the matrix cores with binary32 accumulation; the
binary32 query and softmax weights enter as three bf16 terms, which
represent them to about 2^-25 relative, so the arithmetic is that of
binary32. A score carries an absolute error of at most about
d * 2^-24 * scale * sum_i |q_i k_i| (dot products of d terms), which
perturbs the weights p relatively by the same amount; the weighted sums
add at most ~(tiles + splits) * 2^-24 relative to max |v|. For the inputs
here (|q|, |k| ~ N(0,1) rows, scale 1/sqrt(d)) that is below 1e-5 of
max |v| (measured: below 2e-7 absolute at max |v| ~ 4); the bar is
2e-5 * max|v| per element."""
import math

import numpy as np
import pytest
import torch

import kv_cache_quantization_tq_amd as tq
import oracle as O
from oracle import attention as A

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()
    return torch.device("cuda:0")


def to_dev(planes, dev):
    return {n: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev) for n, a in planes.items()}


def case(dev, *, d, kb, vb, ks=False, g=1, hkv=2, batch=1, width=700, pads=None, seed=0, q_bf16=False,
         out_bf16=False, scale=None, kscale=1.0, zero_key_rows=()):
    print(f"[attention] d={d} k{kb}{'s' if ks else ''} v{vb} g={g} hkv={hkv} batch={batch} width={width} "
          f"pads={pads} q_bf16={q_bf16} out_bf16={out_bf16} zero_key_rows={len(zero_key_rows)}", flush=True)
    rng = np.random.default_rng(seed)
    rows = batch * width * hkv
    k = (rng.standard_normal((rows, d)) * kscale).astype(np.float32)
    k[list(zero_key_rows)] = 0.0
    v = rng.standard_normal((rows, d)).astype(np.float32)
    planes = O.encode_kv(k, v, head_dim=d, k_bits=kb, v_bits=vb, k_signed=ks)
    q = rng.standard_normal((batch, hkv * g, d)).astype(np.float32)
    if q_bf16:
        q = (np.round(q.view(np.uint32) / 65536.0).astype(np.uint32) << 16).view(np.float32)  # any bf16 values
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    kd, vr = A.decoded_cache(planes, rows, d, kb, vb, ks)
    want = A.attention_decode(q.astype(np.float64), kd, vr, batch, width, pads, hkv, np.float64(np.float32(sc)))
    qt = torch.from_numpy(q).to(dev)
    if q_bf16:
        qt = qt.to(torch.bfloat16)
    lp = None if pads is None else torch.tensor(pads, dtype=torch.int32, device=dev)
    got = tq.attention_decode(qt, to_dev(planes, dev), batch=batch, width=width, kv_heads=hkv, head_dim=d,
                              k_bits=kb, v_bits=vb, k_signed=ks, left_pad=lp, scale=sc,
                              out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    vmax = float(np.abs(vr).max()) if vr.size else 1.0
    err = float(np.abs(got - want).max()) if got.size else 0.0
    print(f"    max |err| = {err:.3e}  (max |v| = {vmax:.3f})", flush=True)
    if out_bf16:
        # the output's own rounding to bf16 (2^-9 relative) on top
        assert np.all(np.abs(got - want) <= 2e-5 * vmax + 2 ** -8 * np.abs(want))
    else:
        assert err <= 2e-5 * vmax, err
    return err


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_head_dims_and_groups(dev, d, g):
    case(dev, d=d, kb=4, vb=4, g=g, seed=d + g)


@pytest.mark.parametrize("kb,vb,ks", [(2, 2, False), (3, 3, False), (5, 5, False), (8, 8, False), (8, 3, True)])
def test_bit_widths(dev, kb, vb, ks):
    case(dev, d=128, kb=kb, vb=vb, ks=ks, g=4, seed=10 * kb + vb)


@pytest.mark.parametrize("vb", [3, 5])
def test_value_windows_off_byte_boundaries(dev, vb):
    # at d = 64 a lane's window of 4 odd-width codes starts inside a byte and
    # the lanes differ in how many words it spans
    case(dev, d=64, kb=4, vb=vb, g=4, width=1000, seed=20 + vb)


@pytest.mark.parametrize("kb,ks", [(4, False), (8, True)])
def test_zero_key_groups_take_the_two_step_decode(dev, kb, ks):
    # all-zero key rows give groups of scale 0, for which the fused
    # multiply-add form of the key decode does not apply: a run of 16 tokens
    # of one KV head and scattered single rows of the other
    hkv, width = 2, 700
    rows = [(t * hkv) for t in range(32, 48)] + [t * hkv + 1 for t in (5, 100, 333, 699)]
    case(dev, d=256, kb=kb, vb=5, ks=ks, g=4, hkv=hkv, width=width, seed=30 + kb, zero_key_rows=rows)


def test_left_padded_batch_with_an_empty_sequence(dev):
    case(dev, d=128, kb=4, vb=4, g=2, batch=4, width=700, pads=[0, 300, 699, 700], seed=3)


def test_many_chunks_and_dtypes(dev):
    case(dev, d=256, kb=4, vb=5, g=4, width=5000, seed=4, q_bf16=True)
    case(dev, d=128, kb=4, vb=4, g=4, width=1300, seed=5, out_bf16=True)
    case(dev, d=64, kb=8, vb=2, ks=True, g=8, width=2100, seed=6, scale=0.05)


@pytest.mark.parametrize("d,g", [(512, 8), (64, 1)])
def test_bf16_query_at_the_extreme_head_dims(dev, d, g):
    # the block copies the group's query rows 8 elements per thread: three
    # such steps per thread at d = 512, one at d = 64
    case(dev, d=d, kb=4, vb=8 if d == 512 else 3, g=g, width=900, seed=40 + g, q_bf16=True)


def test_empty_cache_gives_zeros(dev):
    q = torch.randn(2, 4, 128, device=dev)
    planes = tq.empty_planes(0, 128, 4, 4, dev)
    out = tq.attention_decode(q, planes, batch=2, width=0, kv_heads=2, head_dim=128, k_bits=4, v_bits=4)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_full_size_bench_configuration(dev):
    """The bench's attention workload at its full size and launch
    configuration (131072 tokens x 8 KV heads, d 256, V5/K4, 32 bf16 query
    heads, default scale): the same seeded K/V and query as the bench, the
    cache encoded by the codec oracle on the CPU, three query heads (of KV
    heads 0, 3 and 7) compared with the binary64 oracle."""
    from kv_cache_quantization_tq_amd import workloads as W
    w = W.WORKLOADS["long_decode"]
    T, H, d, hq = w.tokens, w.heads, w.head_dim, 32
    print(f"[attention] full size: {T} tokens x {H} KV heads, d={d}, v{w.v_bits}/k{w.k_bits}, {hq} query heads",
          flush=True)
    k, v = W.make_kv(w, dev)
    kh = k.reshape(T * H, d).cpu().numpy()
    vh = v.reshape(T * H, d).cpu().numpy()
    del k, v
    planes = O.encode_kv(kh, vh, head_dim=d, k_bits=w.k_bits, v_bits=w.v_bits)
    del kh, vh
    print("    oracle planes encoded", flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    q = torch.randn((1, hq, d), generator=g, device=dev).to(torch.bfloat16)
    got = tq.attention_decode(q, to_dev(planes, dev), batch=1, width=T, kv_heads=H, head_dim=d, k_bits=w.k_bits,
                              v_bits=w.v_bits)
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    qn = q.float().cpu().numpy().astype(np.float64)
    sc = np.float64(np.float32(1.0 / math.sqrt(d)))
    for h in (0, 13, 31):
        j = h // (hq // H)
        rows = np.arange(T) * H + j
        kd, vr = A.decoded_cache({n: a[rows] for n, a in planes.items()}, T, d, w.k_bits, w.v_bits)
        want = A.attention_decode(qn[:, h:h + 1, :], kd, vr, 1, T, None, 1, sc)[0, 0]
        vmax = float(np.abs(vr).max())
        err = float(np.abs(got[0, h] - want).max())
        print(f"    head {h} (KV head {j}): max |err| = {err:.3e} (max |v| = {vmax:.3f})", flush=True)
        assert err <= 2e-5 * vmax, (h, err)
