"""The codec kernels' tile loop past a wavefront's first tile. With the
default grid (a block for every four tiles) each wavefront takes one tile;
with the grid capped at one block per compute unit (TQ_BLOCKS_PER_CU, read
once per process, so those launches run in a child process) every wavefront
walks several tiles, the decoder's and encoder's later tiles included. The
results must equal the default launch's bit for bit: encoded planes,
decoded K and V (bf16 and rotated) and the un-rotation."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import kv_cache_quantization_tq_amd as tq

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (tokens, heads, head_dim, v_bits, k_bits, k_signed, input dtype): about
# eight tiles per wavefront under the cap (256 compute units x 4
# wavefronts), row counts off the tile size
CASES = [(16383, 8, 128, 4, 4, False, "bf16"), (8191, 32, 64, 2, 8, True, "bf16"),
         (4097, 16, 256, 5, 4, False, "f32")]


def run_cases(out_path):
    """Every case's outputs, as numpy arrays, saved to out_path (.npz)."""
    dev = torch.device("cuda:0")
    res = {}
    for ci, (T, H, d, vb, kb, ks, dt) in enumerate(CASES):
        print(f"[grid-cap] case {ci}: {T} tokens x {H} heads, d={d}, V{vb}/K{kb}{'s' if ks else ''}, {dt}",
              flush=True)
        g = torch.Generator(device=dev)
        g.manual_seed(100 + ci)
        dtype = torch.bfloat16 if dt == "bf16" else torch.float32
        k = torch.randn((T, H, d), generator=g, device=dev).to(dtype)
        v = torch.randn((T, H, d), generator=g, device=dev).to(dtype)
        planes = tq.encode_kv(k, v, v_bits=vb, k_bits=kb, k_signed=ks)
        kw = dict(tokens=T, heads=H, head_dim=d, v_bits=vb, k_bits=kb, k_signed=ks)
        ko, vo = tq.decode_kv(planes, **kw)
        _, vr = tq.decode_kv(planes, keys=False, rotated_v=True, **kw)
        un = tq.unrotate_values(vr.float())
        torch.cuda.synchronize()
        for n, p in planes.items():
            res[f"{ci}_{n}"] = p.cpu().numpy()
        for n, t in (("ko", ko), ("vo", vo), ("vr", vr)):
            res[f"{ci}_{n}"] = t.view(torch.int16).cpu().numpy()
        res[f"{ci}_un"] = un.view(torch.int32).cpu().numpy()
    np.savez(out_path, **res)


def test_capped_grid_walks_several_tiles_per_wavefront(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()
    base = tmp_path / "default.npz"
    run_cases(base)
    capped = tmp_path / "capped.npz"
    env = dict(os.environ, TQ_BLOCKS_PER_CU="1")
    code = (f"import sys; sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r}); "
            f"import test_gpu_grid_cap as m; m.run_cases({str(capped)!r})")
    print("[grid-cap] child process with one block per compute unit", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", code], env=env, cwd=ROOT, timeout=240)
    assert r.returncode == 0, f"child process failed with status {r.returncode}"
    a, b = np.load(base), np.load(capped)
    assert sorted(a.files) == sorted(b.files)
    for n in a.files:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
