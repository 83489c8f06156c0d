"""The device code as compiled for gfx950 with the build's flags (hipcc
cross-compiles without a GPU): no kernel spills registers to scratch
memory. Spills are silent -- results stay right, the kernels slow down --
and the attention kernel's register budget (wavefronts per SIMD) sits at
the edge of the register file, so a change that tips it over is caught here."""
import shutil

import pytest

from kv_cache_quantization_tq_amd import build as B


@pytest.mark.skipif(shutil.which(B.hipcc()) is None, reason="hipcc not available")
def test_no_kernel_spills_registers():
    res = B.kernel_resources()
    assert len(res) > 200, len(res)
    spilled = {k: v for k, v in res.items() if v["scratch"] > 0}
    assert not spilled, spilled
    attn = [v for k, v in res.items() if "attn_partial_kernel" in k]
    assert len(attn) == 120
