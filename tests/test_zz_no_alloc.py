"""kq_qmm_noalloc: the library's fixed scratch array in place of a caller
workspace.  Through the C ABI, two calls in a row (the second smaller, so it
runs on what the first left in the array) must give the same bits as
kq_qmm_ws with a workspace of its own, and agree with the oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TAU, check_tol, empty, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kq():
    from block_quantized_weight_q4_amd import _build, kq as mod

    _build.build_if_missing()
    mod.lib()
    return mod


def _say(*a):
    print("[case]", *a, flush=True)


def _ws_result(kq, kind, w, n, k, x, m, y_dt):
    nb = kq.kq_qmm_workspace_bytes(kind, n, k, m, x.dtype)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=x.device)
    y = empty((m, n), y_dt)
    kq.kq_qmm_ws(kind, w, n, k, x, m, y, ws)
    return y, nb


# (kind, n, k, m, x dtype): the first uses the activation pre-pass and eight
# K splits (about 20 MB of scratch), the second two splits and fp16 rows, the
# third the split-K TQ1 decode product of one row (four pieces, 4.8 KB)
CASES = [("q4_k", 1024, 4096, 512, "bf16"), ("q8_0", 300, 1024, 40, "f16"),
         ("tq1_g128", 300, 8192, 1, "f16")]


def test_noalloc_matches_workspace_twice(kq):
    assert kq.kq_qmm_noalloc_max_bytes() == 64 << 20
    outs = []
    for i, (kind, n, k, m, x_dt) in enumerate(CASES):
        rng = synth.rng_for(4000 + i)
        w = synth.weight_blocks(kind, rng, n, k)
        x = synth.activations(rng, (m, k), x_dt)
        wd, xd = to_dev(w), to_dev(x, x_dt)
        ref_y, nb = _ws_result(kq, kind, wd, n, k, xd, m, "f32")
        assert 0 < nb <= kq.kq_qmm_noalloc_max_bytes()
        _say("noalloc", kind, n, k, m, x_dt, nb)
        y = empty((m, n), "f32")
        kq.kq_qmm_noalloc(kind, wd, n, k, xd, m, y)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref_y.cpu().numpy().view(np.uint32))
        outs.append((kind, w, n, k, x, x_dt, m, to_f64(y)))
    # all against the oracle (the first on sampled outputs)
    for i in (1, 2):
        kind, w, n, k, x, x_dt, m, got = outs[i]
        ref, s = oracle.qmm(kind, w, n, k, x, x_dt, m)
        check_tol(got, ref, s, TAU[x_dt], f"noalloc call {i + 1}")
    kind, w, n, k, x, x_dt, m, got = outs[0]
    rng = np.random.default_rng(1)
    pm, pn = rng.integers(0, m, 500), rng.integers(0, n, 500)
    ref, s = oracle.qmm_points(kind, w, n, k, x, x_dt, m, pm, pn)
    check_tol(got[pm, pn], ref, s, TAU[x_dt], "noalloc first call")


def test_noalloc_rejects_products_past_its_scratch(kq):
    """8192 x 8192 bf16 activations need 128 MiB of converted rows: refused
    before anything is launched; decode shapes need no scratch at all."""
    n, k, m = 256, 8192, 8192
    assert kq.kq_qmm_workspace_bytes("q4_k", n, k, m, torch.bfloat16) > kq.kq_qmm_noalloc_max_bytes()
    dev = torch.device("cuda:0")
    w = torch.zeros(n * (k // 256) * 144, dtype=torch.uint8, device=dev)
    x = torch.zeros((m, k), dtype=torch.bfloat16, device=dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    with pytest.raises(kq.KQError) as e:
        kq.kq_qmm_noalloc("q4_k", w, n, k, x, m, y)
    assert e.value.status == 3
    # m <= 16: the decode kernels, no scratch
    y8 = empty((8, n), "f32")
    kq.kq_qmm_noalloc("q4_k", w, n, k, x[:8], 8, y8)
    torch.cuda.synchronize()
    assert np.all(to_f64(y8) == 0.0)
