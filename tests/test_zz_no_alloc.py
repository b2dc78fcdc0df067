"""coli_moe_forward_noalloc: the forward with the library's static per-GPU
scratch in place of a workspace, for callers that cannot allocate.  Checked
through the C ABI against coli_moe_forward on the same inputs: same kernels,
so bit-identical outputs, on consecutive calls with a shrinking batch (the
scratch keeps the previous call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import LayerPair
from quantized_moe_coli_amd import binding as B
from quantized_moe_coli_amd import inputs

pytestmark = pytest.mark.gpu


def _forward_ws(p, x, lg=None):
    T = x.shape[0]
    s = p.s
    y = torch.empty(T, s.hidden, device="cuda")
    idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, s.top_k, device="cuda")
    ws = B.workspace(p.gpu, T)
    B.coli_moe_forward(p.gpu, x, y, ws, logits_in=lg, idx_out=idx, w_out=w)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _forward_noalloc(p, x, lg=None):
    T = x.shape[0]
    s = p.s
    y = torch.full((T, s.hidden), float("nan"), device="cuda")
    idx = torch.full((T, s.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, s.top_k), float("nan"), device="cuda")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    B.coli_moe_forward_noalloc(p.gpu, x, y, logits_in=lg, idx_out=idx, w_out=w,
                               wait_status_out=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.fixture(scope="module")
def layers():
    assert torch.cuda.is_available()
    return {
        "int8": LayerPair(inputs.TINY, seed=0),
        "grouped_int4": LayerPair(inputs.TINY.with_(n_group=4, topk_group=2, top_k=4,
                                                    bias_std=0.05, bits=4), seed=0),
    }


@pytest.mark.parametrize("name", ["int8", "grouped_int4"])
@pytest.mark.parametrize("sizes", [(40, 3), (5, 1), (1, 1), (70, 9)])
def test_noalloc_matches_forward(layers, name, sizes):
    """Two calls in a row, the second with fewer tokens: each equals
    coli_moe_forward on a workspace of its own, bit for bit."""
    p = layers[name]
    for i, T in enumerate(sizes):
        x = inputs.tokens(p.s, 0, 9000 + 10 * T + i, T).cuda()
        ref = _forward_ws(p, x)
        got = _forward_noalloc(p, x)
        for u, v in zip(got, ref):
            np.testing.assert_array_equal(u, v)


def test_noalloc_supplied_logits_and_glm_decode():
    """Supplied logits on the small layer, then single-token decode and a
    3-token batch of the full GLM-5.2 layer (the single-kernel decode uses
    the scratch's header, which must be back at zero after each call)."""
    p = LayerPair(inputs.TINY.with_(n_group=4, topk_group=2, top_k=4, bias_std=0.05, bits=4),
                  seed=1)
    x = inputs.tokens(p.s, 0, 3, 6).cuda()
    lg = inputs.correlated_logits(4, 6, p.s.n_experts, 0.3).cuda()
    for u, v in zip(_forward_noalloc(p, x, lg), _forward_ws(p, x, lg)):
        np.testing.assert_array_equal(u, v)
    g = LayerPair(inputs.GLM, seed=2, device_gen=True)
    for i, T in enumerate((3, 1, 1)):
        x = inputs.tokens(g.s, 0, 60 + i, T, "cuda")
        for u, v in zip(_forward_noalloc(g, x), _forward_ws(g, x)):
            np.testing.assert_array_equal(u, v)


def test_noalloc_rejects_oversize_batch():
    """A batch whose workspace exceeds the static scratch is refused with
    COLI_ERR_UNSUPPORTED before anything is enqueued; the next call works."""
    p = LayerPair(inputs.GLM.with_(n_experts=16, top_k=4, n_group=4, topk_group=2), seed=3,
                  device_gen=True)
    need = B.coli_moe_workspace_bytes(p.gpu, 512)
    assert need > B.NOALLOC_SCRATCH_BYTES
    x = inputs.tokens(p.s, 0, 1, 512, "cuda")
    y = torch.full((512, p.s.hidden), 3.0, device="cuda")
    with pytest.raises(B.ColiError) as ei:
        B.coli_moe_forward_noalloc(p.gpu, x, y)
    assert ei.value.status == B.COLI_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (y == 3.0).all()
    x1 = x[:2].contiguous()
    for u, v in zip(_forward_noalloc(p, x1), _forward_ws(p, x1)):
        np.testing.assert_array_equal(u, v)
