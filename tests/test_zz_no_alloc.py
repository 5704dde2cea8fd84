"""The allocation-free MoE entry point (moe_forward_static, include/moe.h) against moe_forward, the
entry point with a caller workspace that it shares its kernels with: two calls in a row through the
C ABI, the second with fewer tokens than the first, each equal bit for bit to moe_forward on the same
inputs (same kernels, same reduction order), plus the size limit refused before any launch."""
import numpy as np
import pytest

from synth import moe as smoe
from harness import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _inputs(torch, s, n, seed, gu, dn):
    x = smoe.token_rows(s, n, seed).cuda()
    ids, w = smoe.routing(s, n, seed)
    return x, gu, dn, torch.as_tensor(w).cuda(), torch.as_tensor(np.ascontiguousarray(ids, np.int32)).cuda()


def test_static_workspace_equals_caller_workspace(torch_cuda):
    import graph_replay_amd as g
    torch = torch_cuda
    s = smoe.QWEN3_30B_A3B_MOE
    gu, dn = (t.cuda() for t in smoe.make_moe_weights(s, 2400))
    for n, seed in ((64, 2401), (20, 2402)):      # the second call is smaller than the first
        log("moe_forward_static", n, "tokens")
        x, gu_, dn_, w, ids = _inputs(torch, s, n, seed, gu, dn)
        ref = g.moe_forward(x, gu_, dn_, w, ids)
        out = torch.full_like(x, float("nan"))
        g.moe_forward_static(x, gu_, dn_, w, ids, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), n
        assert float(ref.float().abs().max()) > 0
    # a small, ragged shape right after (another expert count and width in the same workspace)
    r = smoe.MoeShape("ragged", 16, 4, 544, 96, "bf16")
    gur, dnr = (t.cuda() for t in smoe.make_moe_weights(r, 2403))
    x, gu_, dn_, w, ids = _inputs(torch, r, 37, 2403, gur, dnr)
    ref = g.moe_forward(x, gu_, dn_, w, ids)
    out = torch.empty_like(x)
    g.moe_forward_static(x, gu_, dn_, w, ids, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_static_workspace_refuses_layers_past_its_size(torch_cuda):
    import graph_replay_amd as g
    torch = torch_cuda
    s = smoe.QWEN3_30B_A3B_MOE
    gu, dn = (t.cuda() for t in smoe.make_moe_weights(s, 2404))
    x, gu_, dn_, w, ids = _inputs(torch, s, 512, 2404, gu, dn)   # needs ~43 MB > 16 MiB
    out = torch.zeros_like(x)
    with pytest.raises(ValueError, match="static workspace"):
        g.moe_forward_static(x, gu_, dn_, w, ids, out)
    torch.cuda.synchronize()
    assert bool((out == 0).all().item())                         # nothing was launched
