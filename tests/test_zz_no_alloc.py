"""moe_forward_decode_noalloc (the library's static scratch array as the
workspace) against moe_forward_decode with a caller workspace, through the C
ABI: the same kernels, so the outputs, expert indices and gates must be
identical, on two calls in a row, the second with fewer tokens."""
import numpy as np
import pytest

import synth
from moe_testlib import from_dev_bits, log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_ffn_gemv_amd import moe as m
    m.lib()
    return m


def _run(m, L, x_bits, noalloc, ws=None):
    B, H = x_bits.shape
    xd = to_dev(x_bits)
    y = torch.empty((B, H), dtype=torch.int16, device="cuda")
    idx = torch.empty((B, L.k), dtype=torch.int32, device="cuda")
    g = torch.empty((B, L.k), dtype=torch.float32, device="cuda")
    if noalloc:
        m.moe_forward_decode_noalloc(L, xd, y, topk_idx=idx, topk_gate=g)
    else:
        m.moe_forward_decode(L, xd, y, ws, topk_idx=idx, topk_gate=g)
    torch.cuda.synchronize()
    return from_dev_bits(y), idx.cpu().numpy(), g.cpu().numpy()


@pytest.mark.parametrize("name", ["decode_q4", "tiny"])
def test_noalloc_matches_workspace_entry_point(moe, name):
    host = synth.make_layer(name, threads=16)
    L = moe.DeviceLayer(host)
    x = synth.make_tokens(name)
    ws = moe.make_workspace(L, 8, 0)
    for B, t0 in ((5, 0), (1, 7), (3, 9)):  # a call, then smaller ones
        log("%s: no-alloc decode of %d token(s) against the workspace entry point" % (name, B))
        xs = x[t0:t0 + B]
        ya, ia, ga = _run(moe, L, xs, True)
        yb, ib, gb = _run(moe, L, xs, False, ws)
        assert np.array_equal(ia, ib), "expert indices differ"
        assert np.array_equal(ga.view(np.uint32), gb.view(np.uint32)), "gates differ"
        assert np.array_equal(ya, yb), "outputs differ"
    moe.moe_workspace_check(ws)


def test_noalloc_rejects_too_large_a_workspace(moe):
    # a layer whose batch-4 workspace exceeds the 32 MiB scratch array (hidden
    # 4096 takes the four-kernel path, whose partials are per slot and token)
    host = synth.random_layer(16, 16, 4096, 512, "q4", "bf16", seed=31, router_sd=0.05)
    L = moe.DeviceLayer(host)
    need = moe.moe_workspace_bytes(L, 4, 0)
    assert need > 32 << 20
    x = synth.normal_bf16(synth.key(31, 1, 1, 1, 1), (4, 4096), 1.0)
    y = torch.empty((4, 4096), dtype=torch.int16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_decode_noalloc(L, to_dev(x), y)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
