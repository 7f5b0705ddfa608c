"""The batch-1 decode kernel's bounded waits and their report.

Every device-side wait of the one-kernel decode is bounded; one that runs out
sets an error bit and lets its workgroup finish, so the kernel always ends,
and moe_workspace_check reports MOE_ERR_DEVICE. Here the host shrinks the
bound (moe_debug_set_wait_limit) so that the waits give up while their
producers are still running: every workgroup still exits normally (no
fault, no hang), the check reports the time-out once, and the next calls
with the default bound are clean and match the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import check_routing, check_y, from_dev_bits, log, routing_scale, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_expert_ffn_gemv_amd import moe as m
    m.lib()
    return m


def test_wait_limit_reports_and_recovers(moe):
    host = synth.make_layer("decode_q4", threads=16)
    L = moe.DeviceLayer(host)
    x = synth.make_tokens("decode_q4", T=8)
    xd = to_dev(x)
    y = torch.empty_like(xd)
    idx = torch.empty((8, L.k), dtype=torch.int32, device="cuda")
    ws = moe.make_workspace(L, 1, 0)
    try:
        log("decode with a 1-tick wait bound: the waits give up, the kernels end")
        moe.debug_set_wait_limit(1)
        for t in range(4):
            moe.moe_forward_decode(L, xd[t:t + 1], y[t:t + 1], ws)
        torch.cuda.synchronize()
    finally:
        moe.debug_set_wait_limit(0)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_check(ws)
    assert ei.value.status == moe.MOE_ERR_DEVICE
    moe.moe_workspace_check(ws)  # the report was cleared
    log("default bound again: clean calls that match the oracle")
    for t in range(8):
        moe.moe_forward_decode(L, xd[t:t + 1], y[t:t + 1], ws, topk_idx=idx[t:t + 1])
    torch.cuda.synchronize()
    moe.moe_workspace_check(ws)
    y_ref, idx_ref, _ = oracle.moe_forward(host, x)
    _, _, logits = oracle.route(host, x)
    check_routing(idx.cpu().numpy(), idx_ref, logits, "after the time-out", scale=routing_scale(host, x))
    check_y(from_dev_bits(y), y_ref, "after the time-out")
