"""q8_moe_grouped_linear_noalloc (the mixture on the library's fixed device scratch, no
allocation) against q8_moe_grouped_linear (caller workspace): bit-identical outputs on
consecutive calls, the second with fewer tokens, so the scratch keeps the first call's
contents when the second runs."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as wl
from gpu_util import say, to_dev, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q8():
    torch, dev = torch_dev()
    import block_quantized_weight_linear_amd as q8mod
    return q8mod, torch, dev


def _experts(seed, e, f, h):
    gu = np.concatenate([wl.q8_weight(seed + i, 2 * f, h)[0] for i in range(e)])
    dn = np.concatenate([wl.q8_weight(seed + 1000 + i, h, f)[0] for i in range(e)])
    return gu, dn


@pytest.mark.parametrize("e,f,h,k,m1,m2", [(128, 768, 2048, 8, 16, 5), (16, 256, 512, 4, 40, 1),
                                           (8, 512, 256, 2, 300, 17)])
def test_noalloc_matches_workspace_call(q8, e, f, h, k, m1, m2):
    lib, torch, dev = q8
    distinct = min(e, 8)
    gu_h, dn_h = _experts(1100 + e, distinct, f, h)
    gu = to_dev(np.concatenate([gu_h] * (e // distinct)), dev)
    dn = to_dev(np.concatenate([dn_h] * (e // distinct)), dev)
    wr = to_dev(wl.router_weight(1101, e, h, 0.05), dev)
    for m in (m1, m2):
        say(f"noalloc mixture e={e} f={f} h={h} k={k} m={m}")
        x = to_dev(wl.activations(1102 + m, m, h), dev)
        idx, w = lib.moe_route_topk(x, wr, k, True)
        want = lib.q8_moe_grouped_linear(gu, dn, e, f, h, x, idx, w)
        out = torch.full((m, h), float("nan"), device=dev)
        got = lib.q8_moe_grouped_linear_noalloc(gu, dn, e, f, h, x, idx, w, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, want), (m, float((got - want).abs().max()))


def test_noalloc_refuses_oversize(q8):
    lib, torch, dev = q8
    e, f, h, k, m = 128, 768, 2048, 8, 200  # 1600 routed pairs: more than the scratch holds
    gu = torch.zeros(e * 2 * f * (h // 32) * 34, dtype=torch.uint8, device=dev)
    dn = torch.zeros(e * h * (f // 32) * 34, dtype=torch.uint8, device=dev)
    x = torch.zeros((m, h), device=dev)
    idx = torch.zeros((m, k), dtype=torch.int32, device=dev)
    w = torch.zeros((m, k), device=dev)
    with pytest.raises(lib.Q8Error):
        lib.q8_moe_grouped_linear_noalloc(gu, dn, e, f, h, x, idx, w)
