"""GPU test of moe_permute_noalloc, the permute whose histogram table lives in the
library's static device scratch instead of a caller workspace: through the C ABI, its
outputs equal moe_permute's bit for bit (and the oracle's layout) on two calls in a row,
the second one smaller, so stale scratch contents of the first call must not leak into
the second; and with every output buffer supplied the call allocates no device memory."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_amd as rpg
import workloads as W
from oracle import moe_oracle as orc
from tests import _parity as P

pytestmark = pytest.mark.gpu

KEYS = ("x_perm", "counts", "offsets", "dst_row", "src_row", "tile_expert", "dev_err")


def _case(T, D, E, k, seed):
    cfg = W.shrink(W.preset("fine64_shared2_bf16"), T=T, D=D, E=E, k=k, F=128, n_shared=0)
    inp = W.generate(cfg, seed=seed)
    idx, _, _ = orc.route(inp["x"], inp["wg"], k, "bf16")
    idx[::7, 0] = -1   # slots handled elsewhere
    return inp, idx


def _poisoned_out(T, D, E, k, mt, m_cap):
    i32 = dict(dtype=torch.int32, device="cuda")
    return {"x_perm": P.poison(torch.empty((m_cap, D), dtype=torch.bfloat16, device="cuda")),
            "counts": torch.full((E,), -7, **i32), "offsets": torch.full((E + 1,), -7, **i32),
            "dst_row": torch.full((T, k), -7, **i32), "src_row": torch.full((m_cap,), -7, **i32),
            "tile_expert": torch.full((m_cap // mt,), -7, **i32),
            "dev_err": torch.full((1,), -7, **i32)}


def _host(o, used):
    h = {kk: P.to_host(o[kk]) for kk in KEYS}
    h["x_perm"] = h["x_perm"][:used]
    return h


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_permute_equals_the_workspace_permute(order):
    cases = [(3000, 256, 64, 6, 128, 1), (500, 128, 8, 2, 16, 2)]
    if order == "small_then_large":
        cases = cases[::-1]
    for T, D, E, k, mt, seed in cases:
        P.log(f"[noalloc] T={T} D={D} E={E} k={k} m_tile={mt}")
        inp, idx = _case(T, D, E, k, seed)
        x, di = P.to_dev(inp["x"]), P.to_dev(idx)
        m_cap = rpg.moe_capacity(T, k, E, mt)
        a = rpg.moe_permute(x, di, E, mt, m_cap=m_cap, out=_poisoned_out(T, D, E, k, mt, m_cap))
        b = rpg.moe_permute_noalloc(x, di, E, mt, m_cap=m_cap,
                                    out=_poisoned_out(T, D, E, k, mt, m_cap))
        torch.cuda.synchronize()
        lay = orc.dispatch_layout(idx, E, mt, m_cap)
        used = int(lay["offsets"][-1])
        ha, hb = _host(a, used), _host(b, used)
        for kk in KEYS:
            np.testing.assert_array_equal(hb[kk], ha[kk], err_msg=kk)
        for kk in ("counts", "offsets", "dst_row", "src_row", "tile_expert"):
            np.testing.assert_array_equal(hb[kk], lay[kk], err_msg=kk)
        np.testing.assert_array_equal(hb["x_perm"], orc.permute(inp["x"], lay)[:used])
        assert int(hb["dev_err"][0]) == 0


def test_noalloc_permute_allocates_nothing_with_outputs_given():
    T, D, E, k, mt = 700, 128, 16, 4, 128
    inp, idx = _case(T, D, E, k, 5)
    x, di = P.to_dev(inp["x"]), P.to_dev(idx)
    m_cap = rpg.moe_capacity(T, k, E, mt)
    out = _poisoned_out(T, D, E, k, mt, m_cap)
    rpg.moe_permute_noalloc(x, di, E, mt, m_cap=m_cap, out=out)   # first call on the device
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rpg.moe_permute_noalloc(x, di, E, mt, m_cap=m_cap, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    lay = orc.dispatch_layout(idx, E, mt, m_cap)
    np.testing.assert_array_equal(P.to_host(out["dst_row"]), lay["dst_row"])
