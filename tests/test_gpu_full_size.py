"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times: every integer output compared bit for bit with the oracle, x_perm bit for bit,
and the float outputs of sampled tokens (the oracle computes a token's rows one by
one: a row's expert output depends on that row alone)."""
import numpy as np
import pytest

import workloads as W
from oracle import moe_oracle as orc
from tests import _parity as P

pytestmark = pytest.mark.gpu

FULL = ["dense8_bf16", "fine64_shared2_bf16", "skew32_zipf_bf16", "etp_shard32_bf16"]
SAMPLED_TOKENS = 12


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    cfg = W.preset(name)
    P.log(f"[full] {name}: generating inputs")
    inp = W.generate(cfg, seed=0)
    cfg = inp["cfg"]
    T, E, k, mt, dt = cfg.T, cfg.E, cfg.k, cfg.m_tile, cfg.dtype
    P.log(f"[full] {name}: T={T} running the HIP path")
    g = P.run_gpu(inp, k, mt)
    P.log(f"[full] {name}: oracle routing and layout")
    if "topk_idx" in inp:
        idx, w = inp["topk_idx"], inp["topk_w"].astype(np.float64)
        np.testing.assert_array_equal(g["topk_idx"], idx)
    else:
        idx, w, logits = orc.route(inp["x"], inp["wg"], k, dt, inp.get("bias"))
        np.testing.assert_array_equal(g["logits"].view(np.uint32), logits.view(np.uint32))
        np.testing.assert_array_equal(g["topk_idx"], idx)
        np.testing.assert_allclose(g["topk_w"], w, rtol=P.W_RTOL, atol=0)
    lay = orc.dispatch_layout(idx, E, mt)
    for key in ("counts", "offsets", "dst_row", "src_row", "tile_expert"):
        np.testing.assert_array_equal(g[key], lay[key], err_msg=key)
    assert int(g["dev_err"][0]) == 0
    used = int(lay["offsets"][-1])
    xp = orc.permute(inp["x"], lay)
    np.testing.assert_array_equal(g["x_perm"][:used], xp[:used])
    del xp
    pad = lay["src_row"][:used] < 0
    for key in ("h", "y_perm"):
        v = g[key][:used]
        assert np.all(v[pad] == 0), f"{key}: pad rows not zero"
        assert np.all(np.isfinite(orc.values64(v[~pad][:: max(1, used // 4096)])))
    P.log(f"[full] {name}: oracle on {SAMPLED_TOKENS} sampled tokens")
    toks = np.sort(np.random.default_rng(123).choice(T, SAMPLED_TOKENS, replace=False))
    shared = (inp["ws1"], inp["ws3"], inp["ws2"]) if "ws1" in inp else None
    out, hs, ys = orc.token_outputs(toks, inp["x"], idx, w, inp["w1"], inp["w3"], inp["w2"], dt,
                                    shared)
    rows = [lay["dst_row"][t, j] for (t, j) in hs]
    eh = P.rel_err(g["h"][rows], np.stack(list(hs.values())))
    ey = P.rel_err(g["y_perm"][rows], np.stack(list(ys.values())))
    eo = P.rel_err(g["out"][toks], out)
    P.log(f"[full] {name}: rel err h {eh:.2e} y {ey:.2e} out {eo:.2e}")
    tol = P.TOL[dt]
    assert eh <= tol and ey <= tol and eo <= tol
