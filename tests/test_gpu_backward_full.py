"""GPU parity of the backward at the full workload sizes, in the launch configuration the
benchmark times (split-K workspace on). The oracle computes sampled outputs one by one:
the gradients of a few tokens (dx, the top-k weight gradients and every row their slots
occupy in dy_perm, [da | db] and dX), and a few whole rows of dW1 and dW3 and columns
of dW2 of two experts (the hottest and one other), from that expert's rows only. Routing
and layout come from the oracle and must match the GPU's bit for bit first."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_amd as rpg
import workloads as W
from oracle import moe_oracle as orc
from tests import _parity as P

pytestmark = pytest.mark.gpu

FULL = ["dense8_bf16", "fine64_shared2_bf16", "skew32_zipf_bf16", "etp_shard32_bf16"]
SAMPLED_TOKENS = 6
SAMPLED_COLS = 3


def _host(t: torch.Tensor) -> np.ndarray:
    return P.to_host(t.contiguous())


@pytest.mark.parametrize("name", FULL)
def test_full_size_backward_sampled(name):
    cfg = W.preset(name)
    P.log(f"[bwd-full] {name}: generating inputs")
    inp = W.generate(cfg, seed=0)
    cfg = inp["cfg"]
    T, D, F, E, k, mt, dt = cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, cfg.m_tile, cfg.dtype
    dout = W.output_grad(cfg, seed=0)
    if "topk_idx" in inp:
        idx, w = inp["topk_idx"], inp["topk_w"].astype(np.float64)
    else:
        P.log(f"[bwd-full] {name}: oracle routing")
        idx, w, _ = orc.route(inp["x"], inp["wg"], k, dt, inp.get("bias"))
    lay = orc.dispatch_layout(idx, E, mt)

    P.log(f"[bwd-full] {name}: T={T} forward + backward on the GPU")
    d = {n: P.to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    sw = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"]) if "ws1" in d else None
    kw = dict(topk_idx=d["topk_idx"], topk_w=d["topk_w"]) if "topk_idx" in d else \
        dict(wg=d["wg"], bias=d.get("bias"))
    fwd = rpg.moe_layer(d["x"], d["w1"], d["w3"], d["w2"], k, mt, shared=sw,
                        save_for_backward=True, **kw)
    g = rpg.moe_layer_backward(fwd, P.to_dev(dout), d["x"], d["w1"], d["w3"], d["w2"], mt,
                               shared=sw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(fwd["topk_idx"]), idx)
    for key in ("offsets", "dst_row", "src_row"):
        np.testing.assert_array_equal(_host(fwd[key]), lay[key], err_msg=key)
    used = int(lay["offsets"][-1])
    pad = torch.from_numpy(np.nonzero(lay["src_row"][:used] < 0)[0]).cuda()
    for key in ("dy_perm", "dab", "dx_perm"):
        assert bool((g[key][:used].index_select(0, pad).float() == 0).all()), f"{key}: pad rows"
        assert bool(torch.isfinite(g[key][:used].float()).all()), f"{key}: non-finite"
    for key in ("dx", "dtopk_w", "dw1", "dw3", "dw2"):
        assert bool(torch.isfinite(g[key]).all()), f"{key}: non-finite"
    tol = P.TOL[dt]

    P.log(f"[bwd-full] {name}: oracle on {SAMPLED_TOKENS} sampled tokens")
    toks = np.sort(np.random.default_rng(321).choice(T, SAMPLED_TOKENS, replace=False))
    shared = (inp["ws1"], inp["ws3"], inp["ws2"]) if "ws1" in inp else None
    dx, dw, slots = orc.token_backward(toks, inp["x"], idx, w, inp["w1"], inp["w3"], inp["w2"],
                                       dout, dt, shared)
    tt = torch.from_numpy(toks).cuda()
    errs = {"dx": P.rel_err(_host(g["dx"].index_select(0, tt)), dx),
            "dtopk_w": P.rel_err(_host(g["dtopk_w"].index_select(0, tt)), dw)}
    rows = torch.tensor([int(lay["dst_row"][t, j]) for (t, j) in slots], device="cuda")
    for key in ("dy", "dab", "dx_perm"):
        gk = "dy_perm" if key == "dy" else key
        errs[key] = P.rel_err(_host(g[gk].index_select(0, rows)),
                              np.stack([v[key] for v in slots.values()]))

    P.log(f"[bwd-full] {name}: oracle weight-gradient slices")
    counts = lay["counts"]
    rng = np.random.default_rng(654)
    hot = int(np.argmax(counts))
    other = int(rng.choice([e for e in range(E) if counts[e] > 0 and e != hot] or [hot]))
    fs = np.sort(rng.choice(F, SAMPLED_COLS, replace=False))
    ft = torch.from_numpy(fs).cuda()
    for e in sorted({hot, other}):
        sel = np.argwhere(idx == e)
        x_rows = inp["x"][sel[:, 0]]
        dy_rows = orc.round_storage(w[sel[:, 0], sel[:, 1]][:, None] *
                                    orc.values64(dout[sel[:, 0]]), dt)
        d1, d3, d2 = orc.expert_weight_grad_slices(x_rows, dy_rows, inp["w1"][e], inp["w3"][e],
                                                   inp["w2"][e], fs, dt)
        errs[f"dw1[{e}]"] = P.rel_err(_host(g["dw1"][e].index_select(0, ft)), d1)
        errs[f"dw3[{e}]"] = P.rel_err(_host(g["dw3"][e].index_select(0, ft)), d3)
        errs[f"dw2[{e}]"] = P.rel_err(_host(g["dw2"][e].index_select(1, ft)), d2)
    if shared is not None:
        S, Fs, _ = inp["ws1"].shape
        for s in range(S):
            fss = np.sort(rng.choice(Fs, SAMPLED_COLS, replace=False))
            d1, d3, d2 = orc.expert_weight_grad_slices(inp["x"], dout, inp["ws1"][s],
                                                       inp["ws3"][s], inp["ws2"][s], fss, dt)
            ct = torch.from_numpy(s * Fs + fss).cuda()
            errs[f"dws1[{s}]"] = P.rel_err(_host(g["dws1"][0].index_select(0, ct)), d1)
            errs[f"dws3[{s}]"] = P.rel_err(_host(g["dws3"][0].index_select(0, ct)), d3)
            errs[f"dws2[{s}]"] = P.rel_err(_host(g["dws2"][0].index_select(1, ct)), d2)
    P.log(f"[bwd-full] {name}: rel err " + " ".join(f"{k_} {v:.2e}" for k_, v in errs.items()))
    bad = {k_: v for k_, v in errs.items() if not v <= tol}
    assert not bad, bad
