"""Helpers of the GPU parity tests: upload seeded inputs, run the four library calls,
download the results and compare them with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import routing_permute_grouped_amd as rpg
from oracle import moe_oracle as orc

TOL = {"f32": 1e-5, "bf16": 2e-2}   # max|gpu - ref| / max|ref| (fp32 / bf16 with fp32 accumulate)
W_RTOL = 1e-6                        # top-k weights: float32 softmax against float64


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def mx_rows(words: np.ndarray) -> np.ndarray:
    """MX scales in k-step words (uint8 [C/128, R, 4]: word (s, r) holds row r's scale
    bytes of blocks 4s .. 4s+3) back to rows [R, C/32]; index reshuffling only."""
    S, R, _ = words.shape
    return np.ascontiguousarray(words.transpose(1, 0, 2)).reshape(R, 4 * S)


def rel_err(got, ref) -> float:
    g, r = orc.values64(got), np.asarray(ref, dtype=np.float64)
    den = np.abs(r).max()
    return float(np.abs(g - r).max() / (den if den > 0 else 1.0))


def poison(t: torch.Tensor) -> torch.Tensor:
    return t.fill_(float("nan"))


def run_gpu(inp: dict, k: int, m_tile: int, renorm: bool = False, want_logits: bool = True,
            ws_bytes: int | None = None) -> dict:
    """Run route (unless routing is given), permute, grouped SwiGLU (routed and shared)
    and combine; every float output buffer is NaN-poisoned first. The grouped calls get
    a NaN-poisoned workspace of ``ws_bytes`` (default moe_grouped_workspace_bytes(); 0 =
    none, so no split-K tail)."""
    d = {n: to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    E = inp["w1"].shape[0]
    T = inp["x"].shape[0]
    out: dict = {}
    if "topk_idx" in inp:
        idx, w = d["topk_idx"], d["topk_w"]
    else:
        idx, w, logits = rpg.moe_route(d["x"], d["wg"], k, bias=d.get("bias"), renorm=renorm,
                                       want_logits=want_logits)
        out["logits"] = logits
    out["topk_idx"], out["topk_w"] = idx, w
    m_cap = rpg.moe_capacity(T, k, E, m_tile)
    xp = poison(torch.empty((m_cap, inp["x"].shape[1]), dtype=d["x"].dtype, device="cuda"))
    p = rpg.moe_permute(d["x"], idx, E, m_tile, m_cap=m_cap, out={"x_perm": xp})
    out.update(p)
    F = inp["w1"].shape[1]
    if ws_bytes is None:
        ws_bytes = rpg.moe_grouped_workspace_bytes()
    ws = None
    if ws_bytes:
        ws = poison(torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda"))
    h = poison(torch.empty((m_cap, F), dtype=d["x"].dtype, device="cuda"))
    y = poison(torch.empty((m_cap, inp["x"].shape[1]), dtype=d["x"].dtype, device="cuda"))
    rpg.moe_grouped_swiglu(p["x_perm"], p["offsets"], p["tile_expert"], d["w1"], d["w3"], d["w2"],
                           m_tile, m_cap=m_cap, h=h, y_perm=y, workspace=ws, counts=p["counts"])
    out["h"], out["y_perm"] = h, y
    shared = None
    if "ws1" in d:
        sw = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"])
        rows = rpg.DenseRows(T, m_tile, "cuda")
        hs = poison(torch.empty((rows.m_cap, sw.w1.shape[1]), dtype=d["x"].dtype, device="cuda"))
        ys = poison(torch.empty((rows.m_cap, inp["x"].shape[1]), dtype=d["x"].dtype, device="cuda"))
        rpg.moe_grouped_swiglu(d["x"], rows.offsets, rows.tile_expert, sw.w1, sw.w3, sw.w2, m_tile,
                               m_cap=rows.m_cap, h=hs, y_perm=ys, workspace=ws, rows_used=T)
        shared = ys[:T]
        out["shared"] = shared
    o = poison(torch.empty_like(d["x"]))
    out["out"] = rpg.moe_combine(y, p["dst_row"], w, shared=shared, out=o, m_cap=m_cap)
    torch.cuda.synchronize()
    return {kk: (to_host(v) if isinstance(v, torch.Tensor) else v) for kk, v in out.items()}


def compare_layer(g: dict, ref: dict, dtype: str, expect_dev_err: int = 0,
                  verbose: bool = False) -> dict:
    """Element-by-element parity of every output of the layer against the oracle's
    ``forward`` result: logits, routing, layout and x_perm bit for bit; h, y_perm (every
    row in use: all finite, pad rows exactly 0), shared and out within the tolerance.
    Returns the relative errors."""
    tol = TOL[dtype]
    errs = {}
    if "logits" in ref:
        np.testing.assert_array_equal(g["logits"].view(np.uint32), ref["logits"].view(np.uint32))
        np.testing.assert_array_equal(g["topk_idx"], ref["topk_idx"])
        np.testing.assert_allclose(g["topk_w"], ref["topk_w"], rtol=W_RTOL, atol=0)
    for key in ("counts", "offsets", "dst_row", "src_row", "tile_expert"):
        np.testing.assert_array_equal(g[key], ref[key], err_msg=key)
    assert int(g["dev_err"][0]) == expect_dev_err
    used = int(ref["offsets"][-1])
    np.testing.assert_array_equal(g["x_perm"][:used], ref["x_perm"][:used])
    pad = ref["src_row"][:used] < 0
    for key in ("h", "y_perm"):
        vals = orc.values64(g[key][:used])
        assert np.all(np.isfinite(vals)), f"{key}: unwritten rows"
        assert np.all(vals[pad] == 0), f"{key}: pad rows not zero"
        del vals
        errs[key] = rel_err(g[key][:used], ref[key][:used])
    if "shared" in ref:
        assert np.all(np.isfinite(orc.values64(g["shared"]))), "shared: unwritten rows"
        errs["shared"] = rel_err(g["shared"], ref["shared"])
    assert np.all(np.isfinite(orc.values64(g["out"]))), "out: unwritten rows"
    errs["out"] = rel_err(g["out"], ref["out"])
    if verbose:
        log("  rel err " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for key, e in errs.items():
        assert e <= tol, f"{key}: rel err {e:.3e} > {tol}"
    return errs


def check_layer(inp: dict, k: int, m_tile: int, dtype: str, renorm: bool = False,
                expect_dev_err: int = 0, ws_bytes: int | None = None) -> dict:
    """Full element-by-element parity of every output of the layer against the oracle."""
    ref = orc.forward(inp, k=k, m_tile=m_tile, dtype=dtype, renorm=renorm)
    g = run_gpu(inp, k, m_tile, renorm, ws_bytes=ws_bytes)
    compare_layer(g, ref, dtype, expect_dev_err)
    return g
