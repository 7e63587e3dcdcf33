"""GPU parity of the masked (fixed-capacity slab) layout for decode against the oracle.

Bar (shrunk cases spanning several row blocks and ragged slabs, and both decode workloads
at full size): counts, dst_row, src_row and the dropped-slot flag bit-exact; the valid rows of
x_masked bit-exact; h, y and out within max|gpu - ref| / max|ref| <= 2e-2 (bf16) or
1e-5 (float32) on the valid rows; every row past counts[e] left untouched (outputs are
NaN-poisoned first, and those rows must still hold NaN)."""
import dataclasses

import numpy as np
import pytest
import torch

import routing_permute_grouped_amd as rpg
import workloads as W
from oracle import moe_oracle as orc
from tests import _parity as P

pytestmark = pytest.mark.gpu

# The decode GEMM serves bf16 slabs of at most 128 rows when the experts give at least two
# workgroups of 64 output columns per CU (E * min(D, F) / 64 >= 512 on 256 CUs); the
# other cases run on the tile kernel. Both paths are covered here.
CASES = {
    # tile kernel: 8 experts of D=512 are too few workgroups for the decode GEMM
    "decode8": W.shrink(W.preset("decode8_bf16"), D=512, F=1024),
    "tiny_f32_masked": dataclasses.replace(W.preset("tiny_f32"), T=40, cap=16),
    # decode GEMM: one row block per expert, shared experts beside (tile kernel, E=1)
    "decode64_shared2": W.shrink(W.preset("decode64_shared2_bf16"), T=96, D=512, F=512,
                                 F_shared=256, cap=96),
    # the skewed router: its hot experts get far more than cap slots, 20 get none
    "skew_drops": dataclasses.replace(W.shrink(W.preset("skew32_zipf_bf16"), T=128, D=1024,
                                               F=1024), cap=32),
    "etp_given_masked": dataclasses.replace(
        W.shrink(W.preset("etp_shard32_bf16"), D=1024, F=1024, poisson_mean=20.0), cap=48),
    # 3 and 4 row blocks, slabs of 64 with drops
    "mid_slabs": dataclasses.replace(W.shrink(W.preset("decode64_shared2_bf16"), T=600, D=512,
                                              F=512), cap=64, n_shared=0),
    # 5 to 8 row blocks of 16 in slabs of 128, partial last blocks, 13 slots dropped (the
    # decode GEMM's largest bodies)
    "wide_slabs": dataclasses.replace(W.shrink(W.preset("decode64_shared2_bf16"), T=1100,
                                               D=512, F=512), cap=128, n_shared=0),
}


def run_masked(inp, cfg, split_k=True):
    d = {n: P.to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    T, D, F, E, k, cap = inp["x"].shape[0], cfg.D, cfg.F, cfg.E, cfg.k, cfg.cap
    out = {}
    if "topk_idx" in d:
        idx, w = d["topk_idx"], d["topk_w"]
    else:
        idx, w, _ = rpg.moe_route(d["x"], d["wg"], k, bias=d.get("bias"))
    out["topk_idx"] = idx
    xm = P.poison(torch.empty((E * cap, D), dtype=d["x"].dtype, device="cuda"))
    p = rpg.moe_permute_masked(d["x"], idx, E, cap, out={"x_masked": xm})
    out.update(p)
    ws = P.poison(torch.empty(rpg.moe_grouped_workspace_bytes() // 4, dtype=torch.float32,
                              device="cuda")) if split_k else None
    h = P.poison(torch.empty((E * cap, F), dtype=d["x"].dtype, device="cuda"))
    y = P.poison(torch.empty((E * cap, D), dtype=d["x"].dtype, device="cuda"))
    rpg.moe_grouped_swiglu_masked(p["x_masked"], p["counts"], d["w1"], d["w3"], d["w2"], cap,
                                  h=h, y=y, workspace=ws)
    out["h"], out["y_perm"] = h, y
    shared = None
    if "ws1" in d:
        sw = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"])
        rows = rpg.DenseRows(T, 128, "cuda")
        _, ys = rpg.moe_grouped_swiglu(d["x"], rows.offsets, rows.tile_expert, sw.w1, sw.w3, sw.w2,
                                       128, m_cap=rows.m_cap, workspace=ws, rows_used=T)
        shared = ys[:T]
    o = P.poison(torch.empty_like(d["x"]))
    out["out"] = rpg.moe_combine(y, p["dst_row"], w, shared=shared, out=o, m_cap=E * cap)
    torch.cuda.synchronize()
    return {kk: (P.to_host(v) if isinstance(v, torch.Tensor) else v) for kk, v in out.items()}


def check_masked(cfg, split_k=True, label=""):
    """The masked layer on the GPU against the oracle's, on every output."""
    inp = W.generate(cfg, seed=0)
    cfg = inp["cfg"]
    P.log(f"[masked] {label}: oracle")
    ref = orc.forward_masked(inp, cfg.k, cfg.cap, cfg.dtype)
    P.log(f"[masked] {label}: gpu")
    g = run_masked(inp, cfg, split_k)
    np.testing.assert_array_equal(g["topk_idx"], ref["topk_idx"])
    for key in ("counts", "dst_row", "src_row"):
        np.testing.assert_array_equal(g[key], ref[key], err_msg=key)
    assert int(g["dev_err"][0]) == (2 if ref["dropped"] else 0)
    valid = ref["src_row"] >= 0
    np.testing.assert_array_equal(g["x_masked"][valid], ref["x_perm"][valid])
    tol = P.TOL[cfg.dtype]
    errs = {}
    for key in ("h", "y_perm"):
        vals = orc.values64(g[key])
        assert np.all(np.isfinite(vals[valid])), f"{key}: valid rows not written"
        assert np.all(np.isnan(vals[~valid])), f"{key}: rows past counts were written"
        errs[key] = P.rel_err(g[key][valid], ref[key][valid])
    assert np.all(np.isnan(orc.values64(g["x_masked"])[~valid])), "x_masked: unused rows written"
    errs["out"] = P.rel_err(g["out"], ref["out"])
    P.log(f"[masked] {label}: rel err " + " ".join(f"{k_} {v:.2e}" for k_, v in errs.items()))
    bad = {k_: v for k_, v in errs.items() if not v <= tol}
    assert not bad, bad
    return ref


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("split_k", [True, False])
def test_masked_layer_parity(name, split_k):
    cfg = CASES[name]
    ref = check_masked(cfg, split_k, f"{name} split_k={split_k}: {cfg}")
    if name == "skew_drops":
        assert ref["dropped"] > 0


@pytest.mark.parametrize("name", ["decode8_bf16", "decode64_shared2_bf16"])
def test_masked_layer_full_size(name):
    """The decode workloads at their full sizes, in the benchmark's launch configuration
    (split-K workspace given; bf16 slabs of at most 128 rows take the decode GEMM). A
    decode batch is small enough for the oracle to compute every row."""
    check_masked(W.preset(name), True, f"full-size {name}")


# The masked permute alone at its edges: one token, one expert, top-k = E, the largest
# row (float32 rows of 65536 values: more copy items than workgroups, so a workgroup
# copies several), the most slots one launch ranks (256 tokens x top-32 over 1024
# experts) and the first batch size past it (257 tokens: histogram, rank and copy).
EDGES = [(1, 1, 1, 64, 16, "f32"), (1, 8, 8, 64, 16, "bf16"), (256, 3, 3, 65536, 256, "f32"),
         (256, 1024, 32, 64, 16, "bf16"), (257, 16, 4, 128, 32, "bf16"),
         (200, 40, 6, 192, 16, "bf16")]


@pytest.mark.parametrize("T,E,k,D,cap,dt", EDGES)
def test_masked_permute_edges(T, E, k, D, cap, dt):
    P.log(f"[masked] permute edge T={T} E={E} k={k} D={D} cap={cap} {dt}")
    rng = np.random.default_rng(T * 7 + E)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    x32 = rng.standard_normal((T, D)).astype(np.float32)
    x = x32 if dt == "f32" else W.f32_to_bf16_bits(x32)
    ml = orc.masked_layout(idx, E, cap)
    g = rpg.moe_permute_masked(P.to_dev(x), P.to_dev(idx), E, cap)
    torch.cuda.synchronize()
    for key in ("counts", "dst_row", "src_row"):
        np.testing.assert_array_equal(P.to_host(g[key]), ml[key], err_msg=key)
    assert int(P.to_host(g["dev_err"])[0]) == (2 if ml["dropped"] else 0)
    rows = ml["src_row"]
    valid = rows >= 0
    np.testing.assert_array_equal(P.to_host(g["x_masked"])[valid], x[rows[valid] // k])
