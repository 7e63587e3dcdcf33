"""GPU parity of the backward path (the mirror of each forward step) against the oracle.

Each library call is first checked on its own with NaN-poisoned outputs (so an element a
kernel leaves unwritten fails the test), then the whole chain, moe_layer(...,
save_for_backward=True) followed by moe_layer_backward, against oracle.backward on the
same seeded inputs and output gradient.

Bar: dy_perm, dab, dx_perm, dx, dx_shared, the
top-k weight gradients and the float32 weight gradients within max|gpu - ref| / max|ref|
<= 1e-5 (float32 layers) or 2e-2 (bf16 layers, float32 accumulation); pad rows of
dy_perm, dab and dx_perm exactly zero; experts without rows get exactly zero weight
gradients.
"""
import numpy as np
import pytest
import torch

import routing_permute_grouped_amd as rpg
import workloads as W
from oracle import moe_oracle as orc
from tests import _parity as P

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# the single calls, fed with the oracle's forward
# ---------------------------------------------------------------------------

def _small(dt="bf16"):
    if dt == "bf16":
        cfg = W.shrink(W.preset("skew32_zipf_bf16"), T=400, D=256, F=320)
    else:
        cfg = W.shrink(W.preset("tiny_f32"), T=200, D=128, F=192, E=6, k=3, m_tile=64)
    inp = W.generate(cfg, seed=2)
    cfg = inp["cfg"]
    dout = W.output_grad(cfg, seed=2)
    return cfg, inp, dout


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_combine_backward_against_oracle(dt):
    P.log(f"[bwd] combine_backward {dt}")
    cfg, inp, dout = _small(dt)
    ref = orc.backward(inp, dout, cfg.k, cfg.m_tile, dt)
    f = ref["fwd"]
    y = orc.round_storage(f["y_perm"], dt)
    y_st = y.astype(np.float32) if dt == "f32" else W.f32_to_bf16_bits(y.astype(np.float32))
    dev = {n: P.to_dev(np.ascontiguousarray(f[n], dtype=np.int32))
           for n in ("src_row", "offsets", "dst_row")}
    dy = P.poison(torch.empty((f["m_cap"], cfg.D), dtype=torch.float32 if dt == "f32"
                              else torch.bfloat16, device="cuda"))
    dw = P.poison(torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda"))
    rpg.moe_combine_backward(P.to_dev(dout), P.to_dev(y_st), dev["src_row"], dev["offsets"],
                             dev["dst_row"], P.to_dev(f["topk_w"].astype(np.float32)),
                             m_cap=f["m_cap"], dy_perm=dy, dtopk_w=dw)
    torch.cuda.synchronize()
    used = int(f["offsets"][-1])
    g = P.to_host(dy)[:used]
    assert np.all(np.isfinite(orc.values64(g)))
    e = P.rel_err(g, ref["dy_perm"][:used])
    assert e <= P.TOL[dt], e
    assert np.all(orc.values64(g)[f["src_row"][:used] < 0] == 0)
    gw = P.to_host(dw)
    assert np.all(np.isfinite(gw))
    assert np.all(gw[f["dst_row"] < 0] == 0)
    # same stored inputs on both sides: only the float32 summation order differs
    np.testing.assert_allclose(gw, ref["dtopk_w"], rtol=1e-4, atol=1e-4 * np.abs(gw).max())


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("split", [True, False])
def test_dgrad_swiglu_against_oracle(dt, split):
    P.log(f"[bwd] dgrad_swiglu {dt} split={split}")
    cfg, inp, dout = _small(dt)
    ref = orc.backward(inp, dout, cfg.k, cfg.m_tile, dt)
    f = ref["fwd"]
    store = (lambda a: a.astype(np.float32)) if dt == "f32" else \
        (lambda a: W.f32_to_bf16_bits(a.astype(np.float32)))
    M, F = f["m_cap"], cfg.F
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    dab = P.poison(torch.empty((M, 2 * F), dtype=tdt, device="cuda"))
    dh = P.poison(torch.empty((M, F), dtype=tdt, device="cuda"))
    ws = P.poison(torch.empty(rpg.moe_grouped_workspace_bytes() // 4, dtype=torch.float32,
                              device="cuda")) if split else None
    rpg.moe_grouped_dgrad_swiglu(P.to_dev(store(ref["dy_perm"])),
                                 P.to_dev(f["offsets"].astype(np.int32)),
                                 P.to_dev(f["tile_expert"].astype(np.int32)), P.to_dev(inp["w2"]),
                                 P.to_dev(store(ref["ab"])), cfg.m_tile, M, dab=dab, dh=dh,
                                 workspace=ws)
    torch.cuda.synchronize()
    used = int(f["offsets"][-1])
    for name, got in (("dh", dh), ("dab", dab)):
        g = P.to_host(got)[:used]
        assert np.all(np.isfinite(orc.values64(g))), name
        e = P.rel_err(g, ref[name][:used])
        assert e <= P.TOL[dt], (name, e)
        assert np.all(orc.values64(g)[f["src_row"][:used] < 0] == 0), name


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("split", [True, False])
def test_dgrad_fc1_against_oracle(dt, split):
    P.log(f"[bwd] dgrad_fc1 {dt} split={split}")
    cfg, inp, dout = _small(dt)
    ref = orc.backward(inp, dout, cfg.k, cfg.m_tile, dt)
    f = ref["fwd"]
    store = (lambda a: a.astype(np.float32)) if dt == "f32" else \
        (lambda a: W.f32_to_bf16_bits(a.astype(np.float32)))
    M = f["m_cap"]
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    dx = P.poison(torch.empty((M, cfg.D), dtype=tdt, device="cuda"))
    ws = P.poison(torch.empty(rpg.moe_grouped_workspace_bytes() // 4, dtype=torch.float32,
                              device="cuda")) if split else None
    rpg.moe_grouped_dgrad_fc1(P.to_dev(store(ref["dab"])), P.to_dev(f["offsets"].astype(np.int32)),
                              P.to_dev(f["tile_expert"].astype(np.int32)), P.to_dev(inp["w1"]),
                              P.to_dev(inp["w3"]), cfg.m_tile, M, dx_perm=dx, workspace=ws)
    torch.cuda.synchronize()
    used = int(f["offsets"][-1])
    g = P.to_host(dx)[:used]
    assert np.all(np.isfinite(orc.values64(g)))
    e = P.rel_err(g, ref["dx_perm"][:used])
    assert e <= P.TOL[dt], e
    assert np.all(orc.values64(g)[f["src_row"][:used] < 0] == 0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("mt,ragged", [(128, False), (16, False), (128, True)])
def test_wgrad_is_the_per_expert_contraction(dt, mt, ragged):
    """k-grouped GEMM against its definition: an empty expert, a split row NS inside a
    256-row tile, N1 and N2 not multiples of 256, segments of m_tile multiples (and with
    ``ragged`` a last segment ending mid k-step, with NaN rows behind it that must not be
    read)."""
    P.log(f"[bwd] wgrad {dt} mt={mt} ragged={ragged}")
    rng = np.random.default_rng(9)
    E = 5
    idx = rng.integers(0, E - 1, size=(300, 2)).astype(np.int32)   # expert E-1 gets no rows
    lay = orc.dispatch_layout(idx, E, mt)
    M = lay["m_cap"]
    offs = lay["offsets"].copy()
    if ragged:
        offs[E - 1] -= 37     # the last non-empty segment ends 37 rows early
        offs[E] = offs[E - 1]
    N1, N2, NS = 320, 192, 192
    P_ = rng.standard_normal((M, N1)).astype(np.float32)
    Q_ = rng.standard_normal((M, N2)).astype(np.float32)
    used = int(offs[E])
    P_[used:] = np.nan
    Q_[used:] = np.nan
    if dt == "bf16":
        P_, Q_ = W.f32_to_bf16_bits(P_), W.f32_to_bf16_bits(Q_)
    lo = P.poison(torch.empty((E, NS, N2), dtype=torch.float32, device="cuda"))
    hi = P.poison(torch.empty((E, N1 - NS, N2), dtype=torch.float32, device="cuda"))
    rpg.moe_grouped_wgrad(P.to_dev(P_), P.to_dev(Q_), P.to_dev(offs), mt, M, NS=NS, out_lo=lo,
                          out_hi=hi)
    torch.cuda.synchronize()
    got = np.concatenate([P.to_host(lo), P.to_host(hi)], axis=1)
    p64, q64 = orc.values64(P_), orc.values64(Q_)
    ref = np.zeros((E, N1, N2))
    for e in range(E):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        ref[e] = p64[r0:r1].T @ q64[r0:r1]
    assert np.all(np.isfinite(got))
    assert np.all(got[E - 1] == 0)
    e = P.rel_err(got, ref)
    assert e <= 1e-5, e   # same stored operands: float32 accumulation only


# ---------------------------------------------------------------------------
# the whole backward against oracle.backward
# ---------------------------------------------------------------------------

BWD = {
    "tiny_f32": W.preset("tiny_f32"),
    "f32_mt64": W.shrink(W.preset("tiny_f32"), T=300, D=192, F=320, E=6, k=3, m_tile=64),
    "dense8": W.shrink(W.preset("dense8_bf16"), T=512, D=512, F=1024),
    "dense8_mt256": W.shrink(W.preset("dense8_bf16"), T=520, D=256, F=512, m_tile=256),
    "fine64_shared2": W.shrink(W.preset("fine64_shared2_bf16"), T=389, D=256, F=320, F_shared=192),
    "skew32_zipf": W.shrink(W.preset("skew32_zipf_bf16"), T=1024, D=512, F=256),
    "etp_shard32": W.shrink(W.preset("etp_shard32_bf16"), D=1024, F=512, poisson_mean=40.0),
    "bf16_mt64": W.shrink(W.preset("dense8_bf16"), T=900, D=512, F=768, m_tile=64),
    "bf16_mt16": W.shrink(W.preset("skew32_zipf_bf16"), T=500, D=256, F=320, m_tile=16),
}


def run_backward(inp: dict, dout: np.ndarray, cfg, split_k: bool = True) -> dict:
    d = {n: P.to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    sw = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"]) if "ws1" in d else None
    kw = dict(topk_idx=d["topk_idx"], topk_w=d["topk_w"]) if "topk_idx" in d else \
        dict(wg=d["wg"], bias=d.get("bias"))
    fwd = rpg.moe_layer(d["x"], d["w1"], d["w3"], d["w2"], cfg.k, cfg.m_tile, shared=sw,
                        split_k=split_k, save_for_backward=True, **kw)
    bwd = rpg.moe_layer_backward(fwd, P.to_dev(dout), d["x"], d["w1"], d["w3"], d["w2"],
                                 cfg.m_tile, shared=sw, split_k=split_k)
    torch.cuda.synchronize()
    out = {n: P.to_host(v) for n, v in bwd.items()}
    out["offsets"] = P.to_host(fwd["offsets"])
    return out


def check_backward(name: str, cfg, seed: int = 0, split_k: bool = True) -> dict:
    P.log(f"[bwd] layer {name} split_k={split_k}: {cfg}")
    inp = W.generate(cfg, seed=seed)
    cfg = inp["cfg"]
    dout = W.output_grad(cfg, seed=seed)
    dt = cfg.dtype
    ref = orc.backward(inp, dout, cfg.k, cfg.m_tile, dt)
    g = run_backward(inp, dout, cfg, split_k)
    tol = P.TOL[dt]
    f = ref["fwd"]
    np.testing.assert_array_equal(g["offsets"], f["offsets"])
    used = int(f["offsets"][-1])
    pad = f["src_row"][:used] < 0
    for key in ("dy_perm", "dab", "dx_perm"):
        vals = orc.values64(g[key][:used])
        assert np.all(np.isfinite(vals)), f"{key}: non-finite"
        assert np.all(vals[pad] == 0), f"{key}: pad rows not zero"
        e = P.rel_err(g[key][:used], ref[key][:used])
        assert e <= tol, f"{key}: rel err {e:.3e} > {tol}"
    for key in ("dx", "dtopk_w", "dw1", "dw3", "dw2"):
        assert np.all(np.isfinite(orc.values64(g[key]))), key
        e = P.rel_err(g[key], ref[key])
        assert e <= tol, f"{key}: rel err {e:.3e} > {tol}"
    empty = np.nonzero(f["counts"] == 0)[0]
    for key in ("dw1", "dw3", "dw2"):
        assert np.all(g[key][empty] == 0), f"{key}: empty expert not zero"
    if "ws1" in inp:
        S, Fs, D = inp["ws1"].shape
        e = P.rel_err(g["dx_shared"], ref["dx_shared"])
        assert e <= tol, f"dx_shared: rel err {e:.3e}"
        for key, got in (("dws1", g["dws1"].reshape(S, Fs, D)),
                         ("dws3", g["dws3"].reshape(S, Fs, D)),
                         ("dws2", g["dws2"].reshape(D, S, Fs).transpose(1, 0, 2))):
            e = P.rel_err(got, ref[key])
            assert e <= tol, f"{key}: rel err {e:.3e}"
    return g


@pytest.mark.parametrize("name", list(BWD))
def test_layer_backward_parity(name):
    check_backward(name, BWD[name])


def test_layer_backward_without_split_k():
    check_backward("dense8", BWD["dense8"], seed=4, split_k=False)


def test_backward_of_dense_single_expert_with_ragged_rows():
    # E = 1, top-1: the whole backward is one dense SwiGLU FFN backward over 300 rows
    cfg = W.MoEConfig("dense1", T=300, D=256, F=192, E=1, k=1, m_tile=128, dtype="bf16")
    check_backward("dense1", cfg, seed=1)
