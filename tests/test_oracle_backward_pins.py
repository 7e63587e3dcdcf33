"""Pins of the oracle's backward against facts fixed by mathematics.

The backward of the layer (the mirror of every forward step: unpermute for permute,
dispatch for combine, m-grouped dgrad plus k-grouped wgrad for each grouped fc) is
checked, without rounding (storage mode "f64"), against
  * torch float64 autograd of a forward written here independently: per routed slot,
    with no permuted buffer, no tile padding and no segment offsets;
  * central finite differences of the oracle's own forward (itself pinned by brute
    force elsewhere);
  * adjoint identities of the linear steps: <P x, G> = <x, P^T G>;
  * closed forms of silu'.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc


def _routing(rng, T, E, k, holes=True):
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=(T, k))
    if holes:
        drop = rng.random((T, k)) < 0.2
        idx[drop] = -1
        w[drop] = 0.0
    return idx, w


def _case(seed, T=9, D=12, F=10, E=5, k=2, shared=True, holes=True):
    rng = np.random.default_rng(seed)
    idx, w = _routing(rng, T, E, k, holes)
    inp = {
        "x": rng.standard_normal((T, D)),
        "topk_idx": idx,
        "topk_w": w,
        "w1": rng.standard_normal((E, F, D)) / math.sqrt(D),
        "w3": rng.standard_normal((E, F, D)) / math.sqrt(D),
        "w2": rng.standard_normal((E, D, F)) / math.sqrt(F),
    }
    if shared:
        inp["ws1"] = rng.standard_normal((2, 6, D)) / math.sqrt(D)
        inp["ws3"] = rng.standard_normal((2, 6, D)) / math.sqrt(D)
        inp["ws2"] = rng.standard_normal((2, D, 6)) / math.sqrt(6)
    dout = rng.standard_normal((T, D))
    return inp, dout


# ---------------------------------------------------------------------------
# torch autograd of an independent per-slot forward
# ---------------------------------------------------------------------------

def _torch_per_slot(inp, dout):
    """out[t] = sum_j w[t,j] FFN_{idx[t,j]}(x[t]) + sum_s FFN_s(x[t]), slot by slot."""
    leaf = {n: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
            for n, v in inp.items() if n != "topk_idx"}
    idx = torch.tensor(inp["topk_idx"], dtype=torch.int64)
    t_of, j_of = torch.nonzero(idx >= 0, as_tuple=True)
    e = idx[t_of, j_of]
    xs = leaf["x"].index_select(0, t_of)
    xs.retain_grad()
    a = torch.bmm(leaf["w1"][e], xs.unsqueeze(2)).squeeze(2)
    b = torch.bmm(leaf["w3"][e], xs.unsqueeze(2)).squeeze(2)
    a.retain_grad()
    b.retain_grad()
    h = torch.nn.functional.silu(a) * b
    h.retain_grad()
    y = torch.bmm(leaf["w2"][e], h.unsqueeze(2)).squeeze(2)
    y.retain_grad()
    out = torch.zeros_like(leaf["x"]).index_add(0, t_of, leaf["topk_w"][t_of, j_of, None] * y)
    if "ws1" in leaf:
        for s in range(leaf["ws1"].shape[0]):
            hs = torch.nn.functional.silu(leaf["x"] @ leaf["ws1"][s].T) * (leaf["x"] @ leaf["ws3"][s].T)
            out = out + hs @ leaf["ws2"][s].T
    (out * torch.tensor(dout)).sum().backward()
    slots = {"t": t_of.numpy(), "j": j_of.numpy(), "xs": xs.grad.numpy(), "a": a.grad.numpy(),
             "b": b.grad.numpy(), "h": h.grad.numpy(), "y": y.grad.numpy()}
    return {n: v.grad.numpy() for n, v in leaf.items()}, slots


def _close(got, ref, what, rel=1e-10):
    scale = max(1.0, float(np.max(np.abs(ref))) if np.size(ref) else 1.0)
    err = float(np.max(np.abs(np.asarray(got) - np.asarray(ref)))) if np.size(ref) else 0.0
    assert err <= rel * scale, f"{what}: max|diff| {err:.3e} (scale {scale:.3e})"


def _check_backward_against_autograd(o, seed, m_tile=4, **kw):
    inp, dout = _case(seed, **kw)
    k = inp["topk_idx"].shape[1]
    res = o.backward(inp, dout, k, m_tile, "f64")
    g, sl = _torch_per_slot(inp, dout)
    _close(res["dx"], g["x"], "dx")
    _close(res["dtopk_w"], g["topk_w"], "dtopk_w")
    for n in ("w1", "w3", "w2"):
        _close(res["d" + n], g[n], "d" + n)
    if "ws1" in inp:
        for n in ("ws1", "ws3", "ws2"):
            _close(res["d" + n], g[n], "d" + n)
    F = inp["w1"].shape[1]
    rows = res["fwd"]["dst_row"][sl["t"], sl["j"]]
    assert np.all(rows >= 0)
    _close(res["dy_perm"][rows], sl["y"], "dY")
    _close(res["dh"][rows], sl["h"], "dh")
    _close(res["dab"][rows, :F], sl["a"], "da")
    _close(res["dab"][rows, F:], sl["b"], "db")
    _close(res["dx_perm"][rows], sl["xs"], "dX")
    # rows that hold no slot (tile padding, unused capacity) carry zero gradient
    free = np.setdiff1d(np.arange(res["dy_perm"].shape[0]), rows)
    for n in ("dy_perm", "dh", "dab", "dx_perm"):
        assert not np.any(res[n][free]), n


@pytest.mark.parametrize("seed,m_tile,kw", [
    (0, 4, {}),
    (1, 1, {"k": 3, "E": 6}),
    (2, 8, {"shared": False, "holes": False}),
    (3, 4, {"T": 1, "k": 1, "E": 3}),
    (4, 16, {"T": 20, "E": 8, "k": 4, "D": 7, "F": 5}),
])
def test_backward_matches_autograd_of_per_slot_forward(seed, m_tile, kw):
    _check_backward_against_autograd(orc, seed, m_tile, **kw)


def test_expert_without_rows_gets_zero_weight_gradients():
    inp, dout = _case(7, E=6, shared=False, holes=False)
    gone = inp["topk_idx"] == 5
    inp["topk_idx"][gone] = -1
    inp["topk_w"][gone] = 0.0
    res = orc.backward(inp, dout, 2, 4, "f64")
    assert res["fwd"]["counts"][5] == 0
    for n in ("dw1", "dw3", "dw2"):
        assert not np.any(res[n][5])


# ---------------------------------------------------------------------------
# finite differences of the oracle's forward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["x", "topk_w", "w1", "w3", "w2", "ws1", "ws3", "ws2"])
def test_gradient_matches_central_difference(name):
    inp, dout = _case(11, T=4, D=5, F=4, E=3, k=2)
    res = orc.backward(inp, dout, 2, 2, "f64")
    v = np.random.default_rng(12).standard_normal(np.shape(inp[name]))
    if name == "topk_w":
        v[inp["topk_idx"] < 0] = 0.0

    def loss(t):
        p = dict(inp)
        p[name] = np.asarray(inp[name], dtype=np.float64) + t * v
        return float(np.sum(orc.forward(p, 2, 2, "f64")["out"] * dout))

    eps = 1e-5
    fd = (loss(eps) - loss(-eps)) / (2 * eps)
    key = "dtopk_w" if name == "topk_w" else ("dx" if name == "x" else "d" + name)
    an = float(np.sum(res[key] * v))
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


# ---------------------------------------------------------------------------
# adjoint identities of the linear steps
# ---------------------------------------------------------------------------

def test_unpermute_is_the_adjoint_of_permute():
    rng = np.random.default_rng(21)
    idx, _ = _routing(rng, 30, 7, 3)
    lay = orc.dispatch_layout(idx, 7, 8)
    x = rng.standard_normal((30, 6))
    G = rng.standard_normal((lay["m_cap"], 6))
    lhs = float(np.sum(orc.permute(x, lay) * G))
    rhs = float(np.sum(x * orc.permute_backward(G, lay["dst_row"], "f64")))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_combine_backward_is_the_adjoint_of_combine_in_y_and_in_w():
    rng = np.random.default_rng(22)
    idx, w = _routing(rng, 25, 6, 3)
    lay = orc.dispatch_layout(idx, 6, 4)
    Y = rng.standard_normal((lay["m_cap"], 5))
    Y[lay["src_row"] < 0] = 0.0
    g = rng.standard_normal((25, 5))
    dY, dw = orc.combine_backward(g, Y, lay["dst_row"], w, int(lay["offsets"][-1]), "f64")
    # linear in Y: <combine(Y), g> = <Y, dY>
    lhs = float(np.sum(orc.combine(Y, lay["dst_row"], w, "f64") * g))
    assert abs(lhs - float(np.sum(Y * dY))) <= 1e-12 * max(1.0, abs(lhs))
    # linear in w: <combine(Y; dw_dir), g> = <dw_dir, dw>
    vw = rng.standard_normal(w.shape)
    vw[idx < 0] = 0.0
    lhs = float(np.sum(orc.combine(Y, lay["dst_row"], vw, "f64") * g))
    assert abs(lhs - float(np.sum(vw * dw))) <= 1e-12 * max(1.0, abs(lhs))
    assert not np.any(dw[idx < 0])


# ---------------------------------------------------------------------------
# silu' closed forms
# ---------------------------------------------------------------------------

def test_silu_grad_closed_forms():
    assert orc.silu_grad(np.array([0.0]))[0] == 0.5
    a = np.linspace(-12, 12, 97)
    # silu(a) - silu(-a) = a, so silu'(a) + silu'(-a) = 1
    np.testing.assert_allclose(orc.silu_grad(a) + orc.silu_grad(-a), 1.0, atol=1e-14)
    # central difference of silu
    eps = 1e-6
    fd = (orc.silu(a + eps) - orc.silu(a - eps)) / (2 * eps)
    np.testing.assert_allclose(orc.silu_grad(a), fd, atol=1e-8)
    # tails: silu' -> 1 above, -> 0 below; the minimum is near a = -2.3994 (value -0.0998)
    assert abs(orc.silu_grad(np.array([60.0]))[0] - 1.0) < 1e-20
    assert abs(orc.silu_grad(np.array([-60.0]))[0]) < 1e-20
    grid = np.linspace(-3, -2, 100001)
    m = grid[np.argmin(orc.silu_grad(grid))]
    assert abs(m + 2.3994) < 1e-3


# ---------------------------------------------------------------------------
# storage rounding of the bf16 and f32 modes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,rel", [("bf16", 2 ** -5), ("f32", 1e-6)])
def test_stored_gradients_are_representable_and_near_exact(dtype, rel):
    inp, dout = _case(31, T=16, D=32, F=24, E=4, k=2)
    dout = orc.round_storage(dout, dtype)
    for n in ("x", "w1", "w3", "w2", "ws1", "ws3", "ws2"):
        inp[n] = orc.round_storage(inp[n], dtype)
    lo = orc.backward(inp, dout, 2, 4, dtype)
    ex = orc.backward(inp, dout, 2, 4, "f64")
    for n in ("dy_perm", "dh", "dab", "dx_perm", "dx", "dx_shared"):
        assert np.array_equal(orc.round_storage(lo[n], dtype), lo[n]), n
    for n in ("dx", "dw1", "dw3", "dw2", "dtopk_w", "dws1"):
        ref = ex[n]
        err = np.max(np.abs(lo[n] - ref)) / np.max(np.abs(ref))
        assert err < rel, (n, err)


# ---------------------------------------------------------------------------
# the sampled forms used at full size agree with the whole backward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f64"])
def test_token_backward_equals_backward_rows(dtype):
    inp, dout = _case(41, T=12, D=16, F=8, E=4, k=2)
    for n in ("x", "w1", "w3", "w2", "ws1", "ws3", "ws2"):
        inp[n] = orc.round_storage(inp[n], dtype)
    dout = orc.round_storage(dout, dtype)
    res = orc.backward(inp, dout, 2, 4, dtype)
    toks = np.array([0, 5, 11])
    dx, dw, slots = orc.token_backward(toks, inp["x"], inp["topk_idx"], inp["topk_w"], inp["w1"],
                                       inp["w3"], inp["w2"], dout, dtype,
                                       (inp["ws1"], inp["ws3"], inp["ws2"]))
    # the same float64 arithmetic batched differently: equal up to a last-bit rounding flip
    tol = 1e-12 if dtype == "f64" else 2 ** -7
    _close(dx, res["dx"][toks], "dx", tol)
    _close(dw, res["dtopk_w"][toks], "dtopk_w", 1e-12)
    assert len(slots) == int((inp["topk_idx"][toks] >= 0).sum())
    for (t, j), v in slots.items():
        r = res["fwd"]["dst_row"][t, j]
        _close(v["dy"], res["dy_perm"][r], "dy", tol)
        _close(v["dab"], res["dab"][r], "dab", tol)
        _close(v["dx_perm"], res["dx_perm"][r], "dX", tol)


@pytest.mark.parametrize("dtype", ["bf16", "f64"])
def test_weight_grad_slices_equal_backward(dtype):
    inp, dout = _case(42, T=20, D=16, F=12, E=3, k=2, shared=False)
    for n in ("x", "w1", "w3", "w2"):
        inp[n] = orc.round_storage(inp[n], dtype)
    dout = orc.round_storage(dout, dtype)
    res = orc.backward(inp, dout, 2, 4, dtype)
    off = res["fwd"]["offsets"]
    fs = [0, 5, 11]
    for e in range(3):
        r0, r1 = int(off[e]), int(off[e + 1])
        d1, d3, d2 = orc.expert_weight_grad_slices(res["fwd"]["x_perm"][r0:r1],
                                                   res["dy_perm"][r0:r1], inp["w1"][e],
                                                   inp["w3"][e], inp["w2"][e], fs, dtype)
        tol = 1e-12 if dtype == "f64" else 1e-2
        _close(d1, res["dw1"][e][fs], "dW1", tol)
        _close(d3, res["dw3"][e][fs], "dW3", tol)
        _close(d2, res["dw2"][e][:, fs], "dW2", tol)
