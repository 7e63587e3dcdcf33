"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every check here compares the oracle with something other than itself: values the
pages print (the page-4 expert-parallel split example), closed forms, invariants,
special cases that reduce to a library routine, and brute force written as plain
Python loops on tiny inputs.
"""
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


def _tiny_layer(seed, T=7, D=24, F=10, E=5, k=2, dtype="f32", bias=False, shared=False):
    rng = np.random.default_rng(seed)
    inp = {
        "x": rng.standard_normal((T, D)).astype(np.float32),
        "wg": (rng.standard_normal((E, D)) / math.sqrt(D)).astype(np.float32),
        "w1": (rng.standard_normal((E, F, D)) / math.sqrt(D)).astype(np.float32),
        "w3": (rng.standard_normal((E, F, D)) / math.sqrt(D)).astype(np.float32),
        "w2": (rng.standard_normal((E, D, F)) / math.sqrt(F)).astype(np.float32),
    }
    if bias:
        inp["bias"] = rng.standard_normal(E).astype(np.float32)
    if shared:
        inp["ws1"] = (rng.standard_normal((2, 6, D)) / math.sqrt(D)).astype(np.float32)
        inp["ws3"] = (rng.standard_normal((2, 6, D)) / math.sqrt(D)).astype(np.float32)
        inp["ws2"] = (rng.standard_normal((2, D, 6)) / math.sqrt(6)).astype(np.float32)
    return inp


# ---------------------------------------------------------------------------
# brute force: plain Python loops over tokens and experts, float64 throughout
# ---------------------------------------------------------------------------

def _py_silu(a):
    return a / (1.0 + math.exp(-a)) if a > -700 else 0.0


def _py_ffn(xrow, w1e, w3e, w2e):
    D = len(xrow)
    F = len(w1e)
    h = []
    for f in range(F):
        a = sum(float(xrow[d]) * float(w1e[f][d]) for d in range(D))
        b = sum(float(xrow[d]) * float(w3e[f][d]) for d in range(D))
        h.append(_py_silu(a) * b)
    return [sum(h[f] * float(w2e[o][f]) for f in range(F)) for o in range(len(w2e))]


def brute_layer(inp, k, renorm=False):
    """Per-token sum over the top-k experts, no permutation, float64."""
    x, wg = inp["x"], inp["wg"]
    T, D = x.shape
    E = wg.shape[0]
    bias = inp.get("bias")
    outs, idxs, ws = [], [], []
    for t in range(T):
        logits = [sum(float(x[t, d]) * float(wg[e, d]) for d in range(D)) + (float(bias[e]) if bias is not None else 0.0)
                  for e in range(E)]
        order = sorted(range(E), key=lambda e: (-logits[e], e))
        # selection must not hinge on rounding: demand a clear margin at the cut
        if k < E:
            assert logits[order[k - 1]] - logits[order[k]] > 1e-5
        m = max(logits)
        z = [math.exp(l - m) for l in logits]
        s = sum(z)
        p = [v / s for v in z]
        sel = order[:k]
        w = [p[e] for e in sel]
        if renorm:
            tot = sum(w)
            w = [v / tot for v in w]
        o = [0.0] * D
        for j, e in enumerate(sel):
            y = _py_ffn(x[t], inp["w1"][e], inp["w3"][e], inp["w2"][e])
            o = [o[d] + w[j] * y[d] for d in range(D)]
        if "ws1" in inp:
            for s_ in range(inp["ws1"].shape[0]):
                y = _py_ffn(x[t], inp["ws1"][s_], inp["ws3"][s_], inp["ws2"][s_])
                o = [o[d] + y[d] for d in range(D)]
        outs.append(o)
        idxs.append(sel)
        ws.append(w)
    return np.array(outs), np.array(idxs), np.array(ws)


def _check_layer_against_brute(oracle, seed, k, **kw):
    inp = _tiny_layer(seed, k=k, **kw)
    res = oracle.forward(inp, k=k, m_tile=4, dtype="f32", renorm=kw.get("renorm", False))
    out_b, idx_b, w_b = brute_layer(inp, k)
    np.testing.assert_array_equal(res["topk_idx"], idx_b)
    np.testing.assert_allclose(res["topk_w"], w_b, rtol=1e-6, atol=0)
    err = np.abs(res["out"] - out_b).max() / np.abs(out_b).max()
    assert err < 2e-6, err


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_layer_matches_per_token_bruteforce(seed):
    _check_layer_against_brute(orc, seed, k=2)


def test_layer_bruteforce_with_bias_and_shared():
    _check_layer_against_brute(orc, 5, k=3, bias=True, shared=True)


def test_layer_bruteforce_k_equals_e():
    _check_layer_against_brute(orc, 7, k=5)


# ---------------------------------------------------------------------------
# brute force in bf16 storage mode: where the layer rounds, not only what it sums
# ---------------------------------------------------------------------------

def _py_rne_bf16(v):
    """v (a Python float) rounded to the nearest bf16 value, ties to even: 8 significant
    bits; below 2^-126 the spacing stays 2^-133. Python's round() breaks ties to even."""
    if v == 0.0:
        return 0.0
    _, e = math.frexp(v)                  # |v| in [2^(e-1), 2^e)
    q = 2.0 ** (max(e, -125) - 8)
    return round(v / q) * q


def _py_ffn_bf16(xrow, w1e, w3e, w2e):
    """One expert on one row with the bf16 storage points written out: every h value is
    rounded before fc2 reads it, every y value is rounded once. Returns (h, y)."""
    D, F = len(xrow), len(w1e)
    h = []
    for f in range(F):
        a = sum(float(xrow[d]) * float(w1e[f][d]) for d in range(D))
        b = sum(float(xrow[d]) * float(w3e[f][d]) for d in range(D))
        h.append(_py_rne_bf16(_py_silu(a) * b))
    y = [_py_rne_bf16(sum(h[f] * float(w2e[o][f]) for f in range(F))) for o in range(len(w2e))]
    return h, y


def brute_layer_bf16(inp):
    """Per-token layer output for given routing (topk_idx, topk_w; -1 slots skipped) in
    bf16 storage mode: the routed rows' h and y rounded as stored, the shared experts'
    h rounded and their summed output rounded once, then out[t] = sum_j w[t,j] y_j plus
    the stored shared output, rounded once. Returns (out, h per slot, y per slot, shared)."""
    x, idx, w = inp["x"], inp["topk_idx"], inp["topk_w"]
    T, D = x.shape
    out, hs, ys, sh = [], {}, {}, []
    for t in range(T):
        acc = [0.0] * D
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            if e < 0:
                continue
            h, y = _py_ffn_bf16(x[t], inp["w1"][e], inp["w3"][e], inp["w2"][e])
            hs[(t, j)], ys[(t, j)] = h, y
            acc = [acc[d] + float(w[t, j]) * y[d] for d in range(D)]
        s = [0.0] * D
        if "ws1" in inp:
            for s_ in range(inp["ws1"].shape[0]):
                w1s, w3s, w2s = inp["ws1"][s_], inp["ws3"][s_], inp["ws2"][s_]
                hsh = []
                for f in range(len(w1s)):
                    a = sum(float(x[t, d]) * float(w1s[f][d]) for d in range(D))
                    b = sum(float(x[t, d]) * float(w3s[f][d]) for d in range(D))
                    hsh.append(_py_rne_bf16(_py_silu(a) * b))
                s = [s[d] + sum(hsh[f] * float(w2s[d][f]) for f in range(len(w1s)))
                     for d in range(D)]
            s = [_py_rne_bf16(v) for v in s]
        sh.append(s)
        out.append([_py_rne_bf16(acc[d] + s[d]) for d in range(D)])
    return np.array(out), hs, ys, np.array(sh)


def _bf16_given_layer(seed, T=9, D=16, F=12, E=5, k=3, shared=True, holes=True):
    """bf16-representable inputs (values64 of bf16 bit patterns) with given routing,
    some -1 slots, top-k weights in float32."""
    inp = _tiny_layer(seed, T=T, D=D, F=F, E=E, k=k, shared=shared)
    for name in ("x", "w1", "w3", "w2", "ws1", "ws3", "ws2"):
        if name in inp:
            inp[name] = orc.round_bf16(inp[name].astype(np.float64)).astype(np.float32)
    rng = np.random.default_rng(seed + 100)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if holes:
        idx[rng.random((T, k)) < 0.25] = -1
    w = rng.random((T, k)).astype(np.float32)
    w[idx < 0] = 0.0
    inp["topk_idx"], inp["topk_w"] = idx, w
    del inp["wg"]
    return inp


def _check_bf16_storage_points(oracle, seed, **kw):
    inp = _bf16_given_layer(seed, **kw)
    k = inp["topk_idx"].shape[1]
    res = oracle.forward(inp, k=k, m_tile=4, dtype="bf16")
    out_b, hs, ys, sh_b = brute_layer_bf16(inp)
    for (t, j), h in hs.items():
        r = int(res["dst_row"][t, j])
        np.testing.assert_array_equal(res["h"][r], np.array(h), err_msg=f"h of slot {(t, j)}")
        np.testing.assert_array_equal(res["y_perm"][r], np.array(ys[(t, j)]),
                                      err_msg=f"y of slot {(t, j)}")
    if "ws1" in inp:
        np.testing.assert_array_equal(res["shared"], sh_b, err_msg="shared")
    np.testing.assert_array_equal(res["out"], out_b, err_msg="out")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bf16_storage_points_match_bruteforce(seed):
    _check_bf16_storage_points(orc, seed)


def test_bf16_storage_points_without_shared_or_holes():
    _check_bf16_storage_points(orc, 3, shared=False, holes=False, k=2, E=4)


def test_py_rne_bf16_agrees_with_torch_on_float32_values():
    # the brute force's rounding, checked against torch's float32 -> bf16 conversion
    rng = np.random.default_rng(8)
    a = np.concatenate([rng.standard_normal(3000), rng.standard_normal(300) * 1e-38,
                        [0.5 + 2.0 ** -9, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([_py_rne_bf16(float(v)) for v in a])
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(3)
    a = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.round_bf16(a.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_ties_to_even():
    # bf16 spacing at 1 is 2^-7: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1 (even);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6
    assert orc.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert orc.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert orc.round_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)
    # just above the halfway point rounds up
    assert orc.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7


# ---------------------------------------------------------------------------
# router logits: fixed float32 order
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D", [("f32", 128), ("f32", 96), ("f32", 1000), ("bf16", 512), ("bf16", 4096)])
def test_logits_within_forward_error_bound(dtype, D):
    rng = np.random.default_rng(D)
    T, E = 33, 7
    x = rng.standard_normal((T, D)).astype(np.float32)
    w = rng.standard_normal((E, D)).astype(np.float32)
    if dtype == "bf16":
        x = orc.round_bf16(x.astype(np.float64)).astype(np.float32)
        w = orc.round_bf16(w.astype(np.float64)).astype(np.float32)
    got = orc.router_logits(x, w, dtype).astype(np.float64)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    mag = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    V = 4 if dtype == "f32" else 8
    per_lane = math.ceil(D / (64 * V)) * V
    gamma = (per_lane + 6 + 1) * 2.0 ** -24 * 1.01
    assert np.all(np.abs(got - exact) <= gamma * mag)


def test_logits_zero_gate_and_one_hot():
    D, E = 256, 8
    x = np.random.default_rng(0).standard_normal((5, D)).astype(np.float32)
    z = orc.router_logits(x, np.zeros((E, D), np.float32), "f32")
    assert np.all(z == 0)
    wg = np.random.default_rng(1).standard_normal((E, D)).astype(np.float32)
    for d in (0, 3, 77, 255):
        onehot = np.zeros((1, D), np.float32)
        onehot[0, d] = 1.0
        np.testing.assert_array_equal(orc.router_logits(onehot, wg, "f32")[0], wg[:, d])


def test_logits_order_inside_a_lane_is_sequential():
    # D=512 float32: chunk c = d // 4 goes to lane c % 64, so d = 0, 1, 2 sit in lane 0 and
    # are added in that order: (1 + 2^-24) rounds to 1 (tie to even), then + 2^-24 -> 1.
    # Any other grouping of the three, or a correctly rounded sum, gives 1 + 2^-23.
    D = 512
    x = np.zeros((1, D), np.float32)
    w = np.zeros((1, D), np.float32)
    x[0, :3] = 1.0
    w[0, :3] = [1.0, 2.0 ** -24, 2.0 ** -24]
    assert orc.router_logits(x, w, "f32")[0, 0] == np.float32(1.0)
    w2 = w.copy()
    w2[0, :3] = [2.0 ** -24, 2.0 ** -24, 1.0]       # small terms first: they add up first
    assert orc.router_logits(x, w2, "f32")[0, 0] == np.float32(1 + 2.0 ** -23)


def test_logits_butterfly_pairs_far_lanes_first():
    # Lane 0 holds 1 (d = 0), lanes 32 and 48 hold 2^-24 each (d = 128, 192 for float32).
    # The butterfly first adds lane 32 to lane 0 (1 + 2^-24 -> 1) and lane 48 to lane 16,
    # then adds those: 1 + 2^-24 -> 1. A tree that joined lanes 32 and 48 first would
    # give 1 + 2^-23.
    D = 512
    x = np.zeros((1, D), np.float32)
    w = np.zeros((1, D), np.float32)
    for d, v in ((0, 1.0), (128, 2.0 ** -24), (192, 2.0 ** -24)):
        x[0, d] = 1.0
        w[0, d] = v
    assert orc.router_logits(x, w, "f32")[0, 0] == np.float32(1.0)
    # bf16 chunks are 8 wide: d = 256 and 384 are lanes 32 and 48
    xb = np.zeros((1, 1024), np.float32)
    wb = np.zeros((1, 1024), np.float32)
    for d, v in ((0, 1.0), (256, 2.0 ** -9), (384, 2.0 ** -9)):
        xb[0, d] = 2.0 ** -15 if d else 1.0
        wb[0, d] = v
    assert orc.router_logits(xb, wb, "bf16")[0, 0] == np.float32(1.0)


def test_logits_bias_added_last():
    x = np.ones((1, 64), np.float32)
    w = np.ones((2, 64), np.float32)
    b = np.array([0.5, -3.0], np.float32)
    np.testing.assert_array_equal(orc.router_logits(x, w, "f32", b)[0], [64.5, 61.0])


# ---------------------------------------------------------------------------
# softmax and top-k
# ---------------------------------------------------------------------------

def test_softmax_sums_to_one_and_is_shift_invariant():
    l = np.random.default_rng(0).standard_normal((50, 37)).astype(np.float32) * 4
    p = orc.softmax(l)
    assert np.all(np.abs(p.sum(1) - 1) < 37 * 2.0 ** -52)
    np.testing.assert_allclose(orc.softmax(l.astype(np.float64) + 11.5), p, rtol=1e-13)
    assert np.all(p > 0)


@pytest.mark.parametrize("E", [8, 32, 64])
def test_zero_gate_routes_uniformly_to_lowest_indices(E):
    T, D, k = 9, 128, 3
    x = np.random.default_rng(E).standard_normal((T, D)).astype(np.float32)
    idx, w, _ = orc.route(x, np.zeros((E, D), np.float32), k, "f32")
    assert np.all(idx == np.arange(k))
    assert np.all(w == 1.0 / E)          # exact: E is a power of two
    lay = orc.dispatch_layout(idx, E, 16)
    np.testing.assert_array_equal(lay["counts"], [T] * k + [0] * (E - k))


def test_topk_matches_python_sorted_with_ties():
    rng = np.random.default_rng(11)
    l = (rng.integers(-3, 4, size=(400, 9)) * 0.25).astype(np.float32)   # many ties
    l[0] = [0.0, -0.0, 0.0, -0.0, 0.0, -0.0, 0.0, -0.0, 0.0]
    for k in (1, 3, 9):
        idx = orc.select_topk(l, k)
        for t in range(l.shape[0]):
            ref = sorted(range(9), key=lambda e: (-float(l[t, e]), e))[:k]
            assert list(idx[t]) == ref


def test_duplicate_gate_rows_prefer_lower_index():
    D, E = 64, 6
    rng = np.random.default_rng(2)
    wg = rng.standard_normal((E, D)).astype(np.float32)
    wg[4] = wg[1]
    x = rng.standard_normal((40, D)).astype(np.float32)
    idx, _, logits = orc.route(x, wg, E, "f32")
    for t in range(40):
        pos = {e: j for j, e in enumerate(idx[t])}
        assert pos[1] < pos[4]
        assert logits[t, 1] == logits[t, 4]


def test_single_expert_and_renorm():
    x = np.random.default_rng(0).standard_normal((5, 64)).astype(np.float32)
    idx, w, _ = orc.route(x, np.ones((1, 64), np.float32), 1, "f32")
    assert np.all(idx == 0) and np.all(w == 1.0)
    wg = np.random.default_rng(1).standard_normal((8, 64)).astype(np.float32)
    _, w, _ = orc.route(x, wg, 3, "f32", renorm=True)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)


# ---------------------------------------------------------------------------
# dispatch metadata and permute
# ---------------------------------------------------------------------------

def _py_layout(idx, E, mt, m_cap):
    """Stable counting sort written as plain loops."""
    T, k = len(idx), len(idx[0])
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            if idx[t][j] >= 0:
                counts[idx[t][j]] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + (counts[e] + mt - 1) // mt * mt)
    seen = [0] * E
    dst = [[-1] * k for _ in range(T)]
    src = [-1] * m_cap
    for t in range(T):
        for j in range(k):
            e = idx[t][j]
            if e >= 0:
                r = offsets[e] + seen[e]
                seen[e] += 1
                dst[t][j] = r
                src[r] = t * k + j
    tiles = [-1] * (m_cap // mt)
    for q in range(m_cap // mt):
        for e in range(E):
            if offsets[e] <= q * mt < offsets[e + 1]:
                tiles[q] = e
    return counts, offsets, dst, src, tiles


@pytest.mark.parametrize("T,k,E,mt,holes", [(50, 3, 7, 4, False), (33, 2, 5, 16, True), (1, 1, 1, 16, False),
                                            (64, 4, 4, 8, True), (20, 6, 6, 1, False)])
def test_layout_matches_loop_counting_sort(T, k, E, mt, holes):
    rng = np.random.default_rng(T * 7 + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if holes:
        idx[rng.random(idx.shape) < 0.2] = -1
    m_cap = orc.capacity(T, k, E, mt)
    lay = orc.dispatch_layout(idx, E, mt, m_cap)
    c, o, d, s, tiles = _py_layout(idx.tolist(), E, mt, m_cap)
    np.testing.assert_array_equal(lay["counts"], c)
    np.testing.assert_array_equal(lay["offsets"], o)
    np.testing.assert_array_equal(lay["dst_row"], d)
    np.testing.assert_array_equal(lay["src_row"], s)
    np.testing.assert_array_equal(lay["tile_expert"], tiles)


def test_layout_invariants_and_permute_roundtrip():
    rng = np.random.default_rng(5)
    T, k, E, mt, D = 300, 4, 9, 16, 40
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[::7, 1] = -1
    lay = orc.dispatch_layout(idx, E, mt)
    counts, off = lay["counts"].astype(int), lay["offsets"].astype(int)
    assert counts.sum() == (idx >= 0).sum()
    assert np.all(off % mt == 0)
    np.testing.assert_array_equal(np.diff(off), -(-counts // mt) * mt)
    x = rng.standard_normal((T, D)).astype(np.float32)
    xp = orc.permute(x, lay)
    dst, src = lay["dst_row"], lay["src_row"]
    for t in range(T):
        for j in range(k):
            if dst[t, j] >= 0:
                assert src[dst[t, j]] == t * k + j
                assert np.array_equal(xp[dst[t, j]].view(np.uint32), x[t].view(np.uint32))
    # the unpermute (gather back by dst) of the permuted rows is the identity
    back = xp[np.where(dst >= 0, dst, 0)]
    ok = dst >= 0
    np.testing.assert_array_equal(back[ok], np.repeat(x[:, None, :], k, axis=1)[ok])
    pad = src < 0
    assert np.all(xp[pad] == 0)
    # rows inside a segment ascend in flat slot order
    for e in range(E):
        seg = src[off[e]:off[e] + counts[e]]
        assert np.all(np.diff(seg) > 0) and np.all(idx.reshape(-1)[seg] == e)


def test_capacity_is_the_tight_worst_case():
    # the largest padded total over every way of spreading N slots over E experts
    for T, k, E, mt in [(3, 2, 3, 4), (5, 1, 4, 3), (4, 3, 5, 2), (2, 2, 6, 4), (6, 2, 2, 5)]:
        N = T * k

        def best(n, e):
            if e == 1:
                return -(-n // mt) * mt
            return max(-(-c // mt) * mt + best(n - c, e - 1) for c in range(n + 1))
        assert orc.capacity(T, k, E, mt) == best(N, E), (T, k, E, mt)


def test_page4_expert_parallel_split_example():
    g = json.load(open(os.path.join(GOLDEN, "ep_split_worked_example.json")))
    D, eb, per_src = g["D"], g["elem_bytes"], g["tokens_per_source"]
    for name, case in g["cases"].items():
        split = case["per_source_split"]
        idx = np.array([[0]] * split[0] + [[1]] * split[1], dtype=np.int32)
        idx = np.concatenate([idx, idx])                    # two sources, same split
        for mt in (16, 128):
            lay = orc.dispatch_layout(idx, 2, mt)
            np.testing.assert_array_equal(lay["counts"], case["expert_rows"])
            np.testing.assert_array_equal(lay["offsets"], g["offsets_derived"][f"{name}_mtile{mt}"])
        # each source ships its 64 tokens; under skew the hot and cold experts return
        # their rows
        assert per_src * D * eb == g["bytes_KiB"]["dispatch_per_source"] * 1024
        if name == "skewed":
            hot, cold = case["expert_rows"]
            assert hot * D * eb == g["bytes_KiB"]["combine_hot_skewed"] * 1024
            assert cold * D * eb == g["bytes_KiB"]["combine_cold_skewed"] * 1024
        x = np.random.default_rng(0).standard_normal((2 * per_src, D)).astype(np.float32)
        lay = orc.dispatch_layout(idx, 2, 16)
        xp = orc.permute(x, lay)
        off, c = lay["offsets"], lay["counts"]
        for e in range(2):
            assert xp[off[e]:off[e] + c[e]].nbytes == case["expert_rows"][e] * D * eb


def test_out_of_range_index_rejected():
    with pytest.raises(ValueError):
        orc.dispatch_layout(np.array([[0, 3]], np.int32), 3, 4)
    with pytest.raises(ValueError):
        orc.dispatch_layout(np.array([[0, -2]], np.int32), 3, 4)


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------

def test_silu_matches_torch_and_limits():
    a = np.linspace(-30, 30, 2001)
    ref = torch.nn.functional.silu(torch.from_numpy(a)).numpy()
    np.testing.assert_allclose(orc.silu(a), ref, rtol=1e-14, atol=1e-300)
    assert orc.silu(np.array([0.0]))[0] == 0.0
    assert orc.silu(np.array([-800.0]))[0] == 0.0


def test_single_expert_top1_is_a_dense_swiglu_ffn():
    rng = np.random.default_rng(8)
    T, D, F = 20, 32, 48
    inp = {"x": rng.standard_normal((T, D)).astype(np.float32),
           "wg": rng.standard_normal((1, D)).astype(np.float32),
           "w1": rng.standard_normal((1, F, D)).astype(np.float32) / 6,
           "w3": rng.standard_normal((1, F, D)).astype(np.float32) / 6,
           "w2": rng.standard_normal((1, D, F)).astype(np.float32) / 7}
    res = orc.forward(inp, k=1, m_tile=16, dtype="f32")
    xt = torch.from_numpy(inp["x"]).double()
    a = torch.nn.functional.linear(xt, torch.from_numpy(inp["w1"][0]).double())
    b = torch.nn.functional.linear(xt, torch.from_numpy(inp["w3"][0]).double())
    ref = torch.nn.functional.linear(torch.nn.functional.silu(a) * b, torch.from_numpy(inp["w2"][0]).double())
    err = np.abs(res["out"] - ref.numpy()).max() / np.abs(ref.numpy()).max()
    assert err < 1e-6
    assert np.all(res["topk_w"] == 1.0)


def test_shared_experts_concatenated_along_f_equal_their_sum():
    rng = np.random.default_rng(9)
    T, D, Fs = 12, 16, 8
    x = rng.standard_normal((T, D)).astype(np.float32)
    ws1, ws3 = rng.standard_normal((2, 2, Fs, D)).astype(np.float32) / 4
    ws2 = rng.standard_normal((2, D, Fs)).astype(np.float32) / 3
    s = orc.shared_experts(x, ws1, ws3, ws2, "f32")
    cat = orc.shared_experts(x, np.concatenate(ws1)[None], np.concatenate(ws3)[None],
                             np.concatenate(ws2, axis=1)[None], "f32")
    np.testing.assert_allclose(cat, s, rtol=0, atol=2e-7 * np.abs(s).max())


def test_pad_rows_give_exact_zero_and_bf16_storage_points():
    inp = _tiny_layer(4, T=9, D=16, F=8, E=3, k=2)
    for name in ("x", "wg", "w1", "w3", "w2"):
        inp[name] = orc.round_bf16(inp[name].astype(np.float64)).astype(np.float32)
    res = orc.forward(inp, k=2, m_tile=8, dtype="bf16")
    pad = res["src_row"] < 0
    assert np.all(res["h"][pad] == 0) and np.all(res["y_perm"][pad] == 0)
    for key in ("h", "y_perm", "out"):
        np.testing.assert_array_equal(orc.round_bf16(res[key]), res[key])


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------

def _random_routing(rng, T, k, E):
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    return idx, w


def test_combine_is_adjoint_of_weighted_dispatch():
    rng = np.random.default_rng(12)
    T, k, E, D = 40, 3, 6, 10
    idx, w = _random_routing(rng, T, k, E)
    lay = orc.dispatch_layout(idx, E, 4)
    Y = rng.standard_normal((lay["m_cap"], D))
    z = rng.standard_normal((T, D))
    comb = orc.combine(Y, lay["dst_row"], w, "f32")
    # weighted dispatch: row dst[t,j] receives w[t,j] * z[t]
    disp = np.zeros_like(Y)
    for t in range(T):
        for j in range(k):
            disp[lay["dst_row"][t, j]] += w[t, j] * z[t]
    lhs = float((comb * z).sum())
    rhs = float((Y * disp).sum())
    assert abs(lhs - rhs) <= 1e-6 * (np.abs(comb).sum() * np.abs(z).max())


def test_combine_one_hot_weight_copies_rows_exactly():
    rng = np.random.default_rng(13)
    T, k, E, D = 30, 2, 5, 12
    idx, _ = _random_routing(rng, T, k, E)
    w = np.zeros((T, k))
    w[:, 1] = 1.0
    lay = orc.dispatch_layout(idx, E, 4)
    Y = orc.round_bf16(rng.standard_normal((lay["m_cap"], D)))
    out = orc.combine(Y, lay["dst_row"], w, "bf16")
    np.testing.assert_array_equal(out, Y[lay["dst_row"][:, 1]])


def test_combine_skips_missing_slots_and_adds_shared():
    Y = np.arange(12, dtype=np.float64).reshape(4, 3)
    dst = np.array([[2, -1], [-1, 0]], np.int32)
    w = np.array([[0.5, 9.0], [9.0, 2.0]])
    sh = np.ones((2, 3))
    out = orc.combine(Y, dst, w, "f32", sh)
    np.testing.assert_array_equal(out, [[4.0, 4.5, 5.0], [1.0, 3.0, 5.0]])


def test_top_all_experts_without_renorm_is_probability_weighted_mixture():
    inp = _tiny_layer(21, T=6, D=16, F=8, E=4, k=4)
    res = orc.forward(inp, k=4, m_tile=4, dtype="f32")
    p = orc.softmax(res["logits"])
    mix = np.zeros((6, 16))
    for e in range(4):
        _, y = orc.expert_swiglu(inp["x"], inp["w1"][e], inp["w3"][e], inp["w2"][e], "f32")
        mix += p[:, e:e + 1] * y
    np.testing.assert_allclose(res["out"], mix, rtol=0, atol=1e-6 * np.abs(mix).max())


def test_token_outputs_equal_forward_rows():
    inp = _tiny_layer(30, T=15, D=16, F=8, E=4, k=2, shared=True)
    res = orc.forward(inp, k=2, m_tile=4, dtype="f32")
    toks = np.array([0, 4, 14])
    out, hs, ys = orc.token_outputs(toks, inp["x"], res["topk_idx"], res["topk_w"], inp["w1"],
                                    inp["w3"], inp["w2"], "f32",
                                    (inp["ws1"], inp["ws3"], inp["ws2"]))
    np.testing.assert_allclose(out, res["out"][toks], rtol=0, atol=1e-12)
    for (t, j), y in ys.items():
        np.testing.assert_allclose(y, res["y_perm"][res["dst_row"][t, j]], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# masked layout (decode)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E,cap", [(20, 2, 5, 16), (33, 3, 4, 8), (7, 1, 3, 16), (64, 4, 8, 4)])
def test_masked_layout_matches_loop_and_contiguous_ranks(T, k, E, cap):
    rng = np.random.default_rng(T * 7 + cap)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, k)) < 0.15] = -1
    lay = orc.masked_layout(idx, E, cap)
    # plain loops: each expert's slots in flat order t*k+j fill its slab from row e*cap
    fill = [0] * E
    dropped = 0
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                assert lay["dst_row"][t, j] == -1
                continue
            if fill[e] < cap:
                assert lay["dst_row"][t, j] == e * cap + fill[e]
                assert lay["src_row"][e * cap + fill[e]] == t * k + j
            else:
                assert lay["dst_row"][t, j] == -1
                dropped += 1
            fill[e] += 1
    assert lay["dropped"] == dropped
    assert list(lay["counts"]) == [min(c, cap) for c in fill]
    for e in range(E):
        assert np.all(lay["src_row"][e * cap + min(fill[e], cap):(e + 1) * cap] == -1)
    # same stable ranks as the contiguous layout
    con = orc.dispatch_layout(idx, E, 16)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if e >= 0 and lay["dst_row"][t, j] >= 0:
                assert lay["dst_row"][t, j] - e * cap == con["dst_row"][t, j] - con["offsets"][e]


def test_masked_forward_equals_contiguous_forward_when_nothing_drops():
    inp = _tiny_layer(31, T=15, D=16, F=8, E=4, k=2, shared=True)
    a = orc.forward(inp, k=2, m_tile=4, dtype="f32")
    b = orc.forward_masked(inp, k=2, cap=15, dtype="f32")
    assert b["dropped"] == 0
    np.testing.assert_array_equal(a["out"], b["out"])
    for t in range(15):
        for j in range(2):
            np.testing.assert_array_equal(a["y_perm"][a["dst_row"][t, j]],
                                          b["y_perm"][b["dst_row"][t, j]])


def test_masked_forward_drops_slots_past_capacity_like_brute_force():
    inp = _tiny_layer(32, T=12, D=16, F=8, E=3, k=2)
    cap = 3
    res = orc.forward_masked(inp, k=2, cap=cap, dtype="f32")
    assert res["dropped"] > 0
    idx, w = res["topk_idx"], res["topk_w"]
    seen = [0, 0, 0]
    ref = np.zeros((12, 16))
    for t in range(12):
        for j in range(2):
            e = int(idx[t, j])
            if seen[e] < cap:
                ref[t] += w[t, j] * np.asarray(
                    _py_ffn(inp["x"][t], inp["w1"][e], inp["w3"][e], inp["w2"][e]))
            seen[e] += 1
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-5 * np.abs(ref).max())


# ---------------------------------------------------------------------------
# FP8 (e4m3) payload with MX block scales
# ---------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_float8_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3_round_matches_torch_float8_rounding():
    rng = np.random.default_rng(71)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.3, 20000),
                        # exact halfway points between neighbouring codes (ties to even)
                        (orc.e4m3_decode(np.arange(0, 0x7E)) + orc.e4m3_decode(np.arange(1, 0x7F))) / 2,
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -6]])
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.e4m3_round(v), ref)
    codes = orc.e4m3_encode(orc.e4m3_round(v))
    np.testing.assert_array_equal(codes, torch.from_numpy(v).to(torch.float8_e4m3fn)
                                  .view(torch.uint8).numpy())


def test_mx_scale_is_the_smallest_power_that_avoids_saturation():
    rng = np.random.default_rng(72)
    x = (rng.standard_normal((40, 96)) * 10.0 ** rng.uniform(-6, 6, (40, 1))).astype(np.float32)
    x[3] = 0.0                                   # an all-zero row: every block zero
    x[5, :32] = 448.0                            # exactly at the limit: scale 2^0
    x[6, 32:64] = 449.0                          # just above: scale 2^1
    q, s = orc.mx_quantize(x)
    for r in range(40):
        for b in range(3):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                assert s[r, b] == 0 and not np.any(q[r, 32 * b:32 * b + 32] & 0x7F)
                continue
            X = -127
            while amax > 448.0 * 2.0 ** X:        # plain search for the smallest X
                X += 1
            assert s[r, b] == X + 127, (r, b)
            ref = torch.from_numpy(blk / 2.0 ** X).to(torch.float8_e4m3fn).view(torch.uint8)
            np.testing.assert_array_equal(q[r, 32 * b:32 * b + 32], ref.numpy())
    assert s[5, 0] == 127 and s[6, 1] == 128
    d = orc.mx_dequantize(q, s)
    # relative error of e4m3 rounding: at most 2^-4 where the scaled value is normal
    scaled = np.abs(x.astype(np.float64)) / 2.0 ** (np.repeat(s, 32, axis=1) - 127.0)
    normal = scaled >= 2.0 ** -6
    assert np.all(np.abs(d - x)[normal] <= 2.0 ** -4 * np.abs(x[normal]))


def test_mx_fc1_equals_the_swiglu_of_the_dequantized_operands():
    rng = np.random.default_rng(73)
    A = rng.standard_normal((9, 64)).astype(np.float32)
    w1 = (rng.standard_normal((12, 64)) / 8).astype(np.float32)
    w3 = (rng.standard_normal((12, 64)) / 8).astype(np.float32)
    (aq, as_), (q1, s1), (q3, s3) = orc.mx_quantize(A), orc.mx_quantize(w1), orc.mx_quantize(w3)
    got = orc.expert_fc1_mx(aq, as_, q1, s1, q3, s3)
    Ad = torch.from_numpy(orc.mx_dequantize(aq, as_))
    ref = (torch.nn.functional.silu(Ad @ torch.from_numpy(orc.mx_dequantize(q1, s1)).T)
           * (Ad @ torch.from_numpy(orc.mx_dequantize(q3, s3)).T)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_mx_forward_equals_bf16_forward_on_exactly_representable_inputs():
    # inputs that are e4m3 values times one power of two per 32-block quantize exactly,
    # so the FP8 path must reproduce the bf16 layer bit for bit
    rng = np.random.default_rng(74)
    T, D, F, E, k = 20, 64, 32, 4, 2
    pick = lambda shape, p: orc.e4m3_decode(rng.integers(0, 0x70, size=shape)) * \
        np.where(rng.random(shape) < 0.5, -1, 1) * 2.0 ** p
    inp = {"x": pick((T, D), -4).astype(np.float32),
           "wg": (rng.standard_normal((E, D)) / 8).astype(np.float32),
           "w1": pick((E, F, D), -9).astype(np.float32), "w3": pick((E, F, D), -9).astype(np.float32),
           "w2": (rng.standard_normal((E, D, F)) / 8).astype(np.float32)}
    for n in inp:   # every value above is also a bf16 value; round the rest to bf16
        inp[n] = orc.round_bf16(inp[n]).astype(np.float32)
    a = orc.forward(inp, k=k, m_tile=16, dtype="bf16")
    b = orc.forward_mxfp8(inp, k=k, m_tile=16)
    np.testing.assert_array_equal(orc.mx_dequantize(b["xq"], b["xs"]), inp["x"])
    np.testing.assert_array_equal(a["h"], b["h"])
    np.testing.assert_array_equal(a["out"], b["out"])


def test_token_outputs_mx_equal_forward_rows():
    inp = _tiny_layer(33, T=15, D=64, F=16, E=4, k=2, shared=True)
    for n in inp:
        inp[n] = orc.round_bf16(inp[n]).astype(np.float32)
    res = orc.forward_mxfp8(inp, k=2, m_tile=16)
    toks = np.array([1, 7, 14])
    out = orc.token_outputs_mx(toks, inp["x"], res["topk_idx"], res["topk_w"], inp["w1"],
                               inp["w3"], inp["w2"], (inp["ws1"], inp["ws3"], inp["ws2"]))
    # the same float64 arithmetic batched differently: equal up to a last-bit bf16 flip
    np.testing.assert_allclose(out, res["out"][toks], rtol=0, atol=2 ** -7 * np.abs(out).max())
