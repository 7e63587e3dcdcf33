"""GPU parity of the FP8 payload (e4m3 codes with MX block scales) against the oracle.

Bar: codes and scales bit-exact (the quantization is a deterministic rounding), in both
scale layouts (rows, and the GEMM's k-step words, compared after reshuffling them back
into rows); the permute's metadata, code rows and scales bit-exact; fc1's h and the layer output
within max|gpu - ref| / max|ref| <= 2e-2 (float32 accumulation of the same dequantized
products, bf16 storage)."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_amd as rpg
import workloads as W
from oracle import moe_oracle as orc
from tests import _parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", [rpg.MOE_MX_ROWS, rpg.MOE_MX_KSTEPS])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_quantize_matches_oracle_bit_for_bit(dt, layout):
    P.log(f"[mx] quantize {dt} layout {layout}")
    rng = np.random.default_rng(81)
    x = (rng.standard_normal((300, 512)) * 10.0 ** rng.uniform(-8, 8, (300, 1))).astype(np.float32)
    x[4] = 0.0
    x[5, :32] = 448.0
    x[6, 32:64] = -449.0
    x[7, 64:96] = 2.0 ** -20 * rng.integers(-9, 9, 32)
    if dt == "bf16":
        x = W.f32_to_bf16_bits(x)
    q, s = rpg.moe_quantize_mxfp8(P.to_dev(x), layout=layout)
    torch.cuda.synchronize()
    rq, rs = orc.mx_quantize(x)
    s = P.to_host(s)
    np.testing.assert_array_equal(P.mx_rows(s) if layout == rpg.MOE_MX_KSTEPS else s, rs)
    np.testing.assert_array_equal(P.to_host(q), rq)


def _layer_case(name):
    cases = {
        "dense8": W.shrink(W.preset("dense8_bf16"), T=512, D=512, F=1024),
        "fine64_shared2": W.shrink(W.preset("fine64_shared2_bf16"), T=389, D=512, F=320,
                                   F_shared=192),
        "skew32_zipf": W.shrink(W.preset("skew32_zipf_bf16"), T=1024, D=512, F=256),
        "etp_shard32": W.shrink(W.preset("etp_shard32_bf16"), D=1024, F=512, poisson_mean=40.0),
        "dense8_mt256": W.shrink(W.preset("dense8_bf16"), T=520, D=512, F=512, m_tile=256),
        "skew32_mt32": W.shrink(W.preset("skew32_zipf_bf16"), T=700, D=512, F=384, m_tile=32),
    }
    return cases[name]


@pytest.mark.parametrize("name", ["dense8", "fine64_shared2", "skew32_zipf", "etp_shard32",
                                  "dense8_mt256", "skew32_mt32"])
@pytest.mark.parametrize("split_k", [True, False])
def test_mxfp8_layer_parity(name, split_k):
    cfg = _layer_case(name)
    P.log(f"[mx] layer {name} split_k={split_k}: {cfg}")
    inp = W.generate(cfg, seed=0)
    cfg = inp["cfg"]
    ref = orc.forward_mxfp8(inp, cfg.k, cfg.m_tile)
    d = {n: P.to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    sw = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"]) if "ws1" in d else None
    kw = dict(topk_idx=d["topk_idx"], topk_w=d["topk_w"]) if "topk_idx" in d else \
        dict(wg=d["wg"], bias=d.get("bias"))
    mw = rpg.MxWeights.quantize(d["w1"], d["w3"])
    g = rpg.moe_layer_mxfp8(d["x"], mw, d["w2"], cfg.k, cfg.m_tile, shared=sw, split_k=split_k,
                            **kw)
    torch.cuda.synchronize()
    h = {n: P.to_host(v) if isinstance(v, torch.Tensor) else v for n, v in g.items()}
    for key in ("xq", "xs"):
        np.testing.assert_array_equal(h[key], ref[key], err_msg=key)
    for key in ("w1q", "w3q"):
        np.testing.assert_array_equal(P.to_host(getattr(mw, key)), ref[key], err_msg=key)
    for key in ("w1s", "w3s"):   # k-step words over the E*F rows
        got = P.mx_rows(P.to_host(getattr(mw, key))).reshape(ref[key].shape)
        np.testing.assert_array_equal(got, ref[key], err_msg=key)
    for key in ("counts", "offsets", "dst_row", "src_row", "tile_expert"):
        np.testing.assert_array_equal(h[key], ref[key], err_msg=key)
    used = int(ref["offsets"][-1])
    np.testing.assert_array_equal(h["xq_perm"][:used], ref["xq_perm"][:used])
    np.testing.assert_array_equal(P.mx_rows(h["xs_perm"])[:used], ref["xs_perm"][:used])
    pad = ref["src_row"][:used] < 0
    hv = orc.values64(h["h"][:used])
    assert np.all(np.isfinite(hv)) and np.all(hv[pad] == 0)
    e = P.rel_err(h["h"][:used], ref["h"][:used])
    assert e <= P.TOL["bf16"], f"h: rel err {e:.3e}"
    e = P.rel_err(h["out"], ref["out"])
    assert e <= P.TOL["bf16"], f"out: rel err {e:.3e}"


def test_mxfp8_permute_large_table():
    # the FP8 permute with a histogram table large enough to be prefix-summed over its
    # blocks first (16384 tokens over 256 experts: 64 blocks x 256 entries), -1 slots
    # among them: metadata, code rows and scales bit-exact, pad rows zero bytes
    T, E, k, D, mt = 16384, 256, 2, 128, 64
    P.log(f"[mx] permute T={T} E={E} k={k} D={D} m_tile={mt}")
    rng = np.random.default_rng(5)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    idx[rng.random((T, k)) < 0.05] = -1
    xq = rng.integers(0, 256, size=(T, D), dtype=np.uint8)
    xs = rng.integers(100, 140, size=(T, D // 32), dtype=np.uint8)
    lay = orc.dispatch_layout(idx, E, mt)
    g = rpg.moe_permute_mxfp8(P.to_dev(xq), P.to_dev(xs), P.to_dev(idx), E, mt)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "dst_row", "src_row", "tile_expert"):
        np.testing.assert_array_equal(P.to_host(g[key]), lay[key], err_msg=key)
    assert int(P.to_host(g["dev_err"])[0]) == 0
    used = int(lay["offsets"][-1])
    rows = lay["src_row"][:used]
    tok = np.where(rows >= 0, rows // k, 0)
    gq = P.to_host(g["xq_perm"])[:used]
    gs = P.mx_rows(P.to_host(g["xs_perm"]))[:used]
    np.testing.assert_array_equal(gq, np.where((rows >= 0)[:, None], xq[tok], 0))
    np.testing.assert_array_equal(gs, np.where((rows >= 0)[:, None], xs[tok], 0))


def test_mxfp8_full_size_dense8_sampled():
    """The dense 8-expert workload at full size, in the bench's launch configuration:
    routing and layout bit-exact; 4 sampled tokens' outputs against the oracle."""
    cfg = W.preset("dense8_bf16")
    P.log("[mx] full-size dense8: generating")
    inp = W.generate(cfg, seed=0)
    idx, w, _ = orc.route(inp["x"], inp["wg"], cfg.k, "bf16")
    d = {n: P.to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    mw = rpg.MxWeights.quantize(d["w1"], d["w3"])
    g = rpg.moe_layer_mxfp8(d["x"], mw, d["w2"], cfg.k, cfg.m_tile, wg=d["wg"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(P.to_host(g["topk_idx"]), idx)
    lay = orc.dispatch_layout(idx, cfg.E, cfg.m_tile)
    np.testing.assert_array_equal(P.to_host(g["offsets"]), lay["offsets"])
    # tokens whose experts are all among two experts, so the oracle quantizes only those
    rng = np.random.default_rng(5)
    pair = set(rng.choice(cfg.E, 2, replace=False).tolist())
    cand = [t for t in range(cfg.T) if set(idx[t].tolist()) <= pair]
    toks = np.sort(rng.choice(cand, min(4, len(cand)), replace=False))
    P.log(f"[mx] full-size dense8: oracle on tokens {toks.tolist()} (experts {sorted(pair)})")
    out = orc.token_outputs_mx(toks, inp["x"], idx, w, inp["w1"], inp["w3"], inp["w2"])
    got = P.to_host(g["out"].index_select(0, torch.from_numpy(toks).cuda()))
    e = P.rel_err(got, out)
    P.log(f"[mx] full-size dense8: out rel err {e:.2e}")
    assert e <= P.TOL["bf16"]


@pytest.mark.parametrize("name", ["fine64_shared2_bf16", "skew32_zipf_bf16", "etp_shard32_bf16"])
def test_mxfp8_full_size_sampled(name):
    """The other workloads at full size, in the bench's launch configuration (split-K
    workspace): routing and layout bit-exact; sampled tokens' outputs against the oracle,
    which quantizes only the experts those tokens use (tokens are picked among those
    whose experts all lie in the few most-used ones)."""
    cfg = W.preset(name)
    P.log(f"[mx] full-size {name}: generating")
    inp = W.generate(cfg, seed=0)
    cfg = inp["cfg"]
    d = {n: P.to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    if "topk_idx" in inp:
        idx, w = inp["topk_idx"], inp["topk_w"].astype(np.float64)
        kw = dict(topk_idx=d["topk_idx"], topk_w=d["topk_w"])
    else:
        idx, w, _ = orc.route(inp["x"], inp["wg"], cfg.k, "bf16", inp.get("bias"))
        kw = dict(wg=d["wg"], bias=d.get("bias"))
    sw = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"]) if "ws1" in d else None
    mw = rpg.MxWeights.quantize(d["w1"], d["w3"])
    g = rpg.moe_layer_mxfp8(d["x"], mw, d["w2"], cfg.k, cfg.m_tile, shared=sw, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(P.to_host(g["topk_idx"]), idx)
    lay = orc.dispatch_layout(idx, cfg.E, cfg.m_tile)
    for key in ("offsets", "dst_row"):
        np.testing.assert_array_equal(P.to_host(g[key]), lay[key], err_msg=key)
    freq = np.argsort(-np.bincount(idx[idx >= 0].ravel(), minlength=cfg.E), kind="stable")
    T = idx.shape[0]
    for n in (4, 6, 8, 12, 16, 24, cfg.E):
        top = set(freq[:n].tolist())
        cand = [t for t in range(T) if set(idx[t][idx[t] >= 0].tolist()) <= top and
                (idx[t] >= 0).any()]
        if len(cand) >= 4:
            break
    toks = np.sort(np.random.default_rng(7).choice(cand, 4, replace=False))
    P.log(f"[mx] full-size {name}: oracle on tokens {toks.tolist()} ({n} experts)")
    shared = (inp["ws1"], inp["ws3"], inp["ws2"]) if "ws1" in inp else None
    out = orc.token_outputs_mx(toks, inp["x"], idx, w, inp["w1"], inp["w3"], inp["w2"], shared)
    got = P.to_host(g["out"].index_select(0, torch.from_numpy(toks).cuda()))
    e = P.rel_err(got, out)
    P.log(f"[mx] full-size {name}: out rel err {e:.2e}")
    assert e <= P.TOL["bf16"]
