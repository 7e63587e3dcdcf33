"""GPU parity of the HIP path against the CPU oracle, element by element.

Bar: routing indices, logits, counts, offsets and maps bit-exact; x_perm bit-exact;
h, y, shared and out within max|gpu - ref| / max|ref| <= 1e-5 (float32) or 2e-2 (bf16
with float32 accumulation); top-k weights within 1e-6 relative; pad rows exactly zero;
no row left unwritten (outputs are NaN-poisoned before each call)."""
import dataclasses

import numpy as np
import pytest
import torch

import routing_permute_grouped_amd as rpg
import workloads as W
from oracle import moe_oracle as orc
from tests import _parity as P

pytestmark = pytest.mark.gpu

SMALL = {
    # the tiny float32 layer exactly as specified
    "tiny_f32": W.preset("tiny_f32"),
    # the same structures at sizes the oracle finishes in seconds: several tiles and
    # ragged tails (F not a multiple of 128, T not a multiple of 8 or of the M tile)
    "dense8": W.shrink(W.preset("dense8_bf16"), T=512, D=512, F=1024),
    "dense8_mt256": W.shrink(W.preset("dense8_bf16"), T=520, D=256, F=512, m_tile=256),
    "fine64_shared2": W.shrink(W.preset("fine64_shared2_bf16"), T=389, D=256, F=320, F_shared=192),
    "skew32_zipf": W.shrink(W.preset("skew32_zipf_bf16"), T=1024, D=512, F=256),
    "etp_shard32": W.shrink(W.preset("etp_shard32_bf16"), D=1024, F=512, poisson_mean=40.0),
    "f32_mt64": W.shrink(W.preset("tiny_f32"), T=300, D=192, F=320, E=6, k=3, m_tile=64),
    "f32_mt256": W.shrink(W.preset("tiny_f32"), T=77, D=64, F=128, E=5, k=2, m_tile=256),
    # bf16 at the smaller M tiles: segments start at multiples of 16, 32 or 64 rows and
    # end inside the kernel's 256-row tiles (and its 128-row half tiles)
    "bf16_mt16": W.shrink(W.preset("fine64_shared2_bf16"), T=300, D=256, F=320, F_shared=192,
                          m_tile=16),
    "bf16_mt32": W.shrink(W.preset("skew32_zipf_bf16"), T=700, D=256, F=384, m_tile=32),
    "bf16_mt64": W.shrink(W.preset("dense8_bf16"), T=900, D=512, F=768, m_tile=64),
    # the router past 64 experts: 256 experts top-8 (each lane holds 4 logits in the
    # softmax and top-k) and 1024 experts top-4 (16 per lane), a Zipf bias on the latter
    "route256_top8": W.MoEConfig("route256_top8", T=384, D=512, F=128, E=256, k=8, m_tile=16,
                                 dtype="bf16"),
    "route1024_top4": W.MoEConfig("route1024_top4", T=200, D=256, F=64, E=1024, k=4, m_tile=16,
                                  dtype="bf16", zipf_s=1.2),
    "route100_f32": W.MoEConfig("route100_f32", T=150, D=128, F=64, E=100, k=5, m_tile=16,
                                dtype="f32"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity_small(name):
    cfg = SMALL[name]
    P.log(f"[parity] {name}: {cfg}")
    inp = W.generate(cfg, seed=0)
    cfg = inp["cfg"]
    P.check_layer(inp, cfg.k, cfg.m_tile, cfg.dtype)


def test_renormalised_weights():
    cfg = W.shrink(W.preset("dense8_bf16"), T=256, D=256, F=256, k=3)
    P.log("[parity] renorm")
    inp = W.generate(cfg, seed=3)
    g = P.check_layer(inp, 3, 128, "bf16", renorm=True)
    np.testing.assert_allclose(g["topk_w"].sum(1), 1.0, rtol=1e-6)


def _bf16_layer(T, D, F, E, k, seed=1, m_tile=128):
    return W.generate(W.MoEConfig("edge", T=T, D=D, F=F, E=E, k=k, m_tile=m_tile, dtype="bf16"),
                      seed=seed)


def test_single_expert_top1_dense_ffn():
    P.log("[parity] E=1 k=1")
    P.check_layer(_bf16_layer(300, 256, 256, 1, 1), 1, 128, "bf16")


def test_top_all_experts():
    P.log("[parity] k=E=4")
    P.check_layer(_bf16_layer(200, 128, 192, 4, 4), 4, 128, "bf16")


def test_single_token():
    P.log("[parity] T=1")
    P.check_layer(_bf16_layer(1, 128, 128, 8, 2), 2, 128, "bf16")


def test_single_assignment_on_the_decode_gemm():
    """T=1, k=1 over 64 experts of D=F=512: the contiguous buffer holds 128 rows and the
    experts give 512 workgroups of 64 columns, so the grouped call takes the decode GEMM
    (contiguous segments); the one active expert's segment is 1 valid row + 127 pad rows."""
    P.log("[parity] T=1 k=1 E=64 decode GEMM")
    P.check_layer(_bf16_layer(1, 512, 512, 64, 1), 1, 128, "bf16")


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (40, 6), (256, 8), (1024, 3)])
def test_zero_gate_ties_send_every_token_to_lowest_experts(E, k):
    # all logits equal: every pick is a tie, resolved to the lowest index, also where
    # the experts spread over several logits per lane (E > 64)
    P.log(f"[parity] zero gate E={E} k={k}")
    mt = 128 if E <= 64 else 16
    T = 333 if E <= 64 else 64
    inp = _bf16_layer(T, 128, 128, E, k, m_tile=mt)
    inp["wg"][:] = 0
    g = P.check_layer(inp, k, mt, "bf16")
    assert np.all(g["topk_idx"] == np.arange(k))
    np.testing.assert_array_equal(g["counts"], [T] * k + [0] * (E - k))


@pytest.mark.parametrize("T,D,E,k,dtype,zipf", [
    # a whole number of 64-lane chunk steps per lane: the pipelined loop, up to 8
    # experts per wave (one token per wave below ~1000 tokens, two above)
    (333, 1024, 8, 2, "bf16", 0.0),     # one pair per lane
    (1201, 1024, 8, 2, "bf16", 0.0),
    (333, 2048, 8, 2, "bf16", 0.0),
    (130, 3072, 8, 2, "bf16", 0.0),     # three pairs
    (130, 4096, 6, 2, "bf16", 1.1),     # fewer than 8 experts, a bias
    (101, 512, 6, 3, "f32", 0.0),       # float32: 4 values per chunk
    (101, 1024, 8, 3, "f32", 0.0),
    # E > 8 with few tokens: blocks of 8 waves share 4 tokens
    (250, 2048, 32, 4, "bf16", 1.1),    # a bias, T % 4 != 0
    (77, 1024, 256, 8, "bf16", 0.0),    # four logits per lane in the top-k
    (90, 1024, 100, 5, "f32", 0.0),
    (128, 2048, 64, 6, "bf16", 0.0),    # the decode64 router shape
    # E > 8 with many tokens: blocks of 4 waves share 8 tokens
    (1500, 512, 32, 4, "bf16", 1.1),
    (1030, 1024, 256, 8, "bf16", 0.0),
    (1100, 512, 100, 5, "f32", 0.0),
    # an odd number of steps per lane (3 and 5): the last one after the pairs
    (64, 1536, 8, 2, "bf16", 0.0),
    (99, 2560, 40, 6, "bf16", 0.0),
    (70, 256, 8, 3, "f32", 0.0),        # one step per lane, no pair
    # 136 chunks: lanes take different counts, the plain loop
    (64, 1088, 8, 2, "bf16", 0.0),
    (50, 1088, 24, 4, "bf16", 1.1),
])
def test_router_chunk_loops(T, D, E, k, dtype, zipf):
    """The router alone against the oracle: logits and indices bit for bit, weights to
    float rounding, on both of its chunk loops (the pipelined loop, where every lane takes
    the same number of 64-lane steps, and the plain loop)."""
    P.log(f"[parity] router T={T} D={D} E={E} k={k} {dtype}")
    cfg = W.MoEConfig("router", T=T, D=D, F=64, E=E, k=k, m_tile=16, dtype=dtype, zipf_s=zipf)
    inp = W.router_inputs(cfg, seed=7)
    bias = inp.get("bias")
    idx, w, lg = rpg.moe_route(P.to_dev(inp["x"]), P.to_dev(inp["wg"]), k,
                               bias=None if bias is None else P.to_dev(bias), want_logits=True)
    torch.cuda.synchronize()
    ridx, rw, rlg = orc.route(inp["x"], inp["wg"], k, dtype, bias=bias)
    np.testing.assert_array_equal(P.to_host(lg).view(np.uint32), rlg.view(np.uint32))
    np.testing.assert_array_equal(P.to_host(idx), ridx)
    np.testing.assert_allclose(P.to_host(w), rw, rtol=1e-6, atol=1e-7)


def test_out_of_range_expert_ids_are_flagged_and_skipped():
    P.log("[parity] invalid expert ids")
    cfg = W.shrink(W.preset("etp_shard32_bf16"), D=256, F=256, poisson_mean=20.0)
    inp = W.generate(cfg, seed=2)
    bad = inp["topk_idx"].copy()
    bad[3, 0], bad[10, 2], bad[11, 5] = 32, -7, 1000
    clean = np.where((bad >= -1) & (bad < 32), bad, -1).astype(np.int32)
    inp_bad = dict(inp, topk_idx=bad)
    g = P.run_gpu(inp_bad, cfg.k, 128)
    assert int(g["dev_err"][0]) == 1
    ref = orc.forward(dict(inp, topk_idx=clean), k=cfg.k, m_tile=128, dtype="bf16")
    for key in ("counts", "offsets", "dst_row", "src_row", "tile_expert"):
        np.testing.assert_array_equal(g[key], ref[key], err_msg=key)
    assert P.rel_err(g["out"], ref["out"]) <= P.TOL["bf16"]


@pytest.mark.parametrize("T", [100, 300])
def test_masked_out_of_range_expert_ids_are_flagged_and_skipped(T):
    # the masked permute with bad expert ids, in its one-launch form (T <= 256) and its
    # three-launch form: flagged in bit 0 of dev_err, skipped like -1 slots
    P.log(f"[parity] masked permute, invalid expert ids, T={T}")
    E, k, cap = 16, 4, 32
    rng = np.random.default_rng(T)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[3, 0], idx[10, 2], idx[T - 1, 3] = E, -7, 1000
    clean = np.where((idx >= -1) & (idx < E), idx, -1).astype(np.int32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, 128)).astype(np.float32))
    ml = orc.masked_layout(clean, E, cap)
    gm = rpg.moe_permute_masked(P.to_dev(x), P.to_dev(idx), E, cap)
    torch.cuda.synchronize()
    for key in ("counts", "dst_row", "src_row"):
        np.testing.assert_array_equal(P.to_host(gm[key]), ml[key], err_msg=key)
    assert int(P.to_host(gm["dev_err"])[0]) == 1 | (2 if ml["dropped"] else 0)
    valid = ml["src_row"] >= 0
    np.testing.assert_array_equal(P.to_host(gm["x_masked"])[valid],
                                  x[ml["src_row"][valid] // k])


@pytest.mark.parametrize("ws_slots", [0, 10])
def test_grouped_gemm_workspace_sizes(ws_slots):
    # no workspace: every tile whole; 10 slots of 256x256 float32: fc1's 4 tiles split
    # in 2 k-ranges and fc2's 2 tiles in 4, unlike the default size (8 and 4)
    P.log(f"[parity] E=1 k=1 workspace {ws_slots} slots")
    P.check_layer(_bf16_layer(300, 256, 256, 1, 1), 1, 128, "bf16",
                  ws_bytes=ws_slots * 256 * 256 * 4)


def test_split_k_tail_agrees_with_whole_tiles():
    P.log("[parity] split-K tail vs whole tiles")
    inp = W.generate(SMALL["dense8"], seed=5)
    a = P.run_gpu(inp, 2, 128)
    b = P.run_gpu(inp, 2, 128, ws_bytes=0)
    used = int(a["offsets"][-1])
    # only the float32 summation order of the split tiles differs, so the two bf16
    # results are at most a rounding step or two apart
    for key in ("h", "y_perm"):
        assert P.rel_err(a[key][:used], orc.values64(b[key][:used])) <= 2.0 ** -7, key


# More tiles than workgroups: every workgroup runs several tiles back to back (the next
# tile's first k-step loaded during the current one's last step, stages alternating),
# half tiles follow full ones, and the last round is split over k.
MULTI_ROUND = {
    "dense8_multiround": W.shrink(W.preset("dense8_bf16"), T=4096, D=512, F=2048),
    "skew32_multiround": W.shrink(W.preset("skew32_zipf_bf16"), T=4096, D=512, F=1024),
}


@pytest.mark.parametrize("name", list(MULTI_ROUND))
def test_layer_parity_multi_round(name):
    cfg = MULTI_ROUND[name]
    P.log(f"[parity] {name}: {cfg}")
    inp = W.generate(cfg, seed=7)
    cfg = inp["cfg"]
    P.check_layer(inp, cfg.k, cfg.m_tile, cfg.dtype)


def test_max_experts_given_routing():
    # E = 1024 (the largest the library takes): the grouped GEMM's per-expert schedule
    # tables are full; ~1000 one-half-tile segments, F = 192 ragged against 128 columns
    cfg = W.shrink(W.preset("etp_shard32_bf16"), E=1024, k=8, D=128, F=192, poisson_mean=6.0)
    P.log(f"[parity] E=1024 given routing: {cfg}")
    inp = W.generate(cfg, seed=11)
    P.check_layer(inp, 8, 128, "bf16")


def test_grouped_gemm_stays_inside_m_cap_with_bad_offsets():
    # offsets that break the contract (decreasing, negative, past m_cap) only shrink the
    # work: nothing is written at or beyond m_cap rows
    P.log("[parity] grouped GEMM with out-of-contract offsets")
    E, D, F, m_cap, guard = 4, 256, 256, 1024, 256
    g = torch.Generator(device="cuda").manual_seed(3)
    xp = torch.randn(m_cap + guard, D, device="cuda", generator=g).to(torch.bfloat16)
    w1 = (torch.randn(E, F, D, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    w3 = (torch.randn(E, F, D, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(E, D, F, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    te = torch.zeros(m_cap // 128, dtype=torch.int32, device="cuda")
    ws = rpg.grouped_workspace(xp.device)
    for offs in ([0, 640, 256, 768, 5000], [-384, 128, -7, 896, 1024], [0, 384, 384, 2048, 900]):
        h = torch.full((m_cap + guard, F), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = torch.full((m_cap + guard, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        off = torch.tensor(offs, dtype=torch.int32, device="cuda")
        rpg.moe_grouped_swiglu(xp, off, te, w1, w3, w2, 128, m_cap=m_cap, h=h, y_perm=y,
                               workspace=ws)
        torch.cuda.synchronize()
        assert torch.isnan(h[m_cap:].float()).all() and torch.isnan(y[m_cap:].float()).all(), offs


def test_two_call_form_matches_one_call():
    # moe_grouped_fc1_swiglu then moe_grouped_fc2 run the same kernels as
    # moe_grouped_swiglu: identical bits
    P.log("[parity] fc1 + fc2 calls vs one grouped call")
    inp = W.generate(MULTI_ROUND["dense8_multiround"], seed=8)
    d = {n: P.to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    T, k, E = inp["x"].shape[0], 2, inp["w1"].shape[0]
    idx, w, _ = rpg.moe_route(d["x"], d["wg"], k)
    m_cap = rpg.moe_capacity(T, k, E, 128)
    p = rpg.moe_permute(d["x"], idx, E, 128, m_cap=m_cap)
    ws = rpg.grouped_workspace(d["x"].device)
    h1, y1 = rpg.moe_grouped_swiglu(p["x_perm"], p["offsets"], p["tile_expert"], d["w1"], d["w3"],
                                    d["w2"], 128, m_cap=m_cap, workspace=ws)
    F, D = inp["w1"].shape[1], inp["x"].shape[1]
    h2 = torch.empty((m_cap, F), dtype=d["x"].dtype, device="cuda")
    y2 = torch.empty((m_cap, D), dtype=d["x"].dtype, device="cuda")
    rpg.moe_grouped_fc1_swiglu(p["x_perm"], p["offsets"], p["tile_expert"], d["w1"], d["w3"], 128,
                               m_cap, h2, workspace=ws)
    rpg.moe_grouped_fc2(h2, p["offsets"], p["tile_expert"], d["w2"], 128, m_cap, y2, workspace=ws)
    torch.cuda.synchronize()
    used = int(p["offsets"][-1].item())
    assert torch.equal(h1[:used].view(torch.int16), h2[:used].view(torch.int16))
    assert torch.equal(y1[:used].view(torch.int16), y2[:used].view(torch.int16))


def test_two_streams_in_flight_match_serial():
    # the routed experts' grouped call and the shared experts' call in flight at once on
    # two streams, each with its own split-K workspace (the shared call's lone partial
    # round takes the split-K tail here), give the bits the same calls give one after the
    # other on one stream: a call keeps no state beyond the buffers it is handed
    P.log("[parity] routed and shared grouped calls on two streams")
    cfg = W.shrink(W.preset("fine64_shared2_bf16"), T=2048, D=512, F=512, F_shared=512)
    inp = W.generate(cfg, seed=11)
    d = {n: P.to_dev(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
    T, D, E, k = inp["x"].shape[0], inp["x"].shape[1], inp["w1"].shape[0], cfg.k
    dev = d["x"].device
    shared = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"])
    rows = rpg.DenseRows(T, 128, dev)
    idx, _, _ = rpg.moe_route(d["x"], d["wg"], k)
    m_cap = rpg.moe_capacity(T, k, E, 128)
    p = rpg.moe_permute(d["x"], idx, E, 128, m_cap=m_cap)
    ws_main, ws_side = rpg.grouped_workspace(dev), rpg.grouped_workspace(dev)
    F, Fs = inp["w1"].shape[1], shared.w1.shape[1]

    def outputs():
        return (torch.empty((m_cap, F), dtype=d["x"].dtype, device=dev),
                torch.empty((m_cap, D), dtype=d["x"].dtype, device=dev),
                torch.empty((rows.m_cap, Fs), dtype=d["x"].dtype, device=dev),
                torch.empty((rows.m_cap, D), dtype=d["x"].dtype, device=dev))

    def routed(o, ws, stream):
        rpg.moe_grouped_swiglu(p["x_perm"], p["offsets"], p["tile_expert"], d["w1"], d["w3"],
                               d["w2"], 128, m_cap=m_cap, h=o[0], y_perm=o[1], workspace=ws,
                               stream=stream)

    def shared_call(o, ws, stream):
        rpg.moe_grouped_swiglu(d["x"], rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                               shared.w2, 128, m_cap=rows.m_cap, h=o[2], y_perm=o[3],
                               workspace=ws, stream=stream, rows_used=T)

    main = torch.cuda.current_stream()
    a, b = outputs(), outputs()
    torch.cuda.synchronize()
    routed(a, ws_main, main)
    shared_call(a, ws_main, main)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)   # default priority
    go, done = torch.cuda.Event(), torch.cuda.Event()
    go.record(main)
    side.wait_event(go)
    shared_call(b, ws_side, side)
    done.record(side)
    routed(b, ws_main, main)
    main.wait_event(done)
    torch.cuda.synchronize()
    used = int(p["offsets"][-1].item())
    for i, n in ((0, used), (1, used), (2, T), (3, T)):
        assert torch.equal(a[i][:n].view(torch.int16), b[i][:n].view(torch.int16)), i


def test_bitwise_run_to_run_determinism():
    P.log("[parity] determinism")
    inp = W.generate(SMALL["fine64_shared2"], seed=4)
    a = P.run_gpu(inp, 6, 128)
    b = P.run_gpu(inp, 6, 128)
    used = int(a["offsets"][-1])
    for key in ("logits", "topk_idx", "topk_w", "dst_row", "src_row", "shared", "out"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    for key in ("x_perm", "h", "y_perm"):
        np.testing.assert_array_equal(a[key][:used], b[key][:used], err_msg=key)


@pytest.mark.parametrize("split", [True, False])
def test_grouped_calls_skip_pad_rows_given_counts(split):
    # pad rows hold NaN: with counts the tiled kernels must neither read them nor let them
    # reach any output (h, y_perm pad rows exactly 0), while token rows match the oracle;
    # the token rows end at many places inside full (256-row) and half (128-row) tiles
    P.log(f"[parity] grouped calls with counts and NaN pad rows, split={split}")
    D, F, mt = 256, 384, 128
    counts = np.array([1, 31, 32, 33, 100, 127, 129, 200, 255, 256, 257, 383, 0, 64], np.int32)
    E = counts.size
    padded = -(-counts // mt) * mt
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    m_cap = int(offsets[-1])
    rng = np.random.default_rng(21)
    x = W.f32_to_bf16_bits(rng.standard_normal((m_cap, D)).astype(np.float32))
    w1 = W.f32_to_bf16_bits((rng.standard_normal((E, F, D)) / 16).astype(np.float32))
    w3 = W.f32_to_bf16_bits((rng.standard_normal((E, F, D)) / 16).astype(np.float32))
    w2 = W.f32_to_bf16_bits((rng.standard_normal((E, D, F)) / 20).astype(np.float32))
    pad = np.ones(m_cap, bool)
    for e in range(E):
        pad[offsets[e]:offsets[e] + counts[e]] = False
    x_zero = x.copy()
    x_zero[pad] = 0
    x_nan = x.copy()
    x_nan[pad] = 0x7FC0                                     # bf16 quiet NaN
    h_ref, y_ref = orc.grouped_swiglu(x_zero, offsets, w1, w3, w2, "bf16")
    te = np.repeat(np.arange(E, dtype=np.int32), padded // mt)
    ws = rpg.grouped_workspace("cuda") if split else None
    h = P.poison(torch.empty((m_cap, F), dtype=torch.bfloat16, device="cuda"))
    y = P.poison(torch.empty((m_cap, D), dtype=torch.bfloat16, device="cuda"))
    dc = P.to_dev(counts)
    rpg.moe_grouped_swiglu(P.to_dev(x_nan), P.to_dev(offsets), P.to_dev(te), P.to_dev(w1),
                           P.to_dev(w3), P.to_dev(w2), mt, m_cap=m_cap, h=h, y_perm=y,
                           workspace=ws, counts=dc)
    torch.cuda.synchronize()
    for name, got, ref in (("h", h, h_ref), ("y", y, y_ref)):
        v = orc.values64(P.to_host(got))
        assert np.all(v[pad] == 0), f"{name}: pad rows not exactly zero"
        assert np.all(np.isfinite(v)), f"{name}: unwritten or NaN rows"
        e = P.rel_err(P.to_host(got)[~pad], ref[~pad])
        assert e <= P.TOL["bf16"], (name, e)
    # backward: NaN pad rows in dy and in the saved [a | b] must not reach dab, dX or the
    # weight gradients
    ab_ref = orc.preactivations(x_zero, offsets, w1, w3, "bf16")
    dy = W.f32_to_bf16_bits(rng.standard_normal((m_cap, D)).astype(np.float32))
    dy_zero = dy.copy()
    dy_zero[pad] = 0
    dy_nan = dy.copy()
    dy_nan[pad] = 0x7FC0
    ab_st = W.f32_to_bf16_bits(ab_ref.astype(np.float32))
    ab_nan = ab_st.copy()
    ab_nan[pad] = 0x7FC0
    bw = orc.grouped_backward(x_zero, ab_st, h_ref, dy_zero, offsets, w1, w3, w2, "bf16")
    dab = P.poison(torch.empty((m_cap, 2 * F), dtype=torch.bfloat16, device="cuda"))
    rpg.moe_grouped_dgrad_swiglu(P.to_dev(dy_nan), P.to_dev(offsets), P.to_dev(te), P.to_dev(w2),
                                 P.to_dev(ab_nan), mt, m_cap, dab=dab, workspace=ws, counts=dc)
    dab_st = W.f32_to_bf16_bits(bw[1].astype(np.float32))
    dab_nan = dab_st.copy()
    dab_nan[pad] = 0x7FC0
    dx = P.poison(torch.empty((m_cap, D), dtype=torch.bfloat16, device="cuda"))
    rpg.moe_grouped_dgrad_fc1(P.to_dev(dab_nan), P.to_dev(offsets), P.to_dev(te), P.to_dev(w1),
                              P.to_dev(w3), mt, m_cap, dx_perm=dx, workspace=ws, counts=dc)
    x_nan_dev = P.to_dev(x_nan)
    dw1, dw3 = rpg.moe_grouped_wgrad(P.to_dev(dab_nan), x_nan_dev, P.to_dev(offsets), mt, m_cap,
                                     NS=F, counts=dc)
    torch.cuda.synchronize()
    for name, got, ref in (("dab", P.to_host(dab), bw[1]), ("dX", P.to_host(dx), bw[2])):
        v = orc.values64(got)
        assert np.all(v[pad] == 0) and np.all(np.isfinite(v)), name
        e = P.rel_err(got[~pad], ref[~pad])
        assert e <= P.TOL["bf16"], (name, e)
    for name, got, ref in (("dW1", dw1, bw[3]), ("dW3", dw3, bw[4])):
        g = P.to_host(got).astype(np.float64)
        assert np.all(np.isfinite(g)), name
        assert np.all(g[counts == 0] == 0), name
        e = np.abs(g - ref).max() / np.abs(ref).max()
        assert e <= P.TOL["bf16"], (name, e)


@pytest.mark.parametrize("T,E,k,mt", [(700, 64, 32, 128), (1537, 1024, 8, 64), (4097, 3, 2, 256),
                                      (300, 7, 7, 128), (8192, 8, 4, 128), (16384, 1024, 2, 64),
                                      (256, 1024, 32, 64), (97, 5, 3, 16), (16384, 256, 2, 128),
                                      (40000, 200, 3, 32), (65536, 8, 2, 128)])
def test_permute_layout_extremes(T, E, k, mt):
    # the permute alone against the oracle's layout: top-32 routing (the largest k), the
    # largest expert count, several 256-token histogram blocks with a ragged last one,
    # and -1 slots; every map bit-exact, x_perm exact on token rows and zero on pad rows
    # (rows past offsets[E] are not the permute's to write). At most 256 tokens (the last
    # two cases: the most slots one masked launch ranks, and a handful) the masked
    # permute is one launch that ranks every slot in each workgroup. A small histogram table
    # takes the histogram then the rank-and-copy kernel (8192 tokens x top-4 here, like
    # every benchmark workload). Above 2048 table entries the table is first
    # prefix-summed over its histogram blocks and each rank-and-copy workgroup reads two
    # rows of it (16384 tokens over 1024 and 256 experts, 40000 tokens over 200 experts:
    # 157 blocks, a ragged split over the scan's waves); a table of at most 2048 entries
    # too large for every workgroup to read whole (65536 tokens over 8 experts) takes
    # the histogram, rank and copy kernels. The masked layouts above 256 tokens take the
    # rank kernel, with the scan from 1537 tokens over 1024 experts up.
    P.log(f"[parity] permute layout T={T} E={E} k={k} m_tile={mt}")
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, k)) < 0.05] = -1
    x = W.f32_to_bf16_bits(rng.standard_normal((T, 64)).astype(np.float32))
    lay = orc.dispatch_layout(idx, E, mt)
    g = rpg.moe_permute(P.to_dev(x), P.to_dev(idx), E, mt)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "dst_row", "src_row", "tile_expert"):
        np.testing.assert_array_equal(P.to_host(g[key]), lay[key], err_msg=key)
    assert int(P.to_host(g["dev_err"])[0]) == 0
    used = int(lay["offsets"][-1])
    np.testing.assert_array_equal(P.to_host(g["x_perm"])[:used], orc.permute(x, lay)[:used])
    # the masked layout on the same routing, with slabs small enough to drop slots
    cap = max(16, int(np.bincount(idx[idx >= 0], minlength=E).mean() * 0.8) // 16 * 16)
    ml = orc.masked_layout(idx, E, cap)
    gm = rpg.moe_permute_masked(P.to_dev(x), P.to_dev(idx), E, cap)
    torch.cuda.synchronize()
    for key in ("counts", "dst_row", "src_row"):
        np.testing.assert_array_equal(P.to_host(gm[key]), ml[key], err_msg="masked " + key)
    assert int(P.to_host(gm["dev_err"])[0]) == (2 if ml["dropped"] else 0)
