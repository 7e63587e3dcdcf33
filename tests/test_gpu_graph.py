"""The layer's forward step (route, permute, fc1 + SwiGLU, fc2, combine on preallocated
buffers, split-K tail included) captured once in a HIP graph and replayed: every replay
must reproduce the eager step's output bit for bit, with eager steps on other inputs and
host synchronisations between the replays. The step holds kernel launches only (no
memset nodes, no allocation, no host sync), which is what makes it capturable."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_amd as rpg
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _buffers(T, D, F, E, k, mt, dev):
    m_cap = rpg.moe_capacity(T, k, E, mt)
    i32 = dict(dtype=torch.int32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    return m_cap, {
        "idx": torch.empty((T, k), **i32), "w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "x_perm": torch.empty((m_cap, D), **bf), "counts": torch.empty(E, **i32),
        "offsets": torch.empty(E + 1, **i32), "dst_row": torch.empty((T, k), **i32),
        "src_row": torch.empty(m_cap, **i32), "tile_expert": torch.empty(m_cap // mt, **i32),
        "dev_err": torch.empty(1, **i32),
        "workspace": torch.empty(max(4, rpg.moe_permute_workspace_bytes(T, k, E)),
                                 dtype=torch.uint8, device=dev),
        "h": torch.empty((m_cap, F), **bf), "y": torch.empty((m_cap, D), **bf),
        "out": torch.empty((T, D), **bf),
    }


@pytest.mark.parametrize("name,shrink", [
    ("dense8_bf16", dict(T=1000, D=512, F=1024)),          # fc1 on the LDS ring, split-K tail
    ("skew32_zipf_bf16", dict(T=1500, D=512, F=768)),     # two-stage kernel (hot expert)
])
def test_graph_replays_equal_the_eager_step(name, shrink):
    cfg = W.shrink(W.preset(name), **shrink)
    print(f"[graph] {name} {shrink}", flush=True)
    dev = torch.device("cuda", 0)
    inp = [W.generate(cfg, seed=s) for s in (0, 1)]
    d = [{key: P.to_dev(v) for key, v in i.items() if key != "cfg"} for i in inp]
    T, D, F, E, k, mt = cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, cfg.m_tile
    m_cap, buf = _buffers(T, D, F, E, k, mt, dev)
    gws = rpg.grouped_workspace(dev)
    main = torch.cuda.current_stream()
    cap = torch.cuda.Stream()              # capture needs a stream other than the default
    x = torch.empty_like(d[0]["x"])

    def step(stream):
        rpg.moe_route(x, d[0]["wg"], k, bias=d[0].get("bias"), topk_idx=buf["idx"],
                      topk_w=buf["w"], stream=stream)
        rpg.moe_permute(x, buf["idx"], E, mt, m_cap=m_cap, out=buf, stream=stream)
        rpg.moe_grouped_fc1_swiglu(buf["x_perm"], buf["offsets"], buf["tile_expert"], d[0]["w1"],
                                   d[0]["w3"], mt, m_cap, buf["h"], workspace=gws, stream=stream,
                                   counts=buf["counts"])
        rpg.moe_grouped_fc2(buf["h"], buf["offsets"], buf["tile_expert"], d[0]["w2"], mt, m_cap,
                            buf["y"], workspace=gws, stream=stream, counts=buf["counts"])
        rpg.moe_combine(buf["y"], buf["dst_row"], buf["w"], out=buf["out"], m_cap=m_cap,
                        stream=stream)

    eager = []
    for j in (0, 1):                       # eager results for both token batches
        x.copy_(d[j]["x"])
        step(main)
        torch.cuda.synchronize()
        eager.append(buf["out"].clone())
    assert not torch.equal(eager[0], eager[1])

    g = torch.cuda.CUDAGraph()
    x.copy_(d[0]["x"])
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        step(cap)
    for rep in range(4):
        j = rep % 2
        x.copy_(d[j]["x"])
        buf["out"].fill_(float("nan"))
        g.replay()                         # on the default stream
        torch.cuda.synchronize()
        assert torch.equal(buf["out"], eager[j]), f"replay {rep} (batch {j}) differs"
        x.copy_(d[1 - j]["x"])
        step(main)                         # an eager step on the other batch in between
        torch.cuda.synchronize()
    del g
