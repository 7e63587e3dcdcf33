"""The whole layer as one chain of the four library calls on the current stream.

route -> permute -> grouped SwiGLU (routed experts) [-> grouped SwiGLU (shared
experts as one expert over all tokens)] -> combine, following the layer order of
"Expert Parallelism (EP)" (llm-infra-atlas), section 1.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _binding as B


@dataclass
class SharedExperts:
    """Shared experts stored as one expert whose intermediate dimension is the
    concatenation of theirs: sum_s w2_s(silu(w1_s x) * w3_s x) equals the single
    expert with w1, w3 stacked along F and w2 concatenated along its F axis."""
    w1: torch.Tensor       # [1, S*Fs, D]
    w3: torch.Tensor       # [1, S*Fs, D]
    w2: torch.Tensor       # [1, D, S*Fs]

    @staticmethod
    def from_stacked(ws1: torch.Tensor, ws3: torch.Tensor, ws2: torch.Tensor) -> "SharedExperts":
        S, Fs, D = ws1.shape
        return SharedExperts(ws1.reshape(1, S * Fs, D).contiguous(),
                             ws3.reshape(1, S * Fs, D).contiguous(),
                             torch.cat(list(ws2), dim=1).reshape(1, D, S * Fs).contiguous())


class DenseRows:
    """offsets/tile_expert describing one expert over T rows (the shared-expert call)."""

    def __init__(self, T: int, m_tile: int, device):
        self.m_cap = -(-T // m_tile) * m_tile
        self.offsets = torch.tensor([0, T], dtype=torch.int32, device=device)
        self.tile_expert = torch.zeros(self.m_cap // m_tile, dtype=torch.int32, device=device)


def moe_layer(x: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor, k: int,
              m_tile: int, wg: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
              topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
              shared: Optional[SharedExperts] = None, renorm: bool = False,
              check: bool = False, split_k: bool = True) -> dict:
    """Run the layer; returns every intermediate (dict). With routing given
    (``topk_idx``/``topk_w``) the route step is skipped. ``check`` synchronises and
    raises if the permute saw an expert index outside [-1, E). ``split_k`` gives the
    grouped GEMMs a workspace so they can split a partly filled last round of tiles."""
    E = w1.shape[0]
    res = {}
    if topk_idx is None:
        topk_idx, topk_w, _ = B.moe_route(x, wg, k, bias=bias, renorm=renorm)
    res["topk_idx"], res["topk_w"] = topk_idx, topk_w
    p = B.moe_permute(x, topk_idx, E, m_tile)
    res.update(p)
    ws = B.grouped_workspace(x.device) if split_k else None
    h, y = B.moe_grouped_swiglu(p["x_perm"], p["offsets"], p["tile_expert"], w1, w3, w2, m_tile,
                                m_cap=p["m_cap"], workspace=ws)
    res["h"], res["y_perm"] = h, y
    sh = None
    if shared is not None:
        rows = DenseRows(x.shape[0], m_tile, x.device)
        _, ys = B.moe_grouped_swiglu(x, rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                                     shared.w2, m_tile, m_cap=rows.m_cap, workspace=ws)
        sh = ys[: x.shape[0]]
        res["shared"] = sh
    res["out"] = B.moe_combine(y, p["dst_row"], topk_w, shared=sh, m_cap=p["m_cap"])
    if check:
        torch.cuda.current_stream().synchronize()
        if int(p["dev_err"].item()) != 0:
            raise ValueError("topk_idx holds expert indices outside [-1, E)")
    return res
