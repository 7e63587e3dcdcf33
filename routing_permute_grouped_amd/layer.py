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
        self.T = T
        self.m_cap = -(-T // m_tile) * m_tile
        self.offsets = torch.tensor([0, T], dtype=torch.int32, device=device)
        self.tile_expert = torch.zeros(self.m_cap // m_tile, dtype=torch.int32, device=device)


def moe_layer(x: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor, k: int,
              m_tile: int, wg: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
              topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
              shared: Optional[SharedExperts] = None, renorm: bool = False,
              check: bool = False, split_k: bool = True, save_for_backward: bool = False) -> dict:
    """Run the layer; returns every intermediate (dict). With routing given
    (``topk_idx``/``topk_w``) the route step is skipped. ``check`` synchronises and
    raises if the permute saw an expert index outside [-1, E). ``split_k`` gives the
    grouped GEMMs a workspace so they can split a partly filled last round of tiles.
    ``save_for_backward`` also keeps fc1's pre-activations (``ab``, and ``shared_ab`` /
    ``shared_h`` for the shared experts), which ``moe_layer_backward`` reads."""
    E, F, D = w1.shape
    res = {}
    if topk_idx is None:
        topk_idx, topk_w, _ = B.moe_route(x, wg, k, bias=bias, renorm=renorm)
    res["topk_idx"], res["topk_w"] = topk_idx, topk_w
    p = B.moe_permute(x, topk_idx, E, m_tile)
    res.update(p)
    m_cap = p["m_cap"]
    ws = B.grouped_workspace(x.device) if split_k else None
    if save_for_backward:
        h = torch.empty((m_cap, F), dtype=x.dtype, device=x.device)
        ab = torch.empty((m_cap, 2 * F), dtype=x.dtype, device=x.device)
        y = torch.empty((m_cap, D), dtype=x.dtype, device=x.device)
        B.moe_grouped_fc1_swiglu(p["x_perm"], p["offsets"], p["tile_expert"], w1, w3, m_tile,
                                 m_cap, h, ab=ab, workspace=ws, counts=p["counts"])
        B.moe_grouped_fc2(h, p["offsets"], p["tile_expert"], w2, m_tile, m_cap, y, workspace=ws,
                          counts=p["counts"])
        res["ab"] = ab
    else:
        h, y = B.moe_grouped_swiglu(p["x_perm"], p["offsets"], p["tile_expert"], w1, w3, w2,
                                    m_tile, m_cap=m_cap, workspace=ws, counts=p["counts"])
    res["h"], res["y_perm"] = h, y
    sh = None
    if shared is not None:
        rows = DenseRows(x.shape[0], m_tile, x.device)
        if save_for_backward:
            SF = shared.w1.shape[1]
            hs = torch.empty((rows.m_cap, SF), dtype=x.dtype, device=x.device)
            abs_ = torch.empty((rows.m_cap, 2 * SF), dtype=x.dtype, device=x.device)
            ys = torch.empty((rows.m_cap, D), dtype=x.dtype, device=x.device)
            B.moe_grouped_fc1_swiglu(x, rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                                     m_tile, rows.m_cap, hs, ab=abs_, workspace=ws,
                                     rows_used=rows.T)
            B.moe_grouped_fc2(hs, rows.offsets, rows.tile_expert, shared.w2, m_tile, rows.m_cap,
                              ys, workspace=ws)
            res["shared_h"], res["shared_ab"] = hs, abs_
        else:
            _, ys = B.moe_grouped_swiglu(x, rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                                         shared.w2, m_tile, m_cap=rows.m_cap, workspace=ws,
                                         rows_used=rows.T)
        sh = ys[: x.shape[0]]
        res["shared"] = sh
    res["out"] = B.moe_combine(y, p["dst_row"], topk_w, shared=sh, m_cap=m_cap)
    if check:
        torch.cuda.current_stream().synchronize()
        if int(p["dev_err"].item()) != 0:
            raise ValueError("topk_idx holds expert indices outside [-1, E)")
    return res


def moe_layer_masked(x: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor,
                     k: int, cap: int, wg: Optional[torch.Tensor] = None,
                     bias: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                     topk_w: Optional[torch.Tensor] = None,
                     shared: Optional[SharedExperts] = None, renorm: bool = False,
                     split_k: bool = True, shared_m_tile: int = 128) -> dict:
    """The layer on the masked (fixed-capacity) layout for decode: route -> masked
    permute (slabs of ``cap`` rows per expert) -> masked grouped SwiGLU [-> shared
    experts] -> combine. Slots past an expert's cap are dropped (bit 1 of dev_err)."""
    E = w1.shape[0]
    res = {}
    if topk_idx is None:
        topk_idx, topk_w, _ = B.moe_route(x, wg, k, bias=bias, renorm=renorm)
    res["topk_idx"], res["topk_w"] = topk_idx, topk_w
    p = B.moe_permute_masked(x, topk_idx, E, cap)
    res.update(p)
    ws = B.grouped_workspace(x.device) if split_k else None
    h, y = B.moe_grouped_swiglu_masked(p["x_masked"], p["counts"], w1, w3, w2, cap, workspace=ws)
    res["h"], res["y_perm"] = h, y
    sh = None
    if shared is not None:
        rows = DenseRows(x.shape[0], shared_m_tile, x.device)
        _, ys = B.moe_grouped_swiglu(x, rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                                     shared.w2, shared_m_tile, m_cap=rows.m_cap, workspace=ws,
                                     rows_used=rows.T)
        sh = ys[: x.shape[0]]
        res["shared"] = sh
    res["out"] = B.moe_combine(y, p["dst_row"], topk_w, shared=sh, m_cap=p["m_cap"])
    return res


@dataclass
class MxWeights:
    """fc1's weights quantized once for the FP8 payload: e4m3 codes [E,F,D] of w1 and w3,
    and their E8M0 scales in the GEMM's k-step words (uint8 [D/128, E*F, 4]: word (s, r)
    holds row r's scales of values 128*s .. 128*s + 127)."""
    w1q: torch.Tensor
    w1s: torch.Tensor
    w3q: torch.Tensor
    w3s: torch.Tensor

    @staticmethod
    def quantize(w1: torch.Tensor, w3: torch.Tensor) -> "MxWeights":
        w1q, w1s = B.moe_quantize_mxfp8(w1, layout=B.MOE_MX_KSTEPS)
        w3q, w3s = B.moe_quantize_mxfp8(w3, layout=B.MOE_MX_KSTEPS)
        return MxWeights(w1q, w1s, w3q, w3s)


def moe_layer_mxfp8(x: torch.Tensor, mw: MxWeights, w2: torch.Tensor, k: int, m_tile: int,
                    wg: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                    topk_idx: Optional[torch.Tensor] = None,
                    topk_w: Optional[torch.Tensor] = None,
                    shared: Optional[SharedExperts] = None, renorm: bool = False,
                    split_k: bool = True) -> dict:
    """The layer with an FP8 payload (EP page, section 6 "DeepSeek-V3 量级的示例数字": the
    dispatch payload is FP8 e4m3 with scales, the combine stays bf16): route on the bf16 x -> MX-quantize x -> permute codes and scales ->
    fc1 on the scaled-FP8 MFMA -> fc2 (bf16) [-> shared experts, bf16] -> combine."""
    E = mw.w1q.shape[0]
    res = {}
    if topk_idx is None:
        topk_idx, topk_w, _ = B.moe_route(x, wg, k, bias=bias, renorm=renorm)
    res["topk_idx"], res["topk_w"] = topk_idx, topk_w
    xq, xs = B.moe_quantize_mxfp8(x)
    res["xq"], res["xs"] = xq, xs
    p = B.moe_permute_mxfp8(xq, xs, topk_idx, E, m_tile)
    res.update(p)
    m_cap = p["m_cap"]
    ws = B.grouped_workspace(x.device) if split_k else None
    h = B.moe_grouped_fc1_swiglu_mxfp8(p["xq_perm"], p["xs_perm"], p["offsets"], p["tile_expert"],
                                       mw.w1q, mw.w1s, mw.w3q, mw.w3s, m_tile, m_cap,
                                       workspace=ws, counts=p["counts"])
    y = torch.empty((m_cap, x.shape[1]), dtype=x.dtype, device=x.device)
    B.moe_grouped_fc2(h, p["offsets"], p["tile_expert"], w2, m_tile, m_cap, y, workspace=ws,
                      counts=p["counts"])
    res["h"], res["y_perm"] = h, y
    sh = None
    if shared is not None:
        rows = DenseRows(x.shape[0], m_tile, x.device)
        _, ys = B.moe_grouped_swiglu(x, rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                                     shared.w2, m_tile, m_cap=rows.m_cap, workspace=ws,
                                     rows_used=rows.T)
        sh = ys[: x.shape[0]]
        res["shared"] = sh
    res["out"] = B.moe_combine(y, p["dst_row"], topk_w, shared=sh, m_cap=m_cap)
    return res


def _experts_backward(dy, x_rows, ab, h, offsets, tile_expert, w1, w3, w2, m_tile, m_cap, ws,
                      rows_used=None, counts=None):
    """dgrad and wgrad of one grouped SwiGLU FFN over rows [0, m_cap) (section 5 of
    "Expert Parallelism (EP)": the m-grouped fc mirrors into an m-grouped dgrad and a
    k-grouped wgrad). Returns (dab, dX, dw1, dw3, dw2)."""
    F, D = w1.shape[1], w1.shape[2]
    ru, c = rows_used, counts
    dab = B.moe_grouped_dgrad_swiglu(dy, offsets, tile_expert, w2, ab, m_tile, m_cap,
                                     workspace=ws, rows_used=ru, counts=c)
    dX = B.moe_grouped_dgrad_fc1(dab, offsets, tile_expert, w1, w3, m_tile, m_cap, workspace=ws,
                                 rows_used=ru, counts=c)
    dw1, dw3 = B.moe_grouped_wgrad(dab, x_rows, offsets, m_tile, m_cap, NS=F, rows_used=ru,
                                   counts=c)
    dw2, _ = B.moe_grouped_wgrad(dy, h, offsets, m_tile, m_cap, NS=D, rows_used=ru, counts=c)
    return dab, dX, dw1, dw3, dw2


def moe_layer_backward(fwd: dict, dout: torch.Tensor, x: torch.Tensor, w1: torch.Tensor,
                       w3: torch.Tensor, w2: torch.Tensor, m_tile: int,
                       shared: Optional[SharedExperts] = None, split_k: bool = True) -> dict:
    """Backward of ``moe_layer(..., save_for_backward=True)`` for the output gradient
    ``dout`` [T, D], as the mirror of each forward step ("Expert Parallelism (EP)",
    section 5): combine -> dispatch (moe_combine_backward), grouped SwiGLU -> dgrad +
    wgrad, permute -> unpermute (moe_combine without weights). Routing is taken as
    given; its weights get their gradient ``dtopk_w``. Weight gradients are float32
    (``dw1``, ``dw3`` [E,F,D], ``dw2`` [E,D,F]; for the shared experts ``dws1``, ``dws3``
    [1,S*Fs,D] and ``dws2`` [1,D,S*Fs], the concatenated layout of SharedExperts)."""
    m_cap = fwd["m_cap"]
    offs, te = fwd["offsets"], fwd["tile_expert"]
    ws = B.grouped_workspace(x.device) if split_k else None
    res = {}
    dy, dtw = B.moe_combine_backward(dout, fwd["y_perm"], fwd["src_row"], offs, fwd["dst_row"],
                                     fwd["topk_w"], m_cap=m_cap)
    res["dy_perm"], res["dtopk_w"] = dy, dtw
    dab, dX, dw1, dw3, dw2 = _experts_backward(dy, fwd["x_perm"], fwd["ab"], fwd["h"], offs, te,
                                               w1, w3, w2, m_tile, m_cap, ws,
                                               counts=fwd["counts"])
    res.update(dab=dab, dx_perm=dX, dw1=dw1, dw3=dw3, dw2=dw2)
    dxs = None
    if shared is not None:
        T = x.shape[0]
        rows = DenseRows(T, m_tile, x.device)
        _, dXs, dws1, dws3, dws2 = _experts_backward(
            dout, x, fwd["shared_ab"], fwd["shared_h"], rows.offsets, rows.tile_expert,
            shared.w1, shared.w3, shared.w2, m_tile, rows.m_cap, ws, rows_used=T)
        dxs = dXs[:T]
        res.update(dx_shared=dxs, dws1=dws1, dws3=dws3, dws2=dws2)
    res["dx"] = B.moe_combine(dX, fwd["dst_row"], None, shared=dxs, m_cap=m_cap)
    return res
