"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutation is applied with monkeypatch to the oracle module only; the pins are the
checks in test_oracle_pins.py.
"""
import numpy as np
import pytest

from oracle import moe_oracle as orc
from tests import test_oracle_backward_pins as bpins
from tests import test_oracle_pins as pins


def _swapped_gate_up(A, w1e, w3e, w2e, dtype):
    A64 = orc.values64(A)
    a = A64 @ orc.values64(w1e).T
    b = A64 @ orc.values64(w3e).T
    h = orc.round_storage(orc.silu(b) * a, dtype)             # w1 and w3 roles swapped
    return h, orc.round_storage(h @ orc.values64(w2e).T, dtype)


def _no_silu(A, w1e, w3e, w2e, dtype):
    A64 = orc.values64(A)
    h = (A64 @ orc.values64(w1e).T) * (A64 @ orc.values64(w3e).T)   # activation dropped
    return h, h @ orc.values64(w2e).T


def _ties_high(logits, k):
    l = np.asarray(logits)
    order = np.argsort(-l[:, ::-1], axis=1, kind="stable")
    return (l.shape[1] - 1 - order[:, :k]).astype(np.int32)    # ties to the higher index


def _ascending(logits, k):
    return np.argsort(logits, axis=1, kind="stable")[:, :k].astype(np.int32)  # sign flipped


def _unweighted_combine(y_perm, dst_row, topk_w, dtype, shared=None):
    return orc.__dict__["_orig_combine"](y_perm, dst_row, np.ones_like(topk_w), dtype, shared)


def _softmax_over_selected_only(x, wg, k, dtype, bias=None, renorm=False):
    idx, _, logits = orc.__dict__["_orig_route"](x, wg, k, dtype, bias, renorm)
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(1, keepdims=True))
    return idx, z / z.sum(1, keepdims=True), logits


def _bias_dropped(x, wg, dtype, bias=None):
    return orc.__dict__["_orig_router_logits"](x, wg, dtype, None)


def _unstable_layout(topk_idx, E, m_tile, m_cap=None):
    lay = orc.__dict__["_orig_dispatch_layout"](topk_idx, E, m_tile, m_cap)
    # reverse the order of slots inside every segment (an unstable sort)
    src, dst = lay["src_row"].copy(), lay["dst_row"].copy()
    off, c = lay["offsets"], lay["counts"]
    k = dst.shape[1]
    for e in range(E):
        seg = src[off[e]:off[e] + c[e]][::-1].copy()
        src[off[e]:off[e] + c[e]] = seg
        for r, f in enumerate(seg):
            dst[f // k, f % k] = off[e] + r
    lay["src_row"], lay["dst_row"] = src, dst
    return lay


def _first_expert_only_counts(topk_idx, E, m_tile, m_cap=None):
    return orc.__dict__["_orig_dispatch_layout"](np.asarray(topk_idx)[:, :1], E, m_tile, m_cap)


def _silu_grad_dropped_term(a):
    s = 1.0 / (1.0 + np.exp(-np.asarray(a, dtype=np.float64)))
    return s                                                      # the a*s*(1-s) term dropped


def _swiglu_grads_swapped(dh, a, b, dtype):
    da, db = orc.__dict__["_orig_swiglu_backward"](dh, a, b, dtype)
    return db, da                                                 # gate and up gradients swapped


def _dgrad_without_up(A, a, b, h, dY, w1e, w3e, w2e, dtype):
    out = list(orc.__dict__["_orig_expert_backward"](A, a, b, h, dY, w1e, w3e, w2e, dtype))
    out[3] = orc.round_storage(out[1] @ orc.values64(w1e), dtype)  # db w3 term dropped
    return tuple(out)


def _dispatch_unweighted(dout, y_perm, dst_row, topk_w, rows_used, dtype):
    return orc.__dict__["_orig_combine_backward"](dout, y_perm, dst_row, np.ones_like(topk_w),
                                                  rows_used, dtype)


def _unpermute_without_shared(dX, dst_row, dtype, shared=None):
    return orc.__dict__["_orig_permute_backward"](dX, dst_row, dtype, None)


def _wgrad_up_from_gate(A, a, b, h, dY, w1e, w3e, w2e, dtype):
    out = list(orc.__dict__["_orig_expert_backward"](A, a, b, h, dY, w1e, w3e, w2e, dtype))
    out[5] = out[4]                                               # dW3 taken from da
    return tuple(out)


def _masked_keeps_the_last(topk_idx, E, cap):
    # keeps each expert's last cap slots instead of its first
    idx = np.asarray(topk_idx)
    rev = orc.__dict__["_orig_masked_layout"](idx[::-1, ::-1].copy(), E, cap)
    T, k = idx.shape
    dst = rev["dst_row"][::-1, ::-1].copy()
    src = np.where(rev["src_row"] >= 0, T * k - 1 - rev["src_row"], -1).astype(np.int32)
    rev["dst_row"], rev["src_row"] = dst, src
    return rev


def _masked_offsets_by_count(topk_idx, E, cap):
    # packs the slabs back to back (a contiguous layout) instead of at e*cap
    lay = orc.__dict__["_orig_masked_layout"](topk_idx, E, cap)
    start = np.concatenate([[0], np.cumsum(lay["counts"])[:-1]])
    dst = lay["dst_row"].copy()
    ok = dst >= 0
    e = dst[ok] // cap
    dst[ok] = start[e] + dst[ok] % cap
    lay["dst_row"] = dst
    return lay


def _e4m3_truncating(v):
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.clip(e, -6, 8) - 3))
    return np.copysign(np.minimum(np.floor(a / step) * step, 448.0), v)   # rounds toward zero


def _mx_floor_scale(x, block=32):
    # the scale 2^(floor(log2 amax) - 8): the largest values of a block saturate
    v = orc.values64(x)
    R, C = v.shape
    b = v.reshape(R, C // block, block)
    amax = np.abs(b).max(axis=2)
    X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    q = orc.e4m3_round(np.clip(b / 2.0 ** X[:, :, None], -448, 448))
    return orc.e4m3_encode(q).reshape(R, C), (X + 127).astype(np.uint8)


def _combine_rounds_each_slot(y_perm, dst_row, topk_w, dtype, shared=None):
    # every slot's weighted row rounded to storage before the sum (one rounding per slot
    # instead of one for the whole sum)
    Y = orc.values64(y_perm)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    out = np.zeros((dst.shape[0], Y.shape[1]))
    for j in range(dst.shape[1]):
        ok = dst[:, j] >= 0
        out[ok] += orc.round_storage(w[ok, j:j + 1] * Y[dst[ok, j]], dtype)
    if shared is not None:
        out += orc.values64(shared)
    return orc.round_storage(out, dtype)


def _y_from_unrounded_h(A, w1e, w3e, w2e, dtype):
    A64 = orc.values64(A)
    hu = orc.silu(A64 @ orc.values64(w1e).T) * (A64 @ orc.values64(w3e).T)
    # h is stored rounded, but fc2 reads the unrounded values
    return orc.round_storage(hu, dtype), orc.round_storage(hu @ orc.values64(w2e).T, dtype)


def _h_from_rounded_preactivations(A, w1e, w3e, w2e, dtype):
    A64 = orc.values64(A)
    a = orc.round_storage(A64 @ orc.values64(w1e).T, dtype)
    b = orc.round_storage(A64 @ orc.values64(w3e).T, dtype)
    h = orc.round_storage(orc.silu(a) * b, dtype)
    return h, orc.round_storage(h @ orc.values64(w2e).T, dtype)


def _shared_rounded_per_expert(x, ws1, ws3, ws2, dtype):
    total = 0.0
    for s_ in range(ws1.shape[0]):
        total = total + orc.__dict__["_orig_shared_experts"](x, ws1[s_:s_ + 1], ws3[s_:s_ + 1],
                                                              ws2[s_:s_ + 1], dtype)
    return orc.round_storage(total, dtype)


MUTATIONS = {
    "combine_rounds_each_slot": ("combine", _combine_rounds_each_slot, "brute_bf16"),
    "y_from_unrounded_h": ("expert_swiglu", _y_from_unrounded_h, "brute_bf16"),
    "h_from_rounded_ab": ("expert_swiglu", _h_from_rounded_preactivations, "brute_bf16"),
    "shared_rounded_per_expert": ("shared_experts", _shared_rounded_per_expert, "brute_bf16"),
    "e4m3_truncating": ("e4m3_round", _e4m3_truncating, "fp8"),
    "mx_floor_scale": ("mx_quantize", _mx_floor_scale, "fp8"),
    "masked_keeps_last": ("masked_layout", _masked_keeps_the_last, "masked"),
    "masked_packed": ("masked_layout", _masked_offsets_by_count, "masked"),
    "bwd_silu_grad_term": ("silu_grad", _silu_grad_dropped_term, "autograd"),
    "bwd_swiglu_swapped": ("swiglu_backward", _swiglu_grads_swapped, "autograd"),
    "bwd_dgrad_no_up": ("expert_backward", _dgrad_without_up, "autograd"),
    "bwd_dispatch_unweighted": ("combine_backward", _dispatch_unweighted, "autograd"),
    "bwd_unpermute_no_shared": ("permute_backward", _unpermute_without_shared, "autograd"),
    "bwd_wgrad_up_from_gate": ("expert_backward", _wgrad_up_from_gate, "autograd"),
    "swapped_gate_up": ("expert_swiglu", _swapped_gate_up, "brute"),
    "no_silu": ("expert_swiglu", _no_silu, "brute"),
    "ties_high": ("select_topk", _ties_high, "ties"),
    "ascending": ("select_topk", _ascending, "brute"),
    "unweighted_combine": ("combine", _unweighted_combine, "brute"),
    "softmax_over_selected": ("route", _softmax_over_selected_only, "brute"),
    "bias_dropped": ("router_logits", _bias_dropped, "brute_bias"),
    "unstable_layout": ("dispatch_layout", _unstable_layout, "layout"),
    "first_slot_only": ("dispatch_layout", _first_expert_only_counts, "layout"),
}


def _run_pin(kind):
    if kind == "brute":
        pins._check_layer_against_brute(orc, 0, k=2)
    elif kind == "brute_bias":
        pins._check_layer_against_brute(orc, 5, k=3, bias=True, shared=True)
    elif kind == "ties":
        pins.test_topk_matches_python_sorted_with_ties()
    elif kind == "layout":
        pins.test_layout_matches_loop_counting_sort(50, 3, 7, 4, False)
    elif kind == "fp8":
        pins.test_e4m3_round_matches_torch_float8_rounding()
        pins.test_mx_scale_is_the_smallest_power_that_avoids_saturation()
    elif kind == "masked":   # one case with full slabs and drops, one with partly filled slabs
        pins.test_masked_layout_matches_loop_and_contiguous_ranks(33, 3, 4, 8)
        pins.test_masked_layout_matches_loop_and_contiguous_ranks(20, 2, 5, 16)
    elif kind == "brute_bf16":
        for seed in (0, 1, 2):
            pins._check_bf16_storage_points(orc, seed)
    elif kind == "autograd":
        bpins._check_backward_against_autograd(orc, 0)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn, kind = MUTATIONS[name]
    monkeypatch.setitem(orc.__dict__, "_orig_" + attr, getattr(orc, attr))
    monkeypatch.setattr(orc, attr, fn)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _run_pin(kind)


def test_unmutated_pins_pass():
    for kind in ("brute", "brute_bias", "brute_bf16", "ties", "layout", "autograd", "masked",
                 "fp8"):
        _run_pin(kind)
