"""Plain, slow CPU oracle of the single-GPU MoE expert-layer path.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module. The product path (the HIP library and its
Python binding) never imports, calls or links it, and this module imports
nothing from the product.

Sources (cited by page and section):

* "Expert Parallelism (EP)" (llm-infra-atlas), section 1 "MoE layer 的 forward
  通路": the layer is router gating (logits = x·Wg^T over [T,E]), routing
  (top-k plus a score function giving probs and a routing map), metadata
  (tokens per expert), a permute that makes each local expert's tokens
  contiguous, a grouped fc1 -> activation -> fc2, and an unpermute that reduces
  back to token order weighted by the top-k weights, plus shared experts.
* same page, section 2 "三层抽象与三个代码库的分工": the dispatch output must be
  expert-contiguous with every segment aligned to the GEMM M tile (the layout
  contract the grouped GEMM consumes).
* same page, section 5 "forward / backward 的对称性": permute is an index_select
  and unpermute a scatter_add; combine is the transpose of dispatch.
* "Expert Tensor Parallel" design note (HyperParallel issue 104), section 4.3:
  expert weights w1, w3 of shape [E, H, D] and w2 of shape [E, D, H], SwiGLU
  with w1/w3 on the input side and w2 on the output side (H there is this
  module's F).

Readings taken where the pages are silent:

1. Score function: softmax over all E logits; the top-k weights are those
   probabilities at the selected experts, not renormalised (``renorm`` is an
   option, off by default).
2. Selection compares the float32 logits with key (-logit, expert index): the
   lower index wins a tie, results come out best first. -0 and +0 tie.
3. The float32 logits follow one fixed operation order (``router_logits``),
   because the top-k decision must be taken identically on both sides.
4. A router bias is added to the logits, so it moves both the choice and the
   weights.
5. Activation: h = silu(x·w1^T) * (x·w3^T), silu(a) = a / (1 + exp(-a)).
6. Pad rows of every segment are zero, so their h and Y rows are exactly zero.
   Segments of experts with no token are empty (no rows, no tiles).
7. Inside a segment rows follow the flattened (token, slot) order t*k + j.
8. Slots holding -1 (a share that lives on another rank) are skipped by the
   counts, the permute and the combine.
9. Storage points: x, weights, h, Y, the shared-expert output and the layer
   output are stored in the layer dtype (float32 or bf16, round to nearest
   even); all other arithmetic here is float64.

Backward (same page, section 5: every forward operator has a mirror; permute's is an
unpermute (scatter_add), combine's is a dispatch, an m-grouped fc's is an m-grouped
dgrad plus a k-grouped wgrad). Readings:

10. The forward stores the fc1 pre-activations a = X w1^T and b = X w3^T in the
    layer dtype; the backward uses those stored values.
11. Given dout [T, D] (stored), combine's mirror sends w[t,j] * dout[t] to row
    dst[t,j] (stored; pad rows zero) and gives dw[t,j] = <dout[t], Y[dst[t,j]]>.
12. dh = dY w2[e], da = dh * b * silu'(a), db = dh * silu(a), dX = da w1[e] + db w3[e]
    (each stored once); dW2[e] = dY^T h, dW1[e] = da^T X, dW3[e] = db^T X over the
    expert's rows (weight gradients kept in float32 on the device, float64 here).
13. dx[t] = sum_j dX[dst[t,j]] (slots in order j, skipping -1) plus the shared
    experts' input gradient, stored once: permute's mirror is combine with unit
    weights. The shared experts' output gradient is dout itself.
14. The router's own backward (through softmax and top-k) is not part of this path.

Masked layout for decode (same page: decode uses the masked grouped GEMM because each
local expert's row count is known only at run time). Readings:

15. Every expert owns a fixed slab of ``cap`` rows; slot (t, j) of expert e goes to row
    e*cap + rank, rank being its stable rank among e's slots (the contiguous layout's
    rank). A slot whose rank is cap or more is dropped (no row; combine skips it) and
    flagged. counts[e] = min(#slots of e, cap) rows are valid; the rest of a slab is
    neither computed nor read.

FP8 payload (section 6 "DeepSeek-V3 量级的示例数字" of the same page: the dispatch payload
is FP8 e4m3 with scales, the combine stays BF16). Readings:

16. The scales are MX block scales: one power-of-two scale 2^X per 32 consecutive values
    along D (E8M0, stored as X + 127). X is the smallest integer with max|v| <= 448 * 2^X
    (448 is e4m3's largest value), so no value of the block saturates; X = -127 for an
    all-zero block. Each value is v / 2^X rounded to the nearest e4m3 value (OCP E4M3:
    bias 7, no infinities, max 448), ties to even.
17. x is quantized once per token before the permute (the permute copies its rows); the
    fc1 weights w1, w3 are quantized the same way along D; fc1 contracts the dequantized
    values (float64 here, float32 accumulation on the device); h and everything after it
    stay bf16 (fc2 and the combine are the bf16 path).

Float arrays may be passed as float32/float64 values or, for bf16, as uint16
bit patterns; this module widens them itself.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "capacity", "values64", "values32", "round_storage", "round_bf16",
    "router_logits", "softmax", "select_topk", "route",
    "dispatch_layout", "permute", "silu", "expert_swiglu", "grouped_swiglu",
    "shared_experts", "combine", "forward", "token_outputs",
    "silu_grad", "preactivations", "combine_backward", "swiglu_backward",
    "expert_backward", "grouped_backward", "permute_backward", "shared_backward",
    "backward", "token_backward", "expert_weight_grad_slices",
    "masked_layout", "masked_swiglu", "forward_masked",
    "e4m3_decode", "e4m3_round", "e4m3_encode", "mx_quantize", "mx_dequantize",
    "expert_fc1_mx", "grouped_fc1_mx", "forward_mxfp8", "token_outputs_mx",
]

_LANES = 64  # width of one reduction group in the fixed logit order


# ----------------------------------------------------------------------------
# storage types
# ----------------------------------------------------------------------------

def values64(a: np.ndarray) -> np.ndarray:
    """Values of a stored array as float64. uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def values32(a: np.ndarray) -> np.ndarray:
    """Values of a float32 or bf16 (uint16 bits) array as float32 (exact)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if a.dtype != np.float32:
        raise TypeError("router inputs must be float32 values or bf16 bit patterns")
    return a


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits and float32's exponent range; below the
    smallest normal (2^-126) the spacing stays 2^-133. Inputs are finite."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                       # |a| in [2^(e-1), 2^e)
    e = np.maximum(e, -125)
    quantum = np.ldexp(1.0, e - 8)
    return np.rint(a / quantum) * quantum    # np.rint rounds half to even


def round_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Value after storing float64 ``a`` in the layer dtype, as float64. ``"f64"`` keeps
    the value (no rounding): the pins use it to compare derivatives exactly."""
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(a)
    raise ValueError(dtype)


def capacity(T: int, k: int, E: int, m_tile: int) -> int:
    """Rows the permuted buffer needs in the worst case.

    With N = T*k slots and c_e rows per expert, the padded total is
    sum_e ceil(c_e / Mt) * Mt <= N + min(E, N) * (Mt - 1), and it is a multiple of
    Mt, so the largest multiple of Mt not above that bound always suffices."""
    N = T * k
    return ((N + min(E, N) * (m_tile - 1)) // m_tile) * m_tile


# ----------------------------------------------------------------------------
# routing ("Expert Parallelism (EP)", section 1, forward-path figure: gate and top-k)
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, wg: np.ndarray, dtype: str,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, e] = sum_d x[t, d] * Wg[e, d] (+ bias[e]) in float32, fixed order.

    The order (a reading; the pages fix none): elements are taken in chunks of
    V = 16 bytes (V = 4 float32 or 8 bf16 values). Chunk c covers d in
    [c*V, c*V + V) and belongs to lane c mod 64. Each lane starts at +0 and adds
    the rounded products of its chunks in increasing d, one float32 multiply and
    one float32 add per element (no fused multiply-add). The 64 lane sums are
    then combined by a butterfly: for m = 32, 16, 8, 4, 2, 1 every lane adds the
    value of lane (l xor m); all lanes end with the same value. A bias is added
    last in float32.
    """
    x32, w32 = values32(x), values32(wg)
    T, D = x32.shape
    E = w32.shape[0]
    V = 4 if dtype == "f32" else 8
    if D % V:
        raise ValueError("D must be a multiple of the 16-byte chunk")
    chunks = D // V
    Q = -(-chunks // _LANES)
    pad = Q * _LANES * V - D
    wp = np.concatenate([w32, np.zeros((E, pad), np.float32)], axis=1).reshape(E, Q, _LANES, V)
    out = np.empty((T, E), dtype=np.float32)
    partner = {m: np.arange(_LANES) ^ m for m in (32, 16, 8, 4, 2, 1)}
    step = 512
    for t0 in range(0, T, step):
        xb = x32[t0:t0 + step]
        tb = xb.shape[0]
        xp = np.concatenate([xb, np.zeros((tb, pad), np.float32)], axis=1).reshape(tb, Q, _LANES, V)
        acc = np.zeros((tb, E, _LANES), dtype=np.float32)
        for q in range(Q):
            for i in range(V):
                prod = xp[:, None, q, :, i] * wp[None, :, q, :, i]   # rounded float32 product
                acc = acc + prod                                     # rounded float32 sum
        for m in (32, 16, 8, 4, 2, 1):
            acc = acc + acc[:, :, partner[m]]
        out[t0:t0 + tb] = acc[:, :, 0]
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float32)[None, :]
    return out


def softmax(logits: np.ndarray) -> np.ndarray:
    """p_e = exp(l_e - max l) / sum_e' exp(l_e' - max l), in float64."""
    l64 = np.asarray(logits, dtype=np.float64)
    z = np.exp(l64 - l64.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, best first; ties go to the lower index."""
    l = np.asarray(logits)
    if not np.all(np.isfinite(l)):
        raise ValueError("router logits must be finite")
    order = np.argsort(-l, axis=1, kind="stable")   # stable: equal keys keep index order
    return np.ascontiguousarray(order[:, :k].astype(np.int32))


def route(x, wg, k: int, dtype: str, bias=None, renorm: bool = False):
    """Softmax-then-top-k routing. Returns (topk_idx [T,k] int32, topk_w [T,k] float64,
    logits [T,E] float32)."""
    logits = router_logits(x, wg, dtype, bias)
    idx = select_topk(logits, k)
    p = softmax(logits)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w, logits


# ----------------------------------------------------------------------------
# dispatch metadata and permute ("Expert Parallelism (EP)", sections 1, 2, 5)
# ----------------------------------------------------------------------------

def dispatch_layout(topk_idx: np.ndarray, E: int, m_tile: int,
                    m_cap: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Tokens-per-expert metadata and the stable, tile-aligned permutation maps.

    counts[e]     number of slots (t, j) with topk_idx[t, j] == e (-1 slots skipped)
    offsets       exclusive prefix sum of ceil(counts / Mt) * Mt, length E + 1
    dst_row[t,j]  offsets[e] + rank of flat index t*k+j among e's slots (-1 if skipped)
    src_row[r]    t*k + j of the slot placed in row r, -1 for pad and unused rows
    tile_expert   expert owning each Mt-row tile, -1 for tiles past offsets[E]
    """
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    if np.any(flat >= E) or np.any(flat < -1):
        raise ValueError("topk_idx values must lie in [-1, E)")
    if m_cap is None:
        m_cap = capacity(T, k, E, m_tile)
    valid = flat >= 0
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    padded = -(-counts // m_tile) * m_tile
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    if offsets[-1] > m_cap:
        raise ValueError("m_cap too small")
    # stable counting sort of the flat slot order by expert
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")[: int(valid.sum())]
    sorted_e = flat[order]
    first = np.concatenate([[0], np.cumsum(counts)])[:-1]
    rank = np.arange(order.size) - first[sorted_e]
    dst = np.full(T * k, -1, dtype=np.int64)
    dst[order] = offsets[sorted_e] + rank
    src = np.full(m_cap, -1, dtype=np.int64)
    src[dst[order]] = order
    tile_expert = np.full(m_cap // m_tile, -1, dtype=np.int64)
    for e in range(E):
        tile_expert[offsets[e] // m_tile: offsets[e + 1] // m_tile] = e
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "dst_row": dst.reshape(T, k).astype(np.int32),
        "src_row": src.astype(np.int32),
        "tile_expert": tile_expert.astype(np.int32),
        "m_cap": int(m_cap),
    }


def permute(x: np.ndarray, layout: Dict[str, np.ndarray]) -> np.ndarray:
    """X_perm[r] = x[src_row[r] // k] for rows holding a slot, zero elsewhere.

    Copies stored values unchanged (same dtype as ``x``), so it is exact."""
    x = np.asarray(x)
    T, k = layout["dst_row"].shape
    src = layout["src_row"].astype(np.int64)
    out = np.zeros((layout["m_cap"], x.shape[1]), dtype=x.dtype)
    rows = np.nonzero(src >= 0)[0]
    out[rows] = x[src[rows] // k]
    return out


# ----------------------------------------------------------------------------
# experts (section 1, forward-path figure: the routed experts' fc1, activation, fc2;
# ETP note 4.3)
# ----------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a) = a / (1 + exp(-a)), float64."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_swiglu(A, w1e, w3e, w2e, dtype: str):
    """One expert on rows A [M, D]: h = silu(A w1e^T) * (A w3e^T) stored, then
    Y = h w2e^T stored. Returns (h, Y) as float64 values of the stored results."""
    A64 = values64(A)
    a = A64 @ values64(w1e).T
    b = A64 @ values64(w3e).T
    h = round_storage(silu(a) * b, dtype)
    y = round_storage(h @ values64(w2e).T, dtype)
    return h, y


def grouped_swiglu(x_perm, offsets, w1, w3, w2, dtype: str):
    """m-grouped fc1 -> silu(a)*b -> fc2 over the expert-contiguous buffer.

    Segment e is rows [offsets[e], offsets[e+1]) and uses w1[e], w3[e], w2[e].
    Returns (h [m_cap, F], Y [m_cap, D]) as float64 values; rows past offsets[E]
    are zero."""
    M = x_perm.shape[0]
    E, F, D = w1.shape
    h = np.zeros((M, F), dtype=np.float64)
    y = np.zeros((M, D), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            h[r0:r1], y[r0:r1] = expert_swiglu(x_perm[r0:r1], w1[e], w3[e], w2[e], dtype)
    return h, y


def shared_experts(x, ws1, ws3, ws2, dtype: str):
    """Always-active shared experts on every token, summed unweighted and stored once.

    Each shared expert's h is a stored intermediate; the sum of their fc2 outputs is
    rounded once (the shared experts behave as one expert whose F is the
    concatenation of theirs)."""
    x64 = values64(x)
    total = np.zeros((x64.shape[0], ws2.shape[1]), dtype=np.float64)
    for s in range(ws1.shape[0]):
        a = x64 @ values64(ws1[s]).T
        b = x64 @ values64(ws3[s]).T
        h = round_storage(silu(a) * b, dtype)
        total += h @ values64(ws2[s]).T
    return round_storage(total, dtype)


# ----------------------------------------------------------------------------
# combine (section 1, forward-path figure: back to token order, weighted by top-k)
# ----------------------------------------------------------------------------

def combine(y_perm, dst_row, topk_w, dtype: str, shared=None):
    """out[t] = sum_j w[t,j] * Y[dst_row[t,j]] over slots j in order (skipping -1),
    plus shared[t]; float64, stored once in the layer dtype."""
    Y = values64(y_perm)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = dst.shape
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for j in range(k):
        ok = dst[:, j] >= 0
        out[ok] += w[ok, j:j + 1] * Y[dst[ok, j]]
    if shared is not None:
        out += values64(shared)
    return round_storage(out, dtype)


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def forward(inputs: dict, k: int, m_tile: int, dtype: str, renorm: bool = False,
            m_cap: Optional[int] = None) -> dict:
    """Every intermediate of the layer on ``inputs`` (keys as produced by the input
    generator: x, wg or topk_idx/topk_w, w1, w3, w2, optional bias, ws1/ws3/ws2)."""
    x = inputs["x"]
    E = inputs["w1"].shape[0]
    res: dict = {}
    if "topk_idx" in inputs:
        idx = np.asarray(inputs["topk_idx"], dtype=np.int32)
        w = np.asarray(inputs["topk_w"], dtype=np.float64)
    else:
        idx, w, logits = route(x, inputs["wg"], k, dtype, inputs.get("bias"), renorm)
        res["logits"] = logits
    res["topk_idx"], res["topk_w"] = idx, w
    lay = dispatch_layout(idx, E, m_tile, m_cap)
    res.update(lay)
    xp = permute(x, lay)
    res["x_perm"] = xp
    h, y = grouped_swiglu(xp, lay["offsets"], inputs["w1"], inputs["w3"], inputs["w2"], dtype)
    res["h"], res["y_perm"] = h, y
    shared = None
    if "ws1" in inputs:
        shared = shared_experts(x, inputs["ws1"], inputs["ws3"], inputs["ws2"], dtype)
        res["shared"] = shared
    res["out"] = combine(y, lay["dst_row"], w, dtype, shared)
    return res


def token_outputs(tokens, x, topk_idx, topk_w, w1, w3, w2, dtype: str, shared_w=None):
    """Layer output of selected tokens only, without building the permuted buffer.

    A row's expert output depends on that row alone, so out[t] is
    sum_j w[t,j] * FFN_{idx[t,j]}(x[t]) (+ the shared experts on x[t]); the stored
    rounding points are the same as in ``forward``. Returns (out [n,D],
    h {(t,j): [F]}, y {(t,j): [D]})."""
    tokens = np.asarray(tokens, dtype=np.int64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    D = x.shape[1]
    out = np.zeros((tokens.size, D), dtype=np.float64)
    hs, ys = {}, {}
    for e in np.unique(idx[tokens]):
        if e < 0:
            continue
        rows = [(i, j) for i, t in enumerate(tokens) for j in range(idx.shape[1]) if idx[t, j] == e]
        A = np.stack([x[tokens[i]] for i, _ in rows])
        h, y = expert_swiglu(A, w1[e], w3[e], w2[e], dtype)
        for r, (i, j) in enumerate(rows):
            hs[(int(tokens[i]), j)] = h[r]
            ys[(int(tokens[i]), j)] = y[r]
    for i, t in enumerate(tokens):
        for j in range(idx.shape[1]):
            if idx[t, j] >= 0:
                out[i] += w[t, j] * ys[(int(t), j)]
    if shared_w is not None:
        out += shared_experts(x[tokens], *shared_w, dtype)
    return round_storage(out, dtype), hs, ys


# ----------------------------------------------------------------------------
# backward (section 5: each forward operator and its mirror)
# ----------------------------------------------------------------------------

def silu_grad(a: np.ndarray) -> np.ndarray:
    """d silu(a) / da = s + a s (1 - s) with s = 1 / (1 + exp(-a)), float64."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        s_ = 1.0 / (1.0 + np.exp(-a))
    return s_ * (1.0 + a * (1.0 - s_))


def preactivations(x_perm, offsets, w1, w3, dtype: str):
    """The stored fc1 pre-activations ab = [x w1[e]^T | x w3[e]^T] per segment row
    [m_cap, 2F] (rows past offsets[E] zero), as the forward keeps them for the backward."""
    E, F, _ = w1.shape
    xp = values64(x_perm)
    ab = np.zeros((xp.shape[0], 2 * F), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            ab[r0:r1, :F] = xp[r0:r1] @ values64(w1[e]).T
            ab[r0:r1, F:] = xp[r0:r1] @ values64(w3[e]).T
    return round_storage(ab, dtype)


def combine_backward(dout, y_perm, dst_row, topk_w, rows_used: int, dtype: str):
    """Mirror of ``combine``: dY[dst[t,j]] = w[t,j] * dout[t] (stored), zero on every other
    row below ``rows_used``; dw[t,j] = <dout[t], Y[dst[t,j]]> (0 for skipped slots)."""
    G = values64(dout)
    Y = values64(y_perm)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = dst.shape
    dY = np.zeros((Y.shape[0], G.shape[1]), dtype=np.float64)
    dw = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        ok = dst[:, j] >= 0
        dY[dst[ok, j]] = w[ok, j:j + 1] * G[ok]
        dw[ok, j] = np.einsum("td,td->t", G[ok], Y[dst[ok, j]])
    dY[rows_used:] = 0.0
    return round_storage(dY, dtype), dw


def swiglu_backward(dh, a, b, dtype: str):
    """da = dh * b * silu'(a), db = dh * silu(a), each stored (a, b, dh stored values)."""
    dh, a, b = values64(dh), values64(a), values64(b)
    return round_storage(dh * b * silu_grad(a), dtype), round_storage(dh * silu(a), dtype)


def expert_backward(A, a, b, h, dY, w1e, w3e, w2e, dtype: str):
    """One expert's mirror on its rows: returns (dh, da, db, dA, dW1, dW3, dW2); the
    activation gradients are stored values, the weight gradients float64."""
    A64, h64, dY64 = values64(A), values64(h), values64(dY)
    dh = round_storage(dY64 @ values64(w2e), dtype)
    da, db = swiglu_backward(dh, a, b, dtype)
    dA = round_storage(da @ values64(w1e) + db @ values64(w3e), dtype)
    return dh, da, db, dA, da.T @ A64, db.T @ A64, dY64.T @ h64


def grouped_backward(x_perm, ab, h, dY, offsets, w1, w3, w2, dtype: str):
    """``expert_backward`` over every segment [offsets[e], offsets[e+1]) of the
    expert-contiguous buffers; ab = [a | b] per row. Returns dh [m_cap,F],
    dab [m_cap,2F], dX [m_cap,D] (rows past offsets[E] zero) and dW1, dW3 [E,F,D],
    dW2 [E,D,F] (an expert without rows gets zero weight gradients)."""
    E, F, D = w1.shape
    M = np.asarray(x_perm).shape[0]
    ab64 = values64(ab)
    dh = np.zeros((M, F))
    dab = np.zeros((M, 2 * F))
    dX = np.zeros((M, D))
    dW1, dW3, dW2 = np.zeros((E, F, D)), np.zeros((E, F, D)), np.zeros((E, D, F))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        out = expert_backward(x_perm[r0:r1], ab64[r0:r1, :F], ab64[r0:r1, F:], h[r0:r1],
                              dY[r0:r1], w1[e], w3[e], w2[e], dtype)
        dh[r0:r1], dab[r0:r1, :F], dab[r0:r1, F:], dX[r0:r1] = out[:4]
        dW1[e], dW3[e], dW2[e] = out[4:]
    return dh, dab, dX, dW1, dW3, dW2


def permute_backward(dX, dst_row, dtype: str, shared=None):
    """Mirror of ``permute`` (an unpermute / scatter_add): dx[t] = sum_j dX[dst[t,j]] over
    slots in order, skipping -1, plus ``shared``, stored once."""
    dst = np.asarray(dst_row)
    return combine(dX, dst, np.ones(dst.shape), dtype, shared)


def shared_backward(x, ws1, ws3, ws2, dout, dtype: str):
    """Mirror of ``shared_experts`` (the shared experts are summed, so each one's output
    gradient is dout). Returns (dx_shared stored once over all shared experts,
    dws1, dws3, dws2 float64)."""
    x64, G = values64(x), values64(dout)
    S = ws1.shape[0]
    dx = np.zeros_like(x64)
    dws1, dws3, dws2 = np.zeros(ws1.shape), np.zeros(ws3.shape), np.zeros(ws2.shape)
    for s_ in range(S):
        a = x64 @ values64(ws1[s_]).T
        b = x64 @ values64(ws3[s_]).T
        h = round_storage(silu(a) * b, dtype)
        a, b = round_storage(a, dtype), round_storage(b, dtype)
        dh = round_storage(G @ values64(ws2[s_]), dtype)
        da, db = swiglu_backward(dh, a, b, dtype)
        dx += da @ values64(ws1[s_]) + db @ values64(ws3[s_])
        dws1[s_], dws3[s_], dws2[s_] = da.T @ x64, db.T @ x64, G.T @ h
    return round_storage(dx, dtype), dws1, dws3, dws2


def backward(inputs: dict, dout, k: int, m_tile: int, dtype: str, renorm: bool = False,
             m_cap: Optional[int] = None) -> dict:
    """Forward (with the saved pre-activations) and the mirror of every step for the
    output gradient ``dout`` [T, D]. The routing is taken as given (the router's own
    backward is not part of the path): topk_w gets its gradient dtopk_w."""
    fwd = forward(inputs, k, m_tile, dtype, renorm, m_cap)
    x = inputs["x"]
    xp, offs, h, Y = fwd["x_perm"], fwd["offsets"], fwd["h"], fwd["y_perm"]
    ab = preactivations(xp, offs, inputs["w1"], inputs["w3"], dtype)
    res = {"fwd": fwd, "ab": ab}
    dY, dw = combine_backward(dout, Y, fwd["dst_row"], fwd["topk_w"], int(offs[-1]), dtype)
    res["dy_perm"], res["dtopk_w"] = dY, dw
    dh, dab, dX, dW1, dW3, dW2 = grouped_backward(xp, ab, h, dY, offs, inputs["w1"],
                                                 inputs["w3"], inputs["w2"], dtype)
    res.update(dh=dh, dab=dab, dx_perm=dX, dw1=dW1, dw3=dW3, dw2=dW2)
    dxs = None
    if "ws1" in inputs:
        dxs, res["dws1"], res["dws3"], res["dws2"] = shared_backward(
            x, inputs["ws1"], inputs["ws3"], inputs["ws2"], dout, dtype)
        res["dx_shared"] = dxs
    res["dx"] = permute_backward(dX, fwd["dst_row"], dtype, dxs)
    return res


def token_backward(tokens, x, topk_idx, topk_w, w1, w3, w2, dout, dtype: str, shared_w=None):
    """Backward of selected tokens only, without the permuted buffer: a slot's rows of
    dY, dh, [da | db] and dX depend on its own token alone, so each sampled token's slots
    are run one expert at a time with the rounding points of ``backward``. Returns
    (dx [n,D], dtopk_w [n,k], slots {(t, j): {"dy", "dab", "dx_perm"}})."""
    tokens = np.asarray(tokens, dtype=np.int64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    G = values64(dout)
    F = w1.shape[1]
    D = G.shape[1]
    dw = np.zeros((tokens.size, idx.shape[1]))
    acc = np.zeros((tokens.size, D))
    slots = {}
    pos = {int(t): i for i, t in enumerate(tokens)}
    for e in np.unique(idx[tokens]):
        if e < 0:
            continue
        sel = [(int(t), j) for t in tokens for j in range(idx.shape[1]) if idx[t, j] == e]
        A = values64(np.stack([x[t] for t, _ in sel]))
        w1e, w3e, w2e = values64(w1[e]), values64(w3[e]), values64(w2[e])
        a_ = A @ w1e.T
        b_ = A @ w3e.T
        h = round_storage(silu(a_) * b_, dtype)
        y = round_storage(h @ w2e.T, dtype)
        a, b = round_storage(a_, dtype), round_storage(b_, dtype)
        g = np.stack([G[t] for t, _ in sel])
        wj = np.array([w[t, j] for t, j in sel])[:, None]
        dY = round_storage(wj * g, dtype)
        dh = round_storage(dY @ w2e, dtype)
        da, db = swiglu_backward(dh, a, b, dtype)
        dX = round_storage(da @ w1e + db @ w3e, dtype)
        for r, (t, j) in enumerate(sel):
            dw[pos[t], j] = float(np.dot(g[r], y[r]))
            acc[pos[t]] += dX[r]
            slots[(t, j)] = {"dy": dY[r], "dab": np.concatenate([da[r], db[r]]), "dx_perm": dX[r]}
    dxs = None
    if shared_w is not None:
        dxs = shared_backward(x[tokens], *shared_w, G[tokens], dtype)[0]
        acc += dxs
    return round_storage(acc, dtype), dw, slots


def expert_weight_grad_slices(x_rows, dy_rows, w1e, w3e, w2e, fs, dtype: str):
    """Rows f in ``fs`` of dW1 and dW3 and columns f of dW2 for one expert from its rows
    only: x_rows [n, D] are the expert's input rows and dy_rows [n, D] their stored output
    gradients (pad rows, being zero in both, may be left out). The intermediates at
    columns fs (a, b, h, dh, da, db) take the rounding points of ``backward``.
    Returns (dW1[fs, :] [|fs|, D], dW3[fs, :], dW2[:, fs] [D, |fs|]), float64."""
    fs = np.asarray(fs, dtype=np.int64)
    X = values64(x_rows)
    dY = values64(dy_rows)
    w1f, w3f = values64(w1e[fs]), values64(w3e[fs])
    a_ = X @ w1f.T
    b_ = X @ w3f.T
    h = round_storage(silu(a_) * b_, dtype)
    a, b = round_storage(a_, dtype), round_storage(b_, dtype)
    dh = round_storage(dY @ values64(w2e[:, fs]), dtype)
    da, db = swiglu_backward(dh, a, b, dtype)
    return da.T @ X, db.T @ X, dY.T @ h


# ----------------------------------------------------------------------------
# masked layout for decode (section 2: the masked grouped GEMM kernel serves decode;
# section 6 "DeepSeek-V3 量级的示例数字": how many rows each local expert receives is
# known only at run time)
# ----------------------------------------------------------------------------

def masked_layout(topk_idx: np.ndarray, E: int, cap: int) -> Dict[str, np.ndarray]:
    """Fixed slabs of ``cap`` rows per expert.

    counts[e]     valid rows of e's slab: min(#slots of e, cap)
    dst_row[t,j]  e*cap + rank of t*k+j among e's slots, -1 if skipped or dropped
    src_row[r]    t*k + j of the slot in row r, -1 for rows past counts
    dropped       number of slots whose rank reached cap
    m_cap         E*cap
    """
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    if np.any(flat >= E) or np.any(flat < -1):
        raise ValueError("topk_idx values must lie in [-1, E)")
    dst = np.full(T * k, -1, dtype=np.int64)
    src = np.full(E * cap, -1, dtype=np.int64)
    seen = np.zeros(E, dtype=np.int64)
    dropped = 0
    for a, e in enumerate(flat):          # flat slot order: the stable rank
        if e < 0:
            continue
        if seen[e] < cap:
            dst[a] = e * cap + seen[e]
            src[dst[a]] = a
        else:
            dropped += 1
        seen[e] += 1
    return {"counts": np.minimum(seen, cap).astype(np.int32),
            "dst_row": dst.reshape(T, k).astype(np.int32), "src_row": src.astype(np.int32),
            "dropped": int(dropped), "m_cap": int(E * cap)}


def masked_swiglu(x_masked, counts, cap: int, w1, w3, w2, dtype: str):
    """``expert_swiglu`` on the valid rows [e*cap, e*cap + counts[e]) of every slab.
    Returns (h [E*cap, F], Y [E*cap, D]); rows past counts are zero here (the GPU leaves
    them unwritten)."""
    E, F, D = w1.shape
    h = np.zeros((E * cap, F))
    y = np.zeros((E * cap, D))
    for e in range(E):
        r0, r1 = e * cap, e * cap + int(counts[e])
        if r1 > r0:
            h[r0:r1], y[r0:r1] = expert_swiglu(x_masked[r0:r1], w1[e], w3[e], w2[e], dtype)
    return h, y


def forward_masked(inputs: dict, k: int, cap: int, dtype: str, renorm: bool = False) -> dict:
    """The layer on the masked layout: route (or the given routing), masked_layout,
    permute into the slabs, masked_swiglu, shared experts, combine."""
    x = inputs["x"]
    E = inputs["w1"].shape[0]
    res: dict = {}
    if "topk_idx" in inputs:
        idx = np.asarray(inputs["topk_idx"], dtype=np.int32)
        w = np.asarray(inputs["topk_w"], dtype=np.float64)
    else:
        idx, w, logits = route(x, inputs["wg"], k, dtype, inputs.get("bias"), renorm)
        res["logits"] = logits
    res["topk_idx"], res["topk_w"] = idx, w
    lay = masked_layout(idx, E, cap)
    res.update(lay)
    xm = permute(x, lay)
    res["x_perm"] = xm
    h, y = masked_swiglu(xm, lay["counts"], cap, inputs["w1"], inputs["w3"], inputs["w2"], dtype)
    res["h"], res["y_perm"] = h, y
    shared = None
    if "ws1" in inputs:
        shared = shared_experts(x, inputs["ws1"], inputs["ws3"], inputs["ws2"], dtype)
        res["shared"] = shared
    res["out"] = combine(y, lay["dst_row"], w, dtype, shared)
    return res


# ----------------------------------------------------------------------------
# FP8 (e4m3) payload with MX block scales (section 6 "DeepSeek-V3 量级的示例数字": the
# dispatch payload is FP8 e4m3 with scales, the combine stays BF16)
# ----------------------------------------------------------------------------

def e4m3_decode(code) -> np.ndarray:
    """Value of OCP E4M3 codes (bias 7; exponent field 0 is subnormal, m/8 * 2^-6;
    0x7f and 0xff are NaN; no infinities), float64."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return sign * v


def e4m3_round(v) -> np.ndarray:
    """Nearest e4m3 value to float64 ``v`` (ties to an even mantissa), saturating at
    +-448: subnormals are multiples of 2^-9 below 2^-6; a normal binade [2^e, 2^(e+1))
    has steps of 2^(e-3)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.clip(e, -6, 8) - 3))
    q = np.rint(a / step) * step          # np.rint rounds halves to even
    return np.copysign(np.minimum(q, 448.0), v)   # the sign survives rounding to zero


_E4M3_VALUES = e4m3_decode(np.arange(0x7F))   # codes 0x00..0x7e, increasing


def e4m3_encode(v) -> np.ndarray:
    """Code (uint8) of e4m3 values (exact members of the format, e.g. e4m3_round's
    output); -0 encodes as 0x80."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.searchsorted(_E4M3_VALUES, np.abs(v))
    if not np.all(_E4M3_VALUES[np.minimum(mag, 0x7E)] == np.abs(v)):
        raise ValueError("not an e4m3 value")
    return (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def mx_quantize(x, block: int = 32):
    """MX quantization of the rows of ``x`` [R, C] (C a multiple of ``block``), with the
    block scale that lets no value saturate: returns (codes [R, C] uint8 e4m3,
    scales [R, C/block] uint8 = X + 127)."""
    v = values64(x)
    R, C = v.shape
    b = v.reshape(R, C // block, block)
    amax = np.abs(b).max(axis=2)
    # smallest X with amax <= 448 * 2^X: with amax = m * 2^e, 1 <= m < 2, that is e - 8
    # when m <= 1.75 (448 = 1.75 * 2^8) and e - 7 otherwise
    safe = np.where(amax > 0, amax, 1.0)
    e = np.floor(np.log2(safe))
    m = safe / 2.0 ** e
    X = np.where(amax > 0, np.where(m <= 1.75, e - 8, e - 7), -127)
    X = np.clip(X, -127, 127)
    q = e4m3_round(b / 2.0 ** X[:, :, None])
    return e4m3_encode(q).reshape(R, C), (X + 127).astype(np.uint8)


def mx_dequantize(codes, scales, block: int = 32) -> np.ndarray:
    """codes [R, C] e4m3, scales [R, C/block] E8M0 -> float64 values."""
    c = np.asarray(codes)
    R, C = c.shape
    X = np.asarray(scales, dtype=np.float64) - 127.0
    return (e4m3_decode(c).reshape(R, C // block, block) * 2.0 ** X[:, :, None]).reshape(R, C)


def expert_fc1_mx(Aq, As, w1q, w1s, w3q, w3s):
    """h = silu(A w1^T) * (A w3^T) of dequantized MX operands, float64 (rounded by the
    caller)."""
    A = mx_dequantize(Aq, As)
    return silu(A @ mx_dequantize(w1q, w1s).T) * (A @ mx_dequantize(w3q, w3s).T)


def grouped_fc1_mx(xq_perm, xs_perm, offsets, w1q, w1s, w3q, w3s):
    """``expert_fc1_mx`` per segment [offsets[e], offsets[e+1]), stored in bf16; rows past
    offsets[E] zero."""
    E = w1q.shape[0]
    F = w1q.shape[1]
    h = np.zeros((xq_perm.shape[0], F))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            h[r0:r1] = round_bf16(expert_fc1_mx(xq_perm[r0:r1], xs_perm[r0:r1], w1q[e], w1s[e],
                                                w3q[e], w3s[e]))
    return h


def forward_mxfp8(inputs: dict, k: int, m_tile: int, renorm: bool = False) -> dict:
    """The bf16 layer with an FP8 payload: route on the bf16 x, quantize x per token (MX
    e4m3), permute codes and scales, fc1 on the dequantized payload and MX-quantized
    w1, w3, then fc2, shared experts and combine in bf16."""
    x = inputs["x"]
    E, F, D = inputs["w1"].shape
    res: dict = {}
    if "topk_idx" in inputs:
        idx = np.asarray(inputs["topk_idx"], dtype=np.int32)
        w = np.asarray(inputs["topk_w"], dtype=np.float64)
    else:
        idx, w, logits = route(x, inputs["wg"], k, "bf16", inputs.get("bias"), renorm)
        res["logits"] = logits
    res["topk_idx"], res["topk_w"] = idx, w
    lay = dispatch_layout(idx, E, m_tile)
    res.update(lay)
    xq, xs = mx_quantize(x)
    res["xq"], res["xs"] = xq, xs
    res["xq_perm"], res["xs_perm"] = permute(xq, lay), permute(xs, lay)
    wq = {n: [mx_quantize(inputs[n][e]) for e in range(E)] for n in ("w1", "w3")}
    w1q = np.stack([q for q, _ in wq["w1"]]); w1s = np.stack([s_ for _, s_ in wq["w1"]])
    w3q = np.stack([q for q, _ in wq["w3"]]); w3s = np.stack([s_ for _, s_ in wq["w3"]])
    res.update(w1q=w1q, w1s=w1s, w3q=w3q, w3s=w3s)
    h = grouped_fc1_mx(res["xq_perm"], res["xs_perm"], lay["offsets"], w1q, w1s, w3q, w3s)
    y = np.zeros((h.shape[0], D))
    for e in range(E):
        r0, r1 = int(lay["offsets"][e]), int(lay["offsets"][e + 1])
        if r1 > r0:
            y[r0:r1] = round_bf16(h[r0:r1] @ values64(inputs["w2"][e]).T)
    res["h"], res["y_perm"] = h, y
    shared = None
    if "ws1" in inputs:
        shared = shared_experts(x, inputs["ws1"], inputs["ws3"], inputs["ws2"], "bf16")
        res["shared"] = shared
    res["out"] = combine(y, lay["dst_row"], w, "bf16", shared)
    return res


def token_outputs_mx(tokens, x, topk_idx, topk_w, w1, w3, w2, shared_w=None):
    """Layer output of selected tokens on the FP8 payload, one expert at a time: a row's
    quantization and fc1 depend on that row alone, and only the experts the tokens use
    have their w1, w3 quantized. Returns out [n, D] (bf16 values)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    xq, xs = mx_quantize(x[tokens])
    out = np.zeros((tokens.size, x.shape[1]))
    for e in np.unique(idx[tokens]):
        if e < 0:
            continue
        sel = [(i, j) for i, t in enumerate(tokens) for j in range(idx.shape[1]) if idx[t, j] == e]
        rows = [i for i, _ in sel]
        h = round_bf16(expert_fc1_mx(xq[rows], xs[rows], *mx_quantize(w1[e]), *mx_quantize(w3[e])))
        y = round_bf16(h @ values64(w2[e]).T)
        for r, (i, j) in enumerate(sel):
            out[i] += w[tokens[i], j] * y[r]
    if shared_w is not None:
        out += shared_experts(x[tokens], *shared_w, "bf16")
    return round_bf16(out)
