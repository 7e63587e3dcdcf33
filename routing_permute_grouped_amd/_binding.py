"""ctypes binding of libmoe_mi355x.so: argument marshalling only.

Every step of the layer runs in the library's HIP kernels; PyTorch supplies device
memory and the current HIP stream. Output buffers not passed in are allocated with
torch on the input's device. There is no fallback: if the library is missing the
import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_MX_ROWS, MOE_MX_KSTEPS = 0, 1   # moe_mx_layout_t
_STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_ESHAPE", 3: "MOE_ECAPACITY",
           4: "MOE_EWORKSPACE", 5: "MOE_EHIP", 6: "MOE_EUNSUPPORTED", 7: "MOE_ESCRATCH"}

# (name, restype, argtypes) of every symbol include/moe.h declares
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = [
    ("moe_route", _I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    ("moe_permute", _I, [_I, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ,
                         _P, _P]),
    ("moe_permute_noalloc", _I, [_I, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _P, _P, _P, _P, _P,
                                 _P, _P]),
    ("moe_grouped_swiglu", _I, [_I, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _P, _P, _P, _P,
                                _P, _SZ, _P]),
    ("moe_grouped_fc1_swiglu", _I, [_I, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _P, _P, _P,
                                    _P, _SZ, _P]),
    ("moe_grouped_fc2", _I, [_I, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _P, _P, _SZ, _P]),
    ("moe_combine", _I, [_I, _P, _P, _P, _P, _I, _I, _I, _I64, _P, _P]),
    ("moe_quantize_mxfp8", _I, [_I, _P, _I64, _I, _P, _P, _I, _P]),
    ("moe_round_bf16", _I, [_P, _P, _I64, _P]),
    ("moe_permute_mxfp8", _I, [_P, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                               _SZ, _P, _P]),
    ("moe_grouped_fc1_swiglu_mxfp8", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _P, _P,
                                          _P, _P, _P, _SZ, _P]),
    ("moe_permute_masked", _I, [_I, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    ("moe_grouped_swiglu_masked", _I, [_I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ,
                                       _P]),
    ("moe_combine_backward", _I, [_I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _P, _P]),
    ("moe_grouped_dgrad_swiglu", _I, [_I, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _P, _P, _P,
                                      _P, _SZ, _P]),
    ("moe_grouped_dgrad_fc1", _I, [_I, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _P, _P, _P,
                                   _SZ, _P]),
    ("moe_grouped_wgrad", _I, [_I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _P, _P]),
    ("moe_capacity", _I64, [_I, _I, _I, _I]),
    ("moe_grouped_workspace_bytes", _SZ, []),
    ("moe_permute_workspace_bytes", _SZ, [_I, _I, _I]),
    ("moe_status_str", ctypes.c_char_p, [_I]),
]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)} ({text})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python routing_permute_grouped_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoEError(fn, status, lib.moe_status_str(status).decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


# Host-side argument checks. The C ABI sees only pointers and sizes, so it cannot tell
# an int64 index tensor from an int32 one, nor a buffer that is too small for what a
# kernel writes; these run before any pointer is taken and raise TypeError (dtype) or
# ValueError (shape or size) naming the argument.
_LAYER_DTYPES = (torch.float32, torch.bfloat16)


def _dtype(t: Optional[torch.Tensor], name: str, dtype) -> None:
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _dims(t: torch.Tensor, name: str, nd: int) -> None:
    if t.dim() != nd:
        raise ValueError(f"{name}: {t.dim()}-d tensor, expected {nd}-d")


def _exact(t: Optional[torch.Tensor], name: str, shape, dtype=None) -> None:
    """t (if given) has exactly ``shape`` (and ``dtype``)."""
    if t is None:
        return
    if dtype is not None:
        _dtype(t, name, dtype)
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _rows(t: Optional[torch.Tensor], name: str, rows: int, cols: int, dtype=None) -> None:
    """t (if given) is [R, cols] with R >= rows: a row buffer the library writes or reads
    up to row ``rows``."""
    if t is None:
        return
    if dtype is not None:
        _dtype(t, name, dtype)
    _dims(t, name, 2)
    if t.shape[1] != cols or t.shape[0] < rows:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, needs [>= {rows}, {cols}]")


def _numel(t: Optional[torch.Tensor], name: str, n: int, dtype=None) -> None:
    """t (if given) holds at least n elements (and has ``dtype``)."""
    if t is None:
        return
    if dtype is not None:
        _dtype(t, name, dtype)
    if t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements, needs >= {n}")


def _nbytes(t: Optional[torch.Tensor], name: str, n: int) -> None:
    if t is not None and t.numel() * t.element_size() < n:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, needs >= {n}")


def _layer_dtype(t: torch.Tensor, name: str):
    if t.dtype not in _LAYER_DTYPES:
        raise TypeError(f"{name}: dtype {t.dtype}, expected float32 or bfloat16")
    return t.dtype


def _weights(w1, w3, w2, dtype, E, F, D) -> None:
    """w1, w3 [E,F,D] and w2 [E,D,F] in the activations' dtype (any may be None)."""
    for t, n, shp in ((w1, "w1", (E, F, D)), (w3, "w3", (E, F, D)), (w2, "w2", (E, D, F))):
        _exact(t, n, shp, dtype)


# ``rows_used`` (grouped calls): an upper bound, known to the caller, on offsets[E]. The
# kernels read the A operand (and the other row operands they only read) below
# offsets[E] and write the outputs below it, so a caller whose segments end before
# m_cap (the shared experts: one segment of T rows in an m_cap rounded up to the tile)
# may pass shorter read-only operands. Default: m_cap.
def _used(rows_used: Optional[int], m_cap: int) -> int:
    if rows_used is None:
        return m_cap
    if not 0 <= rows_used <= m_cap:
        raise ValueError(f"rows_used {rows_used} outside [0, m_cap={m_cap}]")
    return rows_used


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def moe_capacity(T: int, k: int, E: int, m_tile: int) -> int:
    return int(lib.moe_capacity(T, k, E, m_tile))


def moe_permute_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib.moe_permute_workspace_bytes(T, k, E))


def moe_grouped_workspace_bytes() -> int:
    return int(lib.moe_grouped_workspace_bytes())


def grouped_workspace(device) -> torch.Tensor:
    """A workspace of moe_grouped_workspace_bytes() bytes for the grouped GEMM calls."""
    return torch.empty(moe_grouped_workspace_bytes(), dtype=torch.uint8, device=device)


def _ws(ws: Optional[torch.Tensor]):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def moe_status_str(status: int) -> str:
    return lib.moe_status_str(status).decode()


def moe_route(x: torch.Tensor, wg: torch.Tensor, k: int, bias: Optional[torch.Tensor] = None,
              renorm: bool = False, want_logits: bool = False, topk_idx=None, topk_w=None,
              logits=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    _dims(x, "x", 2)
    _dims(wg, "wg", 2)
    T, D = x.shape
    E = wg.shape[0]
    dt = _layer_dtype(x, "x")
    _exact(wg, "wg", (E, D), dt)
    _exact(bias, "bias", (E,), torch.float32)
    _rows(topk_idx, "topk_idx", T, k, torch.int32)
    _rows(topk_w, "topk_w", T, k, torch.float32)
    _rows(logits, "logits", T, E, torch.float32)
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if logits is None and want_logits:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    _check("moe_route", lib.moe_route(_dt(x), _ptr(x), _ptr(wg), _ptr(bias), T, D, E, k,
                                      int(renorm), _ptr(topk_idx), _ptr(topk_w), _ptr(logits),
                                      _stream(stream)))
    return topk_idx, topk_w, logits


def _check_layout_out(o: dict, T: int, k: int, E: int, m_cap: int, m_tile: Optional[int]) -> None:
    """Metadata buffers given by the caller: counts [E], offsets [E+1], dst_row [T,k],
    src_row [m_cap], tile_expert [m_cap/m_tile] (contiguous layout only), dev_err [1]."""
    i32 = torch.int32
    _numel(o.get("counts"), "counts", E, i32)
    _numel(o.get("offsets"), "offsets", E + 1, i32)
    _rows(o.get("dst_row"), "dst_row", T, k, i32)
    _numel(o.get("src_row"), "src_row", m_cap, i32)
    if m_tile:
        _numel(o.get("tile_expert"), "tile_expert", m_cap // m_tile, i32)
    _numel(o.get("dev_err"), "dev_err", 1, i32)


def _check_idx(topk_idx: torch.Tensor, T: int) -> int:
    _dims(topk_idx, "topk_idx", 2)
    _dtype(topk_idx, "topk_idx", torch.int32)
    if topk_idx.shape[0] != T:
        raise ValueError(f"topk_idx: {topk_idx.shape[0]} rows, x has {T}")
    return topk_idx.shape[1]


def moe_permute(x: torch.Tensor, topk_idx: torch.Tensor, E: int, m_tile: int,
                m_cap: Optional[int] = None, out: Optional[dict] = None, stream=None) -> dict:
    """Returns dict with x_perm, counts, offsets, dst_row, src_row, tile_expert, dev_err,
    workspace and m_cap. Buffers given in ``out`` are reused."""
    _dims(x, "x", 2)
    T, D = x.shape
    dt = _layer_dtype(x, "x")
    k = _check_idx(topk_idx, T)
    dev = x.device
    if m_cap is None:
        m_cap = moe_capacity(T, k, E, m_tile)
    o = dict(out or {})
    _rows(o.get("x_perm"), "x_perm", m_cap, D, dt)
    _check_layout_out(o, T, k, E, m_cap, m_tile)
    ws = max(4, moe_permute_workspace_bytes(T, k, E))
    _nbytes(o.get("workspace"), "workspace", ws)
    i32 = dict(dtype=torch.int32, device=dev)
    o.setdefault("x_perm", torch.empty((m_cap, D), dtype=x.dtype, device=dev))
    o.setdefault("counts", torch.empty(E, **i32))
    o.setdefault("offsets", torch.empty(E + 1, **i32))
    o.setdefault("dst_row", torch.empty((T, k), **i32))
    o.setdefault("src_row", torch.empty(m_cap, **i32))
    o.setdefault("tile_expert", torch.empty(m_cap // m_tile, **i32))
    o.setdefault("dev_err", torch.empty(1, **i32))
    o.setdefault("workspace", torch.empty(ws, dtype=torch.uint8, device=dev))
    _check("moe_permute", lib.moe_permute(
        _dt(x), _ptr(x), _ptr(topk_idx), T, D, E, k, m_tile, m_cap, _ptr(o["x_perm"]),
        _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["dst_row"]), _ptr(o["src_row"]),
        _ptr(o["tile_expert"]), _ptr(o["workspace"]),
        o["workspace"].numel() * o["workspace"].element_size(), _ptr(o["dev_err"]),
        _stream(stream)))
    o["m_cap"] = m_cap
    return o


def moe_permute_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, E: int, m_tile: int,
                        m_cap: Optional[int] = None, out: Optional[dict] = None,
                        stream=None) -> dict:
    """moe_permute without a workspace (the library's static scratch holds its histogram
    table; see moe_permute_noalloc in include/moe.h for the size limit and the rule that
    calls overlapping on one GPU race). Allocates only the output buffers not given in
    ``out``; with all of them given the call allocates nothing."""
    _dims(x, "x", 2)
    T, D = x.shape
    dt = _layer_dtype(x, "x")
    k = _check_idx(topk_idx, T)
    dev = x.device
    if m_cap is None:
        m_cap = moe_capacity(T, k, E, m_tile)
    o = dict(out or {})
    _rows(o.get("x_perm"), "x_perm", m_cap, D, dt)
    _check_layout_out(o, T, k, E, m_cap, m_tile)
    i32 = dict(dtype=torch.int32, device=dev)
    o.setdefault("x_perm", torch.empty((m_cap, D), dtype=x.dtype, device=dev))
    o.setdefault("counts", torch.empty(E, **i32))
    o.setdefault("offsets", torch.empty(E + 1, **i32))
    o.setdefault("dst_row", torch.empty((T, k), **i32))
    o.setdefault("src_row", torch.empty(m_cap, **i32))
    o.setdefault("tile_expert", torch.empty(m_cap // m_tile, **i32))
    o.setdefault("dev_err", torch.empty(1, **i32))
    _check("moe_permute_noalloc", lib.moe_permute_noalloc(
        _dt(x), _ptr(x), _ptr(topk_idx), T, D, E, k, m_tile, m_cap, _ptr(o["x_perm"]),
        _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["dst_row"]), _ptr(o["src_row"]),
        _ptr(o["tile_expert"]), _ptr(o["dev_err"]), _stream(stream)))
    o["m_cap"] = m_cap
    return o


def _check_segments(offsets: torch.Tensor, tile_expert: torch.Tensor, E: int, m_cap: int,
                    m_tile: int) -> None:
    _numel(offsets, "offsets", E + 1, torch.int32)
    _numel(tile_expert, "tile_expert", m_cap // m_tile, torch.int32)


def moe_grouped_swiglu(x_perm: torch.Tensor, offsets: torch.Tensor, tile_expert: torch.Tensor,
                       w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor, m_tile: int,
                       m_cap: Optional[int] = None, h: Optional[torch.Tensor] = None,
                       y_perm: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None,
                       rows_used: Optional[int] = None,
                       counts: Optional[torch.Tensor] = None):
    _dims(w1, "w1", 3)
    E, F, D = w1.shape
    dt = _layer_dtype(x_perm, "x_perm")
    _weights(w1, w3, w2, dt, E, F, D)
    if m_cap is None:
        m_cap = x_perm.shape[0]
    _rows(x_perm, "x_perm", _used(rows_used, m_cap), D, dt)
    _check_segments(offsets, tile_expert, E, m_cap, m_tile)
    _numel(counts, "counts", E, torch.int32)
    _rows(h, "h", m_cap, F, dt)
    _rows(y_perm, "y_perm", m_cap, D, dt)
    dev = x_perm.device
    if h is None:
        h = torch.empty((m_cap, F), dtype=x_perm.dtype, device=dev)
    if y_perm is None:
        y_perm = torch.empty((m_cap, D), dtype=x_perm.dtype, device=dev)
    _check("moe_grouped_swiglu", lib.moe_grouped_swiglu(
        _dt(x_perm), _ptr(x_perm), _ptr(offsets), _ptr(counts), _ptr(tile_expert), E, D, F, m_tile,
        m_cap,
        _ptr(w1), _ptr(w3), _ptr(w2), _ptr(h), _ptr(y_perm), *_ws(workspace), _stream(stream)))
    return h, y_perm


def moe_grouped_fc1_swiglu(x_perm: torch.Tensor, offsets: torch.Tensor, tile_expert: torch.Tensor,
                           w1: torch.Tensor, w3: torch.Tensor, m_tile: int, m_cap: int,
                           h: torch.Tensor, ab: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None,
                           rows_used: Optional[int] = None,
                           counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h = silu(x_perm w1[e]^T) * (x_perm w3[e]^T); with ``ab`` [m_cap, 2F] also the
    pre-activations [a | b] that the backward reads."""
    _dims(w1, "w1", 3)
    E, F, D = w1.shape
    dt = _layer_dtype(x_perm, "x_perm")
    _weights(w1, w3, None, dt, E, F, D)
    _rows(x_perm, "x_perm", _used(rows_used, m_cap), D, dt)
    _check_segments(offsets, tile_expert, E, m_cap, m_tile)
    _numel(counts, "counts", E, torch.int32)
    _rows(h, "h", m_cap, F, dt)
    _rows(ab, "ab", m_cap, 2 * F, dt)
    _check("moe_grouped_fc1_swiglu", lib.moe_grouped_fc1_swiglu(
        _dt(x_perm), _ptr(x_perm), _ptr(offsets), _ptr(counts), _ptr(tile_expert), E, D, F, m_tile,
        m_cap,
        _ptr(w1), _ptr(w3), _ptr(h), _ptr(ab), *_ws(workspace), _stream(stream)))
    return h


def moe_grouped_fc2(h: torch.Tensor, offsets: torch.Tensor, tile_expert: torch.Tensor,
                    w2: torch.Tensor, m_tile: int, m_cap: int, y_perm: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None, stream=None,
                    rows_used: Optional[int] = None,
                    counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dims(w2, "w2", 3)
    E, D, F = w2.shape
    dt = _layer_dtype(h, "h")
    _weights(None, None, w2, dt, E, F, D)
    _rows(h, "h", _used(rows_used, m_cap), F, dt)
    _check_segments(offsets, tile_expert, E, m_cap, m_tile)
    _numel(counts, "counts", E, torch.int32)
    _rows(y_perm, "y_perm", m_cap, D, dt)
    _check("moe_grouped_fc2", lib.moe_grouped_fc2(
        _dt(h), _ptr(h), _ptr(offsets), _ptr(counts), _ptr(tile_expert), E, D, F, m_tile, m_cap,
        _ptr(w2),
        _ptr(y_perm), *_ws(workspace), _stream(stream)))
    return y_perm


def moe_combine(y_perm: torch.Tensor, dst_row: torch.Tensor, topk_w: Optional[torch.Tensor],
                shared: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                m_cap: Optional[int] = None, stream=None) -> torch.Tensor:
    """out[t] = sum_j topk_w[t,j] y_perm[dst_row[t,j]] (+ shared[t]); ``topk_w`` None means
    unit weights (the unpermute-and-sum that is the permute's backward)."""
    _dims(dst_row, "dst_row", 2)
    _dtype(dst_row, "dst_row", torch.int32)
    _dims(y_perm, "y_perm", 2)
    T, k = dst_row.shape
    D = y_perm.shape[1]
    dt = _layer_dtype(y_perm, "y_perm")
    if m_cap is None:
        m_cap = y_perm.shape[0]
    _rows(y_perm, "y_perm", m_cap, D, dt)
    _exact(topk_w, "topk_w", (T, k), torch.float32)
    _rows(shared, "shared", T, D, dt)
    _rows(out, "out", T, D, dt)
    if out is None:
        out = torch.empty((T, D), dtype=y_perm.dtype, device=y_perm.device)
    _check("moe_combine", lib.moe_combine(
        _dt(y_perm), _ptr(y_perm), _ptr(dst_row), _ptr(topk_w), _ptr(shared), T, D, k, m_cap,
        _ptr(out), _stream(stream)))
    return out


def moe_combine_backward(dout: torch.Tensor, y_perm: torch.Tensor, src_row: torch.Tensor,
                         offsets: torch.Tensor, dst_row: torch.Tensor, topk_w: torch.Tensor,
                         m_cap: Optional[int] = None, dy_perm: Optional[torch.Tensor] = None,
                         dtopk_w: Optional[torch.Tensor] = None, stream=None):
    """Returns (dy_perm [m_cap, D], dtopk_w [T, k] float32)."""
    _dims(dst_row, "dst_row", 2)
    _dims(dout, "dout", 2)
    T, k = dst_row.shape
    D = dout.shape[1]
    E = offsets.shape[0] - 1
    dt = _layer_dtype(dout, "dout")
    if m_cap is None:
        m_cap = y_perm.shape[0]
    _rows(dout, "dout", T, D, dt)
    _rows(y_perm, "y_perm", m_cap, D, dt)
    _numel(src_row, "src_row", m_cap, torch.int32)
    _dtype(offsets, "offsets", torch.int32)
    _dtype(dst_row, "dst_row", torch.int32)
    _exact(topk_w, "topk_w", (T, k), torch.float32)
    _rows(dy_perm, "dy_perm", m_cap, D, dt)
    _exact(dtopk_w, "dtopk_w", (T, k), torch.float32)
    if dy_perm is None:
        dy_perm = torch.empty((m_cap, D), dtype=dout.dtype, device=dout.device)
    if dtopk_w is None:
        dtopk_w = torch.empty((T, k), dtype=torch.float32, device=dout.device)
    _check("moe_combine_backward", lib.moe_combine_backward(
        _dt(dout), _ptr(dout), _ptr(y_perm), _ptr(src_row), _ptr(offsets), _ptr(dst_row),
        _ptr(topk_w), T, D, E, k, m_cap, _ptr(dy_perm), _ptr(dtopk_w), _stream(stream)))
    return dy_perm, dtopk_w


def moe_grouped_dgrad_swiglu(dy_perm: torch.Tensor, offsets: torch.Tensor,
                             tile_expert: torch.Tensor, w2: torch.Tensor, ab: torch.Tensor,
                             m_tile: int, m_cap: Optional[int] = None,
                             dab: Optional[torch.Tensor] = None, dh: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, stream=None,
                             rows_used: Optional[int] = None,
                             counts: Optional[torch.Tensor] = None):
    """dab [m_cap, 2F] = [dh*b*silu'(a) | dh*silu(a)] with dh = dy_perm w2[e] (w2 [E,D,F]);
    ``dh`` [m_cap, F], when given, receives dh."""
    _dims(w2, "w2", 3)
    E, D, F = w2.shape
    dt = _layer_dtype(dy_perm, "dy_perm")
    _weights(None, None, w2, dt, E, F, D)
    if m_cap is None:
        m_cap = dy_perm.shape[0]
    ru = _used(rows_used, m_cap)
    _rows(dy_perm, "dy_perm", ru, D, dt)
    _check_segments(offsets, tile_expert, E, m_cap, m_tile)
    _numel(counts, "counts", E, torch.int32)
    _rows(ab, "ab", ru, 2 * F, dt)
    _rows(dab, "dab", m_cap, 2 * F, dt)
    _rows(dh, "dh", m_cap, F, dt)
    if dab is None:
        dab = torch.empty((m_cap, 2 * F), dtype=dy_perm.dtype, device=dy_perm.device)
    _check("moe_grouped_dgrad_swiglu", lib.moe_grouped_dgrad_swiglu(
        _dt(dy_perm), _ptr(dy_perm), _ptr(offsets), _ptr(counts), _ptr(tile_expert), E, D, F,
        m_tile, m_cap,
        _ptr(w2), _ptr(ab), _ptr(dab), _ptr(dh), *_ws(workspace), _stream(stream)))
    return dab


def moe_grouped_dgrad_fc1(dab: torch.Tensor, offsets: torch.Tensor, tile_expert: torch.Tensor,
                          w1: torch.Tensor, w3: torch.Tensor, m_tile: int,
                          m_cap: Optional[int] = None, dx_perm: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None,
                          rows_used: Optional[int] = None,
                          counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dx_perm [m_cap, D] = da w1[e] + db w3[e] for dab = [da | db] (w1, w3 [E,F,D])."""
    _dims(w1, "w1", 3)
    E, F, D = w1.shape
    dt = _layer_dtype(dab, "dab")
    _weights(w1, w3, None, dt, E, F, D)
    if m_cap is None:
        m_cap = dab.shape[0]
    _rows(dab, "dab", _used(rows_used, m_cap), 2 * F, dt)
    _check_segments(offsets, tile_expert, E, m_cap, m_tile)
    _numel(counts, "counts", E, torch.int32)
    _rows(dx_perm, "dx_perm", m_cap, D, dt)
    if dx_perm is None:
        dx_perm = torch.empty((m_cap, D), dtype=dab.dtype, device=dab.device)
    _check("moe_grouped_dgrad_fc1", lib.moe_grouped_dgrad_fc1(
        _dt(dab), _ptr(dab), _ptr(offsets), _ptr(counts), _ptr(tile_expert), E, D, F, m_tile,
        m_cap, _ptr(w1),
        _ptr(w3), _ptr(dx_perm), *_ws(workspace), _stream(stream)))
    return dx_perm


def moe_grouped_wgrad(P: torch.Tensor, Q: torch.Tensor, offsets: torch.Tensor, m_tile: int,
                      m_cap: Optional[int] = None, NS: Optional[int] = None,
                      out_lo: Optional[torch.Tensor] = None, out_hi: Optional[torch.Tensor] = None,
                      stream=None, rows_used: Optional[int] = None,
                      counts: Optional[torch.Tensor] = None):
    """out[e] = P[seg e]^T Q[seg e] in float32 (P [m_cap, N1], Q [m_cap, N2]), rows < NS in
    out_lo [E, NS, N2] and the rest in out_hi [E, N1-NS, N2]. Returns (out_lo, out_hi)."""
    _dims(P, "P", 2)
    _dims(Q, "Q", 2)
    N1, N2 = P.shape[1], Q.shape[1]
    E = offsets.shape[0] - 1
    dt = _layer_dtype(P, "P")
    if m_cap is None:
        m_cap = P.shape[0]
    ru = _used(rows_used, m_cap)
    _rows(P, "P", ru, N1, dt)
    _rows(Q, "Q", ru, N2, dt)
    _dtype(offsets, "offsets", torch.int32)
    _numel(counts, "counts", E, torch.int32)
    NS = N1 if NS is None else NS
    _exact(out_lo, "out_lo", (E, NS, N2), torch.float32)
    _exact(out_hi, "out_hi", (E, N1 - NS, N2), torch.float32)
    f32 = dict(dtype=torch.float32, device=P.device)
    if out_lo is None and NS > 0:
        out_lo = torch.empty((E, NS, N2), **f32)
    if out_hi is None and NS < N1:
        out_hi = torch.empty((E, N1 - NS, N2), **f32)
    _check("moe_grouped_wgrad", lib.moe_grouped_wgrad(
        _dt(P), _ptr(P), _ptr(Q), _ptr(offsets), _ptr(counts), E, N1, N2, NS, m_tile, m_cap,
        _ptr(out_lo),
        _ptr(out_hi), _stream(stream)))
    return out_lo, out_hi


def moe_permute_masked(x: torch.Tensor, topk_idx: torch.Tensor, E: int, cap: int,
                       out: Optional[dict] = None, stream=None) -> dict:
    """The masked layout: returns dict with x_masked [E*cap, D], counts, dst_row, src_row,
    dev_err, workspace, cap and m_cap = E*cap. Buffers given in ``out`` are reused."""
    _dims(x, "x", 2)
    T, D = x.shape
    dt = _layer_dtype(x, "x")
    k = _check_idx(topk_idx, T)
    dev = x.device
    o = dict(out or {})
    _rows(o.get("x_masked"), "x_masked", E * cap, D, dt)
    _check_layout_out(o, T, k, E, E * cap, None)
    ws = max(4, moe_permute_workspace_bytes(T, k, E))
    _nbytes(o.get("workspace"), "workspace", ws)
    i32 = dict(dtype=torch.int32, device=dev)
    o.setdefault("x_masked", torch.empty((E * cap, D), dtype=x.dtype, device=dev))
    o.setdefault("counts", torch.empty(E, **i32))
    o.setdefault("dst_row", torch.empty((T, k), **i32))
    o.setdefault("src_row", torch.empty(E * cap, **i32))
    o.setdefault("dev_err", torch.empty(1, **i32))
    o.setdefault("workspace", torch.empty(ws, dtype=torch.uint8, device=dev))
    _check("moe_permute_masked", lib.moe_permute_masked(
        _dt(x), _ptr(x), _ptr(topk_idx), T, D, E, k, cap, _ptr(o["x_masked"]), _ptr(o["counts"]),
        _ptr(o["dst_row"]), _ptr(o["src_row"]), _ptr(o["workspace"]),
        o["workspace"].numel() * o["workspace"].element_size(), _ptr(o["dev_err"]),
        _stream(stream)))
    o["cap"], o["m_cap"] = cap, E * cap
    return o


def moe_grouped_swiglu_masked(x_masked: torch.Tensor, counts: torch.Tensor, w1: torch.Tensor,
                              w3: torch.Tensor, w2: torch.Tensor, cap: int,
                              h: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None, stream=None):
    """h, y on the valid rows of every slab of the masked layout."""
    _dims(w1, "w1", 3)
    E, F, D = w1.shape
    dt = _layer_dtype(x_masked, "x_masked")
    _weights(w1, w3, w2, dt, E, F, D)
    _rows(x_masked, "x_masked", E * cap, D, dt)
    _numel(counts, "counts", E, torch.int32)
    _rows(h, "h", E * cap, F, dt)
    _rows(y, "y", E * cap, D, dt)
    dev = x_masked.device
    if h is None:
        h = torch.empty((E * cap, F), dtype=x_masked.dtype, device=dev)
    if y is None:
        y = torch.empty((E * cap, D), dtype=x_masked.dtype, device=dev)
    _check("moe_grouped_swiglu_masked", lib.moe_grouped_swiglu_masked(
        _dt(x_masked), _ptr(x_masked), _ptr(counts), E, D, F, cap, _ptr(w1), _ptr(w3), _ptr(w2),
        _ptr(h), _ptr(y), *_ws(workspace), _stream(stream)))
    return h, y


def _bytes_ptr(t: torch.Tensor) -> int:
    if t.dtype != torch.uint8:
        raise TypeError("FP8 codes and scales are uint8 tensors")
    return _ptr(t)


def moe_round_bf16(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """bf16 of float32 x (any shape), rounded as every bf16 value the library stores.
    Returns out (bfloat16, x's shape)."""
    _dtype(x, "x", torch.float32)
    _exact(out, "out", tuple(x.shape), torch.bfloat16)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _check("moe_round_bf16", lib.moe_round_bf16(_ptr(x), _ptr(out), x.numel(), _stream(stream)))
    return out


def moe_quantize_mxfp8(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None, layout: int = 0, stream=None):
    """MX e4m3 codes and E8M0 scales of the rows of x [..., C]. Returns (q uint8 [..., C],
    scales): layout MOE_MX_ROWS, uint8 [..., C/32] (C a multiple of 32); MOE_MX_KSTEPS,
    the GEMM's k-step words as uint8 [C/128, R, 4] (R rows, C a multiple of 128)."""
    _layer_dtype(x, "x")
    C = x.shape[-1]
    R = x.numel() // C
    _numel(q, "q", R * C, torch.uint8)
    _numel(scales, "scales", R * (C // 32), torch.uint8)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        shape = (C // 128, R, 4) if layout == MOE_MX_KSTEPS else (*x.shape[:-1], C // 32)
        scales = torch.empty(shape, dtype=torch.uint8, device=x.device)
    _check("moe_quantize_mxfp8", lib.moe_quantize_mxfp8(
        _dt(x), _ptr(x), R, C, _bytes_ptr(q), _bytes_ptr(scales), layout, _stream(stream)))
    return q, scales


def moe_permute_mxfp8(xq: torch.Tensor, xs: torch.Tensor, topk_idx: torch.Tensor, E: int,
                      m_tile: int, m_cap: Optional[int] = None, out: Optional[dict] = None,
                      stream=None) -> dict:
    """moe_permute for the FP8 payload: dict with xq_perm [m_cap, D], xs_perm (the scales
    in k-step words, uint8 [D/128, m_cap, 4]) and the metadata."""
    _dims(xq, "xq", 2)
    T, D = xq.shape
    _dtype(xq, "xq", torch.uint8)
    _numel(xs, "xs", T * (D // 32), torch.uint8)
    k = _check_idx(topk_idx, T)
    dev = xq.device
    if m_cap is None:
        m_cap = moe_capacity(T, k, E, m_tile)
    o = dict(out or {})
    _rows(o.get("xq_perm"), "xq_perm", m_cap, D, torch.uint8)
    _numel(o.get("xs_perm"), "xs_perm", (D // 128) * m_cap * 4, torch.uint8)
    _check_layout_out(o, T, k, E, m_cap, m_tile)
    ws = max(4, moe_permute_workspace_bytes(T, k, E))
    _nbytes(o.get("workspace"), "workspace", ws)
    i32 = dict(dtype=torch.int32, device=dev)
    o.setdefault("xq_perm", torch.empty((m_cap, D), dtype=torch.uint8, device=dev))
    o.setdefault("xs_perm", torch.empty((D // 128, m_cap, 4), dtype=torch.uint8, device=dev))
    o.setdefault("counts", torch.empty(E, **i32))
    o.setdefault("offsets", torch.empty(E + 1, **i32))
    o.setdefault("dst_row", torch.empty((T, k), **i32))
    o.setdefault("src_row", torch.empty(m_cap, **i32))
    o.setdefault("tile_expert", torch.empty(m_cap // m_tile, **i32))
    o.setdefault("dev_err", torch.empty(1, **i32))
    o.setdefault("workspace", torch.empty(ws, dtype=torch.uint8, device=dev))
    _check("moe_permute_mxfp8", lib.moe_permute_mxfp8(
        _bytes_ptr(xq), _bytes_ptr(xs), _ptr(topk_idx), T, D, E, k, m_tile, m_cap,
        _bytes_ptr(o["xq_perm"]), _bytes_ptr(o["xs_perm"]), _ptr(o["counts"]), _ptr(o["offsets"]),
        _ptr(o["dst_row"]), _ptr(o["src_row"]), _ptr(o["tile_expert"]), _ptr(o["workspace"]),
        o["workspace"].numel() * o["workspace"].element_size(), _ptr(o["dev_err"]),
        _stream(stream)))
    o["m_cap"] = m_cap
    return o


def moe_grouped_fc1_swiglu_mxfp8(xq_perm: torch.Tensor, xs_perm: torch.Tensor,
                                 offsets: torch.Tensor, tile_expert: torch.Tensor,
                                 w1q: torch.Tensor, w1s: torch.Tensor, w3q: torch.Tensor,
                                 w3s: torch.Tensor, m_tile: int, m_cap: Optional[int] = None,
                                 h: Optional[torch.Tensor] = None,
                                 workspace: Optional[torch.Tensor] = None,
                                 stream=None, counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h [m_cap, F] bf16 = silu(a)*b from the FP8 payload and MX-quantized w1, w3 (codes
    [E, F, D], scales in k-step words [D/128, E*F, 4])."""
    _dims(w1q, "w1q", 3)
    E, F, D = w1q.shape
    if m_cap is None:
        m_cap = xq_perm.shape[0]
    _rows(xq_perm, "xq_perm", m_cap, D, torch.uint8)
    _numel(xs_perm, "xs_perm", (D // 128) * m_cap * 4, torch.uint8)
    _exact(w1q, "w1q", (E, F, D), torch.uint8)
    _exact(w3q, "w3q", (E, F, D), torch.uint8)
    _numel(w1s, "w1s", (D // 128) * E * F * 4, torch.uint8)
    _numel(w3s, "w3s", (D // 128) * E * F * 4, torch.uint8)
    _check_segments(offsets, tile_expert, E, m_cap, m_tile)
    _numel(counts, "counts", E, torch.int32)
    _rows(h, "h", m_cap, F, torch.bfloat16)
    if h is None:
        h = torch.empty((m_cap, F), dtype=torch.bfloat16, device=xq_perm.device)
    _check("moe_grouped_fc1_swiglu_mxfp8", lib.moe_grouped_fc1_swiglu_mxfp8(
        _bytes_ptr(xq_perm), _bytes_ptr(xs_perm), _ptr(offsets), _ptr(counts), _ptr(tile_expert), E,
        D, F,
        m_tile, m_cap, _bytes_ptr(w1q), _bytes_ptr(w1s), _bytes_ptr(w3q), _bytes_ptr(w3s), _ptr(h),
        *_ws(workspace), _stream(stream)))
    return h
