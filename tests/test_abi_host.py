"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before touching the GPU. No call here reaches a kernel launch:
every argument set below is invalid, and validation runs before any HIP call."""
import ctypes
import os
import re

import pytest

import routing_permute_grouped_amd as rpg
from oracle import moe_oracle as orc

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_ECAPACITY, MOE_EWORKSPACE, MOE_EUNSUPPORTED = 0, 1, 2, 3, 4, 6
FAKE = 0x10000   # aligned, non-null; never dereferenced because every call is rejected
lib = rpg.lib


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?![\s/*#])[^\n(]*?\b(moe_[a-z_0-9]+)\(", text, re.M)))


def test_header_declares_the_calls_and_helpers():
    assert declared_symbols() == sorted(["moe_route", "moe_permute", "moe_grouped_swiglu",
                                         "moe_grouped_fc1_swiglu", "moe_grouped_fc2",
                                         "moe_combine", "moe_combine_backward",
                                         "moe_grouped_dgrad_swiglu", "moe_grouped_dgrad_fc1",
                                         "moe_grouped_wgrad", "moe_permute_masked",
                                         "moe_grouped_swiglu_masked", "moe_quantize_mxfp8",
                                         "moe_permute_mxfp8", "moe_grouped_fc1_swiglu_mxfp8",
                                         "moe_permute_noalloc", "moe_round_bf16",
                                         "moe_capacity",
                                         "moe_grouped_workspace_bytes",
                                         "moe_permute_workspace_bytes", "moe_status_str"])


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(rpg.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(raw, name), name
    assert sorted(n for n, _, _ in rpg.SIGNATURES) == declared_symbols()


@pytest.mark.parametrize("T,k,E,mt", [(256, 2, 8, 16), (4096, 2, 8, 128), (8192, 6, 64, 128),
                                      (16384, 4, 32, 128), (2049, 8, 32, 128), (1, 1, 1, 16),
                                      (3, 2, 64, 256), (100, 4, 1024, 32)])
def test_capacity_matches_oracle(T, k, E, mt):
    assert rpg.moe_capacity(T, k, E, mt) == orc.capacity(T, k, E, mt)


def test_capacity_and_workspace_reject_bad_sizes():
    assert rpg.moe_capacity(0, 2, 8, 128) == -1
    assert rpg.moe_capacity(8, 2, 8, 100) == -1
    assert rpg.moe_permute_workspace_bytes(8, 2, 0) == 0
    assert rpg.moe_permute_workspace_bytes(8, 2, 2000) == 0
    assert rpg.moe_permute_workspace_bytes(1000, 2, 8) == 4 * (8 + 1) * 4


def test_status_strings():
    for s in range(8):
        assert len(rpg.moe_status_str(s)) > 0
    assert rpg.moe_status_str(99) == "unknown status"


def route(dt=0, x=FAKE, wg=FAKE, bias=None, T=16, D=128, E=8, k=2, renorm=0, idx=FAKE, w=FAKE,
          logits=None):
    return lib.moe_route(dt, x, wg, bias, T, D, E, k, renorm, idx, w, logits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), MOE_EINVAL), (dict(x=None), MOE_EINVAL), (dict(x=FAKE + 8), MOE_EINVAL),
    (dict(idx=None), MOE_EINVAL), (dict(bias=FAKE + 2), MOE_EINVAL), (dict(renorm=2), MOE_EINVAL),
    (dict(T=0), MOE_ESHAPE), (dict(D=100), MOE_ESHAPE), (dict(D=0), MOE_ESHAPE),
    (dict(E=1025), MOE_ESHAPE), (dict(E=0), MOE_ESHAPE), (dict(k=0), MOE_ESHAPE),
    (dict(k=9), MOE_ESHAPE), (dict(E=64, k=33), MOE_ESHAPE),
])
def test_route_validation(kw, code):
    assert route(**kw) == code


def permute(dt=1, x=FAKE, idx=FAKE, T=64, D=128, E=8, k=2, mt=16, m_cap=None, xp=FAKE,
            ws=FAKE, ws_bytes=1 << 20, err=FAKE, counts=FAKE):
    if m_cap is None:
        m_cap = orc.capacity(T, k, E, mt)
    return lib.moe_permute(dt, x, idx, T, D, E, k, mt, m_cap, xp, counts, FAKE, FAKE, FAKE, FAKE,
                           ws, ws_bytes, err, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=-1), MOE_EINVAL), (dict(x=None), MOE_EINVAL), (dict(xp=FAKE + 4), MOE_EINVAL),
    (dict(err=None), MOE_EINVAL), (dict(counts=FAKE + 1), MOE_EINVAL),
    (dict(T=-5), MOE_ESHAPE), (dict(D=96), MOE_ESHAPE), (dict(E=1025), MOE_ESHAPE),
    (dict(k=3, E=2), MOE_ESHAPE), (dict(mt=48), MOE_ESHAPE),
    (dict(m_cap=16), MOE_ECAPACITY), (dict(m_cap=orc.capacity(64, 2, 8, 16) + 8), MOE_ECAPACITY),
    (dict(ws_bytes=3), MOE_EWORKSPACE),
])
def test_permute_validation(kw, code):
    assert permute(**kw) == code


def grouped(dt=1, xp=FAKE, E=8, D=128, F=256, mt=128, m_cap=1024, w1=FAKE, h=FAKE, ws=None,
            ws_bytes=0, counts=None):
    return lib.moe_grouped_swiglu(dt, xp, FAKE, counts, FAKE, E, D, F, mt, m_cap, w1, FAKE, FAKE, h,
                                  FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), MOE_EINVAL), (dict(w1=None), MOE_EINVAL), (dict(h=FAKE + 8), MOE_EINVAL),
    (dict(E=0), MOE_ESHAPE), (dict(F=100), MOE_ESHAPE), (dict(D=32), MOE_ESHAPE),
    (dict(mt=7), MOE_ESHAPE), (dict(m_cap=0), MOE_ECAPACITY), (dict(m_cap=1000), MOE_ECAPACITY),
    (dict(D=65536, F=32768), MOE_ESHAPE), (dict(mt=64, m_cap=1000), MOE_ECAPACITY),
    (dict(mt=16, m_cap=1016), MOE_ECAPACITY), (dict(ws=FAKE + 8, ws_bytes=1 << 20), MOE_EINVAL),
    (dict(dt=7, ws=FAKE, ws_bytes=1 << 20), MOE_EINVAL), (dict(counts=FAKE + 2), MOE_EINVAL),
])
def test_grouped_validation(kw, code):
    assert grouped(**kw) == code


def test_split_grouped_calls_validate():
    assert lib.moe_grouped_fc1_swiglu(1, FAKE, FAKE, None, FAKE, 8, 128, 256, 128, 1024, None, FAKE,
                                      FAKE, None, None, 0, None) == MOE_EINVAL
    assert lib.moe_grouped_fc1_swiglu(1, FAKE, FAKE, None, FAKE, 8, 128, 250, 128, 1024, FAKE, FAKE,
                                      FAKE, None, None, 0, None) == MOE_ESHAPE
    assert lib.moe_grouped_fc1_swiglu(1, FAKE, FAKE, None, FAKE, 8, 128, 256, 128, 1024, FAKE, FAKE,
                                      FAKE, None, FAKE + 4, 1 << 20, None) == MOE_EINVAL
    assert lib.moe_grouped_fc1_swiglu(1, FAKE, FAKE, None, FAKE, 8, 128, 256, 128, 1024, FAKE, FAKE,
                                      FAKE, FAKE + 2, None, 0, None) == MOE_EINVAL
    assert lib.moe_grouped_fc2(1, FAKE, FAKE, None, FAKE, 8, 128, 256, 128, 1000, FAKE, FAKE,
                               None, 0, None) == MOE_ECAPACITY
    assert lib.moe_grouped_fc2(1, FAKE, FAKE, None, FAKE, 8, 128, 256, 64, 1000, FAKE, FAKE,
                               FAKE, 1 << 20, None) == MOE_ECAPACITY


def test_grouped_workspace_size_is_whole_slots():
    n = rpg.moe_grouped_workspace_bytes()
    assert n > 0 and n % (256 * 256 * 4) == 0


def combine(dt=1, y=FAKE, dst=FAKE, w=FAKE, shared=None, T=64, D=128, k=2, m_cap=640, out=FAKE):
    return lib.moe_combine(dt, y, dst, w, shared, T, D, k, m_cap, out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), MOE_EINVAL), (dict(y=None), MOE_EINVAL), (dict(shared=FAKE + 4), MOE_EINVAL),
    (dict(out=FAKE + 2), MOE_EINVAL), (dict(T=0), MOE_ESHAPE), (dict(k=0), MOE_ESHAPE),
    (dict(k=33), MOE_ESHAPE), (dict(D=65), MOE_ESHAPE), (dict(m_cap=0), MOE_ESHAPE),
])
def test_combine_validation(kw, code):
    assert combine(**kw) == code


def test_combine_accepts_missing_weights_only_as_null():
    # NULL weights are the unit-weight unpermute; a misaligned pointer is still rejected
    assert combine(w=FAKE + 2) == MOE_EINVAL
    assert combine(w=None, T=0) == MOE_ESHAPE


@pytest.mark.parametrize("x,y,n,code", [
    (FAKE, FAKE, -1, MOE_ESHAPE), (FAKE, FAKE, 1 << 40, MOE_ESHAPE), (None, FAKE, 10, MOE_EINVAL),
    (FAKE, None, 10, MOE_EINVAL), (FAKE + 2, FAKE, 10, MOE_EINVAL), (FAKE, FAKE + 1, 10, MOE_EINVAL),
    (None, None, 0, 0),   # nothing to round: no pointer is needed and nothing is launched
])
def test_round_bf16_validation(x, y, n, code):
    assert lib.moe_round_bf16(x, y, n, None) == code


def combine_bwd(dt=1, dout=FAKE, y=FAKE, src=FAKE, off=FAKE, dst=FAKE, w=FAKE, T=64, D=128, E=8,
                k=2, m_cap=640, dy=FAKE, dw=FAKE):
    return lib.moe_combine_backward(dt, dout, y, src, off, dst, w, T, D, E, k, m_cap, dy, dw, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), MOE_EINVAL), (dict(dout=None), MOE_EINVAL), (dict(y=FAKE + 4), MOE_EINVAL),
    (dict(src=None), MOE_EINVAL), (dict(off=FAKE + 1), MOE_EINVAL), (dict(w=None), MOE_EINVAL),
    (dict(dy=FAKE + 8), MOE_EINVAL), (dict(dw=None), MOE_EINVAL), (dict(T=0), MOE_ESHAPE),
    (dict(D=96), MOE_ESHAPE), (dict(E=0), MOE_ESHAPE), (dict(E=1025), MOE_ESHAPE),
    (dict(k=0), MOE_ESHAPE), (dict(k=33), MOE_ESHAPE), (dict(m_cap=0), MOE_ESHAPE),
])
def test_combine_backward_validation(kw, code):
    assert combine_bwd(**kw) == code


def dgrad(dt=1, dy=FAKE, E=8, D=128, F=256, mt=128, m_cap=1024, w2=FAKE, ab=FAKE, dab=FAKE,
          dh=None, ws=None, ws_bytes=0):
    return lib.moe_grouped_dgrad_swiglu(dt, dy, FAKE, None, FAKE, E, D, F, mt, m_cap, w2, ab, dab, dh,
                                        ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=9), MOE_EINVAL), (dict(dy=None), MOE_EINVAL), (dict(w2=FAKE + 2), MOE_EINVAL),
    (dict(ab=None), MOE_EINVAL), (dict(dab=None), MOE_EINVAL), (dict(dh=FAKE + 8), MOE_EINVAL),
    (dict(ws=FAKE + 4, ws_bytes=1 << 20), MOE_EINVAL), (dict(E=0), MOE_ESHAPE),
    (dict(F=200), MOE_ESHAPE), (dict(D=65536, F=32768), MOE_ESHAPE),
    (dict(m_cap=1000), MOE_ECAPACITY), (dict(mt=32, m_cap=1000), MOE_ECAPACITY),
])
def test_dgrad_validation(kw, code):
    assert dgrad(**kw) == code


def dgrad_fc1(dt=1, dab=FAKE, E=8, D=128, F=256, mt=128, m_cap=1024, w1=FAKE, w3=FAKE, dx=FAKE,
              ws=None, ws_bytes=0):
    return lib.moe_grouped_dgrad_fc1(dt, dab, FAKE, None, FAKE, E, D, F, mt, m_cap, w1, w3, dx, ws,
                                     ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), MOE_EINVAL), (dict(dab=None), MOE_EINVAL), (dict(w1=None), MOE_EINVAL),
    (dict(w3=FAKE + 2), MOE_EINVAL), (dict(dx=FAKE + 4), MOE_EINVAL),
    (dict(ws=FAKE + 8, ws_bytes=1 << 20), MOE_EINVAL), (dict(E=1025), MOE_ESHAPE),
    (dict(D=100), MOE_ESHAPE), (dict(mt=100), MOE_ESHAPE), (dict(m_cap=0), MOE_ECAPACITY),
    (dict(mt=16, m_cap=1000), MOE_ECAPACITY),
])
def test_dgrad_fc1_validation(kw, code):
    assert dgrad_fc1(**kw) == code


def wgrad(dt=1, P=FAKE, Q=FAKE, off=FAKE, E=8, N1=512, N2=128, NS=256, mt=128, m_cap=1024,
          lo=FAKE, hi=FAKE):
    return lib.moe_grouped_wgrad(dt, P, Q, off, None, E, N1, N2, NS, mt, m_cap, lo, hi, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=4), MOE_EINVAL), (dict(P=None), MOE_EINVAL), (dict(Q=FAKE + 2), MOE_EINVAL),
    (dict(off=None), MOE_EINVAL), (dict(lo=None), MOE_EINVAL), (dict(hi=FAKE + 4), MOE_EINVAL),
    (dict(NS=-1), MOE_ESHAPE), (dict(NS=513), MOE_ESHAPE), (dict(N1=500), MOE_ESHAPE),
    (dict(N2=0), MOE_ESHAPE), (dict(E=0), MOE_ESHAPE), (dict(mt=48), MOE_ESHAPE),
    (dict(m_cap=1000), MOE_ECAPACITY), (dict(m_cap=0), MOE_ECAPACITY),
    (dict(N1=65536, NS=0, m_cap=1 << 15), MOE_ESHAPE),
])
def test_wgrad_validation(kw, code):
    assert wgrad(**kw) == code


def test_wgrad_needs_only_the_output_halves_it_writes():
    # NS = N1: every row goes to out_lo, so out_hi may be NULL (and the reverse); these
    # calls are made invalid by an unrelated size so nothing launches
    assert wgrad(NS=512, hi=None, N2=100) == MOE_ESHAPE
    assert wgrad(NS=0, lo=None, N2=100) == MOE_ESHAPE
    assert wgrad(NS=256, hi=None) == MOE_EINVAL


def permute_masked(dt=1, x=FAKE, idx=FAKE, T=64, D=128, E=8, k=2, cap=16, xm=FAKE, ws=FAKE,
                   ws_bytes=1 << 20):
    return lib.moe_permute_masked(dt, x, idx, T, D, E, k, cap, xm, FAKE, FAKE, FAKE, ws, ws_bytes,
                                  FAKE, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), MOE_EINVAL), (dict(x=None), MOE_EINVAL), (dict(xm=FAKE + 4), MOE_EINVAL),
    (dict(idx=FAKE + 2), MOE_EINVAL), (dict(T=0), MOE_ESHAPE), (dict(D=96), MOE_ESHAPE),
    (dict(k=9), MOE_ESHAPE), (dict(E=1025), MOE_ESHAPE), (dict(cap=0), MOE_ECAPACITY),
    (dict(cap=24), MOE_ECAPACITY), (dict(E=1024, k=2, cap=1 << 21), MOE_ECAPACITY),
    (dict(ws_bytes=0), MOE_EWORKSPACE),
])
def test_permute_masked_validation(kw, code):
    assert permute_masked(**kw) == code


def grouped_masked(dt=1, xm=FAKE, counts=FAKE, E=8, D=128, F=256, cap=32, w1=FAKE, h=FAKE,
                   ws=None, ws_bytes=0):
    return lib.moe_grouped_swiglu_masked(dt, xm, counts, E, D, F, cap, w1, FAKE, FAKE, h, FAKE,
                                         ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), MOE_EINVAL), (dict(xm=None), MOE_EINVAL), (dict(counts=None), MOE_EINVAL),
    (dict(w1=FAKE + 8), MOE_EINVAL), (dict(h=None), MOE_EINVAL),
    (dict(ws=FAKE + 4, ws_bytes=1 << 20), MOE_EINVAL), (dict(E=0), MOE_ESHAPE),
    (dict(F=100), MOE_ESHAPE), (dict(D=65536, F=32768), MOE_ESHAPE), (dict(cap=8), MOE_ECAPACITY),
    (dict(cap=40), MOE_ECAPACITY),
])
def test_grouped_masked_validation(kw, code):
    assert grouped_masked(**kw) == code


def test_mxfp8_calls_validate():
    q = lib.moe_quantize_mxfp8
    assert q(5, FAKE, 16, 64, FAKE, FAKE, 0, None) == MOE_EINVAL
    assert q(1, FAKE + 2, 16, 64, FAKE, FAKE, 0, None) == MOE_EINVAL
    assert q(1, FAKE, 16, 64, FAKE, None, 0, None) == MOE_EINVAL
    assert q(1, FAKE, 16, 64, FAKE, FAKE, 2, None) == MOE_EINVAL     # unknown layout
    assert q(1, FAKE, 0, 64, FAKE, FAKE, 0, None) == MOE_ESHAPE
    assert q(1, FAKE, 16, 48, FAKE, FAKE, 0, None) == MOE_ESHAPE
    assert q(1, FAKE, 16, 96, FAKE, FAKE, 1, None) == MOE_ESHAPE     # k-step words: C % 128
    p = lambda **kw: lib.moe_permute_mxfp8(kw.get("xq", FAKE), FAKE, FAKE, kw.get("T", 64),
                                           kw.get("D", 512), 8, 2, kw.get("mt", 128),
                                           kw.get("m_cap", 2048), FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, FAKE, kw.get("ws", 1 << 20), FAKE, None)
    assert p(xq=None) == MOE_EINVAL
    assert p(D=192) == MOE_ESHAPE           # k-step scale words need D % 128 == 0
    assert p(m_cap=100) == MOE_ECAPACITY
    assert p(ws=0) == MOE_EWORKSPACE
    f = lambda **kw: lib.moe_grouped_fc1_swiglu_mxfp8(
        kw.get("xq", FAKE), FAKE, FAKE, None, FAKE, 8, kw.get("D", 512), kw.get("F", 256),
        kw.get("mt", 128), kw.get("m_cap", 1024), FAKE, FAKE, FAKE, FAKE, kw.get("h", FAKE),
        None, 0, None)
    assert f(xq=FAKE + 4) == MOE_EINVAL
    assert f(h=None) == MOE_EINVAL
    assert f(D=192) == MOE_ESHAPE
    assert f(F=100) == MOE_ESHAPE
    assert f(m_cap=1000) == MOE_ECAPACITY
    assert f(mt=64, m_cap=1000) == MOE_ECAPACITY


def test_binding_raises_on_rejected_call():
    with pytest.raises(rpg.MoEError) as ei:
        rpg._binding._check("moe_route", MOE_ESHAPE)
    assert ei.value.status == MOE_ESHAPE


# ---------------------------------------------------------------------------
# Python binding: dtype and buffer-size checks run on the host before any pointer is
# taken (the C ABI cannot see either), so CPU tensors reach them and no GPU is needed.
# ---------------------------------------------------------------------------
import torch  # noqa: E402

BF = torch.bfloat16


def _perm_args(T=64, D=128, k=2):
    return torch.zeros((T, D), dtype=BF), torch.zeros((T, k), dtype=torch.int32)


def test_binding_rejects_int64_topk_idx():
    x, idx = _perm_args()
    with pytest.raises(TypeError, match="topk_idx"):
        rpg.moe_permute(x, idx.to(torch.int64), 8, 16)


def test_binding_rejects_undersized_x_perm():
    x, idx = _perm_args()
    m_cap = rpg.moe_capacity(64, 2, 8, 16)
    with pytest.raises(ValueError, match="x_perm"):
        rpg.moe_permute(x, idx, 8, 16, out={"x_perm": torch.zeros((m_cap - 1, 128), dtype=BF)})
    with pytest.raises(TypeError, match="x_perm"):
        rpg.moe_permute(x, idx, 8, 16, out={"x_perm": torch.zeros((m_cap, 128))})


@pytest.mark.parametrize("name,bad", [("counts", 7), ("offsets", 8), ("src_row", 10),
                                      ("tile_expert", 1), ("dev_err", 0)])
def test_binding_rejects_undersized_metadata(name, bad):
    x, idx = _perm_args()
    with pytest.raises(ValueError, match=name):
        rpg.moe_permute(x, idx, 8, 16, m_cap=640,
                        out={name: torch.zeros(bad, dtype=torch.int32)})


def test_binding_rejects_topk_idx_row_mismatch():
    x, _ = _perm_args()
    with pytest.raises(ValueError, match="topk_idx"):
        rpg.moe_permute(x, torch.zeros((63, 2), dtype=torch.int32), 8, 16)


def _grouped(E=4, F=256, D=128, m_cap=512, dt=BF):
    return (torch.zeros((m_cap, D), dtype=dt), torch.zeros(E + 1, dtype=torch.int32),
            torch.zeros(m_cap // 128, dtype=torch.int32), torch.zeros((E, F, D), dtype=dt),
            torch.zeros((E, F, D), dtype=dt), torch.zeros((E, D, F), dtype=dt))


def test_binding_rejects_weight_dtype_and_shape():
    xp, off, te, w1, w3, w2 = _grouped()
    with pytest.raises(TypeError, match="w3"):
        rpg.moe_grouped_swiglu(xp, off, te, w1, w3.float(), w2, 128)
    with pytest.raises(ValueError, match="w2"):
        rpg.moe_grouped_swiglu(xp, off, te, w1, w3, w2[:, :64], 128)
    with pytest.raises(TypeError, match="offsets"):
        rpg.moe_grouped_swiglu(xp, off.long(), te, w1, w3, w2, 128)


def test_binding_rejects_undersized_gemm_buffers():
    xp, off, te, w1, w3, w2 = _grouped()
    with pytest.raises(ValueError, match="h:"):
        rpg.moe_grouped_swiglu(xp, off, te, w1, w3, w2, 128, h=torch.zeros((511, 256), dtype=BF))
    with pytest.raises(ValueError, match="x_perm"):
        rpg.moe_grouped_fc1_swiglu(xp[:500], off, te, w1, w3, 128, 512,
                                   torch.zeros((512, 256), dtype=BF))
    with pytest.raises(ValueError, match="tile_expert"):
        rpg.moe_grouped_fc2(torch.zeros((512, 256), dtype=BF), off, te[:3], w2, 128, 512,
                            torch.zeros((512, 128), dtype=BF))
    with pytest.raises(ValueError, match="rows_used"):
        rpg.moe_grouped_swiglu(xp, off, te, w1, w3, w2, 128, rows_used=513)


def test_binding_rows_used_admits_a_shorter_read_operand():
    # the shared experts' call: x holds T rows, m_cap is T rounded up to the tile; the
    # check passes and the call stops only at the device check of the CPU tensor
    xp, off, te, w1, w3, w2 = _grouped()
    with pytest.raises(ValueError, match="must live on the GPU"):
        rpg.moe_grouped_swiglu(xp[:500], off, te, w1, w3, w2, 128, m_cap=512, rows_used=500)
    with pytest.raises(ValueError, match="x_perm"):
        rpg.moe_grouped_swiglu(xp[:500], off, te, w1, w3, w2, 128, m_cap=512)


def test_binding_rejects_combine_dtypes_and_sizes():
    y = torch.zeros((640, 128), dtype=BF)
    dst = torch.zeros((64, 2), dtype=torch.int32)
    w = torch.zeros((64, 2))
    with pytest.raises(TypeError, match="dst_row"):
        rpg.moe_combine(y, dst.long(), w)
    with pytest.raises(TypeError, match="topk_w"):
        rpg.moe_combine(y, dst, w.double())
    with pytest.raises(ValueError, match="out"):
        rpg.moe_combine(y, dst, w, out=torch.zeros((63, 128), dtype=BF))
    with pytest.raises(TypeError, match="shared"):
        rpg.moe_combine(y, dst, w, shared=torch.zeros((64, 128)))


def test_binding_rejects_route_buffers():
    x = torch.zeros((64, 128), dtype=BF)
    wg = torch.zeros((8, 128), dtype=BF)
    with pytest.raises(TypeError, match="wg"):
        rpg.moe_route(x, wg.float(), 2)
    with pytest.raises(TypeError, match="topk_idx"):
        rpg.moe_route(x, wg, 2, topk_idx=torch.zeros((64, 2), dtype=torch.int64))
    with pytest.raises(ValueError, match="topk_w"):
        rpg.moe_route(x, wg, 2, topk_w=torch.zeros((64, 1)))
    with pytest.raises(TypeError, match="bias"):
        rpg.moe_route(x, wg, 2, bias=torch.zeros(8, dtype=torch.float64))


def test_binding_rejects_wgrad_and_mx_buffers():
    P_ = torch.zeros((512, 320), dtype=BF)
    Q_ = torch.zeros((512, 192), dtype=BF)
    off = torch.zeros(5, dtype=torch.int32)
    with pytest.raises(ValueError, match="out_lo"):
        rpg.moe_grouped_wgrad(P_, Q_, off, 128, NS=192, out_lo=torch.zeros((4, 191, 192)))
    with pytest.raises(TypeError, match="Q:"):
        rpg.moe_grouped_wgrad(P_, Q_.float(), off, 128)
    xq = torch.zeros((64, 256), dtype=torch.uint8)
    with pytest.raises(ValueError, match="xs"):
        rpg.moe_permute_mxfp8(xq, torch.zeros((64, 7), dtype=torch.uint8),
                              torch.zeros((64, 2), dtype=torch.int32), 8, 128)


def permute_noalloc(dt=1, x=FAKE, idx=FAKE, T=64, D=128, E=8, k=2, mt=16, m_cap=None, xp=FAKE):
    if m_cap is None:
        m_cap = rpg.moe_capacity(T, k, E, mt)
    return lib.moe_permute_noalloc(dt, x, idx, T, D, E, k, mt, m_cap, xp, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, None)


MOE_ESCRATCH = 7


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), MOE_EINVAL), (dict(x=None), MOE_EINVAL), (dict(xp=FAKE + 4), MOE_EINVAL),
    (dict(T=0), MOE_ESHAPE), (dict(E=1025), MOE_ESHAPE), (dict(mt=100), MOE_ESHAPE),
    (dict(m_cap=16), MOE_ECAPACITY),
    # ceil(T/256) * (E+1) * 4 bytes above the 1 MiB static scratch
    (dict(T=65537, E=1023, k=1), MOE_ESCRATCH), (dict(T=1 << 23, E=8, k=1), MOE_ESCRATCH),
])
def test_permute_noalloc_validation(kw, code):
    assert permute_noalloc(**kw) == code


def test_permute_noalloc_scratch_limit_matches_the_workspace_formula():
    # the largest inputs the static scratch serves are rejected by neither check;
    # validation stops there only at the (FAKE) buffers, which are never touched
    assert rpg.moe_permute_workspace_bytes(65536, 1, 1023) == 1 << 20
    assert rpg.moe_permute_workspace_bytes(65537, 1, 1023) > 1 << 20
    assert "1 MiB" in rpg.moe_status_str(MOE_ESCRATCH)
