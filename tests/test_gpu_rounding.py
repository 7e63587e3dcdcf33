"""The library's float32 -> bf16 rounding, bit for bit against the oracle's.

Every bf16 value the library stores (h, y_perm, the shared output, out, and the
backward's bf16 gradients) goes through one conversion; ``moe_round_bf16`` exposes it.
The patterns cover every upper half-word (sign, exponent and the 7 mantissa bits bf16
keeps) with 16 lower half-words, among them the exact ties 0x8000 and their
neighbours, so ties to even, subnormals, the largest finite values (which round to
infinity past the last tie) and zeros of both signs are all met.
"""
import numpy as np
import pytest
import torch

import routing_permute_grouped_amd as rpg
from oracle import moe_oracle as orc
from tests import _parity as P

pytestmark = pytest.mark.gpu

_LOW = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000, 0x7FFE,
                 0x8002, 0x1234, 0xFEDC, 0x0F0F, 0xF0F0, 0x5555, 0xAAAA], dtype=np.uint32)


def _patterns() -> np.ndarray:
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    return (hi[:, None] | _LOW[None, :]).reshape(-1)


def _oracle_bits(u: np.ndarray) -> np.ndarray:
    """bf16 bits of the oracle's rounding of finite float32 values (float64 arithmetic)."""
    r = orc.round_bf16(u.view(np.float32).astype(np.float64))
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)          # exact for bf16 values; 2^128 becomes inf
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def test_round_bf16_matches_the_oracle_bit_for_bit():
    P.log("[parity] float32 -> bf16 rounding on 2^20 patterns")
    u = _patterns()
    x = torch.from_numpy(u.view(np.float32).copy()).cuda()
    y = rpg.moe_round_bf16(x)
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    mag = u & np.uint32(0x7FFFFFFF)
    finite = mag < np.uint32(0x7F800000)
    np.testing.assert_array_equal(got[finite], _oracle_bits(u[finite]))
    # infinities keep their sign; a NaN stays a NaN
    inf = mag == np.uint32(0x7F800000)
    np.testing.assert_array_equal(got[inf], (u[inf] >> np.uint32(16)).astype(np.uint16))
    nan = mag > np.uint32(0x7F800000)
    assert np.all((got[nan] & 0x7FFF) > 0x7F80)


def test_round_bf16_of_nothing_and_of_one_value():
    P.log("[parity] rounding: n = 0 and n = 1")
    empty = torch.empty(0, dtype=torch.float32, device="cuda")
    assert rpg.moe_round_bf16(empty).numel() == 0
    one = torch.tensor([1.0 + 2.0 ** -8], dtype=torch.float32, device="cuda")   # a tie
    assert rpg.moe_round_bf16(one).float().item() == 1.0                          # to even
