"""CPU checks of the decode-attention tolerance in tests/harness.py.

mla_rel_bound is a first-order rounding bound c (a multiple of S = sum_t p_t
|v_t| / sum_t p_t).  Most of its terms come from the operation itself (the
scores' dot products, exp2, the weighted value sums, the division).  Two
come from the matrix-core kernel's arithmetic: each weight entering the
value product as two bf16 parts (2^-18 relative, twice) and one rescaling
per 32-token block and per merged wave ((L/32 + 8) u).  These tests pin
that c stays under a stated ceiling on the workloads' inputs, and that the
kernel-specific terms are a small part of it, so a change in the kernel
cannot quietly widen the bound that checks it.
"""
import math

import numpy as np
import pytest

from invariant_deterministic_bi_amd import inputs
from harness import mla_rel_bound

CEILING = 5e-3          # stated ceiling of c for N(0,1) inputs, Dqk <= 576, L <= 16384
U = 2.0 ** -24


def _kernel_terms(L):
    return 2 * 2.0 ** -18 + (L / 32 + 8) * U


@pytest.mark.parametrize("Dqk,L", [(576, 1), (576, 1024), (576, 4096), (576, 16384), (128, 4096), (64, 260)])
def test_mla_bound_below_ceiling(Dqk, L):
    H = 16
    q = inputs.randn_bf16((1, H, Dqk), 1.0, tag=(590, Dqk, L))
    kv = inputs.randn_bf16((1, L, Dqk), 1.0, tag=(591, Dqk, L))
    c = mla_rel_bound(q, kv, [L], 1.0 / math.sqrt(192.0))
    assert c.max() <= CEILING, c.max()
    assert c.min() >= 1e-3
    # the kernel-specific terms are under 3% of the bound whenever it exceeds the 1e-3 floor
    raw = c.max() / 1.01
    if raw > 1e-3:
        assert _kernel_terms(L) <= 0.03 * raw, (_kernel_terms(L), raw)


def test_mla_bound_grows_with_the_operation_not_the_kernel():
    """Doubling the scores (scale x2) raises c through the dot-product and
    exp2 terms alone; the kernel-specific part does not depend on scale."""
    q = inputs.randn_bf16((1, 4, 576), 1.0, tag=(592,))
    kv = inputs.randn_bf16((1, 2048, 576), 1.0, tag=(593,))
    c1 = mla_rel_bound(q, kv, [2048], 0.05).max() / 1.01
    c2 = mla_rel_bound(q, kv, [2048], 0.10).max() / 1.01
    fixed = (1.25 * 2048 + 11) * U + U + _kernel_terms(2048) + 2 * 2 * U
    assert c2 - fixed == pytest.approx(2 * (c1 - fixed), rel=1e-9)
