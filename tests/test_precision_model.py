"""Rounding model of the prefill kernels' MFMA operands (CPU, numpy).

The chunk form is run in fp64 with every MFMA operand rounded as the kernels round it (single f16 or
hi/lo pair, at its power-of-two scale, MFMA's subnormal flush included), on the seeded inputs of the
4096-token prefill (16 heads of 128, zero start state) and of the stacked prefill (32 value heads on 16
key heads, saved start states), cut to 2048 tokens and 4 value heads so that it runs in seconds. The
layer's bounds are 2e-3 on outputs and 1e-3 of max |H| on final states. Gated DeltaNet (Yang, Kautz,
Hatamizadeh), section 3.3 on the chunkwise form, fixes the algebra; the operand choices are the kernels'.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

from gdn_inputs import NEXT, SMALL
from tests import bruteforce as bf
from tests import precision_model as pm

OUT_BOUND, STATE_BOUND = 2e-3, 1e-3
SHAPES = {"prefill_4k": (SMALL, 0.0), "stack": (NEXT, 0.05)}


@functools.lru_cache(maxsize=None)
def _case(name):
    dims, h0 = SHAPES[name]
    inp = pm.layer_inputs(1, dims, 2048, 4, h0)
    return inp, {form: pm.run(inp, pm.all_exact(form)) for form in ("fused", "two_phase")}


@pytest.fixture(params=sorted(SHAPES))
def shape(request):
    return (request.param, *_case(request.param))


@pytest.fixture
def small():
    return _case("prefill_4k")


def test_rounding_primitives():
    assert pm.f16(2.0 ** -15) == 0.0 and pm.f16(-(2.0 ** -20)) == 0.0  # subnormals flushed
    assert pm.f16(2.0 ** -14) == 2.0 ** -14
    assert pm.f16(1 + 2.0 ** -11) == 1.0 and pm.f16(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9  # ties to even
    with np.errstate(over="ignore"):
        assert pm.f16(70000.0) == np.inf
    x = np.random.default_rng(0).uniform(-1.0, 1.0, 10000)
    x = x[np.abs(x) > 2.0 ** -6]
    # hi: half an f16 ulp; hi/lo: about 22 bits, but a lo half below 2^-14 flushes, so the pair's error
    # has an absolute floor of 2^-14 / scale
    assert (np.abs(pm.operand(x, "h", 256.0) - x) <= 2.0 ** -11 * np.abs(x)).all()
    err = np.abs(pm.operand(x, "s", 256.0) - x)
    assert (err <= 2.0 ** -21 * np.abs(x) + 2.0 ** -14 / 256.0).all()
    assert (err > 2.0 ** -21 * np.abs(x)).any()  # the floor is reached
    assert np.array_equal(pm.operand(x, "x", 256.0), x)
    # a small entry's lo half falls below 2^-14 without a scale: the pair is then no better than hi
    tiny = np.array([1e-3 + 1e-7])
    assert pm.operand(tiny, "s", 1.0)[0] == pm.operand(tiny, "h", 1.0)[0]
    assert abs(pm.operand(tiny, "s", 256.0)[0] - tiny[0]) < 1e-10


@pytest.mark.parametrize("form", ["fused", "two_phase"])
def test_exact_operands_give_the_closed_form(form):
    """With no operand rounded, both arrangements are the whole-sequence closed form (ragged last chunk,
    ragged last 16-token block)."""
    rng = np.random.default_rng(5)
    L, dk, dv = 203, 32, 24
    q = bf.l2n(rng.standard_normal((L, dk)), 1e-6)
    k = bf.l2n(rng.standard_normal((L, dk)), 1e-6)
    v = rng.standard_normal((L, dv))
    g = -rng.uniform(0.0, 0.3, L)
    beta = rng.uniform(0.05, 1.0, L)
    H0 = rng.standard_normal((dk, dv)) * 0.3
    O, H = pm.head(q, k, v, g, beta, H0, dk ** -0.5, pm.all_exact(form))
    O_ref, H_ref = bf.dense_delta_rule_head(q, k, v, g, beta, H0, dk ** -0.5)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(H, H_ref, rtol=0, atol=1e-10)


def test_chosen_operands_have_margin(shape):
    """The kernels' operand choices spend at most a quarter of the output bound and a twentieth of the
    state bound."""
    name, inp, refs = shape
    for form, cfg, scales in (("fused", pm.FUSED, pm.SCALES), ("two_phase", pm.TWO_PHASE, pm.TWO_PHASE_SCALES)):
        eo, es = pm.errors(refs[form], pm.run(inp, cfg, scales))
        assert eo < 0.25 * OUT_BOUND, (name, form, eo)
        assert es < 0.05 * STATE_BOUND, (name, form, es)


@pytest.mark.parametrize("op", ["U", "Z", "P", "gram"])
def test_single_f16_where_pairs_are_needed(small, op):
    """A single f16 in place of the pair for U, the solve's right-hand sides, P or the Gram operands
    breaks the output bound."""
    inp, refs = small
    eo, _ = pm.errors(refs["fused"], pm.run(inp, dict(pm.FUSED, **{op: "h"})))
    assert eo > OUT_BOUND, (op, eo)


def test_scales_keep_low_halves(small):
    """P at 2^8 flushes the low halves of its small entries (its decays span decades), and so do the
    two-phase record's Q~ and P~ at 2^8 and an unscaled -W: each at least triples the error."""
    inp, refs = small
    base_f, _ = pm.errors(refs["fused"], pm.run(inp, pm.FUSED))
    p8, _ = pm.errors(refs["fused"], pm.run(inp, pm.FUSED, dict(pm.SCALES, P=256.0)))
    assert p8 > 3 * base_f, (p8, base_f)
    base_t, _ = pm.errors(refs["two_phase"], pm.run(inp, pm.TWO_PHASE, pm.TWO_PHASE_SCALES))
    old = dict(pm.TWO_PHASE_SCALES, P=256.0, Q=256.0, W=1.0)
    old_t, _ = pm.errors(refs["two_phase"], pm.run(inp, pm.TWO_PHASE, old))
    assert old_t > 3 * base_t and old_t > 0.4 * OUT_BOUND, (old_t, base_t)


@pytest.mark.parametrize("form,op", [("fused", "kh"), ("fused", "A"), ("two_phase", "X"), ("two_phase", "W"),
                                     ("two_phase", "T")])
def test_dropped_low_halves(small, form, op):
    """The operands kept as a single f16 (K in K H and the off-diagonal -A blocks in the fused kernel;
    beta e^gamma K, -W and T in the two-phase record) would buy back less than a tenth of the output
    bound with their low halves."""
    inp, refs = small
    cfg, scales = (pm.FUSED, pm.SCALES) if form == "fused" else (pm.TWO_PHASE, pm.TWO_PHASE_SCALES)
    assert cfg[op] == "h"
    single, _ = pm.errors(refs[form], pm.run(inp, cfg, scales))
    pair, _ = pm.errors(refs[form], pm.run(inp, dict(cfg, **{op: "s"}), scales))
    assert single - pair < 0.1 * OUT_BOUND, (form, op, single, pair)
