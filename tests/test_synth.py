"""The seeded input generator: determinism, recipe properties and the margin audit."""

import hashlib
import json
import math
import os

import numpy as np
import pytest

from synth import CONFIGS, generate, generate_head, load_repairs
from synth.configs import Spec
from synth.generate import f32_to_bf16_bits
from synth.record_hashes import PATH as HASHES, digest

from oracle import margin, sla
from oracle.make_repairs import boundaries_for


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x7F62]


def test_generation_is_deterministic_and_matches_recorded_hashes():
    with open(HASHES) as f:
        want = json.load(f)
    for name in ("tiny", "short_video"):
        a = generate(CONFIGS[name])
        b = generate(CONFIGS[name], threads=1)
        for t in "qkv":
            np.testing.assert_array_equal(a[t], b[t])
            assert digest(a[t]) == want[name][t]


def test_large_workload_head_hashes():
    with open(HASHES) as f:
        want = json.load(f)
    spec = CONFIGS["wan14b"]
    part = generate_head(spec, 0, 0, repairs=load_repairs(spec.cfg_id))
    for t in "qkv":
        assert digest(part[t]) == want["wan14b/head0"][t]


def test_fourier_fields_have_locality_and_unit_scale():
    spec = CONFIGS["short_video"]
    part = generate_head(spec, 0, 3, repairs=None)
    q = sla.bf16_to_f64(part["q"])
    k = sla.bf16_to_f64(part["k"])
    v = sla.bf16_to_f64(part["v"])
    assert 0.7 < q.var() < 1.5 and 0.7 < v.var() < 1.5
    # Q and K share their field: neighbouring tokens and Q/K at one token correlate
    assert np.corrcoef(q[:-1].ravel(), q[1:].ravel())[0, 1] > 0.8
    assert np.corrcoef(q.ravel(), k.ravel())[0, 1] > 0.8
    assert abs(np.corrcoef(q.ravel(), v.ravel())[0, 1]) < 0.2


def test_repair_touches_only_its_query_block():
    spec = CONFIGS["wan1p3b"]
    base = generate_head(spec, 0, 1, repairs={})
    rep = generate_head(spec, 0, 1, repairs={(0, 1, 5): 2})
    diff = np.nonzero((base["q"] != rep["q"]).any(axis=1))[0]
    assert diff.min() >= 5 * spec.block and diff.max() < 6 * spec.block and len(diff) > 100
    np.testing.assert_array_equal(base["k"], rep["k"])
    np.testing.assert_array_equal(base["v"], rep["v"])


def _audit(spec_names, heads):
    specs = [CONFIGS[n] for n in spec_names]
    spec = specs[0]
    cuts, thr = boundaries_for(specs, spec.nb)
    rep = load_repairs(spec.cfg_id)
    for h in heads:
        part = generate_head(spec, 0, h, ("q", "k"), rep)
        q, k = sla.bf16_to_f64(part["q"]), sla.bf16_to_f64(part["k"])
        s = sla.pooled_scores(sla.pool(q, spec.block), sla.pool(k, spec.block), 1 / math.sqrt(spec.d))
        assert margin.failing_rows(s, cuts, thr) == [], (spec.name, h)


@pytest.mark.parametrize("names,heads", [
    (("tiny",), range(2)), (("short_video",), range(12)), (("wan1p3b",), range(12)),
    (("wan14b",), (0, 39)), (("long_clip_95", "long_clip_90"), (0,)),
])
def test_margin_holds_with_stored_repairs(names, heads):
    _audit(names, heads)


def test_margin_audit_detects_a_near_tie():
    s = np.array([1.0, 0.5, 0.49995, 0.0])
    assert not margin.row_ok(s, [2])
    assert margin.row_ok(s, [1])
    assert margin.row_ok(s, [3])


def test_spec_validation():
    with pytest.raises(ValueError):
        Spec(9, "bad", B=1, H=1, N=10, d=64, block=64, kind="fourier", grid=(1, 2, 3))
    with pytest.raises(ValueError):
        Spec(9, "bad", B=1, H=1, N=10, d=64, block=64, kind="iid", mode="nope")
