"""The seeded input generator: determinism, shapes, the draw recipe and its
single float32 -> bf16 rounding (checked against torch's own conversion)."""

import numpy as np
import pytest

from synthetic import (WORKLOADS, f32_to_bf16_bits, integer_scaled_inputs, make_inputs,
                       special_rows_inputs)


def test_f32_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.3895314e38], np.float32)])
    a = a.astype(np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(a), want)


def test_workload_table():
    assert [w.index for w in WORKLOADS.values()] == [0, 1, 2, 3, 4]
    h = WORKLOADS["llama70b"]
    assert (h.num_tokens, h.hidden, h.num_partials, h.dtype) == (1024, 8192, 8, "bf16")
    assert h.algorithmic_bytes() == 184_549_376
    assert WORKLOADS["tiny"].algorithmic_bytes() == 655_360
    for name in ("qwen72b", "mixtral", "llama405b"):
        assert WORKLOADS[name].algorithmic_bytes() == 738_197_504
    assert WORKLOADS["qwen72b"].eps == 1e-6


def test_make_inputs_deterministic_and_shaped():
    a = make_inputs("tiny")
    b = make_inputs("tiny")
    assert a["partials"].shape == (2, 64, 512) and a["partials"].dtype == np.float32
    assert a["residual"].shape == (64, 512) and a["weight"].shape == (512,)
    for k in ("partials", "residual", "weight"):
        np.testing.assert_array_equal(a[k], b[k])
    c = make_inputs("llama70b", num_tokens=8, hidden=256)
    assert c["partials"].dtype == np.uint16 and c["partials"].shape == (8, 8, 256)
    # the draw recipe: partials ~N(0, 0.5) -> std close to 0.5
    wide = (c["partials"].astype(np.uint32) << 16).view(np.float32)
    assert 0.45 < wide.std() < 0.55


def test_mixtral_outliers():
    d = make_inputs("mixtral", num_tokens=8192, hidden=16)
    rows = d["outlier_rows"]
    assert rows.size == 82 and np.unique(rows).size == 82
    p = (d["partials"].astype(np.uint32) << 16).view(np.float32)
    big = np.abs(p[:, rows]).mean()
    small = np.abs(np.delete(p, rows, axis=1)).mean()
    assert 60 < big / small < 140


def test_special_inputs_exact():
    d = integer_scaled_inputs(3, 4, 32, "bf16", kmax=64)
    v = (d["partials"].astype(np.uint32) << 16).view(np.float32)
    assert np.all(v * 16 == np.round(v * 16)) and np.abs(v).max() <= 4
    s = special_rows_inputs(2, 11, 16, "f32")
    assert set(s["kind"].tolist()) == {0, 1, 2}
