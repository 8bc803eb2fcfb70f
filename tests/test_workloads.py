"""The seeded workload generator (CPU only)."""
import numpy as np
import pytest

from varlen_depthwise_causal_amd import workloads as W


@pytest.mark.parametrize("name", sorted(W.SPECS))
def test_documents(name):
    spec = W.SPECS[name]
    assert spec.C % 8 == 0
    lengths = W.doc_lengths(spec, W._streams(spec.seed)["docs"])
    cu = W.cu_from_lengths(lengths)
    assert cu[0] == 0 and cu[-1] == spec.S and np.all(np.diff(cu) >= 0)
    assert cu.dtype == np.int32
    if spec.docs[0] == "lognormal":
        lo, hi = spec.docs[3], spec.docs[4]
        assert min(lengths) >= lo and max(lengths[:-1]) <= hi and lengths[-1] >= 1
    if spec.docs[0] == "randint":
        assert len(lengths) == spec.docs[1] + 1
        assert max(lengths[:-1]) <= spec.docs[3] and min(lengths) >= 0
        assert any(v == 0 for v in lengths)          # empty documents are present


def test_tiny_exact():
    wl = W.make("tiny")
    assert list(wl.cu) == [0, 0, 1, 3, 6, 11, 28, 278, 1000]
    assert wl.x.shape == (1000, 64) and wl.x.dtype == np.uint16
    assert wl.w.shape == (64, 4) and wl.w.dtype == np.float32 and wl.w_dtype == "f32"
    assert wl.b.shape == (64,) and wl.b_dtype == "f32"
    assert np.all(np.abs(wl.w) <= 0.5)
    again = W.make("tiny")
    for k in ("x", "dy", "w", "b", "cu"):
        assert np.array_equal(getattr(wl, k), getattr(again, k)), k


def test_bf16_rounding_of_inputs():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.0e-39], np.float32)
    bits = W.f32_to_bf16_bits(f)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0021]


def test_stress_saturation():
    spec = W.SPECS["stress"]
    small = W.Spec("stress-small", spec.seed, 8192, spec.C, ("fixed", (8192,)), spec.w, spec.b,
                   spec.policies, spec.sat)
    wl = W.make(small)
    sixty = W.f32_to_bf16_bits(np.array([60.0, -60.0], np.float32))
    hit = (wl.x == sixty[0]) | (wl.x == sixty[1])
    frac = hit.mean()
    assert 0.009 < frac < 0.011
    assert 0.4 < (wl.x == sixty[0]).sum() / hit.sum() < 0.6


def test_param_dtypes():
    wl = W.make(W.Spec("p", 5, 16, 16, ("single",), ("bf16", "U", 0.5), ("bf16", "N", 0.1), ("bf16",)))
    assert wl.w.dtype == np.uint16 and wl.w_dtype == "bf16"
    assert wl.b.dtype == np.uint16 and wl.b_dtype == "bf16"
