"""The precision budget of the projection weight's bf16 split, computed with the
oracle alone (no GPU): the library multiplies the bf16 residual by fn split into
bf16 terms on the matrix cores, and this test measures, in double precision, what
the split by itself does to the gates at the hidden sizes of the pages' workloads.

  * one term (hi = bf16(f)): the gates miss the 1e-4 bar by two orders;
  * two terms (hi + lo, the library's): inside the bar, with a margin of about
    4e-5 at C = 5120 and 6e-5 at C = 16384;
  * three terms: float32 exactly, so no further term could help.
"""
import numpy as np
import pytest

import mhc_inputs as mi
import oracle

GATE_BAR = 1e-4


def _split(f, terms):
    out = np.zeros(f.shape, dtype=np.float64)
    r = f.astype(np.float64)
    for _ in range(terms):
        b = oracle.bf16_to_f64(oracle.bf16_rne(r))
        out += b
        r = r - b
    return out


def _gate_err(d, terms):
    x = d["x"].reshape(d["x"].shape[0], -1)
    lg_e, _ = oracle.logits(x, d["fn"], d["bias"], d["alpha"], d["eps"])
    lg, _ = oracle.logits(x, _split(d["fn"], terms), d["bias"], d["alpha"], d["eps"])
    ge, g = oracle.gates(lg_e, d["iters"]), oracle.gates(lg, d["iters"])
    return max(float(np.max(np.abs(a - b) / np.abs(b))) for a, b in zip(g, ge))


@pytest.mark.parametrize("C,T,lo,hi", [(5120, 64, 2e-5, 7e-5), (16384, 32, 3e-5, 9e-5)])
def test_weight_split_error_budget(C, T, lo, hi):
    d = mi.pre_inputs(T, seed=2, C=C, delayed=True, norm=True, outlier_frac=0.05)
    assert _gate_err(d, 1) > 10 * GATE_BAR
    e2 = _gate_err(d, 2)
    assert lo < e2 < hi < GATE_BAR
    assert np.array_equal(_split(d["fn"], 3), d["fn"].astype(np.float64))
    assert _gate_err(d, 3) == 0.0
