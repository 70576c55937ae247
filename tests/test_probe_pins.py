"""The exact-gather probe (tests/probes.py) pins the oracle's indexing: on
every form pair and causal kind the oracle's output row is the picked V row
to fp64 precision (the other keys weigh e^-64), and rows with no allowed key
are zeros.  The same probe checks the GPU bit for bit."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from tests import probes

FORMS = ["padded_bhnd", "packed_nhd"]


@pytest.mark.parametrize("qf,kf", list(itertools.product(FORMS, FORMS)))
@pytest.mark.parametrize("causal", ["none", "upper_left", "lower_right"])
def test_oracle_gathers_the_picked_row(qf, kf, causal):
    c, expect, ks = probes.gather_probe(11 + FORMS.index(qf) * 6 + FORMS.index(kf) * 3 +
                                        ["none", "upper_left", "lower_right"].index(causal),
                                        qf, kf, causal, torch.float16)
    res = oracle.attention(c.q, c.k, c.v, None, **c.kwargs())
    v = c.v.double()
    empty = 0
    for r, (b, h, i) in enumerate(res.rows.tolist()):
        tgt = expect[(b, h, i)]
        if tgt is None:
            assert np.all(res.out[r] == 0.0), (b, h, i)
            empty += 1
            continue
        g, t = tgt
        want = (v[int(ks[b]) + t, g] if kf == "packed_nhd" else v[b, g, t]).numpy()
        np.testing.assert_allclose(res.out[r], want, rtol=1e-12, atol=0)
    assert len(res.rows) == len(expect)
    if causal == "lower_right":
        assert empty > 0  # some sequences have kv_len < q_len
