"""Golden fixtures for the oracle (CPU only).

* ``golden/pages_constants.json`` - interface constants the pages print,
  each with its citation; the oracle's column split must agree with them.
* ``golden/oracle_regression.json`` - expected values written by
  ``golden/make_golden.py`` from the oracle alone, for formula-defined
  inputs; a drift in the oracle's arithmetic fails here.
"""

import json
import os
import sys

import numpy as np
import pytest

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, HERE)
import regression_inputs  # noqa: E402


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_pages_constants_agree_with_oracle():
    c = load("pages_constants.json")
    assert oracle.SWA_COLUMNS == c["swa_columns"]["value"]
    assert c["nope_dim"]["value"] + c["rope_dim"]["value"] == \
        c["head_dim"]["value"]
    assert all("cite" in v for k, v in c.items() if not k.startswith("_"))


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3fn"])
def test_oracle_regression_fixture(dtype):
    want = load("oracle_regression.json")[dtype]
    r = oracle.sparse_mla_decode(**regression_inputs.case(dtype))
    np.testing.assert_allclose(r["lse"], want["lse"], rtol=1e-13)
    np.testing.assert_allclose(r["out"][:, :, :8], want["out_head8"],
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["out"].sum(-1), want["out_sum"], rtol=1e-11,
                               atol=1e-14)
    np.testing.assert_allclose((r["out"] ** 2).sum(-1), want["out_sumsq"],
                               rtol=1e-12)
    assert r["n_active"].tolist() == want["n_active"]
