"""Write tests/golden/oracle_regression.json by calling only the oracle.

Run from the repository root:  python tests/golden/make_golden.py
The fixture guards against unintended drift of the oracle's arithmetic; a
deliberate change must regenerate it and say why in the commit message.
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, HERE)

import oracle                      # noqa: E402
import regression_inputs           # noqa: E402


def main():
    fixture = {"_about": "Expected oracle outputs for the formula-defined "
                         "inputs in regression_inputs.py; written by "
                         "make_golden.py from the oracle alone."}
    for dtype in ("bf16", "fp8_e4m3fn"):
        c = regression_inputs.case(dtype)
        r = oracle.sparse_mla_decode(**c)
        fixture[dtype] = {
            "lse": r["lse"].tolist(),
            "out_head8": r["out"][:, :, :8].tolist(),
            "out_sum": r["out"].sum(-1).tolist(),
            "out_sumsq": (r["out"] ** 2).sum(-1).tolist(),
            "n_active": r["n_active"].tolist(),
        }
    path = os.path.join(HERE, "oracle_regression.json")
    with open(path, "w") as f:
        json.dump(fixture, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
