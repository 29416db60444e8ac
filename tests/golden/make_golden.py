"""Writes the stored expected values under tests/golden/ (calls only the oracle).

swish_example.json: the worked example of the SwishGrad page ("CANN ops-nn 中 SwishGrad
算子解析", section 4.1, the runnable aclnnSwishBackward sample): shape {2, 3}, gradOutput
all ones, self = 1..6, beta = 1.1 (float32).  The page says the six printed outputs can be
checked by hand against the formula of section 1.2 but does not print them; the expected
values stored here are the oracle's.  The oracle test re-derives them independently at 40
digits.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle.ref import swish_grad_ref  # noqa: E402


def main():
    grad = [1.0] * 6
    x = [1.0, 2.0, 3.0, 4.0, 5.0, 6.0]
    beta = 1.1
    exp = swish_grad_ref(np.array(grad), np.array(x), beta).tolist()
    doc = {
        "source": "SwishGrad page (ops-nn), section 4.1 runnable sample; shape {2,3}",
        "shape": [2, 3], "grad": grad, "x": x, "beta": beta,
        "beta_float32": float(np.float32(beta)),
        "expected": exp,
        "expected_by": "oracle.ref.swish_grad_ref (float64)",
    }
    with open(os.path.join(HERE, "swish_example.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
