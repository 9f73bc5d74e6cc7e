"""Writes tiny_oracle.json: the oracle's float64 outputs on the seeded "tiny" workload.

A regression fixture: it calls only oracle/ and the seeded input generator, so a later
change to the oracle's arithmetic shows up as a diff against this file. Run from the
repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from linear_attention_decode_kda_amd import synth  # noqa: E402


def main():
    w = synth.WORKLOADS["tiny"]
    out = oracle.verify_workload(w, synth.make_inputs(w))
    doc = {
        "what": "oracle outputs for the seeded tiny workload (N=2, T=2, H=HV=2, K=V=16, fp32, softplus gate)",
        "written_by": "tests/golden/make_golden.py (oracle/ + synth only)",
        "o": out["o"].reshape(-1).tolist(),
        "inter_ssm_sum_by_nt": out["inter_ssm"].sum(axis=(2, 3, 4)).reshape(-1).tolist(),
        "inter_ssm_first_row": out["inter_ssm"][:, :, :, 0, :].reshape(-1).tolist(),
        "conv_state": out["conv_state"].reshape(-1).tolist(),
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
