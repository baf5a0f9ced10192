"""Writes tests/golden/tiny_oracle.npz: the oracle's output on the seeded tiny workload.

Calls only the oracle (and the seeded input generator).  The fixture pins the oracle
against silent drift: the pages print no numeric example for this step, so this file
is a regression record, not an external pin (the external pins are in
tests/test_oracle_*.py).  Re-run after a deliberate, justified oracle change:
    python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from prefill_token_amd import inputs  # noqa: E402


def input_digest(inp):
    h = hashlib.sha256()
    for k in ("q", "kv_pool", "indices", "topk_length", "positions", "norm_w"):
        h.update(np.ascontiguousarray(inp[k]).tobytes())
    return h.hexdigest()


def main():
    inp = inputs.make("tiny")
    o, codes, scales = oracle.sparse_mla(
        inp["q"], inp["kv_pool"], inp["kv_scales"], inp["indices"], inp["topk_length"], inp["positions"],
        inp["norm_w"], sm_scale=inp["sm_scale"], eps=inp["eps"], theta=inp["theta"],
        rope_dim=inp["rope_dim"], kv_format=inp["kv_format"])
    np.savez_compressed(os.path.join(HERE, "tiny_oracle.npz"), o=o, codes=codes, scales=scales,
                        digest=np.array(input_digest(inp)))


if __name__ == "__main__":
    main()
