"""Writes oracle_digests.json: SHA-256 digests of the CPU oracle's outputs on small seeded
workloads.  Calls only the oracle and the input generator.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    out = {}
    for name, wl_name, q_dt, k_dt in (("tiny_f32_f16", "tiny", "f32", "f16"),
                                      ("tiny_bf16_f32", "tiny", "bf16", "f32")):
        wl = synth.workloads()[wl_name]
        sp = oracle.spec_from_workload(wl)
        x = synth.qkv_host(wl)
        wq, wk = synth.norm_weights(wl)
        q, k, v = oracle.qk_rmsnorm_rope_permute(sp, x, wl.in_dtype, wq, wk, q_dt, k_dt)
        out[name] = {
            "workload": wl_name, "q_dt": q_dt, "k_dt": k_dt,
            "input_sha256": hashlib.sha256(x.tobytes()).hexdigest(),
            "q_sha256": hashlib.sha256(np.ascontiguousarray(q).tobytes()).hexdigest(),
            "k_sha256": hashlib.sha256(np.ascontiguousarray(k).tobytes()).hexdigest(),
            "v_sha256": hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest(),
        }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digests.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
