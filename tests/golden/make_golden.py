"""Writes tests/golden/synthetic_sha256.json: SHA-256 digests of the first 64 Ki
elements of each seeded tensor of every workload. Calls only the ``synthetic``
generator. Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import synthetic  # noqa: E402

N = 65536


def digests():
    out = {}
    for name in ("tiny_f32", "decode", "int8", "skew"):
        T, d, f, E, k, act, wdt, skew = synthetic.WORKLOADS[name]
        w = synthetic.make(name, T=min(T, 16), f=min(f, 64) if name != "tiny_f32" else f)
        for key in ("x", "router_w", "w_gate", "w_up", "w_down"):
            a = getattr(w, key).ravel()[:N]
            out[f"{name}/{key}"] = hashlib.sha256(a.tobytes()).hexdigest()
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synthetic_sha256.json")
    json.dump({"note": "first 64Ki elements of each tensor; workloads shrunk to T<=16, f<=64 (tiny_f32 full)",
               "digests": digests()}, open(path, "w"), indent=1, sort_keys=True)
    print("wrote", path)
