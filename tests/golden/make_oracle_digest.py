"""Writes oracle_digest.json: SHA-256 digests and a few sampled values of the
oracle's outputs and states on small seeded cases. Calls only ``oracle/`` and
``synthetic``; rerun it only with a commit that names the passage justifying
an oracle change.  Usage: python tests/golden/make_oracle_digest.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthetic  # noqa: E402


def cases():
    yield "single_seq_64ch_f32", synthetic.single_seq_64ch()
    yield "ple_mixed_small", synthetic.ple_mixed_batch(C=64, num_decodes=8, Bp=3, min_len=5,
                                          max_len=70, grid=16, num_slots=64)
    yield "cca_mixed_small", synthetic.cca_case("cca_mixed_small", synthetic.SEED_BASE + 55,
                                           nq=4, nkv=2, hd=16, num_decodes=4,
                                           num_prefills=3, num_prefill_tokens=20,
                                           num_slots=16)


def digest(name, case):
    if isinstance(case, synthetic.CcaCase):
        out, cs, ds, _ = oracle.cca(case, nthreads=1)
        arrays = {"out": out, "conv_state": cs, "delayed_state": ds}
    else:
        out, pool, _ = oracle.conv(case, nthreads=1)
        arrays = {"out": out, "pool": pool}
    rec = {}
    for k, a in arrays.items():
        flat = np.ascontiguousarray(a).reshape(-1)
        idx = np.linspace(0, flat.size - 1, 5).astype(int)
        rec[k] = {"sha256": hashlib.sha256(flat.tobytes()).hexdigest(),
                  "dtype": str(flat.dtype), "shape": list(a.shape),
                  "samples": {str(int(i)): int(flat.view(np.uint16 if flat.dtype == np.uint16 else np.uint32)[i]) for i in idx}}
    return rec


if __name__ == "__main__":
    out = {"_about": "oracle regression digests; written by make_oracle_digest.py from oracle/ only"}
    for name, case in cases():
        out[name] = digest(name, case)
    with open(os.path.join(HERE, "oracle_digest.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print("wrote", os.path.join(HERE, "oracle_digest.json"))
