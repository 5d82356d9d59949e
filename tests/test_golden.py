"""Golden fixtures: shape facts the pages fix, and the oracle's regression digest."""
import json
import os

import numpy as np
import pytest

import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_cca_state_and_output_shapes_follow_page_formulas():
    g = _load("page_shapes.json")
    for c in g["cca_state_shapes"]["cases"]:
        case = synthetic.cca_case("shape", 1, nq=c["num_attention_heads"],
                                  nkv=c["num_key_value_heads"], hd=c["head_dim"],
                                  t0=c["cca_time0"], t1=c["cca_time1"], num_decodes=1,
                                  prefill_lens=[2], num_slots=4)
        assert list(case.conv_state.shape[1:]) == c["conv_state"]
        assert list(case.delayed_state.shape[1:]) == c["delayed_state"]
    for c in g["cca_output_width"]["cases"]:
        case = synthetic.cca_case("shape", 1, nq=c["nq"], nkv=c["nkv"], hd=c["hd"],
                                  num_decodes=1, prefill_lens=[1], num_slots=2)
        assert case.out_width == c["width"]


def test_depthwise_state_len_follows_page_formulas():
    g = _load("page_shapes.json")
    for c in g["ple_state_len"]["cases"]:
        case = synthetic.conv_case("shape", 1, C=8, K=c["kernel"], d=c["dilation"],
                                   dtype="bf16", act="none", w_std=1, bias_std=None,
                                   num_slots=2, prefill_lens=[3])
        assert case.H == c["state_len"] and case.pool.shape[2] == c["state_len"]
    for c in g["gdn_state_len"]["cases"]:
        assert synthetic.varlen_prefill_8seq(C=8, B=1, max_len=4).pool.shape[2] == c["state_len"]


def test_oracle_regression_digest():
    import hashlib
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_oracle_digest", os.path.join(GOLDEN, "make_oracle_digest.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    want = _load("oracle_digest.json")
    for name, case in mod.cases():
        got = mod.digest(name, case)
        for k in got:
            assert got[k]["sha256"] == want[name][k]["sha256"], (name, k)
