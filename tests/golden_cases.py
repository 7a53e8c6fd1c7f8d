"""Loader for the worked examples under tests/golden/ (each file cites the page
section it restates).  Builds bf16 inputs from the small JSON schema."""
from __future__ import annotations

import glob
import json
import os

import numpy as np

from variable_length_flashattention_amd.inputs import bf16_bits

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_files(prefix="plan_"):
    return sorted(glob.glob(os.path.join(GOLDEN_DIR, prefix + "*.json")))


def load(path):
    with open(path) as f:
        return json.load(f)


def build_inputs(g):
    cu = np.asarray(g["cu_seqlens"], dtype=np.int32)
    T, H, D = int(cu[-1]), g["num_heads"], g["head_dim"]

    def per_token(key):
        vals = np.asarray(g[key], dtype=np.float32)
        return np.broadcast_to(vals[:, None, None], (T, H, D)).copy()

    def ramp(step):
        return (np.arange(T * H * D, dtype=np.float64) * step).astype(np.float32).reshape(T, H, D)

    q = per_token("q_token_values") if "q_token_values" in g else ramp(g["q_ramp"])
    k = per_token("k_token_values") if "k_token_values" in g else ramp(g["k_ramp"])
    if g.get("v_onehot_dim_mod"):
        v = np.zeros((T, H, D), np.float32)
        for t in range(T):
            v[t, :, t % D] = 1.0
    elif "v_token_values" in g:
        v = per_token("v_token_values")
    else:
        v = ramp(g["v_ramp"])
    return bf16_bits(q), bf16_bits(k), bf16_bits(v), cu


def check(g, run):
    """``run(q, k, v, cu, scale, causal) -> (out, lse)``; raises AssertionError
    when an expectation of the page fails."""
    q, k, v, cu = build_inputs(g)
    results = {c: run(q, k, v, cu, g["scale"], c) for c in g["causal"]}
    for e in g["expect"]:
        causals = [e["causal"]] if "causal" in e else g["causal"]
        for c in causals:
            out, lse = results[c]
            kind = e["kind"]
            if kind == "rows_equal_value":
                sub = out[e["tokens"]]
                err = float(np.max(np.abs(sub - e["value"])))
                assert err <= e["tol"], f"{kind} causal={c}: max err {err}"
            elif kind == "causal_row_equals_noncausal_row":
                oc, _ = results[True]
                on, _ = results[False]
                err = float(np.max(np.abs(oc[e["tokens"]] - on[e["tokens"]])))
                assert err <= e["tol"], f"{kind}: {err}"
            elif kind == "onehot_weights_sum_to_one":
                D = g["head_dim"]
                for b in range(len(cu) - 1):
                    for t in range(cu[b], cu[b + 1]):
                        dims = [kt % D for kt in range(cu[b], cu[b + 1])]
                        s = out[t][:, dims].sum(axis=-1)
                        assert np.all(np.abs(s - 1.0) <= e["tol"]), f"{kind}: {s}"
            elif kind == "shape":
                assert list(out.shape) == e["out"] and list(lse.shape) == e["lse"], (out.shape, lse.shape)
            elif kind == "all_finite":
                assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), kind
            else:
                raise ValueError(kind)
