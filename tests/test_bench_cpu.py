"""bench.py host logic on the CPU: the algorithmic byte model and the oracle
CPU baseline (including Reindex layers), on a small synthetic layer sequence."""
import importlib.util
import os

import pytest

from fp4_kv_cache_e4m3_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_group_bytes_of_the_decode_group():
    b = _bench()
    nb = b.group_bytes(synth.C2)
    # 32 x 65,536 keys of 128 B plus 32 x 8 x (128 + 4) B of query rows and weights
    assert nb["scan"] == 268_469_248
    # per query: 512 FP4 rows of 288 B, Q 64 KiB, O 128 KiB, Top-K 2 KiB; SWA 128 KiB per sequence
    assert nb["attn_layer"] == 32 * (512 * 288 + 65536 + 131072 + 2048) + 32 * 128 * 1024
    assert nb["total"] == nb["quant"] + nb["scan"] + nb["select"] + 4 * nb["attn_layer"]
    d = b.group_bytes(synth.C6)
    assert d["total"] == d["quant"] + d["scan"] + d["select"] + 4 * d["reindex"] + 20 * d["attn_layer"]


@pytest.mark.parametrize("layers", [("full", "reuse"), ("full", "reuse", "reindex", "reuse"), ("reindex", "reuse")])
def test_cpu_baseline_runs_every_layer_kind(layers):
    b = _bench()
    w = synth.Small(batch=2, kv_len=1024, dim=128, heads=8, layers=layers).workload(wid=97, name="tiny")
    r = b.cpu_baseline(w, max_queries=2, min_seconds=0.0)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    assert "2 of 2 sequences" in r["sample"]
