"""Host-side pieces of bench.py that run without a GPU: the CPU baselines' sampling loops and the
traffic lookup."""
import dataclasses
import importlib.util
import json
import os

import pytest

from workloads import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_search_baseline_stops_at_the_last_block(bench):
    # a budget long enough to reach the end: the sample takes 2048 vectors of each seeded block
    # and must stop after the last (ragged) block instead of asking for a block past the end
    w = dataclasses.replace(gen.EMBED_SEARCH, n=2 * gen.LOWRANK_BLOCK + 100, nq=4)
    r = bench.cpu_baseline_search(w, 2, seconds=1e9)
    assert r["sample"].startswith(f"{2 * 2048 + 100} of {w.n} vectors")
    assert "of 3 seeded blocks" in r["sample"]
    assert r["value"] > 0 and r["kind"] == "oracle"


def test_traffic_lookup_follows_the_source_hash(bench, tmp_path, monkeypatch):
    files = ("score.hip", "score_tile.h", "attention.hip")
    rec = {"+".join(files) + ":decode_attention": {"source_hash": bench.source_hash(*files),
                                                   "bytes_per_launch": 123.0}}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps(rec))
    csrc = tmp_path / "kv_cache_embedding_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in files:
        (csrc / f).write_bytes(open(os.path.join(ROOT, "kv_cache_embedding_amd", "csrc", f), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles(files, "decode_attention") == 123.0
    assert bench.traffic_from_profiles(files, "decode_layer") is None
    (csrc / "attention.hip").write_bytes(b"// changed\n")
    assert bench.traffic_from_profiles(files, "decode_attention") is None
