"""Host-side logic of bench.py, on the CPU: the prefill launch plan it mirrors
to name each event mark, and the rule that drops the HBM traffic figure once
the scan's sources differ from those the counters were taken on."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_prefill_select_kernels_single_sequence():
    # 32768 rows at up to 32768 keys: 1 GiB of scores holds 8192 rows, so four chunks, all scanned
    assert bench.prefill_select_kernels([(0, 32768, 0)], 2048) == ["indexer", "topk"] * 4
    # every row sees at most k keys: no scan
    assert bench.prefill_select_kernels([(0, 2000, 0)], 2048) == ["topk"]
    # one chunk whose later rows see more than k keys
    assert bench.prefill_select_kernels([(0, 2500, 0)], 2048) == ["indexer", "topk"]


def test_prefill_select_kernels_many_sequences():
    # 8 sequences of 4096 rows after prefixes 0, 4096, ...: stride 32768 -> chunks of 8192 rows
    pieces = [(4096 * i, 4096, 4096 * i) for i in range(8)]
    assert bench.prefill_select_kernels(pieces, 2048) == ["indexer", "topk"] * 4
    # 70 one-row sequences: at most 64 pieces per launch, so two chunks; none sees more than k keys
    pieces = [(i, 1, 10) for i in range(70)]
    assert bench.prefill_select_kernels(pieces, 2048) == ["topk", "topk"]
    # only the second chunk has a row past k
    pieces = [(i, 1, 10) for i in range(64)] + [(64, 1, 5000)]
    assert bench.prefill_select_kernels(pieces, 2048) == ["topk", "indexer", "topk"]


def test_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = tmp_path / "dsa_sparse_attention_02_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "indexer.hpp").write_text("kernel v1\n")
    (src / "device_common.hpp").write_text("common\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    key = bench.TRAFFIC_KERNEL + "/w"
    h = bench.source_hash("indexer.hpp", "device_common.hpp")
    (prof / "traffic.json").write_text(json.dumps({key: {"sources": ["indexer.hpp", "device_common.hpp"],
                                                         "source_hash": h, "bytes_per_launch": 123}}))
    assert bench.traffic_from_profiles(key, 1) == 123
    (src / "indexer.hpp").write_text("kernel v2\n")
    assert bench.traffic_from_profiles(key, 1) is None
    assert bench.traffic_from_profiles("other/w", 1) is None
