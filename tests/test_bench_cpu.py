"""bench.py on a machine without a GPU: the one-GPU rule and the host-only
workload (the KV cache manager trace)."""

import json

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_host_cache_manager_workload_prints_one_json_line(capsys):
    assert bench.main(["--only", "KVC"]) == 0
    out = capsys.readouterr().out.strip().splitlines()
    assert len(out) == 1
    d = json.loads(out[0])
    assert d["only"] == "KVC" and d["requests"] == 1024
    assert 0.5 < d["prefix_reuse"] < 1.0            # the shared system prompts are reused
    assert d["requests_per_s"] > 0 and d["cpu_baseline"]["kind"] == "oracle"
