"""Host-side parts of bench.py (no GPU): the one-GPU guard, the byte and
flop formulas the roofline figures rest on, the percentile helper and the
child-process oracle timing."""

import numpy as np
import pytest

import bench
from workloads import generate_host, get_config


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_causal_work_matches_the_closed_form():
    # a sequence with c cached tokens and n new ones: query j sees c + j + 1 keys
    for c, n in ((0, 1), (0, 7), (13, 5), (100, 64)):
        flops, keys = bench.causal_work(np.array([c + n]), np.array([0, n]), 32, 128)
        assert keys == n * c + n * (n + 1) // 2
        assert flops == keys * 32 * 4 * 128
    # queries before position 0 see nothing; two sequences add up
    flops, keys = bench.causal_work(np.array([3, 10]), np.array([0, 5, 7]), 2, 64)
    assert keys == (1 + 2 + 3) + (9 + 10)
    assert flops == keys * 2 * 4 * 64


def test_decode_step_bytes_follow_the_formula():
    cfg = get_config("c1_tiny_f32")
    lens = np.array([35, 16, 1, 100])
    b = bench.step_bytes(cfg, lens)
    row = cfg.kv_heads * cfg.head_dim * 4
    assert b["kv_read"] == int(lens.sum()) * row * 2
    blocks = 3 + 1 + 1 + 7
    assert b["decode"] == b["kv_read"] + 4 * cfg.q_heads * cfg.head_dim * 4 * 2 + blocks * 4 + 4 * 4
    assert b["kv_write"] == 4 * (row * 2 * 2 + 8)
    assert b["shared_repeat"] == 0


def test_block_size_override_is_optional():
    assert bench.parse_args([]).block_size is None
    assert bench.parse_args(["--block-size", "32"]).block_size == 32


def test_percentiles():
    p = bench.percentiles([float(x) for x in range(1, 102)])
    assert p == {"p10": 11.0, "p50": 51.0, "p90": 91.0}


def test_profiles_name_no_traffic_for_an_unprofiled_workload():
    assert bench.profiled_traffic("x1_extend_tiny_bf16") is None


def test_oracle_timing_runs_in_a_child_with_a_worker_pool():
    cfg = get_config("c1_tiny_f32")
    w = generate_host(cfg)
    res = bench.cpu_baseline(cfg, w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, 4)
    assert res["kind"] == "oracle" and res["unit"] == "GB/s"
    assert 1 <= res["cores"] <= min(4, bench.host_workers())
    assert res["workers"] == res["cores"] and res["visible_cores"] == bench.visible_cores()
    assert bench.host_workers() == min(bench.visible_cores(), res["core_share"])
    assert res["value"] > 0 and res["one_core"]["value"] > 0
    with pytest.raises(RuntimeError):
        bench.run_cpu_oracle("decode", {"q": w.q}, [0], scale=0.1, dtype="f32")
