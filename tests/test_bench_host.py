"""Host-side logic of bench.py: byte accounting and the oracle CPU baseline."""
import numpy as np

import bench
from sparse_long_context_page_amd import synth


def test_union_pages_and_bytes():
    w = synth.shrink(synth.WORKLOADS["long_128k"], context=4096, batch=2, n_planted=0, name="t")
    sel = np.full((2, 32, 4), -1, dtype=np.int32)
    sel[0, 0:4, :2] = [[1, 2], [2, 3], [1, 3], [7, 9]]  # group 0 of sequence 0: {1,2,3,7,9}
    sel[1, 4:8, 0] = 5  # group 1 of sequence 1: {5}
    up = bench.union_pages(sel, 4)
    assert up[0, 0] == 5 and up[1, 1] == 1 and up.sum() == 6
    lens = np.array([4096, 4096], dtype=np.int32)
    sup_s = np.ones((2, 32), dtype=np.int32)
    sup_f = np.full((2, 32), 3, dtype=np.int32)
    nb = bench.algorithmic_bytes(w, lens, 4, sel, sup_s, sup_f)
    P = 4096 // 32
    assert nb["bounds"] == 2 * P * 8 * 2 * 128 * 2 + 2 * 32 * 128 * 4 + 2 * P * 4
    assert nb["score_full"] == 2 * 4096 * 8 * 128 * 2 + 2 * 32 * 128 * 4 + 2 * P * 4
    assert nb["score_sparse"] == 6 * 32 * 128 * 2 + 2 * 32 * 128 * 4 + 2 * 32 * 4 * 4 + 2 * P * 4
    assert nb["tau_pv_full"] == 64 * 3 * 128 * 2 + 2 * 32 * 128 * 4
    # the all-K+V view: the union pages' K and V (plus boxes), or all of K and V
    meta_b = 2 * P * 8 * 2 * 128 * 2
    k_sel = 6 * 32 * 128 * 2
    q_b = out_b = 2 * 32 * 128 * 4
    sel_b, bt_b = 2 * 32 * 4 * 4, 2 * P * 4
    # q and the block table are read by the bound and the score kernels
    assert nb["_sparse_all_kv"] == meta_b + 2 * k_sel + 2 * q_b + out_b + sel_b + 2 * bt_b
    assert nb["_full_all_kv"] == 2 * 2 * 4096 * 8 * 128 * 2 + q_b + out_b + bt_b


def test_cpu_baseline_runs_and_matches_oracle_selection():
    w = synth.shrink(synth.WORKLOADS["long_128k"], context=2048, batch=1, n_planted=8, name="t")
    inp = synth.generate(w, 3)
    cb = bench.cpu_baseline(inp, 8, 1.5, n_heads=4)
    assert cb["value"] > 0 and cb["cores"] >= 1 and cb["kind"] == "oracle"
    assert len(cb["_results"]) == 4
    for b, h, dt, sel, rs, rf, near in cb["_results"]:
        assert len(sel) == 8 and rs.shape == (128,) and rf.shape == (128,)
        # the near-tie band always holds the budget-th page itself
        assert len(near) >= 1 and all(0 <= j < 2048 // 32 for j in near)


def test_multi_gpu_request_exits(monkeypatch, capsys):
    import pytest
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_containment_criterion():
    """Equal support size and tau (within 1e-6 relative) count as contained."""
    sup_s = np.array([[3, 3], [2, 5]])
    sup_f = np.array([[3, 4], [2, 5]])
    tau_f = np.array([[1.0, 1.0], [-2.0, 0.5]])
    tau_s = np.array([[1.0, 1.0], [-2.0 - 1e-5, 0.5 + 5e-7]])
    c = bench.contained(sup_s, sup_f, tau_s, tau_f)
    assert c.tolist() == [[True, False], [False, True]]
