"""The seeded generator: determinism, layout, planting and bf16 rounding."""
import numpy as np

from sparse_long_context_page_amd import synth


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9, -2.5, 0.0], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    # 1 + 2^-9 is a tie -> even (1.0); 1 + 3*2^-9 rounds up to 1 + 2^-7
    assert back[0] == 1.0 and back[3] == 1.0 and back[2] == np.float32(1.0 + 2 ** -7)
    assert back[4] == -2.5 and back[5] == 0.0
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    err = np.abs(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(r)) - r)
    assert (err <= np.abs(r) * 2.0 ** -8 + 1e-30).all()


def test_generate_is_deterministic_and_laid_out():
    w = synth.shrink(synth.WORKLOADS["long_128k"], context=2048, batch=2, name="t")
    a = synth.generate(w, 3)
    b = synth.generate(w, 3, threads=1)
    for k in ("q", "k_pool", "v_pool", "block_table", "seq_lens"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["k_pool"].shape == (2 * 64, 8, 32, 128) and a["k_pool"].dtype == np.uint16
    bt = a["block_table"]
    assert sorted(bt[bt >= 0].ravel().tolist()) == list(range(128))
    c = synth.generate(w, 4)
    assert not np.array_equal(a["k_pool"], c["k_pool"])


def test_planted_runs_and_direction():
    w = synth.shrink(synth.WORKLOADS["long_128k"], context=4096, batch=1, name="t")
    inp = synth.generate(w, 3)
    G = 4
    for (b, g), pos in inp["planted"].items():
        assert len(pos) == 128
        runs = np.split(pos, 16)
        for r in runs:
            assert (np.diff(r) == 1).all()
        u = inp["q"][b, g * G:(g + 1) * G].astype(np.float64).mean(0)
        u /= np.linalg.norm(u)
        t = int(pos[0])
        phys = inp["block_table"][b, t // 32]
        k = synth.bf16_bits_to_f32(inp["k_pool"][phys, g, t % 32]).astype(np.float64)
        assert abs(k @ u - 3.0) < 0.5


def test_ragged_tail_fill():
    w = synth.Workload("r", 2, 2, 1, 8, 16, 0, "f32", (1.5,), (2,), 1.0, seq_lens=(20, 0))
    inp = synth.generate(w, 0)
    assert inp["block_table"][1].tolist() == [-1, -1]
    phys = inp["block_table"][0, 1]
    assert (inp["k_pool"][phys, 0, 4:] == synth.TAIL_FILL).all()
    assert (inp["k_pool"][phys, 0, :4] != synth.TAIL_FILL).all()
