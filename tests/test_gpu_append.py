"""Page boxes and page key moments kept current by appends: boxes built for
shorter sequences and then updated with entmaxkv_append_page_meta equal the
oracle's boxes of the longer sequences (value for value), for one-token
decode steps and for multi-token appends that start pages, fill pages and
cross page ends; moments updated with entmaxkv_append_page_moments equal a
full rebuild bit for bit and the oracle's moments within one unit in the
last place."""
import numpy as np
import pytest
import torch

from oracle import entmax_oracle as O
from oracle import gauss_oracle as GO
from sparse_long_context_page_amd import synth
from parity_util import Dev, announce, check_meta_sequence, meta_to_f64

pytestmark = pytest.mark.gpu


def _workload(kv_dtype, D, ps, Hkv, lens):
    return synth.Workload("append", len(lens), 2 * Hkv, Hkv, D, ps, max(lens), kv_dtype, (1.5,),
                          (4,), 4.0 / np.sqrt(D), plant="group_mean", n_planted=2, seq_lens=lens)


def _check_all(inp, meta):
    w = inp["workload"]
    m64 = meta_to_f64(meta, w.kv_dtype)
    for b in range(w.batch):
        if inp["seq_lens"][b] > 0:
            for g in range(w.num_kv_heads):
                check_meta_sequence(inp, m64, b, g)


@pytest.mark.parametrize("kv_dtype,D,ps,Hkv", [
    ("bf16", 128, 32, 2), ("f32", 64, 16, 1), ("bf16", 64, 64, 4), ("f32", 128, 32, 2)])
def test_append_matches_rebuild(kv_dtype, D, ps, Hkv):
    from sparse_long_context_page_amd import entmaxkv as E
    new = (1, ps, ps + 1, 3 * ps - 1, 5 * ps + 7, 40, 2 * ps)
    added = (1, 1, ps, 2, ps + 9, 40, 0)  # tokens appended to each sequence this call
    inp = synth.generate(_workload(kv_dtype, D, ps, Hkv, new), 21)
    dev = Dev(inp)
    announce(f"append {kv_dtype} D{D} ps{ps} Hkv{Hkv}")
    old_np = np.maximum(np.asarray(new) - np.asarray(added), 0).astype(np.int32)
    old = torch.from_numpy(old_np).cuda()
    meta = torch.full((inp["num_phys_pages"], Hkv, 2, D), float("nan"), dtype=dev.kv_torch,
                      device="cuda")
    E.entmaxkv_build_page_meta(dev.shape, dev.k, dev.bt, old, meta)
    E.entmaxkv_append_page_meta(dev.shape, dev.k, dev.bt, old, dev.lens, max(added), meta)
    torch.cuda.synchronize()
    _check_all(inp, meta)


def test_decode_loop_one_token_per_step():
    """A decode loop: every step appends one token per sequence (the page
    boxes grow token by token, starting new pages on the way)."""
    from sparse_long_context_page_amd import entmaxkv as E
    ps = 16
    final = (3 * ps + 5, 2 * ps, ps + 1, 9)
    steps = ps + 6
    inp = synth.generate(_workload("bf16", 128, ps, 2, final), 22)
    dev = Dev(inp)
    announce("append decode loop")
    start = np.maximum(np.asarray(final) - steps, 0).astype(np.int32)
    cur = torch.from_numpy(start).cuda()
    meta = torch.full((inp["num_phys_pages"], 2, 2, 128), float("nan"), dtype=torch.bfloat16,
                      device="cuda")
    E.entmaxkv_build_page_meta(dev.shape, dev.k, dev.bt, cur, meta)
    for _ in range(steps):
        nxt = torch.minimum(cur + 1, dev.lens)
        E.entmaxkv_append_page_meta(dev.shape, dev.k, dev.bt, cur, nxt, 1, meta)
        cur = nxt
    torch.cuda.synchronize()
    assert torch.equal(cur.cpu(), dev.lens.cpu())
    _check_all(inp, meta)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


def _check_moments(inp, mom):
    """Every referenced page's moments against the oracle: within one unit
    in the last place of the stored dtype (bf16: float32 spacing x 2^16)."""
    w = inp["workload"]
    mean, var = GO.page_moments(inp["k_pool"], inp["block_table"], inp["seq_lens"],
                                w.page_size, w.kv_dtype)
    got = meta_to_f64(mom, w.kv_dtype)
    used = sorted({int(inp["block_table"][b, j]) for b in range(w.batch)
                   for j in range(O.num_pages(int(inp["seq_lens"][b]), w.page_size))})
    for side, ref in ((0, mean), (1, var)):
        g, r = got[used, :, side], ref[used]
        sp = np.spacing(np.maximum(np.abs(r), 1e-30).astype(np.float32)).astype(np.float64)
        if w.kv_dtype == "bf16":
            sp *= 65536.0
        assert (np.abs(g - r) <= sp).all(), f"moments side {side}"


@pytest.mark.parametrize("kv_dtype,D,ps,Hkv", [
    ("bf16", 128, 32, 2), ("f32", 64, 16, 1), ("bf16", 64, 64, 4), ("f32", 128, 32, 2)])
def test_append_moments_matches_rebuild(kv_dtype, D, ps, Hkv):
    from sparse_long_context_page_amd import entmaxkv as E
    new = (1, ps, ps + 1, 3 * ps - 1, 5 * ps + 7, 40, 2 * ps)
    added = (1, 1, ps, 2, ps + 9, 40, 0)
    inp = synth.generate(_workload(kv_dtype, D, ps, Hkv, new), 23)
    dev = Dev(inp)
    announce(f"append moments {kv_dtype} D{D} ps{ps} Hkv{Hkv}")
    old = torch.from_numpy(np.maximum(np.asarray(new) - np.asarray(added), 0)
                           .astype(np.int32)).cuda()
    shape = (inp["num_phys_pages"], Hkv, 2, D)
    mom = torch.full(shape, float("nan"), dtype=dev.kv_torch, device="cuda")
    ref = torch.full(shape, float("nan"), dtype=dev.kv_torch, device="cuda")
    E.entmaxkv_build_page_moments(dev.shape, dev.k, dev.bt, old, mom)
    E.entmaxkv_append_page_moments(dev.shape, dev.k, dev.bt, old, dev.lens, max(added), mom)
    E.entmaxkv_build_page_moments(dev.shape, dev.k, dev.bt, dev.lens, ref)
    torch.cuda.synchronize()
    # unreferenced pages stay NaN in both: the whole buffer agrees bit for bit
    assert torch.equal(_bits(mom), _bits(ref))
    _check_moments(inp, mom)


def test_decode_loop_moments_then_gauss_select():
    """A decode loop keeping boxes and moments current one token per step,
    then the Gaussian selection on the maintained moments equals the one on
    rebuilt moments."""
    from sparse_long_context_page_amd import entmaxkv as E
    ps = 16
    final = (3 * ps + 5, 2 * ps, ps + 1, 9)
    steps = ps + 6
    inp = synth.generate(_workload("bf16", 128, ps, 2, final), 24)
    dev = Dev(inp)
    announce("append moments decode loop")
    cur = torch.from_numpy(np.maximum(np.asarray(final) - steps, 0).astype(np.int32)).cuda()
    shape = (inp["num_phys_pages"], 2, 2, 128)
    mom = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    E.entmaxkv_build_page_moments(dev.shape, dev.k, dev.bt, cur, mom)
    for _ in range(steps):
        nxt = torch.minimum(cur + 1, dev.lens)
        E.entmaxkv_append_page_moments(dev.shape, dev.k, dev.bt, cur, nxt, 1, mom)
        cur = nxt
    ref = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    E.entmaxkv_build_page_moments(dev.shape, dev.k, dev.bt, dev.lens, ref)
    torch.cuda.synchronize()
    assert torch.equal(_bits(mom), _bits(ref))
    _check_moments(inp, mom)
    B, H = len(final), dev.w.num_q_heads
    outs = []
    for m in (mom, ref):
        sel = torch.empty((B, H, 4), dtype=torch.int32, device="cuda")
        tau_hat = torch.empty((B, H), device="cuda")
        E.entmaxkv_gauss_select(dev.shape, dev.q, m, dev.bt, dev.lens, 1.5, 1.0, 4, sel, tau_hat)
        outs.append((sel.cpu(), tau_hat.cpu()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_append_without_growth_leaves_pages_alone(kv_dtype):
    """Sequences whose new length is not above the old one (equal, or
    shorter) are left as they are by both append entry points, bit for bit;
    the one sequence that grows is updated."""
    from sparse_long_context_page_amd import entmaxkv as E
    ps, D, Hkv = 16, 64, 2
    lens = (3 * ps + 5, 2 * ps, ps + 1, 9)
    inp = synth.generate(_workload(kv_dtype, D, ps, Hkv, lens), 25)
    dev = Dev(inp)
    announce(f"append without growth {kv_dtype}")
    shape = (inp["num_phys_pages"], Hkv, 2, D)
    meta = torch.full(shape, float("nan"), dtype=dev.kv_torch, device="cuda")
    mom = torch.full(shape, float("nan"), dtype=dev.kv_torch, device="cuda")
    E.entmaxkv_build_page_meta(dev.shape, dev.k, dev.bt, dev.lens, meta)
    E.entmaxkv_build_page_moments(dev.shape, dev.k, dev.bt, dev.lens, mom)
    torch.cuda.synchronize()
    meta0, mom0 = _bits(meta), _bits(mom)
    old = dev.lens.clone()
    new = torch.tensor([lens[0], lens[1] - 3, 0, lens[3] - 1], dtype=torch.int32, device="cuda")
    E.entmaxkv_append_page_meta(dev.shape, dev.k, dev.bt, old, new, 4, meta)
    E.entmaxkv_append_page_moments(dev.shape, dev.k, dev.bt, old, new, 4, mom)
    torch.cuda.synchronize()
    assert torch.equal(_bits(meta), meta0) and torch.equal(_bits(mom), mom0)
    # growing back to the built lengths (3, 17 and 1 rows) recomputes the
    # touched pages to the same bits
    E.entmaxkv_append_page_moments(dev.shape, dev.k, dev.bt, new, dev.lens, lens[2], mom)
    E.entmaxkv_append_page_meta(dev.shape, dev.k, dev.bt, new, dev.lens, lens[2], meta)
    torch.cuda.synchronize()
    assert torch.equal(_bits(mom), mom0)
    _check_all(inp, meta)
