"""Page boxes kept current by appends: boxes built for shorter sequences and
then updated with entmaxkv_append_page_meta equal the oracle's boxes of the
longer sequences (value for value), for one-token decode steps and for
multi-token appends that start pages, fill pages and cross page ends."""
import numpy as np
import pytest
import torch

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
