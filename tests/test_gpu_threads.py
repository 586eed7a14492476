"""Several host threads calling the library at once, each on its own stream
with its own workspaces and outputs: every thread's results equal, bit for
bit, those of one thread calling alone (the calls share no state)."""
import threading

import pytest
import torch

from sparse_long_context_page_amd import synth
from parity_util import Dev, announce

pytestmark = pytest.mark.gpu


def test_concurrent_host_threads_match_single_thread():
    from sparse_long_context_page_amd import entmaxkv as E
    w = synth.shrink(synth.WORKLOADS["gqa_32k"], context=6000, batch=2, n_planted=8)
    inp = synth.generate(w, 2)
    dev = Dev(inp)
    dev.build_meta()
    budget, alpha = 24, 1.5
    B, H, D = w.batch, w.num_q_heads, w.head_dim
    cuda = torch.device("cuda")

    def make_slot():
        sel = torch.empty((B, H, budget), dtype=torch.int32, device=cuda)
        outs = [(torch.empty((B, H, D), device=cuda), torch.empty((B, H), device=cuda),
                 torch.empty((B, H), dtype=torch.int32, device=cuda)) for _ in range(2)]
        ws = [E.workspace(dev.shape, budget, i, cuda) for i in range(3)]
        return sel, outs, ws

    def step(slot, stream):
        sel, outs, ws = slot
        E.entmaxkv_score_select(dev.shape, dev.q, dev.meta, dev.bt, dev.lens, budget, sel,
                                ws=ws[0], stream=stream)
        E.entmaxkv_decode_sparse(dev.shape, dev.q, dev.k, dev.v, dev.bt, dev.lens, sel, budget,
                                 alpha, *outs[0], ws=ws[1], stream=stream)
        E.entmaxkv_decode_full(dev.shape, dev.q, dev.k, dev.v, dev.bt, dev.lens, alpha, *outs[1],
                               ws=ws[2], stream=stream)

    def results(slot):
        sel, outs, _ = slot
        return [x.cpu() for x in (sel, *outs[0], *outs[1])]

    announce("threads: single-thread reference")
    torch.cuda.synchronize()
    ref_slot = make_slot()
    s0 = torch.cuda.Stream()
    step(ref_slot, s0)
    s0.synchronize()
    ref = results(ref_slot)

    n_threads, rounds = 4, 3
    slots = [make_slot() for _ in range(n_threads)]
    streams = [torch.cuda.Stream() for _ in range(n_threads)]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            for _ in range(rounds):
                step(slots[i], streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((i, e))

    announce(f"threads: {n_threads} threads x {rounds} steps")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    names = ("sel", "out sparse", "tau sparse", "support sparse", "out full", "tau full",
             "support full")
    for i in range(n_threads):
        got = results(slots[i])
        for name, a, b in zip(names, ref, got):
            assert torch.equal(a, b), f"thread {i}: {name} differs from the single-thread run"
