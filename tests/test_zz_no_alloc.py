"""moe_dispatch_noalloc (the dispatch for callers that cannot allocate: its
scratch is the library's own device array) against moe_dispatch with a
workspace: the same counts, offsets, permutation and inverse map bit for
bit, on two calls in a row, the second with a smaller batch (and a
capacity limit, so the array holds the first call's values when the second
starts)."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_04_amd import _lib as L
from sparse_mixture_experts_04_amd.configs import MoEConfig

from parity_util import Buffers, desc_for, log, npi

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _topk(T, E, k, seed):
    rng = np.random.default_rng(seed)
    # skewed demand so some experts overflow a capacity limit
    p = 1.0 / np.arange(1, E + 1) ** 0.8
    p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def test_dispatch_noalloc_matches_dispatch_twice():
    for T, cf, seed in ((6000, 0.0, 1), (700, 1.0, 2)):
        cfg = MoEConfig(f"noalloc_{T}", T=T, d=256, F=128, act="bf16", capacity_factor=cf)
        desc = desc_for(cfg)
        log(f"[no-alloc dispatch] T={T} capacity factor {cf}")
        topk = torch.tensor(_topk(T, cfg.E, cfg.k, seed), device=DEV)
        ref = Buffers(desc, DEV)
        got = Buffers(desc, DEV)
        for b in (ref, got):
            b.topk.copy_(topk)
            for t in (b.counts, b.offsets, b.sorted_pair, b.pair_pos):
                t.fill_(-7)
        L.dispatch(desc, ref.topk, ref.counts, ref.offsets, ref.sorted_pair, ref.pair_pos)
        L.dispatch_noalloc(desc, got.topk, got.counts, got.offsets, got.sorted_pair,
                           got.pair_pos)
        torch.cuda.synchronize()
        n_kept = int(ref.offsets[-1].item())
        assert n_kept == T * cfg.k if cf == 0.0 else 0 < n_kept < T * cfg.k
        assert torch.equal(got.counts, ref.counts)
        assert torch.equal(got.offsets, ref.offsets)
        assert torch.equal(got.sorted_pair[:n_kept], ref.sorted_pair[:n_kept])
        assert torch.equal(got.pair_pos, ref.pair_pos)
        if cf:
            assert int((npi(ref.pair_pos) < 0).sum()) > 0     # the capacity dropped pairs


def test_dispatch_noalloc_rejects_batches_past_its_scratch():
    # 1 MiB of scratch holds the counts of 1023 segments of 512 pairs at E=256
    ok = MoEConfig("noalloc_max", T=1023 * 512 // 6, d=256, F=128, act="bf16")
    too_big = MoEConfig("noalloc_over", T=1023 * 512 // 6 + 86, d=256, F=128, act="bf16")
    for cfg, fine in ((ok, True), (too_big, False)):
        desc = desc_for(cfg)
        b = Buffers(desc, DEV)
        b.topk.copy_(torch.tensor(_topk(cfg.T, cfg.E, cfg.k, 3), device=DEV)
                     if fine else torch.zeros_like(b.topk))
        if fine:
            L.dispatch_noalloc(desc, b.topk, b.counts, b.offsets, b.sorted_pair, b.pair_pos)
            ref = Buffers(desc, DEV)
            L.dispatch(desc, b.topk, ref.counts, ref.offsets, ref.sorted_pair, ref.pair_pos)
            torch.cuda.synchronize()
            assert torch.equal(b.counts, ref.counts) and torch.equal(b.pair_pos, ref.pair_pos)
        else:
            with pytest.raises(L.MoEError, match="UNSUPPORTED"):
                L.dispatch_noalloc(desc, b.topk, b.counts, b.offsets, b.sorted_pair, b.pair_pos)
