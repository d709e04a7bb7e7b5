"""Router Balance Lab on the GPU ("Inkling, Dissected", 02g).

A frozen router, one fresh batch per step, a hard capacity per expert and
the selection-only bias of 02e: each step is moe_router -> moe_dispatch
(capacity-limited) -> moe_bias_update through the C ABI, on buffers
allocated once.  The step's outputs (loads, kept pairs, picks, gates) stay
in the buffers below, where a harness reads them to take the lab's
measures; this module computes none of them.
"""
import torch

from . import _lib as L


class BalanceLab:
    """Buffers and calls of the lab's routing step for one workload."""

    def __init__(self, cfg, w_router, gamma, device, capacity_factor=None):
        if cfg.S != 0:
            raise ValueError("the balance lab has no shared experts")
        cf = cfg.capacity_factor if capacity_factor is None else capacity_factor
        self.cfg = cfg
        self.gamma = float(gamma)
        self.desc = L.make_desc(cfg.T, cfg.d, cfg.F, torch.float32, E=cfg.E, S=0, k=cfg.k,
                                capacity_factor=cf)
        T, E, k = cfg.T, cfg.E, cfg.k
        i32, f32 = torch.int32, torch.float32
        self.w_router = w_router
        self.bias = torch.zeros(E, dtype=f32, device=device)
        self.topk = torch.empty((T, k), dtype=i32, device=device)
        self.gates = torch.empty((T, k), dtype=f32, device=device)
        self.counts = torch.empty(E, dtype=i32, device=device)
        self.offsets = torch.empty(E + 1, dtype=i32, device=device)
        self.sorted_pair = torch.empty(T * k, dtype=i32, device=device)
        self.pair_pos = torch.empty(T * k, dtype=i32, device=device)
        self.ws_router = L.alloc_workspace(self.desc, L.CALL_ROUTER, device)
        self.ws_dispatch = L.alloc_workspace(self.desc, L.CALL_DISPATCH, device)

    def reset(self, bias=None):
        if bias is None:
            self.bias.zero_()
        else:
            self.bias.copy_(bias)

    def step(self, x):
        """Route x with the current bias, dispatch under capacity, then move
        the bias by gamma against this step's demand."""
        L.router(self.desc, x, self.w_router, self.bias, self.topk, self.gates,
                 ws=self.ws_router)
        L.dispatch(self.desc, self.topk, self.counts, self.offsets, self.sorted_pair,
                   self.pair_pos, ws=self.ws_dispatch)
        L.bias_update(self.desc, self.counts, self.gamma, self.bias)

    def capture(self, xs):
        """A HIP graph of the routing steps over the device batches ``xs``
        (one step per batch, in order), for replay without per-launch host
        cost.  The graph reads and updates ``self.bias`` in place, so a replay
        continues from whatever bias the buffer holds.  The step's calls
        launch kernels only (no memset, copy, allocation or sync), so they
        capture as they run."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        saved = self.bias.clone()
        with torch.cuda.stream(side):      # warm-up on a side stream before capture
            for x in xs[:2]:
                self.step(x)
        torch.cuda.current_stream().wait_stream(side)
        self.bias.copy_(saved)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for x in xs:
                self.step(x)
        torch.cuda.synchronize()
        self.bias.copy_(saved)
        return g
