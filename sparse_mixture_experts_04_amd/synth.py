"""Seeded synthetic inputs for the MoE layer.

This module only draws random tensors; it holds none of the layer's
arithmetic, so the oracle and the HIP path can both be fed from it.

Recipe (all draws are torch generators seeded from a SHA-256 of
``"<config>/<tensor>/<index>"``, so every tensor and every expert has its own
stream and the result does not depend on generation order):

* ``x``            ~ N(0, 1), one row per token (the RMS-normalised residual
  stream entering the layer has unit RMS);
* ``w_router``     [E+S, d] fp32 ~ N(0, 1/d); rows 0..E-1 are the routed
  experts' routing vectors, rows E, E+1 the shared experts';
* ``w_gate``, ``w_up``  [E, F, d] ~ N(0, 1/d);
* ``w_down``       [E, d, F] ~ N(0, 1/d), or N(0, 1/F) where the workload
  says so;
* shared-expert weights, same shapes with leading dimension S;
* ``bias``         [E] fp32 ~ U[-r, r];
* skewed router (workload E): ``w_router[i] += c_i * u`` for the routed rows,
  ``u`` a seeded unit vector, ``c_i = kappa * r_i ** -s`` with ``r_i`` a seeded
  permutation of the ranks 1..E.

* balance-lab workloads (``lab_head_tail > 0``): E home directions
  ``c_j`` (rows N(0, I) scaled to unit length), router ``w_router =
  lab_kappa * c`` (routed rows only); each step's tokens pick a home
  cluster j with probability proportional to ``(j + 1) ** -a``,
  ``a = ln(lab_head_tail) / ln(E)`` (so expert 0's cluster is
  ``lab_head_tail`` times as common as expert E-1's), and
  ``x_t = c_j + lab_jitter * N(0, I / d)``.  Drawn on the CPU (the same
  values whatever the device), then moved.

Values are drawn in fp32 and rounded to nearest-even into bf16 where the
workload is bf16.  N(0, v) means variance v.
"""
import hashlib
import math

import torch

from .configs import MoEConfig


def _seed(cfg_name: str, tensor: str, index: int = 0) -> int:
    h = hashlib.sha256(f"{cfg_name}/{tensor}/{index}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, cfg_name, tensor, index=0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg_name, tensor, index))
    return g


def act_dtype(cfg: MoEConfig):
    return torch.float32 if cfg.act == "f32" else torch.bfloat16


def normal(shape, std, device, cfg_name, tensor, index=0, dtype=torch.float32):
    g = _gen(device, cfg_name, tensor, index)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(dtype)


def make_x(cfg: MoEConfig, device="cpu", step: int = 0, T: int = None):
    T = cfg.T if T is None else T
    return normal((T, cfg.d), 1.0, device, cfg.name, "x", step, act_dtype(cfg))


def make_bias(cfg: MoEConfig, device="cpu"):
    if cfg.bias_range == 0.0:
        return torch.zeros(cfg.E, dtype=torch.float32, device=device)
    g = _gen(device, cfg.name, "bias")
    u = torch.rand(cfg.E, generator=g, device=device, dtype=torch.float32)
    return (u * 2.0 - 1.0) * cfg.bias_range


def make_router(cfg: MoEConfig, device="cpu"):
    w = normal((cfg.E + cfg.S, cfg.d), 1.0 / math.sqrt(cfg.d), device,
               cfg.name, "w_router")
    if cfg.skew_kappa > 0.0:
        gu = _gen(device, cfg.name, "skew_dir")
        u = torch.randn(cfg.d, generator=gu, device=device, dtype=torch.float64)
        u = (u / u.norm()).to(torch.float32)
        gp = _gen("cpu", cfg.name, "skew_rank")
        ranks = torch.randperm(cfg.E, generator=gp).to(torch.float64) + 1.0
        c = (cfg.skew_kappa * ranks.pow(-cfg.skew_zipf_s)).to(torch.float32)
        w[: cfg.E] += c.to(device)[:, None] * u[None, :]
    return w


def make_expert_weights(cfg: MoEConfig, device="cpu"):
    """Returns a dict of the routed and shared expert weights.

    Each expert's matrices are drawn from their own streams, so any single
    expert can be regenerated alone (see ``expert_matrix``).
    """
    dt = act_dtype(cfg)
    out = {}
    for name, n, shape in (("w_gate", cfg.E, (cfg.F, cfg.d)),
                           ("w_up", cfg.E, (cfg.F, cfg.d)),
                           ("w_down", cfg.E, (cfg.d, cfg.F)),
                           ("ws_gate", cfg.S, (cfg.F, cfg.d)),
                           ("ws_up", cfg.S, (cfg.F, cfg.d)),
                           ("ws_down", cfg.S, (cfg.d, cfg.F))):
        t = torch.empty((n,) + shape, dtype=dt, device=device)
        for e in range(n):
            t[e] = expert_matrix(cfg, name, e, device)
        out[name] = t
    return out


def expert_matrix(cfg: MoEConfig, name: str, e: int, device="cpu"):
    dt = act_dtype(cfg)
    if name in ("w_down", "ws_down") and cfg.wd_std_from_F:
        std = 1.0 / math.sqrt(cfg.F)
    else:
        std = 1.0 / math.sqrt(cfg.d)
    shape = (cfg.d, cfg.F) if name in ("w_down", "ws_down") else (cfg.F, cfg.d)
    return normal(shape, std, device, cfg.name, name, e, dt)


def make_inputs(cfg: MoEConfig, device="cpu"):
    """All inputs of one forward call: x, router, bias and expert weights."""
    inp = {"x": make_x(cfg, device), "w_router": make_router(cfg, device),
           "bias": make_bias(cfg, device)}
    inp.update(make_expert_weights(cfg, device))
    return inp


def lab_directions(cfg: MoEConfig):
    g = _gen("cpu", cfg.name, "lab_home")
    c = torch.randn((cfg.E, cfg.d), generator=g, dtype=torch.float64)
    return c / c.norm(dim=1, keepdim=True)


def make_lab_router(cfg: MoEConfig, device="cpu"):
    """Frozen router of a balance-lab workload: [E, d] fp32."""
    return (cfg.lab_kappa * lab_directions(cfg)).to(torch.float32).to(device)


def make_lab_x(cfg: MoEConfig, step: int, device="cpu", T: int = None):
    """Tokens of step ``step`` of a balance-lab workload: [T, d] fp32."""
    T = cfg.T if T is None else T
    c = lab_directions(cfg)
    a = math.log(cfg.lab_head_tail) / math.log(cfg.E)
    p = torch.arange(1, cfg.E + 1, dtype=torch.float64).pow(-a)
    g = _gen("cpu", cfg.name, "lab_tokens", step)
    home = torch.multinomial(p, T, replacement=True, generator=g)
    noise = torch.randn((T, cfg.d), generator=g, dtype=torch.float64)
    x = c[home] + noise * (cfg.lab_jitter / math.sqrt(cfg.d))
    return x.to(torch.float32).to(device)
