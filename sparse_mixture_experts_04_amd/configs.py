"""Named MoE-layer workloads (shapes, dtypes and value distributions).

Every workload is the DeepSeek-V3-lineage MoE feed-forward layer described in
"Inkling, Dissected" (chapter 02, "Anatomy of one MoE layer"): 256 routed
experts, 2 shared experts, top-6 routing.  The shapes below are synthetic
stand-ins chosen to exercise the regimes that matter on one GPU:

* ``A``  tiny fp32 layer (every tensor fp32), parity only;
* ``B``  a prefill chunk in bf16;
* ``C``  decode-sized: 64 tokens, bound by streaming expert weights;
* ``D``  large batch: 16384 tokens at hidden 7168, bound by matrix cores;
* ``E``  shape of ``D`` with a skewed router, run for 100 bias-update steps;
* ``Ecap`` ``E`` with a hard capacity of 1.25x the ideal load per expert
  (the Router Balance Lab's setting in "Inkling, Dissected" 02g);
* ``Cfp4`` the decode batch of ``C`` with the routed experts' weights in FP4
  (MXFP4 blocks of 32; "Under The Hood: Inkling", quantization);
* ``Lab`` the Router Balance Lab of "Inkling, Dissected" 02g: 64 experts,
  no shared experts, d = 32, 2048 tokens per batch drawn around Zipf-lumpy
  expert home directions, a frozen router, capacity 1.25x, 100 routing
  steps with gamma = 0.01 (routing only: the lab has no expert FFNs, and F
  is a placeholder);
* ``I``  the configuration of "Under The Hood: Inkling" (hidden 6144, expert
  width 3072, gates normalised by logsumexp over log-sigmoids and scaled by
  route_scale = 8 times a global scale; the learned global scale is stood in
  for by 0.8125), at the large batch of ``D``.

No arithmetic of the method lives here.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens in the batch
    d: int                 # hidden size
    F: int                 # expert ffn width (SwiGLU intermediate size)
    E: int = 256           # routed experts
    S: int = 2             # shared experts
    k: int = 6             # routed experts kept per token
    act: str = "bf16"      # dtype of x, y and the expert weights ("f32" or "bf16")
    bias_range: float = 0.05   # balancing bias b ~ U[-bias_range, bias_range]
    wd_std_from_F: bool = False  # W_down ~ N(0, 1/F) instead of N(0, 1/d)
    gamma: float = 1e-3    # bias step size
    skew_kappa: float = 0.0    # router skew strength (workload E only)
    skew_zipf_s: float = 1.2   # exponent of the per-expert router offset
    steps: int = 1         # bias-update steps the workload runs
    gate_norm: str = "ratio"   # "ratio" or "logsumexp"
    gate_scale: float = 1.0    # multiplier of every gate
    capacity_factor: float = 0.0   # per-expert capacity in units of the ideal load (0: none)
    fp4_weights: bool = False      # routed experts' weights in MXFP4
    # Router Balance Lab inputs (tokens around expert "home" directions):
    lab_head_tail: float = 0.0     # home-cluster frequency of expert 0 over expert E-1 (0: off)
    lab_jitter: float = 1.0        # token jitter, in units of the home direction's length
    lab_kappa: float = 4.0         # router weights = lab_kappa * home directions
    extra: dict = field(default_factory=dict)

    @property
    def pairs(self) -> int:
        return self.T * self.k

    def describe(self) -> str:
        return (f"T={self.T} d={self.d} F={self.F} E={self.E}+{self.S} top-{self.k} "
                f"{self.act}")


CONFIGS = {
    "A": MoEConfig("A", T=128, d=512, F=128, act="f32", bias_range=0.1,
                   wd_std_from_F=True),
    "B": MoEConfig("B", T=4096, d=2048, F=768, act="bf16", bias_range=0.05),
    "C": MoEConfig("C", T=64, d=7168, F=2048, act="bf16", bias_range=0.0),
    "D": MoEConfig("D", T=16384, d=7168, F=2048, act="bf16", bias_range=0.05),
    "E": MoEConfig("E", T=16384, d=7168, F=2048, act="bf16", bias_range=0.0,
                   skew_kappa=8.0, steps=100),
    "I": MoEConfig("I", T=16384, d=6144, F=3072, act="bf16", bias_range=0.05,
                   gate_norm="logsumexp", gate_scale=8.0 * 0.8125),
    "Ecap": MoEConfig("Ecap", T=16384, d=7168, F=2048, act="bf16", bias_range=0.0,
                      skew_kappa=8.0, steps=100, capacity_factor=1.25),
    "Lab": MoEConfig("Lab", T=2048, d=32, F=128, E=64, S=0, act="f32", bias_range=0.0,
                     gamma=0.01, steps=100, capacity_factor=1.25, lab_head_tail=30.0),
    "Cfp4": MoEConfig("Cfp4", T=64, d=7168, F=2048, act="bf16", bias_range=0.0,
                      fp4_weights=True),
}


def get(name: str) -> MoEConfig:
    return CONFIGS[name]
