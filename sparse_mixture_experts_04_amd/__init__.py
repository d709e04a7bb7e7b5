"""MI355X-native forward pass of a DeepSeek-V3-lineage MoE feed-forward layer.

The compute lives in ``libmoe.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/moe.h``); ``sparse_mixture_experts_04_amd.ops`` is the
thin torch-facing binding.  ``configs`` and ``synth`` describe and generate
the synthetic workloads and need no GPU.
"""
import importlib

__all__ = ["configs", "synth", "ops"]


def __getattr__(name):
    if name == "ops":
        return importlib.import_module("._lib", __name__)
    if name in ("configs", "synth"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
