"""kimi_k3_attention_amd: the Kimi-K3 attention-residual forward on AMD MI355X.

    from kimi_k3_attention_amd import attnres   # loads libattnres.so (HIP)
    from kimi_k3_attention_amd import workloads # seeded synthetic inputs

The binding is imported lazily so that the workload generator can be used
without the built library; the binding itself refuses to import when the
library is missing (there is no CPU fallback).
"""

__all__ = ["attnres", "workloads", "build"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
