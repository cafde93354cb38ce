"""MI355X-native H2O chunk step: GQA attention over a fixed-capacity KV cache
with exact summed attention weights, H2O score update, bottom-T eviction with a
replay log, and int8/int4 cache buffers.

The compute runs in the HIP library ``libh2o.so`` (C ABI, see include/h2o.h);
this package only marshals arguments to it.  Import ``h2o_kv_cache_sdpa_amd.api``
(or use the names re-exported lazily here) to load the library.
"""

__all__ = ["api", "cache", "workloads"]


def __getattr__(name):
    if name in ("api", "cache"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
