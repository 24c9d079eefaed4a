"""QSA indexer hot path on AMD Instinct MI355X (gfx950).

The compute lives in ``libqsa.so`` (hand-written HIP kernels behind the C ABI of
``include/qsa.h``); ``sparse_attention_indexer_qsa_amd.qsa`` is its thin Python binding and
``sparse_attention_indexer_qsa_amd.workloads`` draws seeded synthetic inputs.  The binding is
loaded on first use so that input generation works on machines without the library.
"""
import importlib

__all__ = ["qsa", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
