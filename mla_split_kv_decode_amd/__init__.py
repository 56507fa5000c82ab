"""MI355X-native absorbed-MLA split-KV decode.

The compute path is the HIP library ``libmla_decode.so`` built from ``csrc/``
for gfx950; ``binding`` is its thin ctypes wrapper.  The library is loaded on
first use, so importing the package (or ``workloads``) does not need it.
"""

__version__ = "0.1.0"


def __getattr__(name):
    if name in ("binding", "workloads"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
