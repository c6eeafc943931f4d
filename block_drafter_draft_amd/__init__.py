"""DFlash2 block-draft-and-verify step for MI355X (gfx950).

The step's five stages are HIP kernels behind the C ABI declared in ``include/dflash2.h``
(``libdflash2.so``). ``block_drafter_draft_amd.dflash2`` is the thin ctypes binding with the
same names; ``workloads`` draws the seeded synthetic inputs. Importing this package loads
nothing; the binding loads the library on first import and fails loudly when it is missing.
"""
import importlib

__all__ = ["dflash2", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
