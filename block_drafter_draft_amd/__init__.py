"""DFlash2 block-draft-and-verify step for MI355X (gfx950).

The step's five stages are HIP kernels behind the C ABI declared in ``include/dflash2.h``
(``libdflash2.so``). ``block_drafter_draft_amd.dflash2`` is the thin ctypes binding with the
same names; ``workloads`` draws the seeded synthetic inputs. Importing this package loads
nothing; the binding loads the library on first use and fails loudly when it is missing.
"""

__all__ = ["dflash2", "workloads"]


def __getattr__(name):
    if name == "dflash2":
        from . import dflash2 as mod
        return mod
    if name == "workloads":
        from . import workloads as mod
        return mod
    raise AttributeError(name)
