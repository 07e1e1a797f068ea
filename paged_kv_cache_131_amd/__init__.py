"""Paged decode attention for MI355X (gfx950).

The compute path is the C-ABI library `libpagedattn.so` (HIP kernels,
declared in include/pagedattn.h); `paged_kv_cache_131_amd.binding` marshals
torch tensors into its calls. `block_manager` is the host-side block
allocator that produces block tables, slot mappings and copy lists;
`workloads` draws seeded synthetic inputs.

Importing this package loads nothing; the library is loaded on first use of
the binding and a missing library is an error, never a fallback.
"""

__all__ = ["binding", "block_manager", "workloads"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
