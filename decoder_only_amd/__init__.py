"""q3: a Qwen3-0.6B-shaped decoder inference engine for AMD Instinct MI355X (gfx950).

The engine is the HIP library ``libq3.so`` behind the C ABI in ``include/q3.h``;
``decoder_only_amd.q3`` is its Python binding (ctypes; torch supplies device
memory and the stream). Build with ``python -m decoder_only_amd.build``.
"""
from . import q3  # noqa: F401
from .q3 import Engine, Q3Error, config, load_library  # noqa: F401
