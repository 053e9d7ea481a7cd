"""MI355X-native (gfx950) HSTU layer forward: jagged, causally masked pointwise attention.

The compute path is libhstu.so (hand-written HIP kernels behind the C ABI in include/hstu.h);
``ops`` is its thin Python binding.  ``inputs`` and ``configs`` hold the seeded synthetic
workloads.  Importing the package loads nothing: the library is loaded on first use and a
missing library raises.
"""
from . import configs, inputs  # noqa: F401


def __getattr__(name):
    if name == "ops":
        from . import _lib
        return _lib
    raise AttributeError(name)
