"""MI355X-native self-conditioning soft embedding (DiffusionGemma).

Submodules
----------
api        tensor-level calls (row statistics, probability slice, soft embedding)
_binding   ctypes binding of libsoftembed.so, one Python function per C entry point
workloads  seeded synthetic inputs
build      hipcc build of libsoftembed.so

``api`` and ``_binding`` load the HIP library on import and raise if it is
missing; ``workloads`` and ``build`` do not need it.
"""
__version__ = "0.1.0"
