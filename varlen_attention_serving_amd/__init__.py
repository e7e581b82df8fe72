"""Unified paged attention for MI355X (gfx950): a HIP kernel family behind the
C boundary of ``include/ua.h``.

``binding`` mirrors that boundary with ctypes (argument marshalling only);
``device`` holds torch-side memory plumbing; ``workloads`` draws seeded
synthetic inputs; ``build`` compiles ``libua.so``.  Importing ``binding``
raises if the library has not been built.
"""
__all__ = ["binding", "device", "workloads", "build"]
