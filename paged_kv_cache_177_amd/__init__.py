"""MI355X (gfx950) paged decode attention: a C-ABI HIP library plus a thin ctypes binding.

Importing the package is cheap: the shared library is loaded on first use of the binding.
"""
