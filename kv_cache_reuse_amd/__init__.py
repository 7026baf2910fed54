"""MAC-Attention decode step on AMD MI355X (gfx950).

The compute path is the HIP library ``libmac.so`` built from ``csrc/``; this
package holds its build script and a ctypes binding (``binding``) whose
functions carry the C entry points' names.
"""

__all__ = ["binding", "build"]
