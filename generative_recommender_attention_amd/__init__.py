"""libhstu: HSTU attention over packed variable-length sequences on MI355X (gfx950).

The compute path is the C-ABI shared library ``libhstu.so`` built from the HIP
sources in ``csrc/``; ``hstu`` is its thin Python binding (argument marshalling
only).  ``workloads`` draws the seeded synthetic inputs.
"""

__all__ = ["hstu", "workloads"]
