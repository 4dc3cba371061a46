"""MI355X-native routed sparse causal attention (the Monodratic mixer's hot path).

The compute path is the gfx950 library libmono.so (C ABI in include/mono.h);
`binding` exposes its calls to Python with the same names.  `configs` and
`synth` describe workloads and draw seeded synthetic inputs.  Importing the
package loads nothing; the first call through `binding` loads the library
and raises if it is missing.
"""
from . import configs  # noqa: F401

__all__ = ["configs", "synth", "binding"]
