"""libaveris: MI355X-native Averis mean-residual split FP4 linear (fwd + dgrad).

The compute path lives in the HIP library built from ``csrc/``; ``averis``
is its thin ctypes binding.  Importing this package loads nothing; the
library is loaded on first use and its absence is an error, never a fallback.
"""

__all__ = ["averis", "workloads"]
