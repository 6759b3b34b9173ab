"""MI355X-native owner-side Muon step (libdmuon_ns).

Submodules:
  dmuon_ns   -- ctypes binding of the C ABI (loads libdmuon_ns.so; no fallback)
  workloads  -- seeded synthetic workloads (shapes, dtypes, distributions)
  build      -- hipcc build of libdmuon_ns.so for gfx950

Importing the package itself loads nothing; import ``dmuon_ns`` to use the
library.
"""

__version__ = "0.1.0"
