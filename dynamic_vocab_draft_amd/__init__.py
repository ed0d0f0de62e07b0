"""Dynamic-vocabulary draft LM head for AMD MI355X (gfx950).

Submodules:
  nanospec   -- ctypes binding of libnanospec.so (the HIP path; loads the library)
  workloads  -- seeded synthetic inputs (no method arithmetic)
  build      -- hipcc build of libnanospec.so
"""
__all__ = ["nanospec", "workloads", "build"]
