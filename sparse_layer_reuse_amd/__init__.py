"""MI355X-native HyLRA decode-phase hybrid attention.

Submodules:
  hylra      -- ctypes binding of the C-ABI library ``libhylra.so`` (the HIP path)
  workloads  -- named decode workloads (shapes, policies, planted structure)
  synth      -- seeded synthetic input generators (no attention arithmetic)
  build      -- hipcc build of ``libhylra.so``

Importing the package loads nothing native; ``sparse_layer_reuse_amd.hylra``
loads the library and raises if it is missing.
"""
__version__ = "0.1.0"
