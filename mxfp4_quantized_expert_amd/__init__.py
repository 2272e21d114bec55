"""MI355X-native MXFP4 mixture-of-experts expert FFN (gfx950 HIP kernels behind a C ABI).

Submodules:
  binding   -- ctypes binding of libmxfp4moe.so (mxfp4_dequantize, moe_mxfp4_route,
               moe_mxfp4_forward); argument marshalling only.
  workloads -- seeded synthetic layers (inputs only, no arithmetic of the method).

Importing the package loads nothing; ``binding.load()`` loads the HIP library
and raises if it has not been built.
"""

__all__ = ["binding", "workloads"]
