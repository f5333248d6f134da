"""MI355X-native decode step of a Qwen-style decoder stack.

Modules:
  inputs   -- model shapes, workloads and seeded synthetic inputs (no HIP)
  build    -- hipcc build of libatd.so for gfx950
  binding  -- ctypes binding of the C ABI (include/atd.h); loading it
              requires the built library
  device   -- torch-allocated device memory around the binding
  runner   -- decode loops (LM, Talker frames, batched) over the C ABI
"""

__all__ = ["inputs", "build", "binding", "device", "runner"]
