"""MI355X (gfx950) packed NR-MMDiT block and rectified-flow wrapper.

Submodules:
  binding    -- ctypes binding of libmmdit.so (the HIP library); importing it
                loads the library and fails loudly if it is not built
  build      -- hipcc build of libmmdit.so in-tree
  configs    -- model widths and packed-batch workloads
  synthetic  -- seeded synthetic inputs (no arithmetic of the method)
  runner     -- device-side helpers that drive whole forward passes through
                the binding (training forward + loss, packed-CFG sampler)
"""
