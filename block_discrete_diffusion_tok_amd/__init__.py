"""Block-diffusion denoising step on MI355X (gfx950).

``dg``     ctypes binding of the C-ABI library libdg.so (include/dg.h,
           include/dg_ops.h); the library is loaded on first use.
``synth``  seeded synthetic inputs (weights, cached K/V, canvas state).
``build``  hipcc build of libdg.so.
"""
__all__ = ["dg", "synth", "build"]
