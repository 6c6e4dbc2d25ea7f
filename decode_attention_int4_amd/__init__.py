"""MI355X (gfx950) ResidualQuant KV cache: quantize-append, reconstruct and fused
decode attention over INT4-anchor / INT2-residual looped-Transformer caches.

The compute lives in the HIP library ``librq.so`` (C ABI declared in
``include/rq.h``); this package only marshals arguments into it.
"""
