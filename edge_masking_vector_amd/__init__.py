"""edge_masking_vector_amd -- tiled, memory-bound f32 maps, copies and row/column reductions for
AMD Instinct MI355X (gfx950), behind the C-ABI library `tilemap` (include/tilemap.h).

Submodules:
  tilemap  -- ctypes binding to libtilemap.so (same names as the C calls); importing it loads the
              HIP library and fails loudly when it has not been built.
  inputs   -- seeded synthetic inputs (no arithmetic of the method).
  _build   -- the hipcc build of libtilemap.so.
"""
