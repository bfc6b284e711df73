"""MI355X (gfx950) tiled 3D Gaussian-splatting rasterizer.

The compute lives in a HIP C-ABI library (``csrc/``, header ``include/gs.h``);
``gaussian_splatting_tile_amd.binding`` marshals torch device tensors into it.
"""
