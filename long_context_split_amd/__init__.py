"""libhysparse: HySparse2 hybrid-block attention for MI355X (gfx950).

The compute path is the HIP library behind include/hysparse.h; `hysparse` is
its ctypes binding and `build` compiles it.
"""
