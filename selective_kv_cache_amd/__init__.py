"""selective_kv_cache_amd: the link step of position-independent KV reuse
(CacheSlide weighted-correction recompute, EPIC LegoLink) on AMD MI355X.

  _lib   - ctypes binding of libkvb.so (the C ABI in include/kvb.h)
  link   - host orchestration of the compile and link steps (LinkEngine)
  build  - in-tree hipcc build of libkvb.so for gfx950
"""
__all__ = ["_lib", "link", "build"]
