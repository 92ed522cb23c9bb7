"""MI355X-native DPO LM-head path: fused completion log-prob sums, sigmoid DPO
loss and head gradients in hand-written HIP for gfx950, behind a C ABI.

Submodules:
  dpo_head   - Python binding of include/dpo_head.h (loads libdpohead.so lazily)
  workloads  - seeded synthetic inputs
  build      - hipcc build of the library
"""
__all__ = ["dpo_head", "workloads", "build"]
