"""Folded multi-branch verify layer (SpecFold) for AMD MI355X.

The compute path is libspecfold.so (hand-written HIP for gfx950, C ABI in
include/specfold.h); `branch_folding_amd._lib` binds it with ctypes and
`branch_folding_amd.runner` marshals device buffers.  Nothing here falls back to a CPU
implementation: calls fail when the library is missing."""
__version__ = "0.1.0"
