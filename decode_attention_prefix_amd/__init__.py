"""Prefix-aware paged decode attention for MI355X (gfx950).

The public API is the C ABI in include/kvattn.h; `kvattn` is its ctypes
binding with the same function names.  Importing this package does not load
the library; importing `decode_attention_prefix_amd.kvattn` does, and fails
loudly when libkvattn.so is not built.
"""
__all__ = ["kvattn", "build"]
