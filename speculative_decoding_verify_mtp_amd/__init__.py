"""MI355X-native multi-token verify step: paged verify attention under chain,
tree or segment masks, greedy acceptance and KV commit.

The compute lives in ``libmtpverify.so`` (hand-written HIP for gfx950) behind
a C ABI; ``lib`` is a thin ctypes binding over it.  Importing the package does
not load the library; ``lib.load()`` does, and fails loudly if it is missing.
"""
__all__ = ["inputs", "lib"]
