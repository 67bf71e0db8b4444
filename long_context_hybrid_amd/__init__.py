"""HySparse hybrid-block attention for one MI355X (gfx950).

The compute path is the C-ABI library ``libhysparse.so`` (hand-written HIP);
``long_context_hybrid_amd.hysparse`` is its thin ctypes binding.  Importing this
package does not load the library; ``inputs`` is the seeded input generator.
"""
__all__ = ["inputs", "hysparse"]
