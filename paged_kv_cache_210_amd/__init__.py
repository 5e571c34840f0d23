"""Exact softmax attention over a paged KV cache for AMD MI355X (gfx950).

The compute lives in the C-ABI library ``libpkv.so`` (hand-written HIP kernels);
``paged_kv_cache_210_amd.lib`` is its thin ctypes binding.  Importing the
package does not load the library; ``lib.load()`` does, and raises if it is
missing."""
