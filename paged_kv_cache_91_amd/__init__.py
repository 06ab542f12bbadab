"""MI355X-native paged KV-cache decode path.

Submodules:

* ``paged_kv_cache_91_amd.pa`` -- the Python binding of the HIP library
  ``libpa.so`` (``pa_write_kv``, ``pa_decode``, ``pa_copy_blocks``); loading
  it fails loudly when the library has not been built;
* ``paged_kv_cache_91_amd.allocator`` -- the host block manager that feeds
  block tables, slot mappings and copy-on-write pairs;
* ``paged_kv_cache_91_amd.workloads`` -- seeded synthetic inputs.
"""

__all__ = ["pa", "allocator", "workloads"]
