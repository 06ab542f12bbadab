"""Float64 CPU oracle for the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct statement of what the GPU library computes.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP library and its Python binding) never
imports, links or calls anything here, and this package imports nothing from
the product.

Pages cited (by title and section; see each function's docstring):

* [ZC] ya.zerocoder.ru, "Что такое PagedAttention" -- sections on the
  block/table mechanism, the worked trace and the structural-vs-factual checks.
* [VL] vasteelab.pages.dev, "PagedAttentionとは？LLMのKV Cacheをblock単位で管理する"
  -- sections on fixed-length blocks, last-block waste, kernel + memory
  manager, Copy-on-Write.
* [GC] gufacode.com/vllm/chapter2, "PagedAttention:KV cache 的页表革命" --
  sections on the mapping, on-demand allocation, prefix sharing, pool size and
  the PagedAttention kernel pseudocode.
* [PD] paweldubiel.com notes, "PagedAttention" -- sections "Mecanismo y
  detalles" and "El orden del texto no es la dirección de memoria".
* [UL] ultralytics.com glossary, "PagedAttention" -- sections on how paging
  works (with the PyTorch pool example), block sharing, related techniques.

Parity status: every function here is pinned by a CPU test to something other
than itself (worked examples printed on the pages, closed forms, brute force,
a library routine on a special case, or the format definition).  None is
"parity unpinned".
"""

from .pa_oracle import (  # noqa: F401
    DTYPES,
    E4M3_MAX,
    e4m3_table,
    e4m3_encode,
    to_float64,
    gather_kv,
    gather_kv_range,
    window_start,
    oracle_decode,
    oracle_prefill,
    oracle_swap,
    oracle_partials,
    oracle_lse_merge,
    oracle_write,
    oracle_copy,
    blocks_needed,
    unused_slots,
    kv_bytes_per_block,
    pool_blocks,
)
