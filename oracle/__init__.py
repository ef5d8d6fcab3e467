"""Plain, slow, fp64 CPU oracle for paged GQA decode attention.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library in
``paged_gqa_decode_kv_amd`` never imports, links or calls anything here, and
nothing here imports the HIP library: the two share no code.  The only module
both sides consume is ``workloads`` (seeded input generators, which hold none of
the attention arithmetic).

Every function states the passage of the source pages it follows:

* "LLM inference optimisation guide" (zhengtianqi.github.io), abbreviated
  *Guide*;
* "LLM inference optimisation in depth" (ybb.press/llm/8022), *In-depth*;
* the devpress.csdn.net tutorial on KV Cache / GQA / vLLM PagedAttention,
  *Tutorial*;
* CS336 lecture 10, "Inference optimisation", *Lecture 10*.

Modules
-------
``kvsize``     the KV-cache size formula.
``storage``    exact decoding of the stored element types (fp32, bf16, int8+scale).
``paging``     block-table translation, de-paging, slot-mapped append, gather.
``attention``  attention over the de-paged cache, verify rows, partitions and the
               log-sum-exp merge.
``quant``      the int8 encoding of a block and the quantising append.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, a library routine or numbers printed on the
pages.  None is "parity unpinned".
"""

from . import attention, kvsize, paging, quant, storage  # noqa: F401
