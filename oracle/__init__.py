"""CPU oracle for the decode megakernel -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct float64 numpy code that states what one decode step
computes (``decode``), how the step is lowered into 64-byte task descriptors and a CSR
edge array (``graph``), and a CPU interpreter that runs those descriptors in any
dependency-respecting order (``interp``).  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product library never
does, and this package imports nothing from the product package.

Sources: the pages "Mega kernel initial" (1y33.com, sections on the graph API, the
lowering, the task descriptor, the edge array, the buffer table and the OpId table)
and "Megakernels" (runhoid.com, section "Hoid's approach to megakernels").

Parity status per function is listed in each module header.  Choices the pages
leave open (RoPE convention, where RoPE runs, the KV-length convention, the
partial format, one combine per (sequence, KV-head group), activation precision)
are conventions both sides obey; they are "parity unpinned" by the pages and pinned
only by the textbook identities the tests check.
"""
