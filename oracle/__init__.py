"""CPU oracle for the wide-beam decode step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (the HIP library and its Python binding)
never imports, links or calls it, and this package imports nothing from the product.

What it computes is the plain definition of the step, not the method's fast route:

* attention: naive softmax attention in float64 over the explicitly concatenated
  prompt + ancestry KV of each beam (xLLM generative-recommendation design doc, §4.2.1
  "KV Cache storage optimisation" and §4.2.2 "Attention compute optimisation": the three
  stages must reproduce exactly this unsplit attention);
* selection: per-beam full stable sort of the trie-valid candidates keeping top_k, then a
  full sort of the beam_width x top_k pool keeping beam_width (same doc, §4.1.1 "model
  input/output characteristics"; FlashRec announcement: illegal semantic IDs are never
  candidates).  Validity is decided from the raw catalog item list, never from a CSR;
* slot-budget batching: first fit in queue order of requests into batches of at most a
  given number of beam rows (FlashRec announcement: scheduling by beam-row slot budget).

Pins (tests/test_oracle_*.py) tie every function to something other than itself:
exhaustive pure-Python enumeration, closed forms, special cases equal to library
routines, and invariants.  No function here is "parity unpinned".
"""
from .numformats import decode_bf16_bits, decode_e4m3fn_bits, decode_stored  # noqa: F401
from .attention import attend_concat, oracle_attention  # noqa: F401
from .select import catalog_prefix_sets, oracle_select, oracle_beam_search  # noqa: F401
from .batching import oracle_plan_batches  # noqa: F401
