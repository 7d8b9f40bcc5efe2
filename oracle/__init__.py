"""FP64 CPU oracle for the CSA2 hot path over an FP4 (E2M1 + E4M3/16) KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
``libcsa2.so`` or its Python binding) imports, links or calls this package;
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, tables or helpers with the HIP
path.

What it computes, and where the pages say so (DeepSeek-V4.1-Flash pages):

* ``formats``  -- FP4 E2M1 and E4M3 decoders from their bit fields (the two
  formats ai-maestro.online names in "FP4 KV, Bounded Replay, and other
  extensions" for the main cache and its per-16-channel multipliers).
* ``quant``    -- the per-16-channel quantiser (same section).
* ``indexer``  -- Full-layer indexer (block max over 8-token blocks, top-2,048
  blocks as the candidate pool, Top-512 positions) and the Reindex layer's
  rescoring of the pool (ai-maestro.online, "Compressed Sparse Attention 2";
  wpnews.pro "What is Compressed Sparse Attention 2 CSA2?").
* ``indexer_fp8`` -- the same indexer over real-valued E4M3 keys and queries
  with fp32 scales (the pages leave the indexer's precision open).
* ``swa8``     -- the 8-bit sliding-window cache rows (E4M3 codes, one
  power-of-two scale per row; kongchang.com "Three Core Innovations" gives
  the window cache an 8-bit format).
* ``attention`` -- sparse attention over the selected entries merged with the
  layer's 128-token sliding window in one softmax (ai-maestro.online, "Causal
  Encoder-Decoder architecture" for the window, "Compressed Sparse
  Attention 2" for the per-layer Q and SWA).

Each reading of a point the pages leave open is stated next to the code that
takes it, numbered R1..R31.

Pins (tests/test_oracle_*.py, run with ``-m "not gpu"``): bit-field decoders
against torch's float8_e4m3fn cast and the E2M1 value fixture; the quantiser
against brute-force nearest-value search in exact rational arithmetic; the
indexer against pure-Python brute force and the pool invariant; the FP8
indexer against the integer indexer it reduces to, power-of-two scale closed
forms, exact-rational brute force and the ReLU sign identities; attention
against closed forms and torch's float64 scaled_dot_product_attention.
No function here is "parity unpinned".
"""
from . import formats, quant, indexer, indexer_fp8, attention, swa8  # noqa: F401
