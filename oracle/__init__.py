"""Plain float64 CPU oracle for the TurboQuant KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or executes anything in this package.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, constants or table generators
with ``compressed_kv_cache_tq_amd``: the HIP side builds its own rotation,
sketch and codebook in C++ and the two are compared in the tests.

Sources (cited by page title and section only):

* noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM open-weight su
  Mac", section "Il metodo TurboQuant, in breve": random rotation, optimal
  scalar quantizer per coordinate, distortion within about 2.7x of the
  information-theoretic minimum, data-oblivious and online, and a 1-bit
  quantized Johnson-Lindenstrauss sketch of the residual for unbiased inner
  products.
* same page, section "Cosa aggiunge turboquant-mlx": Lloyd-Max codebook.
* same page, section "I numeri dichiarati": cosine 0.983 (3-bit) / 0.995
  (4-bit) against FP16.
* GitHub issue "Greetings from TurboQuant-MLX & Some Insights to Share!",
  numbered items 1 and 3: attention sink of about 128 uncompressed tokens;
  skipping V dequantization for attention weight below 1e-6.
* NVIDIA forum "Why TurboQuant saves DGX twice": the two stages are a
  polar/rotation quantizer plus a QJL residual correction, online per token,
  unconventional bit widths.

Modules
-------
rng        SplitMix64 integer stream and Box-Muller Gaussians.
rotation   Haar-random orthogonal matrix from a seeded Gaussian via QR.
codebook   Lloyd-Max quantizer for one coordinate of a uniform unit vector.
quantize   norm, rotation, scalar quantization, QJL residual sketch.
pack       bit layouts of the packed cache (per-token records, 32-token tiles).
attend     single-query decode attention read from the packed cache.
parity     the code/attention comparison rules used against the GPU path.

Every function is a parity-pinned step unless its docstring says
"parity unpinned".
"""
