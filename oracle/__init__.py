"""CPU oracle for the VeriCache draft-then-verify hot path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct
numpy implementation (fp64 accumulation) of what the GPU library computes.
Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import or call it; the product path (the HIP library and
its Python binding) never does, and shares no code with it.

Sources (web pages, cited by title and section):

* "Riepilogo Tecnico: VeriCache" (gist.science, paper 2605.17613, Italian
  summary; an Arabic translation of the same summary adds nothing) --
  section "Algoritmo Principale" (draft with the compressed cache, verify all
  drafted tokens in one full-cache pass, accept up to the first mismatch plus
  a bonus token), "Risultati Sperimentali" (output identical to full-KV
  greedy decoding), "Supporto Architetturale" (eviction and quantization
  compressors behind one interface).
* "Riassunto Tecnico: CentroidKV" (gist.science, paper 2506.11418) --
  section "Componenti Chiave", item 4 "Aggregazione" (attention over merged
  centroids adds the cluster degree as a logarithmic term in the softmax;
  centroids are degree-weighted means), item 2 "Pipeline di Inferenza"
  (attention sinks and recent tokens are kept), item 3 "Chunked Soft
  Matching" (chunks, alternating A/B sets, top-r merging of matched pairs).

Modules:

* :mod:`oracle.formats`   -- exact decoding of bf16 / fp16 / packed-int4 storage.
* :mod:`oracle.attention` -- draft (compressed-cache) and verify (block,
  causal) attention, written as the softmax definition.
* :mod:`oracle.accept`    -- greedy argmax and accept-until-first-mismatch.
* :mod:`oracle.quant`     -- the int4 group quantizer of the compressed cache.
* :mod:`oracle.compress`  -- eviction compaction (the kept rows of a cache).
* :mod:`oracle.csm`       -- one Chunked Soft Matching clustering round
  (CentroidKV, "Componenti Chiave" items 1-4).
* :mod:`oracle.tiny`      -- the tiny random-weight decoder, full-KV greedy
  decoding and the VeriCache loop run step by step.

Parity status of each function is stated in its docstring; functions whose
values no test pins to something outside the oracle say "parity unpinned".
"""
