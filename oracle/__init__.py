"""CPU oracle for the chunked ring-attention and Ulysses layout path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The HIP
library and its Python binding never import this package, and this package
imports nothing from them: the two sides share no code.  Inputs reach both
sides from the seeded generators in ``sequence_kv_chunk_amd.synth`` (which hold
no attention, merge or layout arithmetic); the oracle itself only sees float64
(or raw integer) arrays.

Everything is plain numpy in float64, written for a reader to check against
the pages by eye:

* ``attention``  -- full (non-chunked) softmax attention, the definition the
  chunked method must reproduce exactly up to rounding (also at explicit
  positions, and over packed samples that must not see each other);
* ``ring``       -- the online-softmax / log-sum-exp merge and the ring visit
  over resident chunks, as a self-check of the merge semantics against the full
  definition;
* ``ulysses``    -- the sequence<->head all-to-all as an explicit index copy,
  including GQA key/value head replication;
* ``backward``   -- the gradients of softmax attention (dQ, dK, dV) and one
  chunk pair's share of them given the rows' full log-sum-exp;
* ``zigzag``     -- the zigzag split of the sequence over ring ranks and the
  causal attention of one rank's shard under it;
* ``closed_form``-- the materialised attention-matrix memory formula.

Sources (the pages):
  [RA]  Ring-attention Q&A "Как работает sequence parallelism в контексте LLM?"
        (aivaro.ru, answer 425).
  [UL]  "Метод контекстного параллелизма Ulysses" (Telegram channel stuffynlp,
        post 213).
  [HF]  "Paralelismo de secuencias en 🤗 accelerate" (accelerate concept guide).

Pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
facts other than itself (brute-force loops, closed forms, library routines,
the pages' printed figure); ``tests/test_oracle_mutants.py`` shows that
plausible mistakes fail those pins.  No function is left "parity unpinned".
"""
from .attention import (attention_fp64, attention_at_positions_fp64, attention_packed_fp64, segment_ids,
                        unmasked_pairs)
from .ring import lse_merge_fp64, ring_attention_fp64, ring_visit_order
from .ulysses import (seq_to_head_naive, head_to_seq_naive, replicated_head_source,
                      check_ulysses_shapes)
from .closed_form import attn_matrix_bytes
from .backward import attention_bwd_fp64, chunk_attention_bwd_fp64, rowsum_do_o_fp64
from .zigzag import zigzag_positions, zigzag_shard, zigzag_attention_fp64, zigzag_block_classes

__all__ = [
    "attention_fp64", "attention_at_positions_fp64", "attention_packed_fp64", "segment_ids", "unmasked_pairs",
    "lse_merge_fp64", "ring_attention_fp64", "ring_visit_order",
    "seq_to_head_naive", "head_to_seq_naive", "replicated_head_source",
    "check_ulysses_shapes",
    "attn_matrix_bytes",
    "attention_bwd_fp64", "chunk_attention_bwd_fp64", "rowsum_do_o_fp64",
    "zigzag_positions", "zigzag_shard", "zigzag_attention_fp64", "zigzag_block_classes",
]
