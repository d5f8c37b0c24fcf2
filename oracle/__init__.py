"""Plain, slow fp64 CPU oracle for Dynamic Bifocal RoPE attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or helper with the HIP library, and it imports nothing from it.

Every function follows a passage of the pages about Jet-Long (arXiv 2607.07740),
cited by page and section:

* ResearchPod summary (researchpod.app), 2nd paragraph: nearby keys keep the
  base RoPE; distant positions are folded onto a coarser grid whose step is the
  least integer that holds every folded position inside the trained range; three
  FlashAttention-style passes are combined by inclusion-exclusion.
* ResearchPod transcript, the exchange on the cache: every key stays in the cache
  at the position it was written at; the folding is applied when it is read.
* ResearchPod transcript, the exchange on prefill: the result is built from the
  near keys at base positions, all keys at folded positions, and the near keys
  at folded positions.
* Abstract (engineersofai.com paper page): the base model is recovered exactly at
  short inputs; the merge and the rotation to folded positions run inside the
  attention kernel.
* seventnews.com, "How bifocal attention sidesteps the fixed-scaling trap": the
  long-range factor follows the length s of the sequence at hand; the merge
  joins the branches so that no key is counted twice.

* seventnews.com, "Empirical results that challenge the status quo": the method
  runs inside Qwen3 models (1.7B, 4B, 8B) at up to 128K; ``oracle.layer`` states
  one attention layer of them.

Parity status of each function is listed in the module docstrings of
``oracle.bifocal`` and ``oracle.layer``.
"""

from .bifocal import (  # noqa: F401
    group_factor,
    rope_frequencies,
    rotate_half_pairs,
    rotation_matrix,
    aliased_position,
    correction_offset,
    query_positions,
    plain_causal_attention,
    bifocal_three_pass,
    bifocal_bruteforce,
    bifocal_decode,
    bifocal_decode_varlen,
    plain_decode_varlen,
    bifocal_prefill_varlen,
    gather_pages,
    bifocal_decode_paged,
    sliding_window_attention,
    SCHEDULES,
    seam_group_factor,
    fractional_factor,
    long_range_schedule,
    merge_passes,
)
from .layer import qwen3_attention_layer, rms_norm_heads  # noqa: F401
