"""CPU oracle for the SwitchSD copy-speculation step — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct float64 restatement of what the
copy path computes, written from the SwitchSD pages ("To Copy or Not to Copy:
Controlling Speculative Decoding via Intrinsic Model Signals", arXiv 2609.20186,
and its write-up).  It exists to check the HIP path; it is not part of it.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``copy_draft_verification_amd``)
never imports, calls or links anything here, and this package imports nothing
from the product path: the two share no kernels, helpers, tables or
pre/post-processing.  The only module both sides read is the seeded input
generator ``workloads``, which holds none of the method's arithmetic.

Modules, one per step of the copy path:

* ``probe``   – copy-intent probe score and the probe half of the gate.
* ``kgram``   – kappa-gram suffix match, recency-ordered top-W, candidate gather.
* ``attention`` – block-triangular attention over prefix + own candidate.
* ``lmhead``  – LM-head logits and greedy (T=0) argmax with top-2 margin.
* ``accept``  – longest accepted continuation and the token after it.
* ``commit``  – copying the accepted rows' K/V into the cache, extending the context.
* ``calibration`` – copy-mode labels, batched probe logits, F1-optimal threshold, ROC AUC.
* ``sampling`` – verification at T > 0: candidate trie, recursive rejection with
  point-mass drafts, Gumbel-max residual draws from Philox4x32-10.
* ``forward`` – the verification pass as a full target forward: embedding, decoder
  layers (RMSNorm, projections, RoPE at positions n-1 / n+j, block-triangular
  attention, SwiGLU MLP), final norm and LM head.
* ``bf16``    – exact widening of bfloat16 bit patterns to float64.

Every function states the passage it follows.  Readings of points the pages
leave open are stated where they are used.  Parity pins for every function live
in ``tests/test_oracle_*.py``; no function here is "parity unpinned".
"""

from .bf16 import bf16_bits_to_f64
from .probe import probe_score, logit
from .kgram import kgram_matches, kgram_retrieve
from .attention import allowed_keys, blocktri_attention
from .lmhead import lm_logits, argmax_with_margin, lmhead_argmax
from .accept import accept_longest
from .commit import commit_accepted
from .calibration import copy_labels, probe_logits, threshold_sweep, calibrate
from .sampling import candidate_trie, philox, sample_step, sample_verify
from .forward import decoder_layer, verify_forward

__all__ = [
    "bf16_bits_to_f64", "probe_score", "logit", "kgram_matches", "kgram_retrieve",
    "allowed_keys", "blocktri_attention", "lm_logits",
    "argmax_with_margin", "lmhead_argmax", "accept_longest", "commit_accepted", "copy_labels",
    "probe_logits", "threshold_sweep", "calibrate", "candidate_trie", "philox", "sample_step",
    "sample_verify", "decoder_layer", "verify_forward",
]
