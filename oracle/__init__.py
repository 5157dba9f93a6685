"""CPU oracle for the ragged, confidence-driven verify step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
calls it, and this package imports nothing from the product path.

The oracle is a plain, slow restatement of what the verify step computes, in
fp64 (floating point) and exact Python integers, written from the pages:

* "DSpark in SGLang: Speculative Decoding with Confidence-Driven,
  Variable-Length Verification" (papercache.org summary of the LMSYS blog,
  called *the DSpark-in-SGLang page* below), sections 速读, A2, A3;
* the lshu.cn DSpark explainer (*the explainer page*), sections 1.2, 2.3, 3.3,
  used only for the generic speculative-decoding accept rules.

Five stages, one module each:

=====================  ======================================================
``schedule``           survival products, cost model, per-request windows
``pack``               front-packing into a cu_seqlens buffer + tier rounding
``attention``          varlen causal verify attention over a paged KV cache
``lm_head``            target LM-head logits and argmax
``accept``             greedy / min(1,p/q) acceptance, cap-accept ceiling
``scatter``            compact scatter of committed tokens and KV slots
``dense``              fixed-shape padded verify (the static-graph baseline)
``cost_fit``           least-squares fit of the step-time model's table
``calibration``        per-request confidence statistics and ECE
``estimator``          block-accept estimator of the ceiling truncation hides
=====================  ======================================================

Every array argument is a numpy array; bf16 inputs arrive as their exact
values widened to float32/float64 by the caller.
"""

from .schedule import (STATIC, COMPACT, CAP_ACCEPT, NO_TRIM, FIXED_SHIFT,
                       survival, step_time, schedule)
from .pack import pack, select_tier
from .attention import verify_attention, attention_row
from .lm_head import lm_head_logits, lm_head_pred
from .accept import (GREEDY, REJECTION, accept_greedy, accept_rejection,
                     residual_sample)
from .scatter import compact_scatter
from .dense import dense_padded_verify
from .cost_fit import fit_cost_model, cost_tables
from .calibration import calibration
from .estimator import new_state as estimator_state, estimate_update, open_interval

__all__ = [
    "STATIC", "COMPACT", "CAP_ACCEPT", "NO_TRIM", "FIXED_SHIFT",
    "survival", "step_time", "schedule", "pack", "select_tier",
    "verify_attention", "attention_row", "lm_head_logits", "lm_head_pred",
    "GREEDY", "REJECTION", "accept_greedy", "accept_rejection",
    "residual_sample", "compact_scatter", "dense_padded_verify",
    "fit_cost_model", "cost_tables", "calibration",
    "estimator_state", "estimate_update", "open_interval",
]
