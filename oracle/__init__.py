"""CPU oracle for the dual-flow decode step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 implementation of what the decode path
computes, written from the pages' description of the Dual-Flow Transformer
(Sintesi Tecnica: Dual-Flow Transformers, sections "Architettura Core",
"Meccanismi Chiave" and "Costi di Inferenza vs. Addestramento").

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package. It shares no code with the HIP library: no kernels,
headers, helpers or tables. Its inputs are numpy arrays (bf16 given as uint16
bit patterns); every value is widened exactly to fp64 before any arithmetic.

Functions and their pins (tests/test_oracle_*.py):
  numerics.round_bf16       -- torch's bf16 cast on fp32-exact inputs; hand-derived
                               bit patterns for ties, double-rounding cases, overflow
  attention.decode_attention -- scalar brute force (attention.brute_force), torch
                               SDPA per flow, Q2 = Q1 identities, one-token cache,
                               closed forms, LSE partition merge, paging invariance
  linear.grouped_linear      -- torch.nn.functional.linear per flow, flow independence
  linear.rmsnorm             -- torch.nn.functional.rms_norm
  linear.swiglu_couple       -- torch.nn.functional.silu; b = -1 / b = 0 identities
  cache.kv_append            -- hand-computed slot addresses, bit patterns
  layer.dual_flow_layer      -- textbook pre-norm decoder layer in torch.nn.functional
                               (primary flow), aux = primary identities, cache diff
  step.embed                 -- one-hot matrix product of the tables
  step.dual_flow_step        -- composition of the pinned layer; shared-table / uncoupled
                               aux = primary; primary and caches blind to the aux table
  head.softmax / mixture /   -- torch softmax and argmax; alpha in [1/2, 1], certain primary
       next_token / output_head  -> alpha = 1, flat -> (1 + 1/V) / 2, monotone; Gumbel-max
                               frequencies; torch linear for the projection
  moe.route / moe_mlp        -- torch topk + softmax; equal experts = the dense SwiGLU block
                               composed from the pinned primitives (with b, c and k2 > k1);
                               aux reuses the primary's choice; primary blind to the aux row
  prefill.prefill_attention  -- torch causal SDPA (GQA, cached prefix); prefill_layer = the
       / prefill_layer /       pinned decode layer token by token; chunking invariance; the
       prefill_step            aux started at the last prompt position = aux at every position
  prefill.prefill_dual_      -- torch causal SDPA per flow with Q2 materialised (per-head a);
       attention               primary rows = prefill_attention's; Q2 = Q1 -> O2 = O1
  prefill.prefill_layer_rows -- prefill_layer (from position 0) at the sampled rows, and the
                               keys and values it appends
The placement of the b and c coupling vectors is a reading of the pages (they
name the levels, not the formula); it is pinned only by the identities above:
"parity unpinned" beyond this reading. So is the mixture weight alpha_t = (1 + c_t) / 2
(the pages fix only that it follows the primary's collision probability and stays >= 1/2),
and so are the router-replay readings of moe.py (shared router, the auxiliary's top-k2 taken
from the primary's ranking, softmax over the selected experts, b on shared experts only).
"""
from . import numerics, attention, linear, cache, layer, step, head, moe, prefill  # noqa: F401
