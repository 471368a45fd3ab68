"""fp64 CPU oracle for the joint text+image DiT attention step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import or run
anything in this package.  The product path (the C-ABI library and its Python
binding) never calls it, and this package imports nothing from the product
path: the two share no kernels, helpers, tables or constants.  The only code
both sides use is the seeded input generator in ``workloads``, which holds none
of the method's arithmetic.

What it computes, each step written from its definition on the pages, in
float64 NumPy, slow and plain:

* ``metadata.build_token_metadata`` -- per-token image-block ids (text = -1),
  target-image mask, rotary positions and the exclusive key bound of each
  query (QwenImage21Transformer2DModel API page, ``build_token_metadata``).
* ``qknorm_rope.rms_norm`` / ``qknorm_rope.rope`` -- per-head RMSNorm of Q and
  K, then rotary embedding over the (frame, height, width) axes or the
  Lumina 2D split (NucleusMoE-Image pipeline article, section 6.3; Lumina-Next
  DiT article, configuration table and section 4).
* ``qknorm_rope.layer_norm_across_heads``, the ``linear_factor`` /
  ``ntk_factor`` of ``rope`` and ``qknorm_rope.time_aware_rope_factors`` --
  the Lumina-Next variants: LayerNorm over all heads' channels, and the
  rotary table rescaled per denoising step (Lumina-Next DiT article,
  sections 3 and 4).
* ``attention.attention`` -- softmax attention under the full mask or the
  block-causal rule "q_idx >= kv_idx or same image block", with GQA and an
  optional cached K/V prefix (QwenImage21Transformer2DModel API page, the
  block-causal and causal_condition notes and ``forward``'s kv_cache modes).
* ``attention.attention_multipass`` -- the same masked attention computed
  segment by segment (one pass per text run or image block), the second,
  independent implementation of the mask that the page says gives the same
  result.
* ``attention.attention_bruteforce`` -- quadruple Python loops, tiny inputs.
* ``key_padding.joint_key_valid`` -- the per-sample text mask
  (``encoder_hidden_states_mask``) laid over the joint sequence as per-key
  validity, which ``attention`` and ``attention_bruteforce`` take as
  ``key_valid`` (QwenImage21Transformer2DModel API page, ``forward``).

* ``pipeline.step`` / ``pipeline.extract_cache`` -- the composed step
  (norm and rotation of the query tokens at their logical positions, then the
  masked attention) in the full and the cached form, and the "extract" mode's
  cache (QwenImage21Transformer2DModel API page, forward's kv_cache modes).

* ``cfg.norm_rescaled_cfg`` -- classifier-free guidance whose mixed
  prediction is rescaled, token by token, to the norm of the conditional one
  (NucleusMoE-Image pipeline article, section 4.3).

Pins: every function is pinned by tests under ``tests/`` that do not re-type
its formula: closed forms, invariants (rotation preserves norms, relative
phase), textbook special cases checked against library routines
(``torch.nn.functional.scaled_dot_product_attention`` in float64 on the CPU),
single-pass == multi-pass, cached rows == full rows, brute force on tiny
inputs, and hand-derived token-metadata fixtures under ``tests/golden``.
The pages print no numeric worked example for this step, so no pin is a
printed value; none of the functions is left unpinned.
"""
from . import metadata, qknorm_rope, attention, pipeline, key_padding, cfg  # noqa: F401
