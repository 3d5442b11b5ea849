"""Oracle: a plain, slow, fp64 CPU statement of the video-DiT block hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import or run anything here.  The
product path (the HIP library and its Python binding) never calls it and has
no CPU fallback.  The oracle shares no code with the HIP path: it imports
nothing from the package, and the package imports nothing from here.

Each function writes out the plain definition of what the step computes:

* ``adaln.adaln_modulate``   per-token AdaLN modulation (two-pass LayerNorm)
* ``adaln.adaln_modulate_per_sample``  one modulation row per sample
* ``rope3d.rope3d_apply``    3D RoPE as complex multiplication per band
* ``attention.attention``    naive softmax(Q K^T * scale) V, whole score row
* ``attention.attention_rope`` RoPE on Q and K, then attention
* ``attention.attention_masked``  attention with a padded key range left out
* ``attention.merge_lse``    two partial attentions over disjoint key sets,
  combined through their log-sum-exps

All arithmetic is in float64.  Inputs may be float32 arrays holding the
exact values the device sees (bf16 inputs widened exactly); they are upcast
to float64 here.

Pins (see the ``-m "not gpu"`` tests): LayerNorm against
``torch.nn.functional.layer_norm`` and closed-form rows; RoPE against
closed-form angles, norm preservation and relative-offset invariance;
attention against ``torch.nn.functional.scaled_dot_product_attention``,
``scipy.special.logsumexp`` and closed forms.  The choice of 3D-RoPE family
convention (band order, pairing, per-band frequencies) is a reading of the
pages, which give no formula: against any particular model family the RoPE
convention is parity unpinned; the invariants pin everything else.
"""
from .adaln import adaln_modulate, adaln_modulate_per_sample, layer_norm
from .rope3d import token_positions, rope_angles, rope3d_apply
from .attention import attention, attention_masked, attention_rope, merge_lse

__all__ = [
    "adaln_modulate", "adaln_modulate_per_sample", "layer_norm", "token_positions", "rope_angles",
    "rope3d_apply", "attention", "attention_masked", "attention_rope", "merge_lse",
]
