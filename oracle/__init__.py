"""fp64 CPU oracle for exact attention (test infrastructure only; see attention.py)."""
from .attention import (attention_forward, attention_forward_backward, default_scale,
                        group_forward_backward, head_backward, head_forward,
                        relative_frobenius, tiled_forward, tiled_head_forward, visible)

__all__ = ["attention_forward", "attention_forward_backward", "default_scale",
           "group_forward_backward", "head_backward", "head_forward", "relative_frobenius",
           "tiled_forward", "tiled_head_forward", "visible"]
