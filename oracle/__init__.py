"""fp64 CPU oracle for 3D-RoPE full / Skiparse attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from .core import (MODES, attn3d, attn3d_bwd, attn3d_packed, latent_grid, packed_segments,
                   rope3d, rope3d_transpose, skiparse_groups, skiparse_index, softmax_attention,
                   softmax_attention_bwd, video_coords)

__all__ = ["MODES", "attn3d", "attn3d_bwd", "attn3d_packed", "latent_grid", "packed_segments",
           "rope3d", "rope3d_transpose", "skiparse_groups", "skiparse_index", "softmax_attention",
           "softmax_attention_bwd", "video_coords"]
