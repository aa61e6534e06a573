"""Block-sparse self-attention with summary rows for gfx950 (MI355X)."""
