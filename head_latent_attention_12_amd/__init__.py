"""Absorbed Multi-head Latent Attention decode for MI355X (gfx950)."""
