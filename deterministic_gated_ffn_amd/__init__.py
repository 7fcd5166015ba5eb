"""Deterministic gated FFN for AMD Instinct MI355X (gfx950)."""
