"""Reproducible floating-point add-reductions for AMD Instinct MI355X (gfx950)."""
