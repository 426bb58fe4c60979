"""Unmerged multi-LoRA (SGMV / BGMV) for AMD MI355X (gfx950)."""
