"""Mamba-3 SSM sequence mixer on MI355X (gfx950): Python binding package."""
