"""Circulant softmax attention (CAT 1D and BCCB 2D) for MI355X -- package stub."""
