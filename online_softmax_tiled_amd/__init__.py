"""Exact tiled softmax attention (FlashAttention-style forward) for MI355X."""
