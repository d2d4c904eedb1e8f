"""Windowed-MTP draft attention for MI355X (gfx950): a C-ABI HIP library and its thin binding.

Importing the package loads nothing; ``draft_attention_amd.binding`` loads ``libwmtp.so``.
"""
__all__ = ["binding", "synth"]
