"""Conversions between the d_k x d_v state matrix S and the library's state layout.

The library stores each head's state as S^T, [d_v][d_k] row-major, so that column j of S
(the key-space vector of value channel j) is contiguous: it is both the MFMA operand
fragment the verify kernel loads and the unit the commit kernel updates.
"""
import torch


def state_from_math(S: torch.Tensor) -> torch.Tensor:
    """[..., d_k, d_v] -> contiguous [..., d_v, d_k]."""
    return S.transpose(-1, -2).contiguous()


def state_to_math(St: torch.Tensor) -> torch.Tensor:
    """[..., d_v, d_k] -> contiguous [..., d_k, d_v]."""
    return St.transpose(-1, -2).contiguous()
