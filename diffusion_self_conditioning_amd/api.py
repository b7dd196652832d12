"""Tensor-level calls of libsoftembed.

Each function allocates its outputs with torch on the input's device and calls
the C entry point of the same family through the ctypes binding; all arithmetic
runs in the library's HIP kernels.
"""
from __future__ import annotations

import torch

from ._binding import (SoftEmbedError, se_merge_slices, se_probs_bf16,  # noqa: F401
                       se_quantize_table_fp8, se_row_stats, se_soft_embed, se_soft_embed_fp8,
                       se_soft_embed_fp8_fused, se_soft_embed_fused, se_soft_embed_onepass,
                       se_soft_embed_onepass_workspace_bytes, se_soft_embed_staged,
                       se_soft_embed_step, se_soft_embed_step_fp8, se_soft_embed_step_onepass,
                       se_soft_embed_step_onepass_fp8, se_soft_embed_step_onepass_workspace_bytes,
                       se_soft_embed_staged_workspace_bytes, se_soft_embed_workspace_bytes,
                       se_status_string, se_version)


def row_stats(logits: torch.Tensor, stream=None):
    """(row_max, row_lse, row_entropy, row_argmax) of fp32 logits [L, V] over the full width."""
    n = logits.shape[0]
    f = dict(device=logits.device, dtype=torch.float32)
    mx, lse, ent = torch.empty(n, **f), torch.empty(n, **f), torch.empty(n, **f)
    am = torch.empty(n, device=logits.device, dtype=torch.int32)
    se_row_stats(logits, mx, lse, ent, am, stream=stream)
    return mx, lse, ent, am


def probs_bf16(logits, row_lse, vocab_start, vocab_end, stream=None):
    """bf16 probability matrix [L, V] (a view of a buffer whose row pitch is V rounded up to
    8, as se_probs_bf16 requires); only columns [vocab_start, vocab_end) are written."""
    n, v = logits.shape
    p = torch.zeros((n, (v + 7) // 8 * 8), device=logits.device, dtype=torch.bfloat16)[:, :v]
    se_probs_bf16(logits, row_lse, vocab_start, vocab_end, p, stream=stream)
    return p


def workspace(n_rows, vocab_start, vocab_end, d, device):
    nbytes = se_soft_embed_workspace_bytes(n_rows, vocab_start, vocab_end, d)
    return torch.empty((nbytes + 3) // 4, device=device, dtype=torch.float32) if nbytes else None


def staged_workspace(n_rows, vocab_start, vocab_end, d, device):
    nbytes = se_soft_embed_staged_workspace_bytes(n_rows, vocab_start, vocab_end, d)
    return torch.empty((nbytes + 3) // 4, device=device, dtype=torch.float32) if nbytes else None


def soft_embed(logits, row_lse, vocab_start, vocab_end, w_shard, gamma, *, fused=True,
               out=None, ws=None, stream=None, staged=False):
    """gamma * softmax(logits)[:, s:e] @ w_shard[: e - s]: one rank's partial, fp32 [L, d].
    ``staged=True`` runs se_soft_embed_staged (same result as the fused call)."""
    n, d = logits.shape[0], w_shard.shape[1]
    if out is None:
        out = torch.empty((n, d), device=logits.device, dtype=torch.float32)
    if staged:
        if ws is None:
            ws = staged_workspace(n, vocab_start, vocab_end, d, logits.device)
        se_soft_embed_staged(logits, row_lse, vocab_start, vocab_end, w_shard, gamma, out, ws,
                             stream=stream)
        return out
    if ws is None:
        ws = workspace(n, vocab_start, vocab_end, d, logits.device)
    if fused:
        se_soft_embed_fused(logits, row_lse, vocab_start, vocab_end, w_shard, gamma, out, ws,
                            stream=stream)
    else:
        p = probs_bf16(logits, row_lse, vocab_start, vocab_end, stream=stream)
        se_soft_embed(p, vocab_start, vocab_end, w_shard, gamma, out, ws, stream=stream)
    return out


def quantize_table_fp8(w, stream=None):
    """(codes uint8 [rows, d], row_scale fp32 [rows]): the e4m3 form of a bf16 table."""
    rows, d = w.shape
    codes = torch.empty((rows, d), device=w.device, dtype=torch.uint8)
    scale = torch.empty(rows, device=w.device, dtype=torch.float32)
    se_quantize_table_fp8(w, codes, scale, stream=stream)
    return codes, scale


def soft_embed_fp8(logits, row_lse, vocab_start, vocab_end, w_codes, w_scale, gamma, *,
                   fused=True, out=None, ws=None, stream=None):
    """soft_embed with the shard in e4m3 form (codes [rows, d], power-of-two row scales)."""
    n, d = logits.shape[0], w_codes.shape[1]
    if out is None:
        out = torch.empty((n, d), device=logits.device, dtype=torch.float32)
    if ws is None:
        ws = workspace(n, vocab_start, vocab_end, d, logits.device)
    if fused:
        se_soft_embed_fp8_fused(logits, row_lse, vocab_start, vocab_end, w_codes, w_scale, gamma,
                                out, ws, stream=stream)
    else:
        p = probs_bf16(logits, row_lse, vocab_start, vocab_end, stream=stream)
        se_soft_embed_fp8(p, vocab_start, vocab_end, w_codes, w_scale, gamma, out, ws,
                          stream=stream)
    return out


def onepass_workspace(n_rows, vocab_start, vocab_end, d, device):
    nbytes = se_soft_embed_onepass_workspace_bytes(n_rows, vocab_start, vocab_end, d)
    return torch.empty((nbytes + 3) // 4, device=device, dtype=torch.float32)


def soft_embed_onepass(logits, vocab_start, vocab_end, w_shard, gamma, *, ws=None, stream=None):
    """(out, row_max, row_lse, row_entropy, row_argmax) over the slice [s, e), one logits read."""
    n, d = logits.shape[0], w_shard.shape[1]
    f = dict(device=logits.device, dtype=torch.float32)
    out = torch.empty((n, d), **f)
    mx, lse, ent = torch.empty(n, **f), torch.empty(n, **f), torch.empty(n, **f)
    am = torch.empty(n, device=logits.device, dtype=torch.int32)
    if ws is None:
        ws = onepass_workspace(n, vocab_start, vocab_end, d, logits.device)
    se_soft_embed_onepass(logits, vocab_start, vocab_end, w_shard, gamma, out, mx, lse, ent, am,
                          ws, stream=stream)
    return out, mx, lse, ent, am


def soft_embed_step_fp8(logits, vocab_start, vocab_end, w_codes, w_scale, gamma, *, ws=None,
                        stream=None, onepass=False):
    """se_soft_embed_step_fp8: the whole step against an e4m3 table; returns
    (out, row_max, row_lse, row_entropy, row_argmax).  ``onepass=True`` runs
    se_soft_embed_step_onepass_fp8 (one read of the logits, the row scales carried by the
    staged probabilities; w_scale 16-byte aligned)."""
    n, d = logits.shape[0], w_codes.shape[1]
    f = dict(device=logits.device, dtype=torch.float32)
    out = torch.empty((n, d), **f)
    mx, lse, ent = torch.empty(n, **f), torch.empty(n, **f), torch.empty(n, **f)
    am = torch.empty(n, device=logits.device, dtype=torch.int32)
    if onepass:
        if ws is None:
            ws = step_onepass_workspace(n, logits.shape[1], vocab_start, vocab_end, d,
                                        logits.device)
        se_soft_embed_step_onepass_fp8(logits, vocab_start, vocab_end, w_codes, w_scale, gamma,
                                       out, mx, lse, ent, am, ws, stream=stream)
        return out, mx, lse, ent, am
    if ws is None:
        ws = staged_workspace(n, vocab_start, vocab_end, d, logits.device)
    se_soft_embed_step_fp8(logits, vocab_start, vocab_end, w_codes, w_scale, gamma, out, mx, lse,
                           ent, am, ws, stream=stream)
    return out, mx, lse, ent, am


def step_onepass_workspace(n_rows, vocab, vocab_start, vocab_end, d, device):
    nbytes = se_soft_embed_step_onepass_workspace_bytes(n_rows, vocab, vocab_start, vocab_end, d)
    return torch.empty((nbytes + 3) // 4, device=device, dtype=torch.float32) if nbytes else None


def soft_embed_step(logits, vocab_start, vocab_end, w_shard, gamma, *, ws=None, stream=None,
                    onepass=False):
    """(out, row_max, row_lse, row_entropy, row_argmax): full-width statistics and the slice's
    soft embedding in one call.  ``onepass=True`` runs se_soft_embed_step_onepass (one read
    of the logits; equal to the two-pass step up to rounding)."""
    n, d = logits.shape[0], w_shard.shape[1]
    f = dict(device=logits.device, dtype=torch.float32)
    out = torch.empty((n, d), **f)
    mx, lse, ent = torch.empty(n, **f), torch.empty(n, **f), torch.empty(n, **f)
    am = torch.empty(n, device=logits.device, dtype=torch.int32)
    if onepass:
        if ws is None:
            ws = step_onepass_workspace(n, logits.shape[1], vocab_start, vocab_end, d,
                                        logits.device)
        se_soft_embed_step_onepass(logits, vocab_start, vocab_end, w_shard, gamma, out, mx, lse,
                                   ent, am, ws, stream=stream)
        return out, mx, lse, ent, am
    if ws is None:
        ws = staged_workspace(n, vocab_start, vocab_end, d, logits.device)
    se_soft_embed_step(logits, vocab_start, vocab_end, w_shard, gamma, out, mx, lse, ent, am, ws,
                       stream=stream)
    return out, mx, lse, ent, am
