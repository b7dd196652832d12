"""ctypes binding of libsoftembed (include/softembed.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libsoftembed.so``.  PyTorch supplies device memory and the stream;
the functions below turn tensors into pointers, leading dimensions and sizes,
call the C entry point of the same name, and raise on a non-OK status.  There
is no fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library binds to (same soname)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsoftembed.so")

SE_OK, SE_ERR_NULL, SE_ERR_SHAPE, SE_ERR_SLICE, SE_ERR_ALIGN, SE_ERR_WORKSPACE, SE_ERR_HIP = range(7)
STATUS_NAMES = ["SE_OK", "SE_ERR_NULL", "SE_ERR_SHAPE", "SE_ERR_SLICE", "SE_ERR_ALIGN",
                "SE_ERR_WORKSPACE", "SE_ERR_HIP"]

EXPORTS = ("se_status_string", "se_version", "se_row_stats", "se_probs_bf16",
           "se_soft_embed_workspace_bytes", "se_soft_embed", "se_soft_embed_fused",
           "se_accept_converge", "se_reduce_partials", "se_quantize_table_fp8",
           "se_soft_embed_fp8", "se_soft_embed_fp8_fused", "se_soft_embed_onepass_workspace_bytes",
           "se_soft_embed_onepass", "se_merge_slices", "se_soft_embed_staged_workspace_bytes",
           "se_soft_embed_staged", "se_soft_embed_step",
           "se_soft_embed_step_onepass_workspace_bytes", "se_soft_embed_step_onepass",
           "se_soft_embed_step_fp8", "se_soft_embed_step_onepass_fp8", "se_set_launch_events",
           "se_launch_events_used",
           "se_soft_embed_splits", "se_soft_embed_step_noalloc_max_bytes",
           "se_soft_embed_step_noalloc", "se_mfma_loop")


class SoftEmbedError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _declare(lib):
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    f32 = ctypes.c_float
    lib.se_status_string.argtypes = [ctypes.c_int]
    lib.se_status_string.restype = ctypes.c_char_p
    lib.se_version.argtypes = []
    lib.se_version.restype = ctypes.c_char_p
    lib.se_row_stats.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.se_probs_bf16.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp, i64, vp]
    lib.se_soft_embed_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.se_soft_embed_workspace_bytes.restype = sz
    lib.se_soft_embed.argtypes = [vp, i64, i64, i64, i64, i64, vp, i64, i64, i64, f32, vp, i64,
                                  vp, sz, vp]
    lib.se_soft_embed_fused.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp, i64, i64, i64, f32,
                                        vp, i64, vp, sz, vp]
    f64, i32 = ctypes.c_double, ctypes.c_int32
    lib.se_accept_converge.argtypes = [vp, vp, i64, i64, f64, i32, f64, i32, vp, vp, vp, vp, vp,
                                       vp, vp]
    lib.se_reduce_partials.argtypes = [vp, i64, i64, i64, i64, i64, vp, i64, vp, i64, vp]
    lib.se_quantize_table_fp8.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp]
    lib.se_soft_embed_fp8.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, i64, i64, i64, f32, vp,
                                      i64, vp, sz, vp]
    lib.se_soft_embed_fp8_fused.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp, vp, i64, i64, i64,
                                            f32, vp, i64, vp, sz, vp]
    lib.se_soft_embed_onepass_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.se_soft_embed_onepass_workspace_bytes.restype = sz
    lib.se_soft_embed_onepass.argtypes = [vp, i64, i64, i64, i64, i64, vp, i64, i64, i64, f32, vp,
                                          i64, vp, vp, vp, vp, vp, sz, vp]
    lib.se_merge_slices.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp, vp,
                                    vp, vp, vp]
    lib.se_soft_embed_staged_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.se_soft_embed_staged_workspace_bytes.restype = sz
    lib.se_soft_embed_staged.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp, i64, i64, i64, f32,
                                         vp, i64, vp, sz, vp]
    lib.se_soft_embed_step.argtypes = [vp, i64, i64, i64, i64, i64, vp, i64, i64, i64, f32, vp, i64,
                                       vp, vp, vp, vp, vp, sz, vp]
    lib.se_soft_embed_step_onepass_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.se_soft_embed_step_onepass_workspace_bytes.restype = sz
    lib.se_soft_embed_step_onepass.argtypes = lib.se_soft_embed_step.argtypes
    lib.se_soft_embed_step_fp8.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, i64, i64, i64, f32,
                                           vp, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.se_soft_embed_step_onepass_fp8.argtypes = lib.se_soft_embed_step_fp8.argtypes
    lib.se_soft_embed_step_noalloc_max_bytes.argtypes = []
    lib.se_soft_embed_step_noalloc_max_bytes.restype = sz
    lib.se_soft_embed_step_noalloc.argtypes = [vp, i64, i64, i64, i64, i64, vp, i64, i64, i64,
                                               f32, vp, i64, vp, vp, vp, vp, vp]
    lib.se_soft_embed_splits.argtypes = [i64, i64, i64, i64]
    lib.se_soft_embed_splits.restype = i64
    lib.se_set_launch_events.argtypes = [vp, i32]
    lib.se_launch_events_used.argtypes = []
    lib.se_launch_events_used.restype = i32
    lib.se_mfma_loop.argtypes = [vp, i64, i64, ctypes.c_float, vp]
    for fn in ("se_mfma_loop", "se_soft_embed_step_noalloc", "se_set_launch_events", "se_row_stats", "se_probs_bf16", "se_soft_embed", "se_soft_embed_fused",
               "se_accept_converge", "se_reduce_partials", "se_quantize_table_fp8",
               "se_soft_embed_fp8", "se_soft_embed_fp8_fused", "se_soft_embed_onepass",
               "se_merge_slices", "se_soft_embed_staged", "se_soft_embed_step",
               "se_soft_embed_step_onepass", "se_soft_embed_step_fp8",
               "se_soft_embed_step_onepass_fp8"):
        getattr(lib, fn).restype = ctypes.c_int
    return lib


def load_library(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"libsoftembed.so not built at {path}; run "
                          "`python -m diffusion_self_conditioning_amd.build`")
    return _declare(ctypes.CDLL(path))


lib = load_library()


def _check(fn: str, status: int):
    if status != SE_OK:
        raise SoftEmbedError(fn, status, lib.se_status_string(status).decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _as_u16(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint16) if t.dtype == torch.bfloat16 else t


def se_status_string(status: int) -> str:
    return lib.se_status_string(status).decode()


def se_version() -> str:
    return lib.se_version().decode()


def se_row_stats(logits, row_max, row_lse, row_entropy, row_argmax, *, vocab=None, stream=None):
    """Row max / log-sum-exp / entropy / argmax of fp32 logits [n_rows, >= vocab]."""
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    _check("se_row_stats", lib.se_row_stats(_ptr(logits), _ld(logits), n, vocab, _ptr(row_max),
                                            _ptr(row_lse), _ptr(row_entropy), _ptr(row_argmax),
                                            _stream(stream)))


def se_probs_bf16(logits, row_lse, vocab_start, vocab_end, probs, *, vocab=None, stream=None):
    """probs[:, s:e] = bf16(exp(logits[:, s:e] - lse)); ``probs`` is bf16 or uint16."""
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    probs = _as_u16(probs)
    _check("se_probs_bf16", lib.se_probs_bf16(_ptr(logits), _ld(logits), _ptr(row_lse), n, vocab,
                                              vocab_start, vocab_end, _ptr(probs), _ld(probs),
                                              _stream(stream)))


def se_soft_embed_workspace_bytes(n_rows: int, vocab_start: int, vocab_end: int, d: int) -> int:
    return int(lib.se_soft_embed_workspace_bytes(n_rows, vocab_start, vocab_end, d))


def se_soft_embed_splits(n_rows: int, vocab_start: int, vocab_end: int, d: int) -> int:
    return int(lib.se_soft_embed_splits(n_rows, vocab_start, vocab_end, d))


def se_soft_embed_ranges(n_rows: int, vocab_start: int, vocab_end: int, d: int) -> list:
    """The vocabulary ids [s, b_1, ..., e] bounding the contraction's split ranges (the
    rule stated in include/softembed.h under se_soft_embed_splits)."""
    S = se_soft_embed_splits(n_rows, vocab_start, vocab_end, d)
    K = vocab_end - vocab_start
    nb = (K + 127) // 128
    return [vocab_start + min(128 * ((r * nb) // S), K) for r in range(S)] + [vocab_end]


def se_soft_embed(probs, vocab_start, vocab_end, w_shard, gamma, out, workspace=None, *,
                  vocab=None, d=None, w_rows=None, stream=None):
    """out[:, :d] = gamma * probs[:, s:e] @ w_shard[: e - s, :d]  (bf16 inputs, fp32 out)."""
    probs, w_shard = _as_u16(probs), _as_u16(w_shard)
    n, v = probs.shape
    vocab = v if vocab is None else vocab
    d = w_shard.shape[1] if d is None else d
    w_rows = w_shard.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed", lib.se_soft_embed(
        _ptr(probs), _ld(probs), n, vocab, vocab_start, vocab_end, _ptr(w_shard), w_rows,
        _ld(w_shard), d, float(gamma), _ptr(out), _ld(out), _ptr(workspace), ws_bytes,
        _stream(stream)))


def se_soft_embed_fused(logits, row_lse, vocab_start, vocab_end, w_shard, gamma, out,
                        workspace=None, *, vocab=None, d=None, w_rows=None, stream=None):
    """out[:, :d] = gamma * bf16(softmax(logits))[:, s:e] @ w_shard[: e - s, :d], P never stored."""
    w_shard = _as_u16(w_shard)
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_shard.shape[1] if d is None else d
    w_rows = w_shard.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_fused", lib.se_soft_embed_fused(
        _ptr(logits), _ld(logits), _ptr(row_lse), n, vocab, vocab_start, vocab_end,
        _ptr(w_shard), w_rows, _ld(w_shard), d, float(gamma), _ptr(out), _ld(out),
        _ptr(workspace), ws_bytes, _stream(stream)))


def se_accept_converge(row_entropy, row_argmax, canvas_len, entropy_budget, stable_steps,
                       entropy_tau, step_limit, accepted, prev_argmax, stable_count, step_count,
                       newly_accepted, converged, *, stream=None):
    """Entropy-bound acceptance + convergence test over canvases of ``canvas_len`` rows.

    ``row_entropy`` fp32 / ``row_argmax`` int32 of n_canvas * canvas_len positions; state
    tensors ``accepted`` (uint8), ``prev_argmax`` (int32), ``stable_count`` / ``step_count``
    (int32 per canvas) are updated in place; ``newly_accepted`` (uint8) and ``converged``
    (uint8 per canvas) are written."""
    n = row_entropy.numel()
    if n % canvas_len:
        raise ValueError("row count is not a multiple of canvas_len")
    _check("se_accept_converge", lib.se_accept_converge(
        _ptr(row_entropy), _ptr(row_argmax), n // canvas_len, canvas_len, float(entropy_budget),
        int(stable_steps), float(entropy_tau), int(step_limit), _ptr(accepted),
        _ptr(prev_argmax), _ptr(stable_count), _ptr(step_count), _ptr(newly_accepted),
        _ptr(converged), _stream(stream)))


def se_reduce_partials(parts, out=None, out_bf16=None, *, stream=None):
    """Sum fp32 partials ``parts`` [T, n_rows, >= d] in order r = 0..T-1 into ``out`` (fp32)
    and / or ``out_bf16`` (bfloat16), both [n_rows, >= d]."""
    if parts.dim() != 3 or parts.stride(2) != 1:
        raise ValueError("parts must be [T, rows, d] with unit column stride")
    t, n, d = parts.shape
    dst = out if out is not None else out_bf16
    d = dst.shape[1]
    _check("se_reduce_partials", lib.se_reduce_partials(
        _ptr(parts), t, parts.stride(0), n, d, parts.stride(1), _ptr(out),
        _ld(out) if out is not None else 0, _ptr(out_bf16),
        _ld(out_bf16) if out_bf16 is not None else 0, _stream(stream)))


def se_mfma_loop(out, blocks: int, iters: int, unit: float = 1.0, *, stream=None):
    """The MFMA-rate probe: ``blocks`` workgroups, 8 chains of ``iters`` 32x32x16 bf16 MFMAs
    per wave, one float per lane into ``out`` (fp32, at least blocks * 256)."""
    if out.numel() < blocks * 256:
        raise ValueError("out holds fewer than blocks * 256 floats")
    _check("se_mfma_loop", lib.se_mfma_loop(_ptr(out), blocks, iters, float(unit), _stream(stream)))


def se_quantize_table_fp8(w, codes, row_scale, *, d=None, stream=None):
    """e4m3 codes (uint8 [rows, >= d]) and power-of-two row scales (fp32 [rows]) of the
    bf16 table ``w`` [rows, >= d]."""
    w = _as_u16(w)
    rows = w.shape[0]
    d = w.shape[1] if d is None else d
    _check("se_quantize_table_fp8", lib.se_quantize_table_fp8(
        _ptr(w), _ld(w), rows, d, _ptr(codes), _ld(codes), _ptr(row_scale), _stream(stream)))


def se_soft_embed_fp8(probs, vocab_start, vocab_end, w_codes, w_scale, gamma, out, workspace=None,
                      *, vocab=None, d=None, w_rows=None, stream=None):
    """se_soft_embed with the shard as e4m3 codes [w_rows, >= d] and fp32 row scales."""
    probs = _as_u16(probs)
    n, v = probs.shape
    vocab = v if vocab is None else vocab
    d = w_codes.shape[1] if d is None else d
    w_rows = w_codes.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_fp8", lib.se_soft_embed_fp8(
        _ptr(probs), _ld(probs), n, vocab, vocab_start, vocab_end, _ptr(w_codes), _ptr(w_scale),
        w_rows, _ld(w_codes), d, float(gamma), _ptr(out), _ld(out), _ptr(workspace), ws_bytes,
        _stream(stream)))


def se_soft_embed_fp8_fused(logits, row_lse, vocab_start, vocab_end, w_codes, w_scale, gamma, out,
                            workspace=None, *, vocab=None, d=None, w_rows=None, stream=None):
    """se_soft_embed_fused with the shard as e4m3 codes [w_rows, >= d] and fp32 row scales."""
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_codes.shape[1] if d is None else d
    w_rows = w_codes.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_fp8_fused", lib.se_soft_embed_fp8_fused(
        _ptr(logits), _ld(logits), _ptr(row_lse), n, vocab, vocab_start, vocab_end,
        _ptr(w_codes), _ptr(w_scale), w_rows, _ld(w_codes), d, float(gamma), _ptr(out), _ld(out),
        _ptr(workspace), ws_bytes, _stream(stream)))


def se_soft_embed_onepass_workspace_bytes(n_rows: int, vocab_start: int, vocab_end: int,
                                          d: int) -> int:
    return int(lib.se_soft_embed_onepass_workspace_bytes(n_rows, vocab_start, vocab_end, d))


def se_soft_embed_onepass(logits, vocab_start, vocab_end, w_shard, gamma, out, row_max, row_lse,
                          row_entropy, row_argmax, workspace, *, vocab=None, d=None, w_rows=None,
                          stream=None):
    """Slice-normalised soft embedding and slice row statistics from one read of the logits."""
    w_shard = _as_u16(w_shard)
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_shard.shape[1] if d is None else d
    w_rows = w_shard.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_onepass", lib.se_soft_embed_onepass(
        _ptr(logits), _ld(logits), n, vocab, vocab_start, vocab_end, _ptr(w_shard), w_rows,
        _ld(w_shard), d, float(gamma), _ptr(out), _ld(out), _ptr(row_max), _ptr(row_lse),
        _ptr(row_entropy), _ptr(row_argmax), _ptr(workspace), ws_bytes, _stream(stream)))


def se_merge_slices(outs, part_max, part_lse, part_entropy, part_argmax, out, row_max, row_lse,
                    row_entropy, row_argmax, *, stream=None):
    """Merge T slice results: ``outs`` [T, n_rows, >= d] fp32, statistics [T, n_rows]."""
    if outs.dim() != 3 or outs.stride(2) != 1:
        raise ValueError("outs must be [T, rows, d] with unit column stride")
    t, n, _ = outs.shape
    d = out.shape[1]
    for a in (part_max, part_lse, part_entropy, part_argmax):
        if tuple(a.shape) != (t, n) or not a.is_contiguous():
            raise ValueError("slice statistics must be contiguous [T, rows]")
    _check("se_merge_slices", lib.se_merge_slices(
        _ptr(outs), t, outs.stride(0), n, d, outs.stride(1), _ptr(part_max), _ptr(part_lse),
        _ptr(part_entropy), _ptr(part_argmax), _ptr(out), _ld(out), _ptr(row_max),
        _ptr(row_lse), _ptr(row_entropy), _ptr(row_argmax), _stream(stream)))


def se_soft_embed_staged_workspace_bytes(n_rows: int, vocab_start: int, vocab_end: int,
                                         d: int) -> int:
    return int(lib.se_soft_embed_staged_workspace_bytes(n_rows, vocab_start, vocab_end, d))


def se_soft_embed_staged(logits, row_lse, vocab_start, vocab_end, w_shard, gamma, out, workspace,
                         *, vocab=None, d=None, w_rows=None, stream=None):
    """se_soft_embed_fused's result through probabilities staged in ``workspace``."""
    w_shard = _as_u16(w_shard)
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_shard.shape[1] if d is None else d
    w_rows = w_shard.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_staged", lib.se_soft_embed_staged(
        _ptr(logits), _ld(logits), _ptr(row_lse), n, vocab, vocab_start, vocab_end,
        _ptr(w_shard), w_rows, _ld(w_shard), d, float(gamma), _ptr(out), _ld(out),
        _ptr(workspace), ws_bytes, _stream(stream)))


def se_soft_embed_step_onepass_workspace_bytes(n_rows: int, vocab: int, vocab_start: int,
                                               vocab_end: int, d: int) -> int:
    return int(lib.se_soft_embed_step_onepass_workspace_bytes(n_rows, vocab, vocab_start,
                                                              vocab_end, d))


def se_soft_embed_step_onepass(logits, vocab_start, vocab_end, w_shard, gamma, out, row_max,
                               row_lse, row_entropy, row_argmax, workspace, *, vocab=None,
                               d=None, w_rows=None, stream=None):
    """The step of se_soft_embed_step from one read of the logits (range-wise maxima)."""
    w_shard = _as_u16(w_shard)
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_shard.shape[1] if d is None else d
    w_rows = w_shard.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_step_onepass", lib.se_soft_embed_step_onepass(
        _ptr(logits), _ld(logits), n, vocab, vocab_start, vocab_end, _ptr(w_shard), w_rows,
        _ld(w_shard), d, float(gamma), _ptr(out), _ld(out), _ptr(row_max), _ptr(row_lse),
        _ptr(row_entropy), _ptr(row_argmax), _ptr(workspace), ws_bytes, _stream(stream)))


def se_soft_embed_step_fp8(logits, vocab_start, vocab_end, w_codes, w_scale, gamma, out, row_max,
                           row_lse, row_entropy, row_argmax, workspace, *, vocab=None, d=None,
                           w_rows=None, stream=None):
    """se_soft_embed_step against an e4m3 table (codes + per-row scales)."""
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_codes.shape[1] if d is None else d
    w_rows = w_codes.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_step_fp8", lib.se_soft_embed_step_fp8(
        _ptr(logits), _ld(logits), n, vocab, vocab_start, vocab_end, _ptr(w_codes), _ptr(w_scale),
        w_rows, _ld(w_codes), d, float(gamma), _ptr(out), _ld(out), _ptr(row_max), _ptr(row_lse),
        _ptr(row_entropy), _ptr(row_argmax), _ptr(workspace), ws_bytes, _stream(stream)))


def se_soft_embed_step_onepass_fp8(logits, vocab_start, vocab_end, w_codes, w_scale, gamma, out,
                                   row_max, row_lse, row_entropy, row_argmax, workspace, *,
                                   vocab=None, d=None, w_rows=None, stream=None):
    """se_soft_embed_step_onepass against an e4m3 table (codes + per-row scales)."""
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_codes.shape[1] if d is None else d
    w_rows = w_codes.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_step_onepass_fp8", lib.se_soft_embed_step_onepass_fp8(
        _ptr(logits), _ld(logits), n, vocab, vocab_start, vocab_end, _ptr(w_codes), _ptr(w_scale),
        w_rows, _ld(w_codes), d, float(gamma), _ptr(out), _ld(out), _ptr(row_max), _ptr(row_lse),
        _ptr(row_entropy), _ptr(row_argmax), _ptr(workspace), ws_bytes, _stream(stream)))


def se_soft_embed_step(logits, vocab_start, vocab_end, w_shard, gamma, out, row_max, row_lse,
                       row_entropy, row_argmax, workspace, *, vocab=None, d=None, w_rows=None,
                       stream=None):
    """se_row_stats + se_soft_embed_fused in one call (outputs bit for bit theirs)."""
    w_shard = _as_u16(w_shard)
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_shard.shape[1] if d is None else d
    w_rows = w_shard.shape[0] if w_rows is None else w_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("se_soft_embed_step", lib.se_soft_embed_step(
        _ptr(logits), _ld(logits), n, vocab, vocab_start, vocab_end, _ptr(w_shard), w_rows,
        _ld(w_shard), d, float(gamma), _ptr(out), _ld(out), _ptr(row_max), _ptr(row_lse),
        _ptr(row_entropy), _ptr(row_argmax), _ptr(workspace), ws_bytes, _stream(stream)))


def se_set_launch_events(events) -> None:
    """Arm the calling thread's per-launch timing markers with HIP event handles (ints, e.g.
    ``torch.cuda.Event.cuda_event`` after a first record): each later launch takes two, its
    kernel's start and end.  An empty list disarms them.  The handle array is kept alive
    here until the next call."""
    global _armed
    handles = [int(e) for e in events]
    _armed = (ctypes.c_void_p * max(1, len(handles)))(*handles)
    _check("se_set_launch_events",
           lib.se_set_launch_events(_armed if handles else None, len(handles)))


def se_launch_events_used() -> int:
    return int(lib.se_launch_events_used())


_armed = None


def se_soft_embed_step_noalloc(logits, vocab_start, vocab_end, w_shard, gamma, out, row_max,
                               row_lse, row_entropy, row_argmax, *, vocab=None, d=None,
                               w_rows=None, stream=None):
    """se_soft_embed_step with the library's own device workspace (no allocation)."""
    w_shard = _as_u16(w_shard)
    n, v = logits.shape
    vocab = v if vocab is None else vocab
    d = w_shard.shape[1] if d is None else d
    w_rows = w_shard.shape[0] if w_rows is None else w_rows
    _check("se_soft_embed_step_noalloc", lib.se_soft_embed_step_noalloc(
        _ptr(logits), _ld(logits), n, vocab, vocab_start, vocab_end, _ptr(w_shard), w_rows,
        _ld(w_shard), d, float(gamma), _ptr(out), _ld(out), _ptr(row_max), _ptr(row_lse),
        _ptr(row_entropy), _ptr(row_argmax), _stream(stream)))


def se_soft_embed_step_noalloc_max_bytes() -> int:
    return int(lib.se_soft_embed_step_noalloc_max_bytes())
