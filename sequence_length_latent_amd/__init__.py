"""Python binding of the MI355X Stream-Factorized Attention library.

Thin argument marshalling over the C ABI in ``include/hd_sfa.h``: each function
checks dtype / device / contiguity / shape of its torch tensors, passes raw
device pointers and the current HIP stream, and raises ``HDError`` on a
non-zero status.  Every step of the computation runs in the library's HIP
kernels; PyTorch only provides device memory and the stream.

Expanded position of (token t, stream s) is t*n + s; query head h reads KV
head h // (Hq // Hkv).
"""
from __future__ import annotations

import torch

from ._lib import HDError, check, load  # noqa: F401

__all__ = ["expand", "final_stream_rows", "cyclic_replicate", "stream_attn", "mix_attn",
           "mix_attn_window", "attn_fwd", "split_workspace", "attn_split", "attn_bwd",
           "decode_workspace_size", "decode_step",
           "decode_step_noalloc", "decode_step_paged",
           "HDError", "load", "WITHIN", "MIX"]

WITHIN = 0
MIX = 1


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def expand(ids: torch.Tensor, tables: torch.Tensor, out: torch.Tensor | None = None,
           err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """out[b, t*n+s, :] = tables[s, ids[b, t], :].  ids int32 [B, L],
    tables bf16 [n, V, H] -> out bf16 [B, n*L, H].  ``err_flag`` (int32, one
    element, zeroed by the caller) is set to 1 if an id is out of range."""
    _need(ids, "ids", torch.int32, 2)
    _need(tables, "tables", torch.bfloat16, 3)
    B, L = ids.shape
    n, V, H = tables.shape
    if out is None:
        out = torch.empty((B, n * L, H), dtype=torch.bfloat16, device=tables.device)
    _need(out, "out", torch.bfloat16, 3)
    if tuple(out.shape) != (B, n * L, H):
        raise ValueError(f"out must be {(B, n * L, H)}")
    flag = 0
    if err_flag is not None:
        _need(err_flag, "err_flag", torch.int32, 1)
        flag = err_flag.data_ptr()
    st = load().hd_expand(ids.data_ptr(), B, L, tables.data_ptr(), n, V, H, out.data_ptr(),
                          flag or None, _stream())
    check("hd_expand", st)
    return out


def final_stream_rows(x, n: int, out=None):
    """Rows of the final stream: out[b, t] = x[b, t*n + n-1].  x [B, n*L, H] bf16."""
    _need(x, "x", torch.bfloat16, 3)
    B, N, H = x.shape
    if n < 1 or N % n:
        raise ValueError(f"sequence length {N} is not a multiple of n={n}")
    if out is None:
        out = torch.empty((B, N // n, H), dtype=x.dtype, device=x.device)
    _need(out, "out", torch.bfloat16, 3)
    if tuple(out.shape) != (B, N // n, H):
        raise ValueError("out must be [B, L, H]")
    st = load().hd_final_stream_rows(x.data_ptr(), B, n, N // n, H, out.data_ptr(), _stream())
    check("hd_final_stream_rows", st)
    return out


def cyclic_replicate(tables, n_new: int, out=None):
    """Cyclic Replication Initialization: out[s] = tables[s % n_old], s < n_new.
    tables [n_old, V, H] bf16.  With out=None a new [n_new, V, H] tensor is
    returned; an ``out`` whose storage starts at ``tables`` grows in place."""
    _need(tables, "tables", torch.bfloat16, 3)
    n_old, V, H = tables.shape
    if out is None:
        out = torch.empty((n_new, V, H), dtype=tables.dtype, device=tables.device)
    _need(out, "out", torch.bfloat16, 3)
    if tuple(out.shape) != (n_new, V, H):
        raise ValueError("out must be [n_new, V, H]")
    st = load().hd_cyclic_replicate(tables.data_ptr(), n_old, V, H, out.data_ptr(), n_new,
                                    _stream())
    check("hd_cyclic_replicate", st)
    return out


def _attn(fn_name: str, q, k, v, n: int, scale: float, out, window=None, lse=None, mode=None):
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if n < 1 or N % n:
        raise ValueError(f"sequence length {N} is not a multiple of n={n}")
    if tuple(k.shape) != (B, N, Hkv, D) or tuple(v.shape) != (B, N, Hkv, D):
        raise ValueError("k and v must be [B, n*L, Hkv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 4)
    if out.shape != q.shape:
        raise ValueError("out must match q")
    extra = () if window is None else (int(window),)
    if lse is not None:
        # training forward: mode (sfa_attn_fwd) or window (sfa_attn_fwd_window)
        last = int(mode) if mode is not None else int(window)
        st = getattr(load(), fn_name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr(), B, n, N // n, Hq, Hkv, D, float(scale),
                                      last, _stream())
    else:
        st = getattr(load(), fn_name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      B, n, N // n, Hq, Hkv, D, float(scale), *extra, _stream())
    check(fn_name, st)
    return out


def stream_attn(q, k, v, n: int, scale: float, out=None):
    """Within-stream causal attention.  q [B, n*L, Hq, D], k/v [B, n*L, Hkv, D]."""
    return _attn("sfa_stream_attn", q, k, v, n, scale, out)


def mix_attn(q, k, v, n: int, scale: float, out=None):
    """Mixing attention: full causal over the interleaved n*L order."""
    return _attn("sfa_mix_attn", q, k, v, n, scale, out)


def mix_attn_window(q, k, v, n: int, scale: float, window: int, out=None):
    """Mixing attention, sliding-window pattern: position i sees keys j with
    i - window < j <= i in the interleaved n*L order (window >= 1)."""
    return _attn("sfa_mix_attn_window", q, k, v, n, scale, out, window)


def attn_fwd(q, k, v, n: int, scale: float, mode: int, out=None, lse=None, window=None):
    """Forward of a prefill layer (mode WITHIN or MIX) with its log-sum-exp:
    returns (out [B, n*L, Hq, D] bf16, lse [B, Hq, n*L] fp32, natural log).
    ``window`` (MIX only): the sliding-window layer (sfa_attn_fwd_window)."""
    _need(q, "q", torch.bfloat16, 4)
    B, N, Hq, _ = q.shape
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, 3)
    if tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be [B, Hq, n*L]")
    if window is not None:
        if mode != MIX:
            raise ValueError("a window applies to mixing layers only")
        out = _attn("sfa_attn_fwd_window", q, k, v, n, scale, out, window=window, lse=lse)
    else:
        out = _attn("sfa_attn_fwd", q, k, v, n, scale, out, lse=lse, mode=mode)
    return out, lse


def split_workspace(q, k, n: int, mode: int):
    """A zero-filled workspace for attn_split with these shapes (uint8 tensor;
    empty when no split is possible).  Reuse it across calls: every call
    leaves it ready for the next one."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    B, N, Hq, D = q.shape
    if n < 1 or N % n:
        raise ValueError(f"sequence length {N} is not a multiple of n={n}")
    size = load().sfa_attn_split_workspace_size(B, n, N // n, Hq, k.shape[2], D, int(mode))
    return torch.zeros(max(int(size), 1), dtype=torch.uint8, device=q.device)


def attn_split(q, k, v, n: int, scale: float, mode: int, workspace, out=None, lse=None):
    """Prefill layer (mode WITHIN or MIX) for launches with no more work items
    than compute units: each item's key tiles are taken in two halves by
    different workgroups and merged (sfa_attn_split).  ``workspace`` from
    split_workspace(); ``lse`` optional [B, Hq, n*L] fp32.  Returns out."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if n < 1 or N % n:
        raise ValueError(f"sequence length {N} is not a multiple of n={n}")
    if tuple(k.shape) != (B, N, Hkv, D) or tuple(v.shape) != (B, N, Hkv, D):
        raise ValueError("k and v must be [B, n*L, Hkv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 4)
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, N):
            raise ValueError("lse must be [B, Hq, n*L]")
    if workspace is None or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace: a contiguous device tensor from split_workspace()")
    st = load().sfa_attn_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               None if lse is None else lse.data_ptr(), B, n, N // n, Hq, Hkv,
                               D, float(scale), int(mode), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream())
    check("sfa_attn_split", st)
    return out


def attn_bwd(q, k, v, dout, lse, n: int, scale: float, mode: int, dq=None, dk=None,
             dv=None, workspace=None, window=None):
    """Gradients of a prefill layer: returns (dq, dk, dv) in bf16.  ``lse`` is
    the forward's (attn_fwd with the same arguments).  ``window`` (MIX only):
    the sliding-window layer (sfa_attn_bwd_window)."""
    if window is not None and mode != MIX:
        raise ValueError("a window applies to mixing layers only")
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, nm, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if n < 1 or N % n:
        raise ValueError(f"sequence length {N} is not a multiple of n={n}")
    if tuple(k.shape) != (B, N, Hkv, D) or tuple(v.shape) != (B, N, Hkv, D):
        raise ValueError("k and v must be [B, n*L, Hkv, D] matching q")
    if tuple(dout.shape) != tuple(q.shape):
        raise ValueError("dout must match q")
    if tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be [B, Hq, n*L]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, nm, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _need(t, nm, torch.bfloat16, 4)
        if t.shape != ref.shape:
            raise ValueError(f"{nm} must match its input")
    lib = load()
    need = int(lib.sfa_attn_bwd_workspace_size(B, n, N // n, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    fn = "sfa_attn_bwd" if window is None else "sfa_attn_bwd_window"
    last = int(mode) if window is None else int(window)
    st = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, n, N // n,
                          Hq, Hkv, D, float(scale), last, workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), _stream())
    check(fn, st)
    return dq, dk, dv


def decode_workspace_size(S: int, n: int, Hq: int, Hkv: int, D: int, max_tokens: int) -> int:
    return int(load().sfa_decode_workspace_size(S, n, Hq, Hkv, D, max_tokens))


def _flag_ptr(err_flag):
    if err_flag is None:
        return None
    _need(err_flag, "err_flag", torch.int32, 1)
    return err_flag.data_ptr()


def decode_step(q_new, k_new, v_new, k_cache, v_cache, tokens_before, n: int,
                max_tokens: int, mode: int, scale: float, workspace=None, out=None,
                window=None, err_flag=None):
    """Append the n new stream positions and attend from them (mode WITHIN or
    MIX).  q_new [S, n, Hq, D]; k_new/v_new [S, n, Hkv, D]; caches
    [S, C, Hkv, D] (appended in place); tokens_before int32 [S] on the GPU.
    ``window`` (mode MIX only): sliding window in interleaved positions.
    ``err_flag`` (int32, one element, zeroed by the caller) is set to 1 if a
    tokens_before value lies outside [0, max_tokens]."""
    _need(q_new, "q_new", torch.bfloat16, 4)
    _need(k_new, "k_new", torch.bfloat16, 4)
    _need(v_new, "v_new", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(tokens_before, "tokens_before", torch.int32, 1)
    S, n_, Hq, D = q_new.shape
    if n_ != n:
        raise ValueError("q_new must be [S, n, Hq, D]")
    Hkv = k_new.shape[2]
    C = k_cache.shape[1]
    if tuple(k_new.shape) != (S, n, Hkv, D) or tuple(v_new.shape) != (S, n, Hkv, D):
        raise ValueError("k_new/v_new must be [S, n, Hkv, D]")
    if tuple(k_cache.shape) != (S, C, Hkv, D) or tuple(v_cache.shape) != (S, C, Hkv, D):
        raise ValueError("caches must be [S, C, Hkv, D]")
    if tuple(tokens_before.shape) != (S,):
        raise ValueError("tokens_before must be [S]")
    need = decode_workspace_size(S, n, Hq, Hkv, D, max_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_new.device)
    if out is None:
        out = torch.empty_like(q_new)
    _need(out, "out", torch.bfloat16, 4)
    if out.shape != q_new.shape:
        raise ValueError("out must match q_new")
    if window is not None:
        if mode != MIX:
            raise ValueError("a window applies to the mixing mode only")
        st = load().sfa_decode_step_window(
            q_new.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), tokens_before.data_ptr(), S, n, Hq, Hkv, D, C, max_tokens,
            int(window), float(scale), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), out.data_ptr(), _flag_ptr(err_flag),
            _stream())
        check("sfa_decode_step_window", st)
        return out
    st = load().sfa_decode_step(q_new.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                k_cache.data_ptr(), v_cache.data_ptr(), tokens_before.data_ptr(),
                                S, n, Hq, Hkv, D, C, max_tokens, int(mode), float(scale),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                out.data_ptr(), _flag_ptr(err_flag), _stream())
    check("sfa_decode_step", st)
    return out


def decode_step_noalloc(q_new, k_new, v_new, k_cache, v_cache, tokens_before, n: int,
                        max_tokens: int, mode: int, scale: float, out=None, err_flag=None):
    """decode_step without a workspace (sfa_decode_step_noalloc): the split
    partials live in the library's static 16 MiB per-device scratch, so the
    call allocates nothing given ``out``.  Bitwise the same results as
    decode_step; calls that overlap in time on one GPU race on the scratch."""
    for t, nm in ((q_new, "q_new"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _need(t, nm, torch.bfloat16, 4)
    _need(tokens_before, "tokens_before", torch.int32, 1)
    S, n_, Hq, D = q_new.shape
    if n_ != n:
        raise ValueError("q_new must be [S, n, Hq, D]")
    Hkv = k_new.shape[2]
    C = k_cache.shape[1]
    if tuple(k_new.shape) != (S, n, Hkv, D) or tuple(v_new.shape) != (S, n, Hkv, D):
        raise ValueError("k_new/v_new must be [S, n, Hkv, D]")
    if tuple(k_cache.shape) != (S, C, Hkv, D) or tuple(v_cache.shape) != (S, C, Hkv, D):
        raise ValueError("caches must be [S, C, Hkv, D]")
    if tuple(tokens_before.shape) != (S,):
        raise ValueError("tokens_before must be [S]")
    if out is None:
        out = torch.empty_like(q_new)
    _need(out, "out", torch.bfloat16, 4)
    if out.shape != q_new.shape:
        raise ValueError("out must match q_new")
    st = load().sfa_decode_step_noalloc(q_new.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                        k_cache.data_ptr(), v_cache.data_ptr(),
                                        tokens_before.data_ptr(), S, n, Hq, Hkv, D, C, max_tokens,
                                        int(mode), float(scale), out.data_ptr(),
                                        _flag_ptr(err_flag), _stream())
    check("sfa_decode_step_noalloc", st)
    return out


def decode_step_paged(q_new, k_new, v_new, k_pages, v_pages, page_table, tokens_before, n: int,
                      max_tokens: int, mode: int, scale: float, window=None, workspace=None,
                      out=None, err_flag=None):
    """decode_step over paged caches: pools [num_pages, P, Hkv, D] (appended in
    place), page_table int32 [S, max_pages_per_seq] and tokens_before int32 [S]
    on the GPU.  ``window`` (mode MIX only): sliding window in positions.
    ``err_flag`` as decode_step, also set for a page id outside the pool."""
    for t, nm in ((q_new, "q_new"), (k_new, "k_new"), (v_new, "v_new"), (k_pages, "k_pages"),
                  (v_pages, "v_pages")):
        _need(t, nm, torch.bfloat16, 4)
    _need(page_table, "page_table", torch.int32, 2)
    _need(tokens_before, "tokens_before", torch.int32, 1)
    S, n_, Hq, D = q_new.shape
    if n_ != n:
        raise ValueError("q_new must be [S, n, Hq, D]")
    Hkv = k_new.shape[2]
    num_pages, P = k_pages.shape[0], k_pages.shape[1]
    if tuple(k_new.shape) != (S, n, Hkv, D) or tuple(v_new.shape) != (S, n, Hkv, D):
        raise ValueError("k_new/v_new must be [S, n, Hkv, D]")
    if tuple(k_pages.shape) != (num_pages, P, Hkv, D) or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("page pools must be [num_pages, page_size, Hkv, D]")
    if page_table.shape[0] != S or tuple(tokens_before.shape) != (S,):
        raise ValueError("page_table must be [S, max_pages] and tokens_before [S]")
    need = decode_workspace_size(S, n, Hq, Hkv, D, max_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_new.device)
    if out is None:
        out = torch.empty_like(q_new)
    _need(out, "out", torch.bfloat16, 4)
    st = load().sfa_decode_step_paged(
        q_new.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
        page_table.data_ptr(), tokens_before.data_ptr(), S, n, Hq, Hkv, D, P, num_pages,
        page_table.shape[1], max_tokens, int(mode), 0 if window is None else int(window),
        float(scale), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        out.data_ptr(), _flag_ptr(err_flag), _stream())
    check("sfa_decode_step_paged", st)
    return out
