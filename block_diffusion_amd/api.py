"""Thin Python binding of libdbd (ctypes).  Argument marshalling only: every
step of the round runs in the library's HIP kernels.  PyTorch provides
device memory and the current stream.

The function names are those of the C ABI in include/dbd.h.  A missing or
unloadable libdbd.so raises at import of the library (no fallback).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdbd.so")

DBD_OK, DBD_ERR_INVALID_ARG, DBD_ERR_UNSUPPORTED, DBD_ERR_WORKSPACE, DBD_ERR_HIP = range(5)
DBD_WAITING, DBD_PREFILLING, DBD_DENOISING, DBD_SAVING, DBD_FINISHED = range(5)
DBD_FALLBACK_LEFTMOST, DBD_COMPACT_ONLY = 1, 2
(DBD_RULE_LOW_CONF_DYNAMIC, DBD_RULE_LOW_CONF_STATIC, DBD_RULE_SEQUENTIAL,
 DBD_RULE_ENTROPY_BOUNDED) = 0, 1, 2, 3

_vp, _i32p, _u8p, _fp = C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p


class dbd_round_args(C.Structure):
    _fields_ = [(n, C.c_int) for n in
                ("S", "B", "Hq", "Hkv", "D", "page_size", "max_pages_per_seq", "Hd", "V",
                 "mask_token_id")] + [
        ("dynamic_threshold", C.c_float), ("flags", C.c_uint32), ("softmax_scale", C.c_float),
        ("q", _vp), ("k_blk", _vp), ("v_blk", _vp), ("k_cache", _vp), ("v_cache", _vp),
        ("page_table", _vp), ("prefix_len", _vp), ("attn_out", _vp),
        ("hidden", _vp), ("w_vocab", _vp), ("row_index", _vp), ("num_rows", _vp),
        ("argmax_tok", _vp), ("conf", _vp), ("block_tokens", _vp), ("seq_state", _vp),
        ("num_committed", _vp), ("workspace", _vp), ("workspace_bytes", C.c_size_t),
        ("rule", C.c_int), ("tokens_per_step", C.c_int), ("eb_threshold", C.c_float),
        ("entropy", _vp), ("save_kv", C.c_int), ("num_pages", C.c_int),
        ("token_stream", _vp), ("stream_cap", C.c_int), ("end_len", _vp),
        ("gate_on_rows", C.c_int), ("round_counter", _vp),
        ("sample", C.c_int), ("temperature", C.c_float), ("seed", C.c_uint64), ("step", C.c_uint32),
        ("filter", C.c_int), ("top_k", C.c_int), ("top_p", C.c_float), ("logits", C.c_void_p)]


class DbdError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libdbd status {status}: {msg}")
        self.status = status


_lib = None


ABI_VERSION = 4          # DBD_ABI_VERSION of include/dbd.h that this binding follows


def lib() -> C.CDLL:
    """Load libdbd.so (once).  Raises if it is missing: build it with
    ``python -m block_diffusion_amd.build``."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m block_diffusion_amd.build` "
                          "(there is no CPU fallback)")
    L = C.CDLL(LIB_PATH)
    i, f, u32, sz = C.c_int, C.c_float, C.c_uint32, C.c_size_t
    L.dbd_attn_paged.argtypes = [i] * 7 + [_vp] * 7 + [f, _vp, _vp, sz, _vp]
    L.dbd_attn_paged.restype = i
    L.dbd_attn_workspace_size.argtypes = [i] * 7
    L.dbd_attn_workspace_size.restype = sz
    L.dbd_lmhead_conf.argtypes = [i] * 4 + [_vp] * 6 + [_vp, sz, _vp]
    L.dbd_lmhead_conf.restype = i
    L.dbd_lmhead_workspace_size.argtypes = [i, i]
    L.dbd_lmhead_workspace_size.restype = sz
    L.dbd_remask_commit.argtypes = [i, i, i, f, u32] + [_vp] * 7 + [_vp]
    L.dbd_remask_commit.restype = i
    L.dbd_lmhead_conf_entropy.argtypes = [i] * 4 + [_vp] * 7 + [_vp, sz, _vp]
    L.dbd_lmhead_conf_entropy.restype = i
    L.dbd_remask_commit_rule.argtypes = [i, i, i, i, f, i, f, u32] + [_vp] * 8 + [_vp]
    L.dbd_remask_commit_rule.restype = i
    L.dbd_attn_paged_save.argtypes = [i] * 8 + [_vp] * 8 + [f, _vp, _vp, sz, _vp]
    L.dbd_attn_paged_save.restype = i
    L.dbd_commit_block.argtypes = [i, i, i] + [_vp] * 4 + [i] + [_vp] * 3 + [_vp]
    L.dbd_commit_block.restype = i
    L.dbd_lmhead_sample.argtypes = [i] * 4 + [_vp] * 4 + [f, C.c_uint64, C.c_uint32] + \
        [_vp] * 4 + [sz, _vp]
    L.dbd_lmhead_sample.restype = i
    L.dbd_prefill_attn.argtypes = [i] * 6 + [_vp] * 4 + [f, _vp] + [i] * 3 + [_vp] * 4 + [sz, _vp]
    L.dbd_prefill_attn.restype = i
    L.dbd_prefill_workspace_size.argtypes = [i]
    L.dbd_prefill_workspace_size.restype = sz
    L.dbd_lmhead_logits.argtypes = [i] * 4 + [_vp] * 5 + [_vp]
    L.dbd_lmhead_logits.restype = i
    L.dbd_sample_filtered.argtypes = [i, i, i] + [_vp] * 3 + [f, i, f, C.c_uint64, C.c_uint32] + \
        [_vp, _vp, _vp]
    L.dbd_sample_filtered.restype = i
    L.dbd_stream_read.argtypes = [_vp, sz, _vp, _vp]
    L.dbd_stream_read.restype = i
    L.dbd_stream_read_sink_words.argtypes = []
    L.dbd_stream_read_sink_words.restype = i
    L.dbd_mfma_peak.argtypes = [_vp, i, _vp, _vp]
    L.dbd_mfma_peak.restype = i
    L.dbd_mfma_peak_operand_bytes.argtypes = []
    L.dbd_mfma_peak_operand_bytes.restype = sz
    L.dbd_mfma_peak_sink_floats.argtypes = []
    L.dbd_mfma_peak_sink_floats.restype = i
    L.dbd_mfma_peak_flops.argtypes = [i]
    L.dbd_mfma_peak_flops.restype = C.c_double
    L.dbd_round.argtypes = [C.POINTER(dbd_round_args), _vp]
    L.dbd_round.restype = i
    L.dbd_round_noalloc.argtypes = [C.POINTER(dbd_round_args), _vp]
    L.dbd_round_noalloc.restype = i
    L.dbd_round_workspace_size.argtypes = [C.POINTER(dbd_round_args)]
    L.dbd_round_workspace_size.restype = sz
    L.dbd_graph_create.argtypes = [C.POINTER(dbd_round_args), i, C.POINTER(_vp)]
    L.dbd_graph_create.restype = i
    L.dbd_graph_launch.argtypes = [_vp, _vp]
    L.dbd_graph_launch.restype = i
    L.dbd_graph_destroy.argtypes = [_vp]
    L.dbd_graph_destroy.restype = None
    L.dbd_validate_inputs.argtypes = [i] * 7 + [_vp] * 4
    L.dbd_validate_inputs.restype = i
    L.dbd_last_error.argtypes = []
    L.dbd_last_error.restype = C.c_char_p
    L.dbd_abi_version.argtypes = []
    L.dbd_abi_version.restype = i
    L.dbd_round_args_size.argtypes = []
    L.dbd_round_args_size.restype = sz
    if L.dbd_abi_version() != ABI_VERSION or L.dbd_round_args_size() != C.sizeof(dbd_round_args):
        raise ImportError(f"{LIB_PATH}: ABI {L.dbd_abi_version()} with a {L.dbd_round_args_size()}-byte "
                          f"dbd_round_args, this binding expects ABI {ABI_VERSION} and "
                          f"{C.sizeof(dbd_round_args)} bytes: rebuild the library")
    _lib = L
    return L


def _check(st):
    if st != DBD_OK:
        raise DbdError(st, lib().dbd_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def dbd_attn_workspace_size(S, B, Hq, Hkv, D, page_size, max_pages_per_seq):
    return lib().dbd_attn_workspace_size(S, B, Hq, Hkv, D, page_size, max_pages_per_seq)


def dbd_lmhead_workspace_size(max_rows, V):
    return lib().dbd_lmhead_workspace_size(max_rows, V)


def workspace(nbytes, device="cuda"):
    """A device byte buffer (PyTorch's allocator aligns to 512 B)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _launch_ws(nbytes, device, stream):
    """A workspace the binding allocates for one launch.  When the launch
    goes to a stream the caller names, the allocator is told that stream
    uses the buffer, so that its memory is not handed out again (to work on
    torch's current stream) while the launch may still run."""
    t = workspace(nbytes, device)
    if stream is not None:
        s = torch.cuda.ExternalStream(stream, device=t.device) if isinstance(stream, int) else stream
        t.record_stream(s)
    return t


def dbd_attn_paged(q, k_blk, v_blk, k_cache, v_cache, page_table, prefix_len, out,
                   softmax_scale=0.0, ws=None, stream=None):
    S, B, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    P = k_cache.shape[2]
    maxp = page_table.shape[1]
    for t, n in ((q, "q"), (k_blk, "k_blk"), (v_blk, "v_blk"), (k_cache, "k_cache"),
                 (v_cache, "v_cache"), (out, "out")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous bf16")
    _need(k_blk, torch.bfloat16, (S, B, Hkv, D), "k_blk")
    _need(v_blk, torch.bfloat16, (S, B, Hkv, D), "v_blk")
    _need(v_cache, torch.bfloat16, tuple(k_cache.shape), "v_cache")
    _need(out, torch.bfloat16, (S, B, Hq, D), "out")
    _need(page_table, torch.int32, (S, maxp), "page_table")
    _need(prefix_len, torch.int32, (S,), "prefix_len")
    need = dbd_attn_workspace_size(S, B, Hq, Hkv, D, P, maxp)
    if ws is None and need:
        ws = _launch_ws(need, q.device, stream)
    nbytes = ws.numel() if ws is not None else 0
    _check(lib().dbd_attn_paged(S, B, Hq, Hkv, D, P, maxp, _ptr(q), _ptr(k_blk), _ptr(v_blk),
                                _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                _ptr(prefix_len), float(softmax_scale), _ptr(out), _ptr(ws),
                                nbytes, _stream(stream)))
    return out


def dbd_attn_paged_save(q, k_blk, v_blk, k_cache, v_cache, page_table, prefix_len, seq_state,
                        out, softmax_scale=0.0, ws=None, stream=None):
    """dbd_attn_paged, and the block K/V of SAVING sequences written into
    k_cache / v_cache (in place) at positions prefix_len + j."""
    S, B, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    npages, _, P, _ = k_cache.shape
    maxp = page_table.shape[1]
    for t, n in ((q, "q"), (k_cache, "k_cache")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous bf16")
    _need(k_blk, torch.bfloat16, (S, B, Hkv, D), "k_blk")
    _need(v_blk, torch.bfloat16, (S, B, Hkv, D), "v_blk")
    _need(v_cache, torch.bfloat16, tuple(k_cache.shape), "v_cache")
    _need(out, torch.bfloat16, (S, B, Hq, D), "out")
    _need(page_table, torch.int32, (S, maxp), "page_table")
    _need(prefix_len, torch.int32, (S,), "prefix_len")
    _need(seq_state, torch.uint8, (S,), "seq_state")
    need = dbd_attn_workspace_size(S, B, Hq, Hkv, D, P, maxp)
    if ws is None and need:
        ws = _launch_ws(need, q.device, stream)
    nbytes = ws.numel() if ws is not None else 0
    _check(lib().dbd_attn_paged_save(S, B, Hq, Hkv, D, P, maxp, npages, _ptr(q), _ptr(k_blk),
                                     _ptr(v_blk), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                     _ptr(prefix_len), _ptr(seq_state), float(softmax_scale),
                                     _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    return out


def dbd_commit_block(block_tokens, seq_state, prefix_len, row_index_out, num_rows_out,
                     mask_token_id, token_stream=None, end_len=None, stream=None):
    S, B = block_tokens.shape
    _need(block_tokens, torch.int32, (S, B), "block_tokens")
    _need(seq_state, torch.uint8, (S,), "seq_state")
    _need(prefix_len, torch.int32, (S,), "prefix_len")
    _need(row_index_out, torch.int32, (S * B,), "row_index_out")
    _need(num_rows_out, torch.int32, (1,), "num_rows_out")
    cap = 0
    if token_stream is not None:
        _need(token_stream, torch.int32, (S, token_stream.shape[1]), "token_stream")
        cap = token_stream.shape[1]
    if end_len is not None:
        _need(end_len, torch.int32, (S,), "end_len")
    _check(lib().dbd_commit_block(S, B, int(mask_token_id), _ptr(block_tokens), _ptr(seq_state),
                                  _ptr(prefix_len), _ptr(token_stream), cap, _ptr(end_len),
                                  _ptr(row_index_out), _ptr(num_rows_out), _stream(stream)))


def dbd_lmhead_conf(hidden, w_vocab, num_rows, argmax_tok, conf, mask_token_id,
                    row_index=None, max_rows=None, ws=None, stream=None, entropy=None):
    """entropy (float32, optional): also each listed row's softmax entropy
    (dbd_lmhead_conf_entropy)."""
    V, Hd = w_vocab.shape
    if max_rows is None:
        max_rows = row_index.shape[0] if row_index is not None else hidden.shape[0]
    _need(hidden, torch.bfloat16, (hidden.shape[0], Hd), "hidden")
    _need(w_vocab, torch.bfloat16, (V, Hd), "w_vocab")
    _need(num_rows, torch.int32, (1,), "num_rows")
    if row_index is not None:
        if row_index.dtype != torch.int32 or row_index.numel() < max_rows:
            raise ValueError("row_index must be int32 with at least max_rows entries")
    need = dbd_lmhead_workspace_size(max_rows, V)
    if ws is None and need:
        ws = _launch_ws(need, hidden.device, stream)
    nb = ws.numel() if ws is not None else 0
    if entropy is None:
        _check(lib().dbd_lmhead_conf(max_rows, Hd, V, int(mask_token_id), _ptr(hidden),
                                     _ptr(row_index), _ptr(num_rows), _ptr(w_vocab),
                                     _ptr(argmax_tok), _ptr(conf), _ptr(ws), nb,
                                     _stream(stream)))
    else:
        if entropy.dtype != torch.float32:
            raise ValueError("entropy must be float32")
        _check(lib().dbd_lmhead_conf_entropy(max_rows, Hd, V, int(mask_token_id), _ptr(hidden),
                                             _ptr(row_index), _ptr(num_rows), _ptr(w_vocab),
                                             _ptr(argmax_tok), _ptr(conf), _ptr(entropy),
                                             _ptr(ws), nb, _stream(stream)))


def dbd_lmhead_sample(hidden, w_vocab, num_rows, token, conf, mask_token_id, temperature, seed,
                      step, row_index=None, max_rows=None, ws=None, stream=None, entropy=None):
    """Temperature sampling in the fused LM head: token[row] drawn from
    softmax(l / temperature), conf[row] its probability at temperature 1."""
    V, Hd = w_vocab.shape
    if max_rows is None:
        max_rows = row_index.shape[0] if row_index is not None else hidden.shape[0]
    _need(hidden, torch.bfloat16, (hidden.shape[0], Hd), "hidden")
    _need(w_vocab, torch.bfloat16, (V, Hd), "w_vocab")
    _need(num_rows, torch.int32, (1,), "num_rows")
    need = dbd_lmhead_workspace_size(max_rows, V)
    if ws is None and need:
        ws = _launch_ws(need, hidden.device, stream)
    nb = ws.numel() if ws is not None else 0
    _check(lib().dbd_lmhead_sample(max_rows, Hd, V, int(mask_token_id), _ptr(hidden),
                                   _ptr(row_index), _ptr(num_rows), _ptr(w_vocab),
                                   float(temperature), int(seed) & ((1 << 64) - 1), int(step),
                                   _ptr(token), _ptr(conf), _ptr(entropy), _ptr(ws), nb,
                                   _stream(stream)))


def dbd_prefill_attn(q, k, v, cu_seqlens, out, block_length, softmax_scale=0.0, page_table=None,
                     k_cache=None, v_cache=None, ws=None, stream=None):
    """Block-causal prefill attention over packed prompts; with k_cache /
    v_cache / page_table also the prompts' K/V stored into the pages."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    S = cu_seqlens.shape[0] - 1
    _need(q, torch.bfloat16, (T, Hq, D), "q")
    _need(k, torch.bfloat16, (T, Hkv, D), "k")
    _need(v, torch.bfloat16, (T, Hkv, D), "v")
    _need(out, torch.bfloat16, (T, Hq, D), "out")
    _need(cu_seqlens, torch.int32, (S + 1,), "cu_seqlens")
    P = maxp = npages = 0
    if k_cache is not None:
        npages, _, P, _ = k_cache.shape
        maxp = page_table.shape[1]
        _need(v_cache, torch.bfloat16, tuple(k_cache.shape), "v_cache")
        _need(page_table, torch.int32, (S, maxp), "page_table")
    need = lib().dbd_prefill_workspace_size(S)
    if ws is None:
        ws = _launch_ws(need, q.device, stream)
    _check(lib().dbd_prefill_attn(S, T, Hq, Hkv, D, int(block_length), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(cu_seqlens), float(softmax_scale), _ptr(out), P, maxp,
                                  npages, _ptr(page_table), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(ws), ws.numel(), _stream(stream)))
    return out


def dbd_lmhead_logits(hidden, w_vocab, num_rows, logits, mask_token_id, row_index=None,
                      max_rows=None, stream=None):
    """fp32 logits of the listed rows into logits [max_rows][V]."""
    V, Hd = w_vocab.shape
    if max_rows is None:
        max_rows = row_index.shape[0] if row_index is not None else hidden.shape[0]
    _need(w_vocab, torch.bfloat16, (V, Hd), "w_vocab")
    _need(logits, torch.float32, (logits.shape[0], V), "logits")
    if logits.shape[0] < max_rows:
        raise ValueError("logits needs max_rows rows")
    _check(lib().dbd_lmhead_logits(max_rows, Hd, V, int(mask_token_id), _ptr(hidden),
                                   _ptr(row_index), _ptr(num_rows), _ptr(w_vocab), _ptr(logits),
                                   _stream(stream)))


def dbd_sample_filtered(logits, num_rows, token, conf, mask_token_id, temperature, top_k, top_p,
                        seed, step, row_index=None, max_rows=None, stream=None):
    """Top-k / top-p draw from stored logits (see dbd.h)."""
    M, V = logits.shape
    max_rows = M if max_rows is None else max_rows
    _check(lib().dbd_sample_filtered(max_rows, V, int(mask_token_id), _ptr(logits), _ptr(row_index),
                                     _ptr(num_rows), float(temperature), int(top_k), float(top_p),
                                     int(seed) & ((1 << 64) - 1), int(step), _ptr(token),
                                     _ptr(conf), _stream(stream)))


def dbd_stream_read(data, sink, stream=None):
    """Streaming read of a device buffer (measurement helper)."""
    nbytes = data.numel() * data.element_size()
    _check(lib().dbd_stream_read(_ptr(data), nbytes - nbytes % 16, _ptr(sink), _stream(stream)))


def dbd_mfma_peak(operands, iters, sink, stream=None):
    """Register-resident bf16 MFMA loop (measurement helper); returns the
    launch's floating-point operation count."""
    if operands.numel() * operands.element_size() < lib().dbd_mfma_peak_operand_bytes():
        raise ValueError("operand buffer smaller than dbd_mfma_peak_operand_bytes()")
    if sink.numel() * sink.element_size() < 4 * lib().dbd_mfma_peak_sink_floats():
        raise ValueError("sink smaller than dbd_mfma_peak_sink_floats() floats")
    _check(lib().dbd_mfma_peak(_ptr(operands), int(iters), _ptr(sink), _stream(stream)))
    return lib().dbd_mfma_peak_flops(int(iters))


def dbd_remask_commit(block_tokens, seq_state, argmax_tok, conf, row_index_out, num_rows_out,
                      mask_token_id, dynamic_threshold, flags=0, num_committed=None,
                      stream=None):
    S, B = block_tokens.shape
    _need(block_tokens, torch.int32, (S, B), "block_tokens")
    _need(seq_state, torch.uint8, (S,), "seq_state")
    _need(row_index_out, torch.int32, (S * B,), "row_index_out")
    _need(num_rows_out, torch.int32, (1,), "num_rows_out")
    _check(lib().dbd_remask_commit(S, B, int(mask_token_id), float(dynamic_threshold), int(flags),
                                   _ptr(block_tokens), _ptr(seq_state), _ptr(argmax_tok),
                                   _ptr(conf), _ptr(row_index_out), _ptr(num_rows_out),
                                   _ptr(num_committed), _stream(stream)))


def dbd_remask_commit_rule(block_tokens, seq_state, argmax_tok, conf, row_index_out,
                           num_rows_out, mask_token_id, rule, dynamic_threshold=0.9,
                           tokens_per_step=1, eb_threshold=0.0, entropy=None, flags=0,
                           num_committed=None, stream=None):
    S, B = block_tokens.shape
    _need(block_tokens, torch.int32, (S, B), "block_tokens")
    _need(seq_state, torch.uint8, (S,), "seq_state")
    _need(row_index_out, torch.int32, (S * B,), "row_index_out")
    _need(num_rows_out, torch.int32, (1,), "num_rows_out")
    _check(lib().dbd_remask_commit_rule(S, B, int(mask_token_id), int(rule),
                                        float(dynamic_threshold), int(tokens_per_step),
                                        float(eb_threshold), int(flags), _ptr(block_tokens),
                                        _ptr(seq_state), _ptr(argmax_tok), _ptr(conf),
                                        _ptr(entropy), _ptr(row_index_out), _ptr(num_rows_out),
                                        _ptr(num_committed), _stream(stream)))


@dataclass
class RoundBuffers:
    """Device state of the round that persists across rounds."""
    row_index: torch.Tensor
    num_rows: torch.Tensor
    argmax_tok: torch.Tensor
    conf: torch.Tensor
    block_tokens: torch.Tensor
    seq_state: torch.Tensor
    num_committed: torch.Tensor
    workspace: torch.Tensor


def make_round_args(*, S, B, Hq, Hkv, D, page_size, max_pages_per_seq, Hd, V, mask_token_id,
                    dynamic_threshold, q, k_blk, v_blk, k_cache, v_cache, page_table,
                    prefix_len, attn_out, hidden, w_vocab, bufs: RoundBuffers, flags=0,
                    softmax_scale=0.0, rule=0, tokens_per_step=1, eb_threshold=0.0,
                    entropy=None, save_kv=False, token_stream=None,
                    end_len=None) -> dbd_round_args:
    """The C argument block of one round.  It holds the tensors' raw device
    addresses, not the tensors: the caller keeps every tensor passed here
    alive (and bufs.workspace unchanged) for as long as the block, or a
    graph captured from it, can be launched.  save_kv: the round is a whole
    step for a batch with SAVING sequences (their block K/V go into the
    cache, their blocks are committed)."""
    a = dbd_round_args()
    a.S, a.B, a.Hq, a.Hkv, a.D = S, B, Hq, Hkv, D
    a.page_size, a.max_pages_per_seq, a.Hd, a.V = page_size, max_pages_per_seq, Hd, V
    a.mask_token_id = mask_token_id
    a.dynamic_threshold, a.flags, a.softmax_scale = dynamic_threshold, flags, softmax_scale
    for n, t in (("q", q), ("k_blk", k_blk), ("v_blk", v_blk), ("k_cache", k_cache),
                 ("v_cache", v_cache), ("page_table", page_table), ("prefix_len", prefix_len),
                 ("attn_out", attn_out), ("hidden", hidden), ("w_vocab", w_vocab)):
        setattr(a, n, _ptr(t))
    for n in ("row_index", "num_rows", "argmax_tok", "conf", "block_tokens", "seq_state",
              "num_committed", "workspace"):
        setattr(a, n, _ptr(getattr(bufs, n)))
    a.workspace_bytes = bufs.workspace.numel()
    a.rule, a.tokens_per_step, a.eb_threshold = rule, tokens_per_step, eb_threshold
    a.entropy = _ptr(entropy)
    a.save_kv = int(bool(save_kv))
    a.num_pages = int(k_cache.shape[0]) if save_kv else 0
    a.token_stream = _ptr(token_stream)
    a.stream_cap = int(token_stream.shape[1]) if token_stream is not None else 0
    a.end_len = _ptr(end_len)
    return a


def dbd_round_workspace_size(args: dbd_round_args) -> int:
    return lib().dbd_round_workspace_size(C.byref(args))


def dbd_round(args: dbd_round_args, stream=None):
    _check(lib().dbd_round(C.byref(args), _stream(stream)))


# the static scratch of dbd_round_noalloc (DBD_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def dbd_round_noalloc(args: dbd_round_args, stream=None):
    """dbd_round with the library's static per-device scratch as the
    workspace (args.workspace is not read); allocates nothing."""
    _check(lib().dbd_round_noalloc(C.byref(args), _stream(stream)))


class Graph:
    """n_rounds captured rounds replayed with one launch (dbd_graph_*).  The
    graph keeps the device addresses its rounds were captured with: every
    tensor behind those argument blocks stays alive, at the same address,
    until close()."""

    def __init__(self, args_list):
        arr = (dbd_round_args * len(args_list))(*args_list)
        h = C.c_void_p()
        _check(lib().dbd_graph_create(arr, len(args_list), C.byref(h)))
        self._h = h

    def launch(self, stream=None):
        _check(lib().dbd_graph_launch(self._h, _stream(stream)))

    def close(self):
        if self._h:
            lib().dbd_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dbd_graph_create(args_list):
    return Graph(args_list)


def dbd_validate_inputs(S, B, page_size, max_pages_per_seq, num_pages, V, mask_token_id,
                        page_table=None, prefix_len=None, block_tokens=None, seq_state=None):
    """Host-side check of host (numpy) copies; raises DbdError on a bad input."""
    import numpy as np

    def p(a, dt):
        if a is None:
            return None, None
        a = np.ascontiguousarray(a, dtype=dt)
        return a, a.ctypes.data
    pt, ppt = p(page_table, np.int32)
    pl, ppl = p(prefix_len, np.int32)
    bt, pbt = p(block_tokens, np.int32)
    ss, pss = p(seq_state, np.uint8)
    _check(lib().dbd_validate_inputs(S, B, page_size, max_pages_per_seq, num_pages, V,
                                     mask_token_id, ppt, ppl, pbt, pss))


def dbd_abi_version():
    return lib().dbd_abi_version()
