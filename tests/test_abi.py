"""The C-ABI library on the host: it loads without a GPU, exports every
symbol include/dbd.h declares, and rejects invalid arguments before any HIP
call (so these run with no device)."""
import os
import re
import ctypes
import subprocess

import numpy as np
import pytest

from block_diffusion_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dbd.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\**\s*(dbd_[a-z_0-9]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_round_calls():
    names = declared_functions()
    for n in ("dbd_attn_paged", "dbd_lmhead_conf", "dbd_remask_commit", "dbd_round",
              "dbd_lmhead_conf_entropy", "dbd_remask_commit_rule",
              "dbd_attn_paged_save", "dbd_commit_block", "dbd_lmhead_sample",
              "dbd_prefill_attn", "dbd_prefill_workspace_size", "dbd_lmhead_logits",
              "dbd_sample_filtered", "dbd_stream_read", "dbd_stream_read_sink_words",
              "dbd_mfma_peak", "dbd_mfma_peak_operand_bytes", "dbd_mfma_peak_sink_floats",
              "dbd_mfma_peak_flops",
              "dbd_graph_create", "dbd_graph_launch", "dbd_graph_destroy",
              "dbd_attn_workspace_size", "dbd_lmhead_workspace_size",
              "dbd_round_workspace_size", "dbd_validate_inputs", "dbd_last_error",
              "dbd_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = api.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    assert api.dbd_abi_version() == api.ABI_VERSION == 4
    assert lib.dbd_round_args_size() == ctypes.sizeof(api.dbd_round_args)


def _attn(**kw):
    a = dict(S=2, B=4, Hq=4, Hkv=2, D=64, P=16, maxp=3)
    a.update(kw)
    return api.lib().dbd_attn_paged(a["S"], a["B"], a["Hq"], a["Hkv"], a["D"], a["P"], a["maxp"],
                                    16, 16, 16, 16, 16, 16, 16, 0.0, 16, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), api.DBD_ERR_INVALID_ARG), (dict(B=65), api.DBD_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), api.DBD_ERR_INVALID_ARG), (dict(P=24), api.DBD_ERR_INVALID_ARG),
    (dict(P=0), api.DBD_ERR_INVALID_ARG), (dict(D=96), api.DBD_ERR_UNSUPPORTED),
    (dict(S=0), api.DBD_ERR_INVALID_ARG), (dict(maxp=0), api.DBD_ERR_INVALID_ARG)])
def test_attn_rejects(kw, status):
    assert _attn(**kw) == status
    assert api.lib().dbd_last_error()


def test_attn_null_and_misaligned_pointers():
    L = api.lib()
    st = L.dbd_attn_paged(2, 4, 4, 2, 64, 16, 3, None, 16, 16, 16, 16, 16, 16, 0.0, 16, None, 0, None)
    assert st == api.DBD_ERR_INVALID_ARG and b"q is NULL" in L.dbd_last_error()
    st = L.dbd_attn_paged(2, 4, 4, 2, 64, 16, 3, 16, 18, 16, 16, 16, 16, 16, 0.0, 16, None, 0, None)
    assert st == api.DBD_ERR_INVALID_ARG and b"aligned" in L.dbd_last_error()
    st = L.dbd_attn_paged(2, 4, 4, 2, 64, 16, 3, 16, 16, 16, 16, 16, 16, 16, float("nan"), 16, None, 0, None)
    assert st == api.DBD_ERR_INVALID_ARG


def test_attn_workspace_required():
    L = api.lib()
    need = api.dbd_attn_workspace_size(128, 4, 32, 8, 128, 256, 16)
    assert need > 0
    st = L.dbd_attn_paged(128, 4, 32, 8, 128, 256, 16, 16, 16, 16, 16, 16, 16, 16, 0.0, 16, None, 0, None)
    assert st == api.DBD_ERR_WORKSPACE
    st = L.dbd_attn_paged(128, 4, 32, 8, 128, 256, 16, 16, 16, 16, 16, 16, 16, 16, 0.0, 16, 16, need - 1, None)
    assert st == api.DBD_ERR_WORKSPACE
    # the tile plan and the split-segment partials always need some space
    # (two partial slots per wave of the launch: the SDAR-4B launch above
    # runs fewer, deeper-ringed waves than this small one, so the sizes are
    # not ordered by the problem size)
    small = api.dbd_attn_workspace_size(2, 4, 4, 2, 64, 16, 3)
    assert small > 0
    st = L.dbd_attn_paged(2, 4, 4, 2, 64, 16, 3, 16, 16, 16, 16, 16, 16, 16, 0.0, 16, None, 0, None)
    assert st == api.DBD_ERR_WORKSPACE
    st = L.dbd_attn_paged(2, 4, 4, 2, 64, 16, 3, 16, 16, 16, 16, 16, 16, 16, 0.0, 16, 16, small - 1, None)
    assert st == api.DBD_ERR_WORKSPACE


@pytest.mark.parametrize("args,status", [
    ((16, 100, 1024, 5), api.DBD_ERR_INVALID_ARG),      # Hd not a multiple of 128
    ((16, 192, 1024, 5), api.DBD_ERR_INVALID_ARG),
    ((16, 128, 1, 0), api.DBD_ERR_INVALID_ARG),         # V < 2
    ((16, 128, 1024, 1024), api.DBD_ERR_INVALID_ARG),   # mask id out of range
    ((16, 128, 1024, -1), api.DBD_ERR_INVALID_ARG),
    ((-1, 128, 1024, 5), api.DBD_ERR_INVALID_ARG)])
def test_lmhead_rejects(args, status):
    L = api.lib()
    assert L.dbd_lmhead_conf(*args, 16, None, 16, 16, 16, 16, 256, 1 << 20, None) == status


def _save(**kw):
    a = dict(S=2, B=4, Hq=4, Hkv=2, D=64, P=16, maxp=3, npages=6, state=16, kc=16)
    a.update(kw)
    return api.lib().dbd_attn_paged_save(a["S"], a["B"], a["Hq"], a["Hkv"], a["D"], a["P"],
                                         a["maxp"], a["npages"], 16, 16, 16, a["kc"], 16, 16, 16,
                                         a["state"], 0.0, 16, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), api.DBD_ERR_INVALID_ARG), (dict(D=96), api.DBD_ERR_UNSUPPORTED),
    (dict(npages=0), api.DBD_ERR_INVALID_ARG), (dict(state=None), api.DBD_ERR_INVALID_ARG),
    (dict(kc=None), api.DBD_ERR_INVALID_ARG), (dict(state=17), api.DBD_ERR_INVALID_ARG),
    (dict(), api.DBD_ERR_WORKSPACE)])
def test_attn_save_rejects(kw, status):
    assert _save(**kw) == status


@pytest.mark.parametrize("S,B,prefix,stream,cap,end,status", [
    (0, 4, 16, None, 0, None, api.DBD_ERR_INVALID_ARG),
    (2, 65, 16, None, 0, None, api.DBD_ERR_INVALID_ARG),
    (2, 4, None, None, 0, None, api.DBD_ERR_INVALID_ARG),     # prefix_len is written
    (2, 4, 16, 16, 0, None, api.DBD_ERR_INVALID_ARG),         # a stream needs a capacity
    (2, 4, 16, 18, 8, None, api.DBD_ERR_INVALID_ARG),         # misaligned stream
    (2, 4, 16, None, 0, 20, api.DBD_ERR_INVALID_ARG)])        # misaligned end lengths
def test_commit_block_rejects(S, B, prefix, stream, cap, end, status):
    L = api.lib()
    st = L.dbd_commit_block(S, B, 5, 16, 16, prefix, stream, cap, end, 16, 16, None)
    assert st == status and L.dbd_last_error()


def _prefill(**kw):
    a = dict(S=2, T=40, Hq=8, Hkv=2, D=128, B=4, cu=16, ws=256, wsb=1 << 12, kc=None)
    a.update(kw)
    return api.lib().dbd_prefill_attn(a["S"], a["T"], a["Hq"], a["Hkv"], a["D"], a["B"], 16, 16, 16,
                                      a["cu"], 0.0, 16, 16, 4, 8, 16, a["kc"], 16, a["ws"],
                                      a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(S=0), api.DBD_ERR_INVALID_ARG), (dict(B=0), api.DBD_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), api.DBD_ERR_INVALID_ARG), (dict(Hq=24, Hkv=2), api.DBD_ERR_INVALID_ARG),
    (dict(Hq=512, Hkv=2), api.DBD_ERR_INVALID_ARG),
    (dict(D=96), api.DBD_ERR_UNSUPPORTED), (dict(cu=None), api.DBD_ERR_INVALID_ARG),
    (dict(T=1 << 22, Hkv=8, Hq=8), api.DBD_ERR_INVALID_ARG),
    (dict(ws=None), api.DBD_ERR_WORKSPACE), (dict(wsb=8), api.DBD_ERR_WORKSPACE),
    (dict(ws=272), api.DBD_ERR_INVALID_ARG), (dict(kc=18), api.DBD_ERR_INVALID_ARG)])
def test_prefill_rejects(kw, status):
    assert _prefill(**kw) == status


def test_lmhead_workspace_required():
    L = api.lib()
    assert L.dbd_lmhead_conf(16, 128, 1024, 5, 16, None, 16, 16, 16, 16, None, 0, None) == api.DBD_ERR_WORKSPACE


@pytest.mark.parametrize("S,B,tau,flags,status", [
    (0, 4, 0.9, 0, api.DBD_ERR_INVALID_ARG), (8193, 4, 0.9, 0, api.DBD_ERR_INVALID_ARG),
    (2, 0, 0.9, 0, api.DBD_ERR_INVALID_ARG), (2, 65, 0.9, 0, api.DBD_ERR_INVALID_ARG),
    (2, 4, float("nan"), 0, api.DBD_ERR_INVALID_ARG), (2, 4, 0.9, 8, api.DBD_ERR_INVALID_ARG)])
def test_remask_rejects(S, B, tau, flags, status):
    L = api.lib()
    assert L.dbd_remask_commit(S, B, 5, tau, flags, 16, 16, 16, 16, 16, 16, None, None) == status


@pytest.mark.parametrize("rule,eb,entropy,flags,status", [
    (4, 0.0, 16, 0, api.DBD_ERR_INVALID_ARG),                 # unknown rule
    (-1, 0.0, 16, 0, api.DBD_ERR_INVALID_ARG),
    (3, float("nan"), 16, 0, api.DBD_ERR_INVALID_ARG),        # NaN budget
    (3, 1.0, None, 0, api.DBD_ERR_INVALID_ARG),               # entropy rule needs entropy
    (3, 1.0, 18, 0, api.DBD_ERR_INVALID_ARG),                 # misaligned entropy
    (1, 0.0, None, 4, api.DBD_ERR_INVALID_ARG)])              # unknown flag
def test_remask_rule_rejects(rule, eb, entropy, flags, status):
    L = api.lib()
    st = L.dbd_remask_commit_rule(2, 4, 5, rule, 0.9, 1, eb, flags, 16, 16, 16, 16, entropy,
                                  16, 16, None, None)
    assert st == status and L.dbd_last_error()


@pytest.mark.parametrize("T", [0.0, -1.0, float("inf"), float("nan")])
def test_lmhead_sample_rejects_temperature(T):
    L = api.lib()
    st = L.dbd_lmhead_sample(16, 128, 1024, 5, 16, None, 16, 16, T, 1, 0, 16, 16, None, 256,
                             1 << 20, None)
    assert st == api.DBD_ERR_INVALID_ARG and b"temperature" in L.dbd_last_error()


@pytest.mark.parametrize("T,k,p", [(0.0, 0, 1.0), (1.0, -1, 1.0), (1.0, 0, float("nan"))])
def test_sample_filtered_rejects(T, k, p):
    L = api.lib()
    st = L.dbd_sample_filtered(4, 100, 5, 16, None, 16, T, k, p, 1, 0, 16, 16, None)
    assert st == api.DBD_ERR_INVALID_ARG and L.dbd_last_error()


def test_lmhead_logits_requires_output():
    L = api.lib()
    assert L.dbd_lmhead_logits(16, 128, 1024, 5, 16, None, 16, 16, None, None) == api.DBD_ERR_INVALID_ARG


def test_lmhead_entropy_requires_output():
    L = api.lib()
    st = L.dbd_lmhead_conf_entropy(16, 128, 1024, 5, 16, None, 16, 16, 16, 16, None, 256,
                                   1 << 20, None)
    assert st == api.DBD_ERR_INVALID_ARG and b"entropy is NULL" in L.dbd_last_error()


def test_round_rejects():
    a = api.dbd_round_args()
    a.S, a.B, a.Hq, a.Hkv, a.D, a.page_size, a.max_pages_per_seq = 2, 4, 4, 2, 64, 16, 3
    a.Hd, a.V, a.mask_token_id, a.dynamic_threshold = 256, 1024, 1023, 0.9
    with pytest.raises(api.DbdError) as e:
        api.dbd_round(a, stream=0)
    assert e.value.status == api.DBD_ERR_INVALID_ARG
    with pytest.raises(api.DbdError):
        api.dbd_graph_create([a])
    a.rule, a.eb_threshold = 3, 1.0          # entropy rule without an entropy buffer
    with pytest.raises(api.DbdError) as e:
        api.dbd_round(a, stream=0)
    assert e.value.status == api.DBD_ERR_INVALID_ARG
    # a SAVING step needs the page count it may write to
    a.rule = 0
    for n in ("q", "k_blk", "v_blk", "k_cache", "v_cache", "page_table", "prefix_len",
              "attn_out", "hidden", "w_vocab", "row_index", "num_rows", "argmax_tok", "conf",
              "block_tokens", "seq_state"):
        setattr(a, n, 256)
    a.save_kv, a.num_pages = 1, 0
    with pytest.raises(api.DbdError) as e:
        api.dbd_round(a, stream=0)
    assert b"num_pages" in api.lib().dbd_last_error()
    a.num_pages, a.token_stream, a.stream_cap = 4, 256, 0
    with pytest.raises(api.DbdError) as e:
        api.dbd_round(a, stream=0)
    assert b"stream_cap" in api.lib().dbd_last_error()
    a.token_stream, a.gate_on_rows = None, 1    # a SAVING step is never gated off
    with pytest.raises(api.DbdError) as e:
        api.dbd_round(a, stream=0)
    assert b"gate_on_rows" in api.lib().dbd_last_error()


def test_validate_inputs():
    ok = dict(S=2, B=4, page_size=16, max_pages_per_seq=3, num_pages=4, V=1024, mask_token_id=1023)
    pt = np.array([[1, -1, -1], [0, 3, 2]], np.int32)
    api.dbd_validate_inputs(**ok, page_table=pt, prefix_len=[16, 37],
                            block_tokens=np.full((2, 4), 1023), seq_state=[2, 2])
    with pytest.raises(api.DbdError):
        api.dbd_validate_inputs(**ok, page_table=pt, prefix_len=[17, 37])   # needs page 2 of seq 0
    with pytest.raises(api.DbdError):
        api.dbd_validate_inputs(**ok, page_table=pt, prefix_len=[16, 49])   # > 3 pages * 16
    with pytest.raises(api.DbdError):
        api.dbd_validate_inputs(**ok, block_tokens=np.full((2, 4), 1024))
    with pytest.raises(api.DbdError):
        api.dbd_validate_inputs(**ok, seq_state=[2, 7])
    bad = dict(ok, mask_token_id=1024)
    with pytest.raises(api.DbdError):
        api.dbd_validate_inputs(**bad)


def test_mfma_ceiling_host_checks():
    """The MFMA ceiling helper validates its arguments on the host and
    reports its work: 1024 workgroups x 4 waves x 64 instructions of
    2*32*32*16 flops per iteration."""
    L = api.lib()
    assert L.dbd_mfma_peak_operand_bytes() == 64 * 16 * 64 * 16
    assert L.dbd_mfma_peak_sink_floats() == 1024 * 256
    assert L.dbd_mfma_peak_flops(3) == 1024 * 4 * 3 * 64 * 2 * 32 * 32 * 16
    assert L.dbd_mfma_peak_flops(0) == 0.0
    assert L.dbd_mfma_peak(16, 0, 16, None) == api.DBD_ERR_INVALID_ARG
    assert L.dbd_mfma_peak(16, 4097, 16, None) == api.DBD_ERR_INVALID_ARG
    assert L.dbd_mfma_peak(None, 4, 16, None) == api.DBD_ERR_INVALID_ARG
    assert L.dbd_mfma_peak(16, 4, 8, None) == api.DBD_ERR_INVALID_ARG     # misaligned sink


def test_round_noalloc_rejects():
    """dbd_round_noalloc checks its arguments like dbd_round, ignores the
    workspace fields, and rejects a round whose workspace exceeds its static
    scratch (the SDAR-8B shapes need about 104 MiB) before any HIP call."""
    a = api.dbd_round_args()
    a.S, a.B, a.Hq, a.Hkv, a.D, a.page_size, a.max_pages_per_seq = 64, 16, 32, 8, 128, 256, 32
    a.Hd, a.V, a.mask_token_id, a.dynamic_threshold = 4096, 151936, 151669, 0.75
    with pytest.raises(api.DbdError) as e:
        api.dbd_round_noalloc(a, stream=0)
    assert e.value.status == api.DBD_ERR_INVALID_ARG          # NULL tensors
    for n in ("q", "k_blk", "v_blk", "k_cache", "v_cache", "page_table", "prefix_len",
              "attn_out", "hidden", "w_vocab", "row_index", "num_rows", "argmax_tok", "conf",
              "block_tokens", "seq_state"):
        setattr(a, n, 256)
    a.workspace, a.workspace_bytes = None, 0
    assert api.lib().dbd_round_workspace_size(ctypes.byref(a)) > api.NOALLOC_SCRATCH_BYTES
    with pytest.raises(api.DbdError) as e:
        api.dbd_round_noalloc(a, stream=0)
    assert e.value.status == api.DBD_ERR_WORKSPACE
    assert b"static scratch" in api.lib().dbd_last_error()
