"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and rejects malformed or unsupported arguments before any
launch (these calls never reach the GPU, so they run on a CPU-only host)."""

import ctypes
import os

import pytest
import torch

from gated_block_sparse_attn_amd import _native as nat
from gated_block_sparse_attn_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FAKE = 0x1000  # never dereferenced: validation fails before any launch


def lib():
    return nat.lib()


def prob(**kw):
    base = dict(batch=1, n_q_heads=8, n_kv_heads=2, seq_len=1024, head_dim=128, block_size=64,
                budget_k=4, dtype=nat.SAS_BF16, o_dtype=nat.SAS_FP32, sm_scale=0.0, gate_act=0,
                gate_pos=0, gate_rank=0, n_score_heads=0, seq_lens=None, cu_seqlens=None,
                total_tokens=0)
    base.update(kw)
    return nat.SasProblem(**base)


def fwd(p, cap=4, **ptrs):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lg=FAKE, si=FAKE, sc=FAKE, o=FAKE, lse=FAKE)
    a.update(ptrs)
    return lib().sas_gated_attn_fwd(ctypes.byref(p) if p is not None else None, a["q"], a["k"],
                                    a["v"], a["lg"], a["si"], a["sc"], cap, a["o"], a["lse"],
                                    None)


def thr(p, cap=4, **ptrs):
    a = dict(s=FAKE, lg=FAKE, tau=FAKE, si=FAKE, sc=FAKE)
    a.update(ptrs)
    return lib().sas_gate_threshold(ctypes.byref(p), a["s"], a["lg"], a["tau"], a["si"], a["sc"],
                                    cap, None, None)


def bwd(p, cap=4, ws=FAKE * 256, ws_bytes=1 << 40, **ptrs):
    a = {n: FAKE for n in ("q", "k", "v", "o", "do", "lse", "lg", "si", "sc", "dq", "dk", "dv",
                           "dlg")}
    a.update(ptrs)
    return lib().sas_gated_attn_bwd(ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["do"],
                                    a["lse"], a["lg"], a["si"], a["sc"], cap, a["dq"], a["dk"],
                                    a["dv"], a["dlg"], None, ws, ws_bytes, None)


def test_library_exports_every_header_symbol():
    names = nat.header_symbols()
    assert {"sas_gate_threshold", "sas_gated_attn_fwd", "sas_gated_attn_bwd",
            "sas_gated_attn_bwd_workspace_size", "sas_last_error", "sas_abi_version"} <= set(names)
    handle = ctypes.CDLL(nat.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n


def test_abi_version():
    assert lib().sas_abi_version() == 7
    assert api.abi_version() == 7


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), nat.SAS_E_INVALID),
    (dict(n_q_heads=6, n_kv_heads=4), nat.SAS_E_INVALID),
    (dict(budget_k=-1), nat.SAS_E_INVALID),
    (dict(dtype=7), nat.SAS_E_INVALID),
    (dict(o_dtype=3), nat.SAS_E_INVALID),
    (dict(dtype=nat.SAS_FP32, o_dtype=nat.SAS_BF16), nat.SAS_E_INVALID),
    (dict(sm_scale=float("nan")), nat.SAS_E_INVALID),
    (dict(gate_act=3), nat.SAS_E_INVALID),
    (dict(gate_pos=2), nat.SAS_E_INVALID),
    (dict(gate_rank=2), nat.SAS_E_INVALID),
    (dict(n_score_heads=3), nat.SAS_E_INVALID),                # neither Hkv nor Hq
    (dict(gate_rank=1, gate_act=1), nat.SAS_E_UNSUPPORTED),   # hard gates: softmax only
    (dict(gate_rank=1, gate_pos=1), nat.SAS_E_UNSUPPORTED),   # hard gates: inner only
    (dict(head_dim=96), nat.SAS_E_UNSUPPORTED),
    (dict(block_size=128, seq_len=1024), nat.SAS_E_UNSUPPORTED),
    (dict(seq_len=1000), nat.SAS_E_UNSUPPORTED),          # ragged last block
    (dict(seq_len=64 * 8193), nat.SAS_E_UNSUPPORTED),     # too many blocks
    # packed batches: lengths come from cu_seqlens, T within [1, B * N]
    (dict(cu_seqlens=FAKE, seq_lens=FAKE, total_tokens=100), nat.SAS_E_INVALID),
    (dict(cu_seqlens=FAKE, total_tokens=0), nat.SAS_E_INVALID),
    (dict(cu_seqlens=FAKE, total_tokens=1025), nat.SAS_E_INVALID),   # > batch * seq_len
])
def test_invalid_problems_rejected_by_every_entry_point(kw, code):
    p = prob(**kw)
    assert thr(p) == code
    assert lib().sas_last_error()
    assert fwd(p) == code
    assert bwd(p) == code
    assert lib().sas_gated_attn_bwd_workspace_size(ctypes.byref(p), 4) == 0


def test_null_problem_and_null_pointers():
    assert fwd(None) == nat.SAS_E_INVALID
    p = prob()
    assert fwd(p, q=None) == nat.SAS_E_INVALID
    assert fwd(p, lse=None) == nat.SAS_E_INVALID
    assert thr(p, s=None) == nat.SAS_E_INVALID
    assert bwd(p, dlg=None) == nat.SAS_E_INVALID
    assert b"NULL" in lib().sas_last_error()


def bwd_dq(p, cap=4, ws=FAKE * 256, ws_bytes=1 << 40, **ptrs):
    a = {n: FAKE for n in ("q", "k", "v", "o", "do", "lse", "lg", "si", "sc", "dq")}
    a.update(ptrs)
    return lib().sas_gated_attn_bwd_dq(ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["do"],
                                       a["lse"], a["lg"], a["si"], a["sc"], cap, a["dq"], ws,
                                       ws_bytes, None)


def bwd_dkdv(p, cap=4, ws=FAKE * 256, ws_bytes=1 << 40, **ptrs):
    a = {n: FAKE for n in ("q", "k", "v", "do", "lse", "lg", "si", "sc", "dk", "dv", "dlg")}
    a.update(ptrs)
    return lib().sas_gated_attn_bwd_dkdv(ctypes.byref(p), a["q"], a["k"], a["v"], a["do"],
                                         a["lse"], a["lg"], a["si"], a["sc"], cap, a["dk"],
                                         a["dv"], a["dlg"], None, ws, ws_bytes, None)


def test_staged_backward_validates_its_own_outputs():
    """The query-major stage needs o and dq; the key-major stage needs dk, dv
    and dlog_gate (it writes the block log-gate gradient)."""
    p = prob()
    assert bwd_dq(p, o=None) == nat.SAS_E_INVALID
    assert bwd_dq(p, dq=None) == nat.SAS_E_INVALID
    assert bwd_dkdv(p, dlg=None) == nat.SAS_E_INVALID
    assert bwd_dkdv(p, dk=None) == nat.SAS_E_INVALID
    assert bwd_dq(p, ws=None) == nat.SAS_E_WORKSPACE
    assert bwd_dkdv(p, ws_bytes=16) == nat.SAS_E_WORKSPACE
    assert bwd_dq(prob(head_dim=96)) == nat.SAS_E_UNSUPPORTED
    assert bwd_dkdv(prob(head_dim=96)) == nat.SAS_E_UNSUPPORTED


def test_selection_capacity_must_hold_the_budget():
    p = prob(budget_k=8)               # C = 16 -> need cap >= min(8, 15) = 8
    assert thr(p, cap=7) == nat.SAS_E_INVALID
    assert fwd(p, cap=0) == nat.SAS_E_INVALID
    assert bwd(p, cap=3) == nat.SAS_E_INVALID
    p = prob(budget_k=100)             # K >= C: every historical block, cap >= C - 1 = 15
    assert thr(p, cap=14) == nat.SAS_E_INVALID


def test_workspace_size_and_shortfall():
    p = prob()
    n = lib().sas_gated_attn_bwd_workspace_size(ctypes.byref(p), 4)
    assert n > 0 and n % 256 == 0
    # grows with the selection capacity
    assert lib().sas_gated_attn_bwd_workspace_size(ctypes.byref(p), 15) > n
    assert bwd(p, ws_bytes=n - 1) == nat.SAS_E_WORKSPACE
    assert bwd(p, ws=None) == nat.SAS_E_WORKSPACE
    assert bwd(p, ws=FAKE * 256 + 8, ws_bytes=n) == nat.SAS_E_WORKSPACE   # misaligned
    # fp32 / generic shapes need only the Delta buffer
    p32 = prob(dtype=nat.SAS_FP32, o_dtype=nat.SAS_FP32)
    assert 0 < lib().sas_gated_attn_bwd_workspace_size(ctypes.byref(p32), 4) < n


def test_python_binding_rejects_host_tensors_before_calling():
    p = api.Problem(1, 2, 1, 128, 64, 16, 2, "fp32")
    s = torch.zeros(1, 1, 8, 8)
    with pytest.raises(ValueError, match="device tensor"):
        api.gate_threshold(p, s)


# ---------------------------------------------------------------- sparse decode

def dprob(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=64, max_blocks=16,
                pool_blocks=40, budget_k=4, dtype=nat.SAS_BF16, sm_scale=0.0)
    base.update(kw)
    return nat.SasDecodeProblem(**base)


def dsel(p, cap=4, **ptrs):
    a = dict(s=FAKE, n=FAKE, tau=FAKE, si=FAKE, sc=FAKE)
    a.update(ptrs)
    return lib().sas_decode_select(ctypes.byref(p) if p is not None else None, a["s"], a["n"],
                                   a["tau"], a["si"], a["sc"], cap, None, None)


def dattn(p, cap=4, ws=FAKE * 256, ws_bytes=1 << 40, **ptrs):
    a = {n: FAKE for n in ("q", "kp", "vp", "bt", "n", "si", "sc", "o", "lse")}
    a.update(ptrs)
    return lib().sas_decode_attn(ctypes.byref(p), a["q"], a["kp"], a["vp"], a["bt"], a["n"],
                                 a["si"], a["sc"], cap, a["o"], a["lse"], ws, ws_bytes, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), nat.SAS_E_INVALID),
    (dict(n_q_heads=6, n_kv_heads=4), nat.SAS_E_INVALID),
    (dict(budget_k=-1), nat.SAS_E_INVALID),
    (dict(pool_blocks=0), nat.SAS_E_INVALID),
    (dict(max_blocks=0), nat.SAS_E_INVALID),
    (dict(dtype=5), nat.SAS_E_INVALID),
    (dict(sm_scale=float("inf")), nat.SAS_E_INVALID),
    (dict(head_dim=80), nat.SAS_E_UNSUPPORTED),
    (dict(block_size=8), nat.SAS_E_UNSUPPORTED),
    (dict(max_blocks=16385), nat.SAS_E_UNSUPPORTED),
    (dict(n_q_heads=130, n_kv_heads=2), nat.SAS_E_UNSUPPORTED),   # G = 65
])
def test_decode_invalid_problems_rejected(kw, code):
    p = dprob(**kw)
    assert dsel(p) == code
    assert lib().sas_last_error()
    assert dattn(p) == code
    assert lib().sas_decode_workspace_size(ctypes.byref(p), 4) == 0


def test_decode_null_pointers_capacity_and_workspace():
    assert dsel(None) == nat.SAS_E_INVALID
    p = dprob()
    assert dsel(p, s=None) == nat.SAS_E_INVALID
    assert dsel(p, n=None) == nat.SAS_E_INVALID
    assert dattn(p, bt=None) == nat.SAS_E_INVALID
    assert dattn(p, lse=None) == nat.SAS_E_INVALID
    assert b"NULL" in lib().sas_last_error()
    assert dsel(p, cap=3) == nat.SAS_E_INVALID            # cap < min(K, max_blocks - 1)
    assert dsel(p, cap=65535) == nat.SAS_E_INVALID
    n = lib().sas_decode_workspace_size(ctypes.byref(p), 4)
    assert n > 0 and n % 256 == 0
    assert lib().sas_decode_workspace_size(ctypes.byref(p), 8) > n
    assert dattn(p, ws_bytes=n - 1) == nat.SAS_E_WORKSPACE
    assert dattn(p, ws=None) == nat.SAS_E_WORKSPACE
    assert dattn(p, ws=FAKE * 256 + 4, ws_bytes=n) == nat.SAS_E_WORKSPACE


def dattn_noalloc(p, cap=4, **ptrs):
    a = {n: FAKE for n in ("q", "kp", "vp", "bt", "n", "si", "sc", "o", "lse")}
    a.update(ptrs)
    return lib().sas_decode_attn_noalloc(ctypes.byref(p) if p is not None else None, a["q"],
                                         a["kp"], a["vp"], a["bt"], a["n"], a["si"], a["sc"], cap,
                                         a["o"], a["lse"], None, None)


def test_decode_noalloc_validates_before_launch():
    """The allocation-free decode entry point rejects what sas_decode_attn
    rejects, and a problem whose tile partials exceed its fixed scratch
    (SAS_E_WORKSPACE, with the size in the message), all on the host."""
    assert dattn_noalloc(None) == nat.SAS_E_INVALID
    assert dattn_noalloc(dprob(batch=0)) == nat.SAS_E_INVALID
    assert dattn_noalloc(dprob(head_dim=80)) == nat.SAS_E_UNSUPPORTED
    assert dattn_noalloc(dprob(), lse=None) == nat.SAS_E_INVALID
    assert dattn_noalloc(dprob(), cap=3) == nat.SAS_E_INVALID
    # 64 sequences x 8 kv heads x 65 tiles x G 8 x 130 floats = 138 MB > 32 MiB
    big = dprob(batch=64, n_q_heads=64, n_kv_heads=8, max_blocks=8192, pool_blocks=8192,
                budget_k=64)
    assert lib().sas_decode_workspace_size(ctypes.byref(big), 64) > nat.DECODE_SCRATCH_BYTES
    assert dattn_noalloc(big, cap=64) == nat.SAS_E_WORKSPACE
    assert b"fixed scratch" in lib().sas_last_error()


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "sas.h"

int main(void) {
  sas_problem p;
  memset(&p, 0, sizeof p);
  p.batch = 1; p.n_q_heads = 32; p.n_kv_heads = 8; p.seq_len = 32768; p.head_dim = 128;
  p.block_size = 64; p.budget_k = 16; p.dtype = SAS_BF16; p.o_dtype = SAS_BF16;
  p.gate_act = SAS_GATE_SOFTMAX; p.gate_pos = SAS_GATE_INNER; p.gate_rank = SAS_GATE_SOFT;
  if (sas_abi_version() != SAS_ABI_VERSION) { printf("abi %d\n", sas_abi_version()); return 1; }
  if (sas_gated_attn_bwd_workspace_size(&p, 16) == 0) { printf("size 0: %s\n", sas_last_error()); return 2; }
  p.head_dim = 96;   /* unsupported: size 0 and a message */
  if (sas_gated_attn_bwd_workspace_size(&p, 16) != 0 || strlen(sas_last_error()) == 0) return 3;
  printf("ok\n");
  return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    """include/sas.h is plain C (C99): a C program includes it, links against
    the library and calls its host-side entry points (no GPU needed)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib_dir = os.path.join(ROOT, "gated_block_sparse_attn_amd")
    if not os.path.exists(os.path.join(lib_dir, "libsas.so")):
        pytest.skip("library not built")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", lib_dir, "-lsas", "-Wl,-rpath," + lib_dir, "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
