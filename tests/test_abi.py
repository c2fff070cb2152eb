"""The C-ABI library loads, exports what include/mla.h declares, and rejects
bad arguments on the host (no GPU: no call here reaches a kernel).

Validation reads argument values only, so every rejection is checkable with
placeholder pointer values; the clauses mirror the limits
flydsl_sparse_mla_fp8ds_supported states on the flydsl_sparse_mla page.
"""

import ctypes
import os
import re

import pytest

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd import ops

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
A = 0x100000  # a 256-byte aligned placeholder address (never dereferenced)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(ops.SIGNATURES), names
    lib = mla.lib()
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define MLA_ABI_VERSION (\d+)", open(HEADER).read())
    assert mla.lib().mla_abi_version() == int(m.group(1))


def test_status_strings():
    lib = mla.lib()
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(2) == b"MLA_ERR_UNSUPPORTED"


def fwd(**kw):
    args = dict(q=A, T=4, H=16, qst=16 * 576, qsh=576, kv=A, n=100, pitch=656, indptr=A, indices=A, nnz=10,
                scale=1.0, flags=2, out=A, ost=16 * 512, osh=512, lse=A, ws=None, wsb=0, stream=None)
    args.update(kw)
    lib = mla.lib()
    st = lib.mla_sparse_fwd(args["q"], args["T"], args["H"], args["qst"], args["qsh"], args["kv"], args["n"],
                            args["pitch"], args["indptr"], args["indices"], args["nnz"], args["scale"], args["flags"],
                            args["out"], args["ost"], args["osh"], args["lse"], args["ws"], args["wsb"],
                            args["stream"])
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(H=0), UNSUPPORTED),
    (dict(H=17), UNSUPPORTED),
    (dict(T=-1), INVALID),
    (dict(qst=16 * 576 + 1), UNSUPPORTED),
    (dict(qsh=577), UNSUPPORTED),
    (dict(ost=8191), UNSUPPORTED),
    (dict(osh=-2), INVALID),
    (dict(q=A + 2), UNSUPPORTED),
    (dict(out=A + 2), UNSUPPORTED),
    (dict(kv=A + 8), UNSUPPORTED),
    (dict(pitch=672), UNSUPPORTED),
    (dict(pitch=64 * 672), UNSUPPORTED),
    (dict(n=-1), INVALID),
    (dict(nnz=1 << 29), UNSUPPORTED),
    (dict(nnz=-3), INVALID),
    (dict(flags=1 << 7), INVALID),
    (dict(flags=2, lse=None), INVALID),
    (dict(lse=A + 1), INVALID),
    (dict(indptr=A + 2), INVALID),
    (dict(flags=2 | 4, indices=A + 4), INVALID),
    (dict(q=None), INVALID),
    (dict(out=None), INVALID),
    (dict(indptr=None), INVALID),
    (dict(indices=None), INVALID),
    (dict(T=513, flags=2 | (4 << 16)), UNSUPPORTED),  # forced split-KV: at most 512 rows
    (dict(qst=(1 << 62)), INVALID),                      # the q view would span past 2^62 elements
    (dict(osh=(1 << 60)), INVALID),
])
def test_fwd_rejections(kw, status):
    st, msg = fwd(**kw)
    assert st == status, msg
    assert msg


def test_fwd_zero_tokens_is_a_no_op():
    st, _ = fwd(T=0, q=None, out=None, indptr=None, indices=None, lse=None)
    assert st == OK


def fwd_vp(**kw):
    args = dict(q=A, T=4, H=16, qst=16 * 576, qsh=576, kv=A, n=100, pitch=656, indptr=A, indices=A, nnz=10,
                scale=1.0, flags=2, out=A, ost=16 * 512, osh=512, lse=A, w=A, gate=None, gst=0, vo=A,
                vst=16 * 128, vsh=128, ws=None, wsb=0, stream=None)
    args.update(kw)
    lib = mla.lib()
    st = lib.mla_sparse_fwd_v_up_proj(*args.values())
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(H=17), UNSUPPORTED),                 # the forward's own limits still apply
    (dict(T=-1), INVALID),
    (dict(out=A + 8), UNSUPPORTED),            # the projection reads out 16 bytes at a time
    (dict(ost=16 * 512 + 2), UNSUPPORTED),
    (dict(w=A + 8), UNSUPPORTED),
    (dict(vo=A + 2), UNSUPPORTED),
    (dict(vsh=129), UNSUPPORTED),
    (dict(gate=A, gst=2049), UNSUPPORTED),
    (dict(vst=1 << 61), INVALID),
    (dict(w=None), INVALID),
    (dict(vo=None), INVALID),
])
def test_fwd_v_up_proj_rejections(kw, status):
    st, msg = fwd_vp(**kw)
    assert st == status, msg
    assert msg


def test_fwd_v_up_proj_zero_tokens_is_a_no_op():
    st, _ = fwd_vp(T=0, q=None, out=None, indptr=None, indices=None, lse=None, w=None, vo=None)
    assert st == OK


def insert(**kw):
    args = dict(kv_c=A, kst=512, k_pe=A, pst=64, slots=A, T=8, kv=A, n=100, pitch=656, stream=None)
    args.update(kw)
    lib = mla.lib()
    st = lib.mla_cache_insert(args["kv_c"], args["kst"], args["k_pe"], args["pst"], args["slots"], args["T"],
                              args["kv"], args["n"], args["pitch"], args["stream"])
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), INVALID),
    (dict(kst=511), UNSUPPORTED),
    (dict(pst=-64), INVALID),
    (dict(pitch=660), UNSUPPORTED),
    (dict(kv=A + 4), UNSUPPORTED),
    (dict(kv_c=A + 2), UNSUPPORTED),
    (dict(k_pe=A + 1), UNSUPPORTED),
    (dict(slots=A + 4), INVALID),
    (dict(n=-5), INVALID),
    (dict(kv_c=None), INVALID),
    (dict(slots=None), INVALID),
])
def test_insert_rejections(kw, status):
    st, msg = insert(**kw)
    assert st == status, msg


def test_insert_zero_tokens_is_a_no_op():
    st, _ = insert(T=0, kv_c=None, k_pe=None, slots=None)
    assert st == OK


@pytest.mark.parametrize("tokens,nnz,cus,forced,want", [
    (4096, 4096 * 2048, 256, 0, 0),     # sparse prefill: enough rows, no split
    (1024, 1024 * 1024, 256, 0, 0),     # insert + attend
    (4, 512, 256, 0, 0),                # tiny rows fit one chunk
    (8, 8 * 131072, 256, 0, 512),       # long context: one round of 2 x CUs
    (64, 294912, 256, 0, 512),          # paged decode
    (8, 100, 256, 0, 0),
    (300, 300 * 2048, 256, 0, 0),       # > CU-many equal rows: one chunk each at most, no split
    (300, 300 * 2048 + 1, 256, 0, 512), # unequal rows: the plan balances them
    (256, 256 * 2048, 256, 0, 512),     # CU-many equal rows: two chunks each
    (8, 8 * 131072, 256, 7, 2341 + 8),  # forced 7 tiles: ceil(nnz / 448) + T
    (4096, 100, 256, 1, 2 + 4096),      # forced even with many rows
    (0, 0, 256, 0, 0),
])
def test_split_plan(tokens, nnz, cus, forced, want):
    assert mla.split_workgroups(tokens, nnz, cus, forced) == want


def test_split_plan_depends_only_on_host_values():
    lib = mla.lib()
    assert lib.mla_sparse_fwd_split_workgroups(-1, 0, 256, 0) == -1
    assert lib.mla_sparse_fwd_split_workgroups(8, 0, 256, 1 << 5) == -1  # unknown flag bit
    # beyond the forward's own limits there is nothing to plan
    assert lib.mla_sparse_fwd_split_workgroups(8, 1 << 29, 256, 0) == -1
    assert lib.mla_sparse_fwd_split_workgroups((1 << 31) - 1, 100, 256, 0) == -1
    assert lib.mla_sparse_fwd_split_workgroups(8, (1 << 63) - 1, 256, 1 << 16) == -1


def test_workspace_size_of_forced_chunks_needs_no_device():
    lib = mla.lib()
    a256 = lambda x: (x + 255) // 256 * 256
    # 4-tile (256-entry) chunks: at most ceil(1000 / 256) + 8 = 12 chunks
    bound = 4 + 8
    want = a256(bound * 16 * 512 * 4) + a256(bound * 16 * 4) + a256(9 * 4)
    assert lib.mla_sparse_fwd_workspace_size(8, 16, 1000, 4 << 16, 0) == want
    assert lib.mla_sparse_fwd_workspace_size(0, 16, 0, 4 << 16, 0) == 0
    assert lib.mla_sparse_fwd_workspace_size(8, 17, 1000, 4 << 16, 0) == ctypes.c_size_t(-1).value


def epilogue(**kw):
    args = dict(ql=A, qlt=16 * 512, qlh=512, qp=A, qpt=16 * 64, qph=64, kv=A, kvt=512, kp=A, kpt=64, slots=A, T=8,
                H=16, pos=None, cs=None, maxpos=0, mq=A, mqt=16 * 576, mqh=576, rec=A, n=100, pitch=656, stream=None)
    args.update(kw)
    lib = mla.lib()
    st = lib.mla_decode_q_concat_insert(*args.values())
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(H=0), UNSUPPORTED),
    (dict(H=1025), UNSUPPORTED),
    (dict(T=-1), INVALID),
    (dict(qlh=511), UNSUPPORTED),
    (dict(qpt=-64), INVALID),
    (dict(mqh=577), UNSUPPORTED),
    (dict(ql=A + 2), UNSUPPORTED),
    (dict(mq=A + 2), UNSUPPORTED),
    (dict(pitch=672), UNSUPPORTED),
    (dict(rec=A + 8), UNSUPPORTED),
    (dict(n=-1), INVALID),
    (dict(slots=A + 4), INVALID),
    (dict(pos=A), INVALID),                        # positions without a table
    (dict(cs=A, maxpos=16), INVALID),              # a table without positions
    (dict(pos=A, cs=A, maxpos=0), INVALID),
    (dict(pos=A + 4, cs=A, maxpos=16), INVALID),
    (dict(ql=None), INVALID),
    (dict(mq=None), INVALID),
])
def test_epilogue_rejections(kw, status):
    st, msg = epilogue(**kw)
    assert st == status, msg
    assert msg


def test_epilogue_zero_tokens_is_a_no_op():
    st, _ = epilogue(T=0, ql=None, qp=None, kv=None, kp=None, slots=None, mq=None)
    assert st == OK


def gather(**kw):
    args = dict(rec=A, n=1024, pitch=656, bs=64, bt=A, bts=16, btw=16, cu=A, starts=None, B=8, T=100, dst=A,
                dsts=576, stream=None)
    args.update(kw)
    lib = mla.lib()
    st = lib.mla_gather_upconvert(*args.values())
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), INVALID),
    (dict(n=-1), INVALID),
    (dict(B=-1), INVALID),
    (dict(bs=0), INVALID),
    (dict(pitch=660), UNSUPPORTED),
    (dict(rec=A + 8), UNSUPPORTED),
    (dict(dst=A + 8), UNSUPPORTED),
    (dict(dsts=580), UNSUPPORTED),
    (dict(dsts=512), UNSUPPORTED),
    (dict(bt=A + 2), INVALID),
    (dict(cu=None), INVALID),
    (dict(bt=None), INVALID),
    (dict(dst=None), INVALID),
])
def test_gather_rejections(kw, status):
    st, msg = gather(**kw)
    assert st == status, msg
    assert msg


def test_gather_zero_tokens_is_a_no_op():
    st, _ = gather(T=0, dst=None, cu=None, bt=None)
    assert st == OK


def vproj(prepared=False, **kw):
    args = dict(lat=A, lst=16 * 512, lsh=512, w=A, gate=None, gst=0, T=64, H=16, out=A, ost=16 * 128, osh=128,
                stream=None)
    args.update(kw)
    lib = mla.lib()
    st = (lib.mla_v_up_proj_prepared if prepared else lib.mla_v_up_proj)(*args.values())
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), INVALID),
    (dict(H=0), UNSUPPORTED),
    (dict(H=1025), UNSUPPORTED),
    (dict(lst=-8), INVALID),
    (dict(lsh=516), UNSUPPORTED),
    (dict(lat=A + 8), UNSUPPORTED),
    (dict(out=A + 2), UNSUPPORTED),
    (dict(osh=129), UNSUPPORTED),
    (dict(gate=A + 2, gst=2048), UNSUPPORTED),
    (dict(gate=A, gst=2049), UNSUPPORTED),
    (dict(lat=None), INVALID),
    (dict(w=None), INVALID),
])
def test_v_up_proj_rejections(kw, status):
    st, msg = vproj(**kw)
    assert st == status, msg
    assert msg


def test_v_up_proj_zero_tokens_is_a_no_op():
    st, _ = vproj(T=0, lat=None, w=None, out=None)
    assert st == OK


@pytest.mark.parametrize("kw,status", [
    (dict(H=0), UNSUPPORTED),
    (dict(w=A + 2), UNSUPPORTED),  # prepared weights are read 16 bytes at a time
    (dict(w=None), INVALID),
    (dict(lat=A + 8), UNSUPPORTED),
])
def test_v_up_proj_prepared_rejections(kw, status):
    st, msg = vproj(prepared=True, **kw)
    assert st == status, msg
    assert msg


@pytest.mark.parametrize("args,status", [
    ((A, 0, A + (1 << 24), None), UNSUPPORTED),
    ((A, 1025, A + (1 << 30), None), UNSUPPORTED),
    ((None, 16, A, None), INVALID),
    ((A, 16, None, None), INVALID),
    ((A, 16, A + 8 + (1 << 24), None), UNSUPPORTED),  # output not 16-byte aligned
    ((A, 16, A + 4096, None), INVALID),  # overlapping buffers
])
def test_prepare_weights_rejections(args, status):
    lib = mla.lib()
    st = lib.mla_v_up_proj_prepare_weights(*args)
    assert st == status, lib.mla_last_error().decode()
    assert lib.mla_last_error()


def fwd_ex(**kw):
    args = dict(q=A, T=4, H=16, qst=16 * 576, qsh=576, kv=A, n=100, pitch=656, indptr=A, indices=A, nnz=10,
                sink=None, erec=A, en=50, epitch=656, eptr=A, eidx=A, ennz=10, scale=1.0, flags=2, out=A,
                ost=16 * 512, osh=512, lse=A, ws=None, wsb=0, stream=None)
    args.update(kw)
    lib = mla.lib()
    st = lib.mla_sparse_fwd_ex(*args.values())
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(epitch=672), UNSUPPORTED),
    (dict(en=-1), INVALID),
    (dict(en=(1 << 31) - 2), UNSUPPORTED),
    (dict(ennz=(1 << 29) - 10), UNSUPPORTED),   # both lists together reach 2^29
    (dict(erec=A + 8), UNSUPPORTED),
    (dict(eptr=A + 2), INVALID),
    (dict(eidx=None), INVALID),
    (dict(sink=A + 2), INVALID),
    (dict(H=17), UNSUPPORTED),
])
def test_fwd_ex_rejections(kw, status):
    st, msg = fwd_ex(**kw)
    assert st == status, msg
    assert msg


def test_fwd_ex_zero_tokens_is_a_no_op():
    st, _ = fwd_ex(T=0, q=None, out=None, indptr=None, indices=None, lse=None)
    assert st == OK


def prefill(**kw):
    args = dict(q=A, qst=16 * 192, qsh=192, nope=128, kn=A, knt=16 * 128, knh=128, kv=A, kvt=512, kp=A, kpt=64,
                slots=A, T=8, H=16, pos=None, cs=None, maxpos=0, ko=A, kot=16 * 192, koh=192, rec=A, n=100,
                pitch=656, stream=None)
    args.update(kw)
    lib = mla.lib()
    st = lib.mla_prefill_key_concat_insert(*args.values())
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(nope=0), UNSUPPORTED),
    (dict(nope=100), UNSUPPORTED),
    (dict(nope=2048), UNSUPPORTED),
    (dict(H=0), UNSUPPORTED),
    (dict(knh=129), UNSUPPORTED),
    (dict(qst=-2), INVALID),
    (dict(ko=A + 2), UNSUPPORTED),
    (dict(pos=A), INVALID),
    (dict(pos=A, cs=A, maxpos=16, q=None), INVALID),
    (dict(pitch=672), UNSUPPORTED),
    (dict(kn=None), INVALID),
])
def test_prefill_rejections(kw, status):
    st, msg = prefill(**kw)
    assert st == status, msg
    assert msg


def test_prefill_zero_tokens_is_a_no_op():
    st, _ = prefill(T=0, q=None, kn=None, kv=None, kp=None, slots=None, ko=None)
    assert st == OK


C_PROGRAM = r"""
#include "mla.h"
#include <stdio.h>
#include <string.h>

int main(void) {
  mla_status_t st;
  if (mla_abi_version() != MLA_ABI_VERSION) return 1;
  if (mla_status_string(MLA_OK) == NULL || mla_status_string(MLA_ERR_INVALID_ARGUMENT) == NULL) return 2;
  /* a rejected forward (17 heads): nothing is queued, the message says why */
  st = mla_sparse_fwd(NULL, 4, 17, 17 * MLA_QK_DIM, MLA_QK_DIM, NULL, 0, MLA_RECORD_BYTES, NULL, NULL, 0,
                      1.0f, MLA_FLAG_RETURN_LSE, NULL, 17 * MLA_KV_LORA_RANK, MLA_KV_LORA_RANK, NULL, NULL, 0, NULL);
  if (st == MLA_OK || strlen(mla_last_error()) == 0) return 3;
  /* the split-KV launch size from host values only */
  if (mla_sparse_fwd_split_workgroups(8, 8 * 131072, 256, 0u) != 512) return 4;
  if (mla_sparse_fwd_split_workgroups(4096, (int64_t)4096 * 2048, 256, 0u) != 0) return 5;
  puts("ok");
  return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    """include/mla.h is a C header: a C99 program (pedantic, warnings as
    errors) includes it, links libmla.so and calls host-only entry points."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = mla.lib()  # the built library (loads or raises)
    libdir = os.path.dirname(ops.LIB_PATH)
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run([cc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(exe), "-L", libdir, "-lmla", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
    assert lib is not None
