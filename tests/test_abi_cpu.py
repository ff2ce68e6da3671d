"""The C-ABI library loads without a GPU, exports every declared symbol, and
rejects bad arguments before touching the HIP runtime (no compute calls here)."""
import ctypes
import os
import re

import pytest

from bit_groupwise_weight_amd import lowbit as lb
from bit_groupwise_weight_amd import probe

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADERS = {"lowbit": ["lowbit.h", "lowbit_tuning.h"], "probe": ["lowbit_probe.h"]}

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 6
F32, F16, BF16 = 0, 1, 2
A = 0x10000          # a fake, 256-byte aligned "device" address: never dereferenced


def declared_functions(lib="lowbit"):
    names = set()
    for h in HEADERS[lib]:
        src = open(os.path.join(INCLUDE, h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(lowbit_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_header_and_binding_agree():
    assert declared_functions() == sorted(lb.EXPORTED_SYMBOLS)
    assert declared_functions("probe") == sorted(probe.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lowbit_lib):
    for name in declared_functions():
        assert hasattr(lowbit_lib, name), name
    assert lowbit_lib.lowbit_abi_version() == 3
    plib = probe.load()
    for name in declared_functions("probe"):
        assert hasattr(plib, name), name


def test_probes_are_not_in_the_layer_library(lowbit_lib):
    assert not hasattr(lowbit_lib, "lowbit_probe_stream_read")
    assert not hasattr(lowbit_lib, "lowbit_probe_chase")


def test_size_helpers(lowbit_lib):
    assert lb.lowbit_packed_bytes(4, 4096, 4096) == 4096 * 4096 // 2
    assert lb.lowbit_packed_bytes(3, 10, 96) == 10 * 96 * 3 // 8
    assert lb.lowbit_packed_bytes(8, 10, 96) == 0
    assert lb.lowbit_packed_bytes(3, 10, 100) == 0
    assert lb.lowbit_num_groups(4096, 64) == 64
    assert lb.lowbit_num_groups(4096, 48) == 0
    assert lb.lowbit_num_groups(100, 32) == 0
    assert lb.lowbit_linear_workspace_bytes(4, 64, 1, 4096, 4096, __import__("torch").float16) >= 0


def lin(lib, **kw):
    a = dict(x=A, act=F16, packed=A, scales=A, zeros=A, bias=None, y=A, bits=4, group=64, M=1,
             N=64, K=256, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.lowbit_linear(a["x"], a["act"], a["packed"], a["scales"], a["zeros"], a["bias"],
                             a["y"], a["bits"], a["group"], a["M"], a["N"], a["K"], a["ws"],
                             a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=0), INVALID), (dict(bits=8), INVALID), (dict(group=48), INVALID),
    (dict(group=16), INVALID), (dict(K=96, group=64), INVALID), (dict(N=0), INVALID),
    (dict(K=0), INVALID), (dict(M=-1), INVALID), (dict(x=None), INVALID),
    (dict(packed=None), INVALID), (dict(scales=None), INVALID), (dict(y=None), INVALID),
    (dict(act=7), UNSUPPORTED), (dict(packed=A + 8), MISALIGNED), (dict(x=A + 4), MISALIGNED),
    (dict(y=A + 1), MISALIGNED), (dict(ws=None, ws_bytes=64), WORKSPACE),
    (dict(ws=A + 16, ws_bytes=64), WORKSPACE),
    (dict(M=0), OK),   # M == 0 is a no-op that never reaches the runtime
    (dict(M=0, x=None, y=None), OK), (dict(M=0, packed=None), INVALID),
])
def test_linear_validation(lowbit_lib, kw, status):
    assert lin(lowbit_lib, **kw) == status


def actq(lib, **kw):
    a = dict(x=A, act=BF16, M=4, K=256, xq=A, ascale=A)
    a.update(kw)
    return lib.lowbit_quantize_act_i8(a["x"], a["act"], a["M"], a["K"], a["xq"], a["ascale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(act=3), UNSUPPORTED), (dict(M=-1), INVALID), (dict(K=0), INVALID), (dict(K=48), INVALID),
    (dict(K=(1 << 30) + 32), INVALID), (dict(x=None), INVALID), (dict(xq=None), INVALID),
    (dict(ascale=None), INVALID), (dict(x=A + 8), MISALIGNED), (dict(xq=A + 4), MISALIGNED),
    (dict(ascale=A + 2), MISALIGNED), (dict(M=0), OK), (dict(M=0, x=None, xq=None), OK),
])
def test_quantize_act_validation(lowbit_lib, kw, status):
    assert actq(lowbit_lib, **kw) == status


def lin_a8(lib, **kw):
    a = dict(xq=A, ascale=A, packed=A, scales=A, zeros=A, bias=None, y=A, dt=BF16, bits=4,
             group=32, M=4, N=64, K=256)
    a.update(kw)
    return lib.lowbit_linear_a8(a["xq"], a["ascale"], a["packed"], a["scales"], a["zeros"],
                                a["bias"], a["y"], a["dt"], a["bits"], a["group"], a["M"], a["N"],
                                a["K"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=0), INVALID), (dict(bits=8), INVALID), (dict(group=16), INVALID),
    (dict(K=96, group=64), INVALID), (dict(N=0), INVALID), (dict(M=-1), INVALID),
    (dict(M=16 * 65535 + 1), INVALID), (dict(xq=None), INVALID), (dict(ascale=None), INVALID),
    (dict(y=None), INVALID), (dict(packed=None), INVALID), (dict(zeros=None), INVALID),
    (dict(dt=5), UNSUPPORTED), (dict(xq=A + 4), MISALIGNED), (dict(packed=A + 4), MISALIGNED),
    (dict(ascale=A + 2), MISALIGNED), (dict(y=A + 1), MISALIGNED), (dict(bias=A + 1), MISALIGNED),
    (dict(M=0), OK), (dict(M=0, xq=None, ascale=None, y=None), OK), (dict(M=0, packed=None), INVALID),
])
def test_linear_a8_validation(lowbit_lib, kw, status):
    assert lin_a8(lowbit_lib, **kw) == status
    if status != OK:
        assert lb.lowbit_last_error() != ""


def multi(lib, descs_kw, count=None, **kw):
    a = dict(act=F16, bits=4, group=64, M=1)
    a.update(kw)
    descs = (lb.LinearDesc * max(1, len(descs_kw)))()
    for i, d in enumerate(descs_kw):
        v = dict(x=A, packed=A, scales=A, zeros=A, bias=None, y=A, N=64, K=256)
        v.update(d)
        descs[i] = lb.LinearDesc(v["x"], v["packed"], v["scales"], v["zeros"], v["bias"], v["y"],
                                 v["N"], v["K"])
    n = len(descs_kw) if count is None else count
    return lib.lowbit_linear_multi(descs, n, a["act"], a["bits"], a["group"], a["M"], None)


@pytest.mark.parametrize("descs,kw,status", [
    ([{}], dict(M=0), OK),                                   # M == 0: no launch
    ([], dict(), OK),                                        # count == 0: no launch
    ([{}, {}], dict(M=0), OK),
    ([{}] * 9, dict(M=0), INVALID),                          # more than LOWBIT_MAX_MULTI
    ([{}], dict(M=0, bits=8), INVALID),
    ([{}, dict(K=96)], dict(M=0), INVALID),                  # K % group != 0 in desc 1
    ([{}, dict(packed=A + 8)], dict(M=0), MISALIGNED),
    ([dict(y=None)], dict(M=1), INVALID),
    ([{}], dict(M=0, act=9), UNSUPPORTED),
])
def test_multi_validation(lowbit_lib, descs, kw, status):
    assert multi(lowbit_lib, descs, **kw) == status
    if status != OK:
        assert lb.lowbit_last_error() != ""


def test_multi_negative_count(lowbit_lib):
    assert multi(lowbit_lib, [{}], count=-1, M=0) == INVALID


def test_qmm_path_rejects_fp32(lowbit_lib):
    st = lowbit_lib.lowbit_linear_path(A, F32, A, A, A, None, A, 4, 64, 32, 64, 256, None, 0, 2,
                                       None)
    assert st == UNSUPPORTED
    st = lowbit_lib.lowbit_linear_path(A, F16, A, A, A, None, A, 4, 64, 0, 64, 256, None, 0, 9,
                                       None)
    assert st == INVALID


@pytest.mark.parametrize("args,status", [
    (dict(bits=9), INVALID), (dict(group=100), INVALID), (dict(K=48, group=32), INVALID),
    (dict(w=None), INVALID), (dict(packed=A + 4), MISALIGNED), (dict(w=A + 4), MISALIGNED),
    (dict(sz=5), UNSUPPORTED), (dict(N=-3), INVALID), (dict(wd=3), UNSUPPORTED),
    (dict(wd=F16, w=A + 8), MISALIGNED),
])
def test_quantize_validation(lowbit_lib, args, status):
    a = dict(w=A, wd=F32, bits=4, group=32, N=8, K=64, sz=F16, scales=A, zeros=A, packed=A, codes=None)
    a.update(args)
    st = lowbit_lib.lowbit_quantize_pack(a["w"], a["wd"], a["bits"], a["group"], a["N"], a["K"],
                                         a["sz"], a["scales"], a["zeros"], a["packed"], a["codes"], None)
    assert st == status


def test_tuning_validation(lowbit_lib):
    assert lowbit_lib.lowbit_set_tuning(11, 1) == INVALID
    assert lowbit_lib.lowbit_set_tuning(10, 2) == OK and lowbit_lib.lowbit_set_tuning(10, 0) == OK
    assert lowbit_lib.lowbit_set_tuning(9, 2) == OK and lowbit_lib.lowbit_set_tuning(9, 0) == OK
    assert lowbit_lib.lowbit_set_tuning(7, 2) == OK and lowbit_lib.lowbit_set_tuning(7, 0) == OK
    assert lowbit_lib.lowbit_set_tuning(-1, 1) == INVALID
    assert lowbit_lib.lowbit_set_tuning(0, -2) == INVALID
    assert lowbit_lib.lowbit_set_tuning(3, 0) == OK


def test_library_reads_no_environment():
    """Schedule choices come from the shape and the device only."""
    import subprocess
    syms = subprocess.run(["nm", "-D", "--undefined-only", lb.library_path()], capture_output=True,
                          text=True).stdout
    assert " getenv" not in syms and "secure_getenv" not in syms


def test_status_strings(lowbit_lib):
    for s in range(8):
        assert lb.lowbit_status_string(s)
    assert lb.lowbit_status_string(99) == "unknown status"


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(lb, "_lib", None)
    monkeypatch.setenv("LOWBIT_LIBRARY", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        lb.load()


@pytest.mark.parametrize("args,status", [
    ((None, 1024, 4, A), INVALID), ((A, 1024, 4, None), INVALID), ((A, 0, 4, A), INVALID),
    ((A, 1000, 4, A), INVALID), ((A, 1024, 3, A), INVALID), ((A + 8, 1024, 4, A), MISALIGNED),
    ((A, 1024, 4, A + 2), MISALIGNED)])
def test_probe_stream_read_validation(lowbit_lib, args, status):
    assert probe.load().lowbit_probe_stream_read(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, 16, 4, 0, A), INVALID), ((A, 16, 4, 0, None), INVALID), ((A, 0, 4, 0, A), INVALID),
    ((A, 16, -1, 0, A), INVALID), ((A, 16, (1 << 24) + 1, 0, A), INVALID), ((A, 16, 4, 16, A), INVALID),
    ((A + 2, 16, 4, 0, A), MISALIGNED), ((A, 16, 4, 0, A + 1), MISALIGNED)])
def test_probe_chase_validation(lowbit_lib, args, status):
    assert probe.load().lowbit_probe_chase(*args, None) == status


@pytest.mark.parametrize("M,K,N,bits,group,dtype,planes", [
    (128, 4096, 14336, 4, 128, "bf16", 2),    # bf16 kernel: 112 tiles, split in 2
    (128, 14336, 4096, 4, 128, "bf16", 8),    # bf16 kernel: 32 tiles, split in 8
    (128, 1024, 14336, 4, 128, "bf16", 2),    # bf16 kernel: 128-column tiles at any K
    (128, 1024, 14336, 4, 128, "f16", 0),     # fp16, short loop: 64-column tiles, no split
    (64, 4096, 4096, 4, 64, "f16", 8),        # 4 steps per block: one K group
    (64, 4096, 14336, 4, 64, "f16", 2),       # 16 steps per block: two K groups
    (128, 4096, 14336, 7, 128, "f16", 2),     # 7 bits: 4-wave blocks
    (16, 4096, 4096, 4, 64, "f16", 0),        # fp16 at M <= 16: the small-M kernel, no split
    (32, 4096, 4096, 4, 64, "f16", 8),        # 32-row tiles: split in 8
    (16, 4096, 4096, 4, 64, "bf16", 8),       # bf16 at 16 rows: the tiled kernel
])
def test_mfma_schedule_workspace(lowbit_lib, M, K, N, bits, group, dtype, planes):
    """The MFMA schedule on a 256-CU device, seen through the workspace it asks
    for: one fp32 M x N plane per K split (none without a split)."""
    import torch
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    assert lb.lowbit_linear_workspace_bytes(bits, group, M, N, K, dt) == planes * M * N * 4
