"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before launching anything (no GPU needed)."""

import ctypes
import os
import re

import pytest

from long_context_multimodal_amd import mmsp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmsp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mmsp.LIB_PATH),
                                reason="libmmsp.so not built")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mmsp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert names == sorted(mmsp.SIGNATURES), names
    lib = mmsp.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_abi_version_and_status_strings():
    lib = mmsp.lib()
    assert lib.mmsp_abi_version() == 1
    for code in mmsp.STATUS_NAMES:
        s = lib.mmsp_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.mmsp_status_string(-99).decode() == "unknown status"


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, qp=FAKE, kp=FAKE, sq=128, sk=128, hq=4, hkv=2, d=128,
             scale=0.088, flags=1, o=FAKE, lse=FAKE)
    a.update(kw)
    return mmsp.lib().mmsp_attn_fwd_chunk(a["q"], a["k"], a["v"], a["qp"], a["kp"], a["sq"],
                                          a["sk"], a["hq"], a["hkv"], a["d"], a["scale"],
                                          a["flags"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1), (dict(kp=None), -1),
    (dict(sq=0), -2), (dict(sk=-5), -2), (dict(hq=0), -2), (dict(scale=0.0), -2),
    (dict(scale=-1.0), -2), (dict(scale=float("inf")), -2), (dict(scale=float("nan")), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(flags=8), -3),
    (dict(hq=6, hkv=4), -4), (dict(sq=1 << 30, hq=32), -2),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


def test_fwd_non_causal_allows_null_positions_but_checks_rest():
    assert fwd(flags=0, qp=None, kp=None, d=80) == -3


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, do=FAKE, lse=FAKE, delta=FAKE, qp=FAKE, kp=FAKE, sq=64,
             sk=64, hq=4, hkv=4, d=64, scale=0.125, flags=1, dq=FAKE, dk=FAKE, dv=FAKE)
    a.update(kw)
    return mmsp.lib().mmsp_attn_bwd_chunk(a["q"], a["k"], a["v"], a["do"], a["lse"], a["delta"],
                                          a["qp"], a["kp"], a["sq"], a["sk"], a["hq"], a["hkv"],
                                          a["d"], a["scale"], a["flags"], a["dq"], a["dk"],
                                          a["dv"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), -1), (dict(delta=None), -1), (dict(dq=None), -1), (dict(dv=None), -1),
    (dict(sk=0), -2), (dict(d=32), -3), (dict(hq=7, hkv=2), -4), (dict(flags=16), -3),
    (dict(flags=1 | 4 | 8), -3),                      # both halves skipped
    (dict(flags=1 | 8, dq=None), -1),                 # the dQ half still needs dq_acc
    (dict(flags=1 | 4, dv=None), -1),                 # the dK/dV half still needs dk, dv
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_merge_and_preprocess_reject():
    lib = mmsp.lib()
    assert lib.mmsp_lse_merge(None, FAKE, FAKE, FAKE, 8, 2, 64, None, None) == -1
    assert lib.mmsp_lse_merge(FAKE, FAKE, FAKE, None, 8, 2, 64, None, None) == -1
    assert lib.mmsp_lse_merge(FAKE, FAKE, FAKE, FAKE, 0, 2, 64, None, None) == -2
    assert lib.mmsp_lse_merge(FAKE, FAKE, FAKE, FAKE, 8, 2, 48, None, None) == -3
    # no operand and no bf16 output: nothing to do, nothing launched
    assert lib.mmsp_lse_merge(FAKE, FAKE, None, None, 8, 2, 64, None, None) == 0
    assert lib.mmsp_attn_bwd_preprocess(FAKE, None, 8, 2, 64, FAKE, None, None) == -1
    assert lib.mmsp_attn_bwd_preprocess(FAKE, FAKE, 8, -2, 64, FAKE, None, None) == -2
    assert lib.mmsp_attn_bwd_preprocess(FAKE, FAKE, 8, 2, 100, FAKE, None, None) == -3


def test_shard_balance_rejects_and_workspace():
    lib = mmsp.lib()
    ws = lib.mmsp_shard_balance_workspace_bytes
    assert ws(65536, 8, 0, 0) == 0
    assert ws(65536, 8, 1, 256) == 2 * (65536 // 256) * 4
    sb = lib.mmsp_shard_balance
    assert sb(None, 64, 4, 7, 0, FAKE, None, None, 0, None) == -3        # unknown mode
    assert sb(None, 64, 4, 0, 0, None, None, None, 0, None) == -1        # no perm
    assert sb(None, 64, 4, 1, 4, FAKE, None, FAKE, 1 << 20, None) == -1  # modality w/o labels
    assert sb(None, 0, 4, 0, 0, FAKE, None, None, 0, None) == -2
    assert sb(None, 64, 0, 0, 0, FAKE, None, None, 0, None) == -2
    assert sb(None, 64, 2000, 0, 0, FAKE, None, None, 0, None) == -2     # > 1024 ranks
    assert sb(None, 100, 8, 0, 0, FAKE, None, None, 0, None) == -4       # 100 % 16
    assert sb(FAKE, 96, 4, 1, 8, FAKE, None, FAKE, 1 << 20, None) == -4  # 96 % 64
    assert sb(FAKE, 128, 4, 1, 8, FAKE, None, None, 0, None) == -5       # no workspace
    assert sb(FAKE, 128, 4, 1, 8, FAKE, None, FAKE, 8, None) == -5       # too small
    assert sb(FAKE, 128, 4, 1, 0, FAKE, None, FAKE, 1 << 20, None) == -2


def test_binding_raises_with_code():
    err = mmsp.MMSPError(-4, "where")
    assert err.code == -4 and "MMSP_ERR_DIVISIBILITY" in str(err)


def fwd_packed(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, qp=FAKE, qs=FAKE, kp=FAKE, plan=None, plan_bytes=0, sq=128,
             sk=128, hq=4, hkv=2, d=128, scale=0.088, flags=1, o=FAKE, lse=FAKE)
    a.update(kw)
    return mmsp.lib().mmsp_attn_fwd_chunk_packed(a["q"], a["k"], a["v"], a["qp"], a["qs"],
                                                 a["kp"], a["plan"], a["plan_bytes"], a["sq"],
                                                 a["sk"], a["hq"], a["hkv"], a["d"], a["scale"],
                                                 a["flags"], a["o"], a["lse"], None)


def bwd_packed(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, do=FAKE, lse=FAKE, delta=FAKE, qp=FAKE, qs=FAKE, kp=FAKE,
             plan=None, plan_bytes=0, sq=128, sk=128, hq=4, hkv=2, d=64, scale=0.125, flags=1,
             dq=FAKE, dk=FAKE, dv=FAKE)
    a.update(kw)
    return mmsp.lib().mmsp_attn_bwd_chunk_packed(
        a["q"], a["k"], a["v"], a["do"], a["lse"], a["delta"], a["qp"], a["qs"], a["kp"],
        a["plan"], a["plan_bytes"], a["sq"], a["sk"], a["hq"], a["hkv"], a["d"], a["scale"],
        a["flags"], a["dq"], a["dk"], a["dv"], None)


@pytest.mark.parametrize("fn", [fwd_packed, bwd_packed])
@pytest.mark.parametrize("kw,code", [
    (dict(qs=None), -1), (dict(flags=0), -3), (dict(flags=2), -3), (dict(qp=None), -1),
    (dict(q=None), -1), (dict(sq=0), -2), (dict(d=80), -3), (dict(hq=5, hkv=2), -4),
    (dict(flags=17), -3),  # an undefined bit
    (dict(plan=FAKE, plan_bytes=0), -5), (dict(plan=FAKE, plan_bytes=40), -5),  # plan too small
    (dict(plan=FAKE, plan_bytes=1 << 20, sq=0), -2),
])
def test_packed_attention_rejects(fn, kw, code):
    assert fn(**kw) == code


def test_packed_plan_size_and_rejects():
    lib = mmsp.lib()
    nb = lib.mmsp_attn_packed_plan_bytes
    # header of 8 words, then a list and a work count per tile: forward tiles of
    # 256 query rows, dQ tiles of 128, dK/dV tiles of 128 keys
    assert nb(8192, 8192) == 4 * (8 + 2 * (32 + 64 + 64))
    assert nb(1, 1) == 4 * (8 + 2 * 3)
    assert nb(257, 129) == 4 * (8 + 2 * (2 + 3 + 2))
    assert nb(0, 16) == 0 and nb(16, -1) == 0
    f = lib.mmsp_attn_packed_plan
    need = nb(128, 128)
    assert f(None, FAKE, FAKE, 128, 128, FAKE, need, None) == -1
    assert f(FAKE, None, FAKE, 128, 128, FAKE, need, None) == -1
    assert f(FAKE, FAKE, None, 128, 128, FAKE, need, None) == -1
    assert f(FAKE, FAKE, FAKE, 128, 128, None, need, None) == -1
    assert f(FAKE, FAKE, FAKE, 0, 128, FAKE, need, None) == -2
    assert f(FAKE, FAKE, FAKE, 128, 0, FAKE, need, None) == -2
    assert f(FAKE, FAKE, FAKE, 128, 128, FAKE, need - 4, None) == -5
    g = lib.mmsp_attn_packed_plans  # (q_pos, q_start, k_pos, n_chunks, sq, sk, plans, bytes)
    assert g(None, FAKE, FAKE, 4, 128, 128, FAKE, 4 * need, None) == -1
    assert g(FAKE, FAKE, FAKE, 4, 128, 128, None, 4 * need, None) == -1
    assert g(FAKE, FAKE, FAKE, 0, 128, 128, FAKE, 4 * need, None) == -2
    assert g(FAKE, FAKE, FAKE, 2000, 128, 128, FAKE, 2000 * need, None) == -2   # > 1024 chunks
    assert g(FAKE, FAKE, FAKE, 1024, 128, 1 << 22, FAKE, 1 << 40, None) == -2  # n * sk >= 2^31
    assert g(FAKE, FAKE, FAKE, 4, 128, 128, FAKE, 4 * need - 4, None) == -5    # one plan short


def test_plan_rejected_without_packed_samples():
    import torch
    q = torch.zeros(4, 1, 64, dtype=torch.bfloat16)
    plan = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError):
        mmsp.attn_fwd_chunk(q, q, q, causal=False, plan=plan)
    with pytest.raises(ValueError):
        mmsp.attn_bwd_chunk(q, q, q, q, None, None, None, None, None, causal=False, plan=plan)


def test_packed_shard_balance_rejects():
    f = mmsp.lib().mmsp_shard_balance_packed
    assert f(None, 2, 64, 4, FAKE, None, None, None) == -1
    assert f(FAKE, 2, 64, 4, None, None, None, None) == -1
    assert f(FAKE, 0, 64, 4, FAKE, None, None, None) == -2
    assert f(FAKE, 65, 64, 4, FAKE, None, None, None) == -2
    assert f(FAKE, 2, 0, 4, FAKE, None, None, None) == -2
    assert f(FAKE, 2, 64, 0, FAKE, None, None, None) == -2
    assert f(FAKE, 2, 64, 2048, FAKE, None, None, None) == -2
    assert f(FAKE, 2, 60, 4, FAKE, None, None, None) == -4  # 60 % 8 != 0


def test_rope_rejects():
    f = mmsp.lib().mmsp_rope
    ok = dict(x=FAKE, y=FAKE, dt=0, pos=FAKE, s=16, h=2, d=128, theta=1e7, inv=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["y"], a["dt"], a["pos"], a["s"], a["h"], a["d"], a["theta"], a["inv"],
                 None)
    assert call(x=None) == -1 and call(y=None) == -1 and call(pos=None) == -1
    assert call(dt=2) == -3 and call(inv=2) == -3 and call(d=96) == -3
    assert call(s=0) == -2 and call(h=-1) == -2 and call(theta=1.0) == -2
    assert call(theta=float("inf")) == -2 and call(theta=float("nan")) == -2
    assert call(s=1 << 30, h=32) == -2


def test_device_info_rejects_null():
    lib = mmsp.lib()
    import ctypes
    x = ctypes.c_int32()
    assert lib.mmsp_device_info(0, None, ctypes.byref(x), ctypes.byref(x)) == -1  # MMSP_ERR_NULL
    assert lib.mmsp_device_info(0, ctypes.byref(x), None, ctypes.byref(x)) == -1  # MMSP_ERR_NULL
    assert lib.mmsp_device_info(0, ctypes.byref(x), ctypes.byref(x), None) == -1  # MMSP_ERR_NULL


@pytest.mark.parametrize("name", ["mmsp_shard_gather", "mmsp_shard_scatter"])
def test_shard_gather_scatter_reject(name):
    f = getattr(mmsp.lib(), name)
    # (src, rows_a, idx, rows_b, row_bytes, dst): the row counts swap roles
    assert f(None, 8, FAKE, 8, 256, FAKE, None) == -1
    assert f(FAKE, 8, None, 8, 256, FAKE, None) == -1
    assert f(FAKE, 8, FAKE, 8, 256, None, None) == -1
    assert f(FAKE, 0, FAKE, 8, 256, FAKE, None) == -2
    assert f(FAKE, 8, FAKE, 0, 256, FAKE, None) == -2
    assert f(FAKE, 8, FAKE, 8, 8, FAKE, None) == -2     # under 16 bytes
    assert f(FAKE, 8, FAKE, 8, 264, FAKE, None) == -2   # not a multiple of 16
    assert f(FAKE, 1 << 31, FAKE, 8, 256, FAKE, None) == -2


def test_check_positions_rejects():
    f = mmsp.lib().mmsp_check_positions
    assert f(None, None, 16, FAKE, None) == -1
    assert f(FAKE, None, 16, None, None) == -1
    assert f(FAKE, None, 0, FAKE, None) == -2


def _arr(n, none_at=None):
    a = (ctypes.c_void_p * n)(*([0x1000] * n))
    if none_at is not None:
        a[none_at] = None
    return ctypes.cast(a, ctypes.c_void_p), a


def ring_fwd(**kw):
    n = kw.pop("n", 4)
    ks, ka = _arr(n, kw.pop("k_none_at", None))
    vs, va = _arr(n)
    kps, kpa = _arr(n)
    a = dict(q=FAKE, ks=ks, vs=vs, qp=FAKE, kps=kps, qs=None, n=n, rank=1, sq=128, sk=128, hq=4,
             hkv=2, d=128, scale=0.088, flags=1, o=FAKE, lse=FAKE, of=None)
    a.update(kw)
    return mmsp.lib().mmsp_ring_forward(a["q"], a["ks"], a["vs"], a["qp"], a["kps"], a["qs"],
                                        a["n"], a["rank"], a["sq"], a["sk"], a["hq"], a["hkv"],
                                        a["d"], a["scale"], a["flags"], a["o"], a["lse"], a["of"],
                                        None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=None), -1), (dict(kps=None), -1), (dict(k_none_at=2), -1), (dict(q=None), -1),
    (dict(qp=None), -1), (dict(lse=None), -1),
    (dict(n=0), -2), (dict(rank=4), -2), (dict(rank=-1), -2), (dict(sq=0), -2),
    (dict(scale=0.0), -2),
    (dict(flags=2), -3), (dict(flags=0, qs=FAKE), -3), (dict(d=96), -3),
    (dict(hq=6, hkv=4), -4),
])
def test_ring_forward_rejects(kw, code):
    """Every argument of every chunk is checked before the first launch."""
    assert ring_fwd(**kw) == code


def ring_bwd(**kw):
    n = kw.pop("n", 4)
    ks, ka = _arr(n)
    vs, va = _arr(n)
    kps, kpa = _arr(n)
    dks, dka = _arr(n)
    dvs, dva = _arr(n, kw.pop("dv_none_at", None))
    a = dict(q=FAKE, ks=ks, vs=vs, do=FAKE, o16=FAKE, lse=FAKE, qp=FAKE, kps=kps, qs=None, n=n,
             rank=0, sq=128, sk=128, hq=4, hkv=2, d=128, scale=0.088, flags=1, delta=FAKE,
             dq=FAKE, dks=dks, dvs=dvs)
    a.update(kw)
    return mmsp.lib().mmsp_ring_backward(a["q"], a["ks"], a["vs"], a["do"], a["o16"], a["lse"],
                                         a["qp"], a["kps"], a["qs"], a["n"], a["rank"], a["sq"],
                                         a["sk"], a["hq"], a["hkv"], a["d"], a["scale"],
                                         a["flags"], a["delta"], a["dq"], a["dks"], a["dvs"],
                                         None)


@pytest.mark.parametrize("kw,code", [
    (dict(dks=None), -1), (dict(dv_none_at=3), -1), (dict(do=None), -1), (dict(o16=None), -1),
    (dict(delta=None), -1), (dict(dq=None), -1),
    (dict(n=0), -2), (dict(rank=7), -2), (dict(sk=0), -2),
    (dict(flags=16), -3), (dict(flags=2, qs=FAKE), -3), (dict(d=32), -3),
    (dict(hq=5, hkv=2), -4),
])
def test_ring_backward_rejects(kw, code):
    assert ring_bwd(**kw) == code


def test_native_program_rejects_bad_input(tmp_path):
    """The native C-ABI caller checks its input file before touching the GPU."""
    import subprocess
    from long_context_multimodal_amd.build import TOOL
    if not os.path.exists(TOOL):
        pytest.skip("mmsp_ring_step not built")
    bad = tmp_path / "bad.bin"
    bad.write_bytes(b"\0" * 32)
    r = subprocess.run([TOOL, str(bad), str(tmp_path / "out.bin")], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 1 and "bad header" in r.stderr
    r = subprocess.run([TOOL], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


def test_shard_balance_noalloc_rejects():
    lib = mmsp.lib()
    f = lib.mmsp_shard_balance_noalloc
    assert f(FAKE, 1024, 4, 1, 16, None, None, None) == -1      # no perm
    assert f(None, 1024, 4, 1, 16, FAKE, None, None) == -1      # MODALITY needs labels
    assert f(FAKE, 1024, 4, 7, 16, FAKE, None, None) == -3      # unknown mode
    assert f(FAKE, 0, 4, 0, 0, FAKE, None, None) == -2
    assert f(FAKE, 1000, 4, 1, 16, FAKE, None, None) == -4      # not a multiple of 2*P*g
    # past the static scratch: 131,072 blocks of 16 tokens
    assert f(FAKE, 1 << 21, 8, 1, 16, FAKE, None, None) == -5


def test_header_compiles_as_c(tmp_path):
    """include/mmsp.h is a C header: it compiles as C99 on its own, and as C11
    next to the HIP runtime's header (both declare the same hipStream_t)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = tmp_path / "use.c"
    src.write_text('#include "mmsp.h"\n'
                   "int main(void) { hipStream_t s = 0;\n"
                   "  return mmsp_lse_merge(0, 0, 0, 0, 1, 1, 64, 0, s) == MMSP_ERR_NULL ? 0 : 1; }\n")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c",
                        str(src), "-o", str(tmp_path / "use.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    hip_inc = "/opt/rocm/include"
    if os.path.exists(os.path.join(hip_inc, "hip", "hip_runtime_api.h")):
        src2 = tmp_path / "use_hip.c"
        src2.write_text("#include <hip/hip_runtime_api.h>\n" + src.read_text())
        r = subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                            "-I", hip_inc, "-I", os.path.dirname(HEADER), "-c", str(src2), "-o",
                            str(tmp_path / "use_hip.o")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
