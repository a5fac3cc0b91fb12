"""A native program (``long_context_multimodal_amd/mmsp_ring_step``, built with
the library) runs one rank's training step through the C-ABI alone. Its
process holds no Python or torch: memory comes from hipMalloc, work goes on
the null stream, and the path is shard balance, mmsp_ring_forward and
mmsp_ring_backward. Its outputs must equal, bit for bit, those of the same
step driven through the binding."""

import os
import subprocess

import numpy as np
import pytest

from long_context_multimodal_amd.build import TOOL
from long_context_multimodal_amd.workloads import normal_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from long_context_multimodal_amd import mmsp
    mmsp.lib()
    return mmsp


@pytest.mark.parametrize("causal", [True, False])
def test_native_program_matches_binding(mm, tmp_path, causal):
    import torch
    mmsp = mm
    assert os.path.exists(TOOL), "mmsp_ring_step is not built"
    n, p, rank, hq, hkv, d = 4096, 4, 1, 8, 2, 128
    shard = n // p
    qb, _ = normal_bf16(71, (shard, hq, d))
    kb, _ = normal_bf16(72, (p, shard, hkv, d))
    vb, _ = normal_bf16(73, (p, shard, hkv, d))
    gb, _ = normal_bf16(74, (shard, hq, d))
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        np.array([0x4d4d5350, n, p, rank, hq, hkv, d, int(causal)], dtype="<i4").tofile(f)
        for a in (qb, kb, vb, gb):
            np.ascontiguousarray(a, dtype="<u2").tofile(f)
    print(f"[native-program] n={n} P={p} rank={rank} hq={hq} hkv={hkv} d={d} causal={causal}",
          flush=True)
    r = subprocess.run([TOOL, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(dst, "rb").read()
    sizes = [("o16", "<u2", shard * hq * d), ("lse", "<f4", hq * shard), ("dq", "<f4", shard * hq * d),
             ("dk", "<f4", p * shard * hkv * d), ("dv", "<f4", p * shard * hkv * d)]
    got, off = {}, 0
    for name, dt, cnt in sizes:
        got[name] = np.frombuffer(raw, dtype=dt, count=cnt, offset=off)
        off += cnt * np.dtype(dt).itemsize
    assert off == len(raw)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()
    q, do = dev(qb), dev(gb)
    ks = [dev(kb[c]) for c in range(p)]
    vs = [dev(vb[c]) for c in range(p)]
    perm, _ = mmsp.shard_balance(n, p, with_inverse=False)
    qp = perm[rank * shard:(rank + 1) * shard]
    kps = [perm[c * shard:(c + 1) * shard] for c in range(p)]
    _, lse, o16 = mmsp.ring_forward_native(q, ks, vs, qp, kps, rank=rank, causal=causal)
    dq, dks, dvs = mmsp.ring_backward_native(q, ks, vs, do, o16, lse, qp, kps, rank=rank,
                                             causal=causal)
    torch.cuda.synchronize()
    want = {"o16": o16.view(torch.int16).cpu().numpy().view(np.uint16).ravel(),
            "lse": lse.cpu().numpy().ravel(), "dq": dq.cpu().numpy().ravel(),
            "dk": torch.stack(dks).cpu().numpy().ravel(),
            "dv": torch.stack(dvs).cpu().numpy().ravel()}
    for name in want:
        assert np.array_equal(got[name].view(np.uint32 if got[name].dtype.itemsize == 4
                                             else np.uint16),
                              want[name].view(np.uint32 if want[name].dtype.itemsize == 4
                                              else np.uint16)), f"{name} differs"
