"""The allocation-free full decode (mac_full_decode_noalloc, the library's
static per-GPU scratch instead of a workspace) against mac_full_decode on the
same inputs: bit for bit, on two calls in a row, the second with a smaller
shape (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from attention_reuse_amd import mac
from attention_reuse_amd import workload as wl

pytestmark = pytest.mark.gpu


def _case(batch, ctx, dtype, d):
    cfg = wl.Workload("noalloc", batch, 32, 8, d, dtype, ctx, 2, 64, 16, 0.6, 5e5, 16, 0.1,
                      (0.05, 0.05))
    K, V = wl.gen_kv(cfg)
    _, q, _, _ = wl.gen_queries(cfg)
    return cfg, K, V, q[:, :, cfg.n_warm]


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0").view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def test_noalloc_full_decode_equals_workspace_version():
    stream = torch.cuda.current_stream().cuda_stream
    # Second call smaller: fewer requests, shorter context, other head dim.
    for batch, ctx, dtype, d, m_list in ((6, 9000, "bf16", 128, [8999, 17, 4096, 64, 1000, 7777]),
                                         (2, 1500, "f32", 64, [1499, 300])):
        print("noalloc case: batch %d ctx %d %s d=%d" % (batch, ctx, dtype, d), flush=True)
        cfg, K, V, q = _case(batch, ctx, dtype, d)
        p = mac.make_params(batch, 32, 8, d,
                            mac.MAC_DTYPE_BF16 if dtype == "bf16" else mac.MAC_DTYPE_F32,
                            64, 16, cfg.capacity, 0.6)
        Kd, Vd, qd = _dev(K), _dev(V), _dev(q)
        m = _dev(np.array(m_list, np.int32))
        wsb = mac.mac_workspace_bytes(p)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
        ref_o = torch.empty((batch, 32, d), device="cuda:0")
        ref_l = torch.empty((batch, 32), device="cuda:0")
        mac.mac_full_decode(p, qd, Kd, Vd, m, ref_o, ref_l, ws, wsb, stream)
        out = torch.full((batch, 32, d), float("nan"), device="cuda:0")
        lse = torch.full((batch, 32), float("nan"), device="cuda:0")
        mac.mac_full_decode_noalloc(p, qd, Kd, Vd, m, out, lse, stream)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        assert torch.isfinite(out).all()
