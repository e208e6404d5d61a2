"""The no-allocation decode (zg_attn_decode_noalloc, split partials in the
library's static scratch) against zg_attn_decode with a caller workspace,
through the C ABI: the same kernels and splits, so outputs and appended cache
rows must be equal bit for bit.  Two calls in a row, the second with a
smaller input, so stale scratch contents from the first cannot leak."""

import sys

import numpy as np
import pytest

from global_attention_zg_amd import inputs
from tests import zg_cases as zc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KW = dict(rope_dim=42, rope_theta=10000.0, rms_eps=1e-6)
D = 128


@pytest.fixture(autouse=True)
def _gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def _case(tag, B, Hq, Hkv, cap):
    return dict(
        q=zc.bits((tag, 0, inputs.T_Q), (B, Hq, D)),
        gate=zc.bits((tag, 0, inputs.T_GATE), (B, Hq, D)),
        kc=zc.bits((tag, 0, inputs.T_KCACHE), (B, Hkv, cap, D)),
        vc=zc.bits((tag, 0, inputs.T_VCACHE), (B, Hkv, cap, D)),
        kn=zc.bits((tag, 0, inputs.T_KNEW), (B, Hkv, D)),
        vn=zc.bits((tag, 0, inputs.T_VNEW), (B, Hkv, D)),
        gq=inputs.norm_weight((tag, 0, inputs.T_GQ), D),
        gk=inputs.norm_weight((tag, 0, inputs.T_GK), D),
    )


def _run(fn, c, lens, ring, window, num_splits, gated):
    kc = zc.to_dev(c["kc"], torch)
    vc = zc.to_dev(c["vc"], torch)
    q = zc.to_dev(c["q"], torch)
    out = torch.full_like(q, float("nan"))
    fn(q, zc.to_dev(c["kn"], torch), zc.to_dev(c["vn"], torch), kc, vc,
       torch.tensor(lens, dtype=torch.int32, device="cuda"), ring=ring, window=window,
       gate=zc.to_dev(c["gate"], torch) if gated else None,
       q_norm_w=torch.from_numpy(c["gq"]).cuda(), k_norm_w=torch.from_numpy(c["gk"]).cuda(),
       num_splits=num_splits, out=out, **KW)
    torch.cuda.synchronize()
    return out, kc, vc


# (tag, B, Hq, Hkv, cap, seq_lens, ring, window, num_splits, gated), larger first
CASES = [
    (1301, 16, 32, 8, 2048, [2048, 1, 1500, 777] * 4, 0, 0, 16, False),  # 4.3 MB of partials
    (1302, 4, 32, 8, 3000, [3000, 1, 1777, 2500], 0, 0, 0, False),      # automatic splits
    (1303, 2, 8, 2, 700, [650, 12], 0, 0, 3, False),                    # smaller again
    (1304, 3, 16, 4, 128, [129, 5, 300], 1, 128, 0, True),               # SWA ring: one split
]


def test_noalloc_decode_equals_workspace_decode():
    from global_attention_zg_amd import binding as bd
    for tag, B, Hq, Hkv, cap, lens, ring, window, ns, gated in CASES:
        c = _case(tag, B, Hq, Hkv, cap)
        ref = _run(bd.zg_attn_decode, c, lens, ring, window, ns, gated)
        got = _run(bd.zg_attn_decode_noalloc, c, lens, ring, window, ns, gated)
        for a, b, what in zip(got, ref, ("out", "k_cache", "v_cache")):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (tag, what)
        assert torch.all(torch.isfinite(got[0].float())), tag


def test_noalloc_decode_rejects_too_large_before_launch():
    """64 sequences x 32 heads x 64 splits need 68 MB of partials, more than
    the static array holds: the call is rejected and the output untouched."""
    from global_attention_zg_amd import binding as bd
    c = _case(1305, 64, 32, 8, 256)
    q = zc.to_dev(c["q"], torch)
    out = torch.full_like(q, 7.0)
    with pytest.raises(bd.ZgAttnError) as e:
        bd.zg_attn_decode_noalloc(q, None, None, zc.to_dev(c["kc"], torch),
                                  zc.to_dev(c["vc"], torch),
                                  torch.full((64,), 256, dtype=torch.int32, device="cuda"),
                                  ring=0, window=0, gate=None,
                                  q_norm_w=torch.from_numpy(c["gq"]).cuda(),
                                  k_norm_w=torch.from_numpy(c["gk"]).cuda(), num_splits=64,
                                  out=out, **KW)
    assert e.value.status == bd.ZG_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.all(out.float() == 7.0)
