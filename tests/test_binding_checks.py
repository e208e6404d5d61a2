"""CPU checks of the Python binding's argument checks: a tensor of the wrong
dtype, shape or layout, or one not on a CUDA device, is refused with a
ValueError before its pointer reaches the library (no kernel runs here)."""

import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bd():
    from global_attention_zg_amd import binding
    return binding


def _fwd_args(B=1, S=8, Hq=4, Hkv=1, D=128):
    bf = torch.bfloat16
    return dict(q=torch.zeros(B, S, Hq, D, dtype=bf), k=torch.zeros(B, S, Hkv, D, dtype=bf),
                v=torch.zeros(B, S, Hkv, D, dtype=bf), gate=None,
                q_norm_w=torch.ones(D), k_norm_w=torch.ones(D))


def _call_fwd(bd, a, **kw):
    return bd.zg_attn_fwd(a["q"], a["k"], a["v"], a["gate"], a["q_norm_w"], a["k_norm_w"],
                          window=0, **kw)


@pytest.mark.parametrize("name,bad,msg", [
    ("q", lambda a: a["q"].half(), "torch.bfloat16"),
    ("k", lambda a: a["k"][:, :4], "shape"),
    ("v", lambda a: torch.zeros(1, 8, 1, 256, dtype=torch.bfloat16)[..., :128], "contiguous"),
    ("q_norm_w", lambda a: torch.ones(64), "shape"),
    ("k_norm_w", lambda a: torch.ones(128, dtype=torch.float64), "torch.float32"),
    ("gate", lambda a: torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16), "shape"),
])
def test_fwd_rejects_before_the_library(bd, name, bad, msg):
    a = _fwd_args()
    a[name] = bad(a)
    with pytest.raises(ValueError, match=msg):
        _call_fwd(bd, a)


def test_fwd_rejects_host_tensors_and_bad_outputs(bd):
    a = _fwd_args()
    with pytest.raises(ValueError, match="CUDA device"):
        _call_fwd(bd, a)
    with pytest.raises(ValueError, match="shape"):
        _call_fwd(bd, a, lse=torch.zeros(1, 8, 4))
    with pytest.raises(ValueError, match="torch.bfloat16"):
        _call_fwd(bd, a, out=torch.zeros(1, 8, 4, 128))
    with pytest.raises(ValueError, match="4-d"):
        bd.zg_attn_fwd(torch.zeros(8, 4, 128, dtype=torch.bfloat16), a["k"], a["v"], None,
                       a["q_norm_w"], a["k_norm_w"], window=0)


def test_decode_rejects_before_the_library(bd):
    bf = torch.bfloat16
    q = torch.zeros(2, 8, 128, dtype=bf)
    kc = torch.zeros(2, 2, 64, 128, dtype=bf)
    sl = torch.ones(2, dtype=torch.int32)
    w = torch.ones(128)
    kw = dict(ring=0, window=0, gate=None, q_norm_w=w, k_norm_w=w)
    with pytest.raises(ValueError, match="shape"):
        bd.zg_attn_decode(q, None, None, kc, kc[:, :, :32], sl, **kw)
    with pytest.raises(ValueError, match="torch.int32"):
        bd.zg_attn_decode(q, None, None, kc, kc, sl.long(), **kw)
    with pytest.raises(ValueError, match="sequences"):
        bd.zg_attn_decode(q, None, None, kc[:1], kc[:1], sl, **kw)
    with pytest.raises(ValueError, match="torch.uint8"):
        bd.zg_attn_decode_fp8(q, None, None, kc, kc, sl, k_scale=1.0, v_scale=1.0, **kw)
    with pytest.raises(ValueError, match="shape"):
        bd.zg_attn_decode_noalloc(q, torch.zeros(2, 2, 64, dtype=bf), torch.zeros(2, 2, 64, dtype=bf),
                                  kc, kc, sl, **kw)
    with pytest.raises(ValueError, match="CUDA device"):
        bd.zg_attn_decode_noalloc(q, None, None, kc, kc, sl, **kw)


def test_projection_and_bwd_checks(bd):
    bf = torch.bfloat16
    with pytest.raises(ValueError, match="shape"):
        bd.zg_linear(torch.zeros(4, 256, dtype=bf), torch.zeros(256, 128, dtype=bf))
    with pytest.raises(ValueError, match="contiguous"):
        bd.zg_linear(torch.zeros(256, 4, dtype=bf).t(), torch.zeros(256, 256, dtype=bf).t())
    with pytest.raises(ValueError, match="shape"):
        bd.zg_qkvg_proj(torch.zeros(4, 256, dtype=bf), torch.zeros(10, 256, dtype=bf), 4, 1, True)
    a = _fwd_args()
    with pytest.raises(ValueError, match="shape"):
        bd.zg_attn_bwd(a["q"], a["k"], a["v"], None, a["q_norm_w"], a["k_norm_w"],
                       a["q"], torch.zeros(1, 8, 4), a["q"], window=0)
