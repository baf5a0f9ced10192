"""The Python binding's argument checks (host only, no GPU needed).

The C ABI sees only pointers and sizes, so the binding checks every tensor's dtype,
shape, contiguity and device before the call and raises ValueError for any mismatch.
With host tensors of the right dtypes and shapes the only remaining complaint is the
device, which is checked last: every case here therefore builds host tensors, breaks one
rule and expects that rule's message (the intact set expects the device message)."""
import pytest
import torch

import prefill_token_amd as smla


def fwd_args(s_q=3, h=64, d=512, topk=640, n=100):
    return dict(
        q=torch.zeros((s_q, h, d), dtype=torch.bfloat16),
        kv_pool=torch.zeros((n, d), dtype=torch.uint8),
        kv_scales=torch.zeros((n, d // 32), dtype=torch.uint8),
        indices=torch.zeros((s_q, topk), dtype=torch.int32),
        topk_length=torch.zeros((s_q,), dtype=torch.int32),
        positions=torch.zeros((s_q,), dtype=torch.int32),
        norm_w=torch.zeros((d,), dtype=torch.float32),
        out_fp8=torch.zeros((s_q, h, d), dtype=torch.uint8),
        out_scales=torch.zeros((s_q, h, d // 32), dtype=torch.uint8),
    )


def call_fwd(a, **kw):
    smla.sparse_mla_fwd(a["q"], a["kv_pool"], a["kv_scales"], a["indices"], a["topk_length"], a["positions"],
                        a["norm_w"], a["out_fp8"], a["out_scales"], sm_scale=0.04, rope_dim=64, **kw)


def test_fwd_intact_host_tensors_fail_on_device_only():
    with pytest.raises(ValueError, match="must be on a GPU"):
        call_fwd(fwd_args())


@pytest.mark.parametrize("name,bad,msg", [
    ("q", torch.zeros((3, 64, 512), dtype=torch.float16), "q must have dtype"),
    ("q", torch.zeros((3, 64 * 512), dtype=torch.bfloat16), "q must have 3 dimensions"),
    ("kv_pool", torch.zeros((100, 256), dtype=torch.uint8), "kv_pool rows"),
    ("kv_pool", torch.zeros((100, 512), dtype=torch.int8), "kv_pool must have dtype"),
    ("kv_scales", torch.zeros((99, 16), dtype=torch.uint8), "kv_scales must have shape"),
    ("kv_scales", torch.zeros((100, 16), dtype=torch.int32), "kv_scales must have dtype"),
    ("kv_scales", None, "kv_scales is required"),
    ("indices", torch.zeros((3, 640), dtype=torch.int64), "indices must have dtype"),
    ("indices", torch.zeros((2, 640), dtype=torch.int32), "indices must have 3 rows"),
    ("topk_length", torch.zeros((4,), dtype=torch.int32), "topk_length must have shape"),
    ("positions", torch.zeros((3,), dtype=torch.int64), "positions must have dtype"),
    ("norm_w", torch.zeros((512,), dtype=torch.bfloat16), "norm_w must have dtype"),
    ("norm_w", torch.zeros((128,), dtype=torch.float32), "norm_w must have shape"),
    ("out_fp8", torch.zeros((3, 64, 256), dtype=torch.uint8), "out_fp8 must have shape"),
    ("out_scales", torch.zeros((3, 32, 16), dtype=torch.uint8), "out_scales must have shape"),
])
def test_fwd_rejections(name, bad, msg):
    a = fwd_args()
    a[name] = bad
    with pytest.raises(ValueError, match=msg):
        call_fwd(a)


def test_fwd_non_contiguous_and_optional_outputs():
    a = fwd_args()
    a["indices"] = torch.zeros((640, 3), dtype=torch.int32).t()
    with pytest.raises(ValueError, match="indices must be contiguous"):
        call_fwd(a)
    with pytest.raises(ValueError, match="out_f32 must have shape"):
        call_fwd(fwd_args(), out_f32=torch.zeros((3, 64, 511), dtype=torch.float32))
    with pytest.raises(ValueError, match="workspace must have dtype"):
        call_fwd(fwd_args(), workspace=torch.zeros((1024,), dtype=torch.float32))


def test_fwd_bf16_pool_takes_no_scales():
    a = fwd_args(d=128, h=8)
    a["kv_pool"] = torch.zeros((100, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="kv_scales must be None"):
        call_fwd(a)
    a["kv_scales"] = None
    with pytest.raises(ValueError, match="must be on a GPU"):
        call_fwd(a)


def test_insert_rejections():
    kv = torch.zeros((4, 512), dtype=torch.bfloat16)
    pos = torch.zeros((4,), dtype=torch.int32)
    w = torch.zeros((512,), dtype=torch.float32)
    pool = torch.zeros((100, 512), dtype=torch.uint8)
    sc = torch.zeros((100, 16), dtype=torch.uint8)
    kw = dict(rope_dim=64, n_swa=64)
    with pytest.raises(ValueError, match="must be on a GPU"):
        smla.sparse_mla_kv_insert(kv, pos, w, pool, sc, **kw)
    with pytest.raises(ValueError, match="positions must have shape"):
        smla.sparse_mla_kv_insert(kv, pos[:3], w, pool, sc, **kw)
    with pytest.raises(ValueError, match="kv_scales must have shape"):
        smla.sparse_mla_kv_insert(kv, pos, w, pool, sc[:99], **kw)
    with pytest.raises(ValueError, match="kv must have dtype"):
        smla.sparse_mla_kv_insert(kv.float(), pos, w, pool, sc, **kw)


def test_index_rejections():
    pos = torch.zeros((4,), dtype=torch.int32)
    lg = torch.zeros((4, 2048), dtype=torch.bfloat16)
    nv = torch.zeros((4,), dtype=torch.int32)
    idx = torch.zeros((4, 640), dtype=torch.int32)
    L = torch.zeros((4,), dtype=torch.int32)
    kw = dict(window=128, self_in_window=False, n_swa=8192, cmp_base=8192, k_cmp=512)
    with pytest.raises(ValueError, match="must be on a GPU"):
        smla.sparse_mla_build_index(pos, lg, nv, idx, L, **kw)
    with pytest.raises(ValueError, match="must be on a GPU"):
        smla.sparse_mla_build_index(pos, lg, None, idx, L, **kw)
    with pytest.raises(ValueError, match="indices must have 4 rows"):
        smla.sparse_mla_build_index(pos, lg, nv, idx[:3], L, **kw)
    with pytest.raises(ValueError, match="n_valid must have shape"):
        smla.sparse_mla_build_index(pos, lg, nv[:2], idx, L, **kw)
    with pytest.raises(ValueError, match="logits must have dtype"):
        smla.sparse_mla_build_index(pos, lg.float(), nv, idx, L, **kw)


def test_wo_a_rejections():
    x = torch.zeros((4, 64, 512), dtype=torch.uint8)
    xs = torch.zeros((4, 64, 16), dtype=torch.uint8)
    w = torch.zeros((32, 128, 1024), dtype=torch.uint8)
    ws = torch.zeros((32, 128, 32), dtype=torch.uint8)
    y = torch.zeros((4, 32, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must be on a GPU"):
        smla.sparse_mla_wo_a(x, xs, w, ws, y, heads_per_group=2)
    with pytest.raises(ValueError, match="w_fp8 must have shape"):
        smla.sparse_mla_wo_a(x, xs, w, ws, y, heads_per_group=1)
    with pytest.raises(ValueError, match="heads_per_group must divide"):
        smla.sparse_mla_wo_a(x, xs, w, ws, y, heads_per_group=3)
    with pytest.raises(ValueError, match="y must have shape"):
        smla.sparse_mla_wo_a(x, xs, w, ws, y[:, :16], heads_per_group=2)
    with pytest.raises(ValueError, match="w_scales must have shape"):
        smla.sparse_mla_wo_a(x, xs, w, ws[:, :, :16], y, heads_per_group=2)
