"""The Python binding rejects arguments whose shape or dtype does not match
the sizes it passes to the library, before anything is enqueued (CPU only).

Each case starts from a well-formed argument set of CPU tensors -- which the
binding accepts as far as its shape checks go and then rejects for not being
on the GPU -- and breaks one argument.  The error must come from the shape or
dtype check and name that argument."""
import pytest
import torch

from moe_layer_route_amd import binding

T, H, E, I, k = 5, 64, 4, 96, 2


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _base_bf16():
    return dict(x=_bf(T, H), Wr=_bf(E, H), br=_bf(E), Wgu=_bf(E, H, 2 * I), bgu=_bf(E, 2 * I), Wd=_bf(E, I, H),
                bd=_bf(E, H))


def _base_mxfp4():
    u8 = torch.uint8
    return dict(x=_bf(T, H), Wr=_bf(E, H), br=_bf(E), Wgu_q=torch.zeros((E, 2 * I, H // 2), dtype=u8),
                Wgu_s=torch.zeros((E, H // 32, 2 * I), dtype=u8), bgu=_bf(E, 2 * I),
                Wd_q=torch.zeros((E, H, I // 2), dtype=u8), Wd_s=torch.zeros((E, I // 32, H), dtype=u8),
                bd=_bf(E, H))


def _base_fp8():
    u8 = torch.uint8
    return dict(x=_bf(T, H), Wr=_bf(E, H), br=_bf(E), Wgu_q=torch.zeros((E, 2 * I, H), dtype=u8),
                Wgu_s=torch.ones(E), bgu=_bf(E, 2 * I), Wd_q=torch.zeros((E, H, I), dtype=u8),
                Wd_s=torch.ones(E), bd=_bf(E, H))


def _outs(y_dtype=torch.bfloat16):
    return dict(y=torch.zeros((T, H), dtype=y_dtype), topk_ids=torch.zeros((T, k), dtype=torch.int32),
                topk_w=torch.zeros((T, k), dtype=torch.float32))


def _call(fn, args, **kw):
    with pytest.raises(binding.MoEError) as ei:
        fn(*args.values(), k=k, **kw)
    return str(ei.value)


BROKEN = {
    # argument: (replacement maker given the well-formed tensor)
    "Wr": lambda t: t[:, :-8],
    "br": lambda t: t[:-1],
    "Wgu": lambda t: t[:, :, :-16],
    "bgu": lambda t: t[:-1],
    "Wd": lambda t: t[:, :, :-8],
    "bd": lambda t: t[:, :-8],
    "Wgu_q": lambda t: t[:, :-2],
    "Wgu_s": lambda t: t[:, :-1],
    "Wd_q": lambda t: t[:-1],
    "Wd_s": lambda t: t[:, :, :-4],
}


def _cases(base):
    return [n for n in base() if n in BROKEN]


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "fp8"])
def test_well_formed_arguments_reach_the_device_check(fmt):
    fn, base = {"bf16": (binding.moe_forward, _base_bf16), "mxfp4": (binding.moe_forward_mxfp4, _base_mxfp4),
                "fp8": (binding.moe_forward_fp8, _base_fp8)}[fmt]
    msg = _call(fn, base(), **_outs())
    assert "must be on the GPU" in msg, msg


@pytest.mark.parametrize("fmt,name", [("bf16", n) for n in _cases(_base_bf16)]
                         + [("mxfp4", n) for n in _cases(_base_mxfp4)]
                         + [("fp8", n) for n in _cases(_base_fp8)])
def test_short_weight_is_rejected(fmt, name):
    fn, base = {"bf16": (binding.moe_forward, _base_bf16), "mxfp4": (binding.moe_forward_mxfp4, _base_mxfp4),
                "fp8": (binding.moe_forward_fp8, _base_fp8)}[fmt]
    args = base()
    if fmt == "fp8" and name in ("Wgu_s", "Wd_s"):
        args[name] = torch.ones(E - 1)
    else:
        args[name] = BROKEN[name](args[name]).contiguous()
    msg = _call(fn, args)
    assert "must be on the GPU" not in msg and (name in msg or "Wd" in msg), msg


@pytest.mark.parametrize("out,bad", [
    ("y", torch.zeros((T, H), dtype=torch.float32)),          # float32 y
    ("y", torch.zeros((T - 1, H), dtype=torch.bfloat16)),     # too few rows
    ("topk_ids", torch.zeros((T, k), dtype=torch.int64)),     # int64 ids
    ("topk_ids", torch.zeros((T, k - 1), dtype=torch.int32)),
    ("topk_w", torch.zeros((T, k), dtype=torch.float16)),
    ("topk_w", torch.zeros((T - 1, k), dtype=torch.float32)),
])
@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "fp8"])
def test_bad_output_is_rejected(fmt, out, bad):
    fn, base = {"bf16": (binding.moe_forward, _base_bf16), "mxfp4": (binding.moe_forward_mxfp4, _base_mxfp4),
                "fp8": (binding.moe_forward_fp8, _base_fp8)}[fmt]
    outs = _outs()
    outs[out] = bad
    msg = _call(fn, base(), **outs)
    assert out in msg and "must be on the GPU" not in msg, msg


def test_padded_and_expert_parallel_forms():
    a = _base_bf16()
    # padded: bad y, then a bad n_valid
    msg = _call(binding.moe_forward_padded, a, y=torch.zeros((T, H), dtype=torch.float32))
    assert "y" in msg and "GPU" not in msg
    msg = _call(binding.moe_forward_padded, a, n_valid=torch.zeros(2, dtype=torch.int32))
    assert "n_valid" in msg
    # expert parallel: the local weights must agree with each other, the range with E
    loc = dict(x=a["x"], Wr=a["Wr"], br=a["br"], Wgu=a["Wgu"][:2], bgu=a["bgu"][:2], Wd=a["Wd"][:2],
               bd=a["bd"][:3])
    with pytest.raises(binding.MoEError, match="bd"):
        binding.moe_forward_ep(*loc.values(), 0, k=k)
    loc["bd"] = a["bd"][:2]
    with pytest.raises(binding.MoEError, match="expert range"):
        binding.moe_forward_ep(*loc.values(), 3, k=k)
    with pytest.raises(binding.MoEError, match="y_partial"):
        binding.moe_forward_ep(*loc.values(), 2, k=k, y_partial=torch.zeros((T, H), dtype=torch.bfloat16))
    with pytest.raises(binding.MoEError, match="GPU"):
        binding.moe_forward_ep(*loc.values(), 2, k=k, y_partial=torch.zeros((T, H), dtype=torch.float32))
    m = _base_mxfp4()
    with pytest.raises(binding.MoEError, match="Wd_s"):
        binding.moe_forward_ep_mxfp4(m["x"], m["Wr"], m["br"], m["Wgu_q"][:2], m["Wgu_s"][:2], m["bgu"][:2],
                                     m["Wd_q"][:2], m["Wd_s"][:1], m["bd"][:2], 0, k=k)
    f = _base_fp8()
    with pytest.raises(binding.MoEError, match="Wgu_s"):
        binding.moe_forward_ep_fp8(f["x"], f["Wr"], f["br"], f["Wgu_q"][:2], f["Wgu_s"][:3], f["bgu"][:2],
                                   f["Wd_q"][:2], f["Wd_s"][:2], f["bd"][:2], 0, k=k)


def test_stage_calls():
    a = _base_bf16()
    i32 = torch.int32
    cnt, off = torch.zeros(E, dtype=i32), torch.zeros(E + 1, dtype=i32)
    rows = torch.zeros(T * k, dtype=i32)
    with pytest.raises(binding.MoEError, match="rows"):
        binding.moe_gate_up(a["x"], a["Wgu"], a["bgu"], cnt, off, rows[:-1], k)
    with pytest.raises(binding.MoEError, match="h"):
        binding.moe_gate_up(a["x"], a["Wgu"], a["bgu"], cnt, off, rows, k, h=torch.zeros((T * k, I + 8),
                                                                                        dtype=torch.bfloat16))
    with pytest.raises(binding.MoEError, match="off"):
        binding.moe_gate_up(a["x"], a["Wgu"], a["bgu"], cnt, off[:-1], rows, k)
    h = torch.zeros((T * k, I), dtype=torch.bfloat16)
    with pytest.raises(binding.MoEError, match="o"):
        binding.moe_down(h, a["Wd"], a["bd"], cnt, off, T, k, o=torch.zeros((T * k, H), dtype=torch.bfloat16))
    with pytest.raises(binding.MoEError, match="cnt"):
        binding.moe_down(h, a["Wd"], a["bd"], cnt.long(), off, T, k)
    o = torch.zeros((T * k, H), dtype=torch.float32)
    w = torch.zeros((T, k), dtype=torch.float32)
    with pytest.raises(binding.MoEError, match="pos"):
        binding.moe_combine(o, rows[:-2], w)
    with pytest.raises(binding.MoEError, match="y"):
        binding.moe_combine(o, rows, w, y=torch.zeros((T, H + 8), dtype=torch.bfloat16))
    with pytest.raises(binding.MoEError, match="topk_ids"):
        binding.moe_permute(torch.zeros((T, k), dtype=torch.int64), E)
    with pytest.raises(binding.MoEError, match="topk_w"):
        binding.moe_route(a["x"], a["Wr"], a["br"], k, topk_w=torch.zeros((T, k + 1)))
    with pytest.raises(binding.MoEError, match="GPU"):
        binding.moe_route(a["x"], a["Wr"], a["br"], k)
