"""The C ABI on the host: the library loads, exports every entry point that
include/moe.h declares, and validates arguments with exact status codes
before touching any device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_dispatch_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text, flags=re.M)
    return names


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert len(declared) >= 9
    L = B.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(B.EXPORTED)


def test_status_strings():
    for s in range(7):
        assert B.status_string(s)
    assert "gfx950" in B.status_string(B.MOE_ERR_UNSUPPORTED_DEVICE)


def _cfg(**kw):
    base = dict(T=256, H=256, I=128, E=8, k=2)
    base.update(kw)
    return B.Config(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, B.MOE_OK),
    ({"T": 0}, B.MOE_ERR_INVALID_ARG),
    ({"H": 200}, B.MOE_ERR_INVALID_ARG),          # H must be a multiple of 128
    ({"I": 64}, B.MOE_ERR_INVALID_ARG),
    ({"E": 0}, B.MOE_ERR_INVALID_ARG),
    ({"E": 2048}, B.MOE_ERR_INVALID_ARG),
    ({"k": 9}, B.MOE_ERR_INVALID_ARG),            # k > E
    ({"E": 64, "k": 33}, B.MOE_ERR_INVALID_ARG),  # k > 32
    ({"n_shared": 2}, B.MOE_ERR_INVALID_ARG),
    ({"macrobatch": 100}, B.MOE_ERR_INVALID_ARG),  # does not divide T
    ({"macrobatch": 128, "minibatch": 48}, B.MOE_ERR_INVALID_ARG),
    ({"macrobatch": 128, "minibatch": 64}, B.MOE_OK),
    ({"macrobatch": 128, "capacity_rows": 255}, B.MOE_ERR_CAPACITY),  # < 128 * 2 rows
    ({"macrobatch": 128, "capacity_rows": 256}, B.MOE_OK),
    ({"capacity_rows": -1}, B.MOE_ERR_INVALID_ARG),
    ({"precision": 7}, B.MOE_ERR_INVALID_ARG),
    ({"recompute": True}, B.MOE_OK),
    ({"macrobatch": 64, "acc_experts": 3}, B.MOE_OK),
    ({"macrobatch": 64, "acc_experts": 100}, B.MOE_OK),        # more than E: E
    ({"acc_experts": -1}, B.MOE_ERR_INVALID_ARG),
])
def test_config_validation(kw, status):
    assert B.validate_config(_cfg(**kw)) == status


def test_ring_rows_and_workspace():
    one = _cfg()
    assert B.ring_rows(one) == 256 * 2
    two = _cfg(macrobatch=64)
    assert B.ring_rows(two) == 2 * 64 * 2
    assert B.ring_rows(_cfg(macrobatch=64, capacity_rows=1000)) == 1000
    ws1 = B.workspace_size(one)
    assert ws1 > 256 * 2 * (3 * 128 + 256) * 2          # at least the backward ring (dg|du, hw, dX)
    big = B.Config(T=2048, H=4096, I=1024, E=512, k=10)
    assert B.workspace_size(big) > 20480 * (3 * 1024 + 4096) * 2
    with pytest.raises(B.MoEError):
        B.workspace_size(_cfg(T=0))


def test_entry_points_reject_bad_arguments_before_any_device_work():
    L = B.lib()
    cfg = _cfg().c()
    fake = ctypes.c_void_p(1 << 20)        # never dereferenced: validation fails first
    sched = B.moe_sched()
    # null schedule arrays
    assert L.moe_schedule(ctypes.byref(cfg), fake, ctypes.byref(sched), fake, 1 << 40, None) in (
        B.MOE_ERR_INVALID_ARG, B.MOE_ERR_WORKSPACE)
    # workspace too small
    s_ok = B.moe_sched(*([1 << 20] * 7))
    assert L.moe_schedule(ctypes.byref(cfg), fake, ctypes.byref(s_ok), fake, 16, None) == B.MOE_ERR_WORKSPACE
    # misaligned workspace
    assert L.moe_schedule(ctypes.byref(cfg), fake, ctypes.byref(s_ok), ctypes.c_void_p((1 << 20) + 8),
                          1 << 40, None) == B.MOE_ERR_WORKSPACE
    # bad config
    bad = _cfg(k=99).c()
    assert L.moe_forward(ctypes.byref(bad), ctypes.byref(s_ok), fake, None, fake, None, fake,
                         1 << 40, None) == B.MOE_ERR_INVALID_ARG
    # misaligned activations
    w = B.moe_weights(*([1 << 20] * 6))
    sv = B.moe_saved(*([1 << 20] * 4))
    assert L.moe_forward(ctypes.byref(cfg), ctypes.byref(s_ok), ctypes.c_void_p((1 << 20) + 2),
                         ctypes.byref(w), fake, ctypes.byref(sv), fake, 1 << 40,
                         None) == B.MOE_ERR_INVALID_ARG
    g = B.moe_grads(*([1 << 20] * 6))
    assert L.moe_backward(ctypes.byref(cfg), ctypes.byref(s_ok), ctypes.byref(sv), fake,
                          ctypes.byref(w), fake, fake, ctypes.byref(g), None, None, fake, 1 << 40,
                          None) == B.MOE_ERR_INVALID_ARG      # dw is required
    assert L.moe_check_device_error(None, 0, None, None) == B.MOE_ERR_INVALID_ARG


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "mixture_experts_layer_dispatch_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "synth_inputs" not in text, fn


def test_mx_weight_buffers_match_the_header_layout():
    """alloc_weights_mx gives every field of moe_weights_mx, codes [.., rows, K]
    and K-step-major scales [.., K/128, rows, 4], as include/moe.h lays them out."""
    cfg = B.Config(T=8, H=256, I=384, E=3, k=1, n_shared=1)
    q = B.alloc_weights_mx(cfg, "cpu")
    assert sorted(q) == sorted(B.MX_FIELDS)
    E, H, I = cfg.E, cfg.H, cfg.I
    dims = {"gate_": (I, H), "up_": (I, H), "down_": (H, I),
            "gate_t": (H, I), "up_t": (H, I), "down_t": (I, H)}
    for name, (rows, K) in dims.items():
        for pre, lead in (("w_", (E,)), ("s_", ())):
            assert tuple(q[pre + name + "q"].shape) == (*lead, rows, K)
            assert tuple(q[pre + name + "s"].shape) == (*lead, K // 128, rows, 4)


def test_binding_raises_when_the_library_is_missing(monkeypatch, tmp_path):
    """No fallback: without the built library every entry point raises."""
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libmoe_mi355x.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
    with pytest.raises(RuntimeError, match="missing"):
        B.workspace_size(_cfg())
    with pytest.raises(RuntimeError, match="missing"):
        B.validate_config(_cfg())


def _cpu_buffers(cfg):
    """Correctly shaped buffers of every argument, on the CPU (the binding's
    checks run before any device work, so nothing here reaches the library)."""
    import torch

    bf = torch.bfloat16
    ws = torch.empty(B.workspace_size(cfg), dtype=torch.uint8)
    sched = B.alloc_schedule(cfg, "cpu")
    x = torch.zeros(cfg.T, cfg.H, dtype=bf)
    w = {"w_gate": torch.zeros(cfg.E, cfg.I, cfg.H, dtype=bf),
         "w_up": torch.zeros(cfg.E, cfg.I, cfg.H, dtype=bf),
         "w_down": torch.zeros(cfg.E, cfg.H, cfg.I, dtype=bf)}
    return dict(ws=ws, sched=sched, x=x, y=x.clone(), w=w, saved=B.alloc_saved(cfg, "cpu"),
                grads=B.alloc_grads(cfg, "cpu"), dw=torch.zeros(cfg.T, cfg.k),
                dl=torch.zeros(cfg.T, cfg.E), logits=torch.zeros(cfg.T, cfg.E))


def test_binding_checks_every_tensor_before_the_call():
    """Wrong shape, dtype or layout of any tensor raises ValueError on the host,
    before anything is enqueued (the C side can only see pointers)."""
    import torch

    cfg = _cfg()
    b = _cpu_buffers(cfg)
    # everything right but on the CPU: the device check is the one that fires
    with pytest.raises(ValueError, match="GPU"):
        B.moe_schedule(cfg, b["logits"], b["sched"], b["ws"])
    with pytest.raises(ValueError, match="shape"):
        B.moe_schedule(cfg, torch.zeros(cfg.T, cfg.E + 1), b["sched"], b["ws"])
    with pytest.raises(ValueError, match="dtype"):
        B.moe_schedule(cfg, b["logits"].double(), b["sched"], b["ws"])
    bad = dict(b["sched"], row_of_slot=torch.zeros(cfg.S - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="row_of_slot"):
        B.moe_schedule(cfg, b["logits"], bad, b["ws"])
    with pytest.raises(ValueError, match="workspace"):
        B.moe_schedule(cfg, b["logits"], b["sched"], b["ws"][:16])
    # forward: a non-contiguous x, a y of the wrong shape, weights of another E
    with pytest.raises(ValueError, match="contiguous"):
        B.moe_forward(cfg, b["sched"], torch.zeros(cfg.H, cfg.T, dtype=torch.bfloat16).t(),
                      b["w"], b["y"], b["saved"], b["ws"])
    with pytest.raises(ValueError, match="y: shape"):
        B.moe_forward(cfg, b["sched"], b["x"], b["w"], b["y"][:-1], b["saved"], b["ws"])
    w_bad = dict(b["w"], w_down=torch.zeros(cfg.E + 1, cfg.H, cfg.I, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="w_down"):
        B.moe_forward(cfg, b["sched"], b["x"], w_bad, b["y"], b["saved"], b["ws"])
    # bf16 saved activations handed to an MXFP8 config (which saves fp32)
    mx = B.Config(**{**cfg.__dict__, "precision": B.PREC_MXFP8})
    bmx = _cpu_buffers(mx)
    bmx["w"]["mx"] = B.alloc_weights_mx(mx, "cpu")
    with pytest.raises(ValueError, match="saved\\['g'\\]: dtype"):
        B.moe_forward(mx, bmx["sched"], bmx["x"], bmx["w"], bmx["y"], b["saved"], bmx["ws"])
    with pytest.raises(ValueError, match="mx"):
        B.moe_forward(mx, bmx["sched"], bmx["x"], b["w"], bmx["y"], bmx["saved"], bmx["ws"])
    # backward: dw of [T, k+1], d_logits of [T, k], a gradient of the wrong dtype
    args = (cfg, b["sched"], b["saved"], b["x"], b["w"], b["x"], b["y"], b["grads"])
    with pytest.raises(ValueError, match="dw"):
        B.moe_backward(*args, torch.zeros(cfg.T, cfg.k + 1), b["dl"], b["ws"])
    with pytest.raises(ValueError, match="d_logits"):
        B.moe_backward(*args, b["dw"], torch.zeros(cfg.T, cfg.k), b["ws"])
    g_bad = dict(b["grads"], d_w_up=b["grads"]["d_w_up"].float())
    with pytest.raises(ValueError, match="d_w_up"):
        B.moe_backward(*args[:-1], g_bad, b["dw"], b["dl"], b["ws"])
    with pytest.raises(ValueError, match="GPU"):
        B.moe_backward(*args, b["dw"], None, b["ws"])
    # the quantiser: an output array of the wrong shape
    q = B.alloc_weights_mx(mx, "cpu")
    q["w_up_ts"] = q["w_up_ts"][:-1]
    with pytest.raises(ValueError, match="w_up_ts"):
        B.moe_quantize_weights_mxfp8(mx, b["w"], q)


def test_config_flags_and_recompute_workspace():
    """Unknown flag bits are rejected; recompute mode adds one macrobatch's g, u
    (bf16, or fp32 in MXFP8 mode) to the workspace and saves nothing."""
    bad = _cfg().c()
    bad.flags = 2
    assert B.lib().moe_validate_config(ctypes.byref(bad)) == B.MOE_ERR_INVALID_ARG
    for prec, es in ((B.PREC_BF16, 2), (B.PREC_MXFP8, 4)):
        base = _cfg(macrobatch=64, n_shared=1, precision=prec)
        rc = _cfg(macrobatch=64, n_shared=1, precision=prec, recompute=True)
        extra = B.workspace_size(rc) - B.workspace_size(base)
        assert extra >= 2 * 64 * 2 * 128 * es + 2 * 64 * 128 * es     # routed + shared g, u
        assert B.alloc_saved(rc, "cpu") == {}


def test_workspace_regions_of_the_mx_activation_codes():
    mx = _cfg(precision=B.PREC_MXFP8)
    total = B.workspace_size(mx)
    seen = []
    for name, n in (("x_codes", 256 * 256), ("x_scales", 256 * 256 // 32),
                    ("dy_codes", 256 * 256), ("dy_scales", 256 * 256 // 32)):
        off, nb = B.workspace_region(mx, name)
        assert nb == n and off % 256 == 0 and off + nb <= total
        seen.append((off, off + nb))
    kcap = -(-(256 * 2 + 32 * 8) // 128) * 128          # the macrobatch's rows padded group by group
    for name, n in (("wgrad_x_codes", 256 * kcap), ("wgrad_x_scales", 256 * kcap // 32),
                    ("wgrad_block_offsets", (8 + 1) * 4)):
        off, nb = B.workspace_region(mx, name)
        assert nb >= n and off % 256 == 0 and off + nb <= total
        seen.append((off, off + nb))
    seen.sort()
    assert all(a[1] <= b[0] for a, b in zip(seen, seen[1:]))        # disjoint
    with pytest.raises(B.MoEError):
        B.workspace_region(_cfg(), "x_codes")                        # bf16: no codes
    with pytest.raises(B.MoEError):
        B.workspace_region(mx, "nothing")


def test_noalloc_schedule_rejects_configs_beyond_its_scratch():
    """moe_schedule_noalloc checks its fixed scratch on the host: a schedule
    needing more than 16 MiB of histograms is refused before any device work."""
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)                # never dereferenced
    s_ok = B.moe_sched(*([1 << 20] * 7))
    huge = B.Config(T=262144, H=128, I=128, E=1024, k=10).c()     # 5120 blocks x 1024 experts
    assert L.moe_schedule_noalloc(ctypes.byref(huge), fake, ctypes.byref(s_ok), None) == B.MOE_ERR_WORKSPACE
    assert L.moe_schedule_noalloc(ctypes.byref(_cfg().c()), fake, ctypes.byref(B.moe_sched()),
                                  None) == B.MOE_ERR_INVALID_ARG


def test_mx4_weight_buffers_match_the_header_layout():
    """alloc_weights_mx4 gives every field of moe_weights_mx4: E2M1 codes two per
    byte [.., rows, K/2] and K-step-major scales [.., K/128, rows, 4]."""
    cfg = B.Config(T=8, H=256, I=384, E=3, k=1, n_shared=1, precision=B.PREC_MXFP4)
    q = B.alloc_weights_mx4(cfg, "cpu")
    assert sorted(q) == sorted(B.MX4_FIELDS)
    E, H, I = cfg.E, cfg.H, cfg.I
    for name, (rows, K) in {"gate_": (I, H), "up_": (I, H), "down_": (H, I)}.items():
        for pre, lead in (("w_", (E,)), ("s_", ())):
            assert tuple(q[pre + name + "q"].shape) == (*lead, rows, K // 2)
            assert tuple(q[pre + name + "s"].shape) == (*lead, K // 128, rows, 4)
    assert B.validate_config(cfg) == B.MOE_OK
    assert B.validate_config(B.Config(T=8, H=256, I=384, E=3, k=1, precision=3)) == B.MOE_ERR_INVALID_ARG


def test_accumulators_are_sized_by_acc_experts():
    """Several macrobatches keep fp32 running sums of the weight gradients
    (4 bytes per weight) for acc_experts experts (0 or more than E: E); one
    macrobatch keeps none."""
    E, H, I = 8, 256, 128
    full = B.workspace_size(_cfg(macrobatch=64))
    assert B.workspace_size(_cfg(macrobatch=64, acc_experts=E)) == full
    assert B.workspace_size(_cfg(macrobatch=64, acc_experts=100)) == full
    three = B.workspace_size(_cfg(macrobatch=64, acc_experts=3))
    assert full - three == (E - 3) * 3 * H * I * 4
    assert B.workspace_size(_cfg(acc_experts=3)) == B.workspace_size(_cfg())
