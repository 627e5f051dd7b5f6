"""C-ABI checks that need no GPU: every symbol in include/k3moe.h is exported, and argument and
state errors come back as status codes before any device work."""
import ctypes
import os
import re

import pytest

import latent_width_expert_amd as k3
from latent_width_expert_amd import LayerConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k3moe.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(k3moe_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 12
    L = ctypes.CDLL(k3.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared in k3moe.h but not exported"


def _cfg(**kw):
    base = dict(d_model=256, latent=128, hidden=96, n_experts=16, top_k=4, n_shared=1, shared_hidden=96,
                latent_moe=1, act="bf16", max_tokens=64, rms_eps=1e-6)
    base.update(kw)
    return LayerConfig(**base)


@pytest.mark.parametrize("bad", [dict(d_model=250), dict(latent=100), dict(hidden=0), dict(n_experts=0),
                                 dict(n_experts=4096), dict(top_k=0), dict(top_k=17), dict(top_k=65, n_experts=100),
                                 dict(n_shared=5), dict(max_tokens=0), dict(latent_moe=2), dict(shared_hidden=33)])
def test_create_rejects_bad_config(bad):
    with pytest.raises(k3.K3MoEError) as ei:
        k3.K3MoE(_cfg(**bad))
    assert ei.value.code == k3.EINVAL
    assert str(ei.value)


def test_sizes_and_state_errors():
    m = k3.K3MoE(_cfg())
    assert m.weight_bytes > 0 and m.workspace_bytes > 0
    # forward before pack: state error, no device work
    assert m.forward_raw(None, 4, None, None) == k3.ESTATE
    assert "not packed" in m.last_error()
    # token count checks come first
    assert m.forward_raw(None, 65, None, None) == k3.ETOOBIG
    assert m.forward_raw(None, -1, None, None) == k3.EINVAL
    # pack with NULL weights / buffer
    L = k3.lib()
    assert L.k3moe_pack_weights(m._h, None, None, None) == k3.EINVAL
    w = k3.Weights()
    w.include_dense = 1
    assert L.k3moe_pack_weights(m._h, ctypes.byref(w), 256, None) == k3.EINVAL
    assert "router" in m.last_error()
    w.include_dense = 0
    w.routed_first, w.routed_count = 10, 10
    assert L.k3moe_pack_weights(m._h, ctypes.byref(w), 256, None) == k3.EINVAL
    assert "outside" in m.last_error()


def test_k3_shape_pool_size():
    """At K3 shape the packed routed pool is exactly the canonical MXFP4 size (no padding)."""
    m = k3.K3MoE(LayerConfig(d_model=7168, latent=3584, hidden=3072, n_experts=896, top_k=16, n_shared=2,
                             shared_hidden=3072, max_tokens=8192))
    routed = 896 * (3 * 3584 * 3072 // 2 + 3 * 3584 * 3072 // 32)
    assert routed == 15_722_348_544
    assert routed <= m.weight_bytes < routed + 200_000_000


def test_stage_names():
    assert k3.stage_names() == ["x_gemm", "topk", "route", "gateup", "down", "combine", "y_gemm"]


def test_null_ctx_error_text():
    L = k3.lib()
    assert L.k3moe_create(None, None) == k3.EINVAL
    assert L.k3moe_last_error(None)


def _c_layout(struct, fields):
    """sizeof and offsetof of a C struct of include/k3moe.h, from a small C program built with gcc."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lines = [f'  printf("size %zu\\n", sizeof({struct}));']
    lines += [f'  printf("{f} %zu\\n", offsetof({struct}, {f}));' for f in fields]
    src = "#include <stddef.h>\n#include <stdio.h>\n#include \"k3moe.h\"\nint main(void) {\n" + "\n".join(lines) + \
          "\n  return 0;\n}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), c, "-o", exe],
                       check=True, capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return {k: int(v) for k, v in (line.split() for line in out.splitlines())}


@pytest.mark.parametrize("struct,cls", [("k3moe_config", "Config"), ("k3moe_mx", "MX"), ("k3moe_lora", "Lora"),
                                        ("k3moe_weights", "Weights"), ("k3moe_taps", "Taps")])
def test_struct_layout_matches_header(struct, cls):
    """The binding's ctypes mirrors of the header's structs: every field at the C offset, same size."""
    C = getattr(k3, cls)
    fields = [f for f, _ in C._fields_]
    lay = _c_layout(struct, fields)
    assert lay["size"] == ctypes.sizeof(C), (struct, lay["size"], ctypes.sizeof(C))
    for f in fields:
        assert lay[f] == getattr(C, f).offset, (struct, f, lay[f], getattr(C, f).offset)


def test_new_entry_points_check_arguments_before_any_device_work():
    m = k3.K3MoE(_cfg(lora_rank=16))
    L = k3.lib()
    # expert-parallel split: state and argument errors
    assert L.k3moe_forward_head(m._h, None, 4, None, None, 3, None, None, None, None) == k3.EINVAL
    assert "divide" in m.last_error()
    assert L.k3moe_forward_head(m._h, None, 4, None, None, 4, None, None, None, None) == k3.ESTATE
    assert L.k3moe_experts_forward(m._h, None, None, 4 * 64 + 1, None, None, None, None) == k3.ETOOBIG
    assert L.k3moe_experts_forward(m._h, None, None, 8, None, None, None, None) == k3.ESTATE
    assert L.k3moe_forward_tail(m._h, None, 4, None, None, None) == k3.ESTATE
    assert L.k3moe_forward_tail(m._h, None, 65, None, None, None) == k3.ETOOBIG
    # no-allocation forward: same checks as forward
    assert L.k3moe_forward_noalloc(m._h, None, 4, None, None) == k3.ESTATE
    assert L.k3moe_forward_noalloc(m._h, None, 65, None, None) == k3.ETOOBIG
    # LoRA factors are required when the rank is set
    w = k3.Weights()
    w.routed_first, w.routed_count = 0, 1
    mx1 = (k3.MX * 1)(k3.MX(256, 256))
    w.gate = w.up = w.down = ctypes.cast(mx1, ctypes.POINTER(k3.MX))
    assert L.k3moe_pack_weights(m._h, ctypes.byref(w), 256, None) == k3.EINVAL
    assert "LoRA" in m.last_error()
    # measurement aid
    assert L.k3moe_stream_read(None, 16, None, None) == k3.EINVAL
    assert L.k3moe_stream_read(256, 17, 256, None) == k3.EINVAL


@pytest.mark.parametrize("rank", [4, 33, -8])
def test_create_rejects_bad_lora_rank(rank):
    with pytest.raises(k3.K3MoEError):
        k3.K3MoE(_cfg(lora_rank=rank))


def test_scratch_fits():
    """The static scratch holds a K3-shape decode batch of 64 tokens, not a prefill chunk."""
    m = k3.K3MoE(LayerConfig(d_model=7168, latent=3584, hidden=3072, n_experts=896, top_k=16, n_shared=2,
                             shared_hidden=3072, max_tokens=8192))
    assert m.scratch_fits(64) and not m.scratch_fits(8192)
    assert not m.scratch_fits(8193) and not m.scratch_fits(-1)
