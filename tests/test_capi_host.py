"""Host-only checks of the C ABI library (no GPU): it loads, exports every
function include/moe.h declares, and validates arguments before launching."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_expert_ffn_sigmoid_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|size_t|const char\*)\s+(moe_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 10, names
    L = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(L, n), n


def test_validation_without_gpu():
    from quantized_expert_ffn_sigmoid_amd import capi
    import gen
    cfg = gen.get_config("c2")
    d = capi.make_desc(type("S", (), dict(hidden=6144, inter=2048, n_experts=256, top_k=8,
                                          router=0, n_group=8, topk_group=4,
                                          routed_scaling=2.5, expert_dtype=capi.MOE_I4,
                                          act_dtype=capi.MOE_F32, n_shared=1,
                                          shared_dtype=capi.MOE_BF16, norm_eps=0.0))())
    assert capi.moe_workspace_bytes(d, 1) > 0
    assert capi.moe_workspace_bytes(d, 2048) > capi.moe_workspace_bytes(d, 1)
    # inconsistent descriptors are rejected before anything is launched
    bad = capi.MoeLayerDesc.from_buffer_copy(d)
    bad.topk_group = 9
    assert capi.moe_workspace_bytes(bad, 1) == 0
    with pytest.raises(capi.MoeError) as e:
        capi.moe_route(bad, 0, 0, 0, 1, 0, 0, 0, 0, stream=0)
    assert e.value.status == capi.MOE_EINVAL
    bad = capi.MoeLayerDesc.from_buffer_copy(d)
    bad.hidden = 6144 + 16          # int4 rows must be multiples of 16 bytes
    with pytest.raises(capi.MoeError) as e:
        capi.moe_route(bad, 0, 0, 0, 1, 0, 0, 0, 0, stream=0)
    assert e.value.status == capi.MOE_EUNSUPPORTED
    # zero tokens is a no-op, null pointers otherwise are invalid
    capi.moe_route(d, 0, 0, 0, 0, 0, 0, 0, 0, stream=0)
    with pytest.raises(capi.MoeError) as e:
        capi.moe_route(d, 0, 0, 0, 1, 0, 0, 0, 0, stream=0)
    assert e.value.status == capi.MOE_EINVAL
    # misaligned pointer
    with pytest.raises(capi.MoeError) as e:
        capi.moe_route(d, 0x1004, 0, 0x2000, 1, 0x3000, 0x4000, 0x5000, 1 << 30, stream=0)
    assert e.value.status == capi.MOE_EINVAL
    # workspace too small
    with pytest.raises(capi.MoeError) as e:
        capi.moe_route(d, 0x1000, 0, 0x2000, 1, 0x3000, 0x4000, 0x5000, 16, stream=0)
    assert e.value.status == capi.MOE_EWORKSPACE
    assert "workspace" in capi.status_str(capi.MOE_EWORKSPACE)


def test_noalloc_rejects_large_batches_before_any_launch():
    """moe_layer_forward_noalloc checks its batch against the library's own
    workspace on the host: a batch that needs more is refused with
    MOE_EWORKSPACE and nothing is launched (no device is touched)."""
    from quantized_expert_ffn_sigmoid_amd import capi
    import gen
    cfg = gen.get_config("c2")
    d = capi.make_desc(cfg)
    T = 64
    assert capi.moe_workspace_bytes(d, T) > capi.MOE_NOALLOC_SCRATCH_BYTES
    assert capi.moe_workspace_bytes(d, 40) <= capi.MOE_NOALLOC_SCRATCH_BYTES
    st = dict(gate_up=0x10000, gate_up_stride=1 << 24, gate_up_scale=0x20000,
              gate_up_scale_stride=1 << 24, down=0x30000, down_stride=1 << 24,
              down_scale=0x40000, down_scale_stride=1 << 24)
    w = capi.make_weights(dict(w_router=0x50000, bias=None, routed=st, shared=st))
    with pytest.raises(capi.MoeError) as e:
        capi.moe_layer_forward_noalloc(d, w, 0x60000, T, 0x70000, None, None, stream=0)
    assert e.value.status == capi.MOE_EWORKSPACE
