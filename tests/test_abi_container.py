"""The library's .ninfer v2 directory validator (C ABI, host code) against
the oracle on the containers of tests/container_cases.py: the same accept /
reject decision, the page's error wording, and the same object table."""

import pytest

import ternary_quantized_amd as tq
from oracle import container as C
import container_cases as cc


@pytest.mark.parametrize("label,data,msg", cc.cases(), ids=[c[0] for c in cc.cases()])
def test_validator_matches_oracle(label, data, msg):
    if msg is None:
        off, objs = tq.container_parse(data)
        o_off, o_objs = C.parse(data)
        assert off == o_off
        assert objs == [dict(o) for o in o_objs]
    else:
        with pytest.raises(C.ContainerError):
            C.parse(data)
        with pytest.raises(tq.TQError) as e:
            tq.container_parse(data)
        assert e.value.status == 2  # TQ_ERR_FORMAT
        assert msg in str(e.value)


def test_unsupported_layout_is_its_own_status():
    d = cc.valid_doc()
    d["objects"][2].update(layout="row_scale_v1", format="fp8_e4m3fn_row_bf16")
    with pytest.raises(tq.TQError) as e:
        tq.container_parse(cc.assemble(cc.compact(d)))
    assert e.value.status == 6 and "unsupported layout: row_scale_v1" in str(e.value)


def test_object_at_bounds_and_truncated_file():
    data = cc.assemble(cc.compact(cc.valid_doc()))
    with pytest.raises(tq.TQError) as e:
        tq.container_parse(data[:10])
    assert "bad magic" in str(e.value)
    L = tq.lib()
    o = tq.ContainerObject()
    buf = bytearray(data)
    import ctypes
    arr = (ctypes.c_uint8 * len(buf)).from_buffer(buf)
    assert L.tq_container_object_at(arr, len(buf), 4, ctypes.byref(o)) == 1
    assert L.tq_container_object_at(arr, len(buf), 2, ctypes.byref(o)) == 0
    assert o.name == b"signs" and o.rank == 1 and o.shape[0] == 1024 and o.offset == 1280
