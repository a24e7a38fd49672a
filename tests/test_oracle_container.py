"""Pins of the oracle's .ninfer v2 container reader and writer against
[ninfer-skill] §1: the header layout, the exact member sets, the kinds and
encoding, encoded sizes, ordered aligned ranges and unique names, with the
error wording the page gives.  Containers are assembled byte by byte in
tests/container_cases.py, independently of the oracle's writer."""

import json
import struct

import pytest

from oracle import container as C, geometry as G
import container_cases as cc


def test_valid_container_header_and_directory():
    data = cc.assemble(cc.compact(cc.valid_doc()))
    assert data[:8] == b"NINFER\x00\x02"
    (n,) = struct.unpack("<Q", data[8:16])
    assert json.loads(data[16:16 + n].decode()) == cc.valid_doc()
    off, objs = C.parse(data)
    assert off == 4096 and off % 4096 == 0 and off >= 16 + n
    assert [o["name"] for o in objs] == ["w.pq2", "w.ptq1", "signs", "tok"]


def test_directory_longer_than_one_page_moves_the_payload():
    d = cc.valid_doc()
    d["identity"]["model_id"] = "m" * 5000
    data = cc.assemble(cc.compact(d))
    assert C.parse(data)[0] == 8192


@pytest.mark.parametrize("label,data,msg", cc.cases(), ids=[c[0] for c in cc.cases()])
def test_rules(label, data, msg):
    if msg is None:
        C.parse(data)
    else:
        with pytest.raises(C.ContainerError) as e:
            C.parse(data)
        assert msg in str(e.value)


def test_encoded_sizes():
    # the vocabulary payloads printed by [ninfer-skill] §3
    assert C.encoded_size("row_split_k128_v1", "PQ2_0_G128", [248320, 5120]) == 337715200
    assert C.encoded_size("row_split_k128_v1", "PTQ1_0_G128", [248320, 5120]) == 278118400
    assert C.encoded_size("contiguous_le_v1", "bf16", [5120]) == 10240
    assert C.encoded_size("contiguous_le_v1", "int32", []) == 4
    assert C.encoded_size("contiguous_le_v1", "fp32", [3, 7]) == 84
    with pytest.raises(C.ContainerError, match="unsupported layout"):
        C.encoded_size("row_scale_v1", "fp8_e4m3fn_row_bf16", [4, 4])


def test_writer_places_objects_and_round_trips():
    geo = G.row_split_geometry("PQ2_0_G128", 4, 128)
    pays = [bytes([1]) * geo["payload_bytes"], b"xyz", bytes([2]) * 20]
    objs = [{"name": "a", "kind": "tensor", "shape": [4, 128], "format": "PQ2_0_G128",
             "layout": "row_split_k128_v1"},
            {"name": "r", "kind": "resource", "encoding": "raw-bytes-v1"},
            {"name": "v", "kind": "tensor", "shape": [5], "format": "fp32", "layout": "contiguous_le_v1"}]
    data = C.build({"model_id": "m", "weights_id": "w"}, objs, pays)
    off, out = C.parse(data)
    assert [o["offset"] for o in out] == [0, 264, 512]  # tensors on 256, resources on 1
    for o, p in zip(out, pays):
        assert data[off + o["offset"]:off + o["offset"] + o["bytes"]] == p
