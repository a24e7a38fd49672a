"""Valid and invalid .ninfer v2 containers for the directory tests: each
case is (label, file bytes, expected message fragment or None).  Files are
assembled here byte by byte ([ninfer-skill] §1: magic, little-endian
uint64 directory length, compact JSON, payload at align_up(16+len, 4096)),
not with the oracle's writer, so that the writer and both readers are
checked against the page rather than against each other."""

import json
import struct

MAGIC = b"NINFER\x00\x02"

# PQ2_0 [4, 128]: base 128 B, high at 256 (empty), scale at 256 + 8 B -> 264
# PTQ1_0 [2, 256]: base 96 B, high at 256 (8 B), scale at 512 + 8 B -> 520
W_PQ2 = {"name": "w.pq2", "kind": "tensor", "shape": [4, 128], "format": "PQ2_0_G128",
         "layout": "row_split_k128_v1", "offset": 0, "bytes": 264}
W_PTQ1 = {"name": "w.ptq1", "kind": "tensor", "shape": [2, 256], "format": "PTQ1_0_G128",
          "layout": "row_split_k128_v1", "offset": 512, "bytes": 520}
SIGNS = {"name": "signs", "kind": "tensor", "shape": [1024], "format": "bf16",
         "layout": "contiguous_le_v1", "offset": 1280, "bytes": 2048}
RES = {"name": "tok", "kind": "resource", "encoding": "raw-bytes-v1", "offset": 3328, "bytes": 5}
IDENT = {"model_id": "bonsai-test", "weights_id": "synthetic-1"}
PAYLOAD_BYTES = 3333


def assemble(directory_text, payload_bytes=PAYLOAD_BYTES, magic=MAGIC, declared_len=None):
    raw = directory_text.encode("utf-8")
    n = len(raw) if declared_len is None else declared_len
    start = -(-(16 + len(raw)) // 4096) * 4096
    out = bytearray(start + payload_bytes)
    out[:8] = magic
    out[8:16] = struct.pack("<Q", n)
    out[16:16 + len(raw)] = raw
    for i in range(payload_bytes):
        out[start + i] = (i * 7 + 3) & 0xFF
    return bytes(out)


def compact(doc):
    return json.dumps(doc, separators=(",", ":"))


def valid_doc():
    return {"identity": dict(IDENT), "objects": [dict(W_PQ2), dict(W_PTQ1), dict(SIGNS), dict(RES)]}


def with_obj(i, **kw):
    d = valid_doc()
    o = d["objects"][i]
    for key, v in kw.items():
        if v is None:
            o.pop(key, None)
        else:
            o[key] = v
    return d


def cases():
    out = [("valid", assemble(compact(valid_doc())), None)]
    d = valid_doc()
    d["objects"] = []
    out.append(("valid, no objects", assemble(compact(d), payload_bytes=0), None))
    out.append(("bad magic", assemble(compact(valid_doc()), magic=b"NINFER\x00\x03"), "bad magic"))
    out.append(("directory past end", assemble(compact(valid_doc()), declared_len=1 << 40),
                "directory runs past the end of the file"))
    out.append(("not JSON", assemble('{"identity":'), "not valid JSON"))
    out.append(("whitespace", assemble(json.dumps(valid_doc())), "not compact JSON"))
    d = valid_doc()
    d["extra"] = 1
    out.append(("extra root member", assemble(compact(d)), "root members must be exactly"))
    d = valid_doc()
    del d["identity"]["weights_id"]
    out.append(("missing identity member", assemble(compact(d)), "identity members must be exactly"))
    d = valid_doc()
    d["identity"]["model_id"] = ""
    out.append(("empty model_id", assemble(compact(d)), "identity model_id must be a non-empty string"))
    out.append(("extra tensor member", assemble(compact(with_obj(0, note="x"))), "tensor members must be exactly"))
    out.append(("missing tensor member", assemble(compact(with_obj(0, layout=None))), "tensor members must be exactly"))
    out.append(("bad kind", assemble(compact(with_obj(3, kind="blob"))), "kind must be tensor or resource"))
    out.append(("bad encoding", assemble(compact(with_obj(3, encoding="raw_bytes_v1"))),
                "encoding must be raw-bytes-v1"))
    out.append(("wrong bytes", assemble(compact(with_obj(0, bytes=260))),
                "tensor w.pq2 stores 260 bytes; layout requires 264"))
    out.append(("unknown format", assemble(compact(with_obj(0, format="Q9_0"))), "unknown numeric format: Q9_0"))
    out.append(("unknown layout", assemble(compact(with_obj(0, layout="rowsplit"))), "unknown layout: rowsplit"))
    out.append(("overlap", assemble(compact(with_obj(1, offset=256))),
                "object w.ptq1 overlaps or precedes the previous object"))
    out.append(("misaligned tensor", assemble(compact(with_obj(1, offset=640))),
                "object w.ptq1 offset is not a multiple of 256"))
    out.append(("past payload end", assemble(compact(with_obj(3, offset=3330))),
                "object tok runs past the end of the payload"))
    out.append(("duplicate name", assemble(compact(with_obj(1, name="w.pq2"))), "duplicate object name: w.pq2"))
    out.append(("negative offset", assemble(compact(with_obj(0, offset=-256))), "offset and bytes must be integers"))
    out.append(("zero-sized shape", assemble(compact(with_obj(2, shape=[0], bytes=0))),
                "offset and bytes must be integers"))
    return out
