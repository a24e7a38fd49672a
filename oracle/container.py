"""The .ninfer v2 container: header, JSON directory and its validation
(oracle; test infrastructure only).

Follows [ninfer-skill] §1 (container layout and directory rules):

* offset 0: the 8-byte magic b"NINFER\\x00\\x02"; offset 8: the directory
  length as a little-endian uint64; offset 16: the directory, compact UTF-8
  JSON; the payload starts at align_up(16 + json_bytes, 4096) and object
  offsets in the directory are relative to it;
* the member sets are exact: root {identity, objects}; identity {model_id,
  weights_id}, both non-empty; a tensor {name, kind, shape, format, layout,
  offset, bytes}; a resource {name, kind, encoding, offset, bytes};
* kind is "tensor" or "resource"; a resource's encoding is raw-bytes-v1;
* a tensor's bytes equal the encoded size of (layout, format, shape), else
  "tensor <name> stores N bytes; layout requires M";
* in directory order every object starts at or after the end of the
  previous one, at a multiple of its alignment (256 for tensor layouts, 1
  for resources), and ends inside the payload;
* names are unique ("duplicate object name: <name>").

Readings where the pages are silent (stated, not pinned by the pages):
* layout names are the four of [ninfer-v3] §6.2; encoded sizes are known
  for row_split_k128_v1 with the two ternary formats (the row-split
  geometry of [ninfer-skill] §3) and for contiguous_le_v1 with bf16, fp32
  and int32 (element count times element size; rank 0 is one element);
  other (format, layout) pairs are rejected as unsupported;
* "compact" means no whitespace outside JSON strings; shapes are arrays of
  positive integers (contiguous_le_v1 also allows rank 0); offsets are
  non-negative integers and bytes positive integers.
"""

import json
import struct

from . import geometry

MAGIC = b"NINFER\x00\x02"
PREFIX_BYTES = 16
PAYLOAD_ALIGNMENT = 4096
OBJECT_ALIGNMENT = 256
RESOURCE_ENCODING = "raw-bytes-v1"
LAYOUTS = ("contiguous_le_v1", "row_split_k128_v1", "block_scale_k16_m128x4_v1", "row_scale_v1")
CONTIGUOUS_SIZES = {"bf16": 2, "fp32": 4, "int32": 4}

ROOT_KEYS = {"identity", "objects"}
IDENTITY_KEYS = {"model_id", "weights_id"}
TENSOR_KEYS = {"name", "kind", "shape", "format", "layout", "offset", "bytes"}
RESOURCE_KEYS = {"name", "kind", "encoding", "offset", "bytes"}


class ContainerError(ValueError):
    pass


def _int(v):
    return isinstance(v, int) and not isinstance(v, bool)


def encoded_size(layout, fmt, shape):
    """Encoded byte size of a tensor, or raise ContainerError."""
    if layout not in LAYOUTS:
        raise ContainerError("unknown layout: %s" % layout)
    if layout == "row_split_k128_v1":
        if fmt not in geometry.FORMATS:
            raise ContainerError("unknown numeric format: %s" % fmt)
        if len(shape) != 2:
            raise ContainerError("row_split_k128_v1 needs a rank-2 shape")
        return geometry.row_split_geometry(fmt, shape[0], shape[1])["payload_bytes"]
    if layout == "contiguous_le_v1":
        if fmt not in CONTIGUOUS_SIZES:
            raise ContainerError("unknown numeric format: %s" % fmt)
        if len(shape) > 16:
            raise ContainerError("contiguous_le_v1 allows rank 0..16")
        count = 1
        for d in shape:
            count *= d
        return count * CONTIGUOUS_SIZES[fmt]
    raise ContainerError("unsupported layout: %s" % layout)


def _compact(text):
    """True when there is no whitespace outside JSON strings."""
    in_str = esc = False
    for ch in text:
        if in_str:
            if esc:
                esc = False
            elif ch == "\\":
                esc = True
            elif ch == '"':
                in_str = False
        elif ch == '"':
            in_str = True
        elif ch in " \t\r\n":
            return False
    return True


def _reject_duplicate_keys(pairs):
    keys = [k for k, _ in pairs]
    if len(set(keys)) != len(keys):
        raise ContainerError("directory object repeats a member")
    return dict(pairs)


def parse(data):
    """Validate a whole container; return (payload_offset, objects), where
    objects is the directory's object list in order."""
    data = bytes(data)
    if len(data) < PREFIX_BYTES or data[:8] != MAGIC:
        raise ContainerError("bad magic")
    (json_bytes,) = struct.unpack("<Q", data[8:16])
    if json_bytes > len(data) - PREFIX_BYTES:
        raise ContainerError("directory runs past the end of the file")
    payload_offset = geometry.align_up(PREFIX_BYTES + json_bytes, PAYLOAD_ALIGNMENT)
    if payload_offset > len(data):
        raise ContainerError("payload starts past the end of the file")
    raw = data[PREFIX_BYTES:PREFIX_BYTES + json_bytes]
    try:
        text = raw.decode("utf-8")
        doc = json.loads(text, object_pairs_hook=_reject_duplicate_keys)
    except (UnicodeDecodeError, json.JSONDecodeError):
        raise ContainerError("directory is not valid JSON")
    if not _compact(text):
        raise ContainerError("directory is not compact JSON")
    if not isinstance(doc, dict) or set(doc) != ROOT_KEYS:
        raise ContainerError("root members must be exactly identity, objects")
    ident = doc["identity"]
    if not isinstance(ident, dict) or set(ident) != IDENTITY_KEYS:
        raise ContainerError("identity members must be exactly model_id, weights_id")
    for key in ("model_id", "weights_id"):
        if not isinstance(ident[key], str) or not ident[key]:
            raise ContainerError("identity %s must be a non-empty string" % key)
    objs = doc["objects"]
    if not isinstance(objs, list):
        raise ContainerError("objects must be an array")
    payload_bytes = len(data) - payload_offset
    cursor = 0
    seen = set()
    for o in objs:
        if not isinstance(o, dict) or "kind" not in o:
            raise ContainerError("object entry without a kind")
        kind = o["kind"]
        if kind == "tensor":
            if set(o) != TENSOR_KEYS:
                raise ContainerError("tensor members must be exactly %s" % ", ".join(sorted(TENSOR_KEYS)))
        elif kind == "resource":
            if set(o) != RESOURCE_KEYS:
                raise ContainerError("resource members must be exactly %s" % ", ".join(sorted(RESOURCE_KEYS)))
        else:
            raise ContainerError("kind must be tensor or resource")
        name = o["name"]
        if not isinstance(name, str) or not name:
            raise ContainerError("object name must be a non-empty string")
        if name in seen:
            raise ContainerError("duplicate object name: %s" % name)
        seen.add(name)
        off, nbytes = o["offset"], o["bytes"]
        if not _int(off) or off < 0 or not _int(nbytes) or nbytes <= 0:
            raise ContainerError("object %s: offset and bytes must be integers (bytes > 0)" % name)
        if kind == "tensor":
            shape = o["shape"]
            if not isinstance(shape, list) or not all(_int(d) and d > 0 for d in shape):
                raise ContainerError("tensor %s: shape must be an array of positive integers" % name)
            if not isinstance(o["format"], str) or not isinstance(o["layout"], str):
                raise ContainerError("tensor %s: format and layout must be strings" % name)
            need = encoded_size(o["layout"], o["format"], shape)
            if nbytes != need:
                raise ContainerError("tensor %s stores %d bytes; layout requires %d" % (name, nbytes, need))
            align = OBJECT_ALIGNMENT
        else:
            if o["encoding"] != RESOURCE_ENCODING:
                raise ContainerError("resource %s: encoding must be %s" % (name, RESOURCE_ENCODING))
            align = 1
        if off < cursor:
            raise ContainerError("object %s overlaps or precedes the previous object" % name)
        if off % align:
            raise ContainerError("object %s offset is not a multiple of %d" % (name, align))
        if off + nbytes > payload_bytes:
            raise ContainerError("object %s runs past the end of the payload" % name)
        cursor = off + nbytes
    return payload_offset, objs


def build(identity, objects, payloads):
    """Write a container: identity dict, object dicts (offset and bytes are
    filled in: each object at the next multiple of its alignment), and the
    payload bytes of each object, in the same order."""
    objs = []
    cursor = 0
    for o, p in zip(objects, payloads):
        align = OBJECT_ALIGNMENT if o["kind"] == "tensor" else 1
        off = geometry.align_up(cursor, align)
        o = dict(o, offset=off, bytes=len(p))
        objs.append(o)
        cursor = off + len(p)
    text = json.dumps({"identity": identity, "objects": objs}, separators=(",", ":"))
    raw = text.encode("utf-8")
    payload_offset = geometry.align_up(PREFIX_BYTES + len(raw), PAYLOAD_ALIGNMENT)
    out = bytearray(payload_offset + cursor)
    out[:8] = MAGIC
    out[8:16] = struct.pack("<Q", len(raw))
    out[16:16 + len(raw)] = raw
    for o, p in zip(objs, payloads):
        out[payload_offset + o["offset"]:payload_offset + o["offset"] + len(p)] = p
    return bytes(out)
