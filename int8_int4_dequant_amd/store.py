"""Persisted quantized weights: a folder the packed codes are written to and
loaded from without quantizing again.

Layout (page "量化推理：INT8/INT4 的体积、困惑度与速度为什么不同步", the
script's per-configuration output folder):

* ``<name>.bin``    the payload bytes exactly as ``qw_quantize_pack`` (or
                    ``qw_gptq_quantize_pack``) wrote them;
* ``<name>.scale``  the group scales as little-endian fp32, in group order;
* ``<name>.f32``    a tensor kept unquantized, little-endian fp32, row-major;
* ``manifest.json`` ``{name: {"bits", "group", "shape"}}`` for every
                    quantized tensor -- the same three fields as the page --
                    and, for every unquantized one, ``{"dtype": "f32",
                    "shape"}`` (the page's folder relies on the model
                    definition for those shapes; a loader needs them).

``save`` writes the files and then reads every quantized tensor back,
checking that it decodes to exactly the weights it was saved from (the
decode runs on the GPU through ``qw_unpack``).  ``load`` validates each entry
against its declared bits, group and shape (sizes, a group dividing the
element count) before returning records that ``qw.unpack``, ``qw.gemv`` and
``qw.gemm`` take directly.

File input and output only: no quantization arithmetic happens here.
"""

import json
import os
import re

import numpy as np

MANIFEST = "manifest.json"
_NAME = re.compile(r"^[A-Za-z0-9_.-]+$")


def _check_name(name):
    if not _NAME.match(name) or name in (".", "..") or name == MANIFEST:
        raise ValueError(f"tensor name {name!r} cannot be a file name")


def _host_bytes(a, dtype):
    """A host copy of a numpy array or a torch tensor (on any device)."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _sizes(bits, group, shape):
    count = int(np.prod(shape)) if len(shape) else 1
    if bits not in (4, 8):
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    if group < 1 or count % group:
        raise ValueError(f"group {group} does not divide {count} elements")
    if bits == 4 and count % 2:
        raise ValueError("int4 needs an even element count")
    return count * bits // 8, count // group


def save(folder, tensors, verify=True):
    """Write ``tensors`` ({name: record or fp32 array/tensor}) to ``folder``.

    A record is a dict with ``bits``, ``group``, ``shape``, ``payload`` and
    ``scales`` (numpy arrays or torch tensors).  Returns the manifest.  With
    ``verify`` every quantized tensor is read back from disk and decoded on
    the GPU, and must give exactly the weights of the record it came from."""
    os.makedirs(folder, exist_ok=True)
    manifest = {}
    for name, t in tensors.items():
        _check_name(name)
        if isinstance(t, dict):
            bits, group = int(t["bits"]), int(t["group"])
            shape = [int(d) for d in t["shape"]]
            nb, ns = _sizes(bits, group, shape)
            payload = _host_bytes(t["payload"], np.uint8).reshape(-1)
            scales = _host_bytes(t["scales"], "<f4").reshape(-1)
            if payload.size != nb or scales.size != ns:
                raise ValueError(f"{name}: {payload.size} payload bytes and {scales.size} scales, "
                                 f"expected {nb} and {ns}")
            with open(os.path.join(folder, name + ".bin"), "wb") as f:
                f.write(payload.tobytes())
            with open(os.path.join(folder, name + ".scale"), "wb") as f:
                f.write(scales.tobytes())
            manifest[name] = {"bits": bits, "group": group, "shape": shape}
        else:
            a = _host_bytes(t, "<f4")
            with open(os.path.join(folder, name + ".f32"), "wb") as f:
                f.write(a.tobytes())
            manifest[name] = {"dtype": "f32", "shape": [int(d) for d in a.shape]}
    with open(os.path.join(folder, MANIFEST), "w") as f:
        json.dump(manifest, f, indent=2)
    if verify:
        verify_folder(folder, tensors)
    return manifest


def load(folder, device=None):
    """Read a folder written by ``save``.  Returns {name: record or array}:
    records as ``save`` takes them (payload uint8, scales fp32), arrays fp32
    of their shape; numpy on the host, or torch tensors on ``device``."""
    with open(os.path.join(folder, MANIFEST)) as f:
        manifest = json.load(f)
    out = {}
    for name, m in manifest.items():
        _check_name(name)
        shape = [int(d) for d in m["shape"]]
        if m.get("dtype") == "f32":
            raw = np.fromfile(os.path.join(folder, name + ".f32"), dtype="<f4")
            count = int(np.prod(shape)) if shape else 1
            if raw.size != count:
                raise ValueError(f"{name}.f32 holds {raw.size} values, expected {count}")
            arr = raw.astype(np.float32).reshape(shape)
            out[name] = _to(arr, device)
            continue
        bits, group = int(m["bits"]), int(m["group"])
        nb, ns = _sizes(bits, group, shape)
        payload = np.fromfile(os.path.join(folder, name + ".bin"), dtype=np.uint8)
        scales = np.fromfile(os.path.join(folder, name + ".scale"), dtype="<f4")
        if payload.size != nb:
            raise ValueError(f"{name}.bin holds {payload.size} bytes, expected {nb}")
        if scales.size != ns:
            raise ValueError(f"{name}.scale holds {scales.size} scales, expected {ns}")
        out[name] = dict(bits=bits, group=group, shape=shape, payload=_to(payload, device),
                         scales=_to(scales.astype(np.float32), device))
    return out


def _to(a, device):
    if device is None:
        return a
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def verify_folder(folder, tensors):
    """Read the quantized tensors of ``tensors`` back from ``folder`` and check
    that each decodes (``qw_unpack`` on the GPU) to exactly the weights of the
    record it was saved from; unquantized tensors must round-trip bit for
    bit.  Raises AssertionError on any difference."""
    import torch

    from . import qw

    dev = torch.device("cuda", torch.cuda.current_device())
    loaded = load(folder, device=dev)
    for name, t in tensors.items():
        got = loaded[name]
        if isinstance(t, dict):
            ref = dict(t)
            for key in ("payload", "scales"):
                v = ref[key]
                ref[key] = v.to(dev) if hasattr(v, "to") else torch.from_numpy(
                    np.ascontiguousarray(v)).to(dev)
            a = qw.unpack(got)
            b = qw.unpack(ref)
            torch.cuda.synchronize()
            if not torch.equal(a.view(torch.int32), b.view(torch.int32)):
                raise AssertionError(f"{name}: the persisted codes decode to other weights")
        else:
            a = got.cpu().numpy()
            b = _host_bytes(t, "<f4")
            if not np.array_equal(a.view(np.uint32), b.astype(np.float32).view(np.uint32)):
                raise AssertionError(f"{name}: the persisted fp32 tensor differs")
