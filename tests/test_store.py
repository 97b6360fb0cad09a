"""The persisted format (int8_int4_dequant_amd/store.py), laid out like the
output folder of the script on page "量化推理：INT8/INT4 的体积、困惑度与速度为什么
不同步": <name>.bin payload, <name>.scale little-endian fp32 scales,
<name>.f32 unquantized tensors, manifest.json with bits, group and shape.

CPU tests check the bytes on disk against the format's definition (the
worked example of page "Quantisation, worked as Chapter 23 works it") and
the round trip; the GPU test checks the page's re-read against the oracle:
persisted codes decode exactly as oracle.unpack decodes the bytes on disk,
and the plain records on disk hold the oracle's own payload and scales."""

import json
import os
import struct

import numpy as np
import pytest

import oracle
from int8_int4_dequant_amd import inputs, store


def test_worked_example_bytes_on_disk(tmp_path, golden_dir):
    with open(os.path.join(golden_dir, "chapter23_worked_example.json")) as f:
        w = np.array(json.load(f)["weights"], np.float32)
    rec = oracle.quantize_pack(w, 4, 8)
    store.save(str(tmp_path), {"w": rec}, verify=False)
    # codes 2, -6, 5, -1, 7, -3, 1, -5 (+8, element 2i in the low nibble)
    assert (tmp_path / "w.bin").read_bytes() == bytes.fromhex("2a7d5f39")
    # one fp32 scale 0.072857 (bits 0x3D953620), little-endian
    assert (tmp_path / "w.scale").read_bytes() == struct.pack("<I", 0x3D953620)
    assert json.loads((tmp_path / "manifest.json").read_text()) == {
        "w": {"bits": 4, "group": 8, "shape": [8]}}


def test_round_trip_on_the_host(tmp_path):
    w = inputs.weight([10, 1], 24, 64, 0.02)
    bias = inputs.activations([10, 2], 1, 24)[0]
    recs = {"up": oracle.quantize_pack(w, 4, 32), "down": oracle.quantize_pack(w, 8, 64),
            "bias": bias}
    manifest = store.save(str(tmp_path), recs, verify=False)
    assert manifest["bias"] == {"dtype": "f32", "shape": [24]}
    assert (tmp_path / "bias.f32").read_bytes() == bias.astype("<f4").tobytes()
    back = store.load(str(tmp_path))
    for name in ("up", "down"):
        a, b = recs[name], back[name]
        assert (a["bits"], a["group"], list(a["shape"])) == (b["bits"], b["group"], b["shape"])
        assert np.array_equal(a["payload"], b["payload"])
        assert np.array_equal(a["scales"].view(np.uint32), b["scales"].view(np.uint32))
        assert np.array_equal(oracle.unpack(a).view(np.uint32), oracle.unpack(b).view(np.uint32))
    assert np.array_equal(back["bias"].view(np.uint32), bias.view(np.uint32))


def test_load_rejects_inconsistent_files(tmp_path):
    w = inputs.weight([10, 3], 8, 32, 0.02)
    store.save(str(tmp_path), {"m": oracle.quantize_pack(w, 4, 32)}, verify=False)
    data = (tmp_path / "m.bin").read_bytes()
    (tmp_path / "m.bin").write_bytes(data[:-1])
    with pytest.raises(ValueError):
        store.load(str(tmp_path))
    (tmp_path / "m.bin").write_bytes(data)
    (tmp_path / "m.scale").write_bytes((tmp_path / "m.scale").read_bytes() + b"\0\0\0\0")
    with pytest.raises(ValueError):
        store.load(str(tmp_path))


def test_save_rejects_bad_entries(tmp_path):
    w = inputs.weight([10, 4], 8, 32, 0.02)
    rec = oracle.quantize_pack(w, 4, 32)
    with pytest.raises(ValueError):
        store.save(str(tmp_path), {"../x": rec}, verify=False)
    bad = dict(rec, group=48)
    with pytest.raises(ValueError):
        store.save(str(tmp_path), {"m": bad}, verify=False)
    short = dict(rec, payload=rec["payload"][:-1])
    with pytest.raises(ValueError):
        store.save(str(tmp_path), {"m": short}, verify=False)


@pytest.mark.gpu
def test_persisted_records_decode_like_the_oracle(tmp_path):
    """The page's persist step: the folder is read back and its codes must
    decode exactly to the weights the evaluation used.  Here the reference
    is the oracle, not the HIP path: the plain records on disk must hold the
    oracle's payload and scales for the same weight, the GPU decode of every
    loaded record (plain and GPTQ) must equal oracle.unpack of the bytes on
    disk, and the GEMV of a loaded record must stay within the GEMV bar of
    the oracle's product."""
    import torch

    from int8_int4_dequant_amd import qw

    dev = torch.device("cuda:0")
    w_host = inputs.weight([10, 5], 96, 256, 0.02)
    w = torch.from_numpy(w_host).to(dev)
    xc = torch.from_numpy(inputs.calibration_activations([10, 6], 1024, 256)).to(dev)
    recs = {"plain4": qw.quantize_pack(w, 4, 32), "plain8": qw.quantize_pack(w, 8, 256),
            "gptq4": qw.gptq(w, qw.gptq_hessian(xc), 4, 64), "norm": w[0].clone()}
    store.save(str(tmp_path), recs)           # includes the GPU re-read check
    on_disk = store.load(str(tmp_path))        # host copies of the files
    back = store.load(str(tmp_path), device=dev)
    for name, (bits, group) in (("plain4", (4, 32)), ("plain8", (8, 256))):
        ref = oracle.quantize_pack(w_host, bits, group)
        assert np.array_equal(on_disk[name]["payload"], ref["payload"])
        assert np.array_equal(on_disk[name]["scales"].view(np.uint32), ref["scales"].view(np.uint32))
    x_host = inputs.activations([10, 7], 2, 256)
    x = torch.from_numpy(x_host).to(dev)
    for name in ("plain4", "plain8", "gptq4"):
        want = oracle.unpack(on_disk[name])
        got = qw.unpack(back[name]).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name
        y = qw.gemv(back[name], x).cpu().numpy()
        yr = oracle.gemv_ref(on_disk[name], x_host)
        assert np.all(np.abs(y - yr) <= 1e-5 * oracle.error_base(on_disk[name], x_host)), name
    assert np.array_equal(on_disk["norm"].view(np.uint32), w_host[0].view(np.uint32))
    assert torch.equal(back["norm"], recs["norm"])
