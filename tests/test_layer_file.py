"""CPU checks of the disk stream source's host side: the stack file layout
(blob i at i * stride, stride a multiple of 4 KiB, zero padding), reads back
through the reader threads (direct and buffered), error reporting, and the
`stream_source: auto` choice."""
import os

import numpy as np
import pytest

from qlora_fine_tuning_dequant_amd import binding as b


def _dims(n_layers=3):
    return b.Dims(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, inter=688, vocab=1024, n_layers=n_layers,
                  lora_r=8, lora_alpha=16.0, rms_eps=1e-5, rope_theta=5e5)


def _blobs(d, seed=0):
    _, total = b.blob_layout(d)
    g = np.random.default_rng(seed)
    return [g.integers(0, 256, total, dtype=np.uint8) for _ in range(d.n_layers)]


@pytest.mark.parametrize("buffered", [False, True])
def test_file_layout_and_read_back(tmp_path, buffered):
    d = _dims()
    blobs = _blobs(d)
    path = str(tmp_path / "stack.bin")
    b.LayerFile.write(path, d, blobs)
    f = b.LayerFile(path, d, buffered=buffered)
    info = f.info()
    total = blobs[0].size
    assert info["stride"] % 4096 == 0 and total <= info["stride"] < total + 4096
    assert os.path.getsize(path) == d.n_layers * info["stride"]
    if buffered:
        assert not info["direct"]
    raw = np.fromfile(path, dtype=np.uint8)
    for i, bl in enumerate(blobs):
        s = i * info["stride"]
        assert np.array_equal(raw[s:s + total], bl)
        assert not raw[s + total:s + info["stride"]].any()        # zero padding
        out = np.zeros(total, np.uint8)
        f.read(i, out)
        assert np.array_equal(out, bl)
    # reads in any order, repeated (the streamer's backward runs in reverse)
    for i in (2, 0, 2, 1):
        out = np.empty(total, np.uint8)
        f.read(i, out)
        assert np.array_equal(out, blobs[i])
    f.close()


def test_errors(tmp_path):
    d = _dims()
    L = b.lib()
    missing = str(tmp_path / "none.bin")
    with pytest.raises(b.QlxError) as e:
        b.LayerFile(missing, d)
    assert e.value.code == b.QLX_EIO and "none.bin" in str(e.value)
    # a file shorter than n_layers * stride
    path = str(tmp_path / "short.bin")
    b.LayerFile.write(path, _dims(2), _blobs(_dims(2)))
    with pytest.raises(b.QlxError) as e:
        b.LayerFile(path, d)
    assert e.value.code == b.QLX_EIO and "holds" in str(e.value)
    # bad flags, bad layer index
    import ctypes as C
    h = C.c_void_p()
    assert L.qlx_layer_file_open(C.byref(h), os.fsencode(path), C.byref(_dims(2)), 4) == b.QLX_EINVAL
    f = b.LayerFile(path, _dims(2))
    out = np.zeros(b.blob_layout(_dims(2))[1], np.uint8)
    with pytest.raises(b.QlxError) as e:
        f.read(2, out)
    assert e.value.code == b.QLX_EINVAL
    f.close()
    # NULL blob pointer in the write call
    arr = (C.c_void_p * 2)(None, None)
    assert L.qlx_layer_file_write(os.fsencode(path), C.byref(_dims(2)),
                                  C.cast(arr, C.POINTER(C.c_void_p)), 0) == b.QLX_EINVAL
    # unknown write flags
    assert L.qlx_layer_file_write(os.fsencode(path), C.byref(_dims(2)),
                                  C.cast(arr, C.POINTER(C.c_void_p)), 4) == b.QLX_EINVAL
    # a directory that does not exist
    assert L.qlx_layer_file_write(os.fsencode(str(tmp_path / "no" / "x.bin")), C.byref(_dims(2)),
                                  C.cast((C.c_void_p * 2)(*[bl.ctypes.data for bl in _blobs(_dims(2))]),
                                         C.POINTER(C.c_void_p)), 0) == b.QLX_EIO
    assert L.qlx_layer_file_close(None) == b.QLX_OK


def test_stream_source_auto():
    avail = 0
    for line in open("/proc/meminfo"):
        if line.startswith("MemAvailable:"):
            avail = int(line.split()[1]) * 1024
    assert avail > 0
    assert b.stream_source_auto(0) == b.QLX_STREAMED
    assert b.stream_source_auto(1 << 20) == b.QLX_STREAMED
    assert b.stream_source_auto(1 << 62) == b.QLX_STREAMED_DISK
    assert b.stream_source_auto(1 << 20, 1 << 62) == b.QLX_STREAMED_DISK     # the reserve counts
    assert b.stream_source_auto(2**64 - 1, 2**64 - 1) == b.QLX_STREAMED_DISK  # no overflow
    assert b.stream_source_auto(avail // 4, avail // 4) == b.QLX_STREAMED
