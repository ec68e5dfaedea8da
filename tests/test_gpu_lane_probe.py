"""The hardware lane map of the CDNA4 transposed LDS read
(ds_read_b64_tr_b16), through the C ABI's self-test: every MFMA kernel
builds its 32x32x16 operand fragments with it, assuming that lane l
receives rows 8*(l/32) .. 8*(l/32)+7 of column l % 32 of a K-outer tile
(rocm-libraries PR 11602, "Technical Details"; its gfx1250 follow-up: a
per-lane hardware probe settles the map). The tile holds the code
(row << 8 | column) of every element, so each returned value names where
it came from."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
gcb = pytest.importorskip("grouped_convolution_backward_amd")

pytestmark = pytest.mark.gpu


def test_transposed_read_lane_map():
    out = torch.full((512,), -1, dtype=torch.int16, device="cuda")
    print("[gpu] transposed-read lane probe", flush=True)
    gcb.wgrad_probe_transpose_read(out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 8)
    lane = np.arange(64)[:, None]
    e = np.arange(8)[None, :]
    want = (((lane // 32) * 8 + e) << 8) | (lane % 32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} lane values differ, first (lane, value): {bad[:4].tolist()}, " \
                          f"got {got[tuple(bad[0])]:#06x} want {want[tuple(bad[0])]:#06x}"


def test_probe_rejects_bad_buffers():
    with pytest.raises(ValueError):
        gcb.wgrad_probe_transpose_read(torch.zeros(511, dtype=torch.int16, device="cuda"))
    with pytest.raises(ValueError):
        gcb.wgrad_probe_transpose_read(torch.zeros(512, dtype=torch.int32, device="cuda"))
