"""HIP graph capture of the stateless entry points. The single-pass kernel's workspace returns to
zero by itself and no call issues a memset, so a captured sequence can be replayed as is.

One graph captures, on preallocated outputs: per-tensor current scaling (single-pass path and
the two-kernel path), MX dual, 128x128 groups, MXFP4 dual, NVFP4 with a measured amax (single
pass) and MX de-scaling. It is replayed three times with eager work and synchronizations in
between: as captured, after the inputs were changed in place (x *= 2), and after the outputs
were overwritten. Every replay's outputs equal the eager calls' on the same data, and the
barrier part of the workspace is zero after each replay.
"""
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
from synthetic import mx_gradient, small_tensor
from qf8_test_utils import to_device

pytestmark = pytest.mark.gpu


class Outputs:
    def __init__(self, xl, xs, xm):
        dev = "cuda"
        R, C = xl.shape
        r, c = xm.shape
        u8 = torch.uint8
        f32 = torch.float32
        self.t = {
            "pt_q": torch.empty((R, C), dtype=u8, device=dev), "pt_a": torch.empty(1, dtype=f32, device=dev),
            "pt_s": torch.empty(1, dtype=f32, device=dev),
            "ps_q": torch.empty(xs.shape, dtype=u8, device=dev), "ps_a": torch.empty(1, dtype=f32, device=dev),
            "ps_s": torch.empty(1, dtype=f32, device=dev),
            "mx_qr": torch.empty((r, c), dtype=u8, device=dev), "mx_sr": torch.empty((r, c // 32), dtype=u8, device=dev),
            "mx_qc": torch.empty((c, r), dtype=u8, device=dev), "mx_sc": torch.empty((c, r // 32), dtype=u8, device=dev),
            "bk_q": torch.empty((r, c), dtype=u8, device=dev),
            "bk_s": torch.empty((r // 128, c // 128), dtype=f32, device=dev),
            "f4_qr": torch.empty((r, c // 2), dtype=u8, device=dev), "f4_sr": torch.empty((r, c // 32), dtype=u8, device=dev),
            "f4_qc": torch.empty((c, r // 2), dtype=u8, device=dev), "f4_sc": torch.empty((c, r // 32), dtype=u8, device=dev),
            "nv_q": torch.empty((R, C // 2), dtype=u8, device=dev), "nv_s": torch.empty((R, C // 16), dtype=u8, device=dev),
            "nv_t": torch.empty(1, dtype=f32, device=dev),
            "dq": torch.empty((r, c), dtype=torch.bfloat16, device=dev),
        }

    def snapshot(self):
        return {k: v.clone() for k, v in self.t.items()}

    def poison(self):
        for v in self.t.values():
            if v.dtype == torch.uint8:
                v.fill_(0xA5)
            else:
                v.fill_(-7.0)


def run_all(xl, xs, xm, o, ws_pt, ws_small, ws_nv):
    t = o.t
    qf8.quantize_per_tensor(xl, qf8.E4M3, q=t["pt_q"], amax=t["pt_a"], scale=t["pt_s"], ws=ws_pt)
    qf8.quantize_per_tensor(xs, qf8.E5M2, q=t["ps_q"], amax=t["ps_a"], scale=t["ps_s"], ws=ws_small)
    qf8.quantize_mx_dual(xm, qf8.E4M3, qf8.ROUND_UP, q_row=t["mx_qr"], s_row=t["mx_sr"], q_colT=t["mx_qc"],
                         s_colT=t["mx_sc"])
    qf8.quantize_block(xm, 128, 128, qf8.E4M3, q=t["bk_q"], scales=t["bk_s"], want_amax=False)
    qf8.quantize_mxfp4_dual(xm, qf8.ROUND_DOWN, q_row=t["f4_qr"], s_row=t["f4_sr"], q_colT=t["f4_qc"],
                            s_colT=t["f4_sc"])
    qf8.quantize_nvfp4(xl, q=t["nv_q"], s_blk=t["nv_s"], tensor_scale=t["nv_t"], ws=ws_nv)
    qf8.dequantize_mx(t["mx_qr"], t["mx_sr"], qf8.E4M3, out=t["dq"])


def assert_same(got, want, tag):
    for k in want:
        g, w = got[k], want[k]
        if g.dtype in (torch.float32, torch.bfloat16):
            g, w = g.view(torch.int16 if g.dtype == torch.bfloat16 else torch.int32), \
                w.view(torch.int16 if w.dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(g, w), f"{tag}: {k} differs"


def test_graph_replays_equal_eager_calls():
    xl = to_device(mx_gradient(2048, 4096, seed=61))        # 2^23 elements: single-pass paths
    xs = to_device(small_tensor(256, 512, seed=62))           # two-kernel per-tensor path
    xm = to_device(mx_gradient(1024, 1024, seed=63))
    ws_pt, ws_small, ws_nv = (qf8.workspace(x) for x in (xl, xs, xl))
    o = Outputs(xl, xs, xm)
    run_all(xl, xs, xm, o, ws_pt, ws_small, ws_nv)              # eager, also warms the lazy queries
    torch.cuda.synchronize()
    eager = o.snapshot()

    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=stream):
        run_all(xl, xs, xm, o, ws_pt, ws_small, ws_nv)
    torch.cuda.synchronize()

    def barrier_clean(tag):
        for ws in (ws_pt, ws_nv):
            assert not ws.view(torch.int32)[:qf8.BARRIER_WORDS].any().item(), f"{tag}: workspace not zero"

    o.poison()
    g.replay()
    torch.cuda.synchronize()
    assert_same(o.t, eager, "replay 1")
    barrier_clean("replay 1")

    for x in (xl, xs, xm):                                      # new data in the same buffers
        x.mul_(2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    replayed = o.snapshot()
    run_all(xl, xs, xm, o, ws_pt, ws_small, ws_nv)
    torch.cuda.synchronize()
    assert_same(replayed, o.snapshot(), "replay 2 (inputs doubled)")
    assert not torch.equal(replayed["pt_s"], eager["pt_s"])     # the scale did follow the new data
    barrier_clean("replay 2")

    o.poison()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert_same(o.t, replayed, "replay 3")
    barrier_clean("replay 3")
