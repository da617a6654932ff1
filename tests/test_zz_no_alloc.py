"""The entry point that allocates nothing: rotattn_fp16_fwd_noalloc stages
through the library's static device scratch and must give exactly the output
of rotattn_fp16_fwd (caller workspace), called through the C ABI, on two calls
in a row, the second with a smaller input; the first also against the oracle."""
import ctypes as C

import numpy as np
import pytest

import oracle as O
from video_diffusion_transformers_amd import synth

from gpu_common import check_out, torch_cuda

pytestmark = pytest.mark.gpu


def _call_both(cfg, sel):
    torch = torch_cuda()
    from video_diffusion_transformers_amd import rotattn as R
    L = R.lib()
    shape = R.shape_of(cfg)
    B, H, N, D = cfg.B, cfg.H, cfg.N, cfg.D
    q, k, v = synth.all_heads_qkv(cfg, 0)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    o_na = torch.full((B, H, N, D), float("nan"), dtype=torch.float16, device="cuda")
    o_ws = torch.full((B, H, N, D), float("nan"), dtype=torch.float16, device="cuda")
    ws = torch.empty(R.fp16_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    m = np.ascontiguousarray(sel, np.uint8)
    mp = m.ctypes.data_as(C.c_void_p)
    st = L.rotattn_fp16_fwd_noalloc(C.byref(shape), C.c_void_p(qd.data_ptr()),
                                     C.c_void_p(kd.data_ptr()), C.c_void_p(vd.data_ptr()), mp,
                                     C.c_void_p(o_na.data_ptr()), stream)
    assert st == 0, R.STATUS.get(st, st)
    st = L.rotattn_fp16_fwd(C.byref(shape), C.c_void_p(qd.data_ptr()), C.c_void_p(kd.data_ptr()),
                            C.c_void_p(vd.data_ptr()), mp, C.c_void_p(ws.data_ptr()),
                            ws.numel(), C.c_void_p(o_ws.data_ptr()), stream)
    assert st == 0, R.STATUS.get(st, st)
    torch.cuda.synchronize()
    a = o_na.cpu().numpy()
    b = o_ws.cpu().numpy()
    return (q, k, v), a, b


def test_noalloc_equals_workspace_form_two_calls():
    # call 1: the 720p shape, 31 of 40 heads selected (ten chunks of four
    # heads through the 256 MiB scratch, one chunk with no selected head)
    cfg = synth.CONFIGS["720p"]
    sel = np.ones(cfg.BH, np.uint8)
    sel[[4, 5, 6, 7, 13, 21, 30, 38, 39]] = 0
    (q, k, v), a, b = _call_both(cfg, sel)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    BH, N, D = cfg.BH, cfg.N, cfg.D
    ag = a.reshape(BH, N, D)
    assert np.isnan(ag[~sel.astype(bool)]).all()
    qh, kh, vh = (x.reshape(BH, N, D) for x in (q, k, v))
    for bh in (0, 12, 39 - 2):
        rows = synth.sampled_rows(cfg, bh)
        ref, _ = O.fp16_attention(qh[bh], kh[bh], vh[bh], rows)
        check_out(ag[bh][rows], ref, f"noalloc 720p head {bh}")
    # call 2, right after: a smaller input (the Small shape, every head), so
    # the scratch still holds the first call's staging
    cfg2 = synth.CONFIGS["small"]
    (q2, k2, v2), a2, b2 = _call_both(cfg2, np.ones(cfg2.BH, np.uint8))
    assert np.array_equal(a2.view(np.uint16), b2.view(np.uint16))
    a2g = a2.reshape(cfg2.BH, cfg2.N, cfg2.D)
    rows = np.arange(cfg2.N)
    for bh in range(cfg2.BH):
        ref, _ = O.fp16_attention(q2.reshape(cfg2.BH, cfg2.N, cfg2.D)[bh],
                                  k2.reshape(cfg2.BH, cfg2.N, cfg2.D)[bh],
                                  v2.reshape(cfg2.BH, cfg2.N, cfg2.D)[bh], rows)
        check_out(a2g[bh], ref, f"noalloc small head {bh}")


def test_noalloc_ragged_tail():
    """A ragged shape (N = 306, D = 128) with a partial selection."""
    cfg = synth.custom_config("rag306", 2, 2, (2, 9, 17), 128, (44, 42, 42), cfg_seed=81)
    sel = np.array([1, 0, 1, 1], np.uint8)
    _, a, b = _call_both(cfg, sel)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
