"""vt_attention_varlen_noalloc -- the attention step with its scratch in the
library's fixed device array instead of a caller workspace -- against
vt_attention_varlen on the same inputs, through the C ABI.  Both run the same
kernels, and on these inputs vt_attention_varlen does not cut its last round
of work across workgroups (which the no-allocation call never does), so the
outputs must be equal bit for bit: on two calls in a row, the
second smaller than the first (the array keeps the first call's contents),
in fp32 and bf16 output, and when the call is captured into a HIP graph and
replayed."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_f32, dev_bits, log, rng, window_to_raster

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_transformer_encoder_tiled_amd as m
    return m


def _inputs(vt, grids, seed):
    N = sum(t * h * w for t, h, w in grids)
    qkv = synth.bf16_bits(rng(seed).standard_normal((N, 3840), dtype=np.float32))
    cu = torch.empty(len(grids) + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    return N, qkv, dev_bits(qkv, torch), cu, pos


# The largest packed input that fits the array (seven 448x448 images), then a
# smaller ragged one: the second call runs on what the first left behind.
CASES = [([(1, 32, 32)] * 7, 41), ([(1, 16, 16), (1, 2, 2), (1, 6, 10)], 42)]


def test_noalloc_equals_workspace_entry_point(vt):
    cfg = vt.config()
    for grids, seed in CASES:
        N, qkv_bits, qkv, cu, pos = _inputs(vt, grids, seed)
        max_seq = max(t * h * w for t, h, w in grids)
        log(f"noalloc attention: {len(grids)} images, {N} tokens")
        ws = vt.workspace(vt.vt_block_workspace_size(cfg, N, len(grids), max_seq))
        for dt, tdt in ((vt.VT_FP32, torch.float32), (vt.VT_BF16, torch.int16)):
            ref = torch.empty((N, 1280), dtype=tdt, device="cuda")
            got = torch.full((N, 1280), 7, dtype=tdt, device="cuda")
            vt.vt_attention_varlen(cfg, qkv, cu, pos, len(grids), N, max_seq, ref, dt, ws)
            vt.vt_attention_varlen_noalloc(cfg, qkv, cu, pos, len(grids), N, max_seq, got, dt)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), (grids, dt)
        # and the oracle, on the small case (all rows) and the large one (sampled rows)
        perm = window_to_raster(grids)
        x = np.empty((N, 3, 16, 80), np.float32)
        x[perm] = bf16_f32(qkv_bits).reshape(N, 3, 16, 80)
        axis, inv = oracle.rope_tables()
        p_r, cu_r = oracle.positions(grids), oracle.cu_seqlens(grids)
        q = oracle.apply_rope(x[:, 0], p_r, axis, inv)
        k = oracle.apply_rope(x[:, 1], p_r, axis, inv)
        got32 = torch.empty((N, 1280), dtype=torch.float32, device="cuda")
        vt.vt_attention_varlen_noalloc(cfg, qkv, cu, pos, len(grids), N, max_seq, got32, vt.VT_FP32)
        torch.cuda.synchronize()
        g_r = np.empty((N, 1280), np.float32)
        g_r[perm] = got32.cpu().numpy()
        a, b = int(cu_r[-2]), int(cu_r[-1])     # the last image, every row
        want = oracle.attention_image(q[a:b], k[a:b], x[a:b, 2]).reshape(b - a, 1280)
        err = np.max(np.abs(g_r[a:b] - want))
        log(f"  last image vs oracle: max abs err {err:.3e}")
        assert err <= 2e-3


def test_noalloc_graph_replay(vt):
    """Captured into a HIP graph after one eager call (which resolves the
    array's address), every replay gives the eager bits, with eager calls of
    another size on the same array between the replays."""
    cfg = vt.config()
    grids = [(1, 16, 16), (1, 4, 6)]
    N, _, qkv, cu, pos = _inputs(vt, grids, 43)
    other = [(1, 32, 32)]
    N2, _, qkv2, cu2, pos2 = _inputs(vt, other, 44)
    out = torch.empty((N, 1280), dtype=torch.float32, device="cuda")
    out2 = torch.empty((N2, 1280), dtype=torch.float32, device="cuda")
    call = lambda: vt.vt_attention_varlen_noalloc(cfg, qkv, cu, pos, 2, N, 256, out, vt.VT_FP32)
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        log(f"noalloc graph replay {i}")
        out.zero_()
        vt.vt_attention_varlen_noalloc(cfg, qkv2, cu2, pos2, 1, N2, N2, out2, vt.VT_FP32)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i


def test_noalloc_rejects_oversize(vt):
    cfg = vt.config()
    grids = [(1, 32, 32)] * 8
    N, _, qkv, cu, pos = _inputs(vt, grids, 45)
    out = torch.empty((N, 1280), dtype=torch.float32, device="cuda")
    with pytest.raises(vt.VtError) as e:
        vt.vt_attention_varlen_noalloc(cfg, qkv, cu, pos, 8, N, 1024, out, vt.VT_FP32)
    assert e.value.status == vt.VT_ERR_WORKSPACE
