"""fsattn_head_bounds_noalloc (the bounds with the library's device-resident
workspace) against fsattn_head_bounds with a caller workspace, through the
C ABI: bit-equal records and key means on two calls in a row, the second on
a smaller input, with no change in the device's free memory; and the same
call captured in a HIP graph (the use it exists for), replayed on new
inputs."""
import numpy as np
import pytest
import torch

import frame_block_sparse_amd as fs
import workloads

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _inputs(w, dev, seed):
    q, k, _ = workloads.make_inputs(w, seed=seed)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).to(td).to(dev) for x in (q, k))


def test_noalloc_bounds_match_workspace_entry_then_smaller_input():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    fs.lib()
    big = workloads.workload(2)                                                    # 1 x 8 x 21x960, d 128, bf16
    small = workloads.make_workload("small", 2, 3, 5, 240, 64, "bf16", 1, 0, 4, 48, 80, ref_count=1)
    small_f32 = workloads.make_workload("small_f32", 1, 2, 6, 48, 128, "f32", 1, 1, 0, 16, 16,
                                        ref_queries_global=1)
    cases = [(big, 0), (small, 1), (small_f32, 2)]
    inputs = [(w, *_inputs(w, dev, seed)) for w, seed in cases]
    for w, q, k in inputs:
        assert fs.head_bounds_workspace_bytes(q, w) <= fs.noalloc_max_workspace(), w.name
    # warm: the first call on the device looks up the array's address
    fs.head_bounds_noalloc(inputs[1][1], inputs[1][2], inputs[1][0])
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(dev)[0]
    for w, q, k in inputs:
        _say(f"[noalloc] {w.name}")
        got = fs.head_bounds_noalloc(q, k, w)
        torch.cuda.synchronize()
        ref = fs.head_bounds(q, k, w)
        torch.cuda.synchronize()
        assert torch.equal(got.rec, ref.rec), w.name
        assert torch.equal(got.key_mean, ref.key_mean), w.name
    # the outputs above were allocated by the test before each call; the
    # entry point itself allocated nothing: a call into preallocated outputs
    # leaves the free memory as it was
    w, q, k = inputs[0]
    out = fs.head_bounds(q, k, w)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info(dev)[0]
    fs.head_bounds_noalloc(q, k, w, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info(dev)[0] == free1
    assert free0 > 0


def test_noalloc_rejects_shapes_beyond_its_workspace():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    w = workloads.make_workload("too_big", 1, 64, 16, 1024, 128, "bf16", 15, 15, 0, 64, 64)
    q = torch.zeros((1, 64, 16 * 1024, 128), dtype=torch.bfloat16, device=dev)
    assert fs.head_bounds_workspace_bytes(q, w) > fs.noalloc_max_workspace()
    with pytest.raises(fs.FsattnError) as e:
        fs.head_bounds_noalloc(q, q, w)
    assert e.value.status == 4


def test_noalloc_bounds_in_a_captured_graph():
    """Captured once, replayed three times: before each replay the static
    inputs are overwritten eagerly (and the device synchronised); every
    replay's records equal the eager workspace entry's on the same inputs."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    w = workloads.make_workload("graph", 1, 4, 6, 480, 128, "bf16", 1, 1, 0, 48, 80)
    sets = [_inputs(w, dev, seed) for seed in (11, 12, 13, 14)]
    qs, ks = (t.clone() for t in sets[0])
    out = fs.head_bounds_noalloc(qs, ks, w)          # warm (address lookup) and the output buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fs.head_bounds_noalloc(qs, ks, w, out=out)
    torch.cuda.synchronize()
    for rep, (q, k) in enumerate(sets[1:]):
        _say(f"[noalloc-graph] replay {rep}")
        qs.copy_(q)
        ks.copy_(k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = fs.head_bounds(q, k, w)
        torch.cuda.synchronize()
        assert torch.equal(out.rec, ref.rec), rep
        assert torch.equal(out.key_mean, ref.key_mean), rep

