"""fs_longrange_prefill_noalloc (the prefill with the library's fixed device scratch as
its workspace) against fs_longrange_prefill with a caller workspace: the same kernels
on the same inputs, so outputs, selections and decode states must be bitwise equal.
Two calls in a row, the second with a smaller input (the scratch keeps the first
call's contents), and a shape too large for the scratch is rejected before launch."""
import numpy as np
import pytest

import cell_routed_long_amd as fsl
import synth
from tests import parity_utils as pu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fsl.lib()


def both(w, p, sigma=4.0, lam=1.0, with_state=False):
    host = pu.inputs(w)
    q, k, v = (pu.to_device(host[x], w.dtype) for x in "qkv")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    print(f"[gpu] noalloc vs workspace {w} {p}", flush=True)
    st1 = fsl.new_state(w.batch, w.H, w.d, dt, p) if with_state else None
    st2 = fsl.new_state(w.batch, w.H, w.d, dt, p) if with_state else None
    if with_state:  # the state build leaves padding and free slots unwritten: same bytes there in both
        st1.fill_(0x5A)
        st2.fill_(0x5A)
    out1, sel1, _ = fsl.prefill(q, k, v, p, sigma=sigma, lam=lam, state=st1)
    out2 = torch.full_like(out1, float("nan"))
    sel2 = torch.full_like(sel1, -7)
    fsl.fs_longrange_prefill_noalloc(q, k, v, sigma, lam, None, out2, sel2, st2, p)
    torch.cuda.synchronize()
    assert torch.equal(sel1, sel2)
    assert torch.equal(out1.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       out2.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    if with_state:
        assert torch.equal(st1, st2)
        # and both continue the stream identically
        step = {x: pu.to_device(np.ascontiguousarray(synth.tensor(w, x)[:, :, -1]), w.dtype) for x in "qkv"}
        for _ in range(3):
            o1, s1 = fsl.decode(st1, step["q"], step["k"], step["v"], p, sigma=sigma, lam=lam)
            o2, s2 = fsl.decode(st2, step["q"], step["k"], step["v"], p, sigma=sigma, lam=lam)
            torch.cuda.synchronize()
            assert torch.equal(s1, s2) and torch.equal(o1.float(), o2.float())


def test_noalloc_two_calls_second_smaller():
    # first call: bf16 d128, needles, pruning active; then a smaller fp32 d64 input
    both(synth.Workload(batch=2, H=4, N=3000, d=128, dtype="bf16", seed=301, needle_frac=0.01), fsl.Params(),
         with_state=True)
    both(synth.Workload(batch=1, H=2, N=1000, d=64, dtype="f32", seed=302, needle_frac=0.01), fsl.Params(P=6, W=2))


def test_noalloc_fs_and_ragged():
    both(synth.Workload(batch=1, H=3, N=1300, d=128, dtype="bf16", seed=303), fsl.Params(prune=False))
    both(synth.Workload(batch=1, H=2, N=129, d=64, dtype="bf16", seed=304), fsl.Params(P=3, W=1))


def test_noalloc_rejects_shape_past_scratch():
    cap = fsl.fs_noalloc_scratch_bytes()
    sh = fsl.fs_shape(4, 16, 16384, 128, fsl.FS_BF16)
    assert fsl.fs_prefill_workspace_bytes(sh) > cap
    q = torch.zeros(1, 1, 1, 1, device="cuda")
    with pytest.raises(fsl.FslError) as e:
        # sizes come from the shape; the check happens before anything touches the tensors
        lib = fsl.lib()
        import ctypes
        prm = fsl.Params().c()
        sig = (ctypes.c_float * 16)(*[4.0] * 16)
        lam = (ctypes.c_float * 16)(*[1.0] * 16)
        vp = ctypes.c_void_p(q.data_ptr())
        fsl._check(lib.fs_longrange_prefill_noalloc(ctypes.byref(sh), ctypes.byref(prm), vp, vp, vp, sig, lam, None,
                                                    vp, None, None, 0, None), "fs_longrange_prefill_noalloc")
    assert e.value.status == fsl.FS_ERR_WORKSPACE
