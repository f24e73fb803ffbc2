"""tcl_fused_apply_noalloc (the apply whose workspace is the library's static
device array) against tcl_fused_apply with a caller workspace: bit for bit
on two calls in a row, the second with a smaller batch, so the second reads
what the first left in the shared array only where it writes it first; and a
batch whose workspace exceeds the array is refused before any launch."""
import numpy as np
import pytest
import torch

from gpu_util import make_module, make_plan, rel_err, to_dev
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_parity import TOL, banner, oracle_apply

pytestmark = pytest.mark.gpu


def _both(wl):
    """y after tcl_fused_apply and after tcl_fused_apply_noalloc, from the
    same inputs; returns (reference ys, no-alloc ys, workspace bytes)."""
    plan = make_plan(wl.composites)
    mods = [make_module(m) for m in wl.modules]
    xs = [to_dev(x) for x in wl.x]
    y_ref = [to_dev(y) for y in wl.y_base]
    y_na = [y.clone() for y in y_ref]
    call = tclora.FusedCall(plan, mods, xs, y_ref)
    call()
    na = tclora.FusedCall(plan, mods, xs, y_na, ws=call.ws)
    na.noalloc()
    torch.cuda.synchronize()
    return y_ref, y_na, tclora.workspace_bytes(plan, mods)


def test_noalloc_equals_caller_workspace_twice(monkeypatch):
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    monkeypatch.delenv("TCL_KCHUNK", raising=False)
    # a prefill batch (token-tile expand: tile records and z in the array),
    # then a smaller decode batch (split-K partial z rows)
    big = W.random_case(171, T=600, N=40, d_in=256, d_out=520, r_max=16, max_pairs=4,
                        with_k=True)
    second = W.random_case(172, T=600, N=40, d_in=128, d_out=264, r_max=32, max_pairs=4)
    big.modules.append(second.modules[0])
    big.x.append(second.x[0])
    big.y_base.append(second.y_base[0])
    small = W.random_case(173, T=24, N=40, d_in=4096, d_out=1024, r_max=8, max_pairs=3)
    for label, wl in (("prefill T=600", big), ("decode T=24", small)):
        y_ref, y_na, need = _both(wl)
        banner(f"no-alloc {label}: workspace {need} bytes of {tclora.SCRATCH_BYTES}")
        assert 0 < need <= tclora.SCRATCH_BYTES
        for mi in range(len(wl.modules)):
            assert torch.equal(y_na[mi], y_ref[mi]), (label, mi)
            _, d_ora = oracle_apply(wl, mi)
            got = y_na[mi].double().cpu().numpy() - wl.y_base[mi].astype(np.float64)
            err = rel_err(got, d_ora)
            print(f"  {label} module {mi}: rel {err:.3e}", flush=True)
            assert err <= TOL[wl.dtype]


def test_noalloc_refuses_batches_beyond_the_array(monkeypatch):
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    # 65536 tokens of one pair each: 1024 token tiles of records, more than
    # the static array holds
    T, N = 65536, 8
    rng = np.random.default_rng(174)
    ads = [[int(a)] for a in rng.integers(0, N, T)]
    als = [[1.0] for _ in range(T)]
    wl = W.random_case(174, T=64, N=N, d_in=64, d_out=64, r_max=8, max_pairs=1)
    c = W.csr_from_token_lists(ads, als, N)
    plan = make_plan(c)
    mod = make_module(wl.modules[0])
    need = tclora.workspace_bytes(plan, [mod])
    banner(f"no-alloc refusal: workspace {need} bytes of {tclora.SCRATCH_BYTES}")
    assert need > tclora.SCRATCH_BYTES
    x = torch.zeros(T, 64, dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((T, 64), 3.0, dtype=torch.float32, device="cuda:0")
    call = tclora.FusedCall(plan, [mod], [x], [y])
    with pytest.raises(tclora.TclError) as e:
        call.noalloc()
    assert e.value.code == tclora.ENOSPC
    torch.cuda.synchronize()
    assert bool(torch.all(y == 3.0))
