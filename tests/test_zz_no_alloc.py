"""pa_decode_noalloc, the decode for callers that cannot allocate, through the C
ABI: its output equals pa_decode's (the entry point it is a variant of) and the
oracle's, on two calls in a row, the second with a smaller batch, from the
library's own per-GPU workspace."""
import ctypes

import pytest
import torch

import oracle
import paged_kv_decode_slot_amd as pa
from paged_kv_decode_slot_amd import workloads as W
from tests.gpu_helpers import TOL, GpuCase, dev_bits, log, max_abs_err

pytestmark = pytest.mark.gpu


def _call(fn_name, g: GpuCase, out, workspace=None):
    L = pa.lib()
    c = g.case
    desc = pa.cache_desc(g.k_cache, g.v_cache)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    common = (g.q.data_ptr(), g.k_cache.data_ptr(), g.v_cache.data_ptr(), g.bt.data_ptr(), g.ctx.data_ptr(),
              ctypes.c_float(c.scale), out.data_ptr(), c.S, c.Hq, c.max_blocks_per_seq, ctypes.byref(desc))
    if fn_name == "pa_decode_noalloc":
        return L.pa_decode_noalloc(*common, stream)
    return L.pa_decode(*common, workspace.data_ptr(), workspace.numel(), stream)


def _cases():
    # the Llama-3-8B-shaped batch, then a smaller one of another shape
    big = W.config_case(3)
    small = W.make_case(S=9, Hq=28, Hkv=4, D=128, B=16, dtype="bf16", ctx_range=(100, 3000), seed=77,
                        name="smaller")
    return [big, small]


def test_noalloc_matches_pa_decode_on_two_calls():
    L = pa.lib()
    for i, case in enumerate(_cases()):
        log(f"[noalloc] call {i}: {case.name}, {case.S} sequences")
        g = GpuCase(case)
        g.append()
        desc = pa.cache_desc(g.k_cache, g.v_cache)
        need = int(L.pa_decode_workspace_bytes(case.S, case.Hq, case.max_blocks_per_seq, ctypes.byref(desc)))
        assert 0 < need <= 16 * 1024 * 1024
        ws = pa.new_workspace(need, "cuda:0")
        want = torch.empty_like(g.q)
        got = torch.full_like(g.q, float("nan"))
        assert _call("pa_decode", g, want, ws) == 0
        st = _call("pa_decode_noalloc", g, got)
        assert st == 0, L.pa_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(dev_bits(got), dev_bits(want))
        err = max_abs_err(got, oracle.decode_case(case))
        log(f"[noalloc] call {i}: max abs err vs oracle {err:.3e}")
        assert err <= TOL[case.dtype]
        del g
        torch.cuda.empty_cache()


def test_noalloc_empty_batch_is_a_noop():
    case = W.make_case(S=2, Hq=8, Hkv=2, D=64, B=16, dtype="bf16", ctx=[5, 9], seed=3, name="empty")
    desc = pa.CacheDesc(case.num_blocks, case.B, case.Hkv, case.D, 2)
    assert pa.lib().pa_decode_noalloc(None, None, None, None, None, ctypes.c_float(0.1), None, 0, 8, 1,
                                      ctypes.byref(desc), None) == 0
