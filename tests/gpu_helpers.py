"""Shared plumbing for the GPU parity tests: both sides built from one seeded case.

The GPU side fills NaN-poisoned pools with the library's own pa_write_kv; the
oracle side fills its host pools with the oracle's own write.  Nothing the
GPU computes feeds the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_decode_slot_amd as pa
from paged_kv_decode_slot_amd import workloads as W

# The stated max-abs bounds per dtype.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1.5e-2}

# A tighter, per-element bound for the 16-bit paths, from the kernel's arithmetic.
# The softmax weights enter the P*V product rounded to the storage type, each
# with relative error at most U_P (half an ulp: 2^-8 for bf16, 2^-11 for f16), so
# the weighted sum moves by at most U_P * sum_t w_t |v_t| / sum_t w_t, the softmax
# average of |V| (the oracle's own answer with |V| in place of V).  The rest of
# the arithmetic is the f32 path's, which the f32 twins of the same workloads
# hold within TOL["f32"].  The output is then rounded once: half an ulp of the
# dtype at the value.
U_P = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
_MANT = {"f32": 23, "f16": 10, "bf16": 7}
_MIN_EXP = {"f32": -126, "f16": -14, "bf16": -126}


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -200)))
    e = np.maximum(e, _MIN_EXP[dtype])
    return np.ldexp(0.5, (e - _MANT[dtype]).astype(np.int64))


def derived_bound(dtype: str, ref: np.ndarray, abs_v_avg: np.ndarray) -> np.ndarray:
    core = U_P[dtype] * abs_v_avg + TOL["f32"]
    return core + half_ulp(np.abs(ref) + core, dtype)


def check_output(gpu_out: torch.Tensor, ref: np.ndarray, abs_v_avg: np.ndarray | None, dtype: str,
                 label: str) -> None:
    """Assert the stated bound and, when abs_v_avg is given, the derived per-element bound; log both margins."""
    got = gpu_out.detach().float().cpu().double().numpy()
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    err = np.abs(got - ref)
    emax = float(err.max()) if err.size else 0.0
    msg = f"{label}: max abs err {emax:.3e} (bound {TOL[dtype]:.0e})"
    if abs_v_avg is not None and err.size:
        bound = derived_bound(dtype, ref, abs_v_avg)
        ratio = float((err / bound).max())
        msg += f", worst err / derived bound {ratio:.3f} (derived bound median {float(np.median(bound)):.2e})"
        log(msg)
        assert ratio <= 1.0, msg
    else:
        log(msg)
    assert emax <= TOL[dtype], msg


def log(msg: str) -> None:
    print(msg, flush=True)


class GpuCase:
    """Device copies of a case, with pools written by the library."""

    def __init__(self, case: W.Case, device="cuda:0"):
        self.case = case
        dt = W.DTYPES[case.dtype]
        self.k_cache, self.v_cache = pa.new_cache(case.num_blocks, case.B, case.Hkv, case.D, dt, device)
        ints = torch.int32 if case.elt == 4 else torch.int16
        self.k_cache.view(ints).fill_(W.NAN_BITS[case.dtype])
        self.v_cache.view(ints).fill_(W.NAN_BITS[case.dtype])
        self.q = case.q.to(device)
        self.bt = torch.from_numpy(case.block_tables).to(device)
        self.ctx = torch.from_numpy(case.context_lens).to(device)
        self.k_new = case.k_new.to(device)
        self.v_new = case.v_new.to(device)
        self.slot_new = torch.from_numpy(case.slot_new).to(device)
        if case.k_prefill.shape[0]:
            pa.write_kv(case.k_prefill.to(device), case.v_prefill.to(device),
                        torch.from_numpy(case.slot_prefill).to(device), self.k_cache, self.v_cache)
        self.appended = False

    def append(self):
        """The decode step's KV append of the new token of every sequence."""
        pa.write_kv(self.k_new, self.v_new, self.slot_new, self.k_cache, self.v_cache)
        self.appended = True

    def decode_append(self, num_workers=0, out=None):
        """The fused step: append the new tokens and attend, one launch."""
        assert not self.appended
        self.appended = True
        return pa.decode_append(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache, self.bt, self.ctx,
                                self.case.scale, out, num_workers=num_workers)

    def decode(self, num_workers=0, out=None):
        assert self.appended
        return pa.decode(self.q, self.k_cache, self.v_cache, self.bt, self.ctx, self.case.scale, out,
                         num_workers=num_workers)


def flat_bits(t: torch.Tensor) -> torch.Tensor:
    """A host integer view of a tensor's bytes, so NaN payloads compare too."""
    t = t.detach().contiguous().cpu().view(-1)
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def dev_bits(t: torch.Tensor) -> torch.Tensor:
    """A flat integer view of a tensor's bytes, on its own device."""
    t = t.contiguous().view(-1)
    return t.view({4: torch.int32, 2: torch.int16, 1: torch.uint8}[t.element_size()])


def oracle_pools(case: W.Case):
    return oracle.build_pools(case)


def max_abs_err(gpu_out: torch.Tensor, ref: np.ndarray) -> float:
    got = gpu_out.detach().float().cpu().double().numpy()
    assert got.shape == ref.shape
    if not np.isfinite(got).all():
        return float("inf")
    return float(np.abs(got - ref).max()) if got.size else 0.0
