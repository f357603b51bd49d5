"""The C ABI on the host: the library loads, exports what the header declares,
and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import paged_kv_decode_slot_amd as pa
from paged_kv_decode_slot_amd.binding import CacheDesc, EXPORTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(5)
SYNC = 256 * 1024  # PA_WORKSPACE_SYNC_BYTES


def header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(pa_\w+)\s*\(", text))
    return names


def test_header_declares_the_binding_exports():
    assert header_functions() == set(EXPORTS)


def test_library_exports_every_declared_symbol():
    L = pa.lib()
    for name in header_functions():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    L = pa.lib()
    assert L.pa_abi_version() == 3
    for st in range(6):
        assert L.pa_status_string(st) != b"unknown status"
    assert L.pa_status_string(99) == b"unknown status"


def _desc(**kw):
    d = dict(num_blocks=10, block_size=16, num_kv_heads=2, head_dim=64, dtype=2)
    d.update(kw)
    return CacheDesc(**d)


# fake, suitably aligned device addresses: validation never dereferences them
A = 0x10000


def _write(desc, *, k=A, v=A, slots=A, kc=A, vc=A, T=4):
    return pa.lib().pa_write_kv(k, v, slots, kc, vc, T, ctypes.byref(desc) if desc is not None else None, None)


def _decode(desc, *, q=A, kc=A, vc=A, bt=A, ctx=A, out=A, S=2, Hq=4, maxblk=3, ws=A, ws_bytes=1 << 30,
            workers=64, scale=0.125):
    return pa.lib().pa_decode_ex(q, kc, vc, bt, ctx, scale, out, S, Hq, maxblk,
                                 ctypes.byref(desc) if desc is not None else None, ws, ws_bytes, workers, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(slots=None), INVALID),
    (dict(kc=None), INVALID), (dict(vc=None), INVALID), (dict(T=-1), INVALID),
    (dict(k=A + 8), INVALID), (dict(slots=A + 4), INVALID), (dict(vc=A + 2), INVALID),
])
def test_write_kv_rejects(kw, status):
    assert _write(_desc(), **kw) == status


def test_write_kv_zero_tokens_is_a_noop():
    assert _write(_desc(), T=0) == OK


@pytest.mark.parametrize("desc,status", [
    (None, INVALID),
    (dict(num_blocks=0), INVALID), (dict(num_kv_heads=0), INVALID), (dict(head_dim=-64), INVALID),
    (dict(block_size=8), UNSUPPORTED), (dict(head_dim=96), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
])
def test_cache_descriptor_checks(desc, status):
    d = None if desc is None else _desc(**desc)
    assert _write(d) == status
    assert _decode(d) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(ctx=None), INVALID), (dict(out=None), INVALID),
    (dict(bt=None), INVALID), (dict(q=A + 4), INVALID), (dict(out=A + 8), INVALID), (dict(bt=A + 2), INVALID),
    (dict(Hq=3), INVALID), (dict(S=-1), INVALID), (dict(maxblk=-1), INVALID), (dict(Hq=0), INVALID),
    (dict(Hq=34), UNSUPPORTED),  # G = 17
    (dict(S=8193), UNSUPPORTED),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(workers=-2), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE), (dict(ws=A + 16), WORKSPACE),
])
def test_decode_rejects(kw, status):
    assert _decode(_desc(), **kw) == status


def _append(desc, *, kn=A, vn=A, **kw):
    base = dict(q=A, kc=A, vc=A, bt=A, ctx=A, out=A, S=2, Hq=4, maxblk=3, ws=A, ws_bytes=1 << 30, workers=64,
                scale=0.125)
    base.update(kw)
    b = base
    return pa.lib().pa_decode_append(b["q"], kn, vn, b["kc"], b["vc"], b["bt"], b["ctx"], b["scale"], b["out"],
                                     b["S"], b["Hq"], b["maxblk"], ctypes.byref(desc), b["ws"], b["ws_bytes"],
                                     b["workers"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), INVALID), (dict(vn=None), INVALID), (dict(kn=A + 8), INVALID), (dict(q=None), INVALID),
    (dict(Hq=3), INVALID), (dict(ws=None), WORKSPACE), (dict(S=0, kn=None, vn=None), OK),
])
def test_decode_append_rejects(kw, status):
    assert _append(_desc(), **kw) == status


def _attend_call(desc, *, qs=A, maxq=4, rows=8, **kw):
    base = dict(q=A, kc=A, vc=A, bt=A, ctx=A, out=A, S=2, Hq=4, maxblk=3, ws=A, ws_bytes=1 << 30, workers=64,
                scale=0.125)
    base.update(kw)
    b = base
    return pa.lib().pa_attend(b["q"], b["kc"], b["vc"], b["bt"], b["ctx"], qs, b["scale"], b["out"], b["S"], b["Hq"],
                              b["maxblk"], maxq, rows, ctypes.byref(desc), b["ws"], b["ws_bytes"], b["workers"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qs=None), INVALID), (dict(qs=A + 2), INVALID), (dict(maxq=-1), INVALID), (dict(q=None), INVALID),
    (dict(Hq=3), INVALID), (dict(Hq=34), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(ws_bytes=64), WORKSPACE),
    (dict(maxq=0, qs=None, q=None, out=None), OK), (dict(S=0, qs=None), OK), (dict(rows=-1), INVALID),
    (dict(rows=0, qs=None, q=None, out=None), OK),
])
def test_attend_rejects(kw, status):
    assert _attend_call(_desc(), **kw) == status


def test_attend_workspace_sizes():
    L = pa.lib()
    d = _desc(head_dim=128, num_kv_heads=8)
    W_, S, D, Hkv = 100, 64, 128, 8
    waves = W_ * 2  # a worker has a wave per kv-head of a slice: 2 of the 8 kv-heads here
    r = lambda x: (x + 255) // 256 * 256
    for Hq, cols in [(32, 16), (56, 14), (8, 16), (128, 16)]:  # G = 4, 7, 1, 16: floor(16/G) tokens x G heads
        got = L.pa_attend_workspace_bytes(S, Hq, 256, ctypes.byref(d), W_)
        assert got == SYNC + r(4 * waves * 2 * cols) + 4 * waves * 2 * cols * D
    assert L.pa_attend_workspace_bytes(S, 32, 256, ctypes.byref(d), -1) == SYNC  # the prompt-chunk item counter


@pytest.mark.parametrize("kw,status", [
    (dict(theta=1.0), INVALID), (dict(theta=float("nan")), INVALID), (dict(theta=0.0), INVALID),
    (dict(D=96), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED), (dict(pos=None), INVALID), (dict(q=A + 4), INVALID),
    (dict(T=-1), INVALID), (dict(T=0, q=None, k=None, pos=None), OK), (dict(Hq=0, Hkv=0, q=None, k=None), OK),
])
def test_rope_rejects(kw, status):
    b = dict(q=A, k=A, pos=A, T=4, Hq=4, Hkv=2, D=128, dtype=2, theta=10000.0)
    b.update(kw)
    assert pa.lib().pa_rope(b["q"], b["k"], b["pos"], b["T"], b["Hq"], b["Hkv"], b["D"], b["dtype"], b["theta"],
                            None) == status


@pytest.mark.parametrize("kw,status", [(dict(theta=0.0), INVALID), (dict(theta=0.5), INVALID),
                                       (dict(dtype=0, theta=10000.0), UNSUPPORTED), (dict(S=0, theta=10000.0), OK)])
def test_decode_rope_append_rejects(kw, status):
    d = _desc(dtype=kw.get("dtype", 2))
    S = kw.get("S", 2)
    assert pa.lib().pa_decode_rope_append(A, A, A, A, A, A, A, 0.125, kw["theta"], A, S, 4, 3, ctypes.byref(d), A,
                                          1 << 30, 64, None) == status


def test_decode_zero_sequences_is_a_noop():
    assert _decode(_desc(), S=0) == OK


def test_workspace_sizes():
    L = pa.lib()
    d = _desc(head_dim=128, num_kv_heads=8)
    # one worker per (sequence, kv-head slice): no workspace
    assert L.pa_decode_workspace_bytes_ex(64, 32, 256, ctypes.byref(d), -1) == 0
    # stream split: the fixed synchronisation words, then 2 parts per wave of
    # G lse values and G*D outputs; a worker has a wave per kv-head of its
    # slice (the largest divisor of Hkv up to 2)
    r = lambda x: (x + 255) // 256 * 256
    for Hkv, Hq, sl in [(8, 32, 2), (4, 28, 2), (6, 24, 2), (16, 32, 2), (2, 4, 2), (7, 14, 1), (3, 3, 1), (1, 16, 1)]:
        d = _desc(head_dim=128, num_kv_heads=Hkv)
        W, S, G, D = 100, 64, Hq // Hkv, 128
        got = L.pa_decode_workspace_bytes_ex(S, Hq, 256, ctypes.byref(d), W)
        assert got == SYNC + r(4 * W * sl * 2 * G) + 4 * W * sl * 2 * G * D, (Hkv, Hq)
    d = _desc(head_dim=128, num_kv_heads=8)
    # rejected shapes report 0
    assert L.pa_decode_workspace_bytes_ex(64, 33, 256, ctypes.byref(d), W) == 0


def test_sync_region_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "pagedattn.h")).read()
    m = re.search(r"#define PA_WORKSPACE_SYNC_BYTES \((\d+) \* (\d+)\)", text)
    assert m and int(m.group(1)) * int(m.group(2)) == SYNC == 256 * 1024


def test_worker_count_bounded_by_the_arrival_words():
    # one arrival word per wave of every worker, after 16 header words
    L = pa.lib()
    d = _desc(head_dim=128, num_kv_heads=8)  # slices of 2 kv-heads: 2 waves per worker
    most = (SYNC // 8 - 16) // 2
    assert L.pa_decode_workspace_bytes_ex(64, 32, 256, ctypes.byref(d), most) > 0
    assert L.pa_decode_workspace_bytes_ex(64, 32, 256, ctypes.byref(d), most + 1) == 0
    assert _decode(_desc(num_kv_heads=2), workers=most + 1) == UNSUPPORTED  # rejected before any launch


def test_binding_refuses_cpu_tensors():
    import torch
    k, v = torch.zeros(2, 2, 1, 1024, dtype=torch.bfloat16), torch.zeros(2, 2, 1, 1024, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.write_kv(torch.zeros(1, 2, 64, dtype=torch.bfloat16), torch.zeros(1, 2, 64, dtype=torch.bfloat16),
                    torch.zeros(1, dtype=torch.int64), k, v)


# --- block pool: argument checks (no launch) and the host-side accounting ---

def test_pool_calls_reject_bad_arguments():
    L = pa.lib()
    assert L.pa_pool_init(A, A, 5, 4, None) == pa.binding.PA_ERR_INVALID_ARG  # more free than capacity
    assert L.pa_pool_init(A, A + 4, 2, 4, None) == pa.binding.PA_ERR_INVALID_ARG  # state not 8-byte aligned
    assert L.pa_pool_init(A, None, 2, 4, None) == pa.binding.PA_ERR_INVALID_ARG
    assert L.pa_pool_init(None, A, 0, 4, None) == pa.binding.PA_ERR_INVALID_ARG

    def assign(ctx=A, qs=A, bt=A, free=A, state=A, slots=A, S=2, M=4, B=16, T=3, cap=8):
        return L.pa_assign_slots(ctx, qs, bt, free, state, slots, S, M, B, T, cap, None)
    bad = pa.binding.PA_ERR_INVALID_ARG
    assert assign(S=-1) == bad
    assert assign(qs=None, T=3) == bad       # one row per sequence needs T == S
    assert assign(M=0) == bad
    assert assign(B=0) == bad
    assert assign(M=1 << 28, B=32) == bad    # a row would address more than 2^31 positions
    assert assign(ctx=None) == bad
    assert assign(bt=None) == bad
    assert assign(state=A + 4) == bad
    assert assign(slots=A + 4) == bad
    assert assign(cap=-1) == bad
    assert assign(S=0, T=1) == bad
    assert assign(S=0, T=0) == pa.binding.PA_OK  # nothing to do: no launch

    def release(ids=A, R=2, ctx=A, bt=A, free=A, state=A, S=2, M=4, B=16, cap=8):
        return L.pa_release_seqs(ids, R, ctx, bt, free, state, S, M, B, cap, None)
    assert release(R=-1) == bad
    assert release(ids=None) == bad
    assert release(state=A + 4) == bad
    assert release(B=0) == bad
    assert release(R=0, ids=None) == pa.binding.PA_OK  # nothing to release: no launch


def test_admission_reserves_the_worst_case():
    # B = 16, 10 blocks.  Reservations are ceil(max_tokens / 16): 33 -> 3 blocks,
    # 160 -> 10 (refused beside the 3), 112 -> 7 (exactly fills), 1 -> 1 (refused).
    a = pa.acct_init(10, 16, 4096)
    pa.acct_admit(a, 33)
    with pytest.raises(pa.CapacityError):
        pa.acct_admit(a, 160)
    assert a.reserved_blocks == 3 and a.refused == 1 and a.admitted == 1
    pa.acct_admit(a, 112)
    assert a.reserved_blocks == 10 and a.peak_reserved_blocks == 10
    with pytest.raises(pa.CapacityError):
        pa.acct_admit(a, 1)
    pa.acct_admit(a, 0)  # a request that can never hold a token reserves nothing
    pa.acct_retire(a, 0)
    pa.acct_retire(a, 33)
    assert a.reserved_blocks == 7 and a.admitted == 1 and a.peak_reserved_blocks == 10
    pa.acct_admit(a, 48)
    assert a.reserved_blocks == 10
    with pytest.raises(ValueError):
        pa.acct_retire(a, 1000)  # more than is reserved
    with pytest.raises(ValueError):
        pa.acct_admit(a, -1)


def test_telemetry_from_the_state_record():
    bpb = 2 * 8 * 16 * 128 * 2  # K and V of one block: Hkv 8, B 16, D 128, bf16
    a = pa.acct_init(10, 16, bpb)
    pa.acct_admit(a, 100)
    # 4 free, 2 sequences refused, lowest top 1, 1 release refused
    t = pa.pool_telemetry(a, [4, 2, 1, 1, 0, 0, 0, 0], tokens_stored=80)
    assert t["used_blocks"] == 6 and t["free_blocks"] == 4 and t["peak_used_blocks"] == 9
    assert t["used_bytes"] == 6 * bpb and t["capacity_bytes"] == 10 * bpb
    assert t["empty_slots"] == 6 * 16 - 80 and t["occupancy"] == pytest.approx(0.6)
    assert t["reserved_blocks"] == 7 and t["admitted"] == 1
    assert (t["refused_sequences"], t["refused_releases"], t["refused_admissions"]) == (2, 1, 0)
    with pytest.raises(ValueError):
        pa.pool_telemetry(a, [4, 0, 4, 0, 0, 0, 0, 0], tokens_stored=97)  # more tokens than used slots


def test_rmsnorm_rejects_bad_arguments():
    L = pa.lib()
    bad, uns = pa.binding.PA_ERR_INVALID_ARG, pa.binding.PA_ERR_UNSUPPORTED

    def norm(x=A, res=None, w=A, out=A, rows=4, H=4096, eps=1e-5, dt=2):
        return L.pa_rmsnorm(x, res, w, out, rows, H, ctypes.c_float(eps), dt, None)
    assert norm(rows=-1) == bad
    assert norm(H=0) == bad
    assert norm(eps=-1.0) == bad
    assert norm(eps=float("nan")) == bad
    assert norm(eps=float("inf")) == bad
    assert norm(dt=7) == bad
    assert norm(H=12) == uns            # not whole 16-byte pieces
    assert norm(H=8200) == uns          # wider than 8192 (16-bit)
    assert norm(H=4100, dt=0) == uns    # wider than 4096 (f32)
    assert norm(x=None) == bad
    assert norm(out=A + 8) == bad
    assert norm(res=A + 4) == bad
    assert norm(rows=0, x=None, w=None, out=None) == pa.binding.PA_OK  # nothing to do: no launch


def test_read_probe_rejects_bad_arguments():
    L = pa.lib()

    def probe(src=A, ids=None, n=4, tile=4096, sink=A, waves=8):
        return L.pa_read_probe(src, ids, n, tile, sink, waves, None)
    assert probe(n=-1) == INVALID
    assert probe(tile=0) == INVALID
    assert probe(tile=1000) == INVALID       # not whole 1 KB runs
    assert probe(waves=6) == INVALID         # not whole workgroups of 4 waves
    assert probe(waves=0) == INVALID
    assert probe(sink=None) == INVALID
    assert probe(sink=A + 8) == INVALID
    assert probe(src=A + 4) == INVALID
    assert probe(ids=A + 2) == INVALID


def test_decode_noalloc_rejects_before_any_launch():
    L = pa.lib()

    def call(q=A, S=2, Hq=4, desc=None):
        d = desc or _desc()
        return L.pa_decode_noalloc(q, A, A, A, A, ctypes.c_float(0.125), A, S, Hq, 3, ctypes.byref(d), None)
    assert call(Hq=3) == INVALID
    assert call(Hq=34) == UNSUPPORTED
    assert call(q=None) == INVALID
    assert call(desc=_desc(head_dim=96)) == UNSUPPORTED
    assert call(S=0) == OK
