"""Streams on the GPU: every call is enqueued on the stream it is given and
keeps no state between calls, so sorts on two streams with their own temp
buffers may run at the same time (include/rs.h), and a sort enqueued behind
other work on a stream sees that work's results.  Streams keep the default
priority.  Results are compared bit for bit with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sorting_lsd_radix_amd as rs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def test_two_streams_run_independent_sorts():
    print("streams: 5e6 pairs and 9e6 keys on two streams, 3 rounds", flush=True)
    g = np.random.default_rng(21)
    kp = g.integers(0, 2**32, 5_000_000, dtype=np.uint32)
    vp = np.arange(kp.size, dtype=np.uint32)
    kk = g.integers(0, 2**32, 9_000_000, dtype=np.uint32)
    rk, rv = oracle.sort_u32(kp, vp)
    rkk = oracle.sort_u32(kk)
    tkp, tvp, tkk = (torch.from_numpy(a).to(DEV) for a in (kp, vp, kk))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            ko, vo = rs.sort_pairs_u32(tkp, tvp, stream=s1)
        with torch.cuda.stream(s2):
            kko = rs.sort_keys_u32(tkk, stream=s2)
        outs.append((ko, vo, kko))
    torch.cuda.synchronize()
    for ko, vo, kko in outs:
        assert np.array_equal(ko.cpu().numpy(), rk)
        assert np.array_equal(vo.cpu().numpy(), rv)
        assert np.array_equal(kko.cpu().numpy(), rkk)


def test_sort_is_ordered_after_work_on_its_stream():
    print("streams: upload then sort on one side stream, no sync between", flush=True)
    g = np.random.default_rng(22)
    keys = g.integers(0, 2**32, 7_000_000, dtype=np.uint32)
    vals = np.arange(keys.size, dtype=np.uint32)
    rk, rv = oracle.sort_u32(keys, vals, 3, 29)
    hk = torch.from_numpy(keys).pin_memory()
    hv = torch.from_numpy(vals).pin_memory()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dk = torch.empty(keys.size, dtype=torch.uint32, device=DEV)
        dv = torch.empty(keys.size, dtype=torch.uint32, device=DEV)
        dk.copy_(hk, non_blocking=True)
        dv.copy_(hv, non_blocking=True)
        ko, vo = rs.sort_pairs_u32(dk, dv, 3, 29, stream=s)
    s.synchronize()
    assert np.array_equal(ko.cpu().numpy(), rk)
    assert np.array_equal(vo.cpu().numpy(), rv)


def test_small_sort_paths_on_three_streams():
    """The hybrid path (top-digit pass, bucket sort), its multi-pass LSD
    fallback (skewed keys) and a small LSD sort whose passes use the wide
    look-back (214 tiles of 16384 keys), enqueued together on three streams."""
    print("streams: hybrid 2^20+3 pairs, fallback 2^20+5 pairs, 3.5e6 keys (wide look-back)",
          flush=True)
    g = np.random.default_rng(23)
    kh = g.integers(0, 2**32, (1 << 20) + 3, dtype=np.uint32)
    vh = np.arange(kh.size, dtype=np.uint32)
    # two top-digit values only: every key lands in two buckets of about 2^19
    kf = (g.integers(0, 2, (1 << 20) + 5, dtype=np.uint32) << np.uint32(24)) | \
        g.integers(0, 1 << 24, (1 << 20) + 5, dtype=np.uint32)
    vf = np.arange(kf.size, dtype=np.uint32)
    kw = g.integers(0, 2**32, 3_500_000, dtype=np.uint32)
    rkh, rvh = oracle.sort_u32(kh, vh)
    rkf, rvf = oracle.sort_u32(kf, vf)
    rkw = oracle.sort_u32(kw)
    t = [torch.from_numpy(a).to(DEV) for a in (kh, vh, kf, vf, kw)]
    s = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s[0]):
            a = rs.sort_pairs_u32(t[0], t[1], stream=s[0])
        with torch.cuda.stream(s[1]):
            b = rs.sort_pairs_u32(t[2], t[3], stream=s[1])
        with torch.cuda.stream(s[2]):
            c = rs.sort_keys_u32(t[4], stream=s[2])
        outs.append((a, b, c))
    torch.cuda.synchronize()
    for (ka, va), (kb, vb), kc in outs:
        assert np.array_equal(ka.cpu().numpy(), rkh) and np.array_equal(va.cpu().numpy(), rvh)
        assert np.array_equal(kb.cpu().numpy(), rkf) and np.array_equal(vb.cpu().numpy(), rvf)
        assert np.array_equal(kc.cpu().numpy(), rkw)
