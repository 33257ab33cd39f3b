"""Realized statistics of the seeded input recipes (CPU, reduced sizes)."""

import torch

import workloads


def test_sink_window_statistics():
    wl = workloads.gqa_sink_window(n=4096, heads_q=4, heads_kv=1, dtype=torch.float32)
    q, k = wl.q[0, :, 0].double(), wl.k[0, :, 0].double()
    s = q @ k.T
    dl = torch.arange(4096)[:, None] - torch.arange(4096)[None, :]
    notsink = (torch.arange(4096) >= 4)[None, :]
    win = (dl >= 0) & (dl < 512) & notsink
    far = (dl >= 512) & notsink
    assert abs(s[win].mean().item() - 2.0) < 0.25
    assert abs(s[far].mean().item()) < 0.25
    assert abs(s[:, :4].mean().item() - 6.0) < 0.5


def test_seeded_and_shapes():
    a = workloads.mha_temperature(batch=1, heads=2, n=256)
    b = workloads.mha_temperature(batch=1, heads=2, n=256)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.do, b.do)
    assert a.q.dtype == torch.bfloat16 and a.q.shape == (1, 256, 2, 128)
    c = workloads.decode_cache(batch=2, nk=1024)
    assert c.q.shape == (2, 1, 32, 128) and c.k.shape == (2, 1024, 8, 128)
    assert c.causal_offset == 1023
    s = workloads.small_fp32()
    assert s.q.dtype == torch.float32 and s.block_q == 64


def test_latent_mqa_layout_and_seed():
    wl = workloads.latent_mqa(batch=1, heads=4, n=256, dtype=None)
    assert wl.q.shape == (1, 256, 4, 576) and wl.k.shape == (1, 256, 1, 576)
    assert wl.v.shape == (1, 256, 1, 512)
    # the value is the latent: a view of the first d_v columns of the cached row
    assert wl.v.data_ptr() == wl.k.data_ptr() and torch.equal(wl.v, wl.k[..., :512])
    again = workloads.latent_mqa(batch=1, heads=4, n=256, dtype=None)
    assert torch.equal(wl.q, again.q) and torch.equal(wl.k, again.k)
    t = wl.extra["temperature"]
    assert ((t >= 1.0) & (t <= 4.0)).all()


def test_latent_decode_layout_and_seed():
    wl = workloads.latent_decode(batch=2, heads=16, nk=512, dtype=None)
    assert wl.q.shape == (2, 1, 16, 576) and wl.k.shape == (2, 512, 1, 576)
    assert wl.v.shape == (2, 512, 1, 512)
    assert wl.v.data_ptr() == wl.k.data_ptr() and torch.equal(wl.v, wl.k[..., :512])
    assert wl.block_q == 1 and wl.causal_offset == 511
    again = workloads.latent_decode(batch=2, heads=16, nk=512, dtype=None)
    assert torch.equal(wl.q, again.q) and torch.equal(wl.k, again.k)
    # the sinks: every head of a batch row scores the first keys high
    s = torch.einsum("bhd,bkd->bhk", wl.q[:, 0], wl.k[:, :4, 0])
    assert s.mean() > 4.0


def test_late_sink_statistics():
    q, k, v, do = workloads.late_sink(dtype=torch.float32)
    assert q.shape == k.shape == v.shape == do.shape == (1, 700, 2, 128)
    q2, k2, _, _ = workloads.late_sink(dtype=torch.float32)
    assert torch.equal(q, q2) and torch.equal(k, k2)
    s = torch.einsum("bqhd,bkhd->bhqk", q, k)[0]
    for h, gap in enumerate((15.0, 4.0)):
        generic_max = s[h, -1, 4:].max().item()
        sink_mean = s[h, 4:, :4].mean().item()
        assert 1.5 < generic_max < 4.5
        assert abs(sink_mean - (gap + 3.5)) < 1.5
