"""Dispatch build on the GPU vs the oracle: the four index structures
bit-exact, gates within 1e-6, on the five layer configs and edge shapes."""

import numpy as np
import pytest
import torch

from gpu_helpers import check_dispatch, oracle_dispatch, require_gpu, say
from token_dispatch_expert_amd import workloads as W
from token_dispatch_expert_amd.layer import MoELayerBuffers

pytestmark = pytest.mark.gpu


def _run(cfg, logits):
    dev = require_gpu()
    say(f"  dispatch L={cfg.L} E={cfg.E} K={cfg.K}")
    buf = MoELayerBuffers(cfg, dev)
    buf.build(logits.to(dev))
    torch.cuda.synchronize()
    check_dispatch(buf, oracle_dispatch(logits.cpu().numpy(), cfg))
    return buf


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5])
def test_dispatch_configs(ci):
    cfg = W.CONFIGS[ci]
    dev = require_gpu()
    buf = _run(cfg, W.make_logits(cfg, ci, dev))
    if ci == 4:  # the Zipf-skewed config leaves the last expert empty
        off = buf.offsets.cpu().numpy()
        assert off[cfg.E] == off[cfg.E - 1]


EDGE = [
    # L, E, K, kind
    (1, 8, 2, "normal"),
    (1, 1, 1, "normal"),
    (257, 8, 2, "normal"),          # ragged tile
    (1025, 16, 4, "normal"),        # one full tile + 1
    (3000, 1, 1, "normal"),         # E = 1
    (777, 8, 8, "normal"),          # K = E
    (500, 5, 3, "normal"),          # E not a multiple of 4 (scalar loads)
    (1000, 12, 3, "normal"),        # per-token register path, E below its vector width
    (999, 36, 5, "normal"),         # per-token register path, 64-wide, E = 36
    (513, 20, 20, "ties"),          # K = E on the per-token path, with ties
    (2000, 64, 6, "misaligned"),    # E = 64 with logits not 16-byte aligned
    (999, 100, 7, "normal"),        # 512-token tiles
    (700, 256, 8, "normal"),        # largest E, 256-token tiles
    (300, 256, 255, "normal"),      # largest K
    (2048, 64, 6, "ties"),          # many exact ties
    (4096, 16, 2, "empty_mid"),     # expert 7 never chosen
    (4096, 8, 1, "all_one"),        # every token on expert 3
    (5000, 32, 4, "misaligned"),    # logits not 16-byte aligned
    (1500, 16, 4, "ties"),          # streaming router, ties at the K-th value
    (600, 8, 8, "ties"),            # streaming router, K = E with ties
    (2000, 4, 1, "ties"),           # smallest streaming E, K = 1
    (1024, 32, 3, "signed_zero"),   # -0.0 and +0.0 rank as equal
    (2500, 28, 7, "normal"),        # streaming router, 7 chunks per row
    (3000, 40, 8, "normal"),        # 64-bit expert mask with E < 64
    (3001, 64, 8, "ties"),          # largest streaming E and K
    (64, 64, 6, "normal"),          # one whole part on the 64-expert register-load router
    (65, 64, 2, "normal"),          # its last part read from row 1, 63 rows back
    (63, 64, 4, "normal"),          # fewer than 64 tokens: the direct-to-LDS router
    (1500, 128, 8, "ties"),         # lane-pair router (E <= 128), ties at the K-th value
    (2000, 200, 5, "normal"),       # lane-quad router, last lane partly empty
    (1200, 130, 3, "normal"),       # lane-quad router, E not a multiple of 4
    (1100, 256, 1, "ties"),         # largest E, K = 1, ties
    (900, 96, 8, "signed_zero"),    # lane-pair router, signed zeros
    (3000, 252, 6, "misaligned"),   # lane-quad router, logits not 16-byte aligned
    (2000, 512, 6, "normal"),       # eight mask words per token
    (1500, 1024, 8, "normal"),      # largest E: sixteen mask words, four routing rounds
    (700, 1000, 3, "normal"),       # E not a multiple of 64: last word partly empty
    (999, 777, 8, "ties"),          # ties at the K-th value across sixteen lanes
    (600, 1024, 1, "ties"),         # largest E, K = 1
    (3000, 500, 4, "misaligned"),   # logits not 16-byte aligned, E = 500
    (1000, 300, 2, "signed_zero"),  # signed zeros, eight words
    (5000, 1024, 8, "empty_mid"),   # expert 7 never chosen, 1024 experts
    (4096, 640, 5, "all_one"),      # every token on expert 3
    (1, 1024, 8, "normal"),         # one token
    (129, 65, 8, "normal"),         # smallest wide E, ragged tile
]


@pytest.mark.parametrize("L,E,K,kind", EDGE, ids=[f"{k}-L{l}-E{e}-K{kk}" for l, e, kk, k in EDGE])
def test_dispatch_edges(L, E, K, kind):
    dev = require_gpu()
    cfg = W.small_config(L, 8, 8, E, K)
    g = torch.Generator().manual_seed(L * 1000 + E * 10 + K)
    z = torch.randn(L, E, generator=g)
    if kind == "ties":
        z = torch.randint(-2, 3, (L, E), generator=g).float()
    elif kind == "signed_zero":
        z = torch.randint(-1, 2, (L, E), generator=g).float() * 0.0
        z[torch.rand(L, E, generator=g) < 0.05] = 1.0
    elif kind == "empty_mid":
        z[:, 7] = -1e4
    elif kind == "all_one":
        z[:, 3] += 50.0
    if kind == "misaligned":
        store = torch.empty(L * E + 1, dtype=torch.float32, device=dev)
        zz = store[1:].view(L, E)
        zz.copy_(z.to(dev))
        assert zz.data_ptr() % 16 != 0
        buf = MoELayerBuffers(cfg, dev)
        buf.build(zz)
        torch.cuda.synchronize()
        check_dispatch(buf, oracle_dispatch(z.numpy(), cfg))
        return
    buf = _run(cfg, z)
    off = buf.offsets.cpu().numpy()
    if kind == "empty_mid":
        assert off[8] == off[7]
    if kind == "all_one":
        assert off[4] - off[3] == L


def test_dispatch_repeatable():
    dev = require_gpu()
    cfg = W.CONFIGS[3]
    z = W.make_logits(cfg, 7, dev)
    a = MoELayerBuffers(cfg, dev)
    b = MoELayerBuffers(cfg, dev)
    a.build(z)
    b.ws.fill_(0xFF)          # poisoned workspace must not matter
    b.build(z)
    torch.cuda.synchronize()
    for n in ("eti", "offsets", "tei", "tim", "gates"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n


def check_index_properties(L, E, K, eti, off, tei, tim, step=1 << 25):
    """Properties that fix the four index structures uniquely once the
    expert lists are known, checked on the device in chunks of tokens:
    token_expert_indices rows strictly ascending in [0, E); offsets from 0 to
    L*K with per-expert counts equal to the expert lists' histogram; each
    segment of expert_token_indices strictly ascending; and
    expert_token_indices[token_index_map[t, k]] = t, with token_index_map[t, k]
    inside the segment of token_expert_indices[t, k].  Returns the offsets."""
    dev = eti.device
    R = L * K
    offs = off.cpu().numpy().astype(np.int64)
    assert offs[0] == 0 and offs[E] == R and np.all(np.diff(offs) >= 0), "offsets"
    counts = torch.zeros(E, dtype=torch.int64, device=dev)
    offd = off.to(torch.int64)
    for t0 in range(0, L, step):
        t1 = min(L, t0 + step)
        te = tei[t0:t1].to(torch.int64)
        assert bool((te >= 0).all()) and bool((te < E).all()), "expert id out of range"
        assert bool((te[:, 1:] > te[:, :-1]).all()), "a token's experts not ascending"
        counts += torch.bincount(te.reshape(-1), minlength=E)
        tm = tim[t0:t1].to(torch.int64)
        assert bool((tm >= offd[te]).all()) and bool((tm < offd[te + 1]).all()), \
            "token_index_map outside its expert's segment"
        tok = torch.arange(t0, t1, device=dev, dtype=torch.int64).unsqueeze(1)
        assert bool((eti[tm.reshape(-1)].to(torch.int64).view_as(tm) == tok).all()), \
            "expert_token_indices[token_index_map] != token"
        del te, tm, tok
    assert np.array_equal(counts.cpu().numpy(), np.diff(offs)), "per-expert counts"
    for e in range(E):
        seg = eti[int(offs[e]):int(offs[e + 1])]
        if seg.numel() > 1:
            assert bool((seg[1:] > seg[:-1]).all()), f"expert {e}: tokens not ascending"
    return offs


def test_dispatch_max_size():
    """The largest routing the ABI accepts at K = 8: L = 2^28 - 1 tokens
    (L * K = 2^31 - 8 routes, the last 64-token part ragged), E = 16.  The
    oracle routes a sample of tokens one by one (their expert lists bit-exact,
    gates within 1e-6); everything else is checked through properties that
    fix it uniquely at any size: token_expert_indices rows strictly ascending
    and in range, per-expert counts equal to the offsets, each segment of
    expert_token_indices strictly ascending (so it is the sorted token list),
    and expert_token_indices[token_index_map[t, k]] = t with
    token_index_map[t, k] inside the segment of token_expert_indices[t, k]."""
    import oracle
    from token_dispatch_expert_amd import binding as B

    dev = require_gpu()
    E, K = 16, 8
    L = (2 ** 31 - 1) // K
    R = L * K
    say(f"  dispatch L={L} E={E} K={K} (L*K = {R})")
    g = torch.Generator(device=dev).manual_seed(2024)
    z = torch.randn(L, E, generator=g, device=dev, dtype=torch.float32)
    i32 = dict(dtype=torch.int32, device=dev)
    eti = torch.empty(R, **i32)
    off = torch.empty(E + 1, **i32)
    tei = torch.empty(L, K, **i32)
    tim = torch.empty(L, K, **i32)
    gates = torch.empty(L, K, dtype=torch.float32, device=dev)
    shape = B.make_shape(L, 8, 8, E, K)
    B.moe_dispatch_build(shape, z, eti, off, tei, tim, gates)
    torch.cuda.synchronize()

    check_index_properties(L, E, K, eti, off, tei, tim)
    # sampled tokens against the oracle (first, last and 4,096 random ones)
    gen = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(L - 64, L),
                                     gen.integers(0, L, 4096)]))
    ridx = torch.from_numpy(rows).to(dev)
    ref_tei, ref_gates = oracle.route(z[ridx].cpu().numpy(), K)
    assert np.array_equal(tei[ridx].cpu().numpy(), ref_tei), "sampled token_expert_indices"
    gerr = float(np.abs(gates[ridx].cpu().numpy().astype(np.float64) - ref_gates).max())
    assert gerr <= 1e-6, gerr
    say(f"    {rows.size} sampled tokens bit-exact (gates max-abs {gerr:.1e}); "
        f"properties hold on all {R} routes")


@pytest.mark.parametrize("L,E,K", [
    (3000, 16, 4),      # bit-mask router, direct-to-LDS rows
    (5000, 64, 6),      # 64-expert router, rows through registers
    (2000, 128, 8),     # wide router, two mask words
    (1500, 1024, 8),    # wide router, sixteen mask words
    (700, 32, 12),      # K > 8: byte map, one thread per token
    (800, 200, 12),     # K > 8, E > 64: byte map, lane groups per token
    (600, 30, 10),      # K > 8, E not a multiple of 4: lane groups, scalar loads
])
def test_dispatch_nonfinite_logits(L, E, K):
    """Logits with NaN and infinite entries are outside the contract: the
    results are unspecified but memory-safe, and every token still gets K
    distinct experts, so the index structures keep all their properties.
    Rows of finite logits route exactly as the oracle does."""
    import oracle
    from token_dispatch_expert_amd import binding as B

    dev = require_gpu()
    say(f"  dispatch L={L} E={E} K={K} with NaN / inf logits")
    g = torch.Generator().manual_seed(L + E + K)
    z = torch.randn(L, E, generator=g)
    u = torch.rand(L, E, generator=g)
    bad = torch.rand(L, generator=g) < 0.5          # half the tokens get non-finite entries
    z[bad.unsqueeze(1) & (u < 0.10)] = float("nan")
    z[bad.unsqueeze(1) & (u >= 0.10) & (u < 0.13)] = float("inf")
    z[bad.unsqueeze(1) & (u >= 0.13) & (u < 0.16)] = float("-inf")
    z[0] = float("nan")                             # a token with no finite logit
    i32 = dict(dtype=torch.int32, device=dev)
    eti, off = torch.empty(L * K, **i32), torch.empty(E + 1, **i32)
    tei, tim = torch.empty(L, K, **i32), torch.empty(L, K, **i32)
    gates = torch.empty(L, K, dtype=torch.float32, device=dev)
    B.moe_dispatch_build(B.make_shape(L, 8, 8, E, K), z.to(dev), eti, off, tei, tim, gates)
    torch.cuda.synchronize()
    check_index_properties(L, E, K, eti, off, tei, tim)
    fin = torch.isfinite(z).all(dim=1).numpy()
    rows = np.flatnonzero(fin)
    ref_tei, ref_gates = oracle.route(z.numpy()[rows], K)
    assert np.array_equal(tei.cpu().numpy()[rows], ref_tei), "finite rows routed differently"
    gerr = float(np.abs(gates.cpu().numpy()[rows].astype(np.float64) - ref_gates).max())
    assert gerr <= 1e-6, gerr
    say(f"    {int((~fin).sum())} tokens with non-finite logits: structures valid; "
        f"{rows.size} finite rows bit-exact")
