"""The LM head and attention over packed weights: the packed bytes follow the documented tile
order (rebuilt here with NumPy from the row-major weights), and the packed call
returns exactly what the row-major call returns (same products, same
accumulation order), greedy and sampled, on ragged vocabularies, several
activation tiles and the 8B-shaped head."""
import numpy as np
import pytest
import torch

from tree_verified_block_amd import api

pytestmark = pytest.mark.gpu

WAVES, BLOCKS = 2048, 5  # the head grid's target wave count and blocks per wave


def _grid(V):
    NB = (V + 15) // 16
    per = min(-(-NB // WAVES), BLOCKS)
    NG = -(-NB // per)
    return NB, NG, per


def _pack_numpy(w: np.ndarray) -> np.ndarray:
    """[V][d] uint16 -> [d/64][NG][per][2][64 lanes][8] uint16, zero past V."""
    V, d = w.shape
    _, NG, per = _grid(V)
    out = np.zeros((d // 64, NG, per, 2, 64, 8), dtype=np.uint16)
    l = np.arange(64)
    for t in range(per):
        for G in range(NG):
            rows = (G + t * NG) * 16 + (l & 15)
            ok = rows < V
            for s in range(2):
                cols = 32 * s + 8 * (l >> 4)
                for c in range(d // 64):
                    idx = c * 64 + cols[:, None] + np.arange(8)[None, :]
                    out[c, G, t, s][ok] = w[rows[ok][:, None], idx[ok]]
    return out


def _bf16(shape, scale, gen):
    return (torch.randn(shape, generator=gen, device="cuda") * scale).to(torch.bfloat16)


@pytest.mark.parametrize("V,d", [(1000, 256), (4099, 512)])
def test_pack_layout(V, d):
    g = torch.Generator(device="cuda").manual_seed(V)
    w = _bf16((V, d), 1.0, g)
    packed = api.glance_head_pack(w)
    torch.cuda.synchronize()
    assert packed.numel() == api.head_pack_bytes(V, d)
    want = _pack_numpy(w.cpu().view(torch.int16).numpy().view(np.uint16))
    got = packed.cpu().numpy().view(np.uint16).reshape(want.shape)
    assert np.array_equal(got, want)


def _pack_attn_numpy(wq, wk, wv, wo, Hq, Hkv):
    """Packed q/k/v then wo (at the next 256-byte boundary), uint16, as
    [16-row blocks / 4][64-deep chunks][4 blocks][2 halves][64 lanes][8]: lane l
    of half s of block b, chunk c holds row block_row(b, l%16), columns
    64c + 32s + 8(l/16) .. + 8."""
    def pack(w, rows_of):
        N, K = w.shape
        NB = N // 16
        out = np.zeros((NB // 4, K // 64, 4, 2, 64, 8), dtype=np.uint16)
        l = np.arange(64)
        for b in range(NB):
            rows = rows_of(b, l & 15)
            for s in range(2):
                for c in range(K // 64):
                    cols = 64 * c + 32 * s + 8 * (l >> 4)
                    out[b // 4, c, b % 4, s] = w[rows[:, None], cols[:, None] + np.arange(8)[None, :]]
        return out.reshape(-1)

    nq, nk = Hq * 8, Hkv * 8

    def qkv_row(b, i):
        if b < nq + nk:
            base, bb = (0, b) if b < nq else (Hq * 128, b - nq)
            dim = np.where(i < 8, 8 * (bb & 7) + i, 64 + 8 * (bb & 7) + (i - 8))
            return base + (bb >> 3) * 128 + dim
        return (Hq + Hkv) * 128 + (b - nq - nk) * 16 + i

    a = pack(np.concatenate([wq, wk, wv]), qkv_row)
    pad = (-a.size) % 128  # 256 bytes
    return np.concatenate([a, np.zeros(pad, np.uint16), pack(wo, lambda b, i: 16 * b + i)])


def test_attn_pack_layout():
    Hq, Hkv, d = 8, 2, 512
    g = torch.Generator(device="cuda").manual_seed(11)
    lw = {"wq": _bf16((Hq * 128, d), 1.0, g), "wk": _bf16((Hkv * 128, d), 1.0, g),
          "wv": _bf16((Hkv * 128, d), 1.0, g), "wo": _bf16((d, Hq * 128), 1.0, g)}
    packed = api.glance_attn_pack(lw, Hq, Hkv)
    torch.cuda.synchronize()
    u16 = {k: v.cpu().view(torch.int16).numpy().view(np.uint16) for k, v in lw.items()}
    want = _pack_attn_numpy(u16["wq"], u16["wk"], u16["wv"], u16["wo"], Hq, Hkv)
    got = packed.cpu().numpy().view(np.uint16)
    assert got.size == want.size
    assert np.array_equal(got, want)


def _heads(V, d, R, seed, sample=None):
    g = torch.Generator(device="cuda").manual_seed(seed)
    w = _bf16((V, d), 0.05, g)
    h = _bf16((R, d), 1.0, g)
    packed = api.glance_head_pack(w)
    outs = []
    for use_packed in (False, True):
        o = {k: torch.empty(R, dtype=torch.float32, device="cuda") for k in ("top1", "gap", "H", "sgap")}
        o["am"] = torch.empty(R, dtype=torch.int32, device="cuda")
        o["tok"] = torch.empty(R, dtype=torch.int32, device="cuda")
        o["logits"] = torch.empty((R, V), dtype=torch.float32, device="cuda")
        ws = api.workspace(api.verify_head_ws_bytes(R, V, d, 1), "cuda")
        if use_packed:
            kw = {}
            if sample:
                kw = dict(temperature=sample[0], seed=sample[1], round_id=sample[2],
                          sample_tok=o["tok"], sample_gap=o["sgap"])
            api.glance_verify_head_packed(h, packed, V, o["am"], o["top1"], o["gap"], o["H"], ws,
                                          logits=o["logits"], **kw)
        elif sample:
            api.glance_verify_head_sampled(h, w, sample[0], sample[1], sample[2], o["am"],
                                           o["top1"], o["gap"], o["H"], o["tok"], o["sgap"], ws,
                                           logits=o["logits"])
        else:
            api.glance_verify_head(h, w, o["am"], o["top1"], o["gap"], o["H"], ws,
                                   logits=o["logits"])
        torch.cuda.synchronize()
        outs.append({k: v.cpu().numpy() for k, v in o.items()})
    return outs


# Rows beyond 64 take the packed kernel's two-tile work-groups (each weight chunk
# applied to 128 activation rows): 100 and 150 rows leave the last pair of tiles
# partly or wholly empty, 512 rows are the ragged 8-round batch.
@pytest.mark.parametrize("V,d,R", [(1000, 256, 64), (4099, 512, 100), (4099, 512, 150),
                                   (151936, 4096, 64), (151936, 4096, 512)])
def test_packed_head_equals_row_major(V, d, R):
    ref, got = _heads(V, d, R, seed=V + R)
    for k in ("am", "top1", "gap", "H", "logits"):
        assert np.array_equal(ref[k], got[k]), k


@pytest.mark.parametrize("R", [64, 130])
def test_packed_head_sampled_equals_row_major(R):
    ref, got = _heads(151936, 4096, R, seed=5, sample=(0.8, (1 << 40) + 7, 123))
    for k in ("am", "top1", "gap", "H", "tok", "sgap"):
        assert np.array_equal(ref[k], got[k]), k


@pytest.mark.parametrize("name,seed,kw", [
    ("mini_bf16", 1, {}),
    ("mini_bf16_ragged", 9, dict(draft="topology", n_layers=3, nseq=2, N=63, L=15)),
    ("qwen8b_1layer", 2000, {}),
    ("mini_bf16_full", 3, {}),
])
def test_packed_round_equals_row_major(name, seed, kw):
    """A whole round with the packed head and attention weights (and, for full
    layers, the packed MLP weights): every output equals the row-major round's
    (tree, hidden rows, new cache entries, head statistics, walk)."""
    from synth import gen_round, make_config
    from tree_verified_block_amd.round import DeviceRound
    inp = gen_round(make_config(name, **kw), seed)
    outs = []
    for packed in (False, True):
        dev = DeviceRound(inp, packed_head=packed)
        dev.set_round(0)
        dev.run()
        outs.append(dev.fetch())
        del dev
        torch.cuda.empty_cache()
    ref, got = outs
    for k in ref:
        assert np.array_equal(ref[k], got[k]), k


@pytest.mark.parametrize("name,seed,kw,T", [
    ("mini_bf16_ragged", 9, dict(nseq=3), None),
    ("mini_bf16_ragged", 10, dict(nseq=3), 0.7),
    ("qwen8b_ragged8", 5001, {}, None),
])
def test_fused_walk_equals_head_then_walk(name, seed, kw, T):
    """glance_verify_head_walk (the head's last row to finish walks every round)
    returns what glance_verify_head_packed followed by glance_accept_walk returns,
    greedy and sampled, over several sequences, call after call (the arrival word
    returns to zero)."""
    from synth import gen_round, make_config
    from tree_verified_block_amd.round import DeviceRound
    inp = gen_round(make_config(name, **kw), seed)
    dev = DeviceRound(inp, packed_head=True, temperature=T, seed=77)
    outs = []
    for rep in range(3):
        dev.set_round(0)
        dev.round_id = 5
        dev.step_tree()
        dev.step_attn()
        if rep == 0:
            dev.step_head()
            dev.step_walk()
        else:
            dev.step_verify()
        outs.append(dev.fetch())
    for got in outs[1:]:
        for k in outs[0]:
            assert np.array_equal(np.asarray(got[k]), np.asarray(outs[0][k])), k


def test_head_timing_events_bracket_the_gemm():
    """glance_head_timing: the two events land around the head GEMM (a positive
    span, shorter than the whole call with its row merge), recording changes no
    output, and clearing the hook stops the recording."""
    V, d, R = 4099, 512, 64
    g = torch.Generator(device="cuda").manual_seed(5)
    w = _bf16((V, d), 0.05, g)
    h = _bf16((R, d), 1.0, g)
    packed = api.glance_head_pack(w)
    st = torch.cuda.current_stream()
    outs = []
    for timed in (False, True, False):
        o = {k: torch.empty(R, dtype=torch.float32, device="cuda") for k in ("top1", "gap", "H")}
        o["am"] = torch.empty(R, dtype=torch.int32, device="cuda")
        ws = api.workspace(api.verify_head_ws_bytes(R, V, d, 1), "cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in ev:
            e.record(st)
        torch.cuda.synchronize()
        if timed:
            api.glance_head_timing(ev[1], ev[2])
        ev[0].record(st)
        try:
            api.glance_verify_head_packed(h, packed, V, o["am"], o["top1"], o["gap"], o["H"], ws)
        finally:
            api.glance_head_timing(None, None)
        ev[3].record(st)
        torch.cuda.synchronize()
        if timed:
            inner, outer = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
            assert 0.0 < inner < outer
            assert ev[0].elapsed_time(ev[1]) >= 0.0 and ev[2].elapsed_time(ev[3]) > 0.0
        else:
            # untimed: the events were recorded before the call only
            assert ev[1].elapsed_time(ev[0]) >= 0.0
        outs.append({k: v.cpu().numpy() for k, v in o.items()})
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]) and np.array_equal(outs[0][k], outs[2][k]), k


@pytest.mark.parametrize("nbytes,n_wg", [(16, 1), (4096 + 48, 3), (1 << 22, 257)])
def test_read_probe_reads_every_word(nbytes, n_wg):
    """glance_read_probe reads each 16-byte word once: the XOR of the
    work-groups' words is the XOR of the whole buffer (ragged last step and
    grids larger than the buffer included)."""
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(n_wg, dtype=torch.int32, device="cuda")
    api.glance_read_probe(buf, out, n_wg)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)

