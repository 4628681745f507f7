"""A decode step and a prefill step captured in a HIP graph (torch.cuda.graph)
and replayed.

The library's entry points only enqueue kernels on the caller's stream (no
allocation, no memset, no copy), so a serving loop can capture a step once
and replay it.  Each test captures a step on static buffers, then replays it
several times with new inputs copied into those buffers, with unrelated
eager work and synchronisations between the replays, and checks every replay
bit for bit against the same step run eagerly on the same inputs (every
kernel here is deterministic)."""
import numpy as np
import pytest

from tests import helpers as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from paged_kv_cache_261_amd import pa  # noqa: E402
from paged_kv_cache_261_amd import synthetic as S  # noqa: E402

MFMA, VECTOR = pa.PA_ALGO_MFMA, pa.PA_ALGO_VECTOR
BS, HKV, G, D = 16, 8, 4, 128


def forked_pool(rng, prompts=6, forks=4, prompt_len=304, tail_max=200):
    """Prompts of prompt_len tokens (whole blocks), each forked `forks` times;
    the forks share the prompt's physical blocks and own their tails' blocks.
    Returns the bf16 pool, tables, context lengths, and one new-token slot
    per sequence (its last position, inside its own tail)."""
    nseq = prompts * forks
    tails = rng.integers(1, tail_max + 1, size=nseq)
    ctx = (prompt_len + tails).astype(np.int32)
    max_blocks = int((ctx.max() + BS - 1) // BS)
    need = prompts * (prompt_len // BS) + int(sum((t + BS - 1) // BS for t in tails))
    nb = need + 16
    order = rng.permutation(nb).astype(np.int32)
    nxt = iter(order.tolist())
    kc = np.zeros((nb, HKV, BS, D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    tab = np.full((nseq, max_blocks), -1, dtype=np.int32)

    def put(blocks, pos0, k, v):
        for i in range(k.shape[0]):
            blk, off = blocks[(pos0 + i) // BS], (pos0 + i) % BS
            kc[blk, :, off, :] = k[i]
            vc[blk, :, off, :] = v[i]

    for p in range(prompts):
        pblocks = [next(nxt) for _ in range(prompt_len // BS)]
        put(pblocks, 0, S._normal(rng, (prompt_len, HKV, D), "bf16"),
            S._normal(rng, (prompt_len, HKV, D), "bf16"))
        for f in range(forks):
            b = p * forks + f
            t = int(tails[b])
            blocks = pblocks + [next(nxt) for _ in range((t + BS - 1) // BS)]
            tab[b, :len(blocks)] = blocks
            put(blocks, prompt_len, S._normal(rng, (t, HKV, D), "bf16"),
                S._normal(rng, (t, HKV, D), "bf16"))
    last = ctx - 1
    slots = np.array([int(tab[b, last[b] // BS]) * BS + int(last[b] % BS) for b in range(nseq)],
                     dtype=np.int64)
    return kc, vc, tab, ctx, slots


def _sync_noise():
    """Unrelated eager work between replays."""
    x = torch.randn(1 << 20, device="cuda")
    (x * 2).sum().item()
    torch.cuda.synchronize()


@pytest.mark.parametrize("part,algo,noalloc", [(0, MFMA, False), (512, MFMA, False),
                                               (pa.PA_PARTITION_BALANCED, MFMA, False),
                                               (pa.PA_PARTITION_SHARED, MFMA, False),
                                               (pa.PA_PARTITION_BALANCED, VECTOR, False),
                                               (pa.PA_PARTITION_BALANCED, MFMA, True),
                                               (pa.PA_PARTITION_SHARED, MFMA, True)])
def test_decode_step_graph_replays(part, algo, noalloc):
    """Slot write of each sequence's new token plus decode, captured once and
    replayed four times with new queries and new tokens."""
    rng = np.random.default_rng(900 + (part % 1000) + 10 * algo + 100 * noalloc)
    kc, vc, tab, ctx, slots = forked_pool(rng)
    nseq = len(ctx)
    scale = 1 / np.sqrt(D)
    mc = int(ctx.max())
    kd, vd = H.to_dev(kc), H.to_dev(vc)
    tabd, ctxd, slotd = H.to_dev(tab), H.to_dev(ctx), H.to_dev(slots)
    q = torch.empty((nseq, HKV * G, D), dtype=torch.bfloat16, device="cuda")
    knew = torch.empty((nseq, HKV, D), dtype=torch.bfloat16, device="cuda")
    vnew = torch.empty_like(knew)
    out_g = torch.full_like(q, float("nan"))
    out_e = torch.full_like(q, float("nan"))
    ws_g = None if noalloc else pa.workspace_for(q, kd, mc, part)
    ws_e = pa.workspace_for(q, kd, mc, part)

    def fill(i):
        r = np.random.default_rng(1000 * i + 7)
        q.copy_(H.to_dev(S._normal(r, (nseq, HKV * G, D), "bf16")))
        knew.copy_(H.to_dev(S._normal(r, (nseq, HKV, D), "bf16")))
        vnew.copy_(H.to_dev(S._normal(r, (nseq, HKV, D), "bf16")))

    def step(out, ws, graph_side):
        pa.pa_reshape_and_cache(knew, vnew, kd, vd, slotd)
        if graph_side and noalloc:
            pa.pa_decode_noalloc(out, q, kd, vd, tabd, ctxd, scale, mc, part, algo)
        else:
            pa.pa_decode(out, q, kd, vd, tabd, ctxd, scale, mc, part, ws, algo)

    fill(0)
    step(out_g, ws_g, True)          # eager warm-up (first use of the static scratch)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g, ws_g, True)
    torch.cuda.synchronize()
    for i in range(1, 5):
        fill(i)
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = H.as_bits(out_g).clone()
        _sync_noise()
        out_e.fill_(float("nan"))
        step(out_e, ws_e, False)
        torch.cuda.synchronize()
        assert torch.isfinite(out_e.float()).all()
        assert torch.equal(got, H.as_bits(out_e)), f"replay {i}, mode {part}, algo {algo}"
        _sync_noise()


def test_prefill_step_graph_replays():
    """Slot write of a chunk of new tokens per sequence plus the causal
    prefill of those rows, captured once and replayed with new chunks."""
    rng = np.random.default_rng(950)
    kc, vc, tab, ctx, _ = forked_pool(rng, prompts=4, forks=3)
    nseq = len(ctx)
    chunks = np.minimum(rng.integers(0, 90, size=nseq), ctx).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    total = int(cu[-1])
    # the chunk of sequence b is its last chunks[b] positions
    slots = np.concatenate([
        np.array([int(tab[b, p // BS]) * BS + p % BS
                  for p in range(int(ctx[b] - chunks[b]), int(ctx[b]))], dtype=np.int64)
        for b in range(nseq)])
    scale = 1 / np.sqrt(D)
    mc, mq = int(ctx.max()), int(chunks.max())
    kd, vd = H.to_dev(kc), H.to_dev(vc)
    tabd, ctxd, cud, slotd = H.to_dev(tab), H.to_dev(ctx), H.to_dev(cu), H.to_dev(slots)
    q = torch.empty((total, HKV * G, D), dtype=torch.bfloat16, device="cuda")
    knew = torch.empty((total, HKV, D), dtype=torch.bfloat16, device="cuda")
    vnew = torch.empty_like(knew)
    out_g = torch.full_like(q, float("nan"))
    out_e = torch.full_like(q, float("nan"))

    def fill(i):
        r = np.random.default_rng(2000 * i + 3)
        q.copy_(H.to_dev(S._normal(r, (total, HKV * G, D), "bf16")))
        knew.copy_(H.to_dev(S._normal(r, (total, HKV, D), "bf16")))
        vnew.copy_(H.to_dev(S._normal(r, (total, HKV, D), "bf16")))

    def step(out):
        pa.pa_reshape_and_cache(knew, vnew, kd, vd, slotd)
        pa.pa_prefill(out, q, kd, vd, tabd, cud, ctxd, mc, mq, scale)

    fill(0)
    step(out_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g)
    torch.cuda.synchronize()
    for i in range(1, 4):
        fill(i)
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = H.as_bits(out_g).clone()
        _sync_noise()
        out_e.fill_(float("nan"))
        step(out_e)
        torch.cuda.synchronize()
        assert torch.isfinite(out_e.float()).all()
        assert torch.equal(got, H.as_bits(out_e)), f"replay {i}"
        _sync_noise()
