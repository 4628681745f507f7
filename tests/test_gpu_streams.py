"""Calls on different streams run concurrently and give the bits they give
alone.

The library keeps no state between calls apart from the allocation-free
entry point's per-GPU scratch (documented as shared by every call on a
GPU), so decodes, prefills and slot writes on separate streams, each with
its own outputs and workspace, may overlap freely.  Each test runs its calls
once one after the other for reference outputs, then several times with the
streams interleaved and no synchronisation between the streams, and checks
every output bit for bit."""
import numpy as np
import pytest

from tests import helpers as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from paged_kv_cache_261_amd import pa  # noqa: E402
from paged_kv_cache_261_amd import synthetic as S  # noqa: E402


def _decode_job(seed, part, algo):
    """A bf16 GQA decode problem resident on the GPU, with its own output
    and workspace, and the call that runs it on a given stream."""
    rng = np.random.default_rng(seed)
    hkv, G, d, bs = 8, 4, 128, 16
    ctxs = [int(x) for x in rng.integers(1, 3000, size=40)]
    q = S._normal(rng, (len(ctxs), hkv * G, d), "bf16")
    kl = [S._normal(rng, (n, hkv, d), "bf16") for n in ctxs]
    vl = [S._normal(rng, (n, hkv, d), "bf16") for n in ctxs]
    nb = sum((n + bs - 1) // bs for n in ctxs) + 7
    kc, vc, tab = H.paginate(kl, vl, bs, nb, rng, "bf16")
    qd, kd, vd = H.to_dev(q), H.to_dev(kc), H.to_dev(vc)
    td, cd = H.to_dev(tab), H.to_dev(np.array(ctxs, dtype=np.int32))
    mc = max(ctxs)
    out = torch.full_like(qd, float("nan"))
    ws = pa.workspace_for(qd, kd, mc, part)

    def run(stream):
        pa.pa_decode(out, qd, kd, vd, td, cd, 1 / np.sqrt(d), mc, part, ws, algo, stream=stream)
    return out, run


def _prefill_job(seed):
    rng = np.random.default_rng(seed)
    hkv, G, d, bs = 8, 4, 128, 16
    chunks = [int(x) for x in rng.integers(0, 300, size=12)]
    prefixes = [int(x) for x in rng.integers(0, 1500, size=12)]
    ctxs = [p + c for p, c in zip(prefixes, chunks)]
    q = S._normal(rng, (sum(chunks), hkv * G, d), "bf16")
    kl = [S._normal(rng, (n, hkv, d), "bf16") for n in ctxs]
    vl = [S._normal(rng, (n, hkv, d), "bf16") for n in ctxs]
    nb = sum((n + bs - 1) // bs for n in ctxs) + 5
    kc, vc, tab = H.paginate(kl, vl, bs, nb, rng, "bf16")
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    qd, kd, vd = H.to_dev(q), H.to_dev(kc), H.to_dev(vc)
    td, cd, cud = H.to_dev(tab), H.to_dev(np.array(ctxs, dtype=np.int32)), H.to_dev(cu)
    out = torch.full_like(qd, float("nan"))

    def run(stream):
        pa.pa_prefill(out, qd, kd, vd, td, cud, cd, max(ctxs), max(chunks), 1 / np.sqrt(d),
                      stream=stream)
    return out, run


def _write_job(seed):
    """Slot writes of new tokens into a pool of their own."""
    rng = np.random.default_rng(seed)
    hkv, d, bs, nb = 8, 128, 16, 4096
    n = 20000
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    k = H.to_dev(S._normal(rng, (n, hkv, d), "bf16"))
    v = H.to_dev(S._normal(rng, (n, hkv, d), "bf16"))
    sd = H.to_dev(slots)
    kc = torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)

    def run(stream):
        pa.pa_reshape_and_cache(k, v, kc, vc, sd, stream=stream)
    return kc, run


def test_concurrent_streams_give_the_solo_bits():
    jobs = [_decode_job(11, pa.PA_PARTITION_BALANCED, pa.PA_ALGO_MFMA),
            _decode_job(12, pa.PA_PARTITION_SHARED, pa.PA_ALGO_MFMA),
            _decode_job(13, 512, pa.PA_ALGO_MFMA),
            _decode_job(14, pa.PA_PARTITION_BALANCED, pa.PA_ALGO_VECTOR),
            _prefill_job(15),
            _write_job(16)]
    main = torch.cuda.current_stream()
    for _, run in jobs:
        run(main)
    torch.cuda.synchronize()
    solo = [H.as_bits(out).clone() for out, _ in jobs]
    assert all(torch.isfinite(out.float()).all() for out, _ in jobs[:5])
    streams = [torch.cuda.Stream() for _ in jobs]          # default priority
    for rnd in range(4):
        for out, _ in jobs[:5]:
            out.fill_(float("nan"))
        jobs[5][0].zero_()
        torch.cuda.synchronize()
        for rep in range(3):                                # interleaved launches
            for st, (_, run) in zip(streams, jobs):
                run(st)
        torch.cuda.synchronize()
        for i, (out, _) in enumerate(jobs):
            assert torch.equal(H.as_bits(out), solo[i]), f"round {rnd}, job {i}"
