"""pa_decode_noalloc (decode with the library's static per-GPU scratch)
against pa_decode with a caller-allocated workspace, through the C ABI.

Both run the same kernels on the same inputs, so their outputs must be the
same bits; both must also match the oracle (fp32: max abs error 1e-5; bf16:
per (sequence, head) row, max|d| / max|ref| <= 1e-2).  Each case makes two
calls in a row, the second on a smaller problem, so the second call reads a
scratch that still holds the first call's larger state.
"""
import math
import sys

import numpy as np
import pytest

from tests import helpers as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from oracle import pao  # noqa: E402
from paged_kv_cache_261_amd import pa  # noqa: E402
from paged_kv_cache_261_amd import synthetic as S  # noqa: E402

AUTO, VECTOR, MFMA = pa.PA_ALGO_AUTO, pa.PA_ALGO_VECTOR, pa.PA_ALGO_MFMA


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def problem(seed, dtype, hq, hkv, d, bs, ctxs):
    rng = np.random.default_rng(seed)
    q = S._normal(rng, (len(ctxs), hq, d), dtype)
    kl = [S._normal(rng, (n, hkv, d), dtype) for n in ctxs]
    vl = [S._normal(rng, (n, hkv, d), dtype) for n in ctxs]
    nb = sum((n + bs - 1) // bs for n in ctxs) + 7
    kc, vc, tab = H.paginate(kl, vl, bs, nb, rng, dtype)
    return q, kc, vc, tab, np.array(ctxs, dtype=np.int32)


def both(q, kc, vc, tab, ctx, scale, part, algo):
    """(pa_decode_noalloc output, pa_decode output), both NaN-prefilled."""
    qd, kd, vd = H.to_dev(q), H.to_dev(kc), H.to_dev(vc)
    td, cd = H.to_dev(tab), H.to_dev(ctx)
    mc = int(ctx.max())
    a = torch.full_like(qd, float("nan"))
    b = torch.full_like(qd, float("nan"))
    pa.pa_decode_noalloc(a, qd, kd, vd, td, cd, scale, mc, part, algo)
    ws = pa.workspace_for(qd, kd, mc, part)
    pa.pa_decode(b, qd, kd, vd, td, cd, scale, mc, part, ws, algo)
    torch.cuda.synchronize()
    return a, b


CASES = [   # dtype, algo, partition, (hq, hkv, d, bs), big contexts, small contexts
    ("bf16", MFMA, pa.PA_PARTITION_BALANCED, (32, 8, 128, 16),
     [3000, 17, 0, 2500, 4096, 1, 900] * 4, [5, 300, 0]),
    ("bf16", MFMA, pa.PA_PARTITION_SHARED, (32, 8, 128, 16),
     [2560, 2000, 77, 0, 1500, 16, 3100, 600] * 3, [40, 0, 19]),
    ("bf16", MFMA, 512, (64, 8, 128, 16), [32768, 20000, 513, 0], [512, 1, 1100]),
    ("bf16", AUTO, pa.PA_PARTITION_AUTO, (32, 8, 128, 16), [4000, 33, 1200] * 10, [64, 2]),
    ("bf16", MFMA, 0, (16, 4, 128, 32), [700, 0, 1300], [9]),
    ("bf16", VECTOR, pa.PA_PARTITION_BALANCED, (16, 4, 64, 16), [5000, 0, 333, 2048] * 3,
     [15, 16, 17]),
    ("f32", VECTOR, pa.PA_PARTITION_AUTO, (8, 8, 64, 16), [2048, 1, 700, 1999] * 8, [3, 100]),
    ("f32", VECTOR, 64, (4, 4, 16, 4), [5, 17, 33, 64], [4, 1]),
]


@pytest.mark.parametrize("dtype,algo,part,shape,big,small", CASES)
def test_noalloc_equals_workspace_decode(dtype, algo, part, shape, big, small):
    hq, hkv, d, bs = shape
    scale = 1 / math.sqrt(d)
    for call, ctxs in enumerate((big, small)):
        note(f"[no-alloc] {dtype} algo {algo} partition {part} shape {shape} "
             f"call {call} ({len(ctxs)} sequences, max ctx {max(ctxs)})")
        q, kc, vc, tab, ctx = problem(1000 * call + hq + d + len(big), dtype, hq, hkv, d, bs,
                                      ctxs)
        a, b = both(q, kc, vc, tab, ctx, scale, part, algo)
        assert torch.equal(H.as_bits(a), H.as_bits(b)), "outputs differ"
        got = a.float().cpu().numpy().astype(np.float64)
        ref = pao.decode_concat(q, kc, vc, tab, ctx, scale)
        for i, n in enumerate(ctx):
            if n == 0:
                assert (got[i] == 0).all()
        H.assert_close_to_oracle(got, ref, dtype, f"no-alloc call {call}")


def test_noalloc_rejects_problems_beyond_the_scratch():
    """A fixed-partition split whose workspace exceeds the static scratch
    returns PA_ERR_SCRATCH before anything is enqueued (the output keeps its
    contents); the next call that fits runs normally."""
    B, hq, hkv, d, bs, mc = 64, 64, 8, 128, 16, 16384
    need = pa.pa_decode_workspace_size(B, hq, hkv, d, bs, mc, 16, pa.PA_BF16)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, hq, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((8, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    tab = torch.zeros((B, mc // bs), dtype=torch.int32, device="cuda")
    ctx = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(pa.PAError) as err:
        pa.pa_decode_noalloc(out, q, kc, kc, tab, ctx, 0.1, mc, 16, MFMA)
    assert err.value.status == -8       # PA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    pa.pa_decode_noalloc(out, q, kc, kc, tab, ctx, 0.1, mc, pa.PA_PARTITION_BALANCED, MFMA)
    torch.cuda.synchronize()
    assert bool((out == 0).all())       # K = V = 0: every output is 0
