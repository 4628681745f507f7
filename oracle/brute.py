"""Brute-force paged decode in pure Python (TEST INFRASTRUCTURE ONLY).

For tiny shapes only.  No numpy arithmetic: lists, ``math.exp`` and
``math.fsum`` (exactly rounded sums).  It re-derives every step from the
pages independently of ``pao.c``:

- a token at position ``pos`` of a sequence sits in logical block
  ``pos // block_size`` at offset ``pos % block_size``; the block table turns
  the logical block into a physical one ("PagedAttention实现" page, write_kv);
- the slot of a token is ``physical_block * block_size + offset``
  ("04 - Paged Attention 实现进度", section B.2);
- decode attention takes one softmax over the whole context and returns the
  weighted sum of V (lecture 7 script, demo 2, paper eq. 4).
"""
import math


def bf16_bits_to_float(bits):
    """Exact value of a bfloat16 bit pattern (sign, 8-bit exponent, 7-bit mantissa)."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if man == 0 else math.nan
    if exp == 0:
        return sign * man * 2.0 ** (-133)      # subnormal: man * 2^-7 * 2^-126
    return sign * (1.0 + man / 128.0) * 2.0 ** (exp - 127)


def element(flat_pool, idx, is_bf16):
    v = flat_pool[idx]
    return bf16_bits_to_float(int(v)) if is_bf16 else float(v)


def decode(q, k_pool, v_pool, block_tables, context_lens, scale, num_kv_heads, head_dim,
           block_size, is_bf16=False):
    """q: nested lists [B][Hq][d]; pools: flat lists in [NB][Hkv][bs][d] order;
    block_tables: [B][max_blocks]; returns [B][Hq][d] floats."""
    out = []
    for b, n in enumerate(context_lens):
        hq = len(q[b])
        group = hq // num_kv_heads
        rows = []
        for h in range(hq):
            g = h // group
            qh = [bf16_bits_to_float(int(x)) if is_bf16 else float(x) for x in q[b][h]]
            if n == 0:
                rows.append([0.0] * head_dim)
                continue
            idx_of = []
            for pos in range(n):
                logical, offset = divmod(pos, block_size)
                physical = block_tables[b][logical]
                base = ((physical * num_kv_heads + g) * block_size + offset) * head_dim
                idx_of.append(base)
            scores = [scale * math.fsum(qh[i] * element(k_pool, base + i, is_bf16)
                                        for i in range(head_dim)) for base in idx_of]
            top = max(scores)
            weights = [math.exp(s - top) for s in scores]
            total = math.fsum(weights)
            rows.append([math.fsum(w * element(v_pool, base + i, is_bf16)
                                   for w, base in zip(weights, idx_of)) / total
                         for i in range(head_dim)])
        out.append(rows)
    return out


def prefill(q, cu_seqlens_q, k_pool, v_pool, block_tables, context_lens, scale, num_kv_heads,
            head_dim, block_size, is_bf16=False):
    """Causal prefill of a packed chunk batch: q nested lists [total_q][Hq][d];
    the chunk of sequence b is rows cu[b]..cu[b+1]-1, the last positions of
    its context_lens[b] tokens; row r at position p sees positions 0..p.
    Returns [total_q][Hq][d] floats."""
    out = [None] * len(q)
    for b, n in enumerate(context_lens):
        q0, q1 = cu_seqlens_q[b], cu_seqlens_q[b + 1]
        for r in range(q1 - q0):
            p = n - (q1 - q0) + r
            hq = len(q[q0 + r])
            group = hq // num_kv_heads
            rows = []
            for h in range(hq):
                g = h // group
                qh = [bf16_bits_to_float(int(x)) if is_bf16 else float(x) for x in q[q0 + r][h]]
                bases = []
                for pos in range(p + 1):
                    logical, offset = divmod(pos, block_size)
                    physical = block_tables[b][logical]
                    bases.append(((physical * num_kv_heads + g) * block_size + offset) * head_dim)
                scores = [scale * math.fsum(qh[i] * element(k_pool, base + i, is_bf16)
                                            for i in range(head_dim)) for base in bases]
                top = max(scores)
                weights = [math.exp(s - top) for s in scores]
                total = math.fsum(weights)
                rows.append([math.fsum(w * element(v_pool, base + i, is_bf16)
                                       for w, base in zip(weights, bases)) / total
                             for i in range(head_dim)])
            out[q0 + r] = rows
    return out
