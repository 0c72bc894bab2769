"""Seeded input generator: determinism, shapes and the stated structure (no GPU)."""
import numpy as np
import pytest
import torch

from workloads import (WORKLOAD_NAMES, MODE_NOSA, MODE_RETRIEVAL, MODE_STREAMING,
                       append_tokens, generate, get_workload, query_at_step, small_workload)


def test_full_workload_shapes():
    w = get_workload("tiny")
    assert (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, w.t_cap) == (1, 4, 2, 64, "f32", 2048)
    assert all(p.block == 32 and p.top_k == 8 and p.force_sink and p.force_last for p in w.policies)
    w = get_workload("llama8b_layer")
    assert [p.mode for p in w.policies] == [MODE_STREAMING] * 4 + [MODE_RETRIEVAL] * 4
    assert w.t_cap == 32768 and w.group == 4
    w = get_workload("qwen7b_layer")
    assert w.group == 7 and w.batch == 4 and w.t_cap == 131072
    assert {p.block for p in w.policies} <= {16, 32, 64, 128}
    assert all(0.02 <= p.budget <= 0.10 for p in w.policies)
    # one draw per kv head, shared by every sequence
    assert all(w.policies[b * 4 + h] == w.policies[h] for b in range(4) for h in range(4))
    w = get_workload("nosa_drift")
    assert all(p.mode == MODE_NOSA and p.top_k == 16 and p.k_evict == 48 and p.sub_block == 16
               for p in w.policies)
    assert w.steps == 64 and w.drift == (0.9, 0.44) and w.batch == 32
    w = get_workload("mixed_serving")
    assert w.batch == 64 and all(8192 <= t <= 131072 for t in w.seq_lens)
    modes = {p.mode for p in w.policies}
    assert modes == {MODE_STREAMING, MODE_RETRIEVAL}


def test_block_layout():
    w = get_workload("qwen7b_layer")
    off = w.block_offsets()
    assert off[0] == 0 and off[-1] == sum(-(-w.t_cap // p.block) for p in w.policies)
    mo = w.mask_word_offsets()
    assert all(mo[u + 1] - mo[u] == -(-w.n_cap(u) // 32) for u in range(w.num_units))


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_small_generation_deterministic(name):
    w = small_workload(name)
    a = generate(w, "cpu")
    b = generate(w, "cpu")
    for x, y in ((a.q, b.q), (a.K, b.K), (a.V, b.V)):
        assert torch.equal(x, y)
    if w.has_nosa:
        assert torch.equal(a.logits, b.logits)
        assert a.logits.numel() == w.total_blocks
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    assert a.K.dtype == dt and a.K.shape == (w.batch, w.num_kv_heads, w.t_cap, w.head_dim)
    assert a.q.shape == (w.batch, w.num_q_heads, w.head_dim)
    for bi, T in enumerate(w.seq_lens):
        assert torch.count_nonzero(a.K[bi, :, T:]) == 0           # rows past the length stay zero
        for h in range(w.num_kv_heads):
            g = w.policies[bi * w.num_kv_heads + h].block
            n_tot = -(-T // g)
            nb = a.needles[(bi, h)]
            assert len(set(nb)) == len(nb) and all(0 < j < T // g and j != n_tot - 1 for j in nb)


def test_sink_and_needles_structure():
    w = small_workload("llama8b_layer")
    inp = generate(w, "cpu")
    K = inp.K.float()
    V = inp.V.float()
    # sink tokens 0-3: keys x8, values x0.1
    assert K[0, :, :4].abs().mean() > 5 * K[0, :, 4:64].abs().mean()
    assert V[0, :, :4].abs().mean() < 0.3 * V[0, :, 4:64].abs().mean()
    # needle blocks align with the group's mean query
    G = w.group
    qbar = inp.q.float().reshape(1, w.num_kv_heads, G, -1).mean(dim=2)
    for h in range(w.num_kv_heads):
        g = w.policies[h].block
        for j in inp.needles[(0, h)]:
            blk = K[0, h, j * g:(j + 1) * g]
            cos = torch.nn.functional.cosine_similarity(blk.mean(0), qbar[0, h], dim=0)
            assert cos > 0.9


def test_query_drift():
    w = small_workload("nosa_drift")
    q0 = query_at_step(w, 0).double()
    q1 = query_at_step(w, 1).double()
    q5 = query_at_step(w, 5).double()
    assert torch.equal(query_at_step(w, 5), query_at_step(w, 5))
    c1 = torch.nn.functional.cosine_similarity(q0.flatten(), q1.flatten(), dim=0)
    c5 = torch.nn.functional.cosine_similarity(q0.flatten(), q5.flatten(), dim=0)
    assert 0.8 < c1 < 0.95 and c5 < c1          # correlation 0.9 per step, decaying


def test_append_tokens_writes_one_seeded_row_per_sequence():
    w = small_workload("mixed_serving")
    w = w.replace(t_cap=max(w.seq_lens) + 4)
    a, b = generate(w, "cpu"), generate(w, "cpu")
    lens = list(w.seq_lens)
    K0 = a.K.clone()
    new_a = append_tokens(a, lens, 3)
    new_b = append_tokens(b, lens, 3)
    assert new_a == [T + 1 for T in lens] == new_b
    assert a.seq_lens.tolist() == new_a
    assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V)          # seeded
    for bi, T in enumerate(lens):
        assert torch.any(a.K[bi, :, T] != 0) and torch.any(a.V[bi, :, T] != 0)
        assert torch.equal(a.K[bi, :, :T], K0[bi, :, :T])            # earlier rows untouched
        assert not torch.any(a.K[bi, :, T + 1:] != 0)
    c = generate(w, "cpu")
    append_tokens(c, lens, 4)                                        # another step, other rows
    assert not torch.equal(a.K, c.K)
    full = w.replace(t_cap=max(lens))                                # sequences at capacity stay
    d = generate(full, "cpu")
    longest = int(np.argmax(lens))
    assert append_tokens(d, lens, 0)[longest] == lens[longest]
