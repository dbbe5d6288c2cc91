"""A decode step (cache append, then paged attention), and a prefill,
captured in a HIP graph and replayed: the pages' remedy for launch-bound steps is to record the GPU
work once and resubmit it whole, which needs fixed shapes and fixed addresses
("Fast attention kernels and operator fusion", the-ai.news, section "Fusion
and CUDA Graphs with torch.compile"). Every replay, with eager work and
synchronisations between replays, must give exactly what the same calls give
eagerly, and match the oracle."""

import math

import pytest
import torch

import oracle
import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import inputs
from parity import assert_close, assert_lse_close, ref_decode, ref_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_captured_decode_step_replays_match_eager_and_oracle():
    print("[graph] append + decode step, 4 replays", flush=True)
    num_seqs, Hq, Hkv, d = 32, 8, 2, 128
    b = inputs.paged_inputs(num_seqs, Hq, Hkv, d, seq_len_range=(1, 700), seed=90,
                            max_blocks_per_seq=64)
    max_len = 64 * 16  # host bound baked into the graph: lengths may grow up to it
    static = {k: v.to(DEV) for k, v in b.items() if torch.is_tensor(v)}
    k_new = torch.empty(num_seqs, Hkv, d, dtype=torch.bfloat16, device=DEV)
    v_new = torch.empty_like(k_new)
    o = torch.empty_like(static["q"])
    lse = torch.empty(num_seqs, Hq, device=DEV)
    ws = torch.empty(attn.decode_paged_workspace_size(num_seqs, Hq, Hkv, d, max_len),
                     dtype=torch.uint8, device=DEV)

    def step():
        attn.kv_append(k_new, v_new, static["k_cache"], static["v_cache"], static["block_table"],
                       static["seq_lens"])
        attn.decode_paged(static["q"], static["k_cache"], static["v_cache"],
                          static["block_table"], static["seq_lens"], max_seq_len=max_len, o=o,
                          lse=lse, workspace=ws)

    kn0, vn0 = inputs.new_kv_rows(num_seqs, Hkv, d, 190, device=DEV)
    k_new.copy_(kn0)
    v_new.copy_(vn0)
    step()  # warm-up outside the capture (module load, first launch)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    table_rows = b["block_table"]
    lens = list(b["seq_lens_host"])
    for rep in range(4):
        # new step inputs, written into the captured (static) tensors: the
        # sequences grow by one token, with new q and new K/V rows
        lens = [min(L + 1, max_len) for L in lens]
        table = table_rows.clone()
        free = set(range(b["num_blocks"])) - set(int(x) for x in table_rows.flatten() if x >= 0)
        free = sorted(free)
        for n, L in enumerate(lens):
            nb = -(-L // 16)
            if int(table[n, nb - 1]) < 0:  # the sequence enters a new block
                table[n, nb - 1] = free.pop()
        table_rows = table
        static["block_table"].copy_(table.to(DEV))
        static["seq_lens"].copy_(torch.tensor(lens, dtype=torch.int32, device=DEV))
        q, _ = inputs.new_kv_rows(num_seqs, Hq, d, 300 + rep, device=DEV)  # new queries
        static["q"].copy_(q)
        kn, vn = inputs.new_kv_rows(num_seqs, Hkv, d, 200 + rep, device=DEV)
        k_new.copy_(kn)
        v_new.copy_(vn)
        kc_before = static["k_cache"].clone()
        vc_before = static["v_cache"].clone()
        torch.cuda.synchronize()

        graph.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        kc_g, vc_g = static["k_cache"].clone(), static["v_cache"].clone()

        # eager work between replays, then the same step eagerly from the
        # same starting cache
        junk = torch.randn(1 << 20, device=DEV).sum()
        static["k_cache"].copy_(kc_before)
        static["v_cache"].copy_(vc_before)
        o.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o), f"replay {rep}: o differs from the eager step"
        assert torch.equal(lse_g, lse), f"replay {rep}: lse differs from the eager step"
        assert torch.equal(kc_g.view(torch.int16), static["k_cache"].view(torch.int16))
        assert torch.equal(vc_g.view(torch.int16), static["v_cache"].view(torch.int16))
        del junk

        # and the oracle: append then decode on the CPU
        seq_lens = torch.tensor(lens, dtype=torch.int32)
        rk, rv = oracle.kv_append(kn.cpu(), vn.cpu(), kc_before.cpu(), vc_before.cpu(), table,
                                  seq_lens)
        ro, rl, rb = ref_decode(static["q"].cpu(), torch.from_numpy(rk).view(torch.bfloat16),
                                     torch.from_numpy(rv).view(torch.bfloat16), table, seq_lens,
                                     1.0 / math.sqrt(d))
        assert_close(o_g, ro, torch.bfloat16, f"graph replay {rep}")
        assert_lse_close(lse_g, rl, rb, f"graph replay {rep}")


def test_captured_prefill_replays_match_eager():
    # attn_prefill captured once (fixed shapes and addresses), replayed three
    # times with new q/k/v contents copied into the captured tensors and eager
    # work in between; every replay equals the eager call bit for bit
    print("[graph] prefill, 3 replays", flush=True)
    B, Hq, Hkv, T, d = 2, 8, 2, 700, 128
    q0, k0, v0 = inputs.prefill_inputs(B, Hq, Hkv, T, d, seed=400)
    q, k, v = q0.to(DEV), k0.to(DEV), v0.to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, T, device=DEV)
    attn.prefill(q, k, v, o, causal=True, lse=lse)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        attn.prefill(q, k, v, o, causal=True, lse=lse)
    torch.cuda.synchronize()
    for rep in range(3):
        qn, kn, vn = inputs.prefill_inputs(B, Hq, Hkv, T, d, seed=401 + rep)
        q.copy_(qn.to(DEV))
        k.copy_(kn.to(DEV))
        v.copy_(vn.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        junk = torch.randn(1 << 20, device=DEV).sum()
        o.zero_()
        attn.prefill(q, k, v, o, causal=True, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o), f"replay {rep}: o differs from the eager call"
        assert torch.equal(lse_g, lse), f"replay {rep}: lse differs from the eager call"
        del junk
        if rep == 0:  # and once against the oracle, on two heads
            ro, rl, rb = ref_prefill(qn, kn, vn, 1.0 / math.sqrt(d), causal=True, heads=[0, 5])
            assert_close(o_g[:, [0, 5]], ro[:, [0, 5]], torch.bfloat16, "graph prefill")
            assert_lse_close(lse_g[:, [0, 5]], rl[:, [0, 5]], rb[:, [0, 5]], "graph prefill lse")


def test_captured_mixed_call_replays_match_eager_and_oracle():
    # a paged call with chunk rows (one split along the keys) next to decodes:
    # the planning, chunk, merge, split-KV decode and decode merge kernels all
    # captured in one graph (the plan and partials live in the workspace and
    # are rewritten by every replay). Three replays with new q contents and
    # eager work in between; each equals the eager call bit for bit, the
    # first also the oracle
    print("[graph] mixed paged call, 3 replays", flush=True)
    seq_lens = [6000, 40, 700, 3]
    q_lens = [200, 1, 129, 1]
    Hq, Hkv, d = 8, 2, 128
    b = inputs.paged_inputs(len(seq_lens), Hq, Hkv, d, seq_lens=seq_lens, q_lens=q_lens, seed=95)
    s = {k: v.to(DEV) for k, v in b.items() if torch.is_tensor(v)}
    o = torch.empty_like(s["q"])
    lse = torch.empty(s["q"].shape[0], Hq, device=DEV)
    ws = torch.empty(attn.paged_workspace_size(len(seq_lens), sum(q_lens), Hq, Hkv, d,
                                               b["max_seq_len"], b["max_query_len"]),
                     dtype=torch.uint8, device=DEV)

    def call():
        attn.decode_paged(s["q"], s["k_cache"], s["v_cache"], s["block_table"], s["seq_lens"],
                          max_seq_len=b["max_seq_len"], max_query_len=b["max_query_len"],
                          query_start_loc=s["query_start_loc"], o=o, lse=lse, workspace=ws)

    call()  # warm-up outside the capture (module load, first launch)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        q, _ = inputs.new_kv_rows(sum(q_lens), Hq, d, 500 + rep, device=DEV)
        s["q"].copy_(q)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        junk = torch.randn(1 << 20, device=DEV).sum()
        o.zero_()
        lse.zero_()
        call()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o), f"replay {rep}: o differs from the eager call"
        assert torch.equal(lse_g, lse), f"replay {rep}: lse differs from the eager call"
        del junk
        if rep == 0:
            ro, rl, rb = ref_decode(s["q"].cpu(), b["k_cache"], b["v_cache"], b["block_table"],
                                    b["seq_lens"], 1.0 / math.sqrt(d),
                                    query_start_loc=b["query_start_loc"])
            assert_close(o_g, ro, torch.bfloat16, "graph mixed call")
            assert_lse_close(lse_g, rl, rb, "graph mixed call lse")
