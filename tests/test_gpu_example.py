"""The README's usage example, run as written and checked against the
oracle: a 300-token prompt written into a paged cache (RoPE + cache write,
then the chunked prefill over the cache) and one decode step whose launch
writes its own new token."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import check, f64, say
from workloads import to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_readme_example():
    say("case: the README example (300-token prompt, one decode step)")
    torch.manual_seed(0)
    # ---- the README example, as written there
    Hq, Hkv, D, NB = 12, 2, 128, 1024
    kc = torch.zeros(NB, Hkv, 16, D, dtype=torch.bfloat16, device="cuda")  # K blocks [block][kv head][token][D]
    vc = torch.zeros(NB, Hkv, D, 16, dtype=torch.bfloat16, device="cuda")  # V blocks, token-minor [block][kv head][D][token]
    pool = mi.Pool(NB)                                                     # host block pool, 16-token blocks
    table = np.full((1, 64), -1, dtype=np.int32)                          # block-table row of one sequence

    # prefill: a 300-token prompt
    T = 300
    q, k, v = (torch.randn(T, h, D, dtype=torch.bfloat16, device="cuda") for h in (Hq, Hkv, Hkv))
    slots = pool.seq_reserve(table[0], 0, T)                               # blocks for tokens 0 .. T-1
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    q_in = q.clone()                                                       # (kept for the check below)
    mi.attn_kv_cache_write_rope(q, k, v, pos, torch.from_numpy(slots).cuda(), kc, vc)  # q rotated in place
    o = mi.attn_prefill_paged(q, kc, vc, torch.from_numpy(table).cuda(),
                              torch.tensor([0, T], dtype=torch.int32, device="cuda"),  # cu_seqlens_q
                              torch.tensor([T], dtype=torch.int32, device="cuda"),     # context lengths
                              T)                                                        # max_seqlen_q

    # decode: one new token at position T, rotated and written by the decode launch
    q1, k1, v1 = (torch.randn(1, h, D, dtype=torch.bfloat16, device="cuda") for h in (Hq, Hkv, Hkv))
    slot1 = pool.seq_reserve(table[0], T, 1)
    o1 = mi.attn_decode_paged_rope(q1, k1, v1, torch.tensor([T], dtype=torch.int32, device="cuda"),
                                   torch.from_numpy(slot1).cuda(), kc, vc, torch.from_numpy(table).cuda(),
                                   torch.tensor([T + 1], dtype=torch.int32, device="cuda"), T + 1)
    torch.cuda.synchronize()
    # ---- end of the example

    ks_rot = oracle.round_bf16(oracle.rope(to_f64(k), np.arange(T), 10000.0))
    qs_rot = oracle.round_bf16(oracle.rope(to_f64(q_in), np.arange(T), 10000.0))
    ref = oracle.chunked_prefill([qs_rot], [ks_rot], [to_f64(v)])[0]
    check(f64(o), ref, torch.bfloat16, "example prefill")
    k_all = np.concatenate([ks_rot, oracle.round_bf16(oracle.rope(to_f64(k1), np.array([T]), 10000.0))])
    v_all = np.concatenate([to_f64(v), to_f64(v1)])
    q1_rot = oracle.round_bf16(oracle.rope(to_f64(q1), np.array([T]), 10000.0))
    ref1, _ = oracle.decode(q1_rot, [k_all], [v_all])
    check(f64(o1), ref1, torch.bfloat16, "example decode")
    pool.close()
