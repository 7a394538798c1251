"""The Python binding's own checks, which run before any library call (no GPU needed): tensors that
are not on a GPU are refused, so no host address can reach a kernel."""

import pytest
import torch

import long_context_online_amd as m


def test_prefill_refuses_host_tensors():
    q = torch.zeros(1, 2, 128, 128, dtype=torch.bfloat16)
    k = v = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16)
    o = torch.zeros(1, 2, 128, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        m.blasst_prefill(q, k, v, o, causal=True, block_q=128, block_k=128, lam=0.01)


def test_decode_refuses_host_tensors():
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    kc = torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16)
    vc = torch.zeros(4, 2, 128, 16, dtype=torch.bfloat16)
    table = torch.zeros(2, 2, dtype=torch.int32)
    lens = torch.full((2,), 32, dtype=torch.int32)
    o = torch.zeros(2, 8, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        m.blasst_decode(q, kc, vc, table, lens, o, page_size=16, block_k=64, num_splits=1, lam=0.01)
    with pytest.raises(ValueError, match="GPU tensor"):
        m.blasst_decode_no_alloc(q, kc, vc, table, lens, o, page_size=16, block_k=64, num_splits=1, lam=0.01)


def test_backward_and_paged_prefill_refuse_host_tensors():
    q = torch.zeros(1, 2, 128, 128, dtype=torch.bfloat16)
    k = v = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 128)
    with pytest.raises(ValueError, match="GPU tensor"):
        m.blasst_prefill_backward(q, k, v, q, q, lse, q, k, v, causal=True)
    kc = torch.zeros(16, 1, 16, 128, dtype=torch.bfloat16)
    vc = torch.zeros(16, 1, 128, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        m.blasst_prefill_paged(q, kc, vc, torch.zeros(1, 16, dtype=torch.int32), torch.full((1,), 256, dtype=torch.int32),
                               q, lam=0.01)
