"""The Python binding's checks on GPU tensors: diagnostics buffers too small or of the wrong dtype,
non-contiguous dense decode operands and mismatched shapes are refused before any launch."""

import pytest
import torch

import long_context_online_amd as m

pytestmark = pytest.mark.gpu


def _prefill_args():
    q = torch.zeros(1, 2, 256, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 256, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(1, 2, 256, 128, dtype=torch.float32, device="cuda")
    return q, k, k.clone(), o


def test_prefill_buffer_checks():
    m.lib()
    q, k, v, o = _prefill_args()
    kw = dict(causal=True, block_q=128, block_k=128, lam=0.01)
    with pytest.raises(ValueError, match="skip_mask holds 7"):
        m.blasst_prefill(q, k, v, o, skip_mask=torch.zeros(7, dtype=torch.uint8, device="cuda"), **kw)
    with pytest.raises(TypeError, match="crit"):
        m.blasst_prefill(q, k, v, o, crit=torch.zeros(1, 2, 2, 2, dtype=torch.float64, device="cuda"), **kw)
    with pytest.raises(ValueError, match="lse holds"):
        m.blasst_prefill(q, k, v, o, lse=torch.zeros(1, 2, 255, device="cuda"), **kw)
    with pytest.raises(ValueError, match="o has shape"):
        m.blasst_prefill(q, k, v, o[:, :1], **kw)
    with pytest.raises(ValueError, match="v has shape"):
        m.blasst_prefill(q, k, v[:, :, :128], o, **kw)
    # the right sizes go through
    mask = torch.zeros(1, 2, 2, 2, dtype=torch.uint8, device="cuda")
    m.blasst_prefill(q, k, v, o, skip_mask=mask, lse=torch.zeros(1, 2, 256, device="cuda"), **kw)
    torch.cuda.synchronize()


def test_decode_layout_checks():
    m.lib()
    B, Hq, Hkv, D = 2, 8, 2, 128
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(8, Hkv, 16, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(8, Hkv, D, 16, dtype=torch.bfloat16, device="cuda")
    table = torch.arange(8, dtype=torch.int32, device="cuda").reshape(B, 4)
    lens = torch.full((B,), 64, dtype=torch.int32, device="cuda")
    o = torch.zeros(B, Hq, D, dtype=torch.float32, device="cuda")
    kw = dict(page_size=16, block_k=64, num_splits=1, lam=0.01)
    with pytest.raises(ValueError, match="q must be contiguous"):
        m.blasst_decode(torch.zeros(B, D, Hq, dtype=torch.bfloat16, device="cuda").transpose(1, 2), kc, vc, table,
                        lens, o, **kw)
    with pytest.raises(ValueError, match="o holds"):
        m.blasst_decode(q, kc, vc, table, lens, o[:1], **kw)
    with pytest.raises(TypeError, match="block_table"):
        m.blasst_decode(q, kc, vc, table.long(), lens, o, **kw)
    with pytest.raises(ValueError, match="seq_lens has shape"):
        m.blasst_decode(q, kc, vc, table, lens[:1], o, **kw)
    with pytest.raises(ValueError, match="v_cache has shape"):
        m.blasst_decode(q, kc, vc.transpose(2, 3).contiguous(), table, lens, o, **kw)
    with pytest.raises(ValueError, match="skip_mask holds"):
        m.blasst_decode(q, kc, vc, table, lens, o, skip_mask=torch.zeros(3, dtype=torch.uint8, device="cuda"), **kw)
    m.blasst_decode(q, kc, vc, table, lens, o, skip_mask=torch.zeros(B, Hkv, 1, 1, dtype=torch.uint8, device="cuda"),
                    **kw)
    torch.cuda.synchronize()
