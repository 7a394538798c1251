"""The five workloads, by shape (tiny MHA prefill; GQA prefill at 32K; paged GQA decode; the
calibration sweep with long prefill; latent (MLA-style) decode).  Sizes only, no arithmetic."""

CONFIGS = {
    # tiny MHA prefill that the oracle finishes in seconds; lambda = a / L
    1: dict(kind="prefill", batch=1, hq=2, hkv=2, L=512, d=64, dtype="fp32", causal=True,
            block_q=64, block_k=64, num_splits=1, window=False, a_values=[0.0, 0.5, 2.0, 8.0]),
    # Llama-3.1-8B-shaped GQA prefill
    2: dict(kind="prefill", batch=1, hq=32, hkv=8, L=32768, d=128, dtype="bf16", causal=True,
            block_q=128, block_k=128, num_splits=1, window=True, targets=[0.0, 0.5, 0.75]),
    # GQA decode over a paged KV cache
    3: dict(kind="decode", batch=32, hq=32, hkv=8, ctx_values=[32768, 131072], d=128, dtype="bf16",
            page_size=16, block_k=64, num_splits=16, window=True, target=0.73),
    # calibration sweep + long prefill
    4: dict(kind="calibration", hq=32, hkv=8, d=128, dtype="bf16", causal=True, block_q=128,
            block_k=128, L_values=[4096, 8192, 16384, 32768, 65536, 131072],
            s_values=[0.3, 0.5, 0.7], sample_rows=1024, final_L=131072, final_s=0.75, window=True),
    # latent-attention decode (DeepSeek-shaped): 576-dim scores, V = first 512 latent channels
    5: dict(kind="decode_latent", batch=64, hq=128, hkv=1, ctx=32768, d=576, dv=512,
            dtype="bf16", page_size=16, block_k=64, num_splits=16, window=True,
            targets=[0.5, 0.73]),
}


def config_seed(cfg: int, variant: int = 0) -> int:
    """Seed for a config's inputs: 1000 * config + variant index."""
    return 1000 * cfg + variant
