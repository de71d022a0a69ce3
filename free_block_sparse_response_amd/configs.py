"""The five workload configurations of the SparsePR call, as plain data.

Each entry is one attention call: batch B, heads H, a (T, H, W) latent grid whose
raster order gives the N video tokens, head dimension d, the planner sizes (sampled
queries S, requested key groups C_k and query groups C_q), the probe count M, the
executed-pair density budget rho (probes included) and the ridge strength lambda.
The planner constants that the workloads leave open follow the method configuration
table of the paper (Table C.1: 25 initial k-means iterations, tolerance 1e-4).

Readings taken where a workload is silent (each is listed with its reason in the
design notes): the softmax scale is 1/sqrt(d); the seed is 0; lambda is 1e-3; the
stress workload's grid is 26x45x80 so that it has its stated 93,600 tokens, and its
sampled-query count is 512; the HunyuanVideo-like workload appends 256 text tokens.
"""

CONFIGS = {
    # Tiny fp32 call: 16-component mixture on a 4x16x16 grid.
    "c1": dict(dtype="f32", batch=1, heads=1, grid=(4, 16, 16), text_tokens=0, head_dim=64,
               cells=(4, 2, 2), drift=False, sink_frac=0.0,
               n_sampled=64, n_key_groups=16, n_query_groups=16, n_probes=32,
               density=0.25, ridge_lambda=1e-3, seed=0),
    # Single head group, bf16: 64 components per head on a 16x32x32 grid.
    "c2": dict(dtype="bf16", batch=1, heads=8, grid=(16, 32, 32), text_tokens=0, head_dim=128,
               cells=(4, 4, 4), drift=False, sink_frac=0.0,
               n_sampled=256, n_key_groups=64, n_query_groups=64, n_probes=256,
               density=0.22, ridge_lambda=1e-3, seed=0),
    # Wan-like 720p layer: spatial components whose means drift linearly over T.
    "c3": dict(dtype="bf16", batch=1, heads=40, grid=(21, 45, 80), text_tokens=0, head_dim=128,
               cells=(1, 8, 8), drift=True, sink_frac=0.0,
               n_sampled=512, n_key_groups=256, n_query_groups=256, n_probes=512,
               density=0.22, ridge_lambda=1e-3, seed=0),
    # HunyuanVideo-like 720p layer plus 256 text tokens with uniform random Q/K/V.
    "c4": dict(dtype="bf16", batch=1, heads=24, grid=(33, 45, 80), text_tokens=256, head_dim=128,
               cells=(4, 8, 8), drift=False, sink_frac=0.0,
               n_sampled=512, n_key_groups=384, n_query_groups=384, n_probes=512,
               density=0.24, ridge_lambda=1e-3, seed=0),
    # Tight-budget stress: 10% of tokens carry 3x key norm (attention sinks).
    "c5": dict(dtype="bf16", batch=1, heads=40, grid=(26, 45, 80), text_tokens=0, head_dim=128,
               cells=(4, 8, 8), drift=False, sink_frac=0.10,
               n_sampled=512, n_key_groups=512, n_query_groups=512, n_probes=1024,
               density=0.22, ridge_lambda=1e-3, seed=0),
}

C5_DENSITY_SWEEP = (0.10, 0.16, 0.22, 0.26)

KMEANS_MAX_ITER = 25
KMEANS_TOL = 1e-4


def seq_len(cfg):
    t, h, w = cfg["grid"]
    return t * h * w + cfg["text_tokens"]


def with_overrides(name, **kw):
    cfg = dict(CONFIGS[name])
    cfg.update(kw)
    return cfg
