"""Near-tie rejection for seeded activations.

TEST INFRASTRUCTURE ONLY (used by the test-suite, the smoke check and the
golden-file scripts; never by the HIP path).

Expert selection is an arg-max decided by floating point.  The GPU sums the
router dot products in a different order from the oracle; the two float32
logits differ by about 1e-6 at H=2048.  A token whose k-th and (k+1)-th largest
logits lie closer than that could be routed differently by two correct
implementations.  Reading: such near-ties are treated as measure-zero events of
the input distribution, and a token row whose gap between rank k and rank k+1
is below ``TAU`` (in any layer that reads it) is re-drawn from the next
sub-stream of its seed.  The logits used for the check are the float64 router
products computed with numpy's matrix multiplication.
"""
from __future__ import annotations

import functools

import numpy as np

import moe_synth

TAU = 1e-4


def _f64(bits):
    return moe_synth.bf16_bits_to_f32(bits).astype(np.float64)


def router_logits_f64(x_bits, router_bits, logit_bias=None):
    l = _f64(x_bits) @ _f64(router_bits).T
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, dtype=np.float32).astype(np.float64)[None, :]
    return l


def kth_gap(logits, k):
    """Per token: (k-th largest) - ((k+1)-th largest); +inf when k equals E."""
    E = logits.shape[1]
    if k >= E:
        return np.full(logits.shape[0], np.inf)
    part = -np.partition(-logits, k, axis=1)[:, : k + 1]
    part.sort(axis=1)
    return part[:, 1] - part[:, 0]


def attempts(cfg, routers, T: int | None = None, tau: float = TAU) -> dict:
    """Re-draw counts (token -> attempt) that leave no near-tie under any of the
    given (router bits, logit bias) pairs."""
    k = cfg.shape.top_k
    att: dict[int, int] = {}
    x = moe_synth.token_rows(cfg, T)
    todo = np.arange(x.shape[0])
    for _ in range(64):
        bad = np.zeros(len(todo), dtype=bool)
        for R, b in routers:
            bad |= kth_gap(router_logits_f64(x[todo], R, b), k) < tau
        todo = todo[bad]
        if len(todo) == 0:
            return att
        for t in todo:
            att[int(t)] = att.get(int(t), 0) + 1
        xr = moe_synth.token_rows(cfg, x.shape[0], att)
        x[todo] = xr[todo]
    raise RuntimeError("near-tie rejection did not converge")


@functools.lru_cache(maxsize=None)
def attempts_for(cfg_name: str, T: int | None = None, tau: float = TAU):
    """Re-draw counts for a named config (every layer's router and offset)."""
    cfg = moe_synth.CONFIGS[cfg_name]
    routers = [(moe_synth.router_weights(cfg, l),
                moe_synth.zipf_bias(cfg, l) if cfg.zipf else None) for l in range(cfg.layers)]
    return tuple(sorted(attempts(cfg, routers, T, tau).items()))


def tokens_for(cfg, router, logit_bias=None, T: int | None = None) -> np.ndarray:
    """Activations of an ad-hoc config with near-ties re-drawn."""
    return moe_synth.token_rows(cfg, T, attempts(cfg, [(router, logit_bias)], T))


def tokens(cfg_name: str, T: int | None = None) -> np.ndarray:
    """Seeded activations of a config with near-ties re-drawn."""
    cfg = moe_synth.CONFIGS[cfg_name]
    return moe_synth.token_rows(cfg, T, dict(attempts_for(cfg_name, T)))
