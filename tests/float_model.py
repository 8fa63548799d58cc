"""A textbook llama-style forward pass in float64, for the oracle's sanity pin.

It reads the same artifact, turns every fixed-point quantity into the real
number it stands for (weights (byte - 128) * scale / 2^24, norm weights and
rotary tables / 2^24, 1/sqrt(head) / 2^24) and runs RMSNorm with epsilon
1e-5, rotary on adjacent pairs, causal softmax attention with the true
exponential, a SiLU-gated feed-forward with the true SiLU, and residuals.
The fixed-point pass approximates this; a dropped term, a wrong sign or a
transposed operand in the oracle moves the logits far outside the bound the
test allows.  It shares nothing with the oracle.
"""
from __future__ import annotations

import numpy as np

from workloads import blob as B
from workloads.configs import Shape


class FloatModel:
    def __init__(self, blob: np.ndarray, shape: Shape):
        self.s = shape
        lay = B.plan(shape)
        q24 = float(1 << 24)

        def mat(kind, layer=0):
            w, sc = B.matrix_view(blob, shape, kind, layer)
            return (w.astype(np.float64) - 128.0) * (sc.astype(np.float64)[:, None] / q24)

        self.E = mat(B.KIND_EMBED)
        self.C = mat(B.KIND_CLS)
        self.layers = []
        for l in range(shape.layers):
            self.layers.append({k: mat(k, l) for k in B.LAYER_KINDS})
        o = lay.offsets
        d, L = shape.dim, shape.layers
        half = shape.head_size // 2
        norm = blob[o["norm"]: o["norm"] + 4 * (2 * L + 1) * d].view(np.int32).astype(np.float64) / q24
        self.norm = norm.reshape(2 * L + 1, d)
        n = shape.context * half
        self.cos = blob[o["cos"]: o["cos"] + 4 * n].view(np.int32).astype(np.float64).reshape(-1, half) / q24
        self.sin = blob[o["sin"]: o["sin"] + 4 * n].view(np.int32).astype(np.float64).reshape(-1, half) / q24
        self.inv = float(blob[44:48].view(np.uint32)[0]) / q24
        self.reset()

    def reset(self):
        self.K = [[] for _ in range(self.s.layers)]
        self.V = [[] for _ in range(self.s.layers)]
        self.pos = 0

    @staticmethod
    def rmsnorm(x, g):
        return x * g / np.sqrt(np.mean(x * x) + 1e-5)

    def rope(self, v, pos):
        hs = self.s.head_size
        v = v.reshape(-1, hs // 2, 2).copy()
        c, s = self.cos[pos], self.sin[pos]
        a, b = v[..., 0].copy(), v[..., 1].copy()
        v[..., 0] = a * c - b * s
        v[..., 1] = a * s + b * c
        return v.reshape(-1)

    def step(self, token: int):
        """Feeds one token, returns the logits after it."""
        s, pos = self.s, self.pos
        hs, H, KVH = s.head_size, s.heads, s.kv_heads
        x = self.E[token] * 1.0
        for l, W in enumerate(self.layers):
            xn = self.rmsnorm(x, self.norm[2 * l])
            q = self.rope(W[B.KIND_Q] @ xn, pos)
            k = self.rope(W[B.KIND_K] @ xn, pos)
            v = W[B.KIND_V] @ xn
            self.K[l].append(k)
            self.V[l].append(v)
            Kc = np.stack(self.K[l]).reshape(pos + 1, KVH, hs)
            Vc = np.stack(self.V[l]).reshape(pos + 1, KVH, hs)
            out = np.zeros(s.dim)
            for h in range(H):
                kh = h // (H // KVH)
                sc = Kc[:, kh, :] @ q[h * hs:(h + 1) * hs] * self.inv
                p = np.exp(sc - sc.max())
                p /= p.sum()
                out[h * hs:(h + 1) * hs] = p @ Vc[:, kh, :]
            x = x + W[B.KIND_O] @ out
            xn = self.rmsnorm(x, self.norm[2 * l + 1])
            g = W[B.KIND_GATE] @ xn
            u = W[B.KIND_UP] @ xn
            hdn = g / (1.0 + np.exp(-g)) * u
            x = x + W[B.KIND_DOWN] @ hdn
        self.pos += 1
        return self.C @ self.rmsnorm(x, self.norm[2 * s.layers]), x
