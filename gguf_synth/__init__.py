"""Seeded synthetic inputs for the block-quantized matmul: raw GGUF-layout
weight blocks, fp32 activations and top-k routing tables.

Both the HIP path and the CPU oracle consume the identical buffers made here.
This module holds none of the method's arithmetic: it only places random
draws into block fields (fp16 scale fields at their byte offsets, uniformly
random bytes for packed quants).  Uniform random bytes give uniform 4-bit
quants and, for Q4_K, uniform independent 6-bit scales and mins, because
the 12 scale bytes carry each of their 96 bits in exactly one of the 16
six-bit fields; for Q5_K the same plus uniform 5-bit quants (each qh bit
is the top bit of exactly one quant); for Q6_K, uniform 6-bit quants (every bit of ql and qh
belongs to exactly one quant) and uniform signed 8-bit scales.  TQ2 (2-bit ternary)
codes follow 8:16 structured sparsity: in every 16 consecutive values exactly 8
are non-zero (a uniformly drawn 8-of-16 pattern) with uniform random signs, code
01 for +1 and 11 for -1, 00 for zero, four codes per byte from the low bits up.

Streams: numpy.random.default_rng([20261202, cfg, tensor]) with tensor ids
0 = scales, 1 = quants, 2 = activations, 3 = expert ids, 4 = router logits,
and 100 + 3*e + {0, 1, 2} for expert e's gate / up / down matrices.
"""
import numpy as np

SEED = 20261202

Q4_0, Q4_1, Q8_0, Q4_K, Q5_K, Q6_K, Q1_0, TQ2 = 2, 3, 8, 12, 13, 14, 41, 42
FORMATS = {"q4_0": Q4_0, "q4_1": Q4_1, "q8_0": Q8_0, "q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K,
           "q1_0": Q1_0, "tq2": TQ2}
NAMES = {v: k for k, v in FORMATS.items()}
BLOCK_ELEMS = {Q4_0: 32, Q4_1: 32, Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256, Q1_0: 128, TQ2: 128}
BLOCK_BYTES = {Q4_0: 18, Q4_1: 20, Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210, Q1_0: 18, TQ2: 34}

# scale distributions (fp64 uniform draws, rounded to fp16 by numpy)
D_RANGE = (1e-3, 2e-2)
M_RANGE = (-0.16, 0.0)  # Q4_1 block offset m
D6_RANGE = (1e-5, 2e-4)  # Q6_K super-block d (its 8-bit scales carry the rest)


def rng(cfg, tensor):
    return np.random.default_rng([SEED, int(cfg), int(tensor)])


def row_bytes(fmt, k):
    return k // BLOCK_ELEMS[fmt] * BLOCK_BYTES[fmt]


def _f16_field(g, count, lo, hi):
    return g.uniform(lo, hi, size=count).astype(np.float16).view(np.uint8).reshape(count, 2)


_NM_PATTERNS = None
_SPREAD8 = None


def _nm_patterns():
    """The 12870 16-bit masks with exactly 8 bits set, ascending."""
    global _NM_PATTERNS
    if _NM_PATTERNS is None:
        allm = np.arange(1 << 16, dtype=np.uint32)
        bits = np.unpackbits(allm.astype("<u2").view(np.uint8).reshape(-1, 2), axis=1).sum(axis=1)
        _NM_PATTERNS = allm[bits == 8]
    return _NM_PATTERNS


def _spread16(x):
    """Bit i of each 16-bit value moved to bit 2i (a 32-bit result)."""
    global _SPREAD8
    if _SPREAD8 is None:
        v = np.arange(256, dtype=np.uint32)
        sp = np.zeros(256, np.uint32)
        for i in range(8):
            sp |= ((v >> i) & 1) << (2 * i)
        _SPREAD8 = sp
    x = x.astype(np.uint32)
    return _SPREAD8[x & 0xFF] | (_SPREAD8[x >> 8] << 16)


def weights(fmt, n, k, cfg, tensor=0, d_range=D_RANGE, m_range=M_RANGE):
    """Random GGUF blocks for an [n][k] weight matrix -> uint8 [n][row_bytes]."""
    qk, bs = BLOCK_ELEMS[fmt], BLOCK_BYTES[fmt]
    if k % qk:
        raise ValueError(f"k={k} is not a multiple of {qk}")
    nblk = n * (k // qk)
    gs = rng(cfg, 10 * tensor + 0)  # scale fields
    gq = rng(cfg, 10 * tensor + 1)  # quant bytes
    out = np.empty((nblk, bs), np.uint8)
    if fmt == Q4_0:
        out[:, 0:2] = _f16_field(gs, nblk, *d_range)
        out[:, 2:18] = gq.integers(0, 256, size=(nblk, 16), dtype=np.uint8)
    elif fmt == Q4_1:
        out[:, 0:2] = _f16_field(gs, nblk, *d_range)
        out[:, 2:4] = _f16_field(gs, nblk, *m_range)
        out[:, 4:20] = gq.integers(0, 256, size=(nblk, 16), dtype=np.uint8)
    elif fmt == Q8_0:
        out[:, 0:2] = _f16_field(gs, nblk, *d_range)
        out[:, 2:34] = gq.integers(-127, 128, size=(nblk, 32), dtype=np.int8).view(np.uint8)
    elif fmt == Q4_K:
        out[:, 0:2] = _f16_field(gs, nblk, *d_range)   # d
        out[:, 2:4] = _f16_field(gs, nblk, *d_range)   # dmin
        out[:, 4:144] = gq.integers(0, 256, size=(nblk, 140), dtype=np.uint8)
    elif fmt == Q5_K:
        out[:, 0:2] = _f16_field(gs, nblk, *d_range)   # d
        out[:, 2:4] = _f16_field(gs, nblk, *d_range)   # dmin
        out[:, 4:176] = gq.integers(0, 256, size=(nblk, 172), dtype=np.uint8)  # scales, qh, qs
    elif fmt == Q1_0:
        out[:, 0:2] = _f16_field(gs, nblk, *d_range)
        out[:, 2:18] = gq.integers(0, 256, size=(nblk, 16), dtype=np.uint8)   # sign bits
    elif fmt == TQ2:
        out[:, 0:2] = _f16_field(gs, nblk, *d_range)
        ng = nblk * 8                                    # 16-value groups
        mask = _nm_patterns()[gq.integers(0, 12870, size=ng)]
        sign = gq.integers(0, 1 << 16, size=ng).astype(np.uint32)
        code = _spread16(mask) | (_spread16(mask & sign) << 1)   # 01 = +1, 11 = -1
        out[:, 2:34] = code.astype("<u4").view(np.uint8).reshape(nblk, 32)
    elif fmt == Q6_K:
        # ql[128], qh[64], 16 signed scale bytes: uniform random bytes;
        # d (fp16) last
        out[:, 0:208] = gq.integers(0, 256, size=(nblk, 208), dtype=np.uint8)
        out[:, 208:210] = _f16_field(gs, nblk, *(D6_RANGE if d_range is D_RANGE else d_range))
    else:
        raise ValueError(f"unknown format {fmt}")
    return out.reshape(n, row_bytes(fmt, k))


def activations(m, k, cfg, tensor=2, scale=1.0):
    """fp32 [m][k], standard normal drawn in fp64 then rounded to fp32."""
    return (rng(cfg, tensor).standard_normal((m, k)) * scale).astype(np.float32)


def routing(n_tokens, n_experts, top_k, cfg):
    """Top-k routing table: distinct uniform expert ids per token and softmax
    weights over standard-normal logits (softmax taken over the k chosen
    logits in fp64, stored fp32)."""
    gi = rng(cfg, 3)
    ids = np.stack([gi.choice(n_experts, top_k, replace=False) for _ in range(n_tokens)])
    logits = rng(cfg, 4).standard_normal((n_tokens, top_k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


def expert_weights(fmt, n_experts, n, k, cfg, which):
    """n_experts consecutive [n][k] matrices; which = 0 gate, 1 up, 2 down."""
    return np.concatenate(
        [weights(fmt, n, k, cfg, tensor=100 + 3 * e + which) for e in range(n_experts)], axis=0)


# The workloads.  Sizes are those of real GGUF tensors: a 1B-class attention
# projection, an 8B-class FFN-up, a 128K-vocabulary LM head, and an lfm2moe
# routed FFN (32 experts, top 4, hidden 2048, expert FFN width 1536).
CONFIGS = {
    "q4_0_gemv_2048": dict(cfg=0, kind="gemv", fmt=Q4_0, n=2048, k=2048, batches=(1,)),
    "q8_0_gemv_ffn_up": dict(cfg=1, kind="gemv", fmt=Q8_0, n=14336, k=4096, batches=(1, 5)),
    "q4_1_gemv_ffn_up": dict(cfg=11, kind="gemv", fmt=Q4_1, n=14336, k=4096, batches=(1, 5)),
    "q4_k_gemv_lm_head": dict(cfg=2, kind="gemv", fmt=Q4_K, n=128256, k=4096, batches=(1, 4)),
    # Q1_0 binary weights: the largest matvec of a 27B Q1_0 model
    # (attention QKV 10240 x 5120) at batch 1 and 4
    "q1_0_gemv_qkv": dict(cfg=41, kind="gemv", fmt=Q1_0, n=10240, k=5120, batches=(1, 4)),
    # the tied-embedding LM head in Q6_K
    "q6_k_gemv_lm_head": dict(cfg=22, kind="gemv", fmt=Q6_K, n=128256, k=4096, batches=(1, 4)),
    # Q5_K (the FFN type of Q5_K_M models): decode GEMV and prefill GEMM
    "q5_k_gemv_ffn_up": dict(cfg=15, kind="gemv", fmt=Q5_K, n=14336, k=4096, batches=(1, 5)),
    "q5_k_gemm_prefill_512": dict(cfg=25, kind="gemm", fmt=Q5_K, n=14336, k=4096, m=512),
    # Q6_K prefill GEMM (Q6_K holds the FFN-down and embedding tensors of
    # Q4_K_M models)
    "q6_k_gemm_prefill_512": dict(cfg=26, kind="gemm", fmt=Q6_K, n=14336, k=4096, m=512),
    "q4_0_gemm_prefill_512": dict(cfg=3, kind="gemm", fmt=Q4_0, n=14336, k=4096, m=512),
    "q4_0_gemm_prefill_2048": dict(cfg=13, kind="gemm", fmt=Q4_0, n=14336, k=4096, m=2048),
    "q4_k_moe_ffn": dict(cfg=4, kind="moe", fmt=Q4_K, n_tokens=256, hidden=2048, ffn=1536,
                         n_experts=32, top_k=4),
    # 2-bit sparse ternary (8:16): the FFN gate projection of a 70B-class
    # model, 28672 x 8192, at batch 1 and 4
    "tq2_gemv_70b_gate": dict(cfg=42, kind="gemv", fmt=TQ2, n=28672, k=8192, batches=(1, 4)),
}
