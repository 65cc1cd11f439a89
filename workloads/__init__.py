"""Seeded synthetic inputs for the integrity scan, shared by the tests, the
smoke check and the benchmark.

This module only generates data and writes corruptions into it; it holds none
of the scan's arithmetic.  Values come from ``torch.Generator(device)`` seeded
with the workload's seed; every discrete choice (replica, tensor, element,
bit, NaN positions, sizes, dtypes) comes from ``numpy.random.default_rng``
with the same seed.  Corruptions are written through byte views, so NaN
payloads and every other bit pattern survive exactly.

Workloads (shapes of the training setups these checks run on):
  c1  one fp32 tensor of 1,048,576 elements, N(0, 0.02), 3 replicas, one bit
      flipped in replica 1.
  c2  GPT-style decoder parameter list in fp32 (d_model 2048, 17 layers,
      vocab 50304 tied, ~0.96B parameters), 3 replicas, one bit flipped in a
      seeded replica / tensor / element.
  c3  the gradients of the same shapes, fp32 N(0, 1e-3), with NaN/Inf written
      at rate 1e-7, plus a replay copy that differs by one flipped bit.
  c4  100,000 small tensors, sizes log-uniform in 1..65,536, dtypes mixed
      fp32/bf16/fp16, carved from one byte buffer per replica at element-
      aligned offsets, 3 replicas, 5 single-bit corruptions.
  c5  Llama-70B-shaped bf16 parameter list (d 8192, 80 layers, GQA 64/8 heads,
      FFN 28672, vocab 128256 untied, RMSNorm), ~70.55B parameters, 1 copy.
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch

F32, BF16, F16 = 0, 1, 2
TORCH_OF = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}
ESIZE = {F32: 4, BF16: 2, F16: 2}
CODE_OF = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


@dataclass
class Workload:
    name: str
    R: int                      # replicas (copies) laid out replica-major
    T: int                      # tensors per replica
    tensors: list               # R*T tensors (None allowed), tensor k of replica r at r*T+k
    names: list                 # T names
    seed: int
    injections: list = field(default_factory=list)   # dicts: replica, tensor, index, bit, was
    nonfinite: list = field(default_factory=list)    # (tensor, index, pattern) written
    meta: dict = field(default_factory=dict)
    buffers: list = field(default_factory=list)      # backing storage kept alive

    def replica(self, r):
        return self.tensors[r * self.T:(r + 1) * self.T]

    @property
    def bytes_per_replica(self):
        return sum(t.numel() * t.element_size() for t in self.replica(0) if t is not None)

    @property
    def elems_per_replica(self):
        return sum(t.numel() for t in self.replica(0) if t is not None)


# ---------------------------------------------------------------------------
# corruption helpers (byte views)
# ---------------------------------------------------------------------------
def read_bit(t, index, bit):
    es = t.element_size()
    b = t.detach().reshape(-1).view(torch.uint8)[index * es + bit // 8].item()
    return (b >> (bit % 8)) & 1


def flip_bit(t, index, bit):
    """Flips bit `bit` (0 = least significant) of element `index` in place;
    returns the bit's previous value."""
    es = t.element_size()
    assert 0 <= bit < 8 * es and 0 <= index < t.numel()
    bv = t.detach().reshape(-1).view(torch.uint8)
    pos = index * es + bit // 8
    was = (bv[pos].item() >> (bit % 8)) & 1
    bv[pos] ^= (1 << (bit % 8))
    return was


def write_pattern(t, index, pattern):
    """Writes the raw little-endian bit pattern `pattern` into element `index`."""
    es = t.element_size()
    bv = t.detach().reshape(-1).view(torch.uint8)
    raw = torch.tensor(list(int(pattern).to_bytes(es, "little")), dtype=torch.uint8)
    bv[index * es:(index + 1) * es] = raw.to(bv.device)


def _normal_(t, std, gen):
    return t.normal_(0.0, std, generator=gen)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _is_finite_element(t, index):
    v = t.reshape(-1)[index:index + 1]
    return bool(torch.isfinite(v).item())


# ---------------------------------------------------------------------------
# c1
# ---------------------------------------------------------------------------
def c1(device, seed=1, numel=1 << 20, R=3, corrupt_replica=1):
    rng = np.random.default_rng(seed)
    g = _gen(device, seed)
    base = _normal_(torch.empty(numel, dtype=torch.float32, device=device), 0.02, g)
    reps = [base] + [base.clone() for _ in range(R - 1)]
    i, b = int(rng.integers(0, numel)), int(rng.integers(0, 32))
    was = flip_bit(reps[corrupt_replica], i, b)
    return Workload("c1_fp32_1M_r3", R, 1, reps, ["w"], seed,
                    injections=[dict(replica=corrupt_replica, tensor=0, index=i, bit=b, was=was)])


# ---------------------------------------------------------------------------
# c2 / c3: GPT-style decoder, d_model 2048, 17 layers, vocab 50304 tied
# ---------------------------------------------------------------------------
def gpt_shapes(d=2048, layers=17, vocab=50304):
    """(name, shape, kind) in named-parameter order; kind is 'w' (matrix),
    'b' (bias), 'g' (LayerNorm gain) or 'e' (embedding)."""
    out = [("wte", (vocab, d), "e")]
    for l in range(layers):
        p = f"h{l}."
        out += [(p + "ln1.w", (d,), "g"), (p + "ln1.b", (d,), "b"),
                (p + "qkv.w", (3 * d, d), "w"), (p + "qkv.b", (3 * d,), "b"),
                (p + "out.w", (d, d), "w"), (p + "out.b", (d,), "b"),
                (p + "ln2.w", (d,), "g"), (p + "ln2.b", (d,), "b"),
                (p + "fc.w", (4 * d, d), "w"), (p + "fc.b", (4 * d,), "b"),
                (p + "proj.w", (d, 4 * d), "w"), (p + "proj.b", (d,), "b")]
    out += [("ln_f.w", (d,), "g"), ("ln_f.b", (d,), "b")]
    return out


def c2(device, seed=2, R=3, shapes=None):
    """GPT-style parameters: matrices and embedding N(0, 0.02), biases 0,
    LayerNorm gains 1; R replicas; one seeded bit flip in a seeded replica."""
    shapes = shapes or gpt_shapes()
    rng = np.random.default_rng(seed)
    g = _gen(device, seed)
    base = []
    for name, shape, kind in shapes:
        t = torch.empty(shape, dtype=torch.float32, device=device)
        if kind in ("w", "e"):
            _normal_(t, 0.02, g)
        elif kind == "g":
            t.fill_(1.0)
        else:
            t.zero_()
        base.append(t)
    tensors = list(base)
    for _ in range(R - 1):
        tensors += [t.clone() for t in base]
    T = len(base)
    r = int(rng.integers(0, R))
    k = int(rng.integers(0, T))
    i = int(rng.integers(0, base[k].numel()))
    b = int(rng.integers(0, 32))
    was = flip_bit(tensors[r * T + k], i, b)
    return Workload("c2_gpt0.96b_fp32_r3", R, T, tensors, [s[0] for s in shapes], seed,
                    injections=[dict(replica=r, tensor=k, index=i, bit=b, was=was)])


NAN_PATTERNS = (0x7F800000, 0xFF800000, 0x7FC00000)  # +Inf, -Inf, default quiet NaN


def c3(device, seed=3, rate=1e-7, shapes=None):
    """Gradient list (fp32 N(0, 1e-3)) with NaN/Inf at `rate`, and a replay
    copy that differs from it by one flipped bit at a finite element.
    Laid out as R=2: tensors[0:T] original, tensors[T:2T] replay."""
    shapes = shapes or gpt_shapes()
    rng = np.random.default_rng(seed)
    g = _gen(device, seed)
    grads = [_normal_(torch.empty(s, dtype=torch.float32, device=device), 1e-3, g)
             for _, s, _ in shapes]
    T = len(grads)
    sizes = np.array([t.numel() for t in grads], dtype=np.int64)
    cum = np.concatenate([[0], np.cumsum(sizes)])
    N = int(cum[-1])
    k = int(rng.binomial(N, rate))
    flat = np.sort(rng.choice(N, size=k, replace=False)) if k else np.zeros(0, dtype=np.int64)
    written = []
    for j, pos in enumerate(flat.tolist()):
        tk = int(np.searchsorted(cum, pos, side="right") - 1)
        idx = pos - int(cum[tk])
        if j % 4 < 3:
            pat = NAN_PATTERNS[j % 4]
        else:  # NaN with random sign and random nonzero payload
            pat = (int(rng.integers(0, 2)) << 31) | 0x7F800000 | int(rng.integers(1, 1 << 23))
        write_pattern(grads[tk], idx, pat)
        written.append((tk, idx, pat))
    replay = [t.clone() for t in grads]
    nf_set = {(tk, idx) for tk, idx, _ in written}
    while True:  # a finite, un-injected element
        tk = int(rng.integers(0, T))
        idx = int(rng.integers(0, grads[tk].numel()))
        if (tk, idx) not in nf_set:
            break
    b = int(rng.integers(0, 32))
    was = flip_bit(replay[tk], idx, b)
    return Workload("c3_gpt0.96b_grads_fp32_replay", 2, T, grads + replay, [s[0] for s in shapes],
                    seed, injections=[dict(replica=1, tensor=tk, index=idx, bit=b, was=was)],
                    nonfinite=written, meta={"n_nonfinite": k})


# ---------------------------------------------------------------------------
# c4: 100k small tensors, mixed dtypes, carved from one byte buffer per replica
# ---------------------------------------------------------------------------
def c4_layout(seed=4, n_tensors=100_000, max_numel=65536):
    """Sizes, dtypes and byte offsets of the small-tensor list.
    n = min(max_numel, floor(exp(U[0, ln(max_numel + 1))))), dtype uniform."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.0, math.log(max_numel + 1), size=n_tensors)
    numel = np.minimum(max_numel, np.floor(np.exp(u))).astype(np.int64)
    numel = np.maximum(numel, 1)
    dtypes = rng.integers(0, 3, size=n_tensors)
    offs = np.zeros(n_tensors, dtype=np.int64)
    pos = 0
    for k in range(n_tensors):
        es = ESIZE[int(dtypes[k])]
        pos = (pos + es - 1) // es * es
        offs[k] = pos
        pos += int(numel[k]) * es
    return rng, numel, dtypes, offs, pos


def c4(device, seed=4, n_tensors=100_000, max_numel=65536, R=3, n_corrupt=5):
    rng, numel, dtypes, offs, nbytes = c4_layout(seed, n_tensors, max_numel)
    g = _gen(device, seed)
    flat0 = torch.zeros(max(nbytes, 1) + 16, dtype=torch.uint8, device=device)
    # one value stream per dtype, in dtype order, then copied into the views
    streams = {}
    for d in (F32, BF16, F16):
        n_d = int(numel[dtypes == d].sum())
        streams[d] = (torch.randn(max(n_d, 1), generator=g, device=device, dtype=torch.float32)
                      * 0.02).to(TORCH_OF[d])
    used = {F32: 0, BF16: 0, F16: 0}
    for k in range(n_tensors):
        d, n, o = int(dtypes[k]), int(numel[k]), int(offs[k])
        es = ESIZE[d]
        view = flat0[o:o + n * es].view(TORCH_OF[d])
        view.copy_(streams[d][used[d]:used[d] + n])
        used[d] += n
    del streams
    flats = [flat0] + [flat0.clone() for _ in range(R - 1)]
    tensors = []
    for r in range(R):
        for k in range(n_tensors):
            d, n, o = int(dtypes[k]), int(numel[k]), int(offs[k])
            tensors.append(flats[r][o:o + n * ESIZE[d]].view(TORCH_OF[d]))
    inj = []
    hit = rng.choice(n_tensors, size=min(n_corrupt, n_tensors), replace=False)
    for k in sorted(int(x) for x in hit):
        r = int(rng.integers(0, R))
        i = int(rng.integers(0, int(numel[k])))
        b = int(rng.integers(0, 8 * ESIZE[int(dtypes[k])]))
        was = flip_bit(tensors[r * n_tensors + k], i, b)
        inj.append(dict(replica=r, tensor=k, index=i, bit=b, was=was))
    return Workload("c4_100k_small_mixed_r3", R, n_tensors, tensors,
                    [f"t{k}" for k in range(n_tensors)], seed, injections=inj, buffers=flats,
                    meta={"flat_bytes": nbytes})


# ---------------------------------------------------------------------------
# c5: Llama-70B shapes in bf16
# ---------------------------------------------------------------------------
def llama70b_shapes(d=8192, layers=80, heads=64, kv_heads=8, ffn=28672, vocab=128256):
    hd = d // heads
    kv = kv_heads * hd
    out = [("embed", (vocab, d))]
    for l in range(layers):
        p = f"l{l}."
        out += [(p + "q", (d, d)), (p + "k", (kv, d)), (p + "v", (kv, d)), (p + "o", (d, d)),
                (p + "gate", (ffn, d)), (p + "up", (ffn, d)), (p + "down", (d, ffn)),
                (p + "attn_norm", (d,)), (p + "mlp_norm", (d,))]
    out += [("norm", (d,)), ("lm_head", (vocab, d))]
    return out


def c5(device, seed=5, shapes=None):
    """Every tensor N(0, 0.02) in bf16 (norm gains included, as the setup
    states), one copy."""
    shapes = shapes or llama70b_shapes()
    g = _gen(device, seed)
    ts = [_normal_(torch.empty(s, dtype=torch.bfloat16, device=device), 0.02, g) for _, s in shapes]
    return Workload("c5_llama70b_bf16", 1, len(ts), ts, [s[0] for s in shapes], seed)


def c5_flip(w, seed=55):
    """One seeded flip in the c5 list (after the stored table was taken)."""
    rng = np.random.default_rng(seed)
    k = int(rng.integers(0, w.T))
    i = int(rng.integers(0, w.tensors[k].numel()))
    b = int(rng.integers(0, 16))
    was = flip_bit(w.tensors[k], i, b)
    inj = dict(replica=0, tensor=k, index=i, bit=b, was=was)
    w.injections.append(inj)
    return inj


def recompute_acts(device, seed=6, layers=80, tokens=32768, d=8192):
    """The checkpointed layer outputs of one Llama-70B-shaped micro-batch of
    8 x 4096 tokens: `layers` hidden-state tensors [tokens, d] in bf16,
    N(0, 1) (post-norm activations), 512 MiB each -- the input of the
    recompute audit, one single-tensor scan per layer output."""
    g = _gen(device, seed)
    acts = [_normal_(torch.empty((tokens, d), dtype=torch.bfloat16, device=device), 1.0, g)
            for _ in range(layers)]
    return Workload(f"recompute_llama70b_acts_{layers}x{tokens}x{d}_bf16", 1, layers, acts,
                    [f"layer{i}.out" for i in range(layers)], seed)


BUILDERS = {"c1": c1, "c2": c2, "c3": c3, "c4": c4, "c5": c5}
