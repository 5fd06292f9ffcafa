"""Seeded synthetic workloads: shapes and input generators.

Holds none of the attention or softmax arithmetic; it only names the workloads and
draws their inputs, so both the HIP path and the oracle can be fed the same
tensors.  Recipe: Q, K, V ~ N(0, 1) as float32 from one seeded torch
generator, drawn in the order Q, K, V, then rounded to the workload's dtype.
The ragged workload adds ``k_ramp * j`` to every element of key row j (a
rising key offset pushes the running max up tile after tile).

The generator is torch's CPU generator (``torch.Generator('cpu')``), so the
same seed gives the same inputs on any machine and a host-side
re-derivation reproduces what the GPU ran on; the tensors are then copied
to the target device.  Only tensors of more than HOST_GEN_MAX_ELEMS
elements (the decode workload's K and V, 2^31 elements each) are drawn on
the target device's own generator instead.
"""

import dataclasses
import itertools

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

#: Largest tensor (elements) drawn on the host generator; larger ones are
#: drawn on the target device's generator.
HOST_GEN_MAX_ELEMS = 1 << 28


def generator_device(largest_elems, device):
    """Where inputs whose largest tensor has ``largest_elems`` elements are
    drawn: the host ("cpu") unless that tensor exceeds HOST_GEN_MAX_ELEMS."""
    if str(device) == "cpu" or largest_elems <= HOST_GEN_MAX_ELEMS:
        return "cpu"
    return device


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    dtype: str
    causal: bool
    k_ramp: float = 0.0

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def visible_pairs(self):
        """Query-key pairs with a visible key, summed over (B, H)."""
        if not self.causal:
            per_head = self.Nq * self.Nk
        else:
            off = self.Nk - self.Nq
            per_head = 0
            # rows i see min(Nk, max(0, i + off + 1)) keys
            lo = max(0, -off)                     # first row that sees a key
            full = max(lo, min(self.Nq, self.Nk - off))  # first row that sees all Nk keys
            n = full - lo
            # rows lo..full-1 see i + off + 1 keys: arithmetic series
            per_head += n * (lo + off + 1) + n * (n - 1) // 2
            per_head += (self.Nq - full) * self.Nk
        return self.B * self.H * per_head

    def flops(self):
        """Algorithmic FLOP: 2*D for Q.K^T plus 2*D for P.V per visible pair."""
        return 4 * self.D * self.visible_pairs()

    def bwd_flops(self):
        """Algorithmic FLOP of the backward: 2*D for each of the five products
        per visible pair (Q.K^T recomputed, dO.V^T, P^T dO, dS^T Q, dS K),
        2.5 times the forward's count."""
        return 10 * self.D * self.visible_pairs()

    def bytes(self):
        """Algorithmic HBM bytes: Q, K, V read once and out written once."""
        el = torch.finfo(self.torch_dtype).bits // 8
        return el * self.B * self.H * self.D * (2 * self.Nq + 2 * self.Nk)


WORKLOADS = {w.name: w for w in [
    Workload("tiny_f32", 1, 1, 128, 128, 64, "f32", False),
    Workload("small_causal_bf16", 2, 4, 1024, 1024, 64, "bf16", True),
    Workload("headline_causal_bf16", 4, 16, 4096, 4096, 128, "bf16", True),
    Workload("headline_noncausal_bf16", 4, 16, 4096, 4096, 128, "bf16", False),
    Workload("ragged_causal_f16", 3, 8, 4099, 4099, 64, "f16", True, 0.02),
    Workload("ragged_noncausal_f16", 3, 8, 4099, 4099, 64, "f16", False, 0.02),
    Workload("ragged_nk1_f16", 3, 8, 4099, 1, 64, "f16", False, 0.02),
    Workload("ragged_n1_causal_f16", 3, 8, 1, 1, 64, "f16", True, 0.02),
    Workload("ragged_b0_f16", 0, 8, 4099, 4099, 64, "f16", True, 0.02),
    Workload("long_causal_bf16", 1, 32, 16384, 16384, 128, "bf16", True),
    Workload("decode_bf16", 16, 32, 1, 32768, 128, "bf16", False),
    # A 512-token chunk of new rows over an 8192-token context (causal, the
    # chunk's rows are the context's last 512): few query tiles over many keys.
    Workload("chunked_causal_bf16", 1, 32, 512, 8192, 128, "bf16", True),
]}


def make_qkv(w, seed=0, device="cpu"):
    """Q, K, V for workload ``w``: N(0, 1) float32 from ``seed``, order Q, K, V,
    key ramp added, then rounded to the workload dtype on ``device``."""
    gen_device = generator_device(w.B * w.H * max(w.Nq, w.Nk) * w.D, device)
    g = torch.Generator(device=gen_device)
    g.manual_seed(seed)
    shape_q = (w.B, w.H, w.Nq, w.D)
    shape_k = (w.B, w.H, w.Nk, w.D)
    q = torch.randn(shape_q, generator=g, dtype=torch.float32, device=gen_device)
    k = torch.randn(shape_k, generator=g, dtype=torch.float32, device=gen_device)
    v = torch.randn(shape_k, generator=g, dtype=torch.float32, device=gen_device)
    if w.k_ramp:
        ramp = w.k_ramp * torch.arange(w.Nk, dtype=torch.float32, device=gen_device)
        k = k + ramp[:, None]
    dt = w.torch_dtype
    return (q.to(device=device, dtype=dt), k.to(device=device, dtype=dt),
            v.to(device=device, dtype=dt))


def random_qkv(B, H, Nq, Nk, D, dtype, seed=0, device="cpu", k_ramp=0.0):
    """Same recipe for an ad-hoc shape."""
    return make_qkv(Workload("adhoc", B, H, Nq, Nk, D, dtype, False, k_ramp), seed, device)


def random_dout(shape, dtype, seed=0, device="cpu"):
    """An upstream gradient dO of ``shape``: N(0, 1) float32 from its own
    generator seeded with ``seed``, rounded to ``dtype`` ("f16", "bf16")."""
    numel = 1
    for n in shape:
        numel *= int(n)
    gen_device = generator_device(numel, device)
    g = torch.Generator(device=gen_device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=gen_device)
    return x.to(device=device, dtype=DTYPES[dtype])


def make_paged(B, H, Hkv, Nq, D, page_size, seq_lens, dtype, seed=0, device="cpu",
               spare_pages=3, share_first_page=False):
    """Inputs of a paged-cache decode: (q, k_cache, v_cache, block_table, seq_lens).

    q [B, H, Nq, D] and the caches [num_pages, Hkv, page_size, D] are
    N(0, 1) FP32 from one generator seeded with ``seed`` on ``device``
    (drawn in the order q, K cache, V cache), rounded to ``dtype``.  Each sequence gets
    ceil(len / page_size) pages from a seeded permutation of all pages (plus
    ``spare_pages`` unused ones), so logical order and physical order
    differ; table entries past a sequence's pages are -1 (never read).
    ``share_first_page`` makes sequence 1 reuse sequence 0's first page
    (a shared prefix).
    """
    npp = [(int(n) + page_size - 1) // page_size for n in seq_lens]
    max_pages = max(1, max(npp) if npp else 1)
    total = sum(npp) + spare_pages
    gen_device = generator_device(max(total * Hkv * page_size * D, B * H * Nq * D), device)
    g = torch.Generator(device=gen_device)
    g.manual_seed(seed)
    dt = DTYPES[dtype]
    q = torch.randn((B, H, Nq, D), generator=g, dtype=torch.float32, device=gen_device).to(dt)
    kc = torch.randn((total, Hkv, page_size, D), generator=g, dtype=torch.float32,
                     device=gen_device).to(dt)
    vc = torch.randn((total, Hkv, page_size, D), generator=g, dtype=torch.float32,
                     device=gen_device).to(dt)
    perm = torch.randperm(total, generator=g, device=gen_device).to("cpu")
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    offs = [0]
    for n in npp:
        offs.append(offs[-1] + n)
    for b in range(B):
        table[b, :npp[b]] = perm[offs[b]:offs[b + 1]].to(torch.int32)
    if share_first_page and B > 1 and npp[0] > 0 and npp[1] > 0:
        table[1, 0] = table[0, 0]
    lens = torch.tensor([int(n) for n in seq_lens], dtype=torch.int32)
    return (q.to(device), kc.to(device), vc.to(device), table.to(device), lens.to(device))


def make_varlen(lens_q, lens_k, H, Hkv, D, dtype, seed=0, device="cpu"):
    """Packed variable-length inputs: (q [total_q, H, D], k, v [total_k, Hkv, D],
    cu_q, cu_k int32 [B + 1]); N(0, 1) FP32 from one generator seeded with
    ``seed`` on ``device``, drawn in the order q, k, v, rounded to ``dtype``."""
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    gen_device = generator_device(max(tq * H, tk * Hkv) * D, device)
    g = torch.Generator(device=gen_device)
    g.manual_seed(seed)
    dt = DTYPES[dtype]
    q = torch.randn((tq, H, D), generator=g, dtype=torch.float32, device=gen_device).to(dt)
    k = torch.randn((tk, Hkv, D), generator=g, dtype=torch.float32, device=gen_device).to(dt)
    v = torch.randn((tk, Hkv, D), generator=g, dtype=torch.float32, device=gen_device).to(dt)
    cu_q = torch.tensor([0] + list(itertools.accumulate(int(n) for n in lens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(itertools.accumulate(int(n) for n in lens_k)), dtype=torch.int32)
    return q.to(device), k.to(device), v.to(device), cu_q.to(device), cu_k.to(device)


def varlen_lengths(n_seq, lo, hi, seed=0):
    """Seeded sequence lengths, uniform in [lo, hi] (a mixed-length batch)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n_seq,), generator=g)]


def causal_pairs(nq, nk, window=0):
    """Visible (query, key) pairs of one causal head, keys aligned to the
    end of the query block, with an optional sliding window."""
    off = nk - nq
    total = 0
    for i in range(nq):
        hi = min(nk - 1, i + off)
        lo = 0 if window <= 0 else max(0, i + off - window + 1)
        total += max(0, hi - lo + 1)
    return total


@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    """A wide-row softmax input: x ~ 3 * N(0, 1) float32, rounded to dtype."""
    name: str
    M: int
    N: int
    dtype: str

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def bytes(self):
        """HBM bytes the split method moves: x read twice (partial pass and
        normalising pass), y written once.  A single-pass method would need
        two of these three."""
        el = torch.finfo(self.torch_dtype).bits // 8
        return 3 * el * self.M * self.N


SOFTMAX_WORKLOADS = {w.name: w for w in [
    # The pages' widest row (131072 columns), 1024 rows: 256 MiB of bf16.
    SoftmaxWorkload("wide_softmax_bf16", 1024, 131072, "bf16"),
]}


def make_softmax_input(w, seed=0, device="cpu"):
    """x for softmax workload ``w`` from ``seed`` (drawn as generator_device
    says, then placed on ``device``)."""
    gen_device = generator_device(w.M * w.N, device)
    g = torch.Generator(device=gen_device)
    g.manual_seed(seed)
    x = torch.randn((w.M, w.N), generator=g, dtype=torch.float32, device=gen_device) * 3.0
    return x.to(w.torch_dtype).to(device)
