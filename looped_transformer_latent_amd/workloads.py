"""Named synthetic workloads (shapes + seeded recipes) for tests and bench.

The shapes are Ouro-style looped models as the close reading describes them
(cc.laoqi.cc, 一:动机 item 1 and 方法 item 2: Ouro-1.4B has D = 24 shared layers run
T = 4 times, H = 16 heads, d_head = 128; the 21.3x point stores r_k + r_v = 48
scalars per head, the 4x point 96 + 160).  Trained codecs and real activations
are not available, so every tensor is drawn from the seeded generator in
``gen.py``: decoder parameters mu_t, W_up,t ~ N(0,1)/sqrt(r) (r of their own
K or V side), latents ~ N(0,1), q ~ N(0,1).  Nothing here computes attention.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import gen

F32, BF16 = 0, 1
PER_HEAD, TWO_D = 0, 1
PAGE = 16

STREAMS = dict(mu_k=101, mu_v=102, w_up_k=103, w_up_v=104, w_down_k=111, w_down_v=112,
               k_pool=201, v_pool=202, kr_pool=203, q=301, x_k=401, x_v=402, x_r=403)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    H: int
    d_head: int
    r_k: int
    r_v: int
    variant: int
    dtype: int
    batch: int
    ctx: int            # cached tokens per sequence at decode time
    shuffled: bool      # page table: seeded permutation (True) or identity
    n_new: int          # tokens appended per sequence by one encode call
    seed: int
    ortho_down: bool = False  # W_down orthonormal (QR) and W_up,t its loop-t row slice
    d_rope: int = 0           # > 0: decoupled RoPE (NoPE content + rotary branch of this width)

    @property
    def dims(self) -> dict:
        return dict(T=self.T, D=self.D, H=self.H, d_head=self.d_head, r_k=self.r_k,
                    r_v=self.r_v, variant=self.variant, dtype=self.dtype, page_size=PAGE,
                    rope_base=10000.0)

    @property
    def pages_per_seq(self) -> int:
        return (self.ctx + PAGE - 1) // PAGE

    @property
    def num_pages(self) -> int:
        return self.batch * self.pages_per_seq

    @property
    def groups(self) -> int:
        return self.H if self.variant == PER_HEAD else 1

    @property
    def esize(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def read_bytes(self) -> int:
        """Algorithmic latent bytes of one cached-token read: all heads' (c_k, c_v)
        for per-head LLA, the one shared latent for LLA-2D; plus the token's
        rotary key with decoupled RoPE."""
        return (self.groups * (self.r_k + self.r_v) + self.d_rope) * self.esize

    @property
    def q_width(self) -> int:
        return self.d_head + self.d_rope

    def pool_shape(self, kv: str) -> tuple:
        if kv == "kr":  # decoupled RoPE: one rotary key per (token, layer)
            return (self.D, self.num_pages, PAGE, self.d_rope)
        r = self.r_k if kv == "k" else self.r_v
        if self.variant == PER_HEAD:
            return (self.D, self.num_pages, self.H, PAGE, r)
        return (self.D, self.num_pages, PAGE, r)

    def page_elems(self, kv: str) -> int:
        return int(np.prod(self.pool_shape(kv)[2:]))

    def param_shapes(self) -> dict:
        T, D, H, d, rk, rv = self.T, self.D, self.H, self.d_head, self.r_k, self.r_v
        if self.variant == PER_HEAD:
            return dict(mu_k=(D, H, T, d), mu_v=(D, H, T, d), w_down_k=(D, H, T * d, rk),
                        w_down_v=(D, H, T * d, rv), w_up_k=(D, H, T, d, rk),
                        w_up_v=(D, H, T, d, rv))
        return dict(mu_k=(D, T, H, d), mu_v=(D, T, H, d), w_down_k=(D, T * H * d, rk),
                    w_down_v=(D, T * H * d, rv), w_up_k=(D, T, H, d, rk), w_up_v=(D, T, H, d, rv))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny parity case, fp32 (its codec comes from the SVD fixture in the tests)
    "tiny-fp32": Workload("tiny-fp32", 4, 1, 2, 64, 16, 32, PER_HEAD, F32, 1, 256, False, 0, 1001),
    # Ouro-1.4B-shaped, 21.3x, batch 32, 4k context
    "ouro1.4b-21x-b32": Workload("ouro1.4b-21x-b32", 4, 24, 16, 128, 16, 32, PER_HEAD, BF16,
                                 32, 4096, False, 0, 1002),
    # the high-capacity point: batch 768, 4k context, shuffled 16-token pages
    "ouro1.4b-21x-b768-paged": Workload("ouro1.4b-21x-b768-paged", 4, 24, 16, 128, 16, 32,
                                        PER_HEAD, BF16, 768, 4096, True, 1, 1003),
    # the same with an identity page table (isolates the cost of scattered pages)
    "ouro1.4b-21x-b768-contig": Workload("ouro1.4b-21x-b768-contig", 4, 24, 16, 128, 16, 32,
                                         PER_HEAD, BF16, 768, 4096, False, 1, 1003),
    # 4x compression plus encode/append of 512 tokens per sequence, 8k context
    "ouro1.4b-4x-b64-encode": Workload("ouro1.4b-4x-b64-encode", 4, 24, 16, 128, 96, 160,
                                       PER_HEAD, BF16, 64, 8192, False, 512, 1004, True),
    # decoupled RoPE (appendix J's absorbed kernel), one sequence at 262144 tokens
    "ouro1.4b-21x-ctx256k-decoupled": Workload("ouro1.4b-21x-ctx256k-decoupled", 4, 24, 16, 128, 16, 32,
                                               PER_HEAD, BF16, 1, 262144, True, 1, 1006, d_rope=64),
    # LLA-2D: heads folded into one latent per token and layer
    "lla2d-t8-h32-b128": Workload("lla2d-t8-h32-b128", 8, 4, 32, 128, 256, 256, TWO_D, BF16,
                                  128, 16384, True, 0, 1005),
}


def _gdt(w: Workload) -> str:
    return "bf16" if w.dtype == BF16 else "f32"


def codec_host(w: Workload, ortho_down: bool | None = None) -> dict:
    """Codec parameters as host storage arrays (uint16 bf16 bits or fp32).
    With orthonormal W_down, W_up,t is W_down's loop-t row slice (the SVD-style
    initialisation the close reading describes, 方法 item 3), not a separate draw."""
    ortho_down = w.ortho_down if ortho_down is None else ortho_down
    sh = w.param_shapes()
    out = {}
    for name in ("mu_k", "mu_v", "w_up_k", "w_up_v"):
        r = w.r_k if name.endswith("k") else w.r_v
        out[name] = gen.normal(w.seed, STREAMS[name], sh[name], scale=1.0 / np.sqrt(r), dtype=_gdt(w))
    for name in ("w_down_k", "w_down_v"):
        shape = sh[name]
        if ortho_down:
            g = gen.normal_f32(w.seed, STREAMS[name], int(np.prod(shape))).astype(np.float64)
            flat = g.reshape(-1, shape[-2], shape[-1])
            g = np.stack([np.linalg.qr(x)[0] for x in flat]).reshape(shape)
            g32 = g.astype(np.float32)
            out[name] = gen.f32_to_bf16_bits(g32) if w.dtype == BF16 else g32
        else:
            out[name] = gen.normal(w.seed, STREAMS[name], shape, scale=1.0 / np.sqrt(shape[-2]),
                                   dtype=_gdt(w))
    if ortho_down:
        for kv in ("k", "v"):
            out["w_up_" + kv] = np.ascontiguousarray(out["w_down_" + kv].reshape(sh["w_up_" + kv]))
    return out


def page_table_host(w: Workload) -> np.ndarray:
    if w.shuffled:
        return gen.shuffled_page_table(w.seed, w.batch, w.pages_per_seq)
    return gen.identity_page_table(w.batch, w.pages_per_seq)


def pool_pages_host(w: Workload, kv: str, layer: int, pages) -> np.ndarray:
    """Regenerate physical pages of one layer of the latent pool on the host.
    Element (layer, page, ...) of the pool has generator index equal to its flat
    offset in the [D][num_pages][...] layout."""
    pages = np.asarray(pages, dtype=np.int64)
    pe = w.page_elems(kv)
    base = (layer * w.num_pages + pages) * pe
    idx = (base[:, None] + np.arange(pe, dtype=np.int64)[None, :]).astype(np.uint64)
    v = gen.normal_f32(w.seed, STREAMS[kv + "_pool"], idx.reshape(-1)).reshape((len(pages),) + w.pool_shape(kv)[2:])
    return gen.f32_to_bf16_bits(v) if w.dtype == BF16 else v


def q_host(w: Workload, rows: int | None = None, stream: str = "q") -> np.ndarray:
    rows = w.batch if rows is None else rows
    return gen.normal(w.seed, STREAMS[stream], (rows, w.H, w.q_width), dtype=_gdt(w))


# ---------------------------------------------------------------- device side

def to_device(a: np.ndarray, device="cuda"):
    """Host storage array (uint16 bf16 bits, fp32 or int32) -> device tensor
    (torch.bfloat16 for bf16 bits)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t) -> np.ndarray:
    """Device tensor -> host storage array (bf16 -> uint16 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def device_pool(w: Workload, kv: str, device="cuda"):
    """The whole latent pool of `kv`, filled on the device by the generator."""
    import torch
    from . import lla
    dt = torch.bfloat16 if w.dtype == BF16 else torch.float32
    t = torch.empty(w.pool_shape(kv), dtype=dt, device=device)
    lla.gen_normal_(t, w.seed, STREAMS[kv + "_pool"])
    return t
