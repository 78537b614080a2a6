"""Seeded generators for decode, slot-write and block-copy inputs.

Draw order per decode case (one numpy PCG64 stream seeded with the config's
seed): lengths, pool permutation, then the payload q, K pool, V pool.  Large
cases can draw the payload from a seeded torch CUDA generator instead (same
structure, different numbers); the structure (lengths, tables, which slots
are live) always comes from numpy on the host.

Pool layout (fixed by the library's interface):
    K pool [num_blocks][H_kv][block_size][head_dim]
    V pool [num_blocks][H_kv][head_dim][block_size]
bf16 data is carried as uint16 bit patterns on the numpy side and as
torch.bfloat16 on the torch side.

8-bit pools ("fp8") are a uint8 pair: K [num_blocks][H_kv][B*d + 4*B] (per
(block, kv head) the E4M3 K codes token-major [B][d], then bf16 scales: per
group of 4 slots, 4 K scales then 4 V scales) and V [num_blocks][H_kv][B*d]
(V codes dim-major [d][B]).  Their payload is drawn directly as codes and
scales, with no quantisation arithmetic: magnitude codes uniform over the 127
finite ones (0x00..0x7E), a random sign bit, and scales 2^-7 * U[1, 2)
rounded to bf16, so stored values reach 448 * 2^-6 = 7, the range of the
bf16 cases' normal draws.  Queries and new tokens stay bf16.

Every slot that no sequence's context covers is filled with poison
(K = 64.0, V = 1024.0, both exact in bf16), so reading a slot that should be
masked shows up far above any tolerance.
"""
from dataclasses import dataclass
import math
from typing import Optional

import numpy as np
import torch

from .configs import Config

POISON_K = 64.0
POISON_V = 1024.0


# --- bf16 carriers ---------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """torch tensor (any device) -> numpy array in oracle storage form."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.int32, torch.int64, torch.uint8):
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def from_numpy_storage(a: np.ndarray, dtype: str, device="cpu") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def _torch_dtype(dtype: str):
    """Element type of queries (and of pools other than 8-bit ones)."""
    return torch.float32 if dtype == "f32" else torch.bfloat16


# --- 8-bit regions -----------------------------------------------------------
FP8_POISON_CODE = 0x68          # E4M3 code of 64.0
FP8_POISON_K_SCALE = 1.0        # poison K = 64.0
FP8_POISON_V_SCALE = 16.0       # poison V = 1024.0


def fp8_region_bytes(B: int, d: int):
    """(K region, V region) bytes per (block, kv head) of an 8-bit pool."""
    return B * d + 4 * B, B * d


def fp8_k_codes(k_pool, B: int, d: int):
    """View of the K codes, [nb][H][B*d] (token-major inside)."""
    return k_pool[..., :B * d]


def fp8_scales(k_pool, B: int, d: int):
    """View of the bf16 scale bits in the K buffer, [nb][H][B/4][2][4]:
    per group of 4 slots, side 0 holds the K scales and side 1 the V scales."""
    nb, H = k_pool.shape[0], k_pool.shape[1]
    if isinstance(k_pool, torch.Tensor):
        return k_pool[..., B * d:].view(torch.int16).view(nb, H, B // 4, 2, 4)
    return k_pool[..., B * d:].view(np.uint16).reshape(nb, H, B // 4, 2, 4)


def fp8_codes_np(rng, n):
    mag = rng.integers(0, 0x7F, size=n, dtype=np.uint8)
    sign = (rng.integers(0, 2, size=n, dtype=np.uint8) << 7).astype(np.uint8)
    return mag | sign


def fp8_pools_np(rng, nb, Hkv, B, d):
    """Random 8-bit (K, V) pools: finite codes, bf16 scales 2^-7 * U[1, 2)."""
    rk, rv = fp8_region_bytes(B, d)
    k = np.empty((nb, Hkv, rk), np.uint8)
    v = fp8_codes_np(rng, nb * Hkv * rv).reshape(nb, Hkv, rv)
    fp8_k_codes(k, B, d)[...] = fp8_codes_np(rng, nb * Hkv * B * d).reshape(nb, Hkv, B * d)
    sc = (rng.random((nb, Hkv, B // 4, 2, 4), dtype=np.float32) + 1.0) * np.float32(2.0 ** -7)
    fp8_scales(k, B, d)[...] = f32_to_bf16_bits(sc)
    return k, v


def fp8_pools_torch(g, nb, Hkv, B, d, device):
    rk, rv = fp8_region_bytes(B, d)
    k = torch.empty((nb, Hkv, rk), dtype=torch.uint8, device=device)
    v = torch.empty((nb, Hkv, rv), dtype=torch.uint8, device=device)
    kc, ks = fp8_k_codes(k, B, d), fp8_scales(k, B, d)
    chunk = max(1, (1 << 26) // (Hkv * B * d))

    def codes(n0):
        mag = torch.randint(0, 0x7F, (n0, Hkv, B * d), generator=g, device=device,
                            dtype=torch.uint8)
        sign = torch.randint(0, 2, (n0, Hkv, B * d), generator=g, device=device,
                             dtype=torch.uint8) << 7
        return mag | sign

    for b0 in range(0, nb, chunk):
        b1 = min(nb, b0 + chunk)
        kc[b0:b1] = codes(b1 - b0)
        v[b0:b1] = codes(b1 - b0)
        sc = (torch.rand((b1 - b0, Hkv, B // 4, 2, 4), generator=g, device=device) + 1.0) \
            * 2.0 ** -7
        ks[b0:b1] = sc.to(torch.bfloat16).view(torch.int16)
    return k, v


def fp8_poison(k_pool, v_pool, dead, B, d):
    """Poison the dead token slots (dead: bool [nb][B]) of an 8-bit pool pair:
    K = 64 * 1.0, V = 64 * 16.0."""
    nb, H = k_pool.shape[0], k_pool.shape[1]
    kc = fp8_k_codes(k_pool, B, d)
    sc = fp8_scales(k_pool, B, d)
    if isinstance(k_pool, torch.Tensor):
        kc.view(nb, H, B, d).masked_fill_(dead[:, None, :, None], FP8_POISON_CODE)
        v_pool.view(nb, H, d, B).masked_fill_(dead[:, None, None, :], FP8_POISON_CODE)
        dg = dead.view(nb, B // 4, 4)[:, None, :, :]
        one = torch.tensor(FP8_POISON_K_SCALE, dtype=torch.bfloat16).view(torch.int16).item()
        sixteen = torch.tensor(FP8_POISON_V_SCALE, dtype=torch.bfloat16).view(torch.int16).item()
        sc[:, :, :, 0, :].masked_fill_(dg, one)
        sc[:, :, :, 1, :].masked_fill_(dg, sixteen)
        return
    bi, ri = dead.nonzero()
    kc.reshape(nb, H, B, d)[bi, :, ri, :] = FP8_POISON_CODE
    v_pool.reshape(nb, H, d, B)[bi, :, :, ri] = FP8_POISON_CODE
    sc[bi, :, ri // 4, 0, ri % 4] = f32_to_bf16_bits(np.float32(FP8_POISON_K_SCALE))
    sc[bi, :, ri // 4, 1, ri % 4] = f32_to_bf16_bits(np.float32(FP8_POISON_V_SCALE))


# --- lengths and pools -----------------------------------------------------
def draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Context lengths (including the token being decoded), int32 [S].

    uniform (lo, hi): integers, both ends inclusive.
    lognormal (median, sigma, lo, hi): rint(exp(N(ln median, sigma))) clipped.
    fixed (L,): every sequence has L tokens.
    shared (shared, lo, hi): prompts x samples sequences, each shared + U[lo, hi].
    """
    kind = cfg.lengths[0]
    S = cfg.num_seqs
    if kind == "uniform":
        _, lo, hi = cfg.lengths
        L = rng.integers(lo, hi, size=S, endpoint=True)
    elif kind == "lognormal":
        _, median, sigma, lo, hi = cfg.lengths
        L = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=S))), lo, hi)
    elif kind == "fixed":
        L = np.full(S, cfg.lengths[1])
    elif kind == "shared":
        _, shared, lo, hi = cfg.lengths
        L = shared + rng.integers(lo, hi, size=S, endpoint=True)
    else:
        raise ValueError(kind)
    return L.astype(np.int32)


def _blocks(L, B):
    return (np.asarray(L, dtype=np.int64) + B - 1) // B


def unique_blocks(cfg: Config, lens: np.ndarray) -> int:
    B = cfg.block_size
    if cfg.lengths[0] == "shared":
        shared = cfg.lengths[1]
        n_full = shared // B
        return int(cfg.prompts * n_full + (_blocks(lens, B) - n_full).sum())
    return int(_blocks(lens, B).sum())


def pool_size(cfg: Config, lens: np.ndarray) -> int:
    if cfg.pool[0] == "fixed":
        return int(cfg.pool[1])
    frac = cfg.pool[1]
    return int(math.ceil((1.0 + frac) * unique_blocks(cfg, lens)))


# --- decode case -----------------------------------------------------------
@dataclass
class DecodeCase:
    cfg: Config
    dtype: str
    k_pool: torch.Tensor        # [nb][Hkv][B][d]
    v_pool: torch.Tensor        # [nb][Hkv][d][B]
    q: torch.Tensor             # [S][Hq][d]
    block_tables: torch.Tensor  # int32 [S][maxB]
    context_lens: torch.Tensor  # int32 [S]
    lens: np.ndarray            # host copy of context_lens
    tables: np.ndarray          # host copy of block_tables
    live: np.ndarray            # bool [nb][B]: slot holds a context token
    scale: float

    @property
    def num_blocks(self):
        return self.k_pool.shape[0]

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode reads: sum_s L_s * 2 * H_kv * (bytes
        per token row: d * e, or d codes + one bf16 scale for 8-bit pools)."""
        c = self.cfg
        row = c.head_dim + 2 if self.dtype == "fp8" else \
            c.head_dim * (2 if self.dtype == "bf16" else 4)
        return int(self.lens.astype(np.int64).sum()) * 2 * c.num_kv_heads * row

    def oracle_inputs(self):
        """numpy views for the oracle (uint16 for bf16)."""
        return (to_numpy_storage(self.k_pool), to_numpy_storage(self.v_pool),
                to_numpy_storage(self.q), self.tables.astype(np.int32),
                self.lens.astype(np.int32))


def build_tables(cfg: Config, lens: np.ndarray, perm: np.ndarray):
    """Block tables drawn in order from a shuffled pool.

    Ordinary configs: sequence s takes the next ceil(L_s/B) blocks of perm.
    Prefix-sharing configs: each prompt's full shared blocks are taken once
    and appear in every sample's table; a partly filled shared tail gets one
    block per sample (the state after copy-on-write); private blocks follow.
    Padding entries point at an unused block when one exists.
    Returns (tables int32 [S][width], used block count).
    """
    B, S, W = cfg.block_size, cfg.num_seqs, cfg.table_width
    tables = np.zeros((S, W), dtype=np.int32)
    nblk = _blocks(lens, B)
    if int(nblk.max()) > W:
        raise ValueError("table width too small for the drawn lengths")
    pos = 0
    if cfg.lengths[0] == "shared":
        n_full = cfg.lengths[1] // B
        for p in range(cfg.prompts):
            shared = perm[pos:pos + n_full]
            pos += n_full
            for i in range(cfg.samples):
                s = p * cfg.samples + i
                own = int(nblk[s]) - n_full
                tables[s, :n_full] = shared
                tables[s, n_full:n_full + own] = perm[pos:pos + own]
                pos += own
    else:
        for s in range(S):
            n = int(nblk[s])
            tables[s, :n] = perm[pos:pos + n]
            pos += n
    used = pos
    pad = int(perm[used]) if used < len(perm) else None
    for s in range(S):
        n = int(nblk[s])
        tables[s, n:] = pad if pad is not None else tables[s, 0]
    if cfg.key == "tiny_f32":
        # the tiny config's tables are consecutive chunks of one permutation
        # of the whole pool; entries past a sequence's blocks are its padding
        tables = perm[: S * W].reshape(S, W).astype(np.int32)
        used = S * W
    return tables, used


def live_slots(cfg: Config, lens: np.ndarray, tables: np.ndarray, num_blocks: int):
    B = cfg.block_size
    live = np.zeros((num_blocks, B), dtype=bool)
    for s in range(len(lens)):
        L = int(lens[s])
        n = (L + B - 1) // B
        if n > 1:
            live[tables[s, : n - 1]] = True
        tail = L - (n - 1) * B
        live[tables[s, n - 1], :tail] = True
    return live


def _structure(cfg: Config, rng: np.random.Generator):
    lens = draw_lengths(cfg, rng)
    nb = pool_size(cfg, lens)
    perm = rng.permutation(nb).astype(np.int32)
    tables, _ = build_tables(cfg, lens, perm)
    live = live_slots(cfg, lens, tables, nb)
    return lens, nb, tables, live


def decode_structure(cfg: Config, seed: Optional[int] = None):
    """(lengths, pool size, block tables, live-slot mask) of a decode case,
    without the payload; identical to what ``decode_case`` builds."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    return _structure(cfg, rng)


def decode_case(cfg: Config, payload: str = "numpy", device="cpu",
                seed: Optional[int] = None) -> DecodeCase:
    """Build one decode batch for ``cfg``.

    payload="numpy": q/K/V drawn with numpy on the host (small cases).
    payload="torch": q/K/V drawn with a seeded torch generator on ``device``
    (large cases; the host never holds the pools).
    """
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    B, Hkv, d = cfg.block_size, cfg.num_kv_heads, cfg.head_dim
    lens, nb, tables, live = _structure(cfg, rng)
    tdt = _torch_dtype(cfg.dtype)
    q_shape = (cfg.num_seqs, cfg.num_q_heads, d)
    k_shape = (nb, Hkv, B, d)
    v_shape = (nb, Hkv, d, B)
    if cfg.dtype == "fp8" and payload == "numpy":
        q = torch.from_numpy(rng.standard_normal(q_shape, dtype=np.float32)).to(tdt)
        k_np, v_np = fp8_pools_np(rng, nb, Hkv, B, d)
        fp8_poison(k_np, v_np, ~live, B, d)
        q = q.to(device)
        k = torch.from_numpy(k_np).to(device)
        v = torch.from_numpy(v_np).to(device)
    elif cfg.dtype == "fp8" and payload == "torch":
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        q = torch.randn(q_shape, generator=g, device=device, dtype=torch.float32).to(tdt)
        k, v = fp8_pools_torch(g, nb, Hkv, B, d, device)
        dead = torch.from_numpy(~live).to(device)
        if bool(dead.any()):
            fp8_poison(k, v, dead, B, d)
    elif payload == "numpy":
        q32 = rng.standard_normal(q_shape, dtype=np.float32)
        k32 = rng.standard_normal(k_shape, dtype=np.float32)
        v32 = rng.standard_normal(v_shape, dtype=np.float32)
        dead = ~live
        k32[dead.nonzero()[0], :, dead.nonzero()[1], :] = POISON_K
        v32.transpose(0, 3, 1, 2)[dead] = POISON_V
        q = torch.from_numpy(q32).to(tdt).to(device)
        k = torch.from_numpy(k32).to(tdt).to(device)
        v = torch.from_numpy(v32).to(tdt).to(device)
    elif payload == "torch":
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        q = torch.randn(q_shape, generator=g, device=device, dtype=torch.float32).to(tdt)
        k = torch.empty(k_shape, device=device, dtype=tdt)
        v = torch.empty(v_shape, device=device, dtype=tdt)
        chunk = max(1, (1 << 26) // (Hkv * B * d))
        for b0 in range(0, nb, chunk):
            b1 = min(nb, b0 + chunk)
            k[b0:b1] = torch.randn((b1 - b0,) + k_shape[1:], generator=g, device=device,
                                   dtype=torch.float32).to(tdt)
            v[b0:b1] = torch.randn((b1 - b0,) + v_shape[1:], generator=g, device=device,
                                   dtype=torch.float32).to(tdt)
        dead = torch.from_numpy(~live).to(device)                # [nb][B]
        if bool(dead.any()):
            k.masked_fill_(dead[:, None, :, None], POISON_K)
            v.masked_fill_(dead[:, None, None, :], POISON_V)
    else:
        raise ValueError(payload)
    return DecodeCase(
        cfg=cfg, dtype=cfg.dtype, k_pool=k, v_pool=v, q=q,
        block_tables=torch.from_numpy(tables).to(device),
        context_lens=torch.from_numpy(lens).to(device),
        lens=lens, tables=tables, live=live, scale=cfg.scale)


# --- slot write case -------------------------------------------------------
@dataclass
class KVWriteCase:
    dtype: str
    k_pool: np.ndarray
    v_pool: np.ndarray
    k_new: np.ndarray       # [T][Hkv][d]
    v_new: np.ndarray
    slot_mapping: np.ndarray  # int64 [T]; -1 = skip


def _payload_np(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def kv_write_case(num_blocks, num_kv_heads, head_dim, block_size, T, dtype="bf16",
                  skip_fraction=0.0, seed=0) -> KVWriteCase:
    """Random pools, T new tokens, and T distinct random slots of which about
    ``skip_fraction`` are replaced by -1."""
    rng = np.random.default_rng(seed)
    nb, Hkv, d, B = num_blocks, num_kv_heads, head_dim, block_size
    if T > nb * B:
        raise ValueError("more tokens than slots")
    slots = rng.choice(nb * B, size=T, replace=False).astype(np.int64)
    if skip_fraction > 0:
        slots[rng.random(T) < skip_fraction] = -1
    if dtype == "fp8":  # 8-bit pools take bf16 tokens
        k_pool, v_pool = fp8_pools_np(rng, nb, Hkv, B, d)
        k_new = _payload_np(rng, (T, Hkv, d), "bf16")
        v_new = _payload_np(rng, (T, Hkv, d), "bf16")
        return KVWriteCase(dtype, k_pool, v_pool, k_new, v_new, slots)
    k_pool = _payload_np(rng, (nb, Hkv, B, d), dtype)
    v_pool = _payload_np(rng, (nb, Hkv, d, B), dtype)
    k_new = _payload_np(rng, (T, Hkv, d), dtype)
    v_new = _payload_np(rng, (T, Hkv, d), dtype)
    return KVWriteCase(dtype, k_pool, v_pool, k_new, v_new, slots)


# --- block copy case -------------------------------------------------------
@dataclass
class BlockCopyCase:
    dtype: str
    k_pool: np.ndarray
    v_pool: np.ndarray
    pairs: np.ndarray  # int32 [P][2] (src, dst)


def block_copy_case(num_blocks, num_kv_heads, head_dim, block_size, P, dtype="bf16",
                    seed=0) -> BlockCopyCase:
    """Random pools and P (src, dst) pairs: destinations distinct, no
    destination is also a source; a source may be copied several times (as
    when several forks copy one shared tail)."""
    rng = np.random.default_rng(seed)
    nb, Hkv, d, B = num_blocks, num_kv_heads, head_dim, block_size
    if P >= nb:
        raise ValueError("need more blocks than pairs")
    perm = rng.permutation(nb).astype(np.int32)
    dst = perm[:P]
    src_pool = perm[P:]
    src = src_pool[rng.integers(0, len(src_pool), size=P)]
    pairs = np.stack([src, dst], axis=1).astype(np.int32)
    if dtype == "fp8":
        return BlockCopyCase(dtype, *fp8_pools_np(rng, nb, Hkv, B, d), pairs)
    k_pool = _payload_np(rng, (nb, Hkv, B, d), dtype)
    v_pool = _payload_np(rng, (nb, Hkv, d, B), dtype)
    return BlockCopyCase(dtype, k_pool, v_pool, pairs)
