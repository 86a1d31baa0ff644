"""Shared helpers of the GPU parity tests: device caches, host copies for
the oracle, the attention tolerance check. Not a test module."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import fp8_e4m3_paged_kv_amd as fk

SENTINEL = 0xA5
SCALE_SENTINEL = -7.0

# Attention parity bar (fp32 output against the oracle on the same
# dequantized cache).
MAX_ABS = 2e-3
REL_L2 = 1e-3


def log(msg):
    print(msg, flush=True)


class DevCache:
    """uint8 code buffers [S, H, D] and fp32 scale planes on the device.

    pool "slot": codes stored [S, H, D]; "head": stored [H, S, D] and passed
    as the permuted [S, H, D] view (a KV head's rows of a block contiguous).

    scale_layout "head_major": planes stored [H, S] and passed as the
    transposed [S, H] view (one head's scales contiguous per slot);
    "interleaved": one [H, S, 2] array holding each row's K and V scales
    side by side, passed as two [S, H] views with slot stride 2;
    "slot_major": planes stored [S, H]."""

    def __init__(self, num_slots, H, D, device="cuda",
                 scale_layout="head_major", sentinel=True, pool="slot"):
        self.S, self.H, self.D = num_slots, H, D
        self.layout = scale_layout
        fill = SENTINEL if sentinel else 0
        if pool == "head":
            self.k_cache = torch.full((H, num_slots, D), fill, dtype=torch.uint8,
                                      device=device).permute(1, 0, 2)
            self.v_cache = torch.full((H, num_slots, D), fill, dtype=torch.uint8,
                                      device=device).permute(1, 0, 2)
        else:
            self.k_cache = torch.full((num_slots, H, D), fill, dtype=torch.uint8,
                                      device=device)
            self.v_cache = torch.full_like(self.k_cache, fill)
        sfill = SCALE_SENTINEL if sentinel else 0.0
        if scale_layout == "head_major":
            self.k_plane = torch.full((H, num_slots), sfill, device=device)
            self.v_plane = torch.full_like(self.k_plane, sfill)
            self.k_scale = self.k_plane.t()
            self.v_scale = self.v_plane.t()
        elif scale_layout == "interleaved":
            self.kv_planes = torch.full((H, num_slots, 2), sfill, device=device)
            self.k_plane = self.kv_planes[:, :, 0]
            self.v_plane = self.kv_planes[:, :, 1]
            self.k_scale = self.k_plane.t()
            self.v_scale = self.v_plane.t()
        else:
            self.k_plane = torch.full((num_slots, H), sfill, device=device)
            self.v_plane = torch.full_like(self.k_plane, sfill)
            self.k_scale = self.k_plane
            self.v_scale = self.v_plane

    def host(self):
        """numpy copies with the same element strides as the device views
        (codes always as contiguous [S, H, D])."""
        kc = self.k_cache.contiguous().cpu().numpy()
        vc = self.v_cache.contiguous().cpu().numpy()
        kp = self.k_plane.cpu().numpy()
        vp = self.v_plane.cpu().numpy()
        if self.layout != "slot_major":
            return kc, vc, kp.T, vp.T
        return kc, vc, kp, vp

    def scatter(self, k, v, slots, chunk=1 << 16):
        for i in range(0, k.shape[0], chunk):
            fk.kv_quant_scatter(k[i:i + chunk], v[i:i + chunk],
                                slots[i:i + chunk], self.k_cache,
                                self.v_cache, self.k_scale, self.v_scale)


def host_empty_like(dc: DevCache):
    kc = np.full((dc.S, dc.H, dc.D), SENTINEL, np.uint8)
    vc = np.full_like(kc, SENTINEL)
    if dc.layout != "slot_major":
        kp = np.full((dc.H, dc.S), SCALE_SENTINEL, np.float32)
        vp = np.full_like(kp, SCALE_SENTINEL)
        return kc, vc, kp.T, vp.T
    kp = np.full((dc.S, dc.H), SCALE_SENTINEL, np.float32)
    vp = np.full_like(kp, SCALE_SENTINEL)
    return kc, vc, kp, vp


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> host numpy uint16 view, strides kept."""
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16)


def cache_case(case, device="cuda", scale_layout="head_major", pool="slot"):
    """Build the device cache of a DecodeCase with the GPU quantizer."""
    L = case.layout
    dc = DevCache(L.num_slots, case.num_kv_heads, case.head_dim, device,
                  scale_layout, sentinel=False, pool=pool)
    k = case.k.to(device)
    v = case.v.to(device)
    dc.scatter(k, v, L.token_slots.to(device))
    return dc


def compact_host_cache(case, dc: DevCache, requests):
    """Host copy of just the blocks the given requests use, with the page
    tables remapped onto the compact copy. Returns (cache tuple,
    block_tables, context_lens) for those requests, in the given order."""
    L = case.layout
    bs = L.block_size
    blocks, tables = [], []
    for b in requests:
        nb = (int(L.context_lens[b]) + bs - 1) // bs
        blocks.append(L.block_tables[b, :nb].long())
    uniq = torch.unique(torch.cat(blocks)) if blocks else torch.zeros(0).long()
    remap = {int(x): i for i, x in enumerate(uniq.tolist())}
    maxb = max((len(x) for x in blocks), default=1)
    bt = np.zeros((len(requests), max(maxb, 1)), np.int32)
    for i, blk in enumerate(blocks):
        bt[i, :len(blk)] = [remap[int(x)] for x in blk.tolist()]
    dev_idx = uniq.to(dc.k_cache.device)
    NB = dc.S // bs
    kc = dc.k_cache.view(NB, bs, dc.H, dc.D)[dev_idx].reshape(-1, dc.H, dc.D).cpu().numpy()
    vc = dc.v_cache.view(NB, bs, dc.H, dc.D)[dev_idx].reshape(-1, dc.H, dc.D).cpu().numpy()
    if dc.layout != "slot_major":
        kp = dc.k_plane.view(dc.H, NB, bs)[:, dev_idx].reshape(dc.H, -1).cpu().numpy()
        vp = dc.v_plane.view(dc.H, NB, bs)[:, dev_idx].reshape(dc.H, -1).cpu().numpy()
        ks, vs = kp.T, vp.T
    else:
        ks = dc.k_plane.view(NB, bs, dc.H)[dev_idx].reshape(-1, dc.H).cpu().numpy()
        vs = dc.v_plane.view(NB, bs, dc.H)[dev_idx].reshape(-1, dc.H).cpu().numpy()
    cl = L.context_lens[list(requests)].numpy().astype(np.int32)
    return (kc, vc, ks, vs), bt, cl


def run_decode(case, dc: DevCache, *, out_dtype=torch.float32, ranges=0,
               max_context=None, context_lens=None, q=None, workspace=None):
    L = case.layout
    dev = dc.k_cache.device
    q = (case.q if q is None else q).to(dev)
    cl = (L.context_lens if context_lens is None else context_lens).to(dev)
    if max_context is None:
        max_context = int(L.context_lens.max()) if len(L.context_lens) else 0
    return fk.paged_decode_attn_fp8(
        q, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
        L.block_tables.to(dev), cl, num_kv_heads=case.num_kv_heads,
        block_size=L.block_size, softmax_scale=case.softmax_scale,
        max_context=max_context, num_ranges=ranges,
        out_dtype=out_dtype, workspace=workspace)


def oracle_decode(case, host_cache, rows=None, block_tables=None,
                  context_lens=None, q=None):
    kc, vc, ks, vs = host_cache
    L = case.layout
    bt = L.block_tables.numpy() if block_tables is None else block_tables
    cl = L.context_lens.numpy() if context_lens is None else context_lens
    qb = bf16_bits(case.q if q is None else q)
    return oracle.paged_decode_attn(qb, kc, vc, ks, vs, bt, cl,
                                    case.num_kv_heads, L.block_size,
                                    case.softmax_scale, rows=rows)


def attn_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs = float(np.abs(got - ref).max()) if got.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else max_abs
    return max_abs, rel


def assert_attn_close(got, ref, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel = attn_errors(got, ref)
    log(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= MAX_ABS and rel <= REL_L2, (what, max_abs, rel)


def assert_attn_close_scaled(got, ref, what=""):
    """The attention bar for outputs far from unit magnitude (value rows
    scaled by 100 or by 1e-33): max-abs is taken on the outputs divided by
    the case's largest |reference| value, i.e. 2e-3 in the output's own
    units; rel-L2 does not change under scaling. Rows whose reference stays
    within [-1, 1] must also meet the absolute max-abs bar."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.abs(ref).max())
    assert scale > 0, what
    assert_attn_close(got / scale, ref / scale, f"{what} (scaled by {scale:.3g})")
    rows_ref = ref.reshape(-1, ref.shape[-1])
    rows_got = got.reshape(-1, got.shape[-1])
    small = np.abs(rows_ref).max(axis=1) <= 1.0
    if small.any():
        err = float(np.abs(rows_got[small] - rows_ref[small]).max())
        log(f"  {what}: {int(small.sum())} rows with |ref| <= 1: max_abs={err:.3e}")
        assert err <= MAX_ABS, (what, "unit rows", err)


def oracle_decode_requests(case, dc: DevCache, requests, row_groups=1,
                           threads=16):
    """The oracle on every row of the given requests, on host copies of just
    the blocks each request uses; one task per (request, group of rows) on
    up to `threads` host cores (ctypes releases the GIL). Returns
    {request: [R, Hq, D] float64}."""
    from concurrent.futures import ThreadPoolExecutor
    R, Hq = case.q.shape[1], case.q.shape[2]
    nrows = R * Hq
    tasks = []
    hosts = {}
    for b in requests:
        hosts[b] = compact_host_cache(case, dc, [b])
        per = -(-nrows // row_groups)
        for lo in range(0, nrows, per):
            tasks.append((b, list(range(lo, min(nrows, lo + per)))))

    def run(task):
        b, rows = task
        host, bt, cl = hosts[b]
        return oracle_decode(case, host, rows=rows, block_tables=bt,
                             context_lens=cl, q=case.q[b:b + 1])

    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(tasks)))) as ex:
        parts = list(ex.map(run, tasks))
    out = {b: np.empty((nrows, case.q.shape[3])) for b in requests}
    for (b, rows), part in zip(tasks, parts):
        out[b][rows] = part
    return {b: v.reshape(R, Hq, -1) for b, v in out.items()}


def bf16_rne(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 to bf16, nearest-even (torch's cast does RNE)."""
    return x.to(torch.bfloat16)
