"""Helpers for the GPU tests: upload a workload, call tv_verify_attn through the
C ABI, read results back, and compare against the fp64 oracle."""
from __future__ import annotations

import numpy as np

import tv_workload as W

# Parity bar for the attention output against the fp64 oracle on bf16-rounded
# inputs: max |diff| <= 8e-3 and sum|diff| / sum|ref| <= 2e-3.  A bf16 output is
# also allowed its own rounding, half a bf16 ulp of the reference.
MAX_ABS = 8e-3
MEAN_REL = 2e-3


def p_rounding_bound(w: W.Workload, precise: bool):
    """Per value dim, the most the kernels' deliberate roundings can move an
    output, as u * max_j |v_jd| over the pool rows any request references.
    Probabilities rounded to bf16 move it by sum_j |p~_j - p_j| |v_jd| / sum_j p_j
    <= 2^-8 max_j |v_jd| (8 significant bits), or 2^-16 as a hi + lo pair (precise
    mode).  Without precise mode the partial outputs of a split are also stored as
    fp16 (11 significant bits) under an exact power-of-two scale: each is a convex
    combination of value rows, so that adds at most 2^-11 max_j |v_jd| (fp32
    partials in precise mode add nothing at this scale)."""
    slots = referenced_slots(w)
    v = W.bf16_to_f32(w.kv[slots][:, :512]) if slots.size else np.zeros((1, 512), np.float32)
    u = 2.0 ** -16 if precise else 2.0 ** -8 + 2.0 ** -11
    return u * np.abs(v).max(axis=0).astype(np.float64)


def referenced_slots(w: W.Workload) -> np.ndarray:
    """The pool rows the requests read: every kv_indices entry, or in the
    contiguous-prefix form each prefix as the run from its first slot (its
    other prefix entries are placeholders) followed by the draft slots."""
    if not w.contiguous_prefix:
        return np.unique(w.kv_indices)
    out = []
    for b in range(w.batch):
        k0 = int(w.kv_indptr[b])
        L, n = int(w.kv_lens[b]), int(w.q_lens[b])
        P = L - n
        if P > 0:
            out.append(int(w.kv_indices[k0]) + np.arange(P, dtype=np.int64))
        out.append(w.kv_indices[k0 + P:k0 + L].astype(np.int64))
    return np.unique(np.concatenate(out)) if out else np.zeros(0, np.int64)


def torch_mod():
    import torch
    return torch


def upload(w: W.Workload):
    torch = torch_mod()
    dev = "cuda"
    t = {
        "q": torch.from_numpy(w.q.view(np.int16)).to(dev),
        "kv": torch.from_numpy(w.kv.view(np.int16)).to(dev),
        "kv_indices": torch.from_numpy(np.ascontiguousarray(w.kv_indices, np.int32)).to(dev),
        "kv_indptr": torch.from_numpy(np.ascontiguousarray(w.kv_indptr, np.int32)).to(dev),
        "qo_indptr": torch.from_numpy(np.ascontiguousarray(w.qo_indptr, np.int32)).to(dev),
        "mask": torch.from_numpy(np.ascontiguousarray(w.mask, np.uint8)).to(dev),
        "mask_indptr": torch.from_numpy(np.ascontiguousarray(w.mask_indptr, np.int32)).to(dev),
    }
    if t["kv_indices"].numel() == 0:
        t["kv_indices"] = torch.zeros(1, dtype=torch.int32, device=dev)
    if t["mask"].numel() == 0:
        t["mask"] = torch.zeros(1, dtype=torch.uint8, device=dev)
    return t


def problem_for(w: W.Workload, num_splits: int = 0, out_f32: bool = False, max_q_len=None,
                max_kv_len=None, flags: int = 0):
    import tree_verify_mla_paged_amd as tv
    return tv.make_problem(
        batch=w.batch, num_heads=w.num_heads, total_q=w.total_q,
        max_q_len=w.max_q_len if max_q_len is None else max_q_len,
        max_kv_len=w.max_kv_len if max_kv_len is None else max_kv_len,
        num_slots=w.num_slots, total_kv=int(w.kv_indices.size), total_mask=int(w.mask.size),
        num_splits=num_splits, out_dtype=tv.OUT_F32 if out_f32 else tv.OUT_BF16,
        flags=flags | (tv.FLAG_PREFIX_VISIBLE if w.prefix_visible else 0) |
        (tv.FLAG_CONTIGUOUS_PREFIX if w.contiguous_prefix else 0))


class GpuCall:
    """Device buffers for one problem; call() runs tv_verify_attn on them."""

    def __init__(self, w: W.Workload, num_splits: int = 0, out_f32: bool = False, tensors=None,
                 **kw):  # kw: max_q_len, max_kv_len, flags
        import tree_verify_mla_paged_amd as tv
        torch = torch_mod()
        self.tv = tv
        self.w = w
        self.t = tensors if tensors is not None else upload(w)
        self.p = problem_for(w, num_splits, out_f32, **kw)
        self.plan = tv.plan(self.p)
        N, H = w.total_q, w.num_heads
        self.out = torch.full((N, H, 512), float("nan"),
                              dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
        self.lse = torch.full((N, H), float("nan"), dtype=torch.float32, device="cuda")
        nb = tv.workspace_bytes(self.p)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
        self.ws.fill_(0xA5)  # contents on entry must not matter
        self.out_f32 = out_f32

    def call(self, stream=None):
        t = self.t
        self.tv.verify_attn(self.p, t["q"], t["kv"], t["kv_indices"], t["kv_indptr"],
                            t["qo_indptr"], t["mask"], t["mask_indptr"], float(self.w.sm_scale),
                            self.out, self.lse, self.ws, self.ws.numel(), stream=stream)

    def result(self):
        torch = torch_mod()
        torch.cuda.synchronize()
        if self.out_f32:
            o = self.out.cpu().numpy().astype(np.float64)
        else:
            o = W.bf16_to_f32(self.out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(
                np.float64)
        return o, self.lse.cpu().numpy().astype(np.float64)

    def out_bits(self):
        torch = torch_mod()
        torch.cuda.synchronize()
        if self.out_f32:
            return self.out.view(torch.int32).cpu().numpy()
        return self.out.view(torch.int16).cpu().numpy()


def run(w: W.Workload, num_splits: int = 0, out_f32: bool = False, **kw):
    g = GpuCall(w, num_splits, out_f32, **kw)
    g.call()
    return g.result()


def bf16_half_ulp(x):
    """Half a bf16 spacing at |x| (the output rounding bound)."""
    ax = np.maximum(np.abs(x), 1e-30)
    e = np.floor(np.log2(ax))
    return 0.5 * np.exp2(e - 7)


def compare(o, l, ro, rl, bf16_out: bool, lse_tol: float = 2e-4, label: str = "",
            extra_abs=0.0, mean_rel_max: float = MEAN_REL):
    """Assert the parity bar (plus `extra_abs`, a derived per-element allowance,
    broadcast against the output); returns the statistics."""
    o = np.asarray(o, np.float64).reshape(ro.shape)
    l = np.asarray(l, np.float64).reshape(rl.shape)
    fin = np.isfinite(rl)
    # rows without a visible key: exactly o = 0, lse = -inf
    assert np.all(l[~fin] == -np.inf), label
    assert np.all(o[~fin] == 0), label
    assert np.all(np.isfinite(o)), label
    d = np.abs(o - ro)
    max_abs = float(d.max()) if d.size else 0.0
    mean_rel = float(d.sum() / max(np.abs(ro).sum(), 1e-300)) if d.size else 0.0
    lse_err = float(np.abs(l[fin] - rl[fin]).max()) if fin.any() else 0.0
    bound = MAX_ABS + np.broadcast_to(np.asarray(extra_abs, np.float64), d.shape)
    if bf16_out:
        # the output's own rounding: half an ulp of the value that is rounded
        # (at most |ref| plus the bound above) per element, and in the mean
        # relative error the rounding error of the reference itself
        bound = bound + bf16_half_ulp(np.abs(ro) + bound)
        r16 = W.bf16_to_f32(W.bf16_round(ro.astype(np.float32))).astype(np.float64)
        mean_rel_max = mean_rel_max + float(np.abs(r16 - ro).sum() / max(np.abs(ro).sum(), 1e-300))
    worst = float((d - bound).max()) if d.size else 0.0
    assert worst <= 0, "%s max_abs %.3g (exceeds its bound by %.3g)" % (label, max_abs, worst)
    assert mean_rel <= mean_rel_max, "%s mean_rel %.3g" % (label, mean_rel)
    assert lse_err <= lse_tol * max(1.0, float(np.abs(rl[fin]).max()) if fin.any() else 1.0), \
        "%s lse err %.3g" % (label, lse_err)
    return {"max_abs": max_abs, "mean_rel": mean_rel, "lse_err": lse_err}


def sample_rows(w: W.Workload, n: int, seed: int = 0):
    """Row ids (token * H + head) spread over requests, drafts and heads, always
    including the first and last row of every request."""
    rng = np.random.default_rng(seed)
    H = w.num_heads
    rows = set()
    for b in range(w.batch):
        r0, r1 = int(w.qo_indptr[b]) * H, int(w.qo_indptr[b + 1]) * H
        if r1 > r0:
            rows.update([r0, r1 - 1])
    total = w.total_q * H
    rows.update(int(x) for x in rng.choice(total, size=min(n, total), replace=False))
    return np.array(sorted(rows), dtype=np.int64)
