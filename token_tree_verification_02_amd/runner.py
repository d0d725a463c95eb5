"""Upload a workload (see workloads.make) to the GPU and run one verification step.

One step = tree_build -> tree_attention -> tree_verify_greedy, the whole hot path
of one speculative decoding step for one attention layer, all on one stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib


def _t(a, device, bf16=False, dtype=None):
    """Host array -> device tensor; 16-bit types arrive as raw uint16 bits."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if bf16 or dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "f16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.float16)
    return torch.from_numpy(a).to(device)


def dtype_code(dtype: str) -> int:
    return {"f32": _lib.TV_F32, "bf16": _lib.TV_BF16, "f16": _lib.TV_F16}[dtype]


def upload(w: dict, device="cuda") -> dict:
    cfg = w["cfg"]
    dt = cfg.dtype
    d = dict(cfg=cfg, paged=cfg.paged, num_blocks=int(w.get("num_blocks", 0)))
    for k in ("parent", "depth", "prefix_len", "block_table", "tokens"):
        d[k] = _t(w.get(k), device)
    for k in ("q", "k_tree", "v_tree", "logits"):
        d[k] = _t(w.get(k), device, dtype=dt)
    cdt = "u8" if cfg.kv == "fp8" else dt       # an fp8 cache holds 1-byte codes
    for k in ("k_cache", "v_cache"):
        d[k] = _t(w.get(k), device, dtype=cdt)
    d["k_scale"] = float(w.get("k_scale", 0.0))
    d["v_scale"] = float(w.get("v_scale", 0.0))
    B, n = cfg.B, cfg.n
    d["mask"] = torch.empty((B, n, (n + 63) // 64), dtype=torch.int64, device=device)
    d["pos"] = torch.empty((B, n), dtype=torch.int32, device=device)
    d["status"] = torch.empty((B,), dtype=torch.int32, device=device)
    d["out"] = torch.empty_like(d["q"])
    d["lse"] = torch.empty((B, n, cfg.Hq), dtype=torch.float32, device=device)
    d["attn_status"] = torch.empty((B,), dtype=torch.int32, device=device)
    d["new_len"] = torch.empty((B,), dtype=torch.int32, device=device)
    d["commit_status"] = torch.empty((B,), dtype=torch.int32, device=device)
    desc = attn_desc_of(d)
    ws = _lib.checked_workspace_size(desc)
    d["workspace"] = torch.empty(max(ws, 1), dtype=torch.uint8, device=device) if ws else None
    if cfg.vocab and d.get("logits") is not None:
        d["argmax"] = torch.empty((B, n), dtype=torch.int32, device=device)
        d["path"] = torch.empty((B, n), dtype=torch.int32, device=device)
        d["path_len"] = torch.empty((B,), dtype=torch.int32, device=device)
        d["bonus"] = torch.empty((B,), dtype=torch.int32, device=device)
    return d


def attn_desc_of(d):
    cfg = d["cfg"]
    code = dtype_code(cfg.dtype)
    fp8 = dict(kv_dtype=_lib.TV_FP8_E4M3, k_scale=d["k_scale"], v_scale=d["v_scale"]) if cfg.kv == "fp8" else {}
    if d["paged"]:
        return _lib.attn_desc(cfg.B, cfg.n, cfg.Hq, cfg.Hkv, cfg.D, code, paged=True,
                              max_blocks=d["block_table"].shape[1], num_blocks=d["num_blocks"], **fp8)
    return _lib.attn_desc(cfg.B, cfg.n, cfg.Hq, cfg.Hkv, cfg.D, code, Lmax=d["k_cache"].shape[2], **fp8)


def build(d, stream=None):
    return _lib.tree_build(d["parent"], d["depth"], d["prefix_len"], mask=d["mask"], pos=d["pos"],
                           status=d["status"], stream=stream)


def attention(d, stream=None):
    return _lib.tree_attention(d["q"], d["k_cache"], d["v_cache"], d["prefix_len"], d["k_tree"], d["v_tree"],
                               d["mask"], block_table=d["block_table"], num_blocks=d["num_blocks"],
                               out=d["out"], lse=d["lse"], want_lse=True, status=d["attn_status"],
                               workspace=d["workspace"], k_scale=d["k_scale"], v_scale=d["v_scale"],
                               stream=stream)


def verify(d, stream=None):
    return _lib.tree_verify_greedy(d["logits"], d["tokens"], d["parent"], argmax=d["argmax"], path=d["path"],
                                   path_len=d["path_len"], bonus=d["bonus"], stream=stream)


def commit(d, path=None, path_len=None, stream=None):
    """Commit an accepted path (default: the one tree_verify_greedy wrote) into d's cache."""
    path = d["path"] if path is None else path
    path_len = d["path_len"] if path_len is None else path_len
    return _lib.tree_commit_kv(d["k_cache"], d["v_cache"], d["prefix_len"], d["k_tree"], d["v_tree"], path,
                               path_len, block_table=d["block_table"], num_blocks=d["num_blocks"],
                               new_prefix_len=d["new_len"], status=d["commit_status"], stream=stream)


def step(d, stream=None):
    """One pass of the hot path over the uploaded batch."""
    build(d, stream)
    attention(d, stream)
    if "argmax" in d:
        verify(d, stream)


class Step:
    """One verification step over an uploaded batch with the C-ABI arguments built once.

    Calling it enqueues tree_build, tree_attention and tree_verify_greedy on the
    given (or current) stream with no per-call Python marshalling beyond the
    stream handle; capture() records the same three calls into a HIP graph.
    """

    def __init__(self, d):
        import ctypes
        lib = _lib.load()
        self.d = d
        self.lib = lib
        cfg = d["cfg"]
        P = _lib._ptr
        self.desc = attn_desc_of(d)
        self._desc_ref = ctypes.byref(self.desc)
        ws = d["workspace"]
        wbytes = 0 if ws is None else ws.numel()
        self.build_args = (cfg.B, cfg.n, P(d["parent"]), P(d["depth"]), P(d["prefix_len"]), P(d["mask"]),
                           P(d["pos"]), P(d["status"]))
        self.attn_args = (self._desc_ref, P(d["q"]), P(d["k_cache"]), P(d["v_cache"]), P(d["block_table"]),
                          P(d["prefix_len"]), P(d["k_tree"]), P(d["v_tree"]), P(d["mask"]), P(d["out"]),
                          P(d["lse"]), P(d["attn_status"]), P(ws), wbytes)
        self.verify_args = None
        if "argmax" in d:
            code = dtype_code(cfg.dtype)
            self.verify_args = (cfg.B, cfg.n, cfg.vocab, code, P(d["logits"]), P(d["tokens"]), P(d["parent"]),
                                P(d["argmax"]), P(d["path"]), P(d["path_len"]), P(d["bonus"]))

    def commit_args(self, path, path_len):
        """C-ABI arguments of tree_commit_kv for this batch and the given path tensors."""
        P = _lib._ptr
        d = self.d
        return (self._desc_ref, P(d["k_cache"]), P(d["v_cache"]), P(d["block_table"]), P(d["prefix_len"]),
                P(d["k_tree"]), P(d["v_tree"]), P(path), P(path_len), P(d["new_len"]), P(d["commit_status"]))

    def commit(self, args, sh):
        rc = self.lib.tree_commit_kv(*args, sh)
        if rc:
            _lib._check(rc, "tree_commit_kv")

    def build(self, sh):
        rc = self.lib.tree_build(*self.build_args, sh)
        if rc:
            _lib._check(rc, "tree_build")

    def attention(self, sh):
        rc = self.lib.tree_attention(*self.attn_args, sh)
        if rc:
            _lib._check(rc, "tree_attention")

    def verify(self, sh):
        if self.verify_args is not None:
            rc = self.lib.tree_verify_greedy(*self.verify_args, sh)
            if rc:
                _lib._check(rc, "tree_verify_greedy")

    def __call__(self, stream=None):
        sh = (stream or torch.cuda.current_stream()).cuda_stream
        self.build(sh)
        self.attention(sh)
        self.verify(sh)

    def capture(self):
        """A torch.cuda.CUDAGraph holding one step (replay() re-runs it)."""
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self()  # warm the launch path outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self()
        return g


def capture_steps(steps) -> "torch.cuda.CUDAGraph":
    """One graph that runs the given steps back to back (replay() runs them all)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for st in steps:
            st()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for st in steps:
            st()
    return g


def out_f64(d) -> np.ndarray:
    o = d["out"]
    return o.float().double().cpu().numpy() if o.dtype in (torch.bfloat16, torch.float16) else o.double().cpu().numpy()
