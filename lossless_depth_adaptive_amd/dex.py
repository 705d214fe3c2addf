"""ctypes binding of libdex.so (include/dex.h). Argument marshalling only.

PyTorch provides device memory (the workspace, the caller's weight tensors,
the Gumbel rows) and the HIP stream; every step of the decoding path runs in
the library's HIP kernels. Importing this module without a built library
raises ImportError: there is no fallback implementation.
"""

import ctypes
import os
from typing import Dict, List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; DEX_LIBRARY may name another build of the same sources.
LIB_PATH = os.environ.get("DEX_LIBRARY") or os.path.join(HERE, "libdex.so")

DEX_OK, DEX_EINVAL, DEX_ENOSPC, DEX_ESTATE, DEX_EHIP = 0, -1, -2, -3, -4
DTYPE_F32, DTYPE_BF16 = 0, 1
GREEDY, SAMPLE = 0, 1
EXPORTED = ["dex_workspace_bytes", "dex_create", "dex_prefill", "dex_step", "dex_step_noalloc", "dex_ar_step",
            "dex_debug_anchor", "dex_last_step_rows", "dex_profile", "dex_destroy", "dex_last_error"]
PROF_CLASSES = ["gemm", "attention", "exit_head", "row_ops", "lattice"]


class ModelConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("tied_head", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("adapter_hidden", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class Weights(ctypes.Structure):
    _fields_ = [("tok_embed", ctypes.c_void_p), ("attn_norm", _PP), ("wq", _PP), ("wk", _PP),
                ("wv", _PP), ("wo", _PP), ("ffn_norm", _PP), ("w_gate", _PP), ("w_up", _PP),
                ("w_down", _PP), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("adapter_w1", _PP), ("adapter_b1", _PP), ("adapter_w2", _PP), ("adapter_b2", _PP),
                ("adapter_norm", _PP), ("adapter_alpha", ctypes.POINTER(ctypes.c_float))]


class Options(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("temperature", ctypes.c_float),
                ("decs", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_context", ctypes.c_int32), ("max_new_tokens", ctypes.c_int32),
                ("gumbel", ctypes.c_void_p), ("gumbel_rows", ctypes.c_int32),
                ("debug", ctypes.c_int32), ("single_exit", ctypes.c_int32),
                ("branch_cap", ctypes.c_int32)]


class Commit(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("position", ctypes.c_int32), ("token", ctypes.c_int32),
                ("branch", ctypes.c_int32), ("layers", ctypes.c_int32)]


class KernelStats(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double), ("launches", ctypes.c_int64), ("bytes", ctypes.c_double),
                ("flops", ctypes.c_double)]


class DexError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dex error {code}: {msg}")
        self.code = code


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libdex.so (raises ImportError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m lossless_depth_adaptive_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, vp, P = ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER
    lib.dex_workspace_bytes.argtypes = [P(ModelConfig), P(i32), i32, P(Options), P(ctypes.c_size_t)]
    lib.dex_create.argtypes = [P(ModelConfig), P(Weights), P(i32), i32, i32, P(Options), vp,
                               ctypes.c_size_t, vp, P(vp)]
    lib.dex_prefill.argtypes = [vp, i32, P(i32), P(i32)]
    lib.dex_step.argtypes = [vp, P(Commit), i32, P(i32)]
    lib.dex_ar_step.argtypes = [vp, P(Commit), i32, P(i32)]
    lib.dex_step_noalloc.argtypes = [vp, P(Commit), i32, P(i32)]
    lib.dex_debug_anchor.argtypes = [vp, i32, P(i32), P(ctypes.c_float), P(ctypes.c_float)]
    lib.dex_last_step_rows.argtypes = [vp, P(i32), P(i32)]
    lib.dex_profile.argtypes = [vp, i32, P(KernelStats), i32]
    lib.dex_destroy.argtypes = [vp]
    lib.dex_destroy.restype = None
    lib.dex_last_error.argtypes = [vp]
    lib.dex_last_error.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("dex_destroy", "dex_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _i32_array(vals: Sequence[int]):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


def model_config(n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab, rope_base=10000.0,
                 rms_eps=1e-5, tied_head=False, dtype="bf16", adapter_hidden=0) -> ModelConfig:
    """``adapter_hidden``: m of the inducing adapters (0: none)."""
    return ModelConfig(n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab, rope_base,
                       rms_eps, int(bool(tied_head)), DTYPE_BF16 if dtype == "bf16" else DTYPE_F32,
                       int(adapter_hidden))


def options(mode="greedy", temperature=1.0, decs=True, max_batch=1, max_context=1024,
            max_new_tokens=256, gumbel=None, debug=False, graphs=True, single_exit=False,
            branch_cap=0, span_attention=False) -> Options:
    """``gumbel``: CUDA float32 tensor [max_batch, rows, vocab] or None. ``debug`` keeps the
    final-depth logits of each last commit; ``graphs=False`` launches every round eagerly;
    ``single_exit`` selects the single-exit ablation; ``branch_cap`` > 0 the pruned lattice
    (position children only from explorers below it); ``span_attention`` makes grouped
    attention blocks always run whole spans (same results; for tests)."""
    if gumbel is not None:
        import torch
        if not isinstance(gumbel, torch.Tensor) or gumbel.dtype != torch.float32 or not gumbel.is_cuda:
            raise ValueError("gumbel must be a float32 tensor on the GPU")
        if gumbel.dim() != 3 or not gumbel.is_contiguous():
            raise ValueError("gumbel must be a contiguous [max_batch, rows, vocab] tensor")
        if gumbel.shape[0] < max_batch or gumbel.shape[1] < max_new_tokens:
            raise ValueError(f"gumbel has shape {tuple(gumbel.shape)}: it needs max_batch={max_batch} "
                             f"sequences and at least max_new_tokens={max_new_tokens} rows")
        if gumbel.data_ptr() % 16:
            raise ValueError("gumbel must be 16-byte aligned")
    opt = Options(SAMPLE if mode == "sample" else GREEDY, float(temperature), int(bool(decs)),
                  max_batch, max_context, max_new_tokens,
                  None if gumbel is None else gumbel.data_ptr(),
                  0 if gumbel is None else gumbel.shape[1],
                  int(bool(debug)) | (0 if graphs else 2) | (4 if span_attention else 0),
                  int(bool(single_exit)), int(branch_cap))
    # The library reads the rows through the raw pointer: the options keep the
    # tensor alive, and the context made from them keeps the options.
    opt._gumbel = gumbel
    return opt


def workspace_bytes(cfg: ModelConfig, X: Sequence[int], opt: Options) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    xa = _i32_array(X)
    rc = lib.dex_workspace_bytes(ctypes.byref(cfg), xa, len(X), ctypes.byref(opt), ctypes.byref(out))
    if rc != DEX_OK:
        raise DexError(rc, lib.dex_last_error(None).decode())
    return out.value


class Dex:
    """One library context: dex_create / dex_prefill / dex_step / dex_ar_step.

    ``weights`` is a dict with ``embed``, ``layers`` (list of dicts holding
    ``attn_norm, wq, wk, wv, wo, ffn_norm, w_gate, w_up, w_down``),
    ``final_norm`` and ``lm_head``: CUDA tensors in the storage dtype,
    row-major [out, in]. The library packs them into its workspace.
    ``adapters`` (needed when cfg.adapter_hidden > 0): one dict per non-final
    explorer with CUDA tensors ``w1, b1, w2, b2, norm`` and a float ``alpha``.
    """

    def __init__(self, cfg: ModelConfig, weights: Dict, X: Sequence[int], opt: Options,
                 stream=None, device="cuda", adapters=None):
        import torch
        self.lib = load_library()
        self.cfg, self.opt, self.X = cfg, opt, list(X)
        self.N = len(X)
        self._keep = [opt]
        g = getattr(opt, "_gumbel", None)
        if opt.mode == SAMPLE and g is None and opt.gumbel:
            raise ValueError("sampling options must come from options(), which checks and keeps the Gumbel rows")
        if g is not None:
            if g.shape[0] < opt.max_batch or g.shape[2] != cfg.vocab or g.shape[1] < opt.max_new_tokens + self.N - 1:
                raise ValueError(f"gumbel has shape {tuple(g.shape)}; this context needs "
                                 f"[>= {opt.max_batch}, >= {opt.max_new_tokens + self.N - 1}, {cfg.vocab}]")
            self._keep.append(g)
        nbytes = workspace_bytes(cfg, X, opt)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        L = cfg.n_layers

        def arr(key):
            a = (ctypes.c_void_p * L)(*[weights["layers"][l][key].data_ptr() for l in range(L)])
            self._keep.append(a)
            return ctypes.cast(a, _PP)

        w = Weights(weights["embed"].data_ptr(), arr("attn_norm"), arr("wq"), arr("wk"), arr("wv"),
                    arr("wo"), arr("ffn_norm"), arr("w_gate"), arr("w_up"), arr("w_down"),
                    weights["final_norm"].data_ptr(), weights["lm_head"].data_ptr())
        if cfg.adapter_hidden:
            if adapters is None or len(adapters) != self.N - 1:
                raise ValueError("adapter_hidden > 0 needs one adapter per non-final explorer")

            def aarr(key):
                a = (ctypes.c_void_p * len(adapters))(*[ad[key].data_ptr() for ad in adapters])
                self._keep.append(a)
                return ctypes.cast(a, _PP)

            alpha = (ctypes.c_float * len(adapters))(*[float(ad["alpha"]) for ad in adapters])
            self._keep.append(alpha)
            w.adapter_w1, w.adapter_b1, w.adapter_w2 = aarr("w1"), aarr("b1"), aarr("w2")
            w.adapter_b2, w.adapter_norm = aarr("b2"), aarr("norm")
            w.adapter_alpha = ctypes.cast(alpha, ctypes.POINTER(ctypes.c_float))
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        ctx = ctypes.c_void_p(None)
        rc = self.lib.dex_create(ctypes.byref(cfg), ctypes.byref(w), _i32_array(X), len(X), L,
                                 ctypes.byref(opt), ctypes.c_void_p(self.workspace.data_ptr()),
                                 nbytes, ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(ctx))
        if rc != DEX_OK:
            raise DexError(rc, self.lib.dex_last_error(None).decode())
        self.ctx = ctx
        self.max_batch = opt.max_batch
        self._out = (Commit * max(1, opt.max_batch))()

    def _check(self, rc: int):
        if rc != DEX_OK:
            raise DexError(rc, self.lib.dex_last_error(self.ctx).decode())

    def prefill(self, prompts: List[Sequence[int]]):
        flat = [int(t) for p in prompts for t in p]
        self._check(self.lib.dex_prefill(self.ctx, len(prompts), _i32_array(flat),
                                         _i32_array([len(p) for p in prompts])))

    def _step(self, fn) -> List[dict]:
        n = ctypes.c_int32(0)
        self._check(fn(self.ctx, self._out, len(self._out), ctypes.byref(n)))
        return [dict(seq=c.seq, position=c.position, token=c.token, branch=c.branch, layers=c.layers)
                for c in self._out[:n.value]]

    def step(self) -> List[dict]:
        return self._step(self.lib.dex_step)

    def step_noalloc(self) -> List[dict]:
        """dex_step with the round's scratch in the library's static device
        array and no graph capture (allocates nothing)."""
        return self._step(self.lib.dex_step_noalloc)

    def ar_step(self) -> List[dict]:
        return self._step(self.lib.dex_ar_step)

    def debug_anchor(self, seq: int, want_logits: bool = False):
        u = (ctypes.c_int32 * self.N)()
        m = (ctypes.c_float * self.N)()
        logits = None
        lp = None
        if want_logits:
            import numpy as np
            logits = np.zeros(self.cfg.vocab, dtype=np.float32)
            lp = logits.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
        self._check(self.lib.dex_debug_anchor(self.ctx, seq, u, m, lp))
        return list(u), list(m), logits

    def last_step_rows(self):
        r = (ctypes.c_int32 * self.N)()
        t = ctypes.c_int32(0)
        self._check(self.lib.dex_last_step_rows(self.ctx, r, ctypes.byref(t)))
        return list(r), t.value

    def profile(self, enable: bool = True) -> dict:
        """Turn per-class event timing on/off; returns (and resets) the stats
        gathered since the previous call, keyed by class name."""
        n = len(PROF_CLASSES)
        st = (KernelStats * n)()
        self._check(self.lib.dex_profile(self.ctx, int(bool(enable)), st, n))
        return {PROF_CLASSES[i]: dict(ms=st[i].ms, launches=st[i].launches, bytes=st[i].bytes,
                                      flops=st[i].flops) for i in range(n)}

    def close(self):
        if getattr(self, "ctx", None) is not None and self.ctx.value:
            self.lib.dex_destroy(self.ctx)
            self.ctx = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
