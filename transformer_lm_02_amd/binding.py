"""Thin Python binding over libgpt_hip.so (argument marshalling only).

The C entry points keep their names (gpt_init, gpt_forward_loss,
gpt_backward, gpt_adamw_step, ...).  PyTorch supplies device memory and the
current HIP stream; every step of the computation runs in the library's
kernels.  Importing this module fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

# PyTorch ships its own HIP runtime.  Loading it first makes the library bind to
# that same runtime (it is already loaded under the name the library needs);
# loading the library first would put a second HIP runtime in the process,
# and whichever starts second finds no device.
import torch  # noqa: F401  (imported for its side effect on the loader)

LIB_PATH = os.environ.get("GPT_HIP_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libgpt_hip.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m transformer_lm_02_amd.build`")
lib = ctypes.CDLL(LIB_PATH)

GPT_OK, GPT_EINVAL, GPT_ESEQLEN, GPT_ESTATE, GPT_EHIP, GPT_EUNSUPPORTED = 0, -1, -2, -3, -4, -5
GPT_FP32, GPT_BF16, GPT_FP16 = 0, 1, 2
GPT_FLAG_BAD_TOKEN = 1
GPT_FLAG_BAD_TARGET = 2
GPT_FLAG_HEAD_RANGE = 4
GPT_OPT_FUSED_HEAD_CE = 1
GPT_OPT_TIME_WEIGHT_GRADIENTS = 2


class gpt_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "vocab_size", "padded_vocab", "block_size", "n_layer", "n_head", "n_embd", "mode",
        "max_batch")]


class gpt_dropout(ctypes.Structure):
    _fields_ = [("p", ctypes.c_float), ("step", ctypes.c_uint32), ("seed", ctypes.c_uint64)]


_p, _i32, _i64, _f = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "gpt_query_sizes": [ctypes.POINTER(gpt_config), ctypes.POINTER(_i64), ctypes.POINTER(_i64)],
    "gpt_init": [ctypes.POINTER(_p), ctypes.POINTER(gpt_config), _p, _p, _p, _p, _p, _p,
                 ctypes.c_uint64, _p],
    "gpt_forward_loss": [_p, _p, _p, _i32, _i32, _f, _p, _p, _p],
    "gpt_forward_loss_scaled": [_p, _p, _p, _i32, _i32, _f, _p, _p, _p, _p],
    "gpt_forward_loss_ex": [_p, _p, _p, _i32, _i32, _f, _p, ctypes.POINTER(gpt_dropout), _p, _p,
                            _p],
    "gpt_op_dropout": [_p, _p, _i64, _i32, _f, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                       _p],
    "gpt_amp_step": [_p, _f, _f, _f, _f, _f, _f, _p, _f, _f, _i32, _p, _p],
    "gpt_backward": [_p, _i32, _p],
    "gpt_eval_loss": [_p, _p, _p, _i32, _i32, _p, _p],
    "gpt_estimate_loss": [_p, _p, _p, _i32, _i32, _i32, _p, _p],
    "gpt_adamw_step": [_p, _f, _f, _f, _f, _f, _f, _i32, _i32, _p, _p],
    "gpt_read_flags": [_p, ctypes.POINTER(_i32), _p],
    "gpt_read_timing": [_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)],
    "gpt_set_option": [_p, _i32, _i32],
    "gpt_get_option": [_p, _i32, ctypes.POINTER(_i32)],
    "gpt_op_linear": [_i32, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p],
    "gpt_op_linear_gelu": [_i32, _p, _p, _p, _p, _p, _i32, _i32, _i32, _p],
    "gpt_op_linear_gelu_bwd": [_i32, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _i64, _p],
    "gpt_op_linear_gelu_bwd_noalloc": [_i32, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p],
    "gpt_op_linear_dw": [_i32, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _i64, _p],
    "gpt_op_linear_dw_seq": [_i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _p],
    "gpt_op_linear_dx": [_i32, _p, _p, _p, _i32, _i32, _i32, _p],
    "gpt_op_attention_fwd": [_i32, _p, _p, _p, _i32, _i32, _i32, _i32, _p],
    "gpt_op_attention_bwd": [_i32, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p],
    "gpt_op_layernorm_fwd": [_i32, _p, _p, _p, _p, _p, _p, _i32, _i32, _p],
    "gpt_op_cross_entropy": [_i32, _p, _p, _p, _p, _p, _f, _i32, _i32, _i32, _p],
    "gpt_prefill": [_p, _p, _i32, _i32, _p, _i32, _p, _p],
    "gpt_decode_step": [_p, _p, _i32, _i32, _p, _i32, _p, _p],
    "gpt_sample": [_p, _i32, _i32, _i32, _f, _i32, _p, _p, _p],
}
for _name, _args in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int
lib.gpt_kv_cache_bytes.argtypes = [ctypes.POINTER(gpt_config), _i32, _i32]
lib.gpt_kv_cache_bytes.restype = ctypes.c_int64
lib.gpt_destroy.argtypes = [_p]
lib.gpt_destroy.restype = None
lib.gpt_lr_at.argtypes = [_i64, ctypes.c_double, ctypes.c_double, _i64, _i64]
lib.gpt_lr_at.restype = ctypes.c_double
lib.gpt_strerror.argtypes = [ctypes.c_int]
lib.gpt_strerror.restype = ctypes.c_char_p


class GptError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {lib.gpt_strerror(code).decode()} (code {code})")
        self.code = code


def check(code: int, where: str) -> None:
    if code != GPT_OK:
        raise GptError(code, where)


def make_config(vocab_size, padded_vocab, block_size, n_layer, n_head, n_embd, mode, max_batch):
    return gpt_config(vocab_size, padded_vocab, block_size, n_layer, n_head, n_embd, mode, max_batch)


def query_sizes(cfg: gpt_config):
    n, ws = _i64(), _i64()
    check(lib.gpt_query_sizes(ctypes.byref(cfg), ctypes.byref(n), ctypes.byref(ws)), "gpt_query_sizes")
    return n.value, ws.value


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class GPT:
    """Device buffers (torch tensors) plus the library handle."""

    def __init__(self, dims: dict, mode: int, max_batch: int, init_params=None, seed=0,
                 device="cuda"):
        """init_params: host array of the initial parameters (canonical order),
        or None to draw them on the device from `seed` (gpt_init)."""
        import torch
        self.dims = dict(dims)
        self.mode = mode
        self.cfg = make_config(dims["vocab_size"], dims["padded_vocab"], dims["block_size"],
                               dims["n_layer"], dims["n_head"], dims["n_embd"], mode, max_batch)
        self.n_params, ws_bytes = query_sizes(self.cfg)
        f32 = dict(dtype=torch.float32, device=device)
        self.params = torch.empty(self.n_params, **f32)
        self.grads = torch.empty(self.n_params, **f32)
        self.adam_m = torch.empty(self.n_params, **f32)
        self.adam_v = torch.empty(self.n_params, **f32)
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        self.scalars = torch.zeros(4, **f32)  # loss, norm
        # gpt_loss_scaler {float scale; int32 growth_tracker, steps, found_inf}
        self.scaler = torch.zeros(4, dtype=torch.int32, device=device)
        self.init_scaler()
        init = None
        if init_params is not None:
            init = torch.as_tensor(np.asarray(init_params, dtype=np.float32)).to(device)
            assert init.numel() == self.n_params
        h = ctypes.c_void_p()
        check(lib.gpt_init(ctypes.byref(h), ctypes.byref(self.cfg), _ptr(self.params),
                           _ptr(self.grads), _ptr(self.adam_m), _ptr(self.adam_v),
                           _ptr(self.workspace), _ptr(init), seed, _stream()), "gpt_init")
        self.handle = h
        self._init = init

    @property
    def act_dtype(self):
        import torch
        return {GPT_BF16: torch.bfloat16, GPT_FP16: torch.float16}.get(self.mode, torch.float32)

    def forward(self, idx, targets=None, loss_scale=1.0, logits=False, scaled=False,
                dropout=None):
        """idx/targets: int32 cuda tensors [B, T].  Returns (loss tensor [1] or
        None, logits tensor [B, T, Vp] or None).  scaled: the logits gradient
        is further multiplied by the device loss scale (gpt_forward_loss_scaled).
        dropout: (p, seed, step) for a training forward with dropout
        (gpt_forward_loss_ex); the next backward uses its masks."""
        import torch
        B, T = idx.shape
        out = None
        if logits:
            out = torch.empty((B, T, self.dims["padded_vocab"]), dtype=self.act_dtype, device=idx.device)
        loss = self.scalars[0:1] if targets is not None else None
        if dropout is not None:
            p, seed, step = dropout
            dr = gpt_dropout(p, step, seed)
            check(lib.gpt_forward_loss_ex(self.handle, _ptr(idx), _ptr(targets), B, T, loss_scale,
                                          _ptr(self.scaler) if scaled else None, ctypes.byref(dr),
                                          _ptr(loss), _ptr(out), _stream()), "gpt_forward_loss_ex")
        elif scaled:
            check(lib.gpt_forward_loss_scaled(self.handle, _ptr(idx), _ptr(targets), B, T,
                                              loss_scale, _ptr(self.scaler), _ptr(loss), _ptr(out),
                                              _stream()), "gpt_forward_loss_scaled")
        else:
            check(lib.gpt_forward_loss(self.handle, _ptr(idx), _ptr(targets), B, T, loss_scale,
                                       _ptr(loss), _ptr(out), _stream()), "gpt_forward_loss")
        return loss, out

    # ------------------------------------------------------------ loss scaling
    def init_scaler(self, scale=65536.0, growth_tracker=0, steps=0):
        """Write the device gpt_loss_scaler state."""
        import torch
        st = np.array([0, growth_tracker, steps, 0], np.int32)
        st[0] = np.array([scale], np.float32).view(np.int32)[0]
        self.scaler.copy_(torch.from_numpy(st))

    def scaler_state(self):
        """(scale, growth_tracker, steps, found_inf) read back (synchronises)."""
        st = self.scaler.cpu().numpy()
        return float(st[:1].view(np.float32)[0]), int(st[1]), int(st[2]), int(st[3])

    def amp_step(self, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
                 growth_factor=2.0, backoff_factor=0.5, growth_interval=2000):
        """Unscale, clip, AdamW or skip, scale update: gpt_amp_step.  Returns
        the device norm of the unscaled gradients."""
        norm = self.scalars[1:2]
        check(lib.gpt_amp_step(self.handle, lr, beta1, beta2, eps, weight_decay, max_norm,
                               _ptr(self.scaler), growth_factor, backoff_factor, growth_interval,
                               _ptr(norm), _stream()), "gpt_amp_step")
        return norm

    def eval_loss(self, idx, targets):
        """Mean loss of one batch in eval mode, no gradient (gpt_eval_loss);
        returns a device tensor [1]."""
        B, T = idx.shape
        loss = self.scalars[2:3]
        check(lib.gpt_eval_loss(self.handle, _ptr(idx), _ptr(targets), B, T, _ptr(loss), _stream()),
              "gpt_eval_loss")
        return loss

    def estimate_loss(self, batches):
        """The pages' estimate_loss over one split (gpt_estimate_loss: every
        batch's eval loss and their mean on the device); batches: list of
        (idx, targets) int32 cuda tensors [B, T] of one shape.  Returns the
        mean as a float (read back, as the pages' loop does with loss.item())."""
        import torch
        idx = torch.stack([b[0] for b in batches]).contiguous()
        tgt = torch.stack([b[1] for b in batches]).contiguous()
        n, B, T = idx.shape
        loss = self.scalars[3:4]
        check(lib.gpt_estimate_loss(self.handle, _ptr(idx), _ptr(tgt), n, B, T, _ptr(loss),
                                    _stream()), "gpt_estimate_loss")
        return float(loss.item())

    def backward(self, zero_first=True):
        check(lib.gpt_backward(self.handle, 1 if zero_first else 0, _stream()), "gpt_backward")

    def adamw_step(self, lr, t, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
                   skip_nonfinite=False):
        norm = self.scalars[1:2]
        check(lib.gpt_adamw_step(self.handle, lr, beta1, beta2, eps, weight_decay, max_norm, t,
                                 1 if skip_nonfinite else 0, _ptr(norm), _stream()), "gpt_adamw_step")
        return norm

    # ------------------------------------------------------------ sampling
    def kv_cache(self, B, max_len=None):
        """Device cache for B sequences of up to max_len (default block_size)
        positions; returns (buffer, max_len)."""
        import torch
        max_len = max_len or self.dims["block_size"]
        n = lib.gpt_kv_cache_bytes(ctypes.byref(self.cfg), B, max_len)
        if n < 0:
            raise GptError(GPT_EINVAL, "gpt_kv_cache_bytes")
        return torch.empty(n, dtype=torch.uint8, device=self.params.device), max_len

    def prefill(self, idx, kv, max_len, logits=None):
        """idx: int32 cuda [B, T0].  Returns fp32 logits [B, Vp] of the last position."""
        import torch
        B, T0 = idx.shape
        if logits is None:
            logits = torch.empty((B, self.dims["padded_vocab"]), dtype=torch.float32, device=idx.device)
        check(lib.gpt_prefill(self.handle, _ptr(idx), B, T0, _ptr(kv), max_len, _ptr(logits),
                              _stream()), "gpt_prefill")
        return logits

    def decode_step(self, tok, pos, kv, max_len, logits=None):
        """tok: int32 cuda [B] at position pos.  Returns fp32 logits [B, Vp]."""
        import torch
        B = tok.shape[0]
        if logits is None:
            logits = torch.empty((B, self.dims["padded_vocab"]), dtype=torch.float32, device=tok.device)
        check(lib.gpt_decode_step(self.handle, _ptr(tok), B, pos, _ptr(kv), max_len, _ptr(logits),
                                  _stream()), "gpt_decode_step")
        return logits

    def generate(self, idx, n_new, temperature=0.8, top_k=200, u=None, keep_logits=False):
        """GPT.generate with the cache: idx int32 cuda [B, T0]; u fp32 cuda
        [B, n_new] uniforms in [0, 1) (drawn here from torch when None).
        While a sequence fits in block_size each step feeds one token; past it
        the last block_size tokens are prefilled again (the pages' cropping).
        Returns (tokens [B, T0 + n_new], list of the fp32 logits each draw used
        when keep_logits)."""
        import torch
        bs = self.dims["block_size"]
        B = idx.shape[0]
        if u is None:
            u = torch.rand((B, n_new), dtype=torch.float32, device=idx.device)
        kv, max_len = self.kv_cache(B, bs)
        seq = idx.to(torch.int32).contiguous()
        logits = self.prefill(seq[:, -bs:].contiguous(), kv, max_len)
        kept = []
        for i in range(n_new):
            if keep_logits:
                kept.append(logits.clone())
            tok = sample(logits, self.dims["vocab_size"], temperature, top_k, u[:, i].contiguous())
            seq = torch.cat([seq, tok[:, None]], dim=1)
            if i + 1 == n_new:
                break
            n = seq.shape[1]
            if n <= bs:
                logits = self.decode_step(tok, n - 1, kv, max_len, logits)
            else:
                logits = self.prefill(seq[:, -bs:].contiguous(), kv, max_len, logits)
        return seq, kept

    def set_option(self, option: int, value: int) -> None:
        check(lib.gpt_set_option(self.handle, option, value), "gpt_set_option")

    def get_option(self, option: int) -> int:
        v = _i32()
        check(lib.gpt_get_option(self.handle, option, ctypes.byref(v)), "gpt_get_option")
        return v.value

    def read_flags(self) -> int:
        f = _i32()
        check(lib.gpt_read_flags(self.handle, ctypes.byref(f), _stream()), "gpt_read_flags")
        return f.value

    def read_timing(self):
        """(milliseconds, launches) of the weight-gradient launches timed since
        the last call (GPT_OPT_TIME_WEIGHT_GRADIENTS)."""
        ms, n = ctypes.c_double(), _i64()
        check(lib.gpt_read_timing(self.handle, ctypes.byref(ms), ctypes.byref(n)),
              "gpt_read_timing")
        return ms.value, n.value

    def close(self):
        if getattr(self, "handle", None):
            lib.gpt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lr_at(it, max_lr=6e-4, min_lr=None, warmup=715, decay_end=19073):
    """Learning rate at iteration it (gpt_lr_at); min_lr defaults to a tenth
    of max_lr."""
    return lib.gpt_lr_at(it, max_lr, 0.1 * max_lr if min_lr is None else min_lr, warmup,
                         decay_end)


def sample(logits, vocab_size, temperature, top_k, u):
    """One draw per row of fp32 logits [B, ldv] over ids [0, vocab_size):
    gpt_sample.  u: fp32 cuda [B].  Returns int32 tokens [B]."""
    import torch
    B, ldv = logits.shape
    tok = torch.empty(B, dtype=torch.int32, device=logits.device)
    check(lib.gpt_sample(_ptr(logits), B, vocab_size, ldv, temperature, top_k, _ptr(u), _ptr(tok),
                         _stream()), "gpt_sample")
    return tok


# --------------------------------------------------------------------------- single ops
def _bf(t):
    """GPT_FP32 / GPT_BF16 / GPT_FP16 from a tensor's dtype."""
    import torch
    return {torch.bfloat16: GPT_BF16, torch.float16: GPT_FP16}.get(t.dtype, GPT_FP32)


def op_linear(A, B, bias=None, out_f32=False):
    import torch
    M, K = A.shape
    N = B.shape[0]
    C = torch.empty((M, N), dtype=torch.float32 if out_f32 else A.dtype, device=A.device)
    check(lib.gpt_op_linear(_bf(A), _ptr(A), _ptr(B), _ptr(bias), _ptr(C), int(out_f32), M, N, K,
                            _stream()), "gpt_op_linear")
    return C


def op_linear_gelu(A, W, bias=None):
    """(dgelu, g) = (gelu'(u), gelu(u)) with u = A W^T + bias: gpt_op_linear_gelu."""
    import torch
    M, K = A.shape
    N = W.shape[0]
    dg = torch.empty((M, N), dtype=A.dtype, device=A.device)
    g = torch.empty((M, N), dtype=A.dtype, device=A.device)
    check(lib.gpt_op_linear_gelu(_bf(A), _ptr(A), _ptr(W), _ptr(bias), _ptr(dg), _ptr(g), M, N, K,
                                 _stream()), "gpt_op_linear_gelu")
    return dg, g


def gelu_bwd_scratch_bytes(M, N):
    """Scratch the column sums of gpt_op_linear_gelu_bwd need: ceil(M/128) N fp32."""
    return -(-M // 128) * N * 4


def op_linear_gelu_bwd(dY, Wt, dgelu, dbias=None, accumulate_bias=False, workspace=None):
    """du = (dY Wt^T) * dgelu and dbias (+)= colsum(du): gpt_op_linear_gelu_bwd.
    workspace: fp32 cuda scratch (allocated here when dbias is given and it is None)."""
    import torch
    M, K = dY.shape
    N = Wt.shape[0]
    du = torch.empty((M, N), dtype=dY.dtype, device=dY.device)
    if dbias is not None and workspace is None:
        workspace = torch.empty(gelu_bwd_scratch_bytes(M, N) // 4, dtype=torch.float32,
                                device=dY.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.gpt_op_linear_gelu_bwd(_bf(dY), _ptr(dY), _ptr(Wt), _ptr(dgelu), _ptr(du), _ptr(dbias),
                                     int(accumulate_bias), M, N, K, _ptr(workspace), wsb,
                                     _stream()), "gpt_op_linear_gelu_bwd")
    return du


def op_linear_gelu_bwd_noalloc(dY, Wt, dgelu, dbias=None, accumulate_bias=False):
    """gpt_op_linear_gelu_bwd_noalloc: as op_linear_gelu_bwd, with the library's
    own device scratch in place of a workspace."""
    import torch
    M, K = dY.shape
    N = Wt.shape[0]
    du = torch.empty((M, N), dtype=dY.dtype, device=dY.device)
    check(lib.gpt_op_linear_gelu_bwd_noalloc(_bf(dY), _ptr(dY), _ptr(Wt), _ptr(dgelu), _ptr(du),
                                             _ptr(dbias), int(accumulate_bias), M, N, K,
                                             _stream()), "gpt_op_linear_gelu_bwd_noalloc")
    return du


def op_linear_dw(dY, X, dW=None, workspace=None):
    import torch
    M, N = dY.shape
    K = X.shape[1]
    acc = dW is not None
    if dW is None:
        dW = torch.empty((N, K), dtype=torch.float32, device=dY.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.gpt_op_linear_dw(_bf(dY), _ptr(dY), _ptr(X), _ptr(dW), int(acc), M, N, K,
                               _ptr(workspace), wsb, _stream()), "gpt_op_linear_dw")
    return dW


def op_linear_dw_seq(items, workspace=None):
    """gpt_op_linear_dw_seq over items = [(dY, X, dW, accumulate), ...]
    (dW fp32 [N][K], written or added to)."""
    n = len(items)
    ptrs = lambda ts: (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])
    ints = lambda vs: (ctypes.c_int32 * n)(*vs)
    dt = _bf(items[0][0]) if n else GPT_BF16
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.gpt_op_linear_dw_seq(
        dt, n, ptrs([it[0] for it in items]), ptrs([it[1] for it in items]),
        ptrs([it[2] for it in items]), ints([int(bool(it[3])) for it in items]),
        ints([it[0].shape[0] for it in items]), ints([it[0].shape[1] for it in items]),
        ints([it[1].shape[1] for it in items]), _ptr(workspace), wsb, _stream()),
        "gpt_op_linear_dw_seq")


def op_linear_dx(dY, W):
    import torch
    M, N = dY.shape
    K = W.shape[1]
    dX = torch.empty((M, K), dtype=torch.float32, device=dY.device)
    check(lib.gpt_op_linear_dx(_bf(dY), _ptr(dY), _ptr(W), _ptr(dX), M, N, K, _stream()),
          "gpt_op_linear_dx")
    return dX


def op_attention_fwd(qkv, B, T, H):
    import torch
    C = qkv.shape[-1] // 3
    out = torch.empty((B * T, C), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=qkv.device)
    check(lib.gpt_op_attention_fwd(_bf(qkv), _ptr(qkv), _ptr(out), _ptr(lse), B, T, H, C, _stream()),
          "gpt_op_attention_fwd")
    return out, lse


def op_attention_bwd(qkv, out, lse, dout, B, T, H):
    import torch
    C = qkv.shape[-1] // 3
    dqkv = torch.empty_like(qkv)
    D = torch.empty((2, B, H, T), dtype=torch.float32, device=qkv.device)
    check(lib.gpt_op_attention_bwd(_bf(qkv), _ptr(qkv), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dqkv),
                                   _ptr(D), B, T, H, C, _stream()), "gpt_op_attention_bwd")
    return dqkv


def op_layernorm_fwd(x, w, b, bf16=False, fp16=False):
    import torch
    M, C = x.shape
    dt = torch.bfloat16 if bf16 else torch.float16 if fp16 else torch.float32
    y = torch.empty((M, C), dtype=dt, device=x.device)
    mean = torch.empty(M, dtype=torch.float32, device=x.device)
    rstd = torch.empty(M, dtype=torch.float32, device=x.device)
    check(lib.gpt_op_layernorm_fwd(_bf(y), _ptr(x), _ptr(w), _ptr(b), _ptr(y), _ptr(mean),
                                   _ptr(rstd), M, C, _stream()), "gpt_op_layernorm_fwd")
    return y, mean, rstd


def op_dropout(x, p, seed, step, site_word):
    """y = x times the dropout multipliers of one site (gpt_op_dropout); x fp32
    cuda [rows, cols]."""
    import torch
    rows, cols = x.shape
    y = torch.empty_like(x)
    check(lib.gpt_op_dropout(_ptr(x), _ptr(y), rows, cols, p, seed, step, site_word, _stream()),
          "gpt_op_dropout")
    return y


def op_cross_entropy(logits, targets, V, loss_scale=1.0):
    """In place on logits [N, ldv]; returns (loss [1], row_loss [N], n_valid [1])."""
    import torch
    N, ldv = logits.shape
    loss = torch.empty(1, dtype=torch.float32, device=logits.device)
    row = torch.empty(N, dtype=torch.float32, device=logits.device)
    nv = torch.empty(1, dtype=torch.int32, device=logits.device)
    check(lib.gpt_op_cross_entropy(_bf(logits), _ptr(logits), _ptr(targets), _ptr(loss), _ptr(row),
                                   _ptr(nv), loss_scale, N, V, ldv, _stream()), "gpt_op_cross_entropy")
    return loss, row, nv
