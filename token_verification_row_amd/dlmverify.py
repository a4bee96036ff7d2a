"""ctypes binding of libdlmverify (include/dlmverify.h), same names as the C API.

Argument marshalling only: each function checks device, dtype and layout of
the torch tensors it is given, allocates output tensors where the caller did
not pass them, and calls the C entry point on the current HIP stream. Every
step of the computation runs in the library's HIP kernels. There is no CPU
fallback: without the built library, or without a GPU, the calls raise.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library binds to (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
# DV_LIBRARY may name another build of the same library (the sanitizer build of build_lib.py)
LIB_PATH = os.environ.get("DV_LIBRARY") or os.path.join(_HERE, "libdlmverify.so")

DV_OK, DV_ERR_NULL, DV_ERR_SHAPE, DV_ERR_DTYPE, DV_ERR_ALIGN, DV_ERR_ARG, \
    DV_ERR_WORKSPACE, DV_ERR_UNSUPPORTED, DV_ERR_HIP = range(9)
DV_FP32, DV_BF16 = 0, 1
DV_NONE, DV_KEEP, DV_REPLACE, DV_REMASK = 0, 1, 2, 3
(DV_RULE_TRUST, DV_RULE_KL, DV_RULE_CONF, DV_RULE_KL_OR_CONF, DV_RULE_COVER, DV_RULE_COUPLED_ACCEPT,
 DV_RULE_CONF_DRAFT, DV_RULE_KL_STOCHASTIC) = range(8)
RULES = {"TRUST": 0, "KL": 1, "CONF": 2, "KL_OR_CONF": 3, "COVER": 4, "COUPLED_ACCEPT": 5, "CONF_DRAFT": 6,
         "KL_STOCHASTIC": 7}
# every member of dv_row_stats, in order
STAT_FIELDS = ("lse_v", "lse_d", "kl", "entropy", "conf", "argmax_v", "argmax_d", "tok_v", "tok_d", "kl_rev", "p_tok_d")
# what dv_verify_rows computes unless asked otherwise (kl_rev selects the extended pass)
CORE_FIELDS = STAT_FIELDS[:9]
DV_LOGITS_NEG_INF = 1
_FLOAT_FIELDS = {"lse_v", "lse_d", "kl", "entropy", "conf", "kl_rev", "p_tok_d"}


class DVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class dv_logits(ctypes.Structure):
    _fields_ = [("verifier", ctypes.c_void_p), ("drafter", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("rows", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("ld", ctypes.c_int64)]


class dv_noise(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("reserved", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("pos", ctypes.c_void_p), ("pos_period", ctypes.c_int64)]


class dv_row_stats(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in STAT_FIELDS]


class dv_tuning(ctypes.Structure):
    _fields_ = [("split", ctypes.c_int32), ("shared_noise", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


class dv_decide_args(ctypes.Structure):
    _fields_ = [("rule", ctypes.c_int32), ("tau_kl", ctypes.c_float), ("conf_thr", ctypes.c_float),
                ("mask_token", ctypes.c_int32), ("rows", ctypes.c_int64), ("group_len", ctypes.c_int64),
                ("seed", ctypes.c_uint64), ("pos", ctypes.c_void_p), ("pos_period", ctypes.c_int64)]


class dv_attention(ctypes.Structure):
    _fields_ = [("probs", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("nseq", ctypes.c_int64), ("heads", ctypes.c_int64), ("len", ctypes.c_int64), ("ld", ctypes.c_int64)]


class dv_dual_view_args(ctypes.Structure):
    _fields_ = [("nseq", ctypes.c_int64), ("heads", ctypes.c_int64), ("kv_heads", ctypes.c_int64),
                ("len", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


class dv_tree_args(ctypes.Structure):
    _fields_ = [("ntrees", ctypes.c_int64), ("nodes", ctypes.c_int64), ("block_len", ctypes.c_int64)]


_P = ctypes.c_void_p
_SIGNATURES = {
    "dv_verify_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(dv_logits), ctypes.POINTER(dv_noise),
                                                 ctypes.POINTER(dv_tuning), ctypes.POINTER(ctypes.c_size_t)]),
    "dv_verify_rows": (ctypes.c_int, [ctypes.POINTER(dv_logits), ctypes.POINTER(dv_noise),
                                      ctypes.POINTER(dv_tuning), ctypes.POINTER(dv_row_stats), _P,
                                      ctypes.c_size_t, _P]),
    "dv_verify_rows_noalloc": (ctypes.c_int, [ctypes.POINTER(dv_logits), ctypes.POINTER(dv_noise),
                                              ctypes.POINTER(dv_tuning), ctypes.POINTER(dv_row_stats), _P]),
    "dv_decide": (ctypes.c_int, [ctypes.POINTER(dv_decide_args), ctypes.POINTER(dv_row_stats), _P, _P, _P, _P,
                                 _P, _P, _P]),
    "dv_seed_score": (ctypes.c_int, [ctypes.c_int64, _P, _P, _P, _P, _P, _P]),
    "dv_select_topk": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_float, _P, _P, _P, _P, _P]),
    "dv_seed_select": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P, _P, _P, _P]),
    "dv_decide_seed_select": (ctypes.c_int, [ctypes.POINTER(dv_decide_args), ctypes.POINTER(dv_row_stats)] + [_P] * 6 +
                              [ctypes.c_int64, ctypes.c_int64] + [_P] * 6 +
                              [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float] + [_P] * 5),
    "dv_seed_select_decide": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64] + [_P] * 6 +
                              [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float] + [_P] * 4 +
                              [ctypes.POINTER(dv_decide_args), ctypes.POINTER(dv_row_stats)] + [_P] * 4),
    "dv_tree_accept": (ctypes.c_int, [ctypes.POINTER(dv_tree_args)] + [_P] * 15),
    "dv_dual_view_attention": (ctypes.c_int, [ctypes.POINTER(dv_dual_view_args)] + [_P] * 8),
    "dv_influence_drift_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(dv_attention), ctypes.POINTER(ctypes.c_size_t)]),
    "dv_influence_drift": (ctypes.c_int, [ctypes.POINTER(dv_attention), _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "dv_debug_hash": (ctypes.c_int, [ctypes.c_uint64, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P]),
    "dv_debug_noise": (ctypes.c_int, [ctypes.c_uint64, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "dv_debug_read_probe": (ctypes.c_int, [ctypes.POINTER(dv_logits), ctypes.POINTER(dv_tuning), _P, _P]),
    "dv_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "dv_last_error": (ctypes.c_char_p, []),
    "dv_version": (ctypes.c_int, []),
}

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libdlmverify.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(token_verification_row_amd/build_lib.py)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, call: str):
    if status != DV_OK:
        lib = load_library()
        raise DVError(status, f"{call}: {lib.dv_status_str(status).decode()}: {lib.dv_last_error().decode()}")


def dv_status_str(status: int) -> str:
    return load_library().dv_status_str(status).decode()


def dv_last_error() -> str:
    return load_library().dv_last_error().decode()


def dv_version() -> int:
    return load_library().dv_version()


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")


def _logits_desc(verifier, drafter, vocab):
    _need_cuda(verifier, "verifier")
    _need_cuda(drafter, "drafter")
    if verifier.dim() != 2 or drafter.shape != verifier.shape:
        raise ValueError("verifier and drafter must both be [rows, ld]")
    if verifier.dtype != drafter.dtype or verifier.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits must both be float32 or both bfloat16")
    if verifier.stride() != drafter.stride() or verifier.stride(1) != 1:
        raise ValueError("logit rows must be contiguous with one common row stride")
    rows, width = verifier.shape
    ld = verifier.stride(0) if rows > 0 else width
    vocab = width if vocab is None else int(vocab)
    if vocab > width:
        raise ValueError(f"vocab {vocab} exceeds the row width {width}")
    return dv_logits(verifier=verifier.data_ptr(), drafter=drafter.data_ptr(),
                     dtype=DV_BF16 if verifier.dtype == torch.bfloat16 else DV_FP32, flags=0,
                     rows=rows, vocab=vocab, ld=ld)


def _check_pos(pos, rows):
    """pos: None, or a contiguous device int32 tensor with an entry for each of ``rows`` rows."""
    if pos is None:
        return
    _need_cuda(pos, "pos")
    if pos.dtype != torch.int32 or not pos.is_contiguous():
        raise TypeError("pos must be a contiguous int32 tensor")
    if pos.numel() < rows:
        raise ValueError(f"pos holds {pos.numel()} positions for {rows} rows")


def _noise_desc(temperature, seed, pos, pos_period, rows):
    _check_pos(pos, rows)
    return dv_noise(temperature=float(temperature), reserved=0, seed=int(seed) & 0xFFFFFFFFFFFFFFFF,
                    pos=None if pos is None else pos.data_ptr(), pos_period=int(pos_period))


def _tuning_desc(tuning):
    if tuning is None:
        return None
    t = dict(tuning)
    unknown = set(t) - {"split", "shared_noise"}
    if unknown:
        raise ValueError(f"unknown tuning keys {sorted(unknown)}")
    return dv_tuning(split=int(t.get("split", 0)), shared_noise=int(t.get("shared_noise", -1)))


def dv_verify_workspace_bytes(verifier, drafter, temperature=0.0, seed=0, pos=None, pos_period=0, *,
                              vocab=None, tuning=None) -> int:
    d = _logits_desc(verifier, drafter, vocab)
    n = _noise_desc(temperature, seed, pos, pos_period, d.rows)
    t = _tuning_desc(tuning)
    out = ctypes.c_size_t(0)
    _check(load_library().dv_verify_workspace_bytes(ctypes.byref(d), ctypes.byref(n),
                                                    None if t is None else ctypes.byref(t), ctypes.byref(out)),
           "dv_verify_workspace_bytes")
    return out.value


def dv_verify_rows(verifier, drafter, temperature=0.0, seed=0, pos=None, pos_period=0, *, vocab=None,
                   outputs=CORE_FIELDS, out=None, workspace=None, tuning=None, neg_inf=False):
    """Row statistics of [rows, ld] verifier/drafter logits. Returns a dict of
    tensors (float32 for lse_v, lse_d, kl, entropy, conf, kl_rev, p_tok_d; int32
    for the rest). neg_inf: the logits may hold -inf (DV_LOGITS_NEG_INF)."""
    d = _logits_desc(verifier, drafter, vocab)
    d.flags = DV_LOGITS_NEG_INF if neg_inf else 0
    n = _noise_desc(temperature, seed, pos, pos_period, d.rows)
    t = _tuning_desc(tuning)
    rows, dev = d.rows, verifier.device
    res = {k: v for k, v in (out or {}).items() if not k.startswith("_")}
    for f in outputs:
        if f not in STAT_FIELDS:
            raise KeyError(f)
        if f not in res:
            res[f] = torch.empty(rows, dtype=torch.float32 if f in _FLOAT_FIELDS else torch.int32, device=dev)
    for f, v in res.items():
        _need_cuda(v, f)
        want = torch.float32 if f in _FLOAT_FIELDS else torch.int32
        if v.dtype != want or v.numel() < rows or not v.is_contiguous():
            raise TypeError(f"output {f} must be a contiguous {want} tensor of >= {rows} elements")
    st = dv_row_stats(**{f: (res[f].data_ptr() if f in res else None) for f in STAT_FIELDS})
    lib = load_library()
    need = ctypes.c_size_t(0)
    _check(lib.dv_verify_workspace_bytes(ctypes.byref(d), ctypes.byref(n), None if t is None else ctypes.byref(t),
                                         ctypes.byref(need)), "dv_verify_workspace_bytes")
    if need.value and workspace is None:
        workspace = torch.empty(need.value + 256, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        base = workspace.data_ptr()
        off = (-base) % 256
        ws_ptr, ws_bytes = base + off, workspace.numel() * workspace.element_size() - off
    _check(lib.dv_verify_rows(ctypes.byref(d), ctypes.byref(n), None if t is None else ctypes.byref(t),
                              ctypes.byref(st), ws_ptr, ws_bytes, _stream_handle(dev)), "dv_verify_rows")
    res["_workspace"] = workspace  # keep the scratch alive until the caller drops the result
    return res


DV_NOALLOC_SCRATCH_BYTES = 8 << 20


def dv_verify_rows_noalloc(verifier, drafter, temperature=0.0, seed=0, pos=None, pos_period=0, *, vocab=None,
                           outputs=CORE_FIELDS, out=None, tuning=None, neg_inf=False):
    """dv_verify_rows without a workspace: the library's fixed per-device scratch holds the noise table (the
    C entry point allocates nothing; pass ``out`` to have this wrapper allocate nothing either)."""
    d = _logits_desc(verifier, drafter, vocab)
    d.flags = DV_LOGITS_NEG_INF if neg_inf else 0
    n = _noise_desc(temperature, seed, pos, pos_period, d.rows)
    t = _tuning_desc(tuning)
    rows, dev = d.rows, verifier.device
    res = {k: v for k, v in (out or {}).items() if not k.startswith("_")}
    for f in outputs:
        if f not in STAT_FIELDS:
            raise KeyError(f)
        if f not in res:
            res[f] = torch.empty(rows, dtype=torch.float32 if f in _FLOAT_FIELDS else torch.int32, device=dev)
    for f, v in res.items():
        _need_cuda(v, f)
        want = torch.float32 if f in _FLOAT_FIELDS else torch.int32
        if v.dtype != want or v.numel() < rows or not v.is_contiguous():
            raise TypeError(f"output {f} must be a contiguous {want} tensor of >= {rows} elements")
    st = dv_row_stats(**{f: (res[f].data_ptr() if f in res else None) for f in STAT_FIELDS})
    _check(load_library().dv_verify_rows_noalloc(ctypes.byref(d), ctypes.byref(n),
                                                 None if t is None else ctypes.byref(t), ctypes.byref(st),
                                                 _stream_handle(dev)), "dv_verify_rows_noalloc")
    return res


class VerifyPlan:
    """A dv_verify_rows call whose marshalling is done once: descriptors, output tensors and workspace are
    built at construction, and each call only points the descriptor at new logits of the same shape, dtype
    and row pitch (on the same device) and enters the library. For loops that verify batch after batch."""

    def __init__(self, verifier, drafter, temperature=0.0, seed=0, pos=None, pos_period=0, *, vocab=None,
                 outputs=CORE_FIELDS, tuning=None, neg_inf=False):
        self.out = dv_verify_rows(verifier, drafter, temperature, seed, pos, pos_period, vocab=vocab,
                                  outputs=outputs, tuning=tuning, neg_inf=neg_inf)
        self._desc = _logits_desc(verifier, drafter, vocab)
        self._desc.flags = DV_LOGITS_NEG_INF if neg_inf else 0
        self._noise = _noise_desc(temperature, seed, pos, pos_period, self._desc.rows)
        self._pos = pos                                   # kept alive with the plan
        self._tuning = _tuning_desc(tuning)
        self._stats = dv_row_stats(**{f: (self.out[f].data_ptr() if f in self.out else None) for f in STAT_FIELDS})
        ws = self.out.get("_workspace")
        self._ws_ptr, self._ws_bytes = None, 0
        if ws is not None:
            base = ws.data_ptr()
            off = (-base) % 256
            self._ws_ptr, self._ws_bytes = base + off, ws.numel() - off
        self._key = (tuple(verifier.shape), verifier.dtype, tuple(verifier.stride()), verifier.device)
        self._stream = _stream_handle(verifier.device)
        self._lib = load_library()
        self._args = (ctypes.byref(self._desc), ctypes.byref(self._noise),
                      None if self._tuning is None else ctypes.byref(self._tuning), ctypes.byref(self._stats),
                      self._ws_ptr, self._ws_bytes)

    def prepared(self, verifier, drafter) -> "Prepared":
        """The call on these logits with every argument marshalled (a descriptor of its own), to be repeated."""
        for t in (verifier, drafter):
            if (tuple(t.shape), t.dtype, tuple(t.stride()), t.device) != self._key:
                raise ValueError("logits differ in shape, dtype, pitch or device from the plan's")
        d = dv_logits.from_buffer_copy(self._desc)
        d.verifier, d.drafter = verifier.data_ptr(), drafter.data_ptr()
        return Prepared("dv_verify_rows", ctypes.byref(d), *self._args[1:], self._stream)

    def __call__(self, verifier, drafter):
        """Verify these logits (same shape, dtype, pitch and device as at construction) on the current stream;
        returns the plan's output dict (overwritten by each call)."""
        for t in (verifier, drafter):
            if (tuple(t.shape), t.dtype, tuple(t.stride()), t.device) != self._key:
                raise ValueError("logits differ in shape, dtype, pitch or device from the plan's")
        self._desc.verifier = verifier.data_ptr()
        self._desc.drafter = drafter.data_ptr()
        _check(self._lib.dv_verify_rows(*self._args, _stream_handle(verifier.device)), "dv_verify_rows")
        return self.out


class Prepared:
    """One library call with its arguments marshalled once (ctypes objects built from device pointers that
    stay valid), for loops that repeat the same call on the same buffers: each call only enters the library
    and checks the status."""

    def __init__(self, name: str, *args):
        self._fn = getattr(load_library(), name)
        self._name = name
        self._args = args

    def __call__(self):
        _check(self._fn(*self._args), self._name)


def prepare_seed_score(u, d_in, d_out, eligible, score) -> Prepared:
    """dv_seed_score on fixed buffers (float32 [rows] each, eligible uint8 [rows] or None)."""
    return Prepared("dv_seed_score", u.numel(), _ptr(u), _ptr(d_in), _ptr(d_out), _ptr(eligible), _ptr(score),
                    _stream_handle(u.device))


def prepare_select_topk(score, k, idx, val, cnt, *, eligible=None, mask=None, largest=True) -> Prepared:
    """dv_select_topk of score [nseq, L] into fixed buffers (no threshold)."""
    nseq, L = score.shape
    return Prepared("dv_select_topk", nseq, L, _ptr(score), _ptr(eligible), int(k), int(bool(largest)), 0, 0.0,
                    _ptr(idx), _ptr(val), _ptr(cnt), _ptr(mask), _stream_handle(score.device))


def prepare_seed_select(u, d_in, d_out, seed_eligible, score, k, idx, val, cnt, *, select_eligible=None, mask=None,
                        largest=True) -> Prepared:
    """dv_seed_select on fixed buffers: u, d_in, d_out, score [nseq, L] (no threshold)."""
    nseq, L = u.shape
    return Prepared("dv_seed_select", nseq, L, _ptr(u), _ptr(d_in), _ptr(d_out), _ptr(seed_eligible), _ptr(score),
                    _ptr(select_eligible), int(k), int(bool(largest)), 0, 0.0, _ptr(idx), _ptr(val), _ptr(cnt),
                    _ptr(mask), _stream_handle(u.device))


def prepare_decide_seed_select(decide: Prepared, seed_select: Prepared) -> Prepared:
    """A prepared dv_decide and a prepared dv_seed_select (same stream) as one dv_decide_seed_select call."""
    if decide._name != "dv_decide" or seed_select._name != "dv_seed_select":
        raise TypeError("expects a prepared dv_decide and a prepared dv_seed_select")
    if decide._args[-1] != seed_select._args[-1]:
        raise ValueError("the two calls must use one stream")
    return Prepared("dv_decide_seed_select", *decide._args[:-1], *seed_select._args[:-1], decide._args[-1])


def prepare_decide(rule, stats, decision, out_tok, *, rows, tau_kl=0.0, conf_thr=0.0, mask_token=-1, subject=None,
                   group_len=0, prefix=None, best=None) -> Prepared:
    """dv_decide on fixed buffers; ``stats`` maps dv_row_stats members to device tensors."""
    rule = RULES[rule] if isinstance(rule, str) else int(rule)
    args = dv_decide_args(rule=rule, tau_kl=float(tau_kl), conf_thr=float(conf_thr), mask_token=int(mask_token),
                          rows=int(rows), group_len=int(group_len), seed=0, pos=None, pos_period=0)
    st = dv_row_stats(**{f: (stats[f].data_ptr() if stats.get(f) is not None else None) for f in STAT_FIELDS})
    dev = decision.device
    return Prepared("dv_decide", ctypes.byref(args), ctypes.byref(st), _ptr(subject), None, _ptr(decision),
                    _ptr(out_tok), _ptr(prefix), _ptr(best), _stream_handle(dev))


def _decide_call(rule, stats, *, rows=None, tau_kl=0.0, conf_thr=0.0, mask_token=-1, subject=None, cur_tok=None,
                 group_len=0, want_prefix=False, want_best=False, seed=0, pos=None, pos_period=0):
    """dv_decide's C arguments (without the stream), the outputs they point to and the device."""
    rule = RULES[rule] if isinstance(rule, str) else int(rule)
    ref = next(v for k, v in stats.items() if k in STAT_FIELDS and v is not None)
    rows = ref.numel() if rows is None else int(rows)
    dev = ref.device
    for name, v in (("subject", subject), ("cur_tok", cur_tok), ("pos", pos)):
        if v is not None:
            _need_cuda(v, name)
    if pos is not None and (pos.dtype != torch.int32 or pos.numel() < rows or not pos.is_contiguous()):
        raise TypeError("pos must be a contiguous int32 tensor of >= rows elements")
    if subject is not None and subject.dtype != torch.uint8:
        raise TypeError("subject must be uint8")
    if cur_tok is not None and cur_tok.dtype != torch.int32:
        raise TypeError("cur_tok must be int32")
    decision = torch.empty(rows, dtype=torch.uint8, device=dev)
    out_tok = torch.empty(rows, dtype=torch.int32, device=dev)
    ngroups = rows // group_len if group_len > 0 else 0
    prefix = torch.empty(max(ngroups, 1), dtype=torch.int32, device=dev) if (want_prefix or want_best) else None
    best = torch.empty(1, dtype=torch.int32, device=dev) if want_best else None
    args = dv_decide_args(rule=rule, tau_kl=float(tau_kl), conf_thr=float(conf_thr), mask_token=int(mask_token),
                          rows=rows, group_len=int(group_len), seed=int(seed) & 0xFFFFFFFFFFFFFFFF,
                          pos=None if pos is None else pos.data_ptr(), pos_period=int(pos_period))
    st = dv_row_stats(**{f: (stats[f].data_ptr() if stats.get(f) is not None else None) for f in STAT_FIELDS})
    cargs = (ctypes.byref(args), ctypes.byref(st), _ptr(subject), _ptr(cur_tok), _ptr(decision), _ptr(out_tok),
             _ptr(prefix), _ptr(best))
    if prefix is not None:
        prefix = prefix[:ngroups]
    return cargs, (decision, out_tok, prefix, best), dev


def dv_decide(rule, stats, **kw):
    """Per-position decisions. ``stats`` is a dict with kl / conf / tok_v / tok_d
    tensors. Keywords: rows, tau_kl, conf_thr, mask_token, subject, cur_tok, group_len, want_prefix,
    want_best, seed, pos, pos_period. Returns (decision uint8, out_tok int32, prefix int32 or None,
    best int32[1] or None). seed, pos (int32 [rows]) and pos_period key the draws of KL_STOCHASTIC, as
    in dv_verify_rows."""
    cargs, outs, dev = _decide_call(rule, stats, **kw)
    _check(load_library().dv_decide(*cargs, _stream_handle(dev)), "dv_decide")
    return outs


def dv_seed_score(u, d_in, d_out, eligible=None, *, out=None):
    """COVER seed score u (1 + d_in) / (1 + d_out), -inf where not eligible."""
    for name, v in (("u", u), ("d_in", d_in), ("d_out", d_out)):
        _need_cuda(v, name)
        if v.dtype != torch.float32 or not v.is_contiguous():
            raise TypeError(f"{name} must be contiguous float32")
    rows = u.numel()
    if d_in.numel() != rows or d_out.numel() != rows:
        raise ValueError("u, d_in and d_out must have the same length")
    if eligible is not None:
        _need_cuda(eligible, "eligible")
        if eligible.dtype != torch.uint8:
            raise TypeError("eligible must be uint8")
    score = torch.empty(rows, dtype=torch.float32, device=u.device) if out is None else out
    _check(load_library().dv_seed_score(rows, _ptr(u), _ptr(d_in), _ptr(d_out), _ptr(eligible), _ptr(score),
                                        _stream_handle(u.device)), "dv_seed_score")
    return score


def dv_select_topk(score, k, *, eligible=None, largest=True, use_thr=False, thr=0.0, want_mask=False):
    """Per-sequence top-k of score [nseq, L]. Returns (idx, val, count, mask or None)."""
    _need_cuda(score, "score")
    if score.dim() != 2 or score.dtype != torch.float32 or not score.is_contiguous():
        raise TypeError("score must be a contiguous float32 [nseq, L] tensor")
    nseq, L = score.shape
    if eligible is not None:
        _need_cuda(eligible, "eligible")
        if eligible.dtype != torch.uint8 or eligible.shape != score.shape or not eligible.is_contiguous():
            raise TypeError("eligible must be contiguous uint8 shaped like score")
    dev = score.device
    kk = max(int(k), 1)
    idx = torch.empty((nseq, kk), dtype=torch.int32, device=dev)
    val = torch.empty((nseq, kk), dtype=torch.float32, device=dev)
    cnt = torch.empty(max(nseq, 1), dtype=torch.int32, device=dev)
    mask = torch.empty((nseq, L), dtype=torch.uint8, device=dev) if want_mask else None
    _check(load_library().dv_select_topk(nseq, L, _ptr(score), _ptr(eligible), int(k), int(bool(largest)),
                                         int(bool(use_thr)), float(thr), _ptr(idx), _ptr(val), _ptr(cnt),
                                         _ptr(mask), _stream_handle(dev)), "dv_select_topk")
    return idx, val, cnt[:nseq], mask


def _seed_select_call(u, d_in, d_out, k, *, seed_eligible=None, select_eligible=None, largest=True, use_thr=False,
                      thr=0.0, want_mask=False):
    """dv_seed_select's C arguments (without the stream), the outputs they point to and the device."""
    for name, v in (("u", u), ("d_in", d_in), ("d_out", d_out)):
        _need_cuda(v, name)
        if v.dtype != torch.float32 or not v.is_contiguous():
            raise TypeError(f"{name} must be contiguous float32")
    if u.dim() != 2:
        raise ValueError("u must be [nseq, L]")
    nseq, L = u.shape
    if d_in.numel() != u.numel() or d_out.numel() != u.numel():
        raise ValueError("u, d_in and d_out must have the same number of elements")
    for name, e in (("seed_eligible", seed_eligible), ("select_eligible", select_eligible)):
        if e is not None:
            _need_cuda(e, name)
            if e.dtype != torch.uint8 or e.numel() != u.numel() or not e.is_contiguous():
                raise TypeError(f"{name} must be contiguous uint8 with one entry per position")
    dev = u.device
    kk = max(int(k), 1)
    score = torch.empty((nseq, L), dtype=torch.float32, device=dev)
    idx = torch.empty((nseq, kk), dtype=torch.int32, device=dev)
    val = torch.empty((nseq, kk), dtype=torch.float32, device=dev)
    cnt = torch.empty(max(nseq, 1), dtype=torch.int32, device=dev)
    mask = torch.empty((nseq, L), dtype=torch.uint8, device=dev) if want_mask else None
    cargs = (nseq, L, _ptr(u), _ptr(d_in), _ptr(d_out), _ptr(seed_eligible), _ptr(score), _ptr(select_eligible),
             int(k), int(bool(largest)), int(bool(use_thr)), float(thr), _ptr(idx), _ptr(val), _ptr(cnt), _ptr(mask))
    return cargs, (score, idx, val, cnt[:nseq], mask), dev


def dv_seed_select(u, d_in, d_out, k, **kw):
    """COVER seed scores of u, d_in, d_out [nseq, L] and their per-sequence top-k in one call: the same outputs
    as dv_seed_score followed by dv_select_topk. Keywords: seed_eligible, select_eligible, largest, use_thr,
    thr, want_mask. Returns (score [nseq, L], idx, val, count, mask or None)."""
    cargs, outs, dev = _seed_select_call(u, d_in, d_out, k, **kw)
    _check(load_library().dv_seed_select(*cargs, _stream_handle(dev)), "dv_seed_select")
    return outs


def dv_seed_select_decide(seed_select: dict, decide: dict):
    """COVER's seed step: dv_seed_select, then dv_decide over the same rows with the selected seeds as its
    subject, in one launch up to 2048 positions per sequence. ``seed_select`` holds dv_seed_select's arguments
    by name (u, d_in, d_out, k and its keywords; the mask is always produced), ``decide`` dv_decide's (rule,
    stats, and tau_kl, conf_thr, mask_token, cur_tok, seed, pos, pos_period; no subject, group_len, prefix or
    best). Returns (dv_seed_select's outputs, (decision, out_tok))."""
    sargs, souts, dev = _seed_select_call(**{**seed_select, "want_mask": True})
    for key in ("subject", "group_len", "want_prefix", "want_best"):
        if decide.get(key):
            raise ValueError(f"the decisions over the selected seeds take no {key}")
    dargs, douts, ddev = _decide_call(**decide)
    if ddev != dev:
        raise ValueError("the selection and the decisions must be on one device")
    args, st, _subject, cur, decision, out_tok, _prefix, _best = dargs
    _check(load_library().dv_seed_select_decide(*sargs, args, st, cur, decision, out_tok, _stream_handle(dev)),
           "dv_seed_select_decide")
    return souts, douts[:2]


def prepare_seed_select_decide(seed_select: Prepared, decide: Prepared) -> Prepared:
    """A prepared dv_seed_select (with its mask) and a prepared dv_decide (no subject, prefix or best) as one
    dv_seed_select_decide call."""
    if seed_select._name != "dv_seed_select" or decide._name != "dv_decide":
        raise TypeError("expects a prepared dv_seed_select and a prepared dv_decide")
    if decide._args[-1] != seed_select._args[-1]:
        raise ValueError("the two calls must use one stream")
    a, st, subject, cur, decision, out_tok, prefix, best, stream = decide._args
    if subject is not None or prefix is not None or best is not None:
        raise ValueError("the decisions over the selected seeds take no subject, prefix or best")
    return Prepared("dv_seed_select_decide", *seed_select._args[:-1], a, st, cur, decision, out_tok, stream)


def dv_decide_seed_select(decide: dict, seed_select: dict):
    """dv_decide and dv_seed_select in one call (one launch where both fit it). ``decide`` holds dv_decide's
    arguments by name (rule, stats and its keywords), ``seed_select`` dv_seed_select's (u, d_in, d_out, k and
    its keywords). Returns (dv_decide's outputs, dv_seed_select's outputs)."""
    dargs, douts, dev = _decide_call(**decide)
    sargs, souts, sdev = _seed_select_call(**seed_select)
    if sdev != dev:
        raise ValueError("the decision and the selection must be on one device")
    _check(load_library().dv_decide_seed_select(*dargs, *sargs, _stream_handle(dev)), "dv_decide_seed_select")
    return douts, souts


def dv_tree_accept(parent, node_pos, node_tok, root_masked, conf, tok_v, *, block_tokens=None, update_mask=False):
    """Acceptance over trees of candidate block states (see dlmverify.h).

    parent, node_pos, node_tok: int32 [ntrees, nodes]; root_masked: uint8
    [ntrees, block_len]; conf (float32) and tok_v (int32): [ntrees, nodes,
    block_len] or the flat per-row statistics of those rows. block_tokens
    (int32 [ntrees, block_len]) is updated in place when given; with
    update_mask the committed positions of root_masked are cleared in place.
    Returns a dict: accepted, depth, best_node, commit_pos, commit_tok,
    commit_len.
    """
    for name, t, dt in (("parent", parent, torch.int32), ("node_pos", node_pos, torch.int32),
                        ("node_tok", node_tok, torch.int32), ("root_masked", root_masked, torch.uint8),
                        ("conf", conf, torch.float32), ("tok_v", tok_v, torch.int32)):
        _need_cuda(t, name)
        if t.dtype != dt or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous {dt} tensor")
    if parent.dim() != 2 or root_masked.dim() != 2:
        raise ValueError("parent must be [ntrees, nodes] and root_masked [ntrees, block_len]")
    ntrees, nodes = parent.shape
    L = root_masked.shape[1]
    if node_pos.shape != parent.shape or node_tok.shape != parent.shape or root_masked.shape[0] != ntrees:
        raise ValueError("node arrays and root_masked must agree on ntrees and nodes")
    if conf.numel() != ntrees * nodes * L or tok_v.numel() != ntrees * nodes * L:
        raise ValueError("conf and tok_v must hold ntrees * nodes * block_len entries")
    if block_tokens is not None:
        _need_cuda(block_tokens, "block_tokens")
        if block_tokens.dtype != torch.int32 or tuple(block_tokens.shape) != (ntrees, L) or not block_tokens.is_contiguous():
            raise TypeError("block_tokens must be a contiguous int32 [ntrees, block_len] tensor")
    dev = parent.device
    out = dict(accepted=torch.empty((ntrees, nodes), dtype=torch.uint8, device=dev),
               depth=torch.empty((ntrees, nodes), dtype=torch.int32, device=dev),
               best_node=torch.empty(ntrees, dtype=torch.int32, device=dev),
               commit_pos=torch.empty((ntrees, L), dtype=torch.int32, device=dev),
               commit_tok=torch.empty((ntrees, L), dtype=torch.int32, device=dev),
               commit_len=torch.empty(ntrees, dtype=torch.int32, device=dev))
    args = dv_tree_args(ntrees=ntrees, nodes=nodes, block_len=L)
    _check(load_library().dv_tree_accept(
        ctypes.byref(args), _ptr(parent), _ptr(node_pos), _ptr(node_tok), _ptr(root_masked), _ptr(conf), _ptr(tok_v),
        _ptr(out["accepted"]), _ptr(out["depth"]), _ptr(out["best_node"]), _ptr(out["commit_pos"]),
        _ptr(out["commit_tok"]), _ptr(out["commit_len"]), _ptr(block_tokens),
        _ptr(root_masked) if update_mask else None, _stream_handle(dev)), "dv_tree_accept")
    return out


def _attention_desc(probs):
    _need_cuda(probs, "probs")
    if probs.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("probs must be float32 or bfloat16")
    if probs.dim() != 4 or probs.shape[2] != probs.shape[3]:
        raise ValueError("probs must be [nseq, heads, len, len] (a view with a padded row pitch is fine)")
    B, H, L, _ = probs.shape
    if probs.stride(3) != 1 or probs.stride(1) != L * probs.stride(2) or probs.stride(0) != H * L * probs.stride(2):
        raise ValueError("probs rows must be contiguous and the maps packed ([nseq][heads][len][ld])")
    return dv_attention(probs=probs.data_ptr(), dtype=DV_BF16 if probs.dtype == torch.bfloat16 else DV_FP32,
                        reserved=0, nseq=B, heads=H, len=L, ld=probs.stride(2))


def dv_influence_drift_workspace_bytes(probs) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dv_influence_drift_workspace_bytes(ctypes.byref(_attention_desc(probs)), ctypes.byref(n)),
           "dv_influence_drift_workspace_bytes")
    return n.value


def dv_influence_drift(probs, query_masked, new_cols, *, workspace=None):
    """COVER's d_in and d_out ([nseq, len] float32 each) from attention probabilities
    [nseq, heads, len, len] and the masks query_masked, new_cols (uint8 [nseq, len])."""
    att = _attention_desc(probs)
    B, H, L, _ = probs.shape
    for name, t in (("query_masked", query_masked), ("new_cols", new_cols)):
        _need_cuda(t, name)
        if t.dtype != torch.uint8 or tuple(t.shape) != (B, L) or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous uint8 [nseq, len] tensor")
    dev = probs.device
    d_in = torch.empty((B, L), dtype=torch.float32, device=dev)
    d_out = torch.empty((B, L), dtype=torch.float32, device=dev)
    need = dv_influence_drift_workspace_bytes(probs)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    base = workspace.data_ptr()
    ws_ptr = (base + 255) // 256 * 256
    avail = workspace.numel() - (ws_ptr - base)
    _check(load_library().dv_influence_drift(ctypes.byref(att), _ptr(query_masked), _ptr(new_cols), _ptr(d_in),
                                             _ptr(d_out), ctypes.c_void_p(ws_ptr), avail, _stream_handle(dev)),
           "dv_influence_drift")
    return d_in, d_out


def prepare_influence_drift(probs, query_masked, new_cols, d_in, d_out, workspace) -> Prepared:
    """dv_influence_drift on fixed buffers (d_in, d_out float32 [nseq, len]; workspace uint8 of at least
    dv_influence_drift_workspace_bytes(probs) + 256 bytes), marshalled once."""
    att = _attention_desc(probs)
    B, H, L, _ = probs.shape
    for name, t, dt in (("query_masked", query_masked, torch.uint8), ("new_cols", new_cols, torch.uint8),
                        ("d_in", d_in, torch.float32), ("d_out", d_out, torch.float32)):
        _need_cuda(t, name)
        if t.dtype != dt or tuple(t.shape) != (B, L) or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous {dt} [nseq, len] tensor")
    base = workspace.data_ptr()
    ws_ptr = (base + 255) // 256 * 256
    avail = workspace.numel() - (ws_ptr - base)
    if avail < dv_influence_drift_workspace_bytes(probs):
        raise ValueError("workspace too small")
    call = Prepared("dv_influence_drift", ctypes.byref(att), _ptr(query_masked), _ptr(new_cols), _ptr(d_in),
                    _ptr(d_out), ctypes.c_void_p(ws_ptr), avail, _stream_handle(probs.device))
    call._keep = att  # the descriptor lives as long as the call
    return call


def dv_dual_view_attention(q, k_cur, v_cur, k_prev, v_prev, seed, *, scale=None, out=None):
    """COVER's dual-view attention. q: bf16 [nseq, heads, len, head_dim]; k_cur, v_cur, k_prev,
    v_prev: bf16 [nseq, kv_heads, len, head_dim]; seed: uint8 [nseq, len]. Returns float32
    [nseq, heads, len, head_dim]."""
    for name, t in (("q", q), ("k_cur", k_cur), ("v_cur", v_cur), ("k_prev", k_prev), ("v_prev", v_prev)):
        _need_cuda(t, name)
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bfloat16 [nseq, heads, len, head_dim] tensor")
    B, H, L, D = q.shape
    Hkv = k_cur.shape[1]
    for t in (k_cur, v_cur, k_prev, v_prev):
        if tuple(t.shape) != (B, Hkv, L, D):
            raise ValueError("k/v tensors must be [nseq, kv_heads, len, head_dim] like each other and q")
    _need_cuda(seed, "seed")
    if seed.dtype != torch.uint8 or tuple(seed.shape) != (B, L) or not seed.is_contiguous():
        raise TypeError("seed must be a contiguous uint8 [nseq, len] tensor")
    if out is None:
        out = torch.empty((B, H, L, D), dtype=torch.float32, device=q.device)
    args = dv_dual_view_args(nseq=B, heads=H, kv_heads=Hkv, len=L, head_dim=D,
                             scale=float(D ** -0.5 if scale is None else scale), reserved=0)
    _check(load_library().dv_dual_view_attention(
        ctypes.byref(args), _ptr(q), _ptr(k_cur), _ptr(v_cur), _ptr(k_prev), _ptr(v_prev), _ptr(seed), _ptr(out),
        _stream_handle(q.device)), "dv_dual_view_attention")
    return out


DV_DEBUG_INDEX_WORDS, DV_DEBUG_GROUP_WORDS, DV_DEBUG_NOISE_LOG2, DV_DEBUG_CHUNK_BOUND, DV_DEBUG_TABLE_BOUND = range(5)
DEBUG_NOISE_MODES = {"index_words": 0, "group_words": 1, "noise_log2": 2, "chunk_bound": 3, "table_bound": 4}


def dv_debug_hash(seed, rows, vocab, *, pos=None, pos_period=0, device="cuda"):
    """Noise hash words [rows, vocab] (returned as int32 tensor holding the uint32 bits)."""
    _check_pos(pos, rows)
    if pos is not None:
        device = pos.device
    out = torch.empty((rows, vocab), dtype=torch.int32, device=device)
    _check(load_library().dv_debug_hash(int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(pos), int(pos_period), int(rows),
                                        int(vocab), _ptr(out), _stream_handle(out.device)), "dv_debug_hash")
    return out


def dv_debug_noise(seed, rows, vocab, mode, *, chunk_elems=8, pos=None, pos_period=0, device="cuda"):
    """The shared noise as the kernels derive it (include/dlmverify.h, dv_debug_noise). mode: a name of
    DEBUG_NOISE_MODES. Words come back as int32 tensors holding the uint32 bits, values and bounds as float32:
    [rows, vocab] for index words and noise values, [rows, vocab // 8] for group words, [rows, chunks] for bounds."""
    m = DEBUG_NOISE_MODES[mode] if isinstance(mode, str) else int(mode)
    _check_pos(pos, rows)
    if pos is not None:
        device = pos.device
    nch = -(-int(vocab) // int(chunk_elems))
    width = {0: vocab, 1: vocab // 8, 2: vocab, 3: nch, 4: nch}.get(m, 0)
    dt = torch.int32 if m in (0, 1) else torch.float32
    out = torch.empty((rows, width), dtype=dt, device=device)
    _check(load_library().dv_debug_noise(int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(pos), int(pos_period), int(rows),
                                         int(vocab), m, int(chunk_elems), _ptr(out), _stream_handle(out.device)),
           "dv_debug_noise")
    return out


def dv_debug_read_probe(verifier, drafter, *, sink=None, tuning=None):
    """Read-only streaming probe over both logit matrices in dv_verify_rows's launch shape (measurement only).
    Returns the sink, int32 [rows, 16] holding the uint32 xor of what each wave read."""
    d = _logits_desc(verifier, drafter, None)
    t = _tuning_desc(tuning)
    if sink is None:
        sink = torch.empty((d.rows, 16), dtype=torch.int32, device=verifier.device)
    _check(load_library().dv_debug_read_probe(ctypes.byref(d), None if t is None else ctypes.byref(t), _ptr(sink),
                                              _stream_handle(verifier.device)), "dv_debug_read_probe")
    return sink
