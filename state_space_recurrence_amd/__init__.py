"""ReplaySSM decode step on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libreplayssm.so`` (the C ABI declared in
``include/replayssm.h``).  Every step of the decode path runs in the HIP
kernels of that library; this module only marshals torch tensors (device
memory) and the current HIP stream into the C calls.  There is no fallback:
if the library is missing or fails to load, every call raises.

Method: "NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer"
(devotd.net): per-sequence SSM state = interval checkpoint + buffer of recent
inputs; outputs replay the buffer; the checkpoint is rewritten once per
interval; speculative verify writes no state and rollback moves a position.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "F32", "BF16", "FP8_E4M3", "FP4_E2M1", "NONE", "ReplaySSMError", "lib", "LayerState",
    "step", "verify", "accept", "accept_deferred", "commit", "prefill", "load_checkpoint", "recurrent_step",
    "recurrent_verify", "recurrent_accept", "buffer_capacity", "check_device_errors",
]

F32, BF16, FP8_E4M3, FP4_E2M1, NONE = 0, 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libreplayssm.so")


class ReplaySSMError(RuntimeError):
    pass


class RssmDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("d_state", ctypes.c_int32), ("n_groups", ctypes.c_int32), ("interval", ctypes.c_int32),
        ("max_draft", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("ckpt_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("shared_lowp", ctypes.c_int32), ("layer_id", ctypes.c_int32),
        ("seed", ctypes.c_uint64), ("deferred_commit", ctypes.c_int32), ("n_slots", ctypes.c_int32),
    ]


class RssmState(ctypes.Structure):
    _fields_ = [
        ("ckpt", ctypes.c_void_p), ("out_q", ctypes.c_void_p), ("out_scale", ctypes.c_void_p),
        ("xbuf", ctypes.c_void_p), ("bbuf", ctypes.c_void_p), ("dtbuf", ctypes.c_void_p),
        ("pos", ctypes.c_void_p), ("intv", ctypes.c_void_p), ("work", ctypes.c_void_p),
        ("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("debug_prequant", ctypes.c_void_p),
        ("slot_idx", ctypes.c_void_p), ("commit_list", ctypes.c_void_p),
    ]


def commit_list_words(slots: int) -> int:
    """int32 words of a state's commit list for `slots` slots (RSSM_COMMIT_LIST_WORDS)."""
    return 32 + 4 * slots


_LIB = None
_vp = ctypes.c_void_p
_DP = ctypes.POINTER(RssmDesc)
_SP = ctypes.POINTER(RssmState)


def lib() -> ctypes.CDLL:
    """Load libreplayssm.so (raises ReplaySSMError if it is absent)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ReplaySSMError(
                f"{LIB_PATH} is missing: build it with `python -m state_space_recurrence_amd.build` "
                "(or __graft_entry__.build()); there is no non-HIP fallback")
        L = ctypes.CDLL(LIB_PATH)
        i32 = ctypes.c_int32
        L.replayssm_step.argtypes = [_DP, _SP, _vp, _vp, _vp, _vp, _vp, _vp]
        L.replayssm_step_noalloc.argtypes = [_DP, _SP, _vp, _vp, _vp, _vp, _vp, _vp]
        L.replayssm_verify.argtypes = [_DP, _SP, i32, _vp, _vp, _vp, _vp, _vp, _vp]
        L.replayssm_accept.argtypes = [_DP, _SP, _vp, i32, _vp]
        L.replayssm_accept_deferred.argtypes = [_DP, _SP, _vp, i32, _vp]
        L.replayssm_prefill.argtypes = [_DP, _SP, i32, i32, _vp, _vp, _vp, _vp, _vp, _vp]
        L.replayssm_commit.argtypes = [_DP, _SP, _vp]
        L.replayssm_load_checkpoint.argtypes = [_DP, _SP, _vp, _vp]
        L.replayssm_recurrent_step.argtypes = [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.replayssm_recurrent_verify.argtypes = [_DP, _vp, _vp, i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.replayssm_recurrent_accept.argtypes = [_DP, _vp, _vp, i32, _vp]
        L.replayssm_buffer_capacity.argtypes = [_DP]
        L.replayssm_buffer_capacity.restype = ctypes.c_size_t
        L.replayssm_check_desc.argtypes = [_DP]
        L.replayssm_status_string.argtypes = [ctypes.c_int]
        L.replayssm_status_string.restype = ctypes.c_char_p
        L.replayssm_last_error.argtypes = []
        L.replayssm_last_error.restype = ctypes.c_char_p
        L.replayssm_check_device_errors.argtypes = [_SP, i32, _vp]
        L.replayssm_version.restype = ctypes.c_char_p
        L.replayssm_hbm_probe.argtypes = [i32, _vp, _vp, ctypes.c_size_t, i32, _vp]
        L.replayssm_hbm_probe.restype = ctypes.c_int
        L.replayssm_check_conversions.argtypes = [ctypes.c_uint64, ctypes.c_uint64, _vp, _vp]
        L.replayssm_check_conversions.restype = ctypes.c_int
        for name in ("replayssm_step", "replayssm_step_noalloc", "replayssm_verify", "replayssm_accept", "replayssm_accept_deferred",
                     "replayssm_commit", "replayssm_prefill",
                     "replayssm_load_checkpoint", "replayssm_recurrent_step",
                     "replayssm_recurrent_verify", "replayssm_recurrent_accept",
                     "replayssm_check_desc", "replayssm_check_device_errors"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(rc: int) -> None:
    if rc != 0:
        L = lib()
        raise ReplaySSMError(f"{L.replayssm_status_string(rc).decode()} ({rc}): "
                             f"{L.replayssm_last_error().decode()}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


_IN_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


def _make_desc(batch, heads, head_dim, d_state, groups, interval, max_draft, in_dtype,
               ckpt_dtype=F32, out_dtype=NONE, shared_lowp=0, layer_id=0, seed=0,
               deferred_commit=0) -> RssmDesc:
    return RssmDesc(batch, heads, head_dim, d_state, groups, interval, max_draft,
                    _IN_DTYPES[in_dtype] if isinstance(in_dtype, torch.dtype) else int(in_dtype),
                    ckpt_dtype, out_dtype, shared_lowp, layer_id, seed, int(deferred_commit))


def buffer_capacity(interval: int, max_draft: int = 1) -> int:
    return interval + max_draft - 1


class LayerState:
    """Device state of one SSM layer for the replay path (caller-owned
    memory, allocated with torch on ``device``):

      ckpt [B,H,P,N] fp32 checkpoint;  xbuf [B,Lcap,H,P], bbuf [B,Lcap,G,N],
      dtbuf [B,Lcap,H] (input dtype);  pos, intv [B] int32;  work [B+1] int32;
      A, D [H] fp32.
    Snapshot / restore of the whole logical state is a copy of these tensors.
    """

    #: state formats: name -> (ckpt_dtype, out_dtype, shared_lowp)
    FORMATS = {
        "f32": (F32, NONE, 0),            # fp32 checkpoint (the article's performance setting)
        "split-bf16": (BF16, FP4_E2M1, 0),  # bf16 SR update checkpoint + FP4 output copy
        "split-e4m3": (FP8_E4M3, FP4_E2M1, 0),  # E4M3 SR update checkpoint + FP4 output copy
        "shared-fp4": (NONE, FP4_E2M1, 1),  # the FP4 copy is the only state (ablation)
        "low-bf16": (BF16, NONE, 0),      # one bf16 SR checkpoint for outputs and updates
        "low-e4m3": (FP8_E4M3, NONE, 0),  # one E4M3 SR checkpoint for outputs and updates
    }

    def __init__(self, batch: int, heads: int, groups: int, A: torch.Tensor, D: torch.Tensor, *,
                 head_dim: int = 64, d_state: int = 128, interval: int = 16, max_draft: int = 1,
                 in_dtype: torch.dtype = torch.bfloat16, device="cuda", layer_id: int = 0,
                 seed: int = 0, state_format: str = "f32", debug_prequant: bool = False,
                 deferred_commit: bool = False):
        self.batch, self.heads, self.groups = batch, heads, groups
        self.head_dim, self.d_state, self.interval, self.max_draft = head_dim, d_state, interval, max_draft
        self.in_dtype = in_dtype
        self.layer_id, self.seed = layer_id, seed
        self.lcap = buffer_capacity(interval, max_draft)
        self.state_format = state_format
        ck, od, sh = self.FORMATS[state_format]
        dev = torch.device(device)
        shape = (batch, heads, head_dim, d_state)
        ck_torch = {F32: torch.float32, BF16: torch.int16, FP8_E4M3: torch.uint8}
        self.ckpt = torch.zeros(shape, dtype=ck_torch[ck], device=dev) if ck != NONE else None
        if od == FP4_E2M1:
            self.out_q = torch.zeros(batch, heads, head_dim, d_state // 2, dtype=torch.uint8, device=dev)
            self.out_scale = torch.zeros(batch, heads, head_dim, d_state // 32, dtype=torch.uint8, device=dev)
        else:
            self.out_q = self.out_scale = None
        self.debug_prequant = torch.zeros(shape, dtype=torch.float32, device=dev) if debug_prequant else None
        self.xbuf = torch.zeros(batch, self.lcap, heads, head_dim, dtype=in_dtype, device=dev)
        self.bbuf = torch.zeros(batch, self.lcap, groups, d_state, dtype=in_dtype, device=dev)
        self.dtbuf = torch.zeros(batch, self.lcap, heads, dtype=in_dtype, device=dev)
        self.pos = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.intv = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.work = torch.zeros(batch + 1, dtype=torch.int32, device=dev)
        self.commit_list = torch.zeros(commit_list_words(batch), dtype=torch.int32, device=dev)
        if tuple(A.shape) != (heads,) or tuple(D.shape) != (heads,):
            raise ReplaySSMError(f"A and D must have shape ({heads},), got {tuple(A.shape)}, {tuple(D.shape)}")
        self.A = A.to(device=dev, dtype=torch.float32).contiguous()
        self.D = D.to(device=dev, dtype=torch.float32).contiguous()
        self._desc = _make_desc(batch, heads, head_dim, d_state, groups, interval, max_draft,
                                in_dtype, ckpt_dtype=ck, out_dtype=od, shared_lowp=sh,
                                layer_id=layer_id, seed=seed, deferred_commit=deferred_commit)
        _check(lib().replayssm_check_desc(ctypes.byref(self._desc)))

    def desc(self) -> RssmDesc:
        return self._desc

    def cstate(self) -> RssmState:
        return RssmState(_ptr(self.ckpt), _ptr(self.out_q), _ptr(self.out_scale), _ptr(self.xbuf),
                         _ptr(self.bbuf), _ptr(self.dtbuf), _ptr(self.pos), _ptr(self.intv),
                         _ptr(self.work), _ptr(self.A), _ptr(self.D), _ptr(self.debug_prequant),
                         None, _ptr(self.commit_list))

    def tensors(self):
        t = {"ckpt": self.ckpt, "out_q": self.out_q, "out_scale": self.out_scale, "xbuf": self.xbuf,
             "bbuf": self.bbuf, "dtbuf": self.dtbuf, "pos": self.pos, "intv": self.intv}
        return {k: v for k, v in t.items() if v is not None}

    def snapshot(self):
        return {k: v.clone() for k, v in self.tensors().items()}

    def restore(self, snap) -> None:
        for k, v in self.tensors().items():
            v.copy_(snap[k])


def _need(t: torch.Tensor, shape, dtype, name):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ReplaySSMError(f"{name}: expected contiguous device tensor {tuple(shape)} {dtype}, "
                             f"got {tuple(t.shape)} {t.dtype} contiguous={t.is_contiguous()} "
                             f"device={t.device}")


def _ctx(ls, slots):
    """Descriptor, state struct and row count of one call: every slot of the
    layer in order, or the rows of ``slots`` (int32 device tensor of slot
    indices, -1 = padding row)."""
    if slots is None:
        return ls._desc, ls.cstate(), ls.batch
    _need(slots, (slots.numel(),), torch.int32, "slots")
    d = RssmDesc.from_buffer_copy(ls._desc)
    d.batch = slots.numel()
    d.n_slots = ls.batch
    st = ls.cstate()
    st.slot_idx = slots.data_ptr()
    return d, st, d.batch


def _check_inputs(ls, x, B, C, dt, T=None, rows=None):
    rows = ls.batch if rows is None else rows
    lead = (rows,) if T is None else (rows, T)
    _need(x, lead + (ls.heads, ls.head_dim), ls.in_dtype, "x")
    _need(B, lead + (ls.groups, ls.d_state), ls.in_dtype, "B")
    _need(C, lead + (ls.groups, ls.d_state), ls.in_dtype, "C")
    _need(dt, lead + (ls.heads,), ls.in_dtype, "dt")


def step(ls: LayerState, x, B, C, dt, y=None, stream=None, slots=None) -> torch.Tensor:
    """One decode token per slot (replayssm_step): returns y [rows,H,P] fp32.
    ``slots``: optional int32 device tensor mapping call rows to state slots."""
    d, st, rows = _ctx(ls, slots)
    _check_inputs(ls, x, B, C, dt, rows=rows)
    if y is None:
        y = torch.empty(rows, ls.heads, ls.head_dim, dtype=torch.float32, device=x.device)
    _check(lib().replayssm_step(ctypes.byref(d), ctypes.byref(st), _ptr(x), _ptr(B), _ptr(C),
                                _ptr(dt), _ptr(y), _stream(stream)))
    return y


def step_noalloc(ls: LayerState, x, B, C, dt, y=None, stream=None, slots=None) -> torch.Tensor:
    """replayssm_step_noalloc: the same step with the per-slot arrival
    counters in library scratch (nothing allocated; `y` must be given by
    callers that cannot allocate)."""
    d, st, rows = _ctx(ls, slots)
    _check_inputs(ls, x, B, C, dt, rows=rows)
    if y is None:
        y = torch.empty(rows, ls.heads, ls.head_dim, dtype=torch.float32, device=x.device)
    _check(lib().replayssm_step_noalloc(ctypes.byref(d), ctypes.byref(st), _ptr(x), _ptr(B), _ptr(C),
                                        _ptr(dt), _ptr(y), _stream(stream)))
    return y


def verify(ls: LayerState, x, B, C, dt, y=None, stream=None, slots=None) -> torch.Tensor:
    """Speculative verify of T positions (replayssm_verify): x [rows,T,H,P] etc.;
    returns y [rows,T,H,P] fp32.  No state is written; pos is unchanged."""
    d, st, rows = _ctx(ls, slots)
    T = x.shape[1]
    _check_inputs(ls, x, B, C, dt, T, rows=rows)
    if y is None:
        y = torch.empty(rows, T, ls.heads, ls.head_dim, dtype=torch.float32, device=x.device)
    _check(lib().replayssm_verify(ctypes.byref(d), ctypes.byref(st), T, _ptr(x), _ptr(B),
                                  _ptr(C), _ptr(dt), _ptr(y), _stream(stream)))
    return y


def accept(ls: LayerState, n_keep: torch.Tensor, T: int, stream=None, slots=None) -> None:
    """Keep the first n_keep[row] verified positions (replayssm_accept)."""
    d, st, rows = _ctx(ls, slots)
    _need(n_keep, (rows,), torch.int32, "n_keep")
    _check(lib().replayssm_accept(ctypes.byref(d), ctypes.byref(st), _ptr(n_keep), T, _stream(stream)))


def accept_deferred(ls: LayerState, n_keep: torch.Tensor, T: int, stream=None, slots=None) -> None:
    """Keep the first n_keep[row] verified positions without committing: slots
    reaching the interval length are folded by their next step / verify /
    commit (replayssm_accept_deferred; fp32 checkpoints)."""
    d, st, rows = _ctx(ls, slots)
    _need(n_keep, (rows,), torch.int32, "n_keep")
    _check(lib().replayssm_accept_deferred(ctypes.byref(d), ctypes.byref(st), _ptr(n_keep), T,
                                           _stream(stream)))


def commit(ls: LayerState, stream=None, slots=None) -> None:
    """Flush buffered tokens into the checkpoint (replayssm_commit): every
    slot, or the slots listed in ``slots`` (eviction = flush + copy out)."""
    d, st, _ = _ctx(ls, slots)
    _check(lib().replayssm_commit(ctypes.byref(d), ctypes.byref(st), _stream(stream)))


def prefill(ls: LayerState, x: torch.Tensor, B: torch.Tensor, C: torch.Tensor | None, dt: torch.Tensor, *,
            from_zero: bool = False, outputs: bool = True, y: torch.Tensor | None = None,
            stream=None, slots=None) -> torch.Tensor | None:
    """Run a prompt of Tp tokens per row into the checkpoint (replayssm_prefill):
    x [rows,Tp,H,P], B/C [rows,Tp,G,N], dt [rows,Tp,H]; returns y [rows,Tp,H,P]
    fp32 when ``outputs`` (else None)."""
    d, st, rows = _ctx(ls, slots)
    Tp = x.shape[1] if x.dim() == 4 else 0
    _need(x, (rows, Tp, ls.heads, ls.head_dim), ls.in_dtype, "x")
    _need(B, (rows, Tp, ls.groups, ls.d_state), ls.in_dtype, "B")
    _need(dt, (rows, Tp, ls.heads), ls.in_dtype, "dt")
    if outputs:
        _need(C, (rows, Tp, ls.groups, ls.d_state), ls.in_dtype, "C")
        if y is None:
            y = torch.empty(rows, Tp, ls.heads, ls.head_dim, dtype=torch.float32, device=x.device)
        _need(y, (rows, Tp, ls.heads, ls.head_dim), torch.float32, "y")
    else:
        y = None
    _check(lib().replayssm_prefill(ctypes.byref(d), ctypes.byref(st), Tp, int(from_zero), _ptr(x),
                                   _ptr(B), _ptr(C), _ptr(dt), _ptr(y), _stream(stream)))
    return y


def load_checkpoint(ls: LayerState, src: torch.Tensor, stream=None, slots=None) -> None:
    """Set checkpoints from an fp32 state [rows,H,P,N] and reset their positions
    (quantising into the layer's state format; the rounding stream index is
    the slot's current intv).  With ``slots``, row r goes to slot slots[r]
    (admission into a slot pool)."""
    d, st, rows = _ctx(ls, slots)
    _need(src, (rows, ls.heads, ls.head_dim, ls.d_state), torch.float32, "src")
    _check(lib().replayssm_load_checkpoint(ctypes.byref(d), ctypes.byref(st), _ptr(src), _stream(stream)))


def hbm_probe(mode: int, src: torch.Tensor, dst: torch.Tensor, grid: int, stream=None) -> None:
    """Launch the library's HBM streaming probe (0 = read src, 1 = copy src to dst)."""
    _check(lib().replayssm_hbm_probe(mode, _ptr(src), _ptr(dst), src.numel() * src.element_size(), grid,
                                     _stream(stream)))


def check_conversions(begin: int = 0, end: int = 1 << 32, stream=None) -> tuple:
    """Run the device conversion self-check over fp32 bit patterns
    [begin, end); returns (FP4 conversion mismatches, bf16 rounding
    mismatches, E4M3 rounding mismatches) -- all 0 on a conforming device."""
    counts = torch.zeros(3, dtype=torch.int64, device="cuda")
    _check(lib().replayssm_check_conversions(begin, end, _ptr(counts), _stream(stream)))
    return tuple(int(c) for c in counts.cpu())


def check_device_errors(ls: LayerState, stream=None) -> None:
    st = ls.cstate()
    _check(lib().replayssm_check_device_errors(ctypes.byref(st), ls.batch, _stream(stream)))


def recurrent_step(state, x, B, C, dt, A, D, *, groups: int, y=None, stream=None,
                   max_draft: int = 1) -> torch.Tensor:
    """Conventional per-token update in place (replayssm_recurrent_step)."""
    batch, heads, P, N = state.shape
    _need(state, (batch, heads, P, N), torch.float32, "state")
    _need(x, (batch, heads, P), x.dtype, "x")
    _need(B, (batch, groups, N), x.dtype, "B")
    _need(C, (batch, groups, N), x.dtype, "C")
    _need(dt, (batch, heads), x.dtype, "dt")
    _need(A, (heads,), torch.float32, "A")
    _need(D, (heads,), torch.float32, "D")
    desc = _make_desc(batch, heads, P, N, groups, 1, max_draft, x.dtype)
    if y is None:
        y = torch.empty(batch, heads, P, dtype=torch.float32, device=x.device)
    _check(lib().replayssm_recurrent_step(ctypes.byref(desc), _ptr(state), _ptr(x), _ptr(B), _ptr(C),
                                          _ptr(dt), _ptr(A), _ptr(D), _ptr(y), _stream(stream)))
    return y


def recurrent_verify(pool, sel, x, B, C, dt, A, D, *, groups: int, y=None, stream=None) -> torch.Tensor:
    """Conventional speculative verify with per-token state copies
    (replayssm_recurrent_verify).  pool [B, Tmax+1, H, P, N]; sel [B]."""
    batch, slots, heads, P, N = pool.shape
    T = x.shape[1]
    _need(pool, (batch, slots, heads, P, N), torch.float32, "pool")
    _need(sel, (batch,), torch.int32, "sel")
    _need(x, (batch, T, heads, P), x.dtype, "x")
    _need(B, (batch, T, groups, N), x.dtype, "B")
    _need(C, (batch, T, groups, N), x.dtype, "C")
    _need(dt, (batch, T, heads), x.dtype, "dt")
    _need(A, (heads,), torch.float32, "A")
    _need(D, (heads,), torch.float32, "D")
    desc = _make_desc(batch, heads, P, N, groups, 1, slots - 1, x.dtype)
    if y is None:
        y = torch.empty(batch, T, heads, P, dtype=torch.float32, device=x.device)
    _check(lib().replayssm_recurrent_verify(ctypes.byref(desc), _ptr(pool), _ptr(sel), T, _ptr(x),
                                            _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D), _ptr(y),
                                            _stream(stream)))
    return y


def recurrent_accept(pool_slots: int, sel, n_keep, T: int, *, heads: int = 1, groups: int = 1,
                     stream=None) -> None:
    """Baseline accept: select the kept per-token state copy."""
    batch = sel.shape[0]
    _need(sel, (batch,), torch.int32, "sel")
    _need(n_keep, (batch,), torch.int32, "n_keep")
    desc = _make_desc(batch, heads, 64, 128, groups, 1, pool_slots - 1, torch.float32)
    _check(lib().replayssm_recurrent_accept(ctypes.byref(desc), _ptr(sel), _ptr(n_keep), T,
                                            _stream(stream)))
