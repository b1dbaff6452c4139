"""Python binding of the LoGRA hot path: torch tensors -> liblogra C ABI.

Argument marshalling only: every step of the path runs in the library's HIP
kernels on the tensors' device, asynchronously on torch's current stream.
Tensors must live on the GPU; nothing here falls back to the CPU.

Names follow the pages' notation: X (T x k inputs), dY (T x d output
gradients), S (d x r fp32 sketch), W (d x k bf16 weights), A (r x k
projection), q and alpha of the predicted-KL controller.
"""
import ctypes

import torch

from . import _lib

RADEMACHER = 0
GAUSSIAN = 1
SKETCH_OVERWRITE = 1      # LOGRA_SKETCH_OVERWRITE: S = ... instead of S += ...
SKETCH_DEFER = 2          # LOGRA_SKETCH_DEFER: keep the contribution in the workspace
SKETCH_PENDING = 4        # LOGRA_SKETCH_PENDING: the workspace holds deferred contributions


def _sketch_flags(overwrite, defer, pending):
    return ((SKETCH_OVERWRITE if overwrite else 0) | (SKETCH_DEFER if defer else 0) |
            (SKETCH_PENDING if pending else 0))


# torch's raw current-stream lookup costs well under a microsecond per call; the
# public torch.cuda.current_stream(device) builds a Stream object (a few us,
# a quarter of a sketch call's host time at small sizes)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    if _raw_stream is not None:
        return _raw_stream(t.device.index if t.device.index is not None
                           else torch.cuda.current_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")


def _ws(ws, name="ws"):
    """(device address, bytes) of a caller's workspace: a contiguous GPU tensor
    (a host tensor's address would reach the kernels)."""
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if ws.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {ws.device})")
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _rows(t, name):
    """(rows, cols, row stride) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    rows, cols = t.shape
    # a single row has no meaningful stride; any legal value reads the same bytes
    ld = t.stride(0) if rows > 1 else -(-cols // 8) * 8
    return rows, cols, ld


CHOICE_PROJECT_TILE = 0   # LOGRA_CHOICE_PROJECT_TILE
CHOICE_ACC_WIDE = 1       # LOGRA_CHOICE_ACC_WIDE
CHOICE_AUTO = -1          # LOGRA_CHOICE_AUTO


def set_kernel_choice(which, mode):
    """Force (mode 0 never, 1 always) or release (CHOICE_AUTO) one of the
    sketch's equivalent kernels, process-wide; for tests and measurements."""
    _lib.check(_lib.lib().logra_set_kernel_choice(int(which), int(mode)),
               "logra_set_kernel_choice")


class kernel_choice:
    """Context manager: set_kernel_choice(which, mode) inside, automatic after."""

    def __init__(self, which, mode):
        self.which, self.mode = which, mode

    def __enter__(self):
        set_kernel_choice(self.which, self.mode)
        return self

    def __exit__(self, *exc):
        set_kernel_choice(self.which, CHOICE_AUTO)
        return False


def regen_A(seed, stream, kind, r, k, device="cuda", out=None):
    """A (r x k fp32) exactly as the sketch and merge kernels regenerate it."""
    if out is None:
        out = torch.empty((r, k), dtype=torch.float32, device=device)
    _require(out, "out", torch.float32, 2)
    if not out.is_contiguous() or tuple(out.shape) != (r, k):
        raise ValueError("out must be a contiguous (r, k) float32 tensor")
    st = _lib.lib().logra_regen_A(seed, stream, kind, r, k, out.data_ptr(), _stream(out))
    _lib.check(st, "logra_regen_A")
    return out


def sketch_ws_bytes(T, d, k, r):
    return int(_lib.lib().logra_sketch_ws_bytes(T, d, k, r))


def sketch_workspace(T, d, k, r, device="cuda"):
    """A workspace tensor large enough for sketch_accumulate at these sizes."""
    n = sketch_ws_bytes(T, d, k, r)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def sketch_accumulate(X, dY, S, seed, stream=0, kind=RADEMACHER, ws=None, overwrite=False,
                      defer=False, pending=False):
    """S += dY^T (X A^T) in place for one microbatch; returns S.  With
    overwrite=True (the first microbatch of a step) S = dY^T (X A^T) and S's
    previous contents are ignored.  defer/pending build a deferred chain over
    the microbatches of a step (same ws and sizes throughout): defer keeps the
    contribution in ws and leaves S alone, pending adds the contributions ws
    holds; the last call (pending, not defer) writes S."""
    _require(X, "X", torch.bfloat16, 2)
    _require(dY, "dY", torch.bfloat16, 2)
    _require(S, "S", torch.float32, 2)
    T, k, ldx = _rows(X, "X")
    T2, d, ldd = _rows(dY, "dY")
    if T2 != T:
        raise ValueError(f"X has {T} rows but dY has {T2}")
    if S.shape[0] != d or not S.is_contiguous():
        raise ValueError("S must be a contiguous (d, r) float32 tensor")
    r = S.shape[1]
    if ws is None:
        ws = sketch_workspace(T, d, k, r, X.device)
    st = _lib.lib().logra_sketch_accumulate(
        X.data_ptr(), ldx, dY.data_ptr(), ldd, T, d, k, r, seed, stream, kind,
        _sketch_flags(overwrite, defer, pending), S.data_ptr(), *_ws(ws), _stream(X))
    _lib.check(st, "logra_sketch_accumulate")
    return S


MAX_SHARED = _lib.MAX_SHARED


def sketch_shared_ws_bytes(T, k, r, ds):
    ds = [int(x) for x in ds]
    arr = (ctypes.c_int64 * max(1, len(ds)))(*ds)
    return int(_lib.lib().logra_sketch_shared_ws_bytes(T, k, r, len(ds), arr))


def sketch_accumulate_shared(X, dYs, Ss, seed, stream=0, kind=RADEMACHER, ws=None,
                             overwrite=False, defer=False, pending=False):
    """S_o += dY_o^T (X A^T) in place for outputs sharing the input X and A
    (e.g. q/k/v or gate/up of one layer); returns the list of S.  overwrite,
    defer and pending as in sketch_accumulate, for every S_o."""
    _require(X, "X", torch.bfloat16, 2)
    T, k, ldx = _rows(X, "X")
    if not 1 <= len(dYs) <= MAX_SHARED or len(dYs) != len(Ss):
        raise ValueError(f"between 1 and {MAX_SHARED} (dY, S) pairs")
    ptr_dy, ldds, ds, ptr_s = [], [], [], []
    r = None
    for dY, S in zip(dYs, Ss):
        _require(dY, "dY", torch.bfloat16, 2)
        _require(S, "S", torch.float32, 2)
        T2, d, ldd = _rows(dY, "dY")
        if T2 != T:
            raise ValueError(f"X has {T} rows but a dY has {T2}")
        if S.shape[0] != d or not S.is_contiguous():
            raise ValueError("each S must be a contiguous (d, r) float32 tensor")
        if r is not None and S.shape[1] != r:
            raise ValueError("every S must have the same rank r")
        r = S.shape[1]
        ptr_dy.append(dY.data_ptr())
        ldds.append(ldd)
        ds.append(d)
        ptr_s.append(S.data_ptr())
    n = len(dYs)
    if ws is None:
        ws = torch.empty(max(sketch_shared_ws_bytes(T, k, r, ds), 256), dtype=torch.uint8,
                         device=X.device)
    st = _lib.lib().logra_sketch_accumulate_shared(
        X.data_ptr(), ldx, T, k, r, seed, stream, kind, _sketch_flags(overwrite, defer, pending), n,
        (ctypes.c_void_p * n)(*ptr_dy),
        (ctypes.c_int64 * n)(*ldds), (ctypes.c_int64 * n)(*ds), (ctypes.c_void_p * n)(*ptr_s),
        *_ws(ws), _stream(X))
    _lib.check(st, "logra_sketch_accumulate_shared")
    return list(Ss)


def sketch_p_bytes(T, r):
    return int(_lib.lib().logra_sketch_p_bytes(T, r))


def sketch_project_ws_bytes(k, r):
    return int(_lib.lib().logra_sketch_project_ws_bytes(k, r))


def sketch_project(X, seed, r, stream=0, kind=RADEMACHER, P=None, ws=None):
    """P = X A^T for one microbatch (the first half of sketch_accumulate), in
    the tiled bf16 hi/lo layout of include/logra.h, into a uint8 device tensor
    of sketch_p_bytes(T, r) bytes (allocated when P is None); returns P.  ws:
    scratch for the Gaussian basis (allocated when needed and None)."""
    _require(X, "X", torch.bfloat16, 2)
    T, k, ldx = _rows(X, "X")
    need = sketch_p_bytes(T, r)
    if P is None:
        P = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)
    _require(P, "P", torch.uint8, 1)
    if not P.is_contiguous():
        raise ValueError("P must be a contiguous uint8 buffer")
    if kind == GAUSSIAN and ws is None:
        ws = torch.empty(max(sketch_project_ws_bytes(k, r), 256), dtype=torch.uint8,
                         device=X.device)
    ws_ptr, ws_n = _ws(ws) if ws is not None else (None, 0)
    st = _lib.lib().logra_sketch_project(X.data_ptr(), ldx, T, k, r, seed, stream, kind,
                                         P.data_ptr(), P.numel(), ws_ptr, ws_n, _stream(X))
    _lib.check(st, "logra_sketch_project")
    return P


def sketch_accumulate_p_ws_bytes(T, r, ds):
    ds = [int(x) for x in ds]
    arr = (ctypes.c_int64 * max(1, len(ds)))(*ds)
    return int(_lib.lib().logra_sketch_accumulate_p_ws_bytes(T, r, len(ds), arr))


def sketch_accumulate_p(P, dYs, Ss, ws=None, overwrite=False, defer=False, pending=False):
    """S_o += dY_o^T P in place (the second half of sketch_accumulate, or of
    sketch_accumulate_shared with several outputs) from a P of sketch_project
    with the same T and r; returns the list of S.  overwrite, defer and
    pending as in sketch_accumulate; a deferred chain keeps ws and the
    outputs and may take a different P in every call."""
    _require(P, "P", torch.uint8, 1)
    if not P.is_contiguous():
        raise ValueError("P must be a contiguous uint8 buffer")
    if isinstance(dYs, torch.Tensor):
        dYs, Ss = [dYs], [Ss]
    if not 1 <= len(dYs) <= MAX_SHARED or len(dYs) != len(Ss):
        raise ValueError(f"between 1 and {MAX_SHARED} (dY, S) pairs")
    ptr_dy, ldds, ds, ptr_s = [], [], [], []
    T = r = None
    for dY, S in zip(dYs, Ss):
        _require(dY, "dY", torch.bfloat16, 2)
        _require(S, "S", torch.float32, 2)
        T2, d, ldd = _rows(dY, "dY")
        if T is not None and T2 != T:
            raise ValueError("every dY must have the same number of rows")
        T = T2
        if S.shape[0] != d or not S.is_contiguous():
            raise ValueError("each S must be a contiguous (d, r) float32 tensor")
        if r is not None and S.shape[1] != r:
            raise ValueError("every S must have the same rank r")
        r = S.shape[1]
        ptr_dy.append(dY.data_ptr())
        ldds.append(ldd)
        ds.append(d)
        ptr_s.append(S.data_ptr())
    n = len(dYs)
    if ws is None:
        ws = torch.empty(max(sketch_accumulate_p_ws_bytes(T, r, ds), 256), dtype=torch.uint8,
                         device=P.device)
    st = _lib.lib().logra_sketch_accumulate_p(
        P.data_ptr(), P.numel(), T, r, _sketch_flags(overwrite, defer, pending), n,
        (ctypes.c_void_p * n)(*ptr_dy), (ctypes.c_int64 * n)(*ldds), (ctypes.c_int64 * n)(*ds),
        (ctypes.c_void_p * n)(*ptr_s), *_ws(ws), _stream(P))
    _lib.check(st, "logra_sketch_accumulate_p")
    return list(Ss)


MAX_GROUPS = _lib.MAX_GROUPS
MAX_LAYER_OUT = _lib.MAX_LAYER_OUT


def _group_array(groups):
    """ctypes array of logra_sketch_group from [(X, dYs, Ss, seed, stream)];
    also returns T and r (checked equal across groups)."""
    if not 1 <= len(groups) <= MAX_GROUPS:
        raise ValueError(f"between 1 and {MAX_GROUPS} input groups")
    arr = (_lib.SketchGroup * len(groups))()
    T = r = None
    n_out = 0
    for g, (X, dYs, Ss, seed, stream) in enumerate(groups):
        _require(X, "X", torch.bfloat16, 2)
        Tg, k, ldx = _rows(X, "X")
        if T is not None and Tg != T:
            raise ValueError("every group's X must have the same number of rows")
        T = Tg
        if not 1 <= len(dYs) <= MAX_SHARED or len(dYs) != len(Ss):
            raise ValueError(f"between 1 and {MAX_SHARED} (dY, S) pairs per group")
        n_out += len(dYs)
        q = arr[g]
        q.X, q.ldx, q.k, q.seed, q.stream, q.n_out = X.data_ptr(), ldx, k, seed, stream, len(dYs)
        for o, (dY, S) in enumerate(zip(dYs, Ss)):
            _require(dY, "dY", torch.bfloat16, 2)
            _require(S, "S", torch.float32, 2)
            T2, d, ldd = _rows(dY, "dY")
            if T2 != T:
                raise ValueError(f"X has {T} rows but a dY has {T2}")
            if S.shape[0] != d or not S.is_contiguous():
                raise ValueError("each S must be a contiguous (d, r) float32 tensor")
            if r is not None and S.shape[1] != r:
                raise ValueError("every S must have the same rank r")
            r = S.shape[1]
            q.dY[o], q.ldd[o], q.d[o], q.S[o] = dY.data_ptr(), ldd, d, S.data_ptr()
    if n_out > MAX_LAYER_OUT:
        raise ValueError(f"at most {MAX_LAYER_OUT} outputs in all")
    return arr, T, r


def sketch_layer_ws_bytes(T, r, groups):
    """Workspace bytes of sketch_accumulate_layer; groups: [(k, [d, ...])]."""
    arr = (_lib.SketchGroup * max(1, len(groups)))()
    for g, (k, ds) in enumerate(groups):
        arr[g].k, arr[g].n_out = int(k), len(ds)
        for o, d in enumerate(ds):
            arr[g].d[o] = int(d)
    return int(_lib.lib().logra_sketch_layer_ws_bytes(T, r, len(groups), arr))


def sketch_layer_workspace(T, r, groups, device="cuda"):
    """A workspace tensor for sketch_accumulate_layer; groups: [(k, [d, ...])]."""
    return torch.empty(max(sketch_layer_ws_bytes(T, r, groups), 256), dtype=torch.uint8,
                       device=device)


def sketch_accumulate_layer(groups, kind=RADEMACHER, ws=None, overwrite=False, defer=False,
                            pending=False):
    """The sketches of a layer set for one microbatch in one projection and one
    accumulate launch.  groups: up to 4 entries (X, dYs, Ss, seed, stream), each
    an input X shared by its outputs (dY_o, S_o), up to 8 outputs in all:
    S_o += dY_o^T (X A^T).  overwrite, defer and pending as in
    sketch_accumulate, for every S_o; returns None."""
    arr, T, r = _group_array(groups)
    X0 = groups[0][0]
    if ws is None:
        ws = sketch_layer_workspace(T, r, [(g[0].shape[1], [dy.shape[1] for dy in g[1]])
                                           for g in groups], X0.device)
    st = _lib.lib().logra_sketch_accumulate_layer(
        T, r, kind, _sketch_flags(overwrite, defer, pending), len(groups), arr, *_ws(ws),
        _stream(X0))
    _lib.check(st, "logra_sketch_accumulate_layer")


MAX_MERGE = _lib.MAX_MERGE


def merge_many(items, kind=RADEMACHER, alpha=1.0, eta=1.0):
    """merge for up to 8 weights in one launch; items: [(W, S, seed, stream)],
    every S of the same rank.  Bit-identical to one merge call per item."""
    if not 1 <= len(items) <= MAX_MERGE:
        raise ValueError(f"between 1 and {MAX_MERGE} weights")
    arr = (_lib.MergeItem * len(items))()
    r = None
    for i, (W, S, seed, stream) in enumerate(items):
        _require(W, "W", torch.bfloat16, 2)
        _require(S, "S", torch.float32, 2)
        d, k, ldw = _rows(W, "W")
        if S.shape[0] != d or not S.is_contiguous():
            raise ValueError("each S must be a contiguous (d, r) float32 tensor")
        if r is not None and S.shape[1] != r:
            raise ValueError("every S must have the same rank r")
        r = S.shape[1]
        arr[i].W, arr[i].ldw, arr[i].S, arr[i].d, arr[i].k = W.data_ptr(), ldw, S.data_ptr(), d, k
        arr[i].seed, arr[i].stream = seed, stream
    st = _lib.lib().logra_merge_many(len(items), arr, r, kind, float(alpha), float(eta),
                                     _stream(items[0][0]))
    _lib.check(st, "logra_merge_many")


def merge(W, S, seed, stream=0, kind=RADEMACHER, alpha=1.0, eta=1.0):
    """W <- RNE_bf16(W - alpha * eta * S A) in place; returns W."""
    _require(W, "W", torch.bfloat16, 2)
    _require(S, "S", torch.float32, 2)
    d, k, ldw = _rows(W, "W")
    if S.shape[0] != d or not S.is_contiguous():
        raise ValueError("S must be a contiguous (d, r) float32 tensor")
    r = S.shape[1]
    st = _lib.lib().logra_merge(W.data_ptr(), ldw, S.data_ptr(), d, k, r, seed, stream,
                                kind, float(alpha), float(eta), _stream(W))
    _lib.check(st, "logra_merge")
    return W


UPDATE_SGD = 0
UPDATE_MOMENTUM = 1
UPDATE_ADAM = 2


def sketch_update(rule, S, U=None, m=None, v=None, beta1=0.9, beta2=0.999, eps=1e-8, step=1):
    """U from the sketch S and the sketch-space optimizer state (m, v updated in
    place): UPDATE_SGD U = S; UPDATE_MOMENTUM m <- beta1 m + S, U = m;
    UPDATE_ADAM bias-corrected Adam on S.  U defaults to a new tensor; returns U."""
    _require(S, "S", torch.float32, 2)
    if not S.is_contiguous():
        raise ValueError("S must be a contiguous (d, r) float32 tensor")
    d, r = S.shape
    if U is None:
        U = torch.empty_like(S)
    ptrs = []
    for name, t, need in (("U", U, True), ("m", m, rule in (UPDATE_MOMENTUM, UPDATE_ADAM)),
                          ("v", v, rule == UPDATE_ADAM)):
        if t is None:
            if need:
                raise ValueError(f"rule {rule} needs the state tensor {name}")
            ptrs.append(None)
            continue
        _require(t, name, torch.float32, 2)
        if tuple(t.shape) != (d, r) or not t.is_contiguous() or t.device != S.device:
            raise ValueError(f"{name} must be a contiguous ({d}, {r}) float32 tensor on {S.device}")
        ptrs.append(t.data_ptr())
    st = _lib.lib().logra_sketch_update(rule, S.data_ptr(), ptrs[1], ptrs[2], ptrs[0], d, r,
                                        float(beta1), float(beta2), float(eps), int(step),
                                        _stream(S))
    _lib.check(st, "logra_sketch_update")
    return U


def kl_ws_bytes(n_tok, vocab):
    return int(_lib.lib().logra_kl_ws_bytes(n_tok, vocab))


def predicted_kl(z_cur, z_prop, tau, kl_budget, alpha_max, out=None, kl_tok=None, ws=None):
    """Device tensor [q, alpha]; per-row KL goes to kl_tok when given."""
    _require(z_cur, "z_cur", torch.bfloat16, 2)
    _require(z_prop, "z_prop", torch.bfloat16, 2)
    n, V, ld = _rows(z_cur, "z_cur")
    n2, V2, ld2 = _rows(z_prop, "z_prop")
    if (n2, V2, ld2) != (n, V, ld):
        raise ValueError("z_cur and z_prop must have the same shape and row stride")
    if out is None:
        out = torch.empty(2, dtype=torch.float32, device=z_cur.device)
    _require(out, "out", torch.float32, 1)
    kl_ptr = None
    if kl_tok is not None:
        _require(kl_tok, "kl_tok", torch.float32, 1)
        if kl_tok.numel() != n or not kl_tok.is_contiguous():
            raise ValueError("kl_tok must be a contiguous float32 vector of n_tok entries")
        kl_ptr = kl_tok.data_ptr()
    ws_ptr, ws_n = None, 0
    if kl_tok is None:
        if ws is None:
            ws = torch.empty(max(kl_ws_bytes(n, V), 256), dtype=torch.uint8, device=z_cur.device)
        ws_ptr, ws_n = _ws(ws)
    st = _lib.lib().logra_predicted_kl(z_cur.data_ptr(), z_prop.data_ptr(), n, V, ld,
                                       float(tau), float(kl_budget), float(alpha_max),
                                       out.data_ptr(), kl_ptr, ws_ptr, ws_n, _stream(z_cur))
    _lib.check(st, "logra_predicted_kl")
    return out


MAX_SWEEP = 8


def kl_sweep_ws_bytes(n_tok, n_alpha):
    return int(_lib.lib().logra_kl_sweep_ws_bytes(n_tok, n_alpha))


def predicted_kl_sweep(z, delta, alphas, tau, weight=None, out=None, kl_tok=None, ws=None):
    """Device tensor [n_alpha] of weighted mean KL(p(z) || p(z + alpha_i delta));
    per-row values go to kl_tok ([n_alpha, n_tok], multiplier-major) when given."""
    _require(z, "z", torch.bfloat16, 2)
    _require(delta, "delta", torch.bfloat16, 2)
    n, V, ld = _rows(z, "z")
    if _rows(delta, "delta") != (n, V, ld):
        raise ValueError("z and delta must have the same shape and row stride")
    al = [float(a) for a in alphas]
    if not 1 <= len(al) <= MAX_SWEEP:
        raise ValueError(f"between 1 and {MAX_SWEEP} multipliers")
    c_al = (ctypes.c_float * len(al))(*al)
    if out is None:
        out = torch.empty(len(al), dtype=torch.float32, device=z.device)
    _require(out, "out", torch.float32, 1)
    w_ptr = None
    if weight is not None:
        _require(weight, "weight", torch.float32, 1)
        if weight.numel() != n or not weight.is_contiguous():
            raise ValueError("weight must be a contiguous float32 vector of n_tok entries")
        w_ptr = weight.data_ptr()
    kl_ptr = None
    if kl_tok is not None:
        _require(kl_tok, "kl_tok", torch.float32, 2)
        if tuple(kl_tok.shape) != (len(al), n) or not kl_tok.is_contiguous():
            raise ValueError("kl_tok must be a contiguous float32 [n_alpha, n_tok] tensor")
        kl_ptr = kl_tok.data_ptr()
    ws_ptr, ws_n = None, 0
    if kl_tok is None:
        if ws is None:
            ws = torch.empty(max(kl_sweep_ws_bytes(n, len(al)), 256), dtype=torch.uint8,
                             device=z.device)
        ws_ptr, ws_n = _ws(ws)
    st = _lib.lib().logra_predicted_kl_sweep(z.data_ptr(), delta.data_ptr(), n, V, ld, c_al,
                                             len(al), float(tau), w_ptr, out.data_ptr(), kl_ptr,
                                             ws_ptr, ws_n, _stream(z))
    _lib.check(st, "logra_predicted_kl_sweep")
    return out


def kl_budget_schedule(step, n_steps, start=2e-4, end=2e-5):
    """KL budget at `step` of an annealed run: linear from `start` (step 0) to
    `end` (step n_steps - 1), constant afterwards.  [LoGRA] PKL: the budget may
    be constant or annealed downward (2e-4 to 2e-5 in the pages' LoRA
    comparison); the pages do not give the shape, so it is linear here."""
    if n_steps <= 1 or step >= n_steps - 1:
        return float(end) if n_steps > 1 else float(start)
    if step <= 0:
        return float(start)
    f = step / (n_steps - 1)
    return float(start + (end - start) * f)
