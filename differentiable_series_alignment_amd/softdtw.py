"""PyTorch-facing Soft-DTW on the gfx950 library (libsdtw.so).

API of the README "SoftDTW-CUDA (PyTorch + Numba)": ``SoftDTW(gamma=1.0,
dist="sqeuclidean", fused=False, normalize=False)`` called as
``loss_fn(x, y)`` -> (B,) ("Usage", "Fused Mode", "Normalization") and
``softdtw_barycenter(sequences, gamma, max_iter, lr, fused, early_stopping,
cosine_annealing, grad_clip)`` -> (N, D)
("Time Series Barycenters").  PyTorch provides device memory, streams and
autograd; every Soft-DTW step runs in the library's HIP kernels.
"""
from __future__ import annotations

import math

import torch

from . import _lib as L


def _stream(device: torch.device) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream)


def _validate(x: torch.Tensor, y: torch.Tensor, gamma: float):
    """Input checks of the README's test list ("Tests": gamma, device, empty
    sequences, shape mismatches)."""
    if not isinstance(x, torch.Tensor) or not isinstance(y, torch.Tensor):
        raise ValueError("x and y must be tensors")
    g = float(gamma)
    if not math.isfinite(g) or g <= 0.0:
        raise ValueError(f"gamma must be finite and > 0, got {gamma}")
    if x.dim() != 3 or y.dim() != 3:
        raise ValueError(f"x and y must be (B, N, D) and (B, M, D); got {tuple(x.shape)} and {tuple(y.shape)}")
    if x.shape[0] != y.shape[0]:
        raise ValueError(f"batch sizes differ: {x.shape[0]} vs {y.shape[0]}")
    if x.shape[2] != y.shape[2]:
        raise ValueError(f"feature dimensions differ: {x.shape[2]} vs {y.shape[2]}")
    if min(x.shape) < 1 or min(y.shape) < 1:
        raise ValueError("empty sequences or batch are not supported")
    if x.dtype != torch.float32 or y.dtype != torch.float32:
        raise ValueError("x and y must be float32")
    if x.device.type != "cuda" or y.device.type != "cuda":
        raise ValueError("x and y must be on a GPU (there is no CPU path)")
    if x.device != y.device:
        raise ValueError(f"x and y are on different devices: {x.device} vs {y.device}")


def _workspace(B, N, M, D, mode, device):
    nbytes = L.sdtw_workspace_bytes(B, N, M, D, mode)
    if nbytes == 0:
        raise ValueError(f"unsupported sizes B={B} N={N} M={M} D={D}")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace is not 256-byte aligned")
    return ws


class _SoftDTWFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, y, gamma, mode):
        x = x.contiguous()
        y = y.contiguous()
        B, N, D = x.shape
        M = y.shape[1]
        with torch.cuda.device(x.device):
            ws = _workspace(B, N, M, D, mode, x.device)
            loss = torch.empty(B, dtype=torch.float32, device=x.device)
            L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma,
                                   mode, ws.data_ptr(), ws.numel(), loss.data_ptr(),
                                   _stream(x.device)), "sdtw_forward")
        ctx.save_for_backward(x, y)
        ctx.ws = ws
        ctx.gamma = gamma
        ctx.mode = mode
        return loss

    @staticmethod
    def backward(ctx, grad_loss):
        x, y = ctx.saved_tensors
        B, N, D = x.shape
        M = y.shape[1]
        need_x, need_y = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        gx = torch.empty_like(x) if need_x else None
        gy = torch.empty_like(y) if need_y else None
        gl = grad_loss.contiguous().to(torch.float32)
        ws = ctx.ws
        s = _stream(x.device)
        with torch.cuda.device(x.device):
            # The backward leaves the workspace valid for another backward
            # (retain_graph) in both modes.
            L.check(L.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, ctx.gamma,
                                    ctx.mode, ws.data_ptr(), ws.numel(), gl.data_ptr(),
                                    gx.data_ptr() if gx is not None else None,
                                    gy.data_ptr() if gy is not None else None,
                                    None, s), "sdtw_backward")
        return gx, gy, None, None


def _loss_only(x: torch.Tensor, y: torch.Tensor, gamma: float):
    """The loss through the library's inference mode (no state kept, O(B*N)
    workspace), or None where that mode does not apply (D > 256, or a GPU
    too small for its ring hand-off)."""
    x = x.contiguous()
    y = y.contiguous()
    B, N, D = x.shape
    M = y.shape[1]
    mode = L.SDTW_MODE_INFERENCE
    nbytes = L.sdtw_workspace_bytes(B, N, M, D, mode)
    if nbytes == 0:
        return None
    with torch.cuda.device(x.device):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
        loss = torch.empty(B, dtype=torch.float32, device=x.device)
        st = L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode,
                            ws.data_ptr(), nbytes, loss.data_ptr(), _stream(x.device))
    if st == L.SDTW_ERR_UNSUPPORTED:
        return None
    L.check(st, "sdtw_forward")
    return loss


def choose_mode(fused, B: int, N: int, M: int, D: int, device=None) -> int:
    """The training mode for ``fused``: True -> fused, False -> unfused; None
    or "auto" selects between memory and speed (README "Time Series
    Barycenters", key options: fused auto-selects between memory and speed).
    Reading: the fastest mode whose workspace takes at most half of the free
    device memory, in the order unfused (about 20 bytes per cell),
    low-memory unfused (about 12), fused (8, D <= 256); unfused if none
    does."""
    if fused is None or (isinstance(fused, str) and fused == "auto"):
        free, _ = torch.cuda.mem_get_info(device)
        for mode in (L.SDTW_MODE_UNFUSED, L.SDTW_MODE_UNFUSED_LOWMEM, L.SDTW_MODE_FUSED):
            need = L.sdtw_workspace_bytes(B, N, M, D, mode)
            if 0 < need <= free // 2:
                return mode
        return L.SDTW_MODE_UNFUSED
    if isinstance(fused, str):
        raise ValueError(f"fused must be True, False, None or 'auto', got {fused!r}")
    return L.SDTW_MODE_FUSED if bool(fused) else L.SDTW_MODE_UNFUSED


def choose_fused(fused, B: int, N: int, M: int, D: int, device=None) -> bool:
    """Whether choose_mode picks the fused mode."""
    return choose_mode(fused, B, N, M, D, device) == L.SDTW_MODE_FUSED


def soft_dtw(x: torch.Tensor, y: torch.Tensor, gamma: float = 1.0,
             fused=False, checkpoint: bool = False, low_memory: bool = False) -> torch.Tensor:
    """Per-pair Soft-DTW loss (B,) with autograd support.  When no gradient
    can be asked for (autograd off, or neither input requires one) the loss
    comes from the inference mode, which keeps no state; its value is bitwise
    the one of the other modes.  ``fused``: True, False, or None / "auto"
    (see choose_mode).  ``checkpoint=True`` trains with distances recomputed
    as in fused mode and without the B x N x M forward state: the backward
    recomputes it group by group of rows from checkpoint rows (about
    sqrt(N/64) groups), for a workspace of about sqrt(N/64) x 64 rows of M
    states per pair instead of N.  ``low_memory=True`` (with fused=False)
    trains in the low-memory unfused mode: the sweeps run one after the
    other and the reverse one forms the alignment matrix over the distances
    (about 12 instead of 20 bytes of workspace per cell; same results)."""
    _validate(x, y, gamma)
    if not (torch.is_grad_enabled() and (x.requires_grad or y.requires_grad)):
        loss = _loss_only(x, y, float(gamma))
        if loss is not None:
            return loss
    B, N, D = x.shape
    if checkpoint:
        mode = L.SDTW_MODE_CHECKPOINT
    else:
        mode = choose_mode(fused, B, N, y.shape[1], D, x.device)
        if low_memory and mode == L.SDTW_MODE_UNFUSED:
            mode = L.SDTW_MODE_UNFUSED_LOWMEM
    return _SoftDTWFunction.apply(x, y, float(gamma), mode)


class SoftDTW(torch.nn.Module):
    """``SoftDTW(gamma=1.0, dist="sqeuclidean", fused=False, normalize=False)``.

    ``normalize=True`` returns SoftDTW(x,y) - (SoftDTW(x,x) + SoftDTW(y,y))/2
    and requires x.shape == y.shape (README "Normalization"); the three
    terms run as one batch of 3B pairs."""

    def __init__(self, gamma: float = 1.0, dist: str = "sqeuclidean",
                 fused=False, normalize: bool = False, checkpoint: bool = False,
                 low_memory: bool = False):
        super().__init__()
        if dist != "sqeuclidean":
            raise ValueError(f"only dist='sqeuclidean' is supported, got {dist!r}")
        g = float(gamma)
        if not math.isfinite(g) or g <= 0.0:
            raise ValueError(f"gamma must be finite and > 0, got {gamma}")
        self.gamma = g
        self.dist = dist
        if isinstance(fused, str) and fused != "auto":
            raise ValueError(f"fused must be True, False, None or 'auto', got {fused!r}")
        self.fused = fused if (fused is None or isinstance(fused, str)) else bool(fused)
        self.normalize = bool(normalize)
        self.checkpoint = bool(checkpoint)
        self.low_memory = bool(low_memory)

    def forward(self, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
        if self.normalize:
            if tuple(x.shape) != tuple(y.shape):
                raise ValueError("normalize=True requires x.shape == y.shape")
            _validate(x, y, self.gamma)
            # The three terms as one batch of 3B pairs (x,y), (x,x), (y,y):
            # one pass through the kernels; autograd sums the gradients that
            # reach x and y through the concatenation.
            B = x.shape[0]
            loss = soft_dtw(torch.cat([x, x, y], 0), torch.cat([y, x, y], 0),
                            self.gamma, self.fused, self.checkpoint, self.low_memory)
            return loss[:B] - 0.5 * (loss[B:2 * B] + loss[2 * B:])
        return soft_dtw(x, y, self.gamma, self.fused, self.checkpoint, self.low_memory)

    def extra_repr(self) -> str:
        return (f"gamma={self.gamma}, dist={self.dist!r}, fused={self.fused}, "
                f"normalize={self.normalize}, checkpoint={self.checkpoint}, "
                f"low_memory={self.low_memory}")


def sqeuclidean(x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """The (B, N, M) fp32 squared-Euclidean distance tensor of the unfused
    mode, computed by the library's distance kernel."""
    _validate(x, y, 1.0)
    x = x.contiguous()
    y = y.contiguous()
    B, N, D = x.shape
    M = y.shape[1]
    out = torch.empty((B, N, M), dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        L.check(L.sdtw_dist(x.data_ptr(), y.data_ptr(), out.data_ptr(), B, N, M, D,
                            _stream(x.device)), "sdtw_dist")
    return out


def alignment(x: torch.Tensor, y: torch.Tensor, gamma: float = 1.0,
              fused: bool = False, checkpoint: bool = False):
    """(loss[B], E[B,N,M]): the loss and the alignment matrix dloss/dDist."""
    _validate(x, y, gamma)
    x = x.contiguous()
    y = y.contiguous()
    B, N, D = x.shape
    M = y.shape[1]
    mode = (L.SDTW_MODE_CHECKPOINT if checkpoint else
            L.SDTW_MODE_FUSED if fused else L.SDTW_MODE_UNFUSED)
    s = _stream(x.device)
    with torch.cuda.device(x.device):
        ws = _workspace(B, N, M, D, mode, x.device)
        loss = torch.empty(B, dtype=torch.float32, device=x.device)
        E = torch.empty((B, N, M), dtype=torch.float32, device=x.device)
        gl = torch.ones(B, dtype=torch.float32, device=x.device)
        L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, float(gamma), mode,
                               ws.data_ptr(), ws.numel(), loss.data_ptr(), s), "sdtw_forward")
        L.check(L.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, float(gamma), mode,
                                ws.data_ptr(), ws.numel(), gl.data_ptr(), None, None,
                                E.data_ptr(), s), "sdtw_backward")
    return loss, E


class EarlyStopping:
    """Convergence test of the barycenter loop (README "Time Series
    Barycenters": ``early_stopping=True`` detects convergence; the README's
    "Benchmarking" section reports it saving a large share of the
    iterations).  The pages give no rule; reading: after each iteration,
    an objective below best - tol*|best| becomes the new best, any other
    counts as a stalled iteration, and the loop stops after ``patience``
    stalled iterations in a row."""

    def __init__(self, patience: int = 10, tol: float = 1e-4):
        if int(patience) < 1 or not (float(tol) >= 0.0):
            raise ValueError("patience must be >= 1 and tol >= 0")
        self.patience = int(patience)
        self.tol = float(tol)
        self.best = math.inf
        self.stalled = 0

    def step(self, value: float) -> bool:
        """Record one objective value; True when the loop should stop."""
        v = float(value)
        if self.best == math.inf or v < self.best - self.tol * abs(self.best):
            self.best = v
            self.stalled = 0
        else:
            self.stalled += 1
        return self.stalled >= self.patience


def softdtw_barycenter(sequences: torch.Tensor, gamma: float = 1.0,
                       max_iter: int = 100, lr: float = 0.1, fused=False,
                       early_stopping: bool = False, patience: int = 10,
                       tol: float = 1e-4, cosine_annealing: bool = False,
                       grad_clip=None, return_history: bool = False):
    """Soft-DTW barycenter of K sequences (K, N, D) by Adam (README "Time
    Series Barycenters"; review page, "Proposed method").  The iterate starts
    at the pointwise mean and minimises mean_k SoftDTW(z, X_k).

    Options of the README ("Time Series Barycenters" key options and
    "Benchmarking"): ``fused`` True/False or None/"auto" (choose_mode);
    ``early_stopping`` (EarlyStopping(patience, tol)); ``cosine_annealing``
    (the learning rate follows lr*(1+cos(pi*t/max_iter))/2 over the
    iterations, torch's CosineAnnealingLR); ``grad_clip`` (the gradient's L2
    norm is clipped to this value before each step, as torch's
    clip_grad_norm_ does).  The optimizer is torch's Adam in its fused form.  The pages give no values for these; all are off by
    default so the plain loop is Adam alone."""
    if sequences.dim() != 3:
        raise ValueError("sequences must be (K, N, D)")
    if grad_clip is not None and not (float(grad_clip) > 0.0):
        raise ValueError("grad_clip must be > 0 or None")
    X = sequences.detach().contiguous()
    _validate(X, X, gamma)              # once: every iteration sees the same shapes
    K, N, D = X.shape
    g = float(gamma)
    dev = X.device
    mode = choose_mode(fused, K, N, N, D, dev)
    z = X.mean(dim=0).clone().requires_grad_(True)
    # torch's single-kernel Adam: the same update as the default one, with a
    # fraction of its host time (which bounds this loop: its kernels take
    # about 30 us per iteration).
    opt = torch.optim.Adam([z], lr=lr, fused=True)
    sched = (torch.optim.lr_scheduler.CosineAnnealingLR(opt, T_max=int(max_iter))
             if cosine_annealing and int(max_iter) > 0 else None)
    stop = EarlyStopping(patience, tol) if early_stopping else None
    clip = None if grad_clip is None else float(grad_clip)
    T = int(max_iter)
    # One set of buffers for the whole loop: the iterate broadcast to the K
    # pairs, workspace, per-pair losses, the upstream gradient of the batch
    # mean (1/K per pair), dz per pair and summed, and the objective history.
    # Each iteration is then sdtw_forward + sdtw_backward through the C ABI
    # (the gradient of mean_k SoftDTW(z, X_k) that autograd would assemble
    # from the same calls), a sum over k and the optimizer step.
    with torch.cuda.device(dev):
        ws = _workspace(K, N, N, D, mode, dev)
        loss = torch.empty(K, dtype=torch.float32, device=dev)
        gl = torch.full((K,), 1.0 / K, dtype=torch.float32, device=dev)
        zb = torch.empty_like(X)
        gx = torch.empty_like(X)
        gz = torch.empty_like(z)
        hist = torch.empty(max(T, 1), dtype=torch.float32, device=dev)
        s = _stream(dev)
        args = (zb.data_ptr(), X.data_ptr(), K, N, N, D, g, mode, ws.data_ptr(), ws.numel())
        n = 0
        for it in range(T):
            with torch.no_grad():
                zb.copy_(z.unsqueeze(0).expand_as(X))
            L.check(L.sdtw_forward(*args, loss.data_ptr(), s), "sdtw_forward")
            L.check(L.sdtw_backward(*args, gl.data_ptr(), gx.data_ptr(), None, None, s),
                    "sdtw_backward")
            torch.sum(gx, dim=0, out=gz)
            torch.mean(loss, dim=0, keepdim=True, out=hist[it:it + 1])
            z.grad = gz
            if clip is not None:
                # clip_grad_norm_ for one tensor: scale by min(1, c / (|g| + 1e-6))
                nrm = torch.linalg.vector_norm(gz)
                gz.mul_(torch.clamp(clip / (nrm + 1e-6), max=1.0))
            opt.step()
            if sched is not None:
                sched.step()
            n = it + 1
            if stop is not None and stop.step(hist[it].item()):
                break
    z = z.detach()
    if return_history:
        return z, hist[:n].cpu()
    return z
