"""One K-FAC step over a fixed set of layers: device buffers plus the sequence of
library calls (factors, written packed and as the upper triangle the inversion
reads -> damped inverses -> preconditioning, and the BatchNorm diagonal). Python only allocates and sequences; every number is computed
by libkfac's HIP kernels.

Step order follows Osawa et al. (CVPR 2019): stage 1-2 of their Figure 1 (factors
from the forward activations and backward gradients), eq. (6) (inverses of the
damped factors), eq. (7) (preconditioned gradients) and, when parameters are
given, eq. (8) (the update with learning rate lr); BatchNorm uses the diagonal
Fisher (Section 1, contributions)."""
import math

import torch

from . import _lib as K


def side_split(n_all, min_order=1024):
    """Indices of the matrices whose inverses go to the second stream: those of order
    more than half the largest, when the largest order is at least min_order (a sweep
    of 8 block steps or more; below that the events cost more than the overlap gains)
    and the split leaves matrices on both streams; else none."""
    n_max = max(n_all) if n_all else 0
    long_ = [i for i, n in enumerate(n_all) if 2 * n > n_max + 2]
    if n_max < min_order or len(long_) in (0, len(n_all)):
        return []
    return long_


class KfacStep:
    """Buffers for `layers` (objects with the kfac_layer fields) and `bn_layers`
    (objects with n, hw, c). Tikhonov damping gamma puts sqrt(gamma) on each
    Kronecker factor (float32-rounded) and gamma on the BN diagonal. precond_accum
    "f64" sums the preconditioning products in fp64 (kfac_precondition_ex).
    refine_inverse applies one fp64-residual refinement step to every inverse
    (kfac_invert_refine), which keeps a full symmetric copy of each factor.

    side_stream: when the largest order is 1024 or more, the inverses of the factors
    whose order is more than half the largest order (their block sweep is the long
    tail of the batch, a chain of latency-bound launches that leaves most compute
    units idle) run on a second stream, together with the preconditioning of their
    layers, while the caller's stream inverts the rest, preconditions their layers
    and does the BatchNorm step. The step joins the two streams before it returns;
    results are the same bits as with one stream."""

    def __init__(self, layers, bn_layers=(), device="cuda", damping=1e-3, bn_shift=None,
                 in_dtype=torch.float16, precond_accum="f32", refine_inverse=False, side_stream=True):
        self.layers = list(layers)
        self.bn_layers = list(bn_layers)
        self.device = torch.device(device)
        if precond_accum not in ("f32", "f64"):
            raise ValueError("precond_accum must be 'f32' or 'f64'")
        self.accum = K.KFAC_F64 if precond_accum == "f64" else K.KFAC_F32
        self.shift = float(torch.tensor(math.sqrt(damping), dtype=torch.float32))
        self.bn_shift = float(damping if bn_shift is None else bn_shift)
        self.d_a = [l.c_in * l.kh * l.kw + (1 if l.bias else 0) for l in self.layers]
        self.d_g = [l.c_out for l in self.layers]
        dev = self.device
        f32 = torch.float32
        self.A_packed = [torch.empty(d * (d + 1) // 2, dtype=f32, device=dev) for d in self.d_a]
        self.G_packed = [torch.empty(d * (d + 1) // 2, dtype=f32, device=dev) for d in self.d_g]
        # factor k of the inverse batch: A of every layer, then G of every layer
        self.n_all = self.d_a + self.d_g
        self.full = [torch.empty(d, d, dtype=f32, device=dev) for d in self.n_all]
        self.packed_all = self.A_packed + self.G_packed
        # matrices (indices into n_all) inverted on the second stream, and the layers
        # preconditioned there
        long_ = side_split(self.n_all) if side_stream and not refine_inverse else []
        L = len(self.layers)
        self.side = long_
        self.main = [i for i in range(len(self.n_all)) if i not in long_]
        self.side_layers = sorted({i % L for i in long_})
        self.main_layers = [l for l in range(L) if l not in self.side_layers]
        self._info_main = torch.zeros(len(self.main), dtype=torch.int32, device=dev)
        self._info_side = torch.zeros(len(self.side), dtype=torch.int32, device=dev)
        self.out = [torch.empty(g, a, dtype=f32, device=dev) for g, a in zip(self.d_g, self.d_a)]
        self.refine = bool(refine_inverse)
        self.factor_full = [torch.empty(d, d, dtype=f32, device=dev) for d in self.n_all] if self.refine else []
        self.fisher = [torch.zeros(2, b.c, dtype=f32, device=dev) for b in self.bn_layers]
        self.bn_pre = [torch.empty(2, b.c, dtype=f32, device=dev) for b in self.bn_layers]
        code = K.KFAC_F16 if in_dtype == torch.float16 else K.KFAC_F32
        sizes = [K.kfac_factors_workspace(self.layers, code),
                 K.kfac_pack_sym_workspace(self.n_all),
                 K.kfac_invert_workspace(self.n_all),
                 K.kfac_precondition_workspace(self.d_g, self.d_a)]
        if self.refine:
            sizes.append(K.kfac_invert_refine_workspace(self.n_all))
        if self.bn_layers:
            sizes.append(K.kfac_bn_diag_workspace(self.bn_layers))
        # one workspace serves every call on the caller's stream: they run one after
        # another; the second stream has its own
        self.workspace = torch.empty(max(sizes) + 256, dtype=torch.uint8, device=dev)
        self.stream2 = None
        if self.side:
            sub = lambda v, idx: [v[i] for i in idx]  # noqa: E731
            side_ws = max(K.kfac_invert_workspace(sub(self.n_all, self.side)),
                          K.kfac_precondition_workspace(sub(self.d_g, self.side_layers),
                                                        sub(self.d_a, self.side_layers)))
            self.workspace2 = torch.empty(side_ws + 256, dtype=torch.uint8, device=dev)
            self.stream2 = torch.cuda.Stream(device=dev)

    @property
    def info(self):
        """Breakdown index of every inverse (order of n_all: A factors, then G)."""
        out = torch.zeros(len(self.n_all), dtype=torch.int32, device=self.device)
        if self.main:
            out[self.main] = self._info_main
        if self.side:
            out[self.side] = self._info_side
        return out

    @property
    def A_inv(self):
        return self.full[:len(self.layers)]

    @property
    def G_inv(self):
        return self.full[len(self.layers):]

    def factors(self, act, gout, ema_decay=0.0, stream=None):
        K.kfac_factors(self.layers, act, gout, self.A_packed, self.G_packed, ema_decay,
                       self.workspace, stream)

    def _factors_full(self, act, gout, ema_decay, stream):
        # the packed factors (the stored state) and the upper triangles that kfac_invert
        # reads, from the same kernels: no separate unpack pass
        L = len(self.layers)
        K.kfac_factors_full(self.layers, act, gout, self.A_packed, self.G_packed, self.full[:L], self.full[L:],
                            ema_decay, self.workspace, stream)

    # With the second stream, the caller's stream forms its factors in 2 calls,
    # preconditions in 4 and runs the BatchNorm step in 2 (groups of layers of about
    # equal work). A pivot block of the long sweeps needs a whole compute unit, and while
    # a launch of many small blocks runs, the units it frees go to its own next blocks:
    # the pivot waits for the launch to drain (up to 0.3 ms behind one preconditioning
    # or BatchNorm launch). Shorter launches bound that wait; more calls cost more than
    # they save (measured: 6 preconditioning calls or 3 factor calls were slower).
    MAIN_CALLS = {"factors": 2, "precondition": 4, "bn": 2}

    @staticmethod
    def _groups(idx, cost, parts):
        """idx (in order) cut into at most `parts` runs of about equal summed cost."""
        total = sum(cost(i) for i in idx)
        out, cur, acc = [], [], 0.0
        for i in idx:
            cur.append(i)
            acc += cost(i)
            if len(out) < parts - 1 and acc >= total * (len(out) + 1) / parts:
                out.append(cur)
                cur = []
        if cur:
            out.append(cur)
        return out

    def _sub(self, v, idx):
        return [v[i] for i in idx]

    def _factor_cost(self, l):
        # products of a layer's two factors: rows x order^2, the 3x3 A factors at about a
        # third (formed from shift products)
        L = self.layers[l]
        rows = L.n * L.h_out * L.w_out
        return rows * (self.d_a[l] ** 2 / (3.0 if L.kh == 3 and L.sh == 1 else 1.0) + self.d_g[l] ** 2)

    def _factor_inputs(self, act, gout):
        """(act, gout) lists of the side matrices' factors and of all the others, with
        None where a factor is left to the other call."""
        L = len(self.layers)
        side = set(self.side)
        first = ([a if l in side else None for l, a in enumerate(act)],
                 [g if l + L in side else None for l, g in enumerate(gout)])
        rest = ([None if l in side else a for l, a in enumerate(act)],
                [None if l + L in side else g for l, g in enumerate(gout)])
        return first, rest

    def invert(self, stream=None):
        """Unpacks and inverts every damped factor on `stream` (the side split is
        applied by step())."""
        self._unpack(stream)
        self._invert(self.main, self._info_main, self.workspace, stream)
        if self.side:
            self._invert(self.side, self._info_side, self.workspace, stream)
        self._refine(stream)

    def _unpack(self, stream):
        # kfac_invert reads only the upper triangle: unpack that half
        K.kfac_pack_sym(self.n_all, self.full, self.packed_all, 2, self.workspace, stream)

    def _invert(self, idx, info, ws, stream):
        if idx:
            K.kfac_invert(self._sub(self.n_all, idx), self._sub(self.full, idx), self._sub(self.full, idx),
                          [self.shift] * len(idx), info, None, ws, stream)

    def _refine(self, stream):
        if self.refine:
            K.kfac_pack_sym(self.n_all, self.factor_full, self.packed_all, 1, self.workspace, stream)
            K.kfac_invert_refine(self.n_all, self.factor_full, [self.shift] * len(self.n_all), self.full,
                                 self.workspace, stream)

    def precondition(self, grads, weights=None, lr=0.0, stream=None):
        """self.out <- preconditioned gradients; with weights (fp32 [d_g, d_a] per layer)
        also weights -= lr * self.out, in the same kernel."""
        self._precondition(list(range(len(self.layers))), grads, weights, lr, self.workspace, stream)

    def _precondition(self, ls, grads, weights, lr, ws, stream):
        if not ls:
            return
        sub = self._sub
        d_g, d_a, G, A, g, o = (sub(self.d_g, ls), sub(self.d_a, ls), sub(self.G_inv, ls), sub(self.A_inv, ls),
                                sub(grads, ls), sub(self.out, ls))
        w = sub(weights, ls) if weights is not None else None
        if self.accum == K.KFAC_F64:
            K.kfac_precondition_ex(d_g, d_a, G, A, g, o, w, lr, self.accum, ws, stream)
        elif w is None:
            K.kfac_precondition(d_g, d_a, G, A, g, o, ws, stream)
        else:
            K.kfac_precondition_update(d_g, d_a, G, A, g, o, w, lr, ws, stream)

    def bn(self, xhat, bn_gout, ema_decay=0.0, bn_params=None, lr=0.0, stream=None):
        """BN Fisher and preconditioned gradients; with bn_params (fp32 [2, c]: gamma,
        beta) also bn_params -= lr * self.bn_pre."""
        self._bn(list(range(len(self.bn_layers))), xhat, bn_gout, ema_decay, bn_params, lr, stream)

    def _bn(self, idx, xhat, bn_gout, ema_decay, bn_params, lr, stream):
        if not idx:
            return
        sub = self._sub
        if bn_params is None:
            K.kfac_bn_diag(sub(self.bn_layers, idx), sub(xhat, idx), sub(bn_gout, idx), sub(self.fisher, idx),
                           sub(self.bn_pre, idx), ema_decay, self.bn_shift, self.workspace, stream)
        else:
            K.kfac_bn_update(sub(self.bn_layers, idx), sub(xhat, idx), sub(bn_gout, idx), sub(self.fisher, idx),
                             sub(self.bn_pre, idx), sub(bn_params, idx), lr, ema_decay, self.bn_shift,
                             self.workspace, stream)

    def step(self, act, gout, grads, xhat=(), bn_gout=(), ema_decay=0.0, refresh=True,
             weights=None, bn_params=None, lr=0.0, stream=None):
        """One step. refresh=False is a stale-curvature step: factors and inverses are
        kept, the gradients are preconditioned with them, and BN divides its fresh
        gradient by the stored Fisher (decay 1 keeps it). Given weights and/or
        bn_params, those are updated in place with learning rate lr."""
        if not refresh:
            self.precondition(grads, weights, lr, stream)
            self.bn(xhat, bn_gout, 1.0, bn_params, lr, stream)
            return
        if not self.side:
            self._factors_full(act, gout, ema_decay, stream)
            self._invert(self.main, self._info_main, self.workspace, stream)
            self._refine(stream)
            self.precondition(grads, weights, lr, stream)
            self.bn(xhat, bn_gout, ema_decay, bn_params, lr, stream)
            return
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        side = self.stream2
        # the long sweeps' factors first, so that their inverses start while the other
        # factors are formed (a factor call plans its row splits over every layer,
        # whichever inputs it is given: the same bits as one call)
        first, rest = self._factor_inputs(act, gout)
        self._factors_full(first[0], first[1], ema_decay, main)
        formed = torch.cuda.Event()
        formed.record(main)
        side.wait_event(formed)
        try:
            self._invert(self.side, self._info_side, self.workspace2, side)
            lay = [l for l in range(len(self.layers)) if rest[0][l] is not None or rest[1][l] is not None]
            for part in self._groups(lay, self._factor_cost, self.MAIN_CALLS["factors"]):
                ps = set(part)
                self._factors_full([a if l in ps else None for l, a in enumerate(rest[0])],
                                   [g if l in ps else None for l, g in enumerate(rest[1])], ema_decay, main)
            self._invert(self.main, self._info_main, self.workspace, main)
            main_inverses = torch.cuda.Event()
            main_inverses.record(main)
            pcost = lambda l: self.d_g[l] * self.d_a[l] * (self.d_g[l] + self.d_a[l])  # noqa: E731
            for part in self._groups(self.main_layers, pcost, self.MAIN_CALLS["precondition"]):
                self._precondition(part, grads, weights, lr, self.workspace, main)
            bcost = lambda b: self.bn_layers[b].n * self.bn_layers[b].hw * self.bn_layers[b].c  # noqa: E731
            for part in self._groups(list(range(len(self.bn_layers))), bcost, self.MAIN_CALLS["bn"]):
                self._bn(part, xhat, bn_gout, ema_decay, bn_params, lr, main)
            side.wait_event(main_inverses)  # the side layers' other factor
            self._precondition(self.side_layers, grads, weights, lr, self.workspace2, side)
        finally:
            # whatever was issued on the second stream is ordered before the caller's
            # later work, also when a call above raised
            joined = torch.cuda.Event()
            joined.record(side)
            main.wait_event(joined)
