"""MoELayer: one forward pass of the sparse MoE feed-forward layer as five
libmoe calls (route, permute, routed experts [+ shared experts], combine,
balance statistics).  Buffers are allocated on the first call for a token
count and reused afterwards, so repeated calls allocate nothing.

The shared experts depend on x alone, so by default they run on a second
stream (default priority) beside the routed path, from the start of the call,
where they overlap the latency-bound routing.  When the library streams their
weights (at most 64 tokens) its launches leave room for the routing kernels;
their tiled GEMMs (more tokens) run as persistent launches on half of the
compute units, so that the routing kernels, and then the routed experts'
first workgroups, still find the other half free (a full-width launch would
hold every compute unit until it ends).  In a training forward the shared
experts start once the routing is done, at full width.  The balance
statistics follow them on that stream once the routing is done, and the
combine waits for both.

The layer output excludes the residual ("Every parameter, every token",
section "The gating network": the weighted sum is added back to the residual
stream outside the slot).

``forward(x, train=True)`` also keeps what the backward pass reads (the
experts' pre-activations); ``backward(dy)`` then returns the gradients of
<dy, y> + coef_balance * loss + coef_z * zloss with respect to x and every
weight, through seven more library calls.
"""

from __future__ import annotations

import torch

from . import _lib


# Up to this many rows per group the library runs an expert GEMM as a weight
# stream (few rows, every weight read once) rather than as MFMA tiles; the
# shared experts are one group of T rows.
SHARED_STREAM_ROWS = 64
# Share of the compute units that the shared experts' tiled GEMMs take when
# they start with the call: half (on the fine-grained layer, 8192 tokens and
# four shared experts against eight routed ones per token, half gave the
# fastest step of 96 to 256 workgroups), or their share of the expert FLOPs
# where that is larger, so that they do not end after the routed experts.
SHARED_CU_SHARE = 0.5


class MoELayer:
    def __init__(self, w_router, w_gate, w_up, w_down, k, *, shared=None, logit_bias=None,
                 select_bias=None, capacity=-1, alpha=0.01, gather="fused",
                 overlap_shared=True, balance=None, bias_on_probs=False, relu=False,
                 bypass=None):
        """Weights are device tensors: w_router [E, d]; w_gate, w_up [E, h, d];
        w_down [E, d, h]; ``shared`` is None or (gate [Hs, d], up [Hs, d],
        down [d, Hs]) with the shared experts concatenated along the hidden
        axis.  ``capacity`` < 0 means unlimited.  ``gather`` is "fused" (the
        first expert GEMM reads token rows through the permutation) or "copy"
        (moe_permute writes an expert-ordered copy of x first).  ``overlap_shared``
        runs the shared experts on a second stream (see the module notes).  ``bias_on_probs`` adds
        the selection bias to the routing probability instead of the logit.

        ``balance`` turns on the per-step load-balancing updates that
        ``update_balance()`` applies after a step: a dict with ``bias_step``
        (the selection-bias step; the layer then owns a selection bias, zero
        if none was given), ``ema_decay``, and, for adaptive per-expert
        capacity, ``cf_base`` and ``gamma`` (the budgets start at
        moe_capacity(cf_base) and follow C_e = cf_base + gamma (fbar_e - 1/E)
        from the first update on).

        ``relu`` routes with ReLU gates (at most k experts per token, those
        with a positive logit; no selection bias).  ``bypass`` adds
        zero-computation experts after the FFN experts: a dict with
        ``n_zero``, ``n_copy`` and ``const_rows`` ([n_const, d] in the dtype
        of x, or None); w_router then has E + n_zero + n_copy + n_const rows.
        Neither variant takes balance updates."""
        if gather not in ("fused", "copy"):
            raise ValueError("gather must be 'fused' or 'copy'")
        self.w_router, self.w_gate, self.w_up, self.w_down = w_router, w_gate, w_up, w_down
        self.E, self.h, self.d = w_gate.shape
        self.E_router = w_router.shape[0]
        self.k = k
        self.relu = bool(relu)
        self.bypass = None
        if bypass is not None:
            cr = bypass.get("const_rows")
            self.bypass = dict(n_zero=int(bypass.get("n_zero", 0)),
                               n_copy=int(bypass.get("n_copy", 0)), const_rows=cr,
                               n_const=0 if cr is None else int(cr.shape[0]))
            nz = self.bypass["n_zero"] + self.bypass["n_copy"] + self.bypass["n_const"]
            if self.E + nz != self.E_router:
                raise ValueError("w_router needs E + n_zero + n_copy + n_const rows")
        elif self.E_router != self.E:
            raise ValueError("w_router and the expert weights disagree on E")
        if (self.relu or self.bypass) and balance:
            raise ValueError("the routing variants take no balance updates")
        if self.relu and (select_bias is not None or bias_on_probs):
            raise ValueError("ReLU routing takes no selection bias")
        self.shared = None
        if shared is not None:
            sg, su, sd = shared
            self.shared = (sg.reshape(1, *sg.shape), su.reshape(1, *su.shape),
                           sd.reshape(1, *sd.shape))
        self.logit_bias, self.select_bias = logit_bias, select_bias
        self.capacity = int(capacity)
        self.alpha = alpha
        self.gather = gather
        self.overlap_shared = overlap_shared
        self._bufs = {}
        self._side = {}
        self.bias_on_probs = bias_on_probs
        self.balance = dict(balance) if balance else None
        self.load_ema = None
        self.expert_capacity = None
        if self.balance:
            dev = w_router.device
            self.load_ema = torch.full((self.E,), 1.0 / self.E, dtype=torch.float32, device=dev)
            if self.balance.get("bias_step", 0.0) and self.select_bias is None:
                self.select_bias = torch.zeros(self.E, dtype=torch.float32, device=dev)
        self._last_T = None

    def _buffers(self, x):
        T = x.shape[0]
        key = (T, x.dtype, x.device)
        b = self._bufs.get(key)
        if b is not None:
            return b
        dev, E, k, d, h = x.device, self.E_router, self.k, self.d, self.h
        R = T * k
        dt = _lib._dt(x)
        b = dict(
            logits=torch.empty((T, E), dtype=torch.float32, device=dev),
            topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
            topk_gate=torch.empty((T, k), dtype=torch.float32, device=dev),
            route_ws=torch.empty(max(1, _lib.moe_route_workspace(T, d, E, k, dt)),
                                 dtype=torch.uint8, device=dev),
            expert_count=torch.empty(E, dtype=torch.int32, device=dev),
            expert_offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
            pair_row=torch.empty(R, dtype=torch.int32, device=dev),
            row_pair=torch.empty(R, dtype=torch.int32, device=dev),
            x_perm=(torch.empty((R, d), dtype=x.dtype, device=dev)
                    if self.gather == "copy" else None),
            perm_ws=torch.empty(max(1, _lib.moe_permute_workspace(T, k, E)), dtype=torch.uint8,
                                device=dev),
            hid=torch.empty((R, h), dtype=x.dtype, device=dev),
            y_perm=torch.empty((R, d), dtype=x.dtype, device=dev),
            table_ws=torch.empty(_lib.moe_expert_down_workspace(self.E), dtype=torch.uint8,
                                 device=dev),
            out=torch.empty((T, d), dtype=x.dtype, device=dev),
            f=torch.empty(E, dtype=torch.float32, device=dev),
            P=torch.empty(E, dtype=torch.float32, device=dev),
            loss=torch.empty(1, dtype=torch.float32, device=dev),
            zloss=torch.empty(1, dtype=torch.float32, device=dev),
            stats_ws=torch.empty(max(1, _lib.moe_balance_stats_workspace(T, E)),
                                 dtype=torch.uint8, device=dev),
        )
        if self.bypass is not None:
            # the zero-computation experts take no rows: budget 0
            cap = self.capacity if self.capacity >= 0 else T
            b["bypass_caps"] = torch.tensor([min(cap, T)] * self.E + [0] * (E - self.E),
                                            dtype=torch.int32, device=dev)
        if self.shared is not None:
            Hs = self.shared[0].shape[1]
            b["shared_off"] = torch.tensor([0, T], dtype=torch.int32, device=dev)
            b["shared_y"] = torch.empty((T, d), dtype=x.dtype, device=dev)
            b["shared_ws"] = torch.empty(
                max(1, _lib.moe_expert_swiglu_workspace(T, d, Hs, 1, dt)), dtype=torch.uint8,
                device=dev)
        self._bufs[key] = b
        return b

    def _train_buffers(self, x, b):
        """Buffers of the training forward (pre-activations) and the backward."""
        if "uv" in b:
            return b
        T = x.shape[0]
        dev, E, k, d, h = x.device, self.E, self.k, self.d, self.h
        R = T * k
        dt = _lib._dt(x)
        f32 = torch.float32
        b["uv"] = torch.empty((R, 2 * h), dtype=x.dtype, device=dev)
        b["dgate"] = torch.empty((T, k), dtype=f32, device=dev)
        b["dout"] = torch.empty((R, d), dtype=x.dtype, device=dev)
        Er = self.E_router  # router experts (E plus any zero-computation experts)
        b["dlogits"] = torch.empty((T, Er), dtype=f32, device=dev)
        b["da"] = torch.empty((R, d), dtype=f32, device=dev)
        b["dw_gate"] = torch.empty((E, h, d), dtype=f32, device=dev)
        b["dw_up"] = torch.empty((E, h, d), dtype=f32, device=dev)
        b["dw_down"] = torch.empty((E, d, h), dtype=f32, device=dev)
        b["bwd_ws"] = torch.empty(
            max(1, _lib.moe_expert_swiglu_backward_workspace(R, d, h, E, dt, True)),
            dtype=torch.uint8, device=dev)
        b["dw_router"] = torch.empty((Er, d), dtype=f32, device=dev)
        b["dlogit_bias"] = torch.empty(Er, dtype=f32, device=dev)
        b["dx_acc"] = torch.empty((T, d), dtype=f32, device=dev)
        b["dx"] = torch.empty((T, d), dtype=f32, device=dev)
        b["router_ws"] = torch.empty(max(1, _lib.moe_router_backward_workspace(T, d, Er)),
                                     dtype=torch.uint8, device=dev)
        if self.bypass is not None:
            nk = self.bypass["n_const"]
            b["dconst"] = torch.empty((max(nk, 1), d), dtype=f32, device=dev)
            b["bypass_ws"] = torch.empty(max(1, _lib.moe_bypass_backward_workspace(T, d, nk)),
                                         dtype=torch.uint8, device=dev)
        if self.shared is not None:
            Hs = self.shared[0].shape[1]
            b["shared_hid"] = torch.empty((T, Hs), dtype=x.dtype, device=dev)
            b["shared_uv"] = torch.empty((T, 2 * Hs), dtype=x.dtype, device=dev)
            b["shared_dw_gate"] = torch.empty((1, Hs, d), dtype=f32, device=dev)
            b["shared_dw_up"] = torch.empty((1, Hs, d), dtype=f32, device=dev)
            b["shared_dw_down"] = torch.empty((1, d, Hs), dtype=f32, device=dev)
            b["shared_bwd_ws"] = torch.empty(
                max(1, _lib.moe_expert_swiglu_backward_workspace(T, d, Hs, 1, dt, False)),
                dtype=torch.uint8, device=dev)
        return b

    def _stats(self, b, k, stream):
        _lib.moe_balance_stats(b["logits"], b["expert_count"], k, self.alpha, f=b["f"], P=b["P"],
                               loss=b["loss"], zloss=b["zloss"], ws=b["stats_ws"], stream=stream)

    def _shared_forward(self, x, b, train, stream, max_cus=0):
        sg, su, sd = self.shared
        T = x.shape[0]
        if not train:
            return _lib.moe_expert_swiglu(x, b["shared_off"], T, sg, su, sd, y=b["shared_y"],
                                          ws=b["shared_ws"], stream=stream, max_cus=max_cus)
        table = b["shared_ws"][-_lib.moe_expert_group_workspace(1):]
        _lib.moe_expert_gate_up_train(x, b["shared_off"], T, sg, su, hid=b["shared_hid"],
                                      uv=b["shared_uv"], ws=table, stream=stream)
        return _lib.moe_expert_down(b["shared_hid"], b["shared_off"], T, sd, y=b["shared_y"],
                                    ws=table, stream=stream)

    def forward(self, x, stream=None, mark=None, train=False):
        """Returns a dict of the output and every intermediate the calls produce.
        ``mark(name)``, if given, is called after each library call is enqueued
        (the benchmark records a HIP event there).  ``train`` keeps the experts'
        pre-activations for ``backward`` (bf16 only)."""
        b = self._buffers(x)
        if train:
            self._train_buffers(x, b)
            b["x"] = x
        T = x.shape[0]
        k, E = self.k, self.E
        mark = mark or (lambda name: None)
        main = stream if stream is not None else torch.cuda.current_stream(x.device)
        shared_y = shared_done = side = None
        overlap = self.shared is not None and self.overlap_shared
        early = overlap and (T <= SHARED_STREAM_ROWS or not train)
        if overlap:
            side = self._side.get(x.device)
            if side is None:
                side = self._side[x.device] = torch.cuda.Stream(x.device)
        if early:
            # the side stream starts once everything enqueued so far on the
            # main stream (x, and the previous call's combine, which reads
            # shared_y) is done
            x_ready = torch.cuda.Event()
            x_ready.record(main)
            side.wait_event(x_ready)
            max_cus = 0
            if T > SHARED_STREAM_ROWS:
                ncu = torch.cuda.get_device_properties(x.device).multi_processor_count
                hs = self.shared[0].shape[1]
                share = max(SHARED_CU_SHARE, hs / (hs + self.k * self.h))
                max_cus = max(8, int(ncu * share))
            shared_y = self._shared_forward(x, b, train, side, max_cus=max_cus)
        _lib.moe_route(x, self.w_router, k, self.logit_bias, self.select_bias,
                       logits=b["logits"], topk_idx=b["topk_idx"], topk_gate=b["topk_gate"],
                       bias_on_probs=self.bias_on_probs, relu=self.relu, ws=b["route_ws"],
                       stream=stream)
        mark("route")
        E = self.E_router
        if self.bypass is not None:
            _lib.moe_permute_budgets(b["topk_idx"], E, b["bypass_caps"],
                                     x if self.gather == "copy" else None,
                                     expert_count=b["expert_count"],
                                     expert_offset=b["expert_offset"], pair_row=b["pair_row"],
                                     row_pair=b["row_pair"], x_perm=b["x_perm"], ws=b["perm_ws"],
                                     stream=stream)
        elif self.balance and "gamma" in self.balance:
            if self.expert_capacity is None or self._last_T != T:
                c0 = _lib.moe_capacity(self.balance["cf_base"], T, k, E)
                self.expert_capacity = torch.full((E,), min(c0, T) if c0 >= 0 else T,
                                                  dtype=torch.int32, device=x.device)
            _lib.moe_permute_budgets(b["topk_idx"], E, self.expert_capacity,
                                     x if self.gather == "copy" else None,
                                     expert_count=b["expert_count"],
                                     expert_offset=b["expert_offset"], pair_row=b["pair_row"],
                                     row_pair=b["row_pair"], x_perm=b["x_perm"], ws=b["perm_ws"],
                                     stream=stream)
        else:
            _lib.moe_permute(b["topk_idx"], E, self.capacity,
                             x if self.gather == "copy" else None,
                             expert_count=b["expert_count"], expert_offset=b["expert_offset"],
                             pair_row=b["pair_row"], row_pair=b["row_pair"], x_perm=b["x_perm"],
                             ws=b["perm_ws"], stream=stream)
        self._last_T = T
        self._last_counts = b["expert_count"]
        mark("permute")
        if overlap:
            # the balance statistics need only the logits and the counts: on
            # the side stream, after the shared experts, beside the routed
            # GEMMs (the shared experts themselves start here unless they
            # started with the call)
            routed = torch.cuda.Event()
            routed.record(main)
            side.wait_event(routed)
            if not early:
                shared_y = self._shared_forward(x, b, train, side)
            self._stats(b, k, side)
            shared_done = torch.cuda.Event()
            shared_done.record(side)
        if self.gather == "copy":
            a, a_rows = b["x_perm"], None
        else:
            a, a_rows = x, b["row_pair"]
        off = b["expert_offset"] if self.bypass is None else b["expert_offset"][:self.E + 1]
        if train:
            _lib.moe_expert_gate_up_train(a, off, T * k, self.w_gate, self.w_up,
                                          a_rows=a_rows, a_rows_div=k, hid=b["hid"], uv=b["uv"],
                                          ws=b["table_ws"], stream=stream)
        else:
            _lib.moe_expert_gate_up(a, off, T * k, self.w_gate, self.w_up,
                                    a_rows=a_rows, a_rows_div=k, hid=b["hid"], ws=b["table_ws"],
                                    stream=stream)
        mark("gate_up")
        _lib.moe_expert_down(b["hid"], off, T * k, self.w_down, y=b["y_perm"],
                             ws=b["table_ws"], stream=stream)
        mark("down")
        if self.shared is not None and not self.overlap_shared:
            shared_y = self._shared_forward(x, b, train, stream)
            mark("shared")
        if shared_done is not None:
            main.wait_event(shared_done)
        if self.bypass is not None:
            bp = self.bypass
            _lib.moe_combine_bypass(b["y_perm"], b["pair_row"], b["topk_idx"], b["topk_gate"],
                                    self.E, bp["n_zero"], bp["n_copy"], x, bp["const_rows"],
                                    shared_y, out=b["out"], stream=stream)
        else:
            _lib.moe_combine(b["y_perm"], b["pair_row"], b["topk_gate"], shared_y, out=b["out"],
                             stream=stream)
        mark("combine")
        if shared_done is None:
            self._stats(b, k, stream)
            mark("stats")
        return b

    __call__ = forward

    def update_balance(self, stream=None):
        """The per-step load-balancing updates from the last forward's counts
        (selection bias, rolling load, per-expert budgets for the next step)."""
        if not self.balance:
            raise RuntimeError("the layer was built without balance updates")
        cfg = self.balance
        adaptive = "gamma" in cfg
        if adaptive and self.expert_capacity is None:
            self.expert_capacity = torch.empty(self.E, dtype=torch.int32,
                                               device=self._last_counts.device)
        _lib.moe_balance_update(self._last_counts, self._last_T, self.k, self.load_ema,
                                select_bias=self.select_bias if cfg.get("bias_step", 0.0) else None,
                                bias_step=cfg.get("bias_step", 0.0),
                                ema_decay=cfg.get("ema_decay", 0.0),
                                cf_base=cfg.get("cf_base", 1.0), gamma=cfg.get("gamma", 0.0),
                                expert_capacity=self.expert_capacity if adaptive else None,
                                want_capacity=adaptive, stream=stream)

    def backward(self, dy, coef_balance=0.0, coef_z=0.0, stream=None, mark=None):
        """Gradients after ``forward(x, train=True)`` on the same x: fills and
        returns the buffer dict with dx [T, d], dw_router, dlogit_bias (when the
        layer has a logit bias), dw_gate, dw_up, dw_down, and shared_dw_* (fp32),
        plus the intermediates dgate, dout and dlogits."""
        T = dy.shape[0]
        b = self._bufs[(T, dy.dtype, dy.device)]
        if "x" not in b:
            raise RuntimeError("backward needs forward(x, train=True) first")
        x = b["x"]
        k, E = self.k, self.E
        mark = mark or (lambda name: None)
        bp = self.bypass
        if bp is not None:
            _lib.moe_combine_backward_bypass(dy, b["y_perm"], b["pair_row"], b["topk_idx"],
                                             b["topk_gate"], E, bp["n_zero"], bp["n_copy"], x,
                                             bp["const_rows"], dgate=b["dgate"], dout=b["dout"],
                                             stream=stream)
        else:
            _lib.moe_combine_backward(dy, b["y_perm"], b["pair_row"], k, b["topk_gate"],
                                      dgate=b["dgate"], dout=b["dout"], stream=stream)
        mark("combine_bwd")
        _lib.moe_route_backward(b["logits"], b["topk_idx"], b["topk_gate"], b["dgate"],
                                b["expert_count"], self.alpha, coef_balance, coef_z,
                                relu=self.relu, dlogits=b["dlogits"], stream=stream)
        mark("route_bwd")
        _lib.moe_expert_swiglu_backward(
            x, b["expert_offset"][:E + 1], T * k, b["dout"], b["uv"], b["hid"], self.w_gate,
            self.w_up,
            self.w_down, a_rows=b["row_pair"], a_rows_div=k, da=b["da"], dw_gate=b["dw_gate"],
            dw_up=b["dw_up"], dw_down=b["dw_down"], ws=b["bwd_ws"], stream=stream)
        mark("experts_bwd")
        if self.shared is not None:
            sg, su, sd = self.shared
            _lib.moe_expert_swiglu_backward(
                x, b["shared_off"], T, dy, b["shared_uv"], b["shared_hid"], sg, su, sd,
                da=b["dx_acc"], dw_gate=b["shared_dw_gate"], dw_up=b["shared_dw_up"],
                dw_down=b["shared_dw_down"], ws=b["shared_bwd_ws"], stream=stream)
            mark("shared_bwd")
        _lib.moe_router_backward(x, self.w_router, b["dlogits"], dw_router=b["dw_router"],
                                 dlogit_bias=b["dlogit_bias"] if self.logit_bias is not None else None,
                                 dx=b["dx_acc"], accumulate_dx=self.shared is not None,
                                 want=("dw", "dx"), ws=b["router_ws"], stream=stream)
        mark("router_bwd")
        if bp is not None:
            # copy slots add g dy to dx; constant experts collect their rows' gradient
            _lib.moe_bypass_backward(dy, b["topk_idx"], b["topk_gate"], E, bp["n_zero"],
                                     bp["n_copy"], bp["n_const"], dx_acc=b["dx_acc"],
                                     dconst=b["dconst"][:bp["n_const"]] if bp["n_const"] else None,
                                     ws=b["bypass_ws"], stream=stream)
            mark("bypass_bwd")
        _lib.moe_combine(b["da"], b["pair_row"], None, b["dx_acc"], out=b["dx"], k=k,
                         stream=stream)
        mark("dx")
        return b
