"""The hot path end to end on one GPU: device buffers plus the sequence of
C-ABI calls for the three workload shapes (up-projection, gated FFN
forward, backward).  Buffer management and call order only -- every
arithmetic step runs in libmoefp8's kernels.

Forward ("Quantize activations before EP all gather", description and
review comments): quantize tokens -> sort/gather fp8 rows -> gmm(s) ->
[SiLU*mul requantize -> gmm] -> weighted gather-reduce.  Backward
("Support quantization for tokamax gmm v2", gmm2 / tgmm2): dX = gmm(dY,
W^T) and dW = tgmm(X, dY).

Expert parallelism is modelled as one GPU's slice: experts
[group_offset, group_offset + num_local_experts) are local; the sorted
buffers hold only their rows (compact window).  With ``share`` the step
quantizes only this GPU's 1/share of the tokens into its slot of the
token buffer; the other slots stand for what the all-gather would bring and
are quantized once at setup.
"""

import numpy as np
import torch

from . import (MOE_ACT_NONE, MOE_ACT_SILU_MUL, MOE_BF16, MOE_E4M3FN, MOE_F32, MOE_OP_GATHER_REDUCE, MOE_OP_GMM,
               MOE_OP_QUANTIZE_ROWS, MOE_OP_SORT_BY_EXPERT, MOE_OP_TGMM, MOE_SCALE_ROW_DYNAMIC, MOE_SCALE_TENSOR_DYNAMIC,
               MOE_SCALE_TENSOR_FROM_ROW_AMAX, MOE_SCALE_TENSOR_STATIC, moe_gather_reduce, moe_gather_reduce_backward,
               moe_gmm_fp8, moe_quantize_rows, moe_quantize_rows_strided, moe_quantize_sort_by_expert,
               moe_quantize_weights, moe_silu_mul_backward, moe_sort_by_expert, moe_sort_gather_transposed,
               moe_tgmm_fp8, moe_tgmm_fp8_xt, tgmm_xt_cols, workspace)


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """bfloat16 bit patterns (uint16 numpy) -> bfloat16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class QuantizedWeight:
    """An expert weight [E, K, N] quantized on the GPU with [E, kb, 1, nb]
    scales; stored [E, N, K] when ``nk`` (contraction dim contiguous)."""

    def __init__(self, w_bf16: torch.Tensor, kb: int, nb: int, static_scale=None, nk=True, stream=None):
        E, K, N = w_bf16.shape
        self.E, self.K, self.N, self.kb, self.nb, self.nk = E, K, N, kb, nb, nk
        dev = w_bf16.device
        self.q = torch.empty((E, N, K) if nk else (E, K, N), dtype=torch.uint8, device=dev)
        self.scale = torch.empty((E, kb, 1, nb), dtype=torch.float32, device=dev)
        mode = MOE_SCALE_TENSOR_STATIC if static_scale is not None else MOE_SCALE_ROW_DYNAMIC
        moe_quantize_weights(w_bf16, E, K, N, kb, nb, mode, static_scale or 0.0, 1 if nk else 0, self.q,
                             self.scale, stream=stream)


def concat_columns(w0: QuantizedWeight, w1: QuantizedWeight) -> QuantizedWeight:
    """The two input projections of the gated FFN as one weight of 2N output
    columns ([w0 | w1] along N, scales likewise): one grouped matmul then
    produces a and b side by side, reading each lhs tile once."""
    assert (w0.E, w0.K, w0.N, w0.kb, w0.nb, w0.nk) == (w1.E, w1.K, w1.N, w1.kb, w1.nb, w1.nk)
    w = QuantizedWeight.__new__(QuantizedWeight)
    w.E, w.K, w.N, w.kb, w.nb, w.nk = w0.E, w0.K, 2 * w0.N, w0.kb, 2 * w0.nb, w0.nk
    w.q = torch.cat([w0.q, w1.q], dim=1 if w0.nk else 2).contiguous()
    w.scale = torch.cat([w0.scale, w1.scale], dim=3).contiguous()
    return w


class ForwardPath:
    """Up-projection (``cfg.pipeline == 'up'``) or gated FFN forward."""

    def __init__(self, cfg, data, device="cuda", static_act=None, static_weight=None, nk=True, m_cap=None,
                 share=1, weights_dev=None, fused_quantize=None):
        self.cfg, self.dev = cfg, device
        T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
        self.T, self.H, self.k, self.E = T, H, k, E
        self.g0, self.El = cfg.group_offset, cfg.E_loc
        self.M = T * k
        self.m_cap = self.M if m_cap is None else m_cap
        self.act_mode = MOE_SCALE_TENSOR_STATIC if static_act is not None else MOE_SCALE_ROW_DYNAMIC
        self.static_act = static_act or 0.0
        self.share = share
        # one GPU's own tokens: quantize and sort in one pass (moe_quantize_sort_by_expert); with an
        # expert-parallel share the sort reads the all-gathered fp8 rows, so the two stay separate
        self.fused_quantize = (share == 1) if fused_quantize is None else bool(fused_quantize)
        self.x = bf16_tensor(data["x"], device)
        self.ids = torch.from_numpy(np.ascontiguousarray(data["ids"], dtype=np.int32)).to(device)
        self.topk_w = torch.from_numpy(np.ascontiguousarray(data["topk_w"], dtype=np.float32)).to(device)
        # weights: quantized once on the GPU (setup, not part of a step)
        self.w = {}
        src = weights_dev if weights_dev is not None else {n: bf16_tensor(w, device) for n, w in data["weights"].items()}
        for name, wt in src.items():
            _, K, N = wt.shape
            kb, nb = cfg.scale_blocks(K, N)
            self.w[name] = QuantizedWeight(wt, kb, nb, static_scale=static_weight, nk=nk)
        del src
        N_out = cfg.I if cfg.pipeline == "up" else H
        self.N_out = N_out
        u8, f32, i32, bf = torch.uint8, torch.float32, torch.int32, torch.bfloat16
        self.xq = torch.empty((T, H), dtype=u8, device=device)
        self.xscale = torch.empty((T if self.act_mode == MOE_SCALE_ROW_DYNAMIC else 1,), dtype=f32, device=device)
        self.perm = torch.empty(self.M, dtype=i32, device=device)
        self.inv_pos = torch.empty(self.M, dtype=i32, device=device)
        self.group_sizes = torch.empty(E, dtype=i32, device=device)
        self.xs = torch.empty((self.m_cap, H), dtype=u8, device=device)
        self.ss = torch.empty((self.m_cap,), dtype=f32, device=device)
        self.xamax = torch.empty((T,), dtype=f32, device=device)      # tokens' absmax (fused row-mode pass)
        if cfg.pipeline == "ffn":
            # a and b are the column halves of one [m_cap, 2I] output
            self.w01 = concat_columns(self.w["wi_0"], self.w["wi_1"])
            self.ab = torch.empty((self.m_cap, 2 * cfg.I), dtype=bf, device=device)
            self.a, self.b = self.ab[:, :cfg.I], self.ab[:, cfg.I:]
            self.hq = torch.empty((self.m_cap, cfg.I), dtype=u8, device=device)
            self.hs = torch.empty((self.m_cap,), dtype=f32, device=device)
            self.hamax = torch.empty((self.m_cap,), dtype=f32, device=device)   # rows' absmax of h
        self.y = torch.empty((self.m_cap, N_out), dtype=bf, device=device)
        self.out = torch.empty((T, N_out), dtype=bf, device=device)
        self.ws_q = workspace(MOE_OP_QUANTIZE_ROWS, T, H, self.act_mode, device=device)
        self.ws_sort = workspace(MOE_OP_SORT_BY_EXPERT, self.M, 0, 0, E, device=device)
        self.ws_gmm = workspace(MOE_OP_GMM, self.m_cap, H, N_out, E, device=device)
        if share > 1:
            # slots of the other GPUs: quantized once, as the all-gather would deliver them
            self._quantize(0, T)

    # -- steps -------------------------------------------------------------
    def _quantize(self, r0, rows):
        H = self.H
        xs = self.xscale[r0:r0 + rows] if self.act_mode == MOE_SCALE_ROW_DYNAMIC else self.xscale
        moe_quantize_rows(self.x[r0:r0 + rows], None, MOE_ACT_NONE, rows, H, self.act_mode, self.static_act,
                          self.xq[r0:r0 + rows], xs, None, self.ws_q)

    def quantize(self):
        if self.fused_quantize:
            return                     # done by sort()
        rows = self.T // self.share
        self._quantize(0, rows)        # this GPU's share sits in slot 0

    def sort(self):
        if self.fused_quantize:
            row = self.act_mode == MOE_SCALE_ROW_DYNAMIC
            moe_quantize_sort_by_expert(self.x, self.T, self.H, self.act_mode, self.static_act, self.ids, self.k,
                                        self.E, self.g0, self.El, self.m_cap, self.perm, self.inv_pos,
                                        self.group_sizes, self.xs, self.ss if row else None,
                                        None if row else self.xscale, self.ws_sort,
                                        row_amax=self.xamax if row else None)
            return
        moe_sort_by_expert(self.ids, self.T, self.k, self.E, self.g0, self.El, self.xq, self.xscale,
                           self.act_mode, self.H, self.m_cap, self.perm, self.inv_pos, self.group_sizes,
                           self.xs, self.ss if self.act_mode == MOE_SCALE_ROW_DYNAMIC else None, self.ws_sort)

    def gmm(self, lhs, lhs_scale, lhs_mode, w: QuantizedWeight, out, out_dtype=MOE_BF16):
        moe_gmm_fp8(lhs, lhs_scale, lhs_mode, w.q, w.scale, w.kb, w.nb, 1 if w.nk else 0, self.group_sizes,
                    self.E, self.g0, self.El, self.m_cap, w.K, w.N, out_dtype, out, self.ws_gmm)

    def experts(self):
        ls = self.ss if self.act_mode == MOE_SCALE_ROW_DYNAMIC else self.xscale
        if self.cfg.pipeline == "up":
            self.gmm(self.xs, ls, self.act_mode, self.w["w_up"], self.y)
            return
        self.gmm_gate_up(ls)
        self.silu_quant()
        self.gmm(self.hq, self.hs, MOE_SCALE_ROW_DYNAMIC, self.w["wo"], self.y)

    def gmm_gate_up(self, ls):
        """a = x W0 and b = x W1 for every routed row, as one grouped matmul."""
        self.gmm(self.xs, ls, self.act_mode, self.w01, self.ab)

    def silu_quant(self):
        I = self.cfg.I
        moe_quantize_rows_strided(self.a, self.b, 2 * I, MOE_ACT_SILU_MUL, self.m_cap, I, MOE_SCALE_ROW_DYNAMIC,
                                  0.0, self.hq, self.hs, self.hamax, None)

    def combine(self):
        moe_gather_reduce(self.y, MOE_BF16, self.inv_pos, self.topk_w, self.T, self.k, self.N_out, MOE_BF16,
                          self.out)

    def step(self):
        self.quantize()
        self.sort()
        self.experts()
        self.combine()

    # -- HIP graph of one step ------------------------------------------------
    def capture_graph(self, warmup=2):
        """Record one step (every launch of the path, on one stream) into a HIP
        graph; replay() then runs the step with a single submission.  Every
        buffer a step writes is fully rewritten by it, so replays are
        identical to eager steps."""
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()

    # -- accounting ----------------------------------------------------------
    def gmm_flops(self, n_local):
        """Algorithmic GMM flops of one step for n_local routed local rows."""
        return sum(2 * n_local * w.K * w.N for w in self.w.values())


class BackwardPath:
    """Config-5 backward: dX = gmm(dY, W^T), dW = tgmm(X_sorted, dY)."""

    def __init__(self, cfg, data, static_act, static_weight, device="cuda", dw_dtype=MOE_F32, fused_quantize=True,
                 transposed_x=False):
        self.cfg, self.dev = cfg, device
        # X quantized with its static scale inside the sort's gather (True), or
        # to [T, H] codes by a pass of its own first
        self.fused_quantize = bool(fused_quantize)
        # transposed_x: no sorted X rows at all -- the sort's metadata, then X quantized on its way into the
        # weight-gradient product's transposed layout (moe_sort_gather_transposed), read by moe_tgmm_fp8_xt
        self.transposed_x = bool(transposed_x)
        T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
        self.T, self.H, self.E, self.k, self.I = T, H, E, k, I
        self.M = T * k
        self.g0, self.El = cfg.group_offset, cfg.E_loc
        self.static_act = static_act
        u8, f32, i32, bf = torch.uint8, torch.float32, torch.int32, torch.bfloat16
        self.x = bf16_tensor(data["x"], device)
        self.ids = torch.from_numpy(np.ascontiguousarray(data["ids"], dtype=np.int32)).to(device)
        self.dy = bf16_tensor(data["dy"], device)
        w = bf16_tensor(data["weights"]["w_up"], device)
        # W [E, H, I] is the forward up weight; for dX it is the rhs stored [E, N=H, K=I]
        self.w = QuantizedWeight(w, 1, 1, static_scale=static_weight, nk=False)
        del w
        self.xq = torch.empty((T, H), dtype=u8, device=device)
        self.xscale = torch.empty(1, dtype=f32, device=device)
        self.perm = torch.empty(self.M, dtype=i32, device=device)
        self.inv_pos = torch.empty(self.M, dtype=i32, device=device)
        self.group_sizes = torch.empty(E, dtype=i32, device=device)
        if self.transposed_x:
            self.xt = torch.empty((H, tgmm_xt_cols(self.M, E)), dtype=u8, device=device)
            self.ws_xt = workspace(MOE_OP_GATHER_REDUCE, device=device)
        else:
            self.xs = torch.empty((self.M, H), dtype=u8, device=device)
        self.dyq_r = torch.empty((self.M, I), dtype=u8, device=device)
        self.dys_r = torch.empty(self.M, dtype=f32, device=device)
        self.dyq_t = torch.empty((self.M, I), dtype=u8, device=device)
        self.dys_t = torch.empty(1, dtype=f32, device=device)
        self.dy_amax = torch.empty(self.M, dtype=f32, device=device)
        self.dx = torch.empty((self.M, H), dtype=bf, device=device)
        self.dw_dtype = dw_dtype
        self.dw = torch.empty((self.El, H, I), dtype=f32 if dw_dtype == MOE_F32 else bf, device=device)
        self.ws_q = workspace(MOE_OP_QUANTIZE_ROWS, self.M, I, MOE_SCALE_TENSOR_DYNAMIC, device=device)
        self.ws_sort = workspace(MOE_OP_SORT_BY_EXPERT, self.M, 0, 0, E, device=device)
        self.ws_gmm = workspace(MOE_OP_GMM, self.M, I, H, E, device=device)
        self.ws_tgmm = workspace(MOE_OP_TGMM, self.M, H, I, E, device=device)

    def quantize_and_sort(self):
        if self.transposed_x:
            # (fused_quantize: the bf16 rows are quantized on their way into the layout; otherwise the [T, H]
            # codes come first and the gather moves bytes)
            moe_sort_by_expert(self.ids, self.T, self.k, self.E, self.g0, self.El, None, None, MOE_SCALE_TENSOR_STATIC,
                               self.H, self.M, self.perm, self.inv_pos, self.group_sizes, None, None, self.ws_sort)
            if self.fused_quantize:
                moe_sort_gather_transposed(self.x, MOE_BF16, self.static_act, self.T, self.k, self.H, self.perm,
                                           self.group_sizes, self.E, self.g0, self.El, self.M, self.xt, self.xscale,
                                           self.ws_xt)
            else:
                moe_quantize_rows(self.x, None, MOE_ACT_NONE, self.T, self.H, MOE_SCALE_TENSOR_STATIC,
                                  self.static_act, self.xq, self.xscale, None, None)
                moe_sort_gather_transposed(self.xq, MOE_E4M3FN, 1.0, self.T, self.k, self.H, self.perm,
                                           self.group_sizes, self.E, self.g0, self.El, self.M, self.xt, None,
                                           self.ws_xt)
            return
        if self.fused_quantize:
            moe_quantize_sort_by_expert(self.x, self.T, self.H, MOE_SCALE_TENSOR_STATIC, self.static_act, self.ids,
                                        self.k, self.E, self.g0, self.El, self.M, self.perm, self.inv_pos,
                                        self.group_sizes, self.xs, None, self.xscale, self.ws_sort)
            return
        moe_quantize_rows(self.x, None, MOE_ACT_NONE, self.T, self.H, MOE_SCALE_TENSOR_STATIC, self.static_act,
                          self.xq, self.xscale, None, None)
        moe_sort_by_expert(self.ids, self.T, self.k, self.E, self.g0, self.El, self.xq, self.xscale,
                           MOE_SCALE_TENSOR_STATIC, self.H, self.M, self.perm, self.inv_pos, self.group_sizes,
                           self.xs, None, self.ws_sort)

    def quantize_dy(self):
        # per-row codes (for dX), then per-tensor codes (for dW) scaled from the row pass's maxima
        moe_quantize_rows(self.dy, None, MOE_ACT_NONE, self.M, self.I, MOE_SCALE_ROW_DYNAMIC, 0.0, self.dyq_r,
                          self.dys_r, self.dy_amax, None)
        moe_quantize_rows(self.dy, None, MOE_ACT_NONE, self.M, self.I, MOE_SCALE_TENSOR_FROM_ROW_AMAX, 0.0,
                          self.dyq_t, self.dys_t, self.dy_amax, None)

    def grad_input(self):
        moe_gmm_fp8(self.dyq_r, self.dys_r, MOE_SCALE_ROW_DYNAMIC, self.w.q, self.w.scale, 1, 1, 1,
                    self.group_sizes, self.E, self.g0, self.El, self.M, self.I, self.H, MOE_BF16, self.dx,
                    self.ws_gmm)

    def grad_weight(self):
        if self.transposed_x:
            moe_tgmm_fp8_xt(self.xt, self.xscale, 1, self.dyq_t, self.dys_t, 1, self.group_sizes, self.E, self.g0,
                            self.El, self.M, self.H, self.I, self.dw_dtype, self.dw, self.ws_tgmm)
            return
        moe_tgmm_fp8(self.xs, self.xscale, 1, self.dyq_t, self.dys_t, 1, self.group_sizes, self.E, self.g0,
                     self.El, self.M, self.H, self.I, self.dw_dtype, self.dw, self.ws_tgmm)

    def step(self):
        self.quantize_and_sort()
        self.quantize_dy()
        self.grad_input()
        self.grad_weight()

    @property
    def OUTPUTS(self):
        x_out = (() if self.fused_quantize else ("xq",)) + (("xt",) if self.transposed_x else ("xs",))
        return (x_out + ("xscale", "perm", "inv_pos", "group_sizes", "dyq_r", "dys_r", "dyq_t", "dys_t", "dy_amax",
                         "dx", "dw"))

    def capture_graph(self, warmup=1):
        """Record one backward step into a HIP graph (every buffer it writes is
        fully rewritten by it, so replays equal eager steps)."""
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()


class FFNBackwardPath:
    """The gated FFN's backward after a forward step of ``fwd`` (a
    ForwardPath with ``pipeline == 'ffn'``), for an upstream gradient
    ``dout`` [T, H] bf16 of the combined token rows:

      combine backward  dy = w * dout to the sorted rows, dw_router per slot
      dh   = gmm(dy, wo^T)            per-row dy scales, wo^T quantized per channel
      dwo  = tgmm(h, dy)              h requantized with one tensor scale
      da, db = SiLU*mul backward(a, b, dh), written as [da | db]
      dxs  = gmm([da | db], [W0 | W1]^T)   one launch, K = 2I
      dw01 = tgmm(x, [da | db])       x requantized with one tensor scale
      dx   = unit-weight gather-reduce of dxs back to token rows

    The forward's per-output-channel weight scales vary along the backward's
    contraction, so the backward quantizes the transposed weights with scales
    per its own output channel; tgmm needs scales constant along the
    contracted rows, so its operands use per-tensor dynamic scales (per-row
    scales serve the gmm inputs).  Weight gradients come out in float32
    ([E, I, H] for wo, [E, H, 2I] for [W0 | W1])."""

    def __init__(self, fwd, data, dout: torch.Tensor, device="cuda", fuse_dy_quant=True, transposed_x=False):
        cfg = fwd.cfg
        assert cfg.pipeline == "ffn"
        # dy's per-row quantization formed by the combine backward (True) or as a pass of its own
        self.fuse_dy_quant = fuse_dy_quant
        # transposed_x: dW01's x as [T, H] codes with one tensor scale, gathered by the forward's sort
        # straight into the weight-gradient product's transposed layout (no second sort, no sorted x rows)
        self.transposed_x = bool(transposed_x)
        T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
        self.fwd, self.cfg = fwd, cfg
        self.T, self.H, self.E, self.k, self.I = T, H, E, k, I
        Mc = fwd.m_cap
        self.m_cap = Mc
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        self.dout = dout
        # backward weights (set-up): transposed, quantized per channel of the backward's output
        wo = bf16_tensor(data["weights"]["wo"], device)                       # [E, I, H]
        self.woT = QuantizedWeight(wo.transpose(1, 2).contiguous(), 1, I)      # as [E, K=H, N=I]
        del wo
        w01 = torch.cat([bf16_tensor(data["weights"]["wi_0"], device), bf16_tensor(data["weights"]["wi_1"], device)],
                        dim=2)                                                  # [E, H, 2I]
        self.w01T = QuantizedWeight(w01.transpose(1, 2).contiguous(), 1, H)    # as [E, K=2I, N=H]
        del w01
        self.ones = torch.ones((T, k), dtype=f32, device=device)
        self.dy = torch.empty((Mc, H), dtype=bf, device=device)
        self.dw_router = torch.empty((T, k), dtype=f32, device=device)
        self.dyq_r = torch.empty((Mc, H), dtype=u8, device=device)
        self.dys_r = torch.empty((Mc,), dtype=f32, device=device)
        self.dyq_t = torch.empty((Mc, H), dtype=u8, device=device)
        self.dys_t = torch.empty((1,), dtype=f32, device=device)
        self.dy_amax = torch.empty((Mc,), dtype=f32, device=device)
        self.dh = torch.empty((Mc, I), dtype=bf, device=device)
        self.hq_t = torch.empty((Mc, I), dtype=u8, device=device)
        self.hs_t = torch.empty((1,), dtype=f32, device=device)
        self.dwo = torch.empty((cfg.E_loc, I, H), dtype=f32, device=device)
        self.dab = torch.empty((Mc, 2 * I), dtype=bf, device=device)
        self.dabq_r = torch.empty((Mc, 2 * I), dtype=u8, device=device)
        self.dabs_r = torch.empty((Mc,), dtype=f32, device=device)
        self.dabq_t = torch.empty((Mc, 2 * I), dtype=u8, device=device)
        self.dabs_t = torch.empty((1,), dtype=f32, device=device)
        self.dab_amax = torch.empty((Mc,), dtype=f32, device=device)
        self.dxs = torch.empty((Mc, H), dtype=bf, device=device)
        self.xq_t = torch.empty((T, H), dtype=u8, device=device)
        self.xs_scale = torch.empty((1,), dtype=f32, device=device)
        if self.transposed_x:
            self.xt = torch.empty((H, tgmm_xt_cols(Mc, E)), dtype=u8, device=device)
            self.ws_xt = workspace(MOE_OP_GATHER_REDUCE, device=device)
        else:
            self.perm = torch.empty(T * k, dtype=torch.int32, device=device)
            self.inv_pos = torch.empty(T * k, dtype=torch.int32, device=device)
            self.group_sizes = torch.empty(E, dtype=torch.int32, device=device)
            self.xs_t = torch.empty((Mc, H), dtype=u8, device=device)
        self.dw01 = torch.empty((cfg.E_loc, H, 2 * I), dtype=f32, device=device)
        self.dx = torch.empty((T, H), dtype=bf, device=device)
        C = max(H, 2 * I)
        self.ws_q = workspace(MOE_OP_QUANTIZE_ROWS, Mc, C, MOE_SCALE_TENSOR_DYNAMIC, device=device)
        self.ws_qx = workspace(MOE_OP_QUANTIZE_ROWS, T, H, MOE_SCALE_TENSOR_DYNAMIC, device=device)
        self.ws_sort = workspace(MOE_OP_SORT_BY_EXPERT, T * k, 0, 0, E, device=device)
        self.ws_gmm_h = workspace(MOE_OP_GMM, Mc, H, I, E, device=device)
        self.ws_gmm_x = workspace(MOE_OP_GMM, Mc, 2 * I, H, E, device=device)
        self.ws_tgmm_o = workspace(MOE_OP_TGMM, Mc, I, H, E, device=device)
        self.ws_tgmm_01 = workspace(MOE_OP_TGMM, Mc, H, 2 * I, E, device=device)

    def _gmm(self, lhs, ls, w: QuantizedWeight, out, ws):
        f = self.fwd
        moe_gmm_fp8(lhs, ls, MOE_SCALE_ROW_DYNAMIC, w.q, w.scale, w.kb, w.nb, 1, f.group_sizes, self.E, f.g0, f.El,
                    self.m_cap, w.K, w.N, MOE_BF16, out, ws)

    def _tgmm(self, lhs, ls, rhs, rs, K, N, out, ws):
        f = self.fwd
        moe_tgmm_fp8(lhs, ls, 1, rhs, rs, 1, f.group_sizes, self.E, f.g0, f.El, self.m_cap, K, N, MOE_F32, out, ws)

    # -- steps -------------------------------------------------------------
    def combine_backward(self):
        f = self.fwd
        fq = self.fuse_dy_quant
        # dy, and (fused) its per-row codes, scales and row maxima from the same registers
        moe_gather_reduce_backward(self.dout, f.y, f.inv_pos, f.topk_w, self.T, self.k, self.H, f.group_sizes,
                                   self.E, f.g0, f.El, self.m_cap, self.dy, self.dw_router,
                                   self.dyq_r if fq else None, self.dys_r if fq else None,
                                   self.dy_amax if fq else None)

    def quantize_dy(self):
        """Per-row codes of dy unless the combine backward formed them, then
        per-tensor codes whose scale comes from the row maxima (the
        tensor-dynamic result without an absmax pass)."""
        Mc, H = self.m_cap, self.H
        if not self.fuse_dy_quant:
            moe_quantize_rows(self.dy, None, MOE_ACT_NONE, Mc, H, MOE_SCALE_ROW_DYNAMIC, 0.0, self.dyq_r, self.dys_r,
                              self.dy_amax)
        moe_quantize_rows(self.dy, None, MOE_ACT_NONE, Mc, H, MOE_SCALE_TENSOR_FROM_ROW_AMAX, 0.0, self.dyq_t,
                          self.dys_t, self.dy_amax)

    def grad_h(self):
        self._gmm(self.dyq_r, self.dys_r, self.woT, self.dh, self.ws_gmm_h)

    def grad_wo(self):
        f, I = self.fwd, self.I
        # h with one tensor scale, from the row maxima of h that the forward's requantization wrote
        moe_quantize_rows_strided(f.a, f.b, 2 * I, MOE_ACT_SILU_MUL, self.m_cap, I, MOE_SCALE_TENSOR_FROM_ROW_AMAX,
                                  0.0, self.hq_t, self.hs_t, f.hamax)
        self._tgmm(self.hq_t, self.hs_t, self.dyq_t, self.dys_t, I, self.H, self.dwo, self.ws_tgmm_o)

    def silu_backward(self):
        f, I = self.fwd, self.I
        moe_silu_mul_backward(f.a, f.b, 2 * I, self.dh, self.m_cap, I, self.dab[:, :I], self.dab[:, I:], 2 * I)

    def quantize_dab(self):
        Mc, C = self.m_cap, 2 * self.I
        moe_quantize_rows(self.dab, None, MOE_ACT_NONE, Mc, C, MOE_SCALE_ROW_DYNAMIC, 0.0, self.dabq_r, self.dabs_r,
                          self.dab_amax)
        moe_quantize_rows(self.dab, None, MOE_ACT_NONE, Mc, C, MOE_SCALE_TENSOR_FROM_ROW_AMAX, 0.0, self.dabq_t,
                          self.dabs_t, self.dab_amax)

    def grad_x_sorted(self):
        self._gmm(self.dabq_r, self.dabs_r, self.w01T, self.dxs, self.ws_gmm_x)

    def grad_w01(self):
        f, T, H = self.fwd, self.T, self.H
        if self.transposed_x:
            if f.fused_quantize and f.act_mode == MOE_SCALE_ROW_DYNAMIC:   # the scale from the forward's maxima
                moe_quantize_rows(f.x, None, MOE_ACT_NONE, T, H, MOE_SCALE_TENSOR_FROM_ROW_AMAX, 0.0, self.xq_t,
                                  self.xs_scale, f.xamax)
            else:
                moe_quantize_rows(f.x, None, MOE_ACT_NONE, T, H, MOE_SCALE_TENSOR_DYNAMIC, 0.0, self.xq_t,
                                  self.xs_scale, None, self.ws_qx)
            moe_sort_gather_transposed(self.xq_t, MOE_E4M3FN, 1.0, T, self.k, H, f.perm, f.group_sizes, self.E,
                                       f.g0, f.El, self.m_cap, self.xt, None, self.ws_xt)
            moe_tgmm_fp8_xt(self.xt, self.xs_scale, 1, self.dabq_t, self.dabs_t, 1, f.group_sizes, self.E, f.g0,
                            f.El, self.m_cap, H, 2 * self.I, MOE_F32, self.dw01, self.ws_tgmm_01)
            return
        if f.fused_quantize and f.act_mode == MOE_SCALE_ROW_DYNAMIC:
            # x with one tensor scale (from the token maxima the forward's fused pass wrote), quantized
            # straight into the sorted rows
            moe_quantize_sort_by_expert(f.x, T, H, MOE_SCALE_TENSOR_FROM_ROW_AMAX, 0.0, f.ids, self.k, self.E, f.g0,
                                        f.El, self.m_cap, self.perm, self.inv_pos, self.group_sizes, self.xs_t, None,
                                        self.xs_scale, self.ws_sort, row_amax=f.xamax)
        else:
            moe_quantize_rows(f.x, None, MOE_ACT_NONE, T, H, MOE_SCALE_TENSOR_DYNAMIC, 0.0, self.xq_t, self.xs_scale,
                              None, self.ws_qx)
            moe_sort_by_expert(f.ids, T, self.k, self.E, f.g0, f.El, self.xq_t, self.xs_scale,
                               MOE_SCALE_TENSOR_DYNAMIC, H, self.m_cap, self.perm, self.inv_pos, self.group_sizes,
                               self.xs_t, None, self.ws_sort)
        self._tgmm(self.xs_t, self.xs_scale, self.dabq_t, self.dabs_t, H, 2 * self.I, self.dw01, self.ws_tgmm_01)

    def grad_x(self):
        moe_gather_reduce(self.dxs, MOE_BF16, self.fwd.inv_pos, self.ones, self.T, self.k, self.H, MOE_BF16, self.dx)

    def step(self):
        self.combine_backward()
        self.quantize_dy()
        self.grad_h()
        self.grad_wo()
        self.silu_backward()
        self.quantize_dab()
        self.grad_x_sorted()
        self.grad_w01()
        self.grad_x()

    @property
    def OUTPUTS(self):
        x_out = ("xq_t", "xt") if self.transposed_x else ("perm", "inv_pos", "group_sizes", "xs_t")
        return (("dy", "dw_router", "dyq_r", "dys_r", "dyq_t", "dys_t", "dy_amax", "dh", "hq_t", "hs_t", "dwo", "dab",
                 "dabq_r", "dabs_r", "dabq_t", "dabs_t", "dab_amax", "dxs", "xs_scale") + x_out + ("dw01", "dx"))

    def capture_graph(self, warmup=1):
        """Record one backward step into a HIP graph (every buffer it writes is
        fully rewritten by it, so replays equal eager steps)."""
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()
