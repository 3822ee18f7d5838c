"""GroupedLinear-style training wrapper over the C ABI: the expert layer whose
forward is the grouped forward GEMM and whose backward is the grouped input
gradient plus the variable-K weight gradient, with

- the weights quantized once per weight version and reused by every
  microbatch until the optimizer changes them (a cache keyed on the tensor's
  storage and version counter);
- the weight gradient accumulated in place into an fp32 ``main_grad`` (the
  fused accumulation of the pages' GroupedLinear integration), so autograd
  sees no weight gradient;
- an optional delayed weight gradient: its quantized operands are kept and
  ``backward_dw()`` launches them later (for pipeline schedules that split
  the input and weight gradients);
- ``is_first_microbatch`` (None: quantize whenever the weight changed; True:
  quantize now; False: reuse the cached quantization, and fail loudly if
  there is none or it does not fit the layer);
- ``weight.overwrite_main_grad``: when True at a backward, that backward's
  weight gradient overwrites ``main_grad`` (experts with no tokens become
  zero) instead of adding to it -- the first microbatch of an accumulation;
- caller-provided ``out`` (forward output) and ``dgrad_out`` (input gradient)
  buffers, written in place and returned (aliased).

Pages: "Triton mxfp4 (and a8w4) grouped GEMM kernel" (the GroupedLinear
integration, a4w4 and a8w4), "Add ROCm Triton blockwise FP8 grouped GEMM"
(blockwise FP8, the weight-quantization cache across microbatches with
is_first_microbatch, fused main_grad accumulation and the first-microbatch
logic, overwrite_main_grad) and "route te.GroupedLinear through #723; a8w4
fwd-only" (its review: preallocated out and dgrad_out buffers are honoured). Every step runs in libmxgg's kernels; this file only
orders the calls and keeps the quantized operands between forward and
backward. Tensors must live on the GPU: the library rejects anything else.

Recipes (activation, weight, gradient formats):
  "a4w4"      MXFP4 x MXFP4 everywhere;
  "a8w4"      activations and output gradients MXFP8, weights MXFP4 (the
              weight gradient contracts two MXFP8 operands);
  "blockwise" 1x128 activations / gradients and 128x128 weights, E4M3 with
              power-of-two scales (the input gradient reads the weights'
              blocks transposed).
When in_features and out_features are multiples of 128, the MX recipes keep
every row-wise code tensor (activations, output gradients, weights along K)
and the weights along N in 64-byte K blocks (MXGG_KBLOCK_ROWS /
MXGG_KBLOCK_COLS: the forward's and the input gradient's operand stages
become contiguous runs; the results are the same bits); the weight
gradient's column-wise operands stay in rows. Blockwise codes are always
K-blocked.
"""
import torch

from . import _lib as L

RECIPES = {
    "a4w4": dict(act="mxfp4", wgt="mxfp4", grad="mxfp4"),
    "a8w4": dict(act="mxfp8", wgt="mxfp4", grad="mxfp8"),
    "blockwise": dict(act="fp8_1x128_p2", wgt="fp8_128x128_p2", grad="fp8_1x128_p2"),
}


def _formats(recipe, N, K):
    """The format (with its code-layout bits) of each call of a recipe for a
    layer of K inputs and N outputs."""
    r = RECIPES[recipe]
    if recipe == "blockwise" or K % 128 or N % 128:
        return dict(act=r["act"], wgt_q=r["wgt"], fwd_w=r["wgt"], grad=r["grad"], dgrad=r["grad"], wgrad=r["grad"])
    kr, kc = L.KBLOCK_ROWS, L.KBLOCK_COLS
    act, wgt, grad = L.FORMATS[r["act"]], L.FORMATS[r["wgt"]], L.FORMATS[r["grad"]]
    return dict(act=act | kr, wgt_q=wgt | kr | kc, fwd_w=wgt | kr, grad=grad | kr, dgrad=grad | kr | kc, wgrad=grad)


def _code_rows(q):
    """Rows of a code tensor: [rows, bytes] or K-blocked [bytes/64, rows, 64]."""
    return q.shape[1] if q.dim() == 3 else q.shape[0]


class _WeightCache:
    """Quantized weights of one parameter for the forward and for the input
    gradient, rebuilt when the parameter's storage or version changes."""

    def __init__(self):
        self.key = None
        self.fwd = None   # (q, s)
        self.dgrad = None  # (q, s)

    def get(self, weight, recipe, G, N, K, is_first_microbatch=None):
        key = (weight.data_ptr(), weight._version, recipe)
        if is_first_microbatch is False:
            # reuse without checking the version (the caller promises the
            # weight is unchanged); refuse a cache that cannot serve the layer
            if self.fwd is None or self.key[2] != recipe or self.key[0] != weight.data_ptr() \
                    or self.fwd[0].device != weight.device or _code_rows(self.fwd[0]) != G * N:
                raise RuntimeError("is_first_microbatch=False but no compatible cached weight quantization exists "
                                   "(run a microbatch with is_first_microbatch=True or None first)")
            return self.fwd, self.dgrad
        if is_first_microbatch or key != self.key:
            f = _formats(recipe, N, K)
            if recipe == "blockwise":
                q, s = L.mxgg_quantize_rowwise(weight, f["wgt_q"])
                self.fwd = (q, s)
                self.dgrad = L.mxgg_transpose_128x128(q, s, G, N, K)
            else:
                # row-wise along K for the forward, along N (segments of N
                # rows per expert) for the input gradient, from one read
                qr, sr, qc, sc, _ = L.mxgg_quantize_dual(weight, [N] * G, f["wgt_q"])
                self.fwd, self.dgrad = (qr, sr), (qc, sc)
            self.key = key
        return self.fwd, self.dgrad


def _quantize_act(x, m_splits, fmt, need_col):
    """Row-wise (forward or input gradient) and, when needed, column-wise
    segment-padded (weight gradient) quantization of an activation or a
    gradient; both from one read when both are needed (MX and blockwise)."""
    if need_col:
        qr, sr, qc, sc, mpad = L.mxgg_quantize_dual(x, m_splits, fmt)
        return (qr, sr), (qc, sc, mpad)
    return L.mxgg_quantize_rowwise(x, fmt), None


class _GroupedLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, m_splits, module, is_first_microbatch, out, dgrad_out):
        G, N, K, recipe = module.num_experts, module.out_features, module.in_features, module.recipe
        f = _formats(recipe, N, K)
        (wq, ws), wdgrad = module._cache.get(weight, recipe, G, N, K, is_first_microbatch)
        need_wgrad = ctx.needs_input_grad[1]
        xrow, xcol = _quantize_act(x, m_splits, f["act"], need_wgrad)
        y = L.mxgg_grouped_fwd(xrow[0], xrow[1], wq, ws, m_splits, N, K, a_fmt=f["act"], w_fmt=f["fwd_w"], out=out)
        ctx.module, ctx.m_splits, ctx.wdgrad, ctx.xcol = module, m_splits, wdgrad, xcol
        ctx.need_dx = ctx.needs_input_grad[0]
        ctx.dgrad_out = dgrad_out
        if out is not None:
            ctx.mark_dirty(out)
        return y

    @staticmethod
    def backward(ctx, dy):
        module, m_splits = ctx.module, ctx.m_splits
        G, N, K, recipe = module.num_experts, module.out_features, module.in_features, module.recipe
        f = _formats(recipe, N, K)
        dy = dy.contiguous()
        need_wgrad = ctx.xcol is not None
        drow, dcol = _quantize_act(dy, m_splits, f["grad"], need_wgrad)
        dx = None
        if ctx.need_dx:
            dx = L.mxgg_grouped_dgrad(drow[0], drow[1], ctx.wdgrad[0], ctx.wdgrad[1], m_splits, N, K,
                                      fmt=f["dgrad"], dx=ctx.dgrad_out)
        if need_wgrad:
            # the accumulation mode is the one in force at this backward
            accumulate = not getattr(module.weight, "overwrite_main_grad", False)
            job = (dcol[0], dcol[1], ctx.xcol[0], ctx.xcol[1], m_splits, dcol[2], accumulate)
            if module.delay_wgrad:
                module._pending.append(job)
            else:
                module._run_wgrad(job)
        ctx.xcol = ctx.wdgrad = ctx.dgrad_out = None
        return dx, None, None, None, None, None, None


class GroupedLinear(torch.nn.Module):
    """y[r] = x[r] . W_g^T for the rows r of expert g; weight bf16 [G*N, K]
    (expert g owns rows [g*N, (g+1)*N)), main_grad fp32 [G, N, K]."""

    def __init__(self, num_experts, in_features, out_features, recipe="a4w4", delay_wgrad=False, device=None,
                 weight_std=0.02, generator=None):
        super().__init__()
        if recipe not in RECIPES:
            raise ValueError(f"recipe {recipe!r} is not one of {sorted(RECIPES)}")
        self.num_experts, self.in_features, self.out_features = num_experts, in_features, out_features
        self.recipe, self.delay_wgrad = recipe, delay_wgrad
        device = torch.device("cuda") if device is None else torch.device(device)
        w = torch.randn((num_experts * out_features, in_features), device=device, generator=generator) * weight_std
        self.weight = torch.nn.Parameter(w.to(torch.bfloat16))
        self.weight.main_grad = torch.zeros((num_experts, out_features, in_features), dtype=torch.float32,
                                            device=device)
        self.weight.overwrite_main_grad = False
        self._cache = _WeightCache()
        self._pending = []

    def forward(self, x, m_splits, is_first_microbatch=None, out=None, dgrad_out=None):
        """x bf16 [M, K]; out: optional bf16 [M, N] written and returned;
        dgrad_out: optional bf16 [M, K] that receives the input gradient."""
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != self.in_features:
            raise ValueError(f"x must be bf16 [M, {self.in_features}], got {tuple(x.shape)} {x.dtype}")
        M = x.shape[0]
        for name, buf, shape in (("out", out, (M, self.out_features)), ("dgrad_out", dgrad_out, (M, self.in_features))):
            if buf is not None and (buf.dtype != torch.bfloat16 or tuple(buf.shape) != shape
                                    or not buf.is_contiguous() or buf.device != x.device):
                raise ValueError(f"{name} must be a contiguous bf16 {shape} tensor on {x.device}")
        m_splits = [int(m) for m in m_splits]
        return _GroupedLinearFn.apply(x, self.weight, m_splits, self, is_first_microbatch, out, dgrad_out)

    def _run_wgrad(self, job):
        dq, ds, xq, xs, m_splits, mpad, accumulate = job
        L.mxgg_grouped_wgrad(dq, ds, xq, xs, m_splits, self.out_features, self.in_features, mpad,
                             self.weight.main_grad, accumulate=accumulate, fmt=_formats(self.recipe, self.out_features, self.in_features)["wgrad"])

    def backward_dw(self):
        """Launch the delayed weight gradients, oldest first."""
        jobs, self._pending = self._pending, []
        for job in jobs:
            self._run_wgrad(job)
