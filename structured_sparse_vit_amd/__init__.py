"""SparseSAM encoder-block hot path on MI355X: Python binding of libsparsesam.so.

Argument marshalling only: every step of the path runs in the HIP kernels behind
the C ABI in include/sparsesam.h. torch provides device memory and the current
stream. If the library is not built, every call raises.

    plan = Plan.from_config(cfg)              # static pattern + sizes
    imp = importance(img)                     # [b, H, W] fp32 -> [b, tokens]
    perm, inv, routed = permute(plan, imp)    # stripe-sort + keep-set
    block(plan, weights, x, perm, routed)     # one encoder block, in place on x
    forward(plan, weights, img, x)            # importance + permute + block in one call
    encoder(plan_g, plan_w, layers, kinds, x, perms)   # a stack of blocks, in place on x
"""
import ctypes

import torch

from . import _lib
from ._lib import SPARSESAM_BF16, SPARSESAM_F32, SparseSAMError, check

__all__ = ["Plan", "importance", "permute", "attn", "mlp", "block", "forward", "block_noalloc",
           "noalloc_scratch_bytes", "route_topk", "block_dynamic", "encoder", "SparseSAMError", "library_path",
           "weights_to_device"]


def library_path() -> str:
    return _lib.LIB_PATH


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


# token orders ahead of the stripe-sort, in the C enum's order (sparsesam_ordering)
ORDERINGS = ("importance", "zorder", "hilbert", "random")
# how a block picks its MLP keep-set, in the C enum's order (sparsesam_routing)
ROUTINGS = ("importance", "update")


class Plan:
    """Static description of one block type: segments, stripe-sort pattern, keep-set size."""

    def __init__(self, grid_h, grid_w, window, stripes, block, global_tokens, band_radius, attn_density,
                 mlp_density, channels, heads, head_dim, mlp_hidden, max_batch, dtype, ordering="importance",
                 order_seed=0, rel_pos=False, routing="importance", mlp_merge=False):
        lib = _lib.load()
        self._lib = lib
        self.dtype = dtype
        if ordering not in ORDERINGS:
            raise ValueError("ordering must be one of %s" % (ORDERINGS,))
        if routing not in ROUTINGS:
            raise ValueError("routing must be one of %s" % (ROUTINGS,))
        self.routing = routing
        self.desc = _lib.PlanDesc(grid_h, grid_w, window, stripes, block, global_tokens, band_radius,
                                  attn_density, mlp_density, channels, heads, head_dim, mlp_hidden, max_batch,
                                  SPARSESAM_BF16 if dtype == "bf16" else SPARSESAM_F32, ORDERINGS.index(ordering),
                                  order_seed & 0xFFFFFFFF, 1 if rel_pos else 0, ROUTINGS.index(routing),
                                  1 if mlp_merge else 0)
        h = ctypes.c_void_p()
        check(lib.sparsesam_plan_create(ctypes.byref(self.desc), ctypes.byref(h)), "sparsesam_plan_create")
        self._h = h
        info = _lib.PlanInfo()
        check(lib.sparsesam_plan_get_info(self._h, ctypes.byref(info)), "sparsesam_plan_get_info")
        self.info = {f: getattr(info, f) for f, _ in _lib.PlanInfo._fields_ if f != "reserved0"}
        self.device = torch.device("cuda", info.device) if info.has_device_copy else None

    @classmethod
    def from_config(cls, cfg, max_batch=None, rel_pos=False):
        return cls(cfg.grid, cfg.grid, cfg.window, cfg.stripes, cfg.block, cfg.global_tokens, cfg.band_radius,
                   cfg.attn_density, cfg.mlp_density, cfg.channels, cfg.heads, cfg.head_dim, cfg.mlp_hidden,
                   max_batch or cfg.batch, cfg.dtype, getattr(cfg, "ordering", "importance"),
                   getattr(cfg, "order_seed", 0), rel_pos, getattr(cfg, "routing", "importance"),
                   bool(getattr(cfg, "mlp_merge", False)))

    @property
    def handle(self):
        return self._h

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def tile_list(self):
        import numpy as np
        rp = np.zeros(self.info["tiles"] + 1, np.int32)
        ci = np.zeros(max(1, self.info["tiles_kept"]), np.int32)
        check(self._lib.sparsesam_plan_tile_list(self._h, rp.ctypes.data_as(ctypes.c_void_p),
                                                 ci.ctypes.data_as(ctypes.c_void_p)), "sparsesam_plan_tile_list")
        return rp, ci[:self.info["tiles_kept"]]

    def close(self):
        if getattr(self, "_h", None):
            self._lib.sparsesam_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def importance(img, patch=16, out=None):
    """Sobel-magnitude token importance: img [b, H, W] fp32 -> [b, (H/patch)*(W/patch)] fp32."""
    lib = _lib.load()
    if img.dim() != 3:
        raise ValueError("img must be [batch, height, width]")
    _need(img, "img", torch.float32)
    b, H, W = img.shape
    if out is None:
        out = torch.empty(b, (H // patch) * (W // patch), dtype=torch.float32, device=img.device)
    _need(out, "out", torch.float32, (b, (H // patch) * (W // patch)), img.device)
    check(lib.sparsesam_importance(_ptr(img), b, H, W, patch, _ptr(out), _stream(img.device)),
          "sparsesam_importance")
    return out


def permute(plan, imp, out=None):
    """Stripe-sort permutation and keep-set: returns (perm, inv, routed), int32 on the device."""
    lib = _lib.load()
    tokens = plan.desc.grid_h * plan.desc.grid_w
    _need(imp, "imp", torch.float32, device=plan.device)
    if imp.dim() != 2 or imp.shape[1] != tokens:
        raise ValueError("imp must be [batch, %d]" % tokens)
    b = imp.shape[0]
    n, segs, rpi = plan.info["seq_len"], plan.info["segments_per_image"], plan.info["routed_per_image"]
    if out is None:
        perm = torch.empty(b * segs, n, dtype=torch.int32, device=imp.device)
        inv = torch.empty_like(perm)
        routed = torch.empty(b * rpi, dtype=torch.int32, device=imp.device)
    else:
        perm, inv, routed = out
    _need(perm, "perm", torch.int32, (b * segs, n), imp.device)
    _need(inv, "inv", torch.int32, (b * segs, n), imp.device)
    _need(routed, "routed", torch.int32, (b * rpi,), imp.device)
    check(lib.sparsesam_permute(plan.handle, _ptr(imp), b, _ptr(perm), _ptr(inv), _ptr(routed),
                                _stream(imp.device)), "sparsesam_permute")
    return perm, inv, routed


def attn(plan, q, k, vt, scale=None, out=None, workspace=None):
    """Block-sparse attention on stripe-sorted tokens.

    q, k [segments, heads, N, D]; vt [segments, heads, D, N_pad] -> o [segments, N, heads * D].
    """
    lib = _lib.load()
    dt = plan.torch_dtype
    H, D, n = plan.desc.heads, plan.desc.head_dim, plan.info["seq_len"]
    n_pad = (n + 7) // 8 * 8
    segs = q.shape[0]
    _need(q, "q", dt, (segs, H, n, D), plan.device)
    _need(k, "k", dt, (segs, H, n, D), plan.device)
    _need(vt, "vt", dt, (segs, H, D, n_pad), plan.device)
    if out is None:
        out = torch.empty(segs, n, H * D, dtype=dt, device=q.device)
    _need(out, "out", dt, (segs, n, H * D), plan.device)
    scale = D ** -0.5 if scale is None else float(scale)
    per_seg = plan.info["attn_workspace_bytes"] // max(1, plan.desc.max_batch * plan.info["segments_per_image"])
    ws = _workspace(per_seg * segs, q.device, workspace)
    check(lib.sparsesam_attn(plan.handle, segs, _ptr(q), _ptr(k), _ptr(vt), _ptr(out), scale, _ptr(ws), ws.numel(),
                             _stream(q.device)), "sparsesam_attn")
    return out


def attn_relpos(plan, q, k, vt, perm, rel_h, rel_w, scale=None, out=None, workspace=None):
    """Block-sparse attention with the decomposed relative-position bias.

    q, k [segments, heads, N, D]; vt [segments, heads, D, N_pad]; perm [segments, N] int32
    (slot of each position); rel_h [2 Sh - 1, D], rel_w [2 Sw - 1, D] fp32 -> o [segments,
    N, heads * D].
    """
    lib = _lib.load()
    dt = plan.torch_dtype
    H, D, n = plan.desc.heads, plan.desc.head_dim, plan.info["seq_len"]
    n_pad = (n + 7) // 8 * 8
    segs = q.shape[0]
    sh_, sw_ = (plan.desc.window, plan.desc.window) if plan.desc.window else (plan.desc.grid_h, plan.desc.grid_w)
    _need(q, "q", dt, (segs, H, n, D), plan.device)
    _need(k, "k", dt, (segs, H, n, D), plan.device)
    _need(vt, "vt", dt, (segs, H, D, n_pad), plan.device)
    _need(perm, "perm", torch.int32, (segs, n), plan.device)
    _need(rel_h, "rel_h", torch.float32, (2 * sh_ - 1, D), plan.device)
    _need(rel_w, "rel_w", torch.float32, (2 * sw_ - 1, D), plan.device)
    if out is None:
        out = torch.empty(segs, n, H * D, dtype=dt, device=q.device)
    _need(out, "out", dt, (segs, n, H * D), plan.device)
    scale = D ** -0.5 if scale is None else float(scale)
    per_seg = plan.info["relpos_workspace_bytes"] // max(1, plan.desc.max_batch * plan.info["segments_per_image"])
    ws = _workspace(per_seg * segs, q.device, workspace)
    check(lib.sparsesam_attn_relpos(plan.handle, segs, _ptr(q), _ptr(k), _ptr(vt), _ptr(out), scale, _ptr(perm),
                                    _ptr(rel_h), _ptr(rel_w), _ptr(ws), ws.numel(), _stream(q.device)),
          "sparsesam_attn_relpos")
    return out


def _workspace(nbytes, device, workspace):
    if workspace is None:
        return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
    _need(workspace, "workspace", torch.uint8, device=device)
    return workspace


def mlp(plan, x, routed, ln_g, ln_b, w1, b1, w2, b2, workspace=None):
    """Residual-Consistency MLP in place on x [rows, C] fp32 for the rows in `routed`."""
    lib = _lib.load()
    dt = plan.torch_dtype
    C, Hm = plan.desc.channels, plan.desc.mlp_hidden
    x2 = x.view(-1, C)
    _need(x, "x", torch.float32, device=plan.device)
    _need(routed, "routed", torch.int32, device=plan.device)
    _need(ln_g, "ln_g", torch.float32, (C,), plan.device)
    _need(ln_b, "ln_b", torch.float32, (C,), plan.device)
    _need(w1, "w1", dt, (Hm, C), plan.device)
    _need(b1, "b1", torch.float32, (Hm,), plan.device)
    _need(w2, "w2", dt, (C, Hm), plan.device)
    _need(b2, "b2", torch.float32, (C,), plan.device)
    ws = _workspace(plan.info["mlp_workspace_bytes"], x.device, workspace)
    check(lib.sparsesam_mlp(plan.handle, _ptr(x), x2.shape[0], _ptr(routed), routed.numel(), _ptr(ln_g), _ptr(ln_b),
                            _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(ws), ws.numel(), _stream(x.device)),
          "sparsesam_mlp")
    return x


_WEIGHT_NAMES = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2")
_MATRICES = ("w_qkv", "w_proj", "w1", "w2")


def weights_to_device(w, plan, device=None):
    """Host arrays (numpy or torch) -> device tensors in the plan's layout and dtypes."""
    device = device or plan.device
    out = {}
    for name in _WEIGHT_NAMES:
        t = torch.as_tensor(w[name])
        dt = plan.torch_dtype if name in _MATRICES else torch.float32
        out[name] = t.to(device=device, dtype=dt).contiguous()
    for name, src in (("rel_pos_h", "rel_h"), ("rel_pos_w", "rel_w")):
        if w.get(src) is not None:
            out[name] = torch.as_tensor(w[src]).to(device=device, dtype=torch.float32).contiguous()
    return out


def _block_weights(plan, w, what=""):
    """The C struct of one layer's weights; the relative-position tables are passed
    when the plan adds the bias (their shapes checked) and must be absent otherwise."""
    rel = [w.get("rel_pos_h"), w.get("rel_pos_w")]
    if plan.desc.rel_pos:
        D = plan.desc.head_dim
        sh_, sw_ = ((plan.desc.window, plan.desc.window) if plan.desc.window
                    else (plan.desc.grid_h, plan.desc.grid_w))
        _need(rel[0], what + "rel_pos_h", torch.float32, (2 * sh_ - 1, D), plan.device)
        _need(rel[1], what + "rel_pos_w", torch.float32, (2 * sw_ - 1, D), plan.device)
        ptrs = [t.data_ptr() for t in rel]
    else:
        if rel[0] is not None or rel[1] is not None:
            raise ValueError(what + "rel_pos_h / rel_pos_w given to a plan without rel_pos")
        ptrs = [None, None]
    return _lib.BlockWeights(*([w[name].data_ptr() for name in _WEIGHT_NAMES] + ptrs))


def _block_args(plan, weights, x, perm, routed):
    """Checks of block() / block_noalloc(); returns (batch, C weight struct)."""
    dt = plan.torch_dtype
    C, Hm = plan.desc.channels, plan.desc.mlp_hidden
    gh, gw = plan.desc.grid_h, plan.desc.grid_w
    _need(x, "x", torch.float32, device=plan.device)
    b = x.shape[0]
    if tuple(x.shape) != (b, gh, gw, C):
        raise ValueError("x must be [batch, %d, %d, %d]" % (gh, gw, C))
    shapes = {"ln1_g": (C,), "ln1_b": (C,), "w_qkv": (3 * C, C), "b_qkv": (3 * C,), "w_proj": (C, C),
              "b_proj": (C,), "ln2_g": (C,), "ln2_b": (C,), "w1": (Hm, C), "b1": (Hm,), "w2": (C, Hm), "b2": (C,)}
    for name in _WEIGHT_NAMES:
        _need(weights[name], name, dt if name in _MATRICES else torch.float32, shapes[name], plan.device)
    n, segs, rpi = plan.info["seq_len"], plan.info["segments_per_image"], plan.info["routed_per_image"]
    _need(perm, "perm", torch.int32, (b * segs, n), plan.device)
    _need(routed, "routed", torch.int32, (b * rpi,), plan.device)
    return b, _block_weights(plan, weights)


def block(plan, weights, x, perm, routed, workspace=None):
    """One SparseSAM encoder block in place on x [batch, grid_h, grid_w, C] fp32."""
    lib = _lib.load()
    b, bw = _block_args(plan, weights, x, perm, routed)
    ws = _workspace(plan.info["block_workspace_bytes"], x.device, workspace)
    check(lib.sparsesam_block(plan.handle, ctypes.byref(bw), _ptr(x), b, _ptr(perm), _ptr(routed), _ptr(ws),
                              ws.numel(), _stream(x.device)), "sparsesam_block")
    return x


def forward(plan, weights, img, x, patch=16, out=None, workspace=None):
    """The whole step of one block: importance of img [batch, H, W] fp32, the permutation,
    then the block in place on x [batch, grid_h, grid_w, C] -- importance(), permute() and
    block() in one call, bit for bit. Returns (imp, perm, inv, routed)."""
    lib = _lib.load()
    _need(img, "img", torch.float32, device=plan.device)
    if img.dim() != 3:
        raise ValueError("img must be [batch, height, width]")
    b, H, W = img.shape
    tokens = plan.desc.grid_h * plan.desc.grid_w
    n, segs, rpi = plan.info["seq_len"], plan.info["segments_per_image"], plan.info["routed_per_image"]
    if out is None:
        imp = torch.empty(b, tokens, dtype=torch.float32, device=img.device)
        perm = torch.empty(b * segs, n, dtype=torch.int32, device=img.device)
        inv = torch.empty_like(perm)
        routed = torch.empty(b * rpi, dtype=torch.int32, device=img.device)
    else:
        imp, perm, inv, routed = out
    _need(imp, "imp", torch.float32, (b, tokens), plan.device)
    _need(inv, "inv", torch.int32, (b * segs, n), plan.device)
    bx, bw = _block_args(plan, weights, x, perm, routed)
    if bx != b:
        raise ValueError("img and x must hold the same number of images")
    ws = _workspace(plan.info["block_workspace_bytes"], x.device, workspace)
    check(lib.sparsesam_forward(plan.handle, ctypes.byref(bw), _ptr(img), b, H, W, patch, _ptr(x), _ptr(imp),
                                _ptr(perm), _ptr(inv), _ptr(routed), _ptr(ws), ws.numel(), _stream(x.device)),
          "sparsesam_forward")
    return imp, perm, inv, routed


def route_topk(plan, score, out=None):
    """Keep-set by score: per segment the K tokens with the largest score [b, tokens] fp32
    (ties to the lower slot); returns routed int32 [b * routed_per_image]."""
    lib = _lib.load()
    tokens = plan.desc.grid_h * plan.desc.grid_w
    _need(score, "score", torch.float32, device=plan.device)
    if score.dim() != 2 or score.shape[1] != tokens:
        raise ValueError("score must be [batch, %d]" % tokens)
    b = score.shape[0]
    if out is None:
        out = torch.empty(b * plan.info["routed_per_image"], dtype=torch.int32, device=score.device)
    _need(out, "out", torch.int32, (b * plan.info["routed_per_image"],), plan.device)
    check(lib.sparsesam_route_topk(plan.handle, _ptr(score), b, _ptr(out), _stream(score.device)),
          "sparsesam_route_topk")
    return out


def block_dynamic(plan, weights, x, perm, routed_out=None, score_out=None, workspace=None, want_score=True):
    """One block of a plan with routing "update", in place on x: the keep-set of every
    segment is chosen from this block's attention update. Returns (x, routed, score);
    score is None when want_score is False and no score_out is given."""
    lib = _lib.load()
    if plan.routing != "update":
        raise ValueError("block_dynamic needs a plan with routing='update'")
    b = x.shape[0]
    rpi, tokens = plan.info["routed_per_image"], plan.desc.grid_h * plan.desc.grid_w
    if routed_out is None:
        routed_out = torch.empty(b * rpi, dtype=torch.int32, device=x.device)
    if score_out is None and want_score:
        score_out = torch.empty(b, tokens, dtype=torch.float32, device=x.device)
    b, bw = _block_args(plan, weights, x, perm, routed_out)
    if score_out is not None:
        _need(score_out, "score_out", torch.float32, (b, tokens), plan.device)
    ws = _workspace(plan.info["block_workspace_bytes"], x.device, workspace)
    check(lib.sparsesam_block_dynamic(plan.handle, ctypes.byref(bw), _ptr(x), b, _ptr(perm), _ptr(routed_out),
                                      _ptr(score_out), _ptr(ws), ws.numel(), _stream(x.device)),
          "sparsesam_block_dynamic")
    return x, routed_out, score_out


def block_noalloc(plan, weights, x, perm, routed):
    """block() without a workspace: the library's fixed per-GPU scratch serves instead
    (sparsesam_block_noalloc; for callers that cannot allocate). Calls on one GPU must
    not overlap."""
    lib = _lib.load()
    b, bw = _block_args(plan, weights, x, perm, routed)
    check(lib.sparsesam_block_noalloc(plan.handle, ctypes.byref(bw), _ptr(x), b, _ptr(perm), _ptr(routed),
                                      _stream(x.device)), "sparsesam_block_noalloc")
    return x


def noalloc_scratch_bytes():
    """Size of the library's per-GPU scratch used by block_noalloc()."""
    return int(_lib.load().sparsesam_noalloc_scratch_bytes())


def encoder(global_plan, window_plan, layers, kinds, x, global_perm=None, window_perm=None, workspace=None,
            sorted_stream=False):
    """A stack of blocks in place on x [batch, grid_h, grid_w, C] fp32.

    layers: list of weight dicts (weights_to_device); kinds: list of 1 (global block)
    or 0 (windowed block); global_perm / window_perm: (perm, routed) of permute() for
    the plan of that block type, computed once and reused by every layer of the type;
    with sorted_stream=True they are (perm, inv) and the residual stream stays in
    stripe-sorted order between blocks (sparsesam_encoder_permuted).
    """
    lib = _lib.load()
    n = len(layers)
    if len(kinds) != n:
        raise ValueError("layers and kinds must have the same length")
    plans = [p for p in (global_plan, window_plan) if p is not None]
    if not plans:
        raise ValueError("at least one plan is needed")
    ref = plans[0]
    for p in plans:
        _need(x, "x", torch.float32, device=p.device)
        for f in ("grid_h", "grid_w", "channels", "heads", "head_dim", "mlp_hidden", "dtype"):
            if getattr(p.desc, f) != getattr(ref.desc, f):
                raise ValueError("global_plan and window_plan must share %s" % f)
    gh, gw, C = ref.desc.grid_h, ref.desc.grid_w, ref.desc.channels
    b = x.shape[0] if x.dim() == 4 else -1
    if x.dim() != 4 or tuple(x.shape) != (b, gh, gw, C):
        raise ValueError("x must be [batch, %d, %d, %d], got %s" % (gh, gw, C, tuple(x.shape)))
    for p in plans:
        if b > p.desc.max_batch:
            raise ValueError("batch %d exceeds the plan's max_batch %d" % (b, p.desc.max_batch))
    ptrs = {}
    for name, plan, pr in (("global", global_plan, global_perm), ("window", window_plan, window_perm)):
        if plan is None or pr is None:
            ptrs[name] = (ctypes.c_void_p(0), ctypes.c_void_p(0))
            continue
        perm, second = pr
        n_seq, segs, rpi = plan.info["seq_len"], plan.info["segments_per_image"], plan.info["routed_per_image"]
        _need(perm, name + "_perm", torch.int32, (b * segs, n_seq), plan.device)
        if sorted_stream:
            _need(second, name + "_inv", torch.int32, (b * segs, n_seq), plan.device)
        else:
            _need(second, name + "_routed", torch.int32, (b * rpi,), plan.device)
        ptrs[name] = (_ptr(perm), _ptr(second))
    dt, C, Hm = ref.torch_dtype, ref.desc.channels, ref.desc.mlp_hidden
    shapes = {"ln1_g": (C,), "ln1_b": (C,), "w_qkv": (3 * C, C), "b_qkv": (3 * C,), "w_proj": (C, C),
              "b_proj": (C,), "ln2_g": (C,), "ln2_b": (C,), "w1": (Hm, C), "b1": (Hm,), "w2": (C, Hm), "b2": (C,)}
    arr = (_lib.BlockWeights * max(1, n))()
    for l, w in enumerate(layers):
        for name in _WEIGHT_NAMES:
            _need(w[name], "layer %d %s" % (l, name), dt if name in _MATRICES else torch.float32, shapes[name],
                  ref.device)
        arr[l] = _block_weights(global_plan if int(kinds[l]) else window_plan, w, "layer %d " % l)
    kind_arr = (ctypes.c_uint8 * max(1, n))(*[int(k) for k in kinds])
    gh_ = global_plan.handle if global_plan is not None else None
    wh_ = window_plan.handle if window_plan is not None else None
    if sorted_stream:
        need = ctypes.c_size_t()
        check(lib.sparsesam_encoder_permuted_workspace(gh_, wh_, b, ctypes.byref(need)),
              "sparsesam_encoder_permuted_workspace")
        ws = _workspace(need.value, x.device, workspace)
        check(lib.sparsesam_encoder_permuted(gh_, wh_, arr, kind_arr, n, _ptr(x), b, ptrs["global"][0],
                                             ptrs["global"][1], ptrs["window"][0], ptrs["window"][1], _ptr(ws),
                                             ws.numel(), _stream(x.device)), "sparsesam_encoder_permuted")
        return x
    need = max(p.info["block_workspace_bytes"] for p in plans)
    ws = _workspace(need, x.device, workspace)
    check(lib.sparsesam_encoder(global_plan.handle if global_plan is not None else None,
                                window_plan.handle if window_plan is not None else None, arr, kind_arr, n, _ptr(x),
                                b, ptrs["global"][0], ptrs["global"][1], ptrs["window"][0], ptrs["window"][1],
                                _ptr(ws), ws.numel(), _stream(x.device)), "sparsesam_encoder")
    return x
