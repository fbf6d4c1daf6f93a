"""ctypes binding of libuno (include/uno.h).

Argument marshalling only: every step of the decode runs in the HIP library.
torch supplies device memory (tensors) and the HIP stream.  The library is loaded
on first use; a missing library raises (there is no fallback path).
"""
import ctypes as C
import os

import numpy as np

from . import synth

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libuno.so")

UNO_OK = 0
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "OUT_OF_PAGES", 3: "STATE", 4: "NUMERIC",
          5: "DEVICE", 6: "UNSUPPORTED"}
PROJ = synth.PROJ

EXPORTED = ("uno_query_sizes", "uno_init", "uno_prefill", "uno_draft", "uno_verify",
            "uno_step", "uno_accept", "uno_sample", "uno_forward", "uno_kv_import",
            "uno_kv_export", "uno_seq_state", "uno_release", "uno_sync", "uno_free_pages",
            "uno_last_error", "uno_destroy", "uno_timing", "uno_timing_every", "uno_timing_read",
            "uno_distill_forward", "uno_pack_weight", "uno_top_p", "uno_accept_noalloc",
            "uno_set_trace", "uno_query_backward_bytes", "uno_set_distill_checkpoint",
            "uno_tv_backward", "uno_lm_head_backward", "uno_lora_layer_backward",
            "uno_distill_backward", "uno_tree_draft", "uno_tree_verify", "uno_tree_step",
            "uno_tree_accept", "uno_stream_read")

# kernel classes of uno_timing (uno_kernel_class)
KC = {"linear": 0, "linear_swiglu": 1, "lora_down": 2, "attention": 3, "lm_head": 4,
      "sampling": 5, "misc": 6}


class UnoError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class UnoConfigC(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads",
                                         "head_dim", "ffn_dim", "vocab", "mask_id",
                                         "lora_rank")] + \
               [("lora_alpha", C.c_float), ("rope_theta", C.c_float), ("rms_eps", C.c_float)] + \
               [(n, C.c_int32) for n in ("block_size", "page_size", "max_seqs", "max_seq_len",
                                         "n_pages", "max_rows", "dtype")] + \
               [("seed", C.c_uint64), ("top_p", C.c_float), ("qk_norm", C.c_int32),
                ("tree_chains", C.c_int32)]


PP = C.POINTER(C.c_void_p)


class UnoTraceLayerC(C.Structure):
    _fields_ = [("layer", C.c_int32), ("x_in", C.c_void_p), ("q", C.c_void_p),
                ("attn", C.c_void_p), ("x_mid", C.c_void_p), ("act", C.c_void_p),
                ("x_out", C.c_void_p)]


class UnoTraceC(C.Structure):
    _fields_ = [("n", C.c_int32), ("layer", UnoTraceLayerC * 4), ("logits", C.c_void_p)]

TRACE_FIELDS = ("x_in", "q", "attn", "x_mid", "act", "x_out")


class UnoWeightsC(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("final_norm", C.c_void_p),
                ("attn_norm", PP), ("mlp_norm", PP),
                ("w", PP * 7), ("lora_a", PP * 7), ("lora_b", PP * 7),
                ("q_norm", PP), ("k_norm", PP)]


_lib = None


def lib():
    """Load libuno.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m diffusion_drafted_lora_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, u64 = C.c_void_p, C.c_int32, C.c_uint64
        P = C.POINTER
        L.uno_query_sizes.argtypes = [P(UnoConfigC), P(C.c_size_t), P(C.c_size_t)]
        L.uno_init.argtypes = [P(UnoConfigC), P(UnoWeightsC), vp, C.c_size_t, vp, C.c_size_t, vp,
                               P(vp)]
        L.uno_prefill.argtypes = [vp, i32, P(i32), vp, P(i32)]
        L.uno_draft.argtypes = [vp, i32, P(i32), vp, vp]
        L.uno_verify.argtypes = [vp, i32, P(i32), vp, vp, vp]
        L.uno_step.argtypes = [vp, i32, P(i32), vp, vp]
        L.uno_tree_draft.argtypes = [vp, i32, P(i32), i32, vp, vp]
        L.uno_tree_verify.argtypes = [vp, i32, P(i32), vp, vp, vp, vp]
        L.uno_tree_step.argtypes = [vp, i32, P(i32), i32, vp, vp]
        L.uno_tree_accept.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.uno_accept.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.uno_sample.argtypes = [vp, i32, vp, vp, vp, vp, i32, vp]
        L.uno_accept_noalloc.argtypes = [u64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp]
        L.uno_forward.argtypes = [vp, i32, P(i32), i32, vp, vp, vp, vp, vp, vp]
        L.uno_set_trace.argtypes = [vp, P(UnoTraceC)]
        L.uno_kv_import.argtypes = [vp, i32, i32, vp, vp, i32, i32]
        L.uno_kv_export.argtypes = [vp, i32, i32, vp, vp]
        L.uno_seq_state.argtypes = [vp, i32, P(i32), P(i32), P(i32)]
        L.uno_release.argtypes = [vp, i32]
        L.uno_sync.argtypes = [vp]
        L.uno_free_pages.argtypes = [vp]
        L.uno_free_pages.restype = i32
        L.uno_last_error.argtypes = [vp]
        L.uno_last_error.restype = C.c_char_p
        L.uno_destroy.argtypes = [vp]
        L.uno_destroy.restype = None
        L.uno_query_backward_bytes.argtypes = [P(UnoConfigC), i32, i32, P(C.c_size_t)]
        L.uno_set_distill_checkpoint.argtypes = [vp, vp, vp, vp, i32, i32]
        L.uno_tv_backward.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
        L.uno_lm_head_backward.argtypes = [vp, i32, vp, vp, vp, vp, C.c_size_t]
        L.uno_lora_layer_backward.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                              P(vp), P(vp), vp, C.c_size_t]
        L.uno_distill_backward.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                           P(vp), P(vp), vp, C.c_size_t]
        L.uno_timing.argtypes = [vp, C.c_uint32]
        L.uno_stream_read.argtypes = [vp, C.c_size_t, C.c_size_t, i32, i32, i32, i32, vp, vp]
        L.uno_timing_read.argtypes = [vp, i32, P(C.c_int64), P(C.c_double), P(C.c_double),
                                      P(C.c_double)]
        for name in EXPORTED:
            f = getattr(L, name)
            if f.restype is C.c_int:  # default restype: status codes
                f.restype = C.c_int32
        _lib = L
    return _lib


def make_config(cfg, max_seqs=1, max_seq_len=None, n_pages=None, max_rows=None, seed=0,
                top_p=0.0, tree_chains=0):
    """uno_config for a configs.UnoConfig plus decoding limits."""
    max_seq_len = max_seq_len or cfg.max_len
    pages_per_seq = -(-max_seq_len // cfg.page_size)
    c = UnoConfigC()
    c.n_layers, c.d_model = cfg.n_layers, cfg.d_model
    c.n_q_heads, c.n_kv_heads, c.head_dim = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    c.ffn_dim, c.vocab, c.mask_id = cfg.ffn_dim, cfg.vocab, cfg.mask_id
    c.lora_rank, c.lora_alpha = cfg.lora_rank, cfg.lora_alpha
    c.rope_theta, c.rms_eps = cfg.rope_theta, cfg.rms_eps
    c.block_size, c.page_size = cfg.block_size, cfg.page_size
    c.max_seqs, c.max_seq_len = max_seqs, max_seq_len
    c.n_pages = n_pages or max_seqs * pages_per_seq
    c.max_rows = max_rows or max_seqs * cfg.block_size
    c.dtype = 1 if cfg.dtype == "bf16" else 0
    c.seed = seed
    c.top_p = top_p
    c.qk_norm = 1 if getattr(cfg, "qk_norm", False) else 0
    c.tree_chains = tree_chains
    return c


def query_sizes(ccfg):
    kv, ws = C.c_size_t(), C.c_size_t()
    st = lib().uno_query_sizes(C.byref(ccfg), C.byref(kv), C.byref(ws))
    if st != UNO_OK:
        raise UnoError(st, lib().uno_last_error(None).decode())
    return kv.value, ws.value


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def _ptr(t):
    return C.c_void_p(0) if t is None else C.c_void_p(t.data_ptr())


class Engine:
    """A libuno context over torch-allocated device memory."""

    def __init__(self, cfg, weights, max_seqs=1, max_seq_len=None, n_pages=None, max_rows=None,
                 seed=0, device="cuda", stream=None, top_p=0.0, tree_chains=0):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.ccfg = make_config(cfg, max_seqs, max_seq_len, n_pages, max_rows, seed, top_p,
                                tree_chains)
        self.n_pages = self.ccfg.n_pages
        kv_bytes, ws_bytes = query_sizes(self.ccfg)
        self.kv = torch.empty(max(kv_bytes, 1), dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=self.device)
        self.stream = stream or torch.cuda.current_stream(self.device)
        self._keep = []
        wc = UnoWeightsC()
        self.weights = weights

        def arr(ts):
            a = (C.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
            self._keep.append(a)
            return C.cast(a, PP)

        for t in self._all_tensors(weights):
            if not t.is_contiguous() or t.device != self.device:
                raise ValueError("weights must be contiguous tensors on the engine's device")
        weights = pack_weights(cfg, weights)
        self.weights = weights      # the context reads these tensors: keep them alive
        wc.embed = weights["embed"].data_ptr() if "embed" in weights else None
        wc.lm_head = weights["lm_head"].data_ptr() if "lm_head" in weights else None
        wc.final_norm = weights["final_norm"].data_ptr()
        L = weights["layers"]
        wc.attn_norm = arr([l["attn_norm"] for l in L])
        wc.mlp_norm = arr([l["mlp_norm"] for l in L])
        if self.ccfg.qk_norm:
            wc.q_norm = arr([l["q_norm"] for l in L])
            wc.k_norm = arr([l["k_norm"] for l in L])
        has_lora = "la" in L[0] and len(L[0]["la"]) == 7
        for i, p in enumerate(PROJ):
            wc.w[i] = arr([l["w"][p] for l in L])
            if has_lora:
                wc.lora_a[i] = arr([l["la"][p] for l in L])
                wc.lora_b[i] = arr([l["lb"][p] for l in L])
        self._wc = wc
        h = C.c_void_p()
        st = lib().uno_init(C.byref(self.ccfg), C.byref(wc), _ptr(self.kv), kv_bytes,
                            _ptr(self.ws), ws_bytes, C.c_void_p(self.stream.cuda_stream),
                            C.byref(h))
        if st != UNO_OK:
            raise UnoError(st, lib().uno_last_error(None).decode())
        self.h = h

    @staticmethod
    def _all_tensors(w):
        for k in ("embed", "lm_head", "final_norm"):
            if k in w:
                yield w[k]
        for l in w["layers"]:
            yield l["attn_norm"]
            yield l["mlp_norm"]
            for k in ("q_norm", "k_norm"):
                if k in l:
                    yield l[k]
            for d in ("w", "la", "lb"):
                for t in l.get(d, {}).values():
                    yield t

    # ------------------------------------------------------------------ helpers
    def _check(self, st):
        if st != UNO_OK:
            raise UnoError(st, lib().uno_last_error(self.h).decode())

    def _empty(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, device=self.device)

    # -------------------------------------------------------------------- calls
    def prefill(self, seq_ids, prompts):
        """prompts: list of 1-D int arrays (host) or one int32 device tensor per seq."""
        torch = self.torch
        ids, pids = _i32(seq_ids)
        lens, plens = _i32([len(p) for p in prompts])
        cat = torch.cat([torch.as_tensor(np.asarray(p, dtype=np.int32)) if not torch.is_tensor(p)
                         else p.to(torch.int32).cpu() for p in prompts]).to(self.device)
        self._check(lib().uno_prefill(self.h, len(ids), pids, _ptr(cat), plens))
        self._keep_alive = cat  # the copy stays valid until the stream reaches it

    def draft(self, seq_ids, want_probs=False):
        ids, pids = _i32(seq_ids)
        B, V = self.cfg.block_size, self.cfg.vocab
        dr = self._empty((len(ids), B), self.torch.int32)
        pr = self._empty((len(ids), B, V), self.torch.float32) if want_probs else None
        self._check(lib().uno_draft(self.h, len(ids), pids, _ptr(dr), _ptr(pr)))
        return dr, pr

    def verify(self, seq_ids, want_probs=False):
        ids, pids = _i32(seq_ids)
        B, V = self.cfg.block_size, self.cfg.vocab
        out = self._empty((len(ids), B + 1), self.torch.int32)
        n_out = self._empty((len(ids),), self.torch.int32)
        pr = self._empty((len(ids), B, V), self.torch.float32) if want_probs else None
        self._check(lib().uno_verify(self.h, len(ids), pids, _ptr(out), _ptr(n_out), _ptr(pr)))
        return out, n_out, pr

    def step(self, seq_ids, out=None, n_out=None):
        ids, pids = _i32(seq_ids)
        B = self.cfg.block_size
        if out is None:
            out = self._empty((len(ids), B + 1), self.torch.int32)
        if n_out is None:
            n_out = self._empty((len(ids),), self.torch.int32)
        self._check(lib().uno_step(self.h, len(ids), pids, _ptr(out), _ptr(n_out)))
        return out, n_out

    def accept(self, p, q, draft, seq_ids, pos, iters):
        """Accept kernel on given tensors: p [n,B,V], q [n,B-1,V], draft [n,B]; seq_ids,
        pos, iters device int32 [n]."""
        n, B = draft.shape
        out = self._empty((n, B + 1), self.torch.int32)
        n_out = self._empty((n,), self.torch.int32)
        self._check(lib().uno_accept(self.h, n, _ptr(p), _ptr(q), _ptr(draft), _ptr(seq_ids),
                                     _ptr(pos), _ptr(iters), _ptr(out), _ptr(n_out)))
        return out, n_out

    def tree_draft(self, seq_ids, n_chains, want_probs=False):
        """uno_tree_draft: (chains [n, K, B], draft laws [n, B, V] or None)."""
        ids, pids = _i32(seq_ids)
        B, V = self.cfg.block_size, self.cfg.vocab
        ch = self._empty((len(ids), n_chains, B), self.torch.int32)
        pr = self._empty((len(ids), B, V), self.torch.float32) if want_probs else None
        self._check(lib().uno_tree_draft(self.h, len(ids), pids, n_chains, _ptr(ch), _ptr(pr)))
        return ch, pr

    def tree_verify(self, seq_ids, n_chains, want_probs=False):
        """uno_tree_verify: (out [n, B+1], n_out [n], kstar [n], verify laws
        [n, 1 + K (B-1), V] or None); n_chains is the pending draft's K."""
        ids, pids = _i32(seq_ids)
        B, V = self.cfg.block_size, self.cfg.vocab
        n = len(ids)
        out = self._empty((n, B + 1), self.torch.int32)
        n_out = self._empty((n,), self.torch.int32)
        kstar = self._empty((n,), self.torch.int32)
        pr = self._empty((n, 1 + n_chains * (B - 1), V), self.torch.float32) if want_probs else None
        self._check(lib().uno_tree_verify(self.h, n, pids, _ptr(out), _ptr(n_out), _ptr(kstar),
                                          _ptr(pr)))
        return out, n_out, kstar, pr

    def tree_step(self, seq_ids, n_chains, out=None, n_out=None):
        ids, pids = _i32(seq_ids)
        B = self.cfg.block_size
        if out is None:
            out = self._empty((len(ids), B + 1), self.torch.int32)
        if n_out is None:
            n_out = self._empty((len(ids),), self.torch.int32)
        self._check(lib().uno_tree_step(self.h, len(ids), pids, n_chains, _ptr(out), _ptr(n_out)))
        return out, n_out

    def tree_accept(self, p, q, chains, seq_ids, pos, iters):
        """Tree acceptance on given tensors: p [n, 1 + K (B-1), V], q [n, B, V],
        chains [n, K, B]; seq_ids, pos, iters device int32 [n].  Returns (out, n_out,
        kstar)."""
        n, K, B = chains.shape
        out = self._empty((n, B + 1), self.torch.int32)
        n_out = self._empty((n,), self.torch.int32)
        kstar = self._empty((n,), self.torch.int32)
        self._check(lib().uno_tree_accept(self.h, n, K, _ptr(p), _ptr(q), _ptr(chains), _ptr(seq_ids),
                                          _ptr(pos), _ptr(iters), _ptr(out), _ptr(n_out),
                                          _ptr(kstar)))
        return out, n_out, kstar

    def sample(self, w, seq_ids, pos, iters, stream_id):
        rows = w.shape[0]
        idx = self._empty((rows,), self.torch.int32)
        self._check(lib().uno_sample(self.h, rows, _ptr(w), _ptr(seq_ids), _ptr(pos),
                                     _ptr(iters), stream_id, _ptr(idx)))
        return idx

    def forward(self, seq_ids, rows_per_seq, pos, gate, tokens=None, hidden_in=None,
                want_hidden=False, want_logits=False):
        ids, pids = _i32(seq_ids)
        R = len(ids) * rows_per_seq
        hid = self._empty((R, self.cfg.d_model), self.torch.float32) if want_hidden else None
        lg = self._empty((R, self.cfg.vocab), self.torch.float32) if want_logits else None
        self._check(lib().uno_forward(self.h, len(ids), pids, rows_per_seq, _ptr(tokens),
                                      _ptr(hidden_in), _ptr(pos), _ptr(gate), _ptr(hid), _ptr(lg)))
        return hid, lg

    def distill_forward(self, x, B, teacher=None, student=None, tv_row=None, tv_block=None,
                        want_logits=True):
        """[x, MASK^L] forward of each row of x (device int32 [batch, L]) with block
        size B.  Returns (teacher, student, tv_row, tv_block); logits are allocated
        unless passed in (or want_logits is False: then None, only TV formed)."""
        torch = self.torch
        batch, L = x.shape
        V = self.cfg.vocab
        if want_logits:
            if teacher is None:
                teacher = self._empty((batch, L, V), torch.float32)
            if student is None:
                student = self._empty((batch, L, V), torch.float32)
        if tv_row is None:
            tv_row = self._empty((batch, L), torch.float32)
        if tv_block is None:
            tv_block = self._empty((batch, L // B), torch.float32)
        self._check(lib().uno_distill_forward(self.h, batch, L, B, _ptr(x), _ptr(teacher),
                                              _ptr(student), _ptr(tv_row), _ptr(tv_block)))
        return teacher, student, tv_row, tv_block

    # ---- distillation backward (gradient of L_TV with respect to the LoRA)

    def backward_scratch(self, batch, L):
        """Device scratch for a backward over batch x L z1 rows (cached, grown)."""
        n = C.c_size_t(0)
        self._check(lib().uno_query_backward_bytes(C.byref(self.ccfg), batch, L, C.byref(n)))
        cur = getattr(self, "_bw_scratch", None)
        if cur is None or cur.numel() < n.value:
            self._bw_scratch = None
            self._bw_scratch = self._empty((n.value,), self.torch.uint8)
        return self._bw_scratch

    def set_distill_checkpoint(self, batch, L):
        """Arm the activation checkpoint for distillation forwards of batch x L and
        return its buffers {"x", "k", "v"}; batch None disarms."""
        torch = self.torch
        if batch is None:
            self._check(lib().uno_set_distill_checkpoint(self.h, None, None, None, 0, 0))
            self._ckpt = None
            return None
        cfg = self.cfg
        ck = {"x": self._empty((cfg.n_layers + 1, batch * L, cfg.d_model), torch.float32),
              "k": self._empty((batch, cfg.n_layers, L, cfg.n_kv_heads, cfg.head_dim), torch.bfloat16),
              "v": self._empty((batch, cfg.n_layers, L, cfg.n_kv_heads, cfg.head_dim), torch.bfloat16)}
        self._check(lib().uno_set_distill_checkpoint(self.h, _ptr(ck["x"]), _ptr(ck["k"]),
                                                     _ptr(ck["v"]), batch, L))
        self._ckpt = ck
        return ck

    def _grad_bufs(self, layers):
        torch = self.torch
        shapes = synth.proj_shapes(self.cfg)
        r = self.cfg.lora_rank
        lead = () if layers is None else (layers,)
        ga = {p: self._empty(lead + (r, shapes[p][1]), torch.float32) for p in PROJ}
        gb = {p: self._empty(lead + (shapes[p][0], r), torch.float32) for p in PROJ}
        arr = lambda d: (C.c_void_p * 7)(*[C.c_void_p(d[p].data_ptr()) for p in PROJ])
        return ga, gb, arr(ga), arr(gb)

    def lm_head_backward(self, x_final, dlogits):
        """uno_lm_head_backward: dx [rows, d] of the final residual stream."""
        rows = x_final.shape[0]
        dx = self._empty((rows, self.cfg.d_model), self.torch.float32)
        sc = self.backward_scratch(1, rows)
        self._check(lib().uno_lm_head_backward(self.h, rows, _ptr(x_final), _ptr(dlogits), _ptr(dx),
                                               _ptr(sc), sc.numel()))
        return dx

    def lora_layer_backward(self, layer, B, x_in, k_ctx, v_ctx, dy, dx=None):
        """uno_lora_layer_backward over the z1 rows of k_ctx.shape[0] sequences of
        L = k_ctx.shape[1] rows.  Returns (dx, {proj: dA}, {proj: dB})."""
        batch, L = k_ctx.shape[0], k_ctx.shape[1]
        if dx is None:
            dx = self._empty((batch * L, self.cfg.d_model), self.torch.float32)
        ga, gb, pa, pb = self._grad_bufs(None)
        sc = self.backward_scratch(batch, L)
        self._check(lib().uno_lora_layer_backward(self.h, layer, batch, L, B, _ptr(x_in), _ptr(k_ctx),
                                                  _ptr(v_ctx), _ptr(dy), _ptr(dx), pa, pb, _ptr(sc),
                                                  sc.numel()))
        return dx, ga, gb

    def distill_backward(self, B, teacher, student, ckpt=None, tv_row=None):
        """uno_distill_backward after a checkpointed distill_forward.  Returns
        (loss [1], tv_row [batch * L], {proj: dA [layers, r, in]}, {proj: dB})."""
        torch = self.torch
        ckpt = ckpt or self._ckpt
        batch, L = teacher.shape[0], teacher.shape[1]
        loss = self._empty((1,), torch.float32)
        if tv_row is None:
            tv_row = self._empty((batch * L,), torch.float32)
        ga, gb, pa, pb = self._grad_bufs(self.cfg.n_layers)
        sc = self.backward_scratch(batch, L)
        self._check(lib().uno_distill_backward(self.h, batch, L, B, _ptr(teacher), _ptr(student),
                                               _ptr(ckpt["x"]), _ptr(ckpt["k"]), _ptr(ckpt["v"]),
                                               _ptr(loss), _ptr(tv_row), pa, pb, _ptr(sc),
                                               sc.numel()))
        return loss, tv_row, ga, gb

    def set_trace(self, rows, layers=(), logits=False):
        """Arm the stage capture for forwards of `rows` rows: for each layer index
        in `layers` (at most four) device buffers for x_in, q, attn, x_mid, act and
        x_out, plus the logits when asked; returns {layer: {field: tensor}} and
        (under the key "logits") the logits tensor.  rows=None disarms."""
        torch = self.torch
        if rows is None:
            self._check(lib().uno_set_trace(self.h, None))
            self._trace = None
            return None
        cfg = self.cfg
        st = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        f32 = torch.float32
        shapes = {"x_in": (cfg.d_model, f32), "q": (cfg.q_dim, st), "attn": (cfg.q_dim, st),
                  "x_mid": (cfg.d_model, f32), "act": (cfg.ffn_dim, st),
                  "x_out": (cfg.d_model, f32)}
        tc = UnoTraceC()
        tc.n = len(layers)
        bufs = {}
        for i, l in enumerate(layers):
            tc.layer[i].layer = l
            bufs[l] = {}
            for f in TRACE_FIELDS:
                cols, dt = shapes[f]
                t = self._empty((rows, cols), dt)
                bufs[l][f] = t
                setattr(tc.layer[i], f, t.data_ptr())
        if logits:
            bufs["logits"] = self._empty((rows, cfg.vocab), f32)
            tc.logits = bufs["logits"].data_ptr()
        self._check(lib().uno_set_trace(self.h, C.byref(tc)))
        self._trace = bufs          # the library writes into these: keep them alive
        return bufs

    def kv_import(self, seq_id, k, v, pending, iteration=0):
        """k, v: device tensors [layers, len, Hkv, hd] of the storage dtype."""
        self._check(lib().uno_kv_import(self.h, seq_id, k.shape[1], _ptr(k), _ptr(v), pending,
                                        iteration))

    def kv_export(self, seq_id, length):
        cfg = self.cfg
        dt = self.torch.bfloat16 if cfg.dtype == "bf16" else self.torch.float32
        shape = (cfg.n_layers, length, cfg.n_kv_heads, cfg.head_dim)
        k, v = self._empty(shape, dt), self._empty(shape, dt)
        self._check(lib().uno_kv_export(self.h, seq_id, length, _ptr(k), _ptr(v)))
        return k, v

    def seq_state(self, seq_id):
        a, b, c = C.c_int32(), C.c_int32(), C.c_int32()
        self._check(lib().uno_seq_state(self.h, seq_id, C.byref(a), C.byref(b), C.byref(c)))
        return a.value, b.value, c.value

    def release(self, seq_id):
        self._check(lib().uno_release(self.h, seq_id))

    def sync(self):
        self._check(lib().uno_sync(self.h))

    def timing(self, classes=(), every=1):
        """Start recording launches of the named kernel classes (empty: stop),
        the first of every `every` calls of each class."""
        mask = 0
        for c in classes:
            mask |= 1 << KC[c]
        self._check(lib().uno_timing_every(self.h, int(every)))
        self._check(lib().uno_timing(self.h, mask))

    def timing_read(self, cls):
        """(launches, total ms, algorithmic bytes, flops) recorded for a class."""
        n, ms, b, f = C.c_int64(), C.c_double(), C.c_double(), C.c_double()
        self._check(lib().uno_timing_read(self.h, KC[cls], C.byref(n), C.byref(ms), C.byref(b),
                                          C.byref(f)))
        return n.value, ms.value, b.value, f.value

    def free_pages(self):
        return lib().uno_free_pages(self.h)

    def close(self):
        if getattr(self, "h", None):
            lib().uno_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def top_p(probs, p, out=None):
    """Top-p truncation of the rows of a float32 device tensor [..., V] (see
    uno_top_p); in place when out is probs."""
    import torch
    if not (probs.is_cuda and probs.is_contiguous() and probs.dtype == torch.float32):
        raise ValueError("top_p needs a contiguous float32 device tensor")
    if out is None:
        out = torch.empty_like(probs)
    V = probs.shape[-1]
    st = lib().uno_top_p(_ptr(probs), _ptr(out), probs.numel() // V, V, C.c_float(p),
                         C.c_void_p(torch.cuda.current_stream(probs.device).cuda_stream))
    if st != UNO_OK:
        raise UnoError(st, lib().uno_last_error(None).decode())
    return out


def stream_read(src, nbytes, workgroups, threads, loads, sink, reps=1):
    """uno_stream_read: `reps` read-only launches of nbytes each, over windows
    rotating through the device tensor src (sink: int32 device tensor of at least
    `workgroups` entries), on the current stream."""
    import torch
    region = src.numel() * src.element_size()
    if not (src.is_cuda and sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= workgroups
            and nbytes <= region):
        raise ValueError("stream_read: device buffers of the right sizes required")
    st = lib().uno_stream_read(_ptr(src), int(region), int(nbytes), int(reps), int(workgroups),
                               int(threads), int(loads), _ptr(sink),
                               C.c_void_p(torch.cuda.current_stream(src.device).cuda_stream))
    if st != UNO_OK:
        raise UnoError(st, lib().uno_last_error(None).decode())


def tv_backward(teacher, student, n_rows_total=None, dlogits=None, tv_row=None):
    """uno_tv_backward on float32 device logits [rows, V] (no context): returns
    (dL_TV/d student logits, per-row TV)."""
    import torch
    V = teacher.shape[-1]
    rows = teacher.numel() // V
    if dlogits is None:
        dlogits = torch.empty_like(student)
    if tv_row is None:
        tv_row = torch.empty(rows, dtype=torch.float32, device=teacher.device)
    st = lib().uno_tv_backward(_ptr(teacher), _ptr(student), rows, V, n_rows_total or rows,
                               _ptr(dlogits), _ptr(tv_row),
                               C.c_void_p(torch.cuda.current_stream(teacher.device).cuda_stream))
    if st != UNO_OK:
        raise UnoError(st, lib().uno_last_error(None).decode())
    return dlogits, tv_row


def accept_noalloc(seed, p, q, draft, seq_ids, pos, iters, out, n_out, err=None, stream=None):
    """uno_accept_noalloc on device tensors: p [n,B,V], q [n,B-1,V] (or None when B
    is 1), draft [n,B]; seq_ids, pos, iters int32 [n]; outputs out [n,B+1] and n_out
    [n] are caller-allocated, err an optional int32 [1] that receives the device
    error bits.  Enqueued on `stream` (default: the current torch stream)."""
    import torch
    n, B = draft.shape
    V = p.shape[-1]
    s = stream or torch.cuda.current_stream(p.device)
    st = lib().uno_accept_noalloc(C.c_uint64(seed), n, B, V, _ptr(p), _ptr(q), _ptr(draft),
                                  _ptr(seq_ids), _ptr(pos), _ptr(iters), _ptr(out), _ptr(n_out),
                                  _ptr(err), C.c_void_p(s.cuda_stream))
    if st != UNO_OK:
        raise UnoError(st, lib().uno_last_error(None).decode())
    return out, n_out


def pack_weights(cfg, w):
    """For bf16 models, a copy of the device weight dict `w` with the LM head, the
    projections and the LoRA matrices in the fragment-tiled layout of
    uno_pack_weight (q / k / v and their LoRA up with the rotary pair order);
    float32 models, or an already packed dict, are returned as they are."""
    if cfg.dtype != "bf16" or w.get("_packed"):
        return w
    import torch

    def pk(t, pair_hd):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == torch.bfloat16 and t.dim() == 2):
            raise ValueError("pack_weights needs contiguous 2-D bf16 device tensors")
        out = torch.empty_like(t)
        st = lib().uno_pack_weight(_ptr(t), _ptr(out), t.shape[0], t.shape[1], pair_hd,
                                   C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream))
        if st != UNO_OK:
            raise UnoError(st, lib().uno_last_error(None).decode())
        return out

    out = {k: w[k] for k in ("embed", "final_norm") if k in w}
    if "lm_head" in w:
        out["lm_head"] = pk(w["lm_head"], 0)
    out["layers"] = []
    for lw in w["layers"]:
        d = {"attn_norm": lw["attn_norm"], "mlp_norm": lw["mlp_norm"], "w": {}}
        d.update({k: lw[k] for k in ("q_norm", "k_norm") if k in lw})
        for p, t in lw["w"].items():
            d["w"][p] = pk(t, cfg.head_dim if p in ("q", "k", "v") else 0)
        if "la" in lw:
            d["la"] = {p: pk(t, 0) for p, t in lw["la"].items()}
            d["lb"] = {p: pk(t, cfg.head_dim if p in ("q", "k", "v") else 0)
                       for p, t in lw["lb"].items()}
        out["layers"].append(d)
    out["_packed"] = True
    return out


def to_device(weights_np, cfg, device="cuda"):
    """Copy a synth.weights_numpy dict to device tensors of the storage dtype."""
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(device)

    out = {k: t(weights_np[k]) for k in ("embed", "lm_head", "final_norm") if k in weights_np}
    out["layers"] = []
    for lw in weights_np["layers"]:
        d = {"attn_norm": t(lw["attn_norm"]), "mlp_norm": t(lw["mlp_norm"]),
             "w": {p: t(a) for p, a in lw["w"].items()}}
        d.update({k: t(lw[k]) for k in ("q_norm", "k_norm") if k in lw})
        if "la" in lw:
            d["la"] = {p: t(a) for p, a in lw["la"].items()}
            d["lb"] = {p: t(a) for p, a in lw["lb"].items()}
        out["layers"].append(d)
    return out
