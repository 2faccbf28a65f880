"""ctypes binding of libspecdec.so (the gfx950 block-verify path).

Argument marshalling only: PyTorch provides device memory and the stream;
every step of the path runs in the library's HIP kernels.  Importing this
module raises if the library has not been built; nothing falls back to a
CPU implementation.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

from .shapes import ModelShape

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecdec.so")

OK, EINVAL, ECAPACITY, ESHAPE, EHIP, EDEVICE, EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
DERR_CAPACITY, DERR_TRIM, DERR_NONFINITE, DERR_TABLE, DERR_OUTPUT, DERR_SYNC, DERR_TREE = 1, 2, 4, 8, 16, 32, 64
W_BF16, W_Q4G64 = 0, 1
GREEDY, STOCHASTIC, RELAXED = 0, 1, 2
SCHEDULE_A, SCHEDULE_B = 0, 1
DRAFT_TABLE, DRAFT_MODEL, DRAFT_NOISY_SELF, DRAFT_Q4_SELF = 0, 1, 2, 3
MAX_ROWS = 32
MAX_K = 16
MAX_TREE = 512

EXPORTED = [
    "specdec_tensor_count", "specdec_weights_bytes", "specdec_weights_pack", "specdec_model_create",
    "specdec_model_destroy", "specdec_cache_bytes", "specdec_cache_create", "specdec_cache_destroy",
    "specdec_kv_trim", "specdec_workspace_bytes", "specdec_workspace_init", "specdec_decode_step",
    "specdec_prefill", "specdec_round_state_bytes", "specdec_round_ws_bytes", "specdec_round_create",
    "specdec_round_destroy", "specdec_round_prefill", "specdec_round_reset", "specdec_verify_round",
    "specdec_check", "specdec_last_hip_error", "specdec_status_str", "specdec_philox4x64",
    "specdec_round_graph", "specdec_round_graph_launch", "specdec_round_debug_view", "specdec_stream_read",
    "specdec_decode_step_noalloc", "specdec_static_init", "specdec_tree_verify", "specdec_tree_accept",
    "specdec_tree_draft",
]


class SpecdecError(RuntimeError):
    pass


class ModelDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("rope_theta", C.c_float), ("rms_eps", C.c_float),
                ("weight_format", C.c_int32)]


class RoundState(C.Structure):
    _fields_ = [("n_committed", C.c_int32), ("round", C.c_int32), ("m_last", C.c_int32),
                ("last_tok", C.c_int32), ("saved_argmax", C.c_int32), ("saved_lse", C.c_float),
                ("accepted_total", C.c_int32), ("cap", C.c_int32), ("n_target", C.c_int32),
                ("reserved", C.c_int32 * 7)]


class RoundDesc(C.Structure):
    _fields_ = [("target", C.c_void_p), ("target_cache", C.c_void_p), ("draft", C.c_void_p),
                ("draft_cache", C.c_void_p), ("k", C.c_int32), ("mode", C.c_int32), ("bonus", C.c_int32),
                ("schedule", C.c_int32), ("draft_source", C.c_int32), ("d_draft_table", C.c_void_p),
                ("table_len", C.c_int32), ("d_noise", C.c_void_p), ("noise_rows", C.c_int32),
                ("philox_seed", C.c_uint64), ("d_state", C.c_void_p), ("d_ws", C.c_void_p),
                ("ws_bytes", C.c_size_t), ("d_draft_ws", C.c_void_p), ("draft_ws_bytes", C.c_size_t),
                ("d_round_ws", C.c_void_p), ("round_ws_bytes", C.c_size_t), ("state_cap", C.c_int32),
                ("events", C.POINTER(C.c_void_p)), ("n_events", C.c_int32), ("temperature", C.c_float),
                ("top_k", C.c_int32), ("top_p", C.c_float), ("relax_delta", C.c_float)]


def load_library(path: str = _LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise SpecdecError(f"{path} is missing: build it with `python -m block_verify_amd.build`")
    lib = C.CDLL(path)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    P = C.POINTER
    sig = {
        "specdec_tensor_count": (i32, [P(ModelDesc)]),
        "specdec_weights_bytes": (C.c_int, [P(ModelDesc), P(sz)]),
        "specdec_weights_pack": (C.c_int, [P(ModelDesc), i32, vp, vp, vp]),
        "specdec_model_create": (C.c_int, [P(ModelDesc), vp, vp, P(vp)]),
        "specdec_model_destroy": (None, [vp]),
        "specdec_cache_bytes": (C.c_int, [P(ModelDesc), i32, P(sz)]),
        "specdec_cache_create": (C.c_int, [P(ModelDesc), vp, sz, i32, vp, P(vp)]),
        "specdec_cache_destroy": (None, [vp]),
        "specdec_kv_trim": (C.c_int, [vp, i32, vp, vp]),
        "specdec_workspace_bytes": (C.c_int, [P(ModelDesc), i32, i32, P(sz)]),
        "specdec_workspace_init": (C.c_int, [vp, sz, vp]),
        "specdec_decode_step": (C.c_int, [vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]),
        "specdec_prefill": (C.c_int, [vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]),
        "specdec_round_state_bytes": (C.c_int, [i32, P(sz)]),
        "specdec_round_ws_bytes": (C.c_int, [P(ModelDesc), i32, P(sz)]),
        "specdec_round_create": (C.c_int, [P(RoundDesc), P(vp)]),
        "specdec_round_destroy": (None, [vp]),
        "specdec_round_prefill": (C.c_int, [vp, vp, i32, i32, vp]),
        "specdec_round_reset": (C.c_int, [vp, i32, vp]),
        "specdec_verify_round": (C.c_int, [vp, vp]),
        "specdec_check": (C.c_int, [vp, P(i32), vp]),
        "specdec_last_hip_error": (i32, []),
        "specdec_status_str": (C.c_char_p, [C.c_int]),
        "specdec_philox4x64": (C.c_int, [vp, vp, i32, vp, vp]),
        "specdec_round_graph": (C.c_int, [vp]),
        "specdec_round_graph_launch": (C.c_int, [vp, i32, vp]),
        "specdec_round_debug_view": (C.c_int, [vp, i32, P(vp), P(sz)]),
        "specdec_stream_read": (C.c_int, [vp, sz, i32, vp, vp]),
        "specdec_decode_step_noalloc": (C.c_int, [vp, vp, vp, i32, vp, vp, vp, vp, vp]),
        "specdec_static_init": (C.c_int, [vp]),
        "specdec_tree_verify": (C.c_int, [vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]),
        "specdec_tree_accept": (C.c_int, [vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp]),
        "specdec_tree_draft": (C.c_int, [vp, vp, vp, i32, i32, C.c_float, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def check(rc: int, what: str = "") -> None:
    if rc != OK:
        msg = lib().specdec_status_str(rc).decode()
        extra = f" (hipError {lib().specdec_last_hip_error()})" if rc == EHIP else ""
        raise SpecdecError(f"{what}: {msg} [{rc}]{extra}")


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def desc_of(shape: ModelShape, weight_format: int = W_BF16) -> ModelDesc:
    return ModelDesc(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                     shape.ffn, shape.vocab, shape.rope_theta, shape.rms_eps, weight_format)


def _dev_bytes(n: int, device) -> torch.Tensor:
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


class Model:
    """Packed decoder weights on the device + the library's model handle.

    tensors: the canonical list (ModelShape.tensor_specs order) of bf16 bit
    arrays.  For weight_format=W_Q4G64 the linear entries other than lm_head
    are (codes uint8 [N][K/2], scale fp16 [N][K/64], zero fp16 [N][K/64])
    tuples; with `share` (a Model) the embedding, final norm and LM head come
    from that model and their entries may be None.
    """

    def __init__(self, shape: ModelShape, tensors, device="cuda", stream=None, weight_format: int = W_BF16,
                 share: "Model | None" = None):
        self.shape = shape
        self.desc = desc_of(shape, weight_format)
        self.share = share
        L = lib()
        nbytes = C.c_size_t()
        check(L.specdec_weights_bytes(C.byref(self.desc), C.byref(nbytes)), "weights_bytes")
        self.blob = _dev_bytes(nbytes.value, device)
        s = _stream(stream)
        for i, t in enumerate(tensors):
            if t is None:
                continue
            if isinstance(t, tuple):
                codes, sc, zc = t
                raw = np.concatenate([np.ascontiguousarray(codes, np.uint8).ravel(),
                                      np.ascontiguousarray(sc, np.float16).view(np.uint8).ravel(),
                                      np.ascontiguousarray(zc, np.float16).view(np.uint8).ravel()])
                src = torch.from_numpy(raw).to(device)
            else:
                src = torch.from_numpy(np.ascontiguousarray(t).view(np.int16)).to(device)
            check(L.specdec_weights_pack(C.byref(self.desc), i, src.data_ptr(), self.blob.data_ptr(), s), f"pack {i}")
            torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
            del src
        h = C.c_void_p()
        check(L.specdec_model_create(C.byref(self.desc), self.blob.data_ptr(), share.handle if share else None,
                                     C.byref(h)), "model_create")
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.specdec_model_destroy(self.handle)
            self.handle = None


class Cache:
    """KV cache of max_len positions; the length lives in device memory."""

    def __init__(self, shape: ModelShape, max_len: int, device="cuda"):
        L = lib()
        self.shape = shape
        self.desc = desc_of(shape)
        self.max_len = max_len
        nbytes = C.c_size_t()
        check(L.specdec_cache_bytes(C.byref(self.desc), max_len, C.byref(nbytes)), "cache_bytes")
        self.mem = _dev_bytes(nbytes.value, device)
        self.len = torch.zeros(1, dtype=torch.int32, device=device)
        h = C.c_void_p()
        check(L.specdec_cache_create(C.byref(self.desc), self.mem.data_ptr(), nbytes.value, max_len,
                                     self.len.data_ptr(), C.byref(h)), "cache_create")
        self.handle = h

    def length(self) -> int:
        return int(self.len.item())

    def kv_bytes(self) -> int:
        """Bytes of the K and V arrays at the start of the cache memory."""
        sh = self.shape
        lp = (self.max_len + 127) // 128 * 128
        return 2 * sh.n_layers * sh.n_kv_heads * lp * sh.head_dim * 2

    def kv(self):
        """bf16 bit views (int16) of the cache: K [L][n_kv][max_len][hd] and V [L][n_kv][max_len][hd].

        V is stored transposed ([n_kv][hd][lp] per layer); the view returned
        here is transposed back (a strided view, no copy).
        """
        sh = self.shape
        lp = (self.max_len + 127) // 128 * 128
        per = sh.n_kv_heads * lp * sh.head_dim
        raw = self.mem[: 2 * sh.n_layers * 2 * per].view(torch.int16).view(sh.n_layers, 2, per)
        k = raw[:, 0].view(sh.n_layers, sh.n_kv_heads, lp, sh.head_dim)[:, :, : self.max_len]
        v = raw[:, 1].view(sh.n_layers, sh.n_kv_heads, sh.head_dim, lp).transpose(2, 3)[:, :, : self.max_len]
        return k, v

    def trim(self, new_len: int, ws: "Workspace", stream=None) -> None:
        check(lib().specdec_kv_trim(self.handle, new_len, ws.mem.data_ptr(), _stream(stream)), "kv_trim")

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.specdec_cache_destroy(self.handle)
            self.handle = None


class Workspace:
    def __init__(self, shape: ModelShape, max_len: int, max_rows: int = MAX_ROWS, device="cuda"):
        L = lib()
        nbytes = C.c_size_t()
        d = desc_of(shape)
        check(L.specdec_workspace_bytes(C.byref(d), max_rows, max_len, C.byref(nbytes)), "workspace_bytes")
        self.nbytes = nbytes.value
        self.mem = _dev_bytes(self.nbytes, device)
        check(L.specdec_workspace_init(self.mem.data_ptr(), self.nbytes, _stream(None)), "workspace_init")

    def error_bits(self, stream=None) -> int:
        bits = C.c_int32()
        lib().specdec_check(self.mem.data_ptr(), C.byref(bits), _stream(stream))
        return bits.value


def decode_step(model: Model, cache: Cache, tokens: torch.Tensor, ws: Workspace, logits=None, argmax=None,
                lse=None, rows=None, stream=None) -> None:
    rows = int(tokens.numel()) if rows is None else rows
    check(lib().specdec_decode_step(model.handle, cache.handle, tokens.data_ptr(), rows, _ptr(logits),
                                    _ptr(argmax), _ptr(lse), ws.mem.data_ptr(), ws.nbytes, _stream(stream)),
          "decode_step")


def tree_verify(model: Model, cache: Cache, tokens: torch.Tensor, parents: torch.Tensor, ws: Workspace, logits=None,
                argmax=None, lse=None, stream=None) -> None:
    check(lib().specdec_tree_verify(model.handle, cache.handle, tokens.data_ptr(), parents.data_ptr(),
                                    int(tokens.numel()), _ptr(logits), _ptr(argmax), _ptr(lse), ws.mem.data_ptr(),
                                    ws.nbytes, _stream(stream)), "tree_verify")


def tree_accept(cache: Cache, tokens: torch.Tensor, parents: torch.Tensor, argmax: torch.Tensor,
                out_tokens: torch.Tensor, out_count: torch.Tensor, err: torch.Tensor, root=None, log=None,
                n=None, stream=None) -> None:
    """``log``: int32 [1 + cap] job log (entry 0 counts the tokens stored from entry 1)."""
    n = int(tokens.numel()) if n is None else n
    cap = int(log.numel()) - 1 if log is not None else 0
    check(lib().specdec_tree_accept(cache.handle, tokens.data_ptr(), parents.data_ptr(), n, argmax.data_ptr(),
                                    out_tokens.data_ptr(), out_count.data_ptr(), _ptr(root), _ptr(log), cap,
                                    err.data_ptr(), _stream(stream)), "tree_accept")


def tree_draft(draft: Model, cache: Cache, root: torch.Tensor, k: int, depth: int, tokens: torch.Tensor,
               parents: torch.Tensor, scores: torch.Tensor, ws: Workspace, temperature: float = 0.2,
               stream=None) -> None:
    n = 1 + k * depth
    if tokens.numel() < n or parents.numel() < n or scores.numel() < n:
        raise ValueError(f"tree_draft: outputs need {n} entries")
    check(lib().specdec_tree_draft(draft.handle, cache.handle, root.data_ptr(), k, depth, float(temperature),
                                   tokens.data_ptr(), parents.data_ptr(), scores.data_ptr(), ws.mem.data_ptr(),
                                   ws.nbytes, _stream(stream)), "tree_draft")


def static_init(stream=None) -> None:
    check(lib().specdec_static_init(_stream(stream)), "static_init")


def decode_step_noalloc(model: Model, cache: Cache, tokens: torch.Tensor, err: torch.Tensor, logits=None,
                        argmax=None, lse=None, rows=None, stream=None) -> None:
    rows = int(tokens.numel()) if rows is None else rows
    check(lib().specdec_decode_step_noalloc(model.handle, cache.handle, tokens.data_ptr(), rows, _ptr(logits),
                                            _ptr(argmax), _ptr(lse), err.data_ptr(), _stream(stream)),
          "decode_step_noalloc")


def prefill(model: Model, cache: Cache, tokens: torch.Tensor, ws: Workspace, chunk: int = MAX_ROWS,
            logits=None, argmax=None, lse=None, stream=None) -> None:
    check(lib().specdec_prefill(model.handle, cache.handle, tokens.data_ptr(), int(tokens.numel()), chunk,
                                _ptr(logits), _ptr(argmax), _ptr(lse), ws.mem.data_ptr(), ws.nbytes,
                                _stream(stream)), "prefill")


def stream_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 2048, stream=None) -> None:
    """Read every byte of `buf` once (the stream-read ceiling probe)."""
    check(lib().specdec_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), workgroups, sink.data_ptr(),
                                    _stream(stream)), "stream_read")


def philox4x64(counters: np.ndarray, keys: np.ndarray, device="cuda") -> np.ndarray:
    n = counters.shape[0]
    c = torch.from_numpy(counters.astype(np.uint64).view(np.int64)).to(device)
    k = torch.from_numpy(keys.astype(np.uint64).view(np.int64)).to(device)
    out = torch.empty((n, 4), dtype=torch.int64, device=device)
    check(lib().specdec_philox4x64(c.data_ptr(), k.data_ptr(), n, out.data_ptr(), _stream(None)), "philox")
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint64)


class Round:
    """One speculative decoding job: caches, state and the round handle."""

    def __init__(self, target: Model, k: int, *, mode=GREEDY, bonus=True, schedule=SCHEDULE_A,
                 draft_source=DRAFT_TABLE, table: np.ndarray | None = None, draft: Model | None = None,
                 noise: np.ndarray | None = None, seed: int = 3, max_len: int, cap: int = 1024, device="cuda",
                 events=None, n_events: int = 0, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                 relax_delta: float = 0.0):
        L = lib()
        self.target, self.draft, self.k = target, draft, k
        self.schedule, self.mode, self.draft_source = schedule, mode, draft_source
        sh = target.shape
        self.tcache = Cache(sh, max_len, device)
        self.ws = Workspace(sh, max_len, device=device)
        self.dcache = self.dws = None
        if draft_source == DRAFT_MODEL:
            self.dcache = Cache(draft.shape, max_len, device)
            self.dws = Workspace(draft.shape, max_len, device=device)
        nb = C.c_size_t()
        check(L.specdec_round_state_bytes(cap, C.byref(nb)), "state_bytes")
        self.state = _dev_bytes(nb.value, device)
        self.state.zero_()
        check(L.specdec_round_ws_bytes(C.byref(target.desc), k, C.byref(nb)), "round_ws_bytes")
        self.rws = _dev_bytes(nb.value, device)
        self.rws.zero_()
        self.table = torch.from_numpy(np.asarray(table, np.int32)).to(device) if table is not None else None
        self.noise = torch.from_numpy(np.ascontiguousarray(noise, np.float32)).to(device) if noise is not None else None
        d = RoundDesc()
        d.target, d.target_cache = target.handle, self.tcache.handle
        d.draft = draft.handle if draft is not None else None
        d.draft_cache = self.dcache.handle if self.dcache is not None else None
        d.k, d.mode, d.bonus, d.schedule, d.draft_source = k, mode, 1 if bonus else 0, schedule, draft_source
        d.d_draft_table = _ptr(self.table)
        d.table_len = int(self.table.numel()) if self.table is not None else 0
        d.d_noise = _ptr(self.noise)
        d.noise_rows = int(self.noise.shape[0]) if self.noise is not None else 0
        d.philox_seed = seed
        d.d_state = self.state.data_ptr()
        d.d_ws, d.ws_bytes = self.ws.mem.data_ptr(), self.ws.nbytes
        if self.dws is not None:
            d.d_draft_ws, d.draft_ws_bytes = self.dws.mem.data_ptr(), self.dws.nbytes
        d.d_round_ws, d.round_ws_bytes = self.rws.data_ptr(), self.rws.numel()
        d.state_cap = cap
        d.temperature, d.top_k, d.top_p, d.relax_delta = temperature, top_k, top_p, relax_delta
        if events is not None:
            d.events = C.cast(events, C.POINTER(C.c_void_p))
            d.n_events = n_events
        self._events = events
        self._calls = 0
        self.desc = d
        h = C.c_void_p()
        check(L.specdec_round_create(C.byref(d), C.byref(h)), "round_create")
        self.handle = h
        self.cap = cap

    def prefill(self, prompt: np.ndarray, chunk: int = MAX_ROWS, stream=None) -> None:
        self.prompt = torch.from_numpy(np.asarray(prompt, np.int32)).to(self.state.device)
        check(lib().specdec_round_prefill(self.handle, self.prompt.data_ptr(), int(self.prompt.numel()), chunk,
                                          _stream(stream)), "round_prefill")

    def reset(self, n_target: int, stream=None) -> None:
        check(lib().specdec_round_reset(self.handle, n_target, _stream(stream)), "round_reset")

    def step(self, stream=None) -> None:
        check(lib().specdec_verify_round(self.handle, _stream(stream)), "verify_round")
        self._calls += 1

    def calls(self) -> int:
        """Rounds enqueued so far (the index the library uses for its event ring)."""
        return self._calls

    def debug_view(self, which: int, dtype=torch.float32) -> torch.Tensor:
        """A torch view (no copy) of an internal round buffer (see specdec_round_debug_view)."""
        ptr, nb = C.c_void_p(), C.c_size_t()
        check(lib().specdec_round_debug_view(self.handle, which, C.byref(ptr), C.byref(nb)), "debug_view")
        base = self.rws.data_ptr()
        off = ptr.value - base
        assert 0 <= off and off + nb.value <= self.rws.numel()
        return self.rws[off:off + nb.value].view(dtype)

    def read_state(self):
        raw = self.state.cpu().numpy()
        st = RoundState.from_buffer_copy(raw[:C.sizeof(RoundState)].tobytes())
        toks = raw[C.sizeof(RoundState):].view(np.int32)
        return st, toks[: min(st.n_committed, self.cap)].copy()

    def capture(self) -> None:
        """Capture the round as four HIP graphs (replayed by run(graph=True))."""
        check(lib().specdec_round_graph(self.handle), "round_graph")

    def committed(self) -> int:
        return int(self.state[:4].view(torch.int32).item())

    def run(self, n_new: int, stream=None, graph: bool = False, max_rounds: int = 100000):
        """Reset to the post-prefill state and run rounds until n_new tokens are committed.

        Each host check launches ceil((n_new - n) / (k + 1)) rounds first: a
        round commits at most k + 1 tokens, so every one of them is needed
        (rounds past the target would return at once on the device anyway).
        """
        self.reset(n_new, stream)
        rounds, n = 0, 0
        while rounds < max_rounds and n < n_new:
            batch = max(1, -(-(n_new - n) // (self.k + 1)))
            if graph:
                check(lib().specdec_round_graph_launch(self.handle, batch, _stream(stream)), "round_graph_launch")
                self._calls += batch
            else:
                for _ in range(batch):
                    self.step(stream)
            rounds += batch
            n = self.committed()
        return self.read_state()

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.specdec_round_destroy(self.handle)
            self.handle = None
