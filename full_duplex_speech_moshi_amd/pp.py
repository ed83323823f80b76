"""Python binding of libpp.so (ctypes): the C entry points under the same
names, plus an Engine class that owns the device buffers (torch tensors) a
handle needs.  Argument marshalling only: every step of the tick runs in the
library's HIP kernels.  Importing works without a GPU; creating an Engine
without the built library or without a GPU raises."""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpp.so")

PP_OK, PP_EINVAL, PP_EBUSY, PP_ENOSPC, PP_EDEVICE = 0, -1, -2, -3, -4
PP_MAX_BATCH = 32
PP_MAX_WINDOW = 4096
PP_MAX_QUEUE = 4096
PP_MAX_DELAY = 4
TO_STRIDE = 32

EXPORTS = ("pp_arena_bytes", "pp_create", "pp_prefill_forced", "pp_prefill_embed", "pp_step", "pp_step_static",
           "pp_set_acoustic_delay", "pp_agent_frames", "pp_set_sampling", "pp_slot_seed", "pp_slot_reset",
           "pp_ring_fill", "pp_taps",
           "pp_time_kernel", "pp_time_graph", "pp_set_depformer_loop", "pp_depformer_loop_active", "pp_destroy",
           "pp_last_error", "pp_packed_elems", "pp_pack_matrix")

KERNELS = {"qkv": 0, "attention": 1, "out_proj": 2, "gate_up": 3, "down": 4, "text_head": 5}


class PPDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("d", "n_layers", "n_heads", "ffn", "text_card", "audio_card", "n_q",
                 "dep_d", "dep_layers", "dep_heads", "dep_ffn", "dep_q")] + \
               [("norm_eps", ctypes.c_float), ("rope_base", ctypes.c_float)]


WEIGHT_FIELDS = ("emb_text", "emb_audio", "attn_norm", "wqkv", "wo", "mlp_norm", "w_in", "w_out",
                 "out_norm", "text_head", "dep_in_proj", "dep_emb_text", "dep_emb_audio",
                 "dep_attn_norm", "dep_wqkv", "dep_wo", "dep_mlp_norm", "dep_w_in", "dep_w_out",
                 "dep_out_norm", "dep_heads")


class PPWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class PPTaps(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_void_p), ("text_logits", ctypes.c_void_p),
                ("dep_logits", ctypes.c_void_p), ("tokens", ctypes.c_void_p)]


class PPSampling(ctypes.Structure):
    _fields_ = [("text_temperature", ctypes.c_float), ("audio_temperature", ctypes.c_float),
                ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float), ("repetition_penalty", ctypes.c_float)]


class PPError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpp.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run `python -m full_duplex_speech_moshi_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.pp_arena_bytes.argtypes = [ctypes.POINTER(PPDims), I, I, ctypes.POINTER(SZ)]
    lib.pp_create.argtypes = [ctypes.POINTER(PPDims), I, I, ctypes.POINTER(PPWeights), P, SZ, P,
                              ctypes.POINTER(P)]
    lib.pp_prefill_forced.argtypes = [P, I, P, I]
    lib.pp_prefill_embed.argtypes = [P, I, P, P, I]
    lib.pp_set_acoustic_delay.argtypes = [P, I]
    lib.pp_agent_frames.argtypes = [P, P, P]
    lib.pp_set_sampling.argtypes = [P, ctypes.POINTER(PPSampling)]
    lib.pp_slot_seed.argtypes = [P, I, ctypes.c_uint64]
    lib.pp_step.argtypes = [P, P, P]
    lib.pp_step_static.argtypes = [P, P, P]
    lib.pp_slot_reset.argtypes = [P, I]
    lib.pp_ring_fill.argtypes = [P, I, I, P, P]
    lib.pp_taps.argtypes = [P, ctypes.POINTER(PPTaps)]
    lib.pp_time_kernel.argtypes = [P, I, I, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    lib.pp_time_graph.argtypes = [P, I, ctypes.POINTER(ctypes.c_float)]
    lib.pp_set_depformer_loop.argtypes = [P, I]
    lib.pp_depformer_loop_active.argtypes = [P]
    lib.pp_destroy.argtypes = [P]
    lib.pp_destroy.restype = None
    lib.pp_last_error.argtypes = [P]
    lib.pp_last_error.restype = ctypes.c_char_p
    lib.pp_packed_elems.argtypes = [I, I]
    lib.pp_packed_elems.restype = SZ
    lib.pp_pack_matrix.argtypes = [P, I, I, P, P]
    for n in EXPORTS:
        if n not in ("pp_destroy", "pp_last_error", "pp_packed_elems"):
            getattr(lib, n).restype = I
    _lib = lib
    return lib


def make_dims(dm) -> PPDims:
    return PPDims(dm.d, dm.n_layers, dm.n_heads, dm.ffn, dm.text_card, dm.audio_card, dm.n_q,
                  dm.dep_d, dm.dep_layers, dm.dep_heads, dm.dep_ffn, dm.dep_q,
                  float(dm.norm_eps), float(dm.rope_base))


def _check(rc, handle=None):
    if rc != PP_OK:
        msg = load_library().pp_last_error(handle).decode(errors="replace")
        raise PPError(rc, msg)


def _i32(a, shape):
    a = np.ascontiguousarray(a, dtype=np.int32)
    if a.shape != shape:
        a = a.reshape(shape)
    return a


# ------------------------------------------------------------------ C entry points

def pp_arena_bytes(dims: PPDims, B: int, window: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().pp_arena_bytes(ctypes.byref(dims), B, window, ctypes.byref(out)))
    return out.value


def pp_create(dims: PPDims, B: int, window: int, weights: PPWeights, arena_ptr: int, arena_bytes: int,
              stream_ptr: int) -> int:
    h = ctypes.c_void_p()
    _check(load_library().pp_create(ctypes.byref(dims), B, window, ctypes.byref(weights),
                                    ctypes.c_void_p(arena_ptr), arena_bytes, ctypes.c_void_p(stream_ptr),
                                    ctypes.byref(h)))
    return h.value


def pp_prefill_forced(h: int, slot: int, frames) -> None:
    f = np.ascontiguousarray(frames, dtype=np.int32).reshape(-1, 17)
    _check(load_library().pp_prefill_forced(h, slot, f.ctypes.data, f.shape[0]), h)


def pp_prefill_embed(h: int, slot: int, x, force=None) -> None:
    xv = np.ascontiguousarray(x, dtype=np.float32)
    n = xv.shape[0] if xv.ndim == 2 else 1
    f = None if force is None else np.ascontiguousarray(force, dtype=np.int32).reshape(n, 9)
    _check(load_library().pp_prefill_embed(h, slot, xv.ctypes.data, None if f is None else f.ctypes.data, n), h)


def pp_set_acoustic_delay(h: int, frames: int) -> None:
    _check(load_library().pp_set_acoustic_delay(h, frames), h)


def pp_set_sampling(h: int, text_temperature=None, audio_temperature=0.0, top_k=0, top_p=1.0,
                    repetition_penalty=1.0) -> None:
    """text_temperature None: back to greedy."""
    if text_temperature is None:
        _check(load_library().pp_set_sampling(h, None), h)
        return
    sp = PPSampling(text_temperature, audio_temperature, top_k, top_p, repetition_penalty)
    _check(load_library().pp_set_sampling(h, ctypes.byref(sp)), h)


def pp_slot_seed(h: int, slot: int, seed: int) -> None:
    _check(load_library().pp_slot_seed(h, slot, seed), h)


def pp_agent_frames(h: int, B: int):
    frames = np.empty((B, 8), np.int32)
    valid = np.empty(B, np.int32)
    _check(load_library().pp_agent_frames(h, frames.ctypes.data, valid.ctypes.data), h)
    return frames, valid.astype(bool)


def pp_step(h: int, user_codes, B: int) -> np.ndarray:
    u = _i32(user_codes, (B, 8))
    tok = np.empty((B, 9), np.int32)
    _check(load_library().pp_step(h, u.ctypes.data, tok.ctypes.data), h)
    return tok


def pp_step_static(h: int, user_codes, B: int) -> np.ndarray:
    u = _i32(user_codes, (B, 8))
    tok = np.empty((B, 9), np.int32)
    _check(load_library().pp_step_static(h, u.ctypes.data, tok.ctypes.data), h)
    return tok


def pp_slot_reset(h: int, slot: int) -> None:
    _check(load_library().pp_slot_reset(h, slot), h)


def pp_ring_fill(h: int, slot: int, k_bits, v_bits) -> None:
    k = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    if k.shape != v.shape or k.ndim != 4:
        raise ValueError("k and v must both be [L, n, H, head_dim]")
    _check(load_library().pp_ring_fill(h, slot, k.shape[1], k.ctypes.data, v.ctypes.data), h)


def pp_taps(h: int) -> PPTaps:
    t = PPTaps()
    _check(load_library().pp_taps(h, ctypes.byref(t)), h)
    return t


def pp_time_kernel(h: int, which: int, iters: int):
    ms = ctypes.c_float()
    by = ctypes.c_double()
    _check(load_library().pp_time_kernel(h, which, iters, ctypes.byref(ms), ctypes.byref(by)), h)
    return ms.value, by.value


def pp_time_graph(h: int, iters: int) -> float:
    ms = ctypes.c_float()
    _check(load_library().pp_time_graph(h, iters, ctypes.byref(ms)), h)
    return ms.value


def pp_set_depformer_loop(h: int, on: bool) -> None:
    _check(load_library().pp_set_depformer_loop(h, 1 if on else 0), h)


def pp_depformer_loop_active(h: int) -> bool:
    rc = load_library().pp_depformer_loop_active(h)
    if rc < 0:
        _check(rc, h)
    return rc == 1


def pp_packed_elems(M: int, K: int) -> int:
    return load_library().pp_packed_elems(M, K)


def pp_pack_matrix(src_ptr: int, M: int, K: int, dst_ptr: int, stream_ptr: int) -> None:
    _check(load_library().pp_pack_matrix(ctypes.c_void_p(src_ptr), M, K, ctypes.c_void_p(dst_ptr),
                                         ctypes.c_void_p(stream_ptr)))


def pp_destroy(h: int) -> None:
    if h:
        load_library().pp_destroy(h)


# ------------------------------------------------------------------ device weights

def _per_layer_groups(dm):
    """(field, manifest name pattern, count) of the stacked weight tensors."""
    L, Ld, Q = dm.n_layers, dm.dep_layers, dm.dep_q
    return [("emb_text", "emb.text", None), ("emb_audio", "emb.audio.{}", (0, 2 * dm.n_q)),
            ("attn_norm", "layers.{}.attn_norm", (0, L)), ("wqkv", "layers.{}.wqkv", (0, L)),
            ("wo", "layers.{}.wo", (0, L)), ("mlp_norm", "layers.{}.mlp_norm", (0, L)),
            ("w_in", "layers.{}.w_in", (0, L)), ("w_out", "layers.{}.w_out", (0, L)),
            ("out_norm", "out_norm", None), ("text_head", "text_head", None),
            ("dep_in_proj", "dep.in_proj.{}", (0, Q)), ("dep_emb_text", "dep.emb.text", None),
            ("dep_emb_audio", "dep.emb.audio.{}", (1, Q)),
            ("dep_attn_norm", "dep.layers.{}.attn_norm", (0, Ld)), ("dep_wqkv", "dep.layers.{}.wqkv", (0, Ld)),
            ("dep_wo", "dep.layers.{}.wo", (0, Ld)), ("dep_mlp_norm", "dep.layers.{}.mlp_norm", (0, Ld)),
            ("dep_w_in", "dep.layers.{}.w_in", (0, Ld)), ("dep_w_out", "dep.layers.{}.w_out", (0, Ld)),
            ("dep_out_norm", "dep.out_norm", None), ("dep_heads", "dep.head.{}", (0, Q))]


def _matrix_shape(dm, field):
    """(rows, cols) of each matrix of a stacked matrix field, or None for
    tables and alphas (which stay row-major)."""
    d, F, dd, dF = dm.d, dm.ffn, dm.dep_d, dm.dep_ffn
    return {"wqkv": (3 * d, d), "wo": (d, d), "w_in": (2 * F, d), "w_out": (d, F),
            "text_head": (dm.text_card, d), "dep_in_proj": (dd, d), "dep_wqkv": (3 * dd, dd),
            "dep_wo": (dd, dd), "dep_w_in": (2 * dF, dd), "dep_w_out": (dd, dF),
            "dep_heads": (dm.audio_card, dd)}.get(field)


def upload_weights(dm, w: dict, device):
    """Copy manifest-named host weights to device tensors in the library's
    stacked layout, one manifest entry at a time; matrices are packed into the
    tile layout on the device by pp_pack_matrix."""
    import torch
    stream = torch.cuda.current_stream(device)
    tensors = {}
    for field, pat, rng in _per_layer_groups(dm):
        names = [pat] if rng is None else [pat.format(i) for i in range(*rng)]
        first = w[names[0]]
        shape = _matrix_shape(dm, field)
        if shape is None:
            tdt = torch.int16 if first.dtype == np.uint16 else torch.float32
            tshape = first.shape if rng is None else (len(names),) + first.shape
            t = torch.empty(tshape, dtype=tdt, device=device)
            for i, n in enumerate(names):
                a = w[n]
                src = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
                (t if rng is None else t[i]).copy_(src)
        else:
            M, K = shape
            pe = pp_packed_elems(M, K)
            t = torch.empty(len(names) * pe, dtype=torch.int16, device=device)
            for i, n in enumerate(names):
                src = torch.from_numpy(w[n].view(np.int16)).to(device)
                pp_pack_matrix(src.data_ptr(), M, K, t.data_ptr() + 2 * i * pe, stream.cuda_stream)
                stream.synchronize()
                del src
        tensors[field] = t
    ptrs = PPWeights(**{f: tensors[f].data_ptr() for f in WEIGHT_FIELDS})
    return tensors, ptrs


class Engine:
    """A lockstep engine of B slots on one GPU.  Owns the weight tensors, the
    arena and a stream (default priority); the handle is destroyed by close()."""

    def __init__(self, dm, weights: dict, B: int, window: int, device="cuda:0", device_weights=None):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("no GPU visible: the lockstep engine runs only on the HIP device")
        load_library()
        self.dm, self.B, self.W = dm, int(B), int(window)
        self.device = torch.device(device)
        self.dims = make_dims(dm)
        if device_weights is None:
            device_weights = upload_weights(dm, weights, self.device)
        self.wt, self.wptrs = device_weights
        nbytes = pp_arena_bytes(self.dims, self.B, self.W)
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.Stream(device=self.device)
        torch.cuda.synchronize(self.device)
        self.h = pp_create(self.dims, self.B, self.W, self.wptrs, self.arena.data_ptr(), nbytes,
                           self.stream.cuda_stream)

    # thin wrappers
    def prefill_forced(self, slot, frames):
        pp_prefill_forced(self.h, slot, frames)

    def prefill_embed(self, slot, x, force=None):
        pp_prefill_embed(self.h, slot, x, force)

    def set_acoustic_delay(self, frames):
        pp_set_acoustic_delay(self.h, frames)

    def agent_frames(self):
        return pp_agent_frames(self.h, self.B)

    def set_sampling(self, text_temperature=None, audio_temperature=0.0, top_k=0, top_p=1.0, repetition_penalty=1.0):
        pp_set_sampling(self.h, text_temperature, audio_temperature, top_k, top_p, repetition_penalty)

    def slot_seed(self, slot, seed):
        pp_slot_seed(self.h, slot, seed)

    def step(self, user_codes) -> np.ndarray:
        return pp_step(self.h, user_codes, self.B)

    def step_static(self, user_codes) -> np.ndarray:
        return pp_step_static(self.h, user_codes, self.B)

    def slot_reset(self, slot):
        pp_slot_reset(self.h, slot)

    def ring_fill(self, slot, k_bits, v_bits):
        pp_ring_fill(self.h, slot, k_bits, v_bits)

    def time_kernel(self, name, iters=20):
        return pp_time_kernel(self.h, KERNELS[name], iters)

    def time_graph(self, iters=10):
        return pp_time_graph(self.h, iters)

    def set_depformer_loop(self, on: bool):
        pp_set_depformer_loop(self.h, on)

    def depformer_loop_active(self) -> bool:
        return pp_depformer_loop_active(self.h)

    def taps(self) -> dict:
        """Host copies of the last tick's taps."""
        import torch
        t = pp_taps(self.h)
        dm, B = self.dm, self.B
        base = self.arena.data_ptr()
        torch.cuda.synchronize(self.device)

        def view(ptr, dtype, shape):
            n = int(np.prod(shape))
            isz = 4
            off = ptr - base
            return self.arena[off:off + n * isz].view(dtype).reshape(shape).cpu().numpy()

        tok = view(t.tokens, torch.int32, (B, TO_STRIDE))
        return dict(hidden=view(t.hidden, torch.float32, (dm.n_layers + 1, B, dm.d)),
                    text_logits=view(t.text_logits, torch.float32, (B, dm.text_card)),
                    dep_logits=view(t.dep_logits, torch.float32, (B, dm.dep_q, dm.audio_card)),
                    tokens=tok[:, 0:9], user_pred=tok[:, 9:17], chosen=tok[:, 17:26])

    def close(self):
        if getattr(self, "h", None):
            pp_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
