"""Python binding of the streaming codec (decoder and encoder) in libpp.so
(include/codec.h): the C entry points under the same names, plus a
CodecEngine that owns the device buffers (torch tensors) a handle needs.
Argument marshalling only: every step runs in the library's HIP kernels."""
from __future__ import annotations

import ctypes

import numpy as np

from full_duplex_speech_moshi_amd import pp

PP_CODEC_MAX_STAGES = 6
PP_CODEC_MAX_BATCH = 32
PP_CODEC_MAX_WINDOW = 256

EXPORTS = ("pp_codec_samples", "pp_codec_arena_bytes", "pp_codec_create", "pp_codec_decode", "pp_codec_encode",
           "pp_codec_reset", "pp_codec_time", "pp_codec_time_encode", "pp_codec_taps", "pp_codec_destroy",
           "pp_codec_last_error")

_S = PP_CODEC_MAX_STAGES


class PPCodecDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_q", "card", "d", "n_layers", "n_heads", "ffn", "window", "conv_k", "res_k", "n_stages")] + \
               [("strides", ctypes.c_int32 * _S), ("channels", ctypes.c_int32 * (_S + 1)),
                ("norm_eps", ctypes.c_float), ("rope_base", ctypes.c_float)]


CODEC_WEIGHT_FIELDS = ("codebooks", "attn_norm", "wqkv", "wo", "mlp_norm", "w_in", "w_out", "out_norm",
                       "conv_in_w", "conv_in_b")
CODEC_STAGE_FIELDS = ("up_w", "up_b", "res_a_w", "res_a_b", "res_b_w", "res_b_b")


class PPCodecTaps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ring", "z", "enc_ring", "enc_y", "enc_z")]


ENC_STAGE_FIELDS = ("enc_res_a_w", "enc_res_a_b", "enc_res_b_w", "enc_res_b_b", "enc_down_w", "enc_down_b")
ENC_TAIL_FIELDS = ("enc_conv_out_w", "enc_conv_out_b", "enc_attn_norm", "enc_wqkv", "enc_wo", "enc_mlp_norm",
                   "enc_w_in", "enc_w_out", "enc_out_norm")


class PPCodecWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in CODEC_WEIGHT_FIELDS] + \
               [(n, ctypes.c_void_p * _S) for n in CODEC_STAGE_FIELDS] + \
               [("conv_out_w", ctypes.c_void_p), ("conv_out_b", ctypes.c_void_p),
                ("enc_conv_in_w", ctypes.c_void_p), ("enc_conv_in_b", ctypes.c_void_p)] + \
               [(n, ctypes.c_void_p * _S) for n in ENC_STAGE_FIELDS] + \
               [(n, ctypes.c_void_p) for n in ENC_TAIL_FIELDS]


_ready = False


def _lib() -> ctypes.CDLL:
    global _ready
    lib = pp.load_library()
    if not _ready:
        P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.pp_codec_samples.argtypes = [ctypes.POINTER(PPCodecDims)]
        lib.pp_codec_arena_bytes.argtypes = [ctypes.POINTER(PPCodecDims), I, ctypes.POINTER(SZ)]
        lib.pp_codec_create.argtypes = [ctypes.POINTER(PPCodecDims), I, ctypes.POINTER(PPCodecWeights), P, SZ, P,
                                        ctypes.POINTER(P)]
        lib.pp_codec_decode.argtypes = [P, P, P]
        lib.pp_codec_encode.argtypes = [P, P, P]
        lib.pp_codec_time_encode.argtypes = [P, I, ctypes.POINTER(ctypes.c_float)]
        lib.pp_codec_reset.argtypes = [P, I]
        lib.pp_codec_time.argtypes = [P, I, ctypes.POINTER(ctypes.c_float)]
        lib.pp_codec_taps.argtypes = [P, ctypes.POINTER(PPCodecTaps)]
        lib.pp_codec_destroy.argtypes = [P]
        lib.pp_codec_destroy.restype = None
        lib.pp_codec_last_error.argtypes = [P]
        lib.pp_codec_last_error.restype = ctypes.c_char_p
        for n in EXPORTS:
            if n not in ("pp_codec_destroy", "pp_codec_last_error"):
                getattr(lib, n).restype = I
        _ready = True
    return lib


def _check(rc, handle=None):
    if rc != pp.PP_OK:
        raise pp.PPError(rc, _lib().pp_codec_last_error(handle).decode(errors="replace"))


def make_codec_dims(cd) -> PPCodecDims:
    n = len(cd.strides)
    st = (ctypes.c_int32 * _S)(*(list(cd.strides) + [0] * (_S - n)))
    ch = (ctypes.c_int32 * (_S + 1))(*(list(cd.channels) + [0] * (_S + 1 - len(cd.channels))))
    return PPCodecDims(cd.n_q, cd.card, cd.d, cd.n_layers, cd.n_heads, cd.ffn, cd.window, cd.conv_k, cd.res_k, n,
                       st, ch, float(cd.norm_eps), float(cd.rope_base))


# ------------------------------------------------------------------ C entry points

def pp_codec_samples(dims: PPCodecDims) -> int:
    rc = _lib().pp_codec_samples(ctypes.byref(dims))
    _check(min(rc, 0))
    return rc


def pp_codec_arena_bytes(dims: PPCodecDims, B: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib().pp_codec_arena_bytes(ctypes.byref(dims), B, ctypes.byref(out)))
    return out.value


def pp_codec_create(dims: PPCodecDims, B: int, weights: PPCodecWeights, arena_ptr: int, arena_bytes: int,
                    stream_ptr: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib().pp_codec_create(ctypes.byref(dims), B, ctypes.byref(weights), arena_ptr, arena_bytes, stream_ptr,
                                  ctypes.byref(h)))
    return h.value


def pp_codec_decode(h: int, codes, B: int, n_q: int, samples: int) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.int32).reshape(B, n_q)
    pcm = np.empty((B, samples), np.float32)
    _check(_lib().pp_codec_decode(h, c.ctypes.data, pcm.ctypes.data), h)
    return pcm


def pp_codec_encode(h: int, pcm, B: int, n_q: int, samples: int) -> np.ndarray:
    x = np.ascontiguousarray(pcm, dtype=np.float32).reshape(B, samples)
    codes = np.empty((B, n_q), np.int32)
    _check(_lib().pp_codec_encode(h, x.ctypes.data, codes.ctypes.data), h)
    return codes


def pp_codec_time_encode(h: int, iters: int) -> float:
    ms = ctypes.c_float()
    _check(_lib().pp_codec_time_encode(h, iters, ctypes.byref(ms)), h)
    return ms.value


def pp_codec_reset(h: int, slot: int) -> None:
    _check(_lib().pp_codec_reset(h, slot), h)


def pp_codec_time(h: int, iters: int) -> float:
    ms = ctypes.c_float()
    _check(_lib().pp_codec_time(h, iters, ctypes.byref(ms)), h)
    return ms.value


def pp_codec_taps(h: int) -> PPCodecTaps:
    t = PPCodecTaps()
    _check(_lib().pp_codec_taps(h, ctypes.byref(t)), h)
    return t


def pp_codec_destroy(h: int) -> None:
    _lib().pp_codec_destroy(h)


# ------------------------------------------------------------------ weights and engine

def upload_codec_weights(cd, w: dict, device):
    """Copy the codec's manifest-named host weights to device tensors: the
    codebooks stacked, the transformer matrices stacked per layer and packed
    into the tile layout on the device (pp_pack_matrix), the rest as they are."""
    import torch
    stream = torch.cuda.current_stream(device)
    t = {}

    def dev(a):
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else np.ascontiguousarray(a)).to(device)

    t["codebooks"] = dev(np.stack([w[f"codebook.{q}"] for q in range(cd.n_q)]))
    shapes = {"wqkv": (3 * cd.d, cd.d), "wo": (cd.d, cd.d), "w_in": (2 * cd.ffn, cd.d), "w_out": (cd.d, cd.ffn)}
    for pre in ("", "enc."):
        for k in ("attn_norm", "mlp_norm"):
            t[pre + k] = dev(np.stack([w[f"{pre}layers.{l}.{k}"] for l in range(cd.n_layers)]))
        for k, (M, K) in shapes.items():
            pe = pp.pp_packed_elems(M, K)
            out = torch.empty(cd.n_layers * pe, dtype=torch.int16, device=device)
            for l in range(cd.n_layers):
                src = dev(w[f"{pre}layers.{l}.{k}"])
                pp.pp_pack_matrix(src.data_ptr(), M, K, out.data_ptr() + 2 * l * pe, stream.cuda_stream)
                stream.synchronize()
            t[pre + k] = out
        t[pre + "out_norm"] = dev(w[pre + "out_norm"])
    for k in ("conv_in.w", "conv_in.b", "conv_out.w", "conv_out.b", "enc.conv_in.w", "enc.conv_in.b",
              "enc.conv_out.w", "enc.conv_out.b"):
        t[k] = dev(w[k])
    for i in range(len(cd.strides)):
        for k in ("w", "b"):
            for name in (f"up.{i}", f"res.{i}.a", f"res.{i}.b", f"enc.res.{i}.a", f"enc.res.{i}.b", f"enc.down.{i}"):
                t[f"{name}.{k}"] = dev(w[f"{name}.{k}"])
    torch.cuda.synchronize(device)
    p = PPCodecWeights()
    for k in ("codebooks", "attn_norm", "wqkv", "wo", "mlp_norm", "w_in", "w_out", "out_norm"):
        setattr(p, k, t[k].data_ptr())
    p.conv_in_w, p.conv_in_b = t["conv_in.w"].data_ptr(), t["conv_in.b"].data_ptr()
    p.conv_out_w, p.conv_out_b = t["conv_out.w"].data_ptr(), t["conv_out.b"].data_ptr()
    for i in range(len(cd.strides)):
        p.up_w[i], p.up_b[i] = t[f"up.{i}.w"].data_ptr(), t[f"up.{i}.b"].data_ptr()
        p.res_a_w[i], p.res_a_b[i] = t[f"res.{i}.a.w"].data_ptr(), t[f"res.{i}.a.b"].data_ptr()
        p.res_b_w[i], p.res_b_b[i] = t[f"res.{i}.b.w"].data_ptr(), t[f"res.{i}.b.b"].data_ptr()
        p.enc_res_a_w[i], p.enc_res_a_b[i] = t[f"enc.res.{i}.a.w"].data_ptr(), t[f"enc.res.{i}.a.b"].data_ptr()
        p.enc_res_b_w[i], p.enc_res_b_b[i] = t[f"enc.res.{i}.b.w"].data_ptr(), t[f"enc.res.{i}.b.b"].data_ptr()
        p.enc_down_w[i], p.enc_down_b[i] = t[f"enc.down.{i}.w"].data_ptr(), t[f"enc.down.{i}.b"].data_ptr()
    p.enc_conv_in_w, p.enc_conv_in_b = t["enc.conv_in.w"].data_ptr(), t["enc.conv_in.b"].data_ptr()
    p.enc_conv_out_w, p.enc_conv_out_b = t["enc.conv_out.w"].data_ptr(), t["enc.conv_out.b"].data_ptr()
    for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_in", "w_out", "out_norm"):
        setattr(p, "enc_" + k, t["enc." + k].data_ptr())
    return t, p


class CodecEngine:
    """A streaming codec decoder of B slots on one GPU.  Owns the weight
    tensors, the arena and a stream (default priority)."""

    def __init__(self, cd, weights: dict, B: int, device="cuda:0", device_weights=None):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("no GPU visible: the codec decoder runs only on the HIP device")
        _lib()
        self.cd, self.B = cd, int(B)
        self.device = torch.device(device)
        self.dims = make_codec_dims(cd)
        self.samples = pp_codec_samples(self.dims)
        if device_weights is None:
            device_weights = upload_codec_weights(cd, weights, self.device)
        self.wt, self.wptrs = device_weights
        nbytes = pp_codec_arena_bytes(self.dims, self.B)
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.Stream(device=self.device)
        torch.cuda.synchronize(self.device)
        self.h = pp_codec_create(self.dims, self.B, self.wptrs, self.arena.data_ptr(), nbytes,
                                 self.stream.cuda_stream)

    def decode(self, codes) -> np.ndarray:
        return pp_codec_decode(self.h, codes, self.B, self.cd.n_q, self.samples)

    def encode(self, pcm) -> np.ndarray:
        return pp_codec_encode(self.h, pcm, self.B, self.cd.n_q, self.samples)

    def time_encode(self, iters=20) -> float:
        return pp_codec_time_encode(self.h, iters)

    def reset(self, slot):
        pp_codec_reset(self.h, slot)

    def time(self, iters=20) -> float:
        return pp_codec_time(self.h, iters)

    def taps(self) -> dict:
        """Host copies of the decoder's state after the last call: the
        transformer's stored keys and values as bf16 bits [B][L][2][H][W][Dh]
        and the last output norm z [B][d]."""
        import torch
        t = pp_codec_taps(self.h)
        cd, B = self.cd, self.B
        base = self.arena.data_ptr()
        torch.cuda.synchronize(self.device)

        def view(ptr, dtype, isz, shape):
            off, n = ptr - base, int(np.prod(shape))
            return self.arena[off:off + n * isz].view(dtype).reshape(shape).cpu().numpy()

        shape = (B, cd.n_layers, 2, cd.n_heads, cd.window, cd.head_dim)
        return {"ring": view(t.ring, torch.int16, 2, shape).view(np.uint16),
                "z": view(t.z, torch.float32, 4, (B, cd.d)),
                "enc_ring": view(t.enc_ring, torch.int16, 2, shape).view(np.uint16),
                "enc_y": view(t.enc_y, torch.float32, 4, (B, cd.d)),
                "enc_z": view(t.enc_z, torch.float32, 4, (B, cd.d))}

    def close(self):
        if getattr(self, "h", None):
            pp_codec_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
