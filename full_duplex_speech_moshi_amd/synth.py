"""Seeded synthetic inputs for the lockstep tick: model shapes, weights, token
streams, pre-filled ring contents and session schedules.

This module holds random draws and the fp32 -> bf16 round-to-nearest-even
conversion that turns a draw into a stored bf16 value, and nothing of the
tick's own arithmetic.  Both the CPU oracle and the GPU harness take their
inputs from here, so the two sides see bit-identical weights and streams.

Shapes follow the PersonaPlex recipe ("Architecture (Moshi RQ-Transformer, all
native)": 4096-d / 32 layers / 32 heads temporal, 1024-d / 6 layers / 16 heads
depformer, 16 codebooks of cardinality 2048, 17-row token column, 3000-frame
sliding window) and the frame-layout constants of the vLLM-Omni PersonaPlex
article ("帧 token 布局": TEXT_INITIAL_TOKEN 32000, AUDIO_INITIAL_TOKEN 2048,
AUDIO_SILENCE_FRAME_CNT 6).

RNG: numpy.random.Generator(PCG64(SeedSequence(...))).  Weights draw one child
stream per manifest entry (SeedSequence([seed, index])); every other stream is
named by its integer seed.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

N_ROWS = 17          # token column: 1 text + 8 agent audio + 8 user audio
N_AGENT = 8
N_USER = 8
SILENCE_FRAMES = 6   # AUDIO_SILENCE_FRAME_CNT: 0.5 s at 12.5 Hz
FREE = -1            # "not forced" marker in a forced frame


@dataclasses.dataclass(frozen=True)
class Dims:
    d: int
    n_layers: int
    n_heads: int
    ffn: int
    text_card: int
    audio_card: int
    n_q: int            # audio codebooks per stream in the column (8)
    dep_d: int
    dep_layers: int
    dep_heads: int
    dep_ffn: int
    dep_q: int          # depformer codebooks per frame (16)
    norm_eps: float = 1e-5
    rope_base: float = 10000.0

    @property
    def head_dim(self) -> int:
        return self.d // self.n_heads

    @property
    def dep_head_dim(self) -> int:
        return self.dep_d // self.dep_heads


# Tiny RQ-Transformer used for exhaustive CPU checks (ring window 32 wraps).
TINY = Dims(d=256, n_layers=2, n_heads=4, ffn=704, text_card=1000, audio_card=2048,
            n_q=8, dep_d=128, dep_layers=1, dep_heads=4, dep_ffn=352, dep_q=16)
TINY_WINDOW = 32

# Full 7B shape.
FULL = Dims(d=4096, n_layers=32, n_heads=32, ffn=11264, text_card=32000, audio_card=2048,
            n_q=8, dep_d=1024, dep_layers=6, dep_heads=16, dep_ffn=2816, dep_q=16)
FULL_WINDOW = 3000


# ---------------------------------------------------------------- manifest

def manifest(dm: Dims):
    """Ordered list of (name, shape, kind); kind is 'bf16' (N(0,0.02) weight or
    table, stored as bf16 bits) or 'alpha' (RMSNorm scale 1+N(0,0.01), fp32)."""
    d, F, Vt, A = dm.d, dm.ffn, dm.text_card, dm.audio_card
    dd, dF = dm.dep_d, dm.dep_ffn
    m = [("emb.text", (Vt + 1, d), "bf16")]
    for r in range(2 * dm.n_q):
        m.append((f"emb.audio.{r}", (A + 1, d), "bf16"))
    for l in range(dm.n_layers):
        m += [(f"layers.{l}.attn_norm", (d,), "alpha"),
              (f"layers.{l}.wqkv", (3 * d, d), "bf16"),
              (f"layers.{l}.wo", (d, d), "bf16"),
              (f"layers.{l}.mlp_norm", (d,), "alpha"),
              (f"layers.{l}.w_in", (2 * F, d), "bf16"),
              (f"layers.{l}.w_out", (d, F), "bf16")]
    m += [("out_norm", (d,), "alpha"), ("text_head", (Vt, d), "bf16")]
    for k in range(dm.dep_q):
        m.append((f"dep.in_proj.{k}", (dd, d), "bf16"))
    m.append(("dep.emb.text", (Vt + 1, dd), "bf16"))
    for k in range(1, dm.dep_q):
        m.append((f"dep.emb.audio.{k}", (A + 1, dd), "bf16"))
    for l in range(dm.dep_layers):
        m += [(f"dep.layers.{l}.attn_norm", (dd,), "alpha"),
              (f"dep.layers.{l}.wqkv", (3 * dd, dd), "bf16"),
              (f"dep.layers.{l}.wo", (dd, dd), "bf16"),
              (f"dep.layers.{l}.mlp_norm", (dd,), "alpha"),
              (f"dep.layers.{l}.w_in", (2 * dF, dd), "bf16"),
              (f"dep.layers.{l}.w_out", (dd, dF), "bf16")]
    m.append(("dep.out_norm", (dd,), "alpha"))
    for k in range(dm.dep_q):
        m.append((f"dep.head.{k}", (A, dd), "bf16"))
    return m


# ---------------------------------------------------------------- bf16 storage

_CHUNK = 1 << 20


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    shape = x.shape
    x = x.reshape(-1)
    out = np.empty(x.size, dtype=np.uint16)
    tmp = np.empty(min(_CHUNK, x.size), dtype=np.uint32)
    for s in range(0, x.size, _CHUNK):
        u = x[s:s + _CHUNK].view(np.uint32)
        t = tmp[:u.size]
        np.right_shift(u, 16, out=t)
        np.bitwise_and(t, 1, out=t)
        t += np.uint32(0x7FFF)
        t += u
        np.right_shift(t, 16, out=t)
        out[s:s + _CHUNK] = t
    return out.reshape(shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they denote (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(*seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))


def _normal_bf16(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    buf = np.empty(min(_CHUNK * 8, max(n, 1)), dtype=np.float32)
    for s in range(0, n, buf.size):
        b = buf[:min(buf.size, n - s)]
        rng.standard_normal(out=b, dtype=np.float32)
        if scale != 1.0:
            b *= np.float32(scale)
        out[s:s + b.size] = to_bf16_bits(b)
    return out.reshape(shape)


def _make_tensor(seed: int, index: int, shape, kind: str) -> np.ndarray:
    rng = _rng(seed, index)
    if kind == "bf16":
        return _normal_bf16(rng, shape, 0.02)
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(0.01)
    a += np.float32(1.0)
    return a


def make_weights(dm: Dims, seed: int = 0, threads: int | None = None) -> dict:
    """All weights of the model, name -> array (uint16 bf16 bits or fp32 alpha).
    Each tensor is drawn from its own child stream, so the result does not
    depend on the thread count."""
    man = manifest(dm)
    threads = threads or min(16, os.cpu_count() or 1)
    out = {}
    with ThreadPoolExecutor(threads) as ex:
        futs = {ex.submit(_make_tensor, seed, i, shp, kind): name
                for i, (name, shp, kind) in enumerate(man)}
        for f, name in futs.items():
            out[name] = f.result()
    return out


# ---------------------------------------------------------------- codec

@dataclasses.dataclass(frozen=True)
class CodecDims:
    """A streaming codec decoder of the SoundStream / EnCodec family with a
    transformer (the chenxutan.com PersonaPlex article, section 2.3 on Mimi:
    24 kHz audio <-> 12.5 Hz tokens, 1.1 kbps, causal, transformers in the
    encoder and decoder; the recipe's "Architecture": 8 codebooks of 2048,
    1920 samples per 80 ms frame).  Everything else here is a choice made
    where the pages are silent: they give neither the layer structure nor the
    weights."""
    n_q: int = 8                  # codebooks per frame (agent rows 1-8)
    card: int = 2048              # entries per codebook
    d: int = 512                  # latent width = transformer width
    n_layers: int = 8
    n_heads: int = 8
    ffn: int = 2048
    window: int = 250             # transformer context, frames (20 s)
    conv_k: int = 7               # first and last convolutions
    res_k: int = 3                # first convolution of each residual unit
    strides: tuple = (2, 8, 6, 5, 4)
    channels: tuple = (512, 256, 128, 64, 32, 16)   # after the first convolution, then after each stage
    norm_eps: float = 1e-5
    rope_base: float = 10000.0

    @property
    def head_dim(self) -> int:
        return self.d // self.n_heads

    @property
    def samples(self) -> int:
        """Output samples per frame."""
        return int(np.prod(self.strides))


CODEC = CodecDims()
CODEC_TINY = CodecDims(d=128, n_layers=2, n_heads=2, ffn=256, window=8, strides=(2, 3, 4),
                       channels=(64, 32, 16, 8))


def codec_manifest(cd: CodecDims):
    """Ordered list of (name, shape, kind, scale).  kind 'bf16': N(0, scale)
    stored as bf16 bits; 'alpha': RMSNorm scale 1 + N(0, 0.01), fp32; 'bias':
    N(0, scale), fp32.  Convolution weights are [C_out][C_in][K] for both the
    causal and the transposed convolutions, drawn with scale 1/sqrt(fan-in)
    so that activations stay of order one."""
    d, F = cd.d, cd.ffn
    m = [(f"codebook.{q}", (cd.card, d), "bf16", 1.0 / np.sqrt(cd.n_q)) for q in range(cd.n_q)]
    for l in range(cd.n_layers):
        m += [(f"layers.{l}.attn_norm", (d,), "alpha", 0.0),
              (f"layers.{l}.wqkv", (3 * d, d), "bf16", 0.02),
              (f"layers.{l}.wo", (d, d), "bf16", 0.02),
              (f"layers.{l}.mlp_norm", (d,), "alpha", 0.0),
              (f"layers.{l}.w_in", (2 * F, d), "bf16", 0.02),
              (f"layers.{l}.w_out", (d, F), "bf16", 0.02)]
    m.append(("out_norm", (d,), "alpha", 0.0))
    c = cd.channels
    m += [("conv_in.w", (c[0], d, cd.conv_k), "bf16", 1.0 / np.sqrt(d * cd.conv_k)),
          ("conv_in.b", (c[0],), "bias", 0.01)]
    for i, st in enumerate(cd.strides):
        ci, co = c[i], c[i + 1]
        m += [(f"up.{i}.w", (co, ci, 2 * st), "bf16", 1.0 / np.sqrt(2 * ci)),
              (f"up.{i}.b", (co,), "bias", 0.01),
              (f"res.{i}.a.w", (co // 2, co, cd.res_k), "bf16", 1.0 / np.sqrt(co * cd.res_k)),
              (f"res.{i}.a.b", (co // 2,), "bias", 0.01),
              (f"res.{i}.b.w", (co, co // 2, 1), "bf16", 0.5 / np.sqrt(co // 2)),
              (f"res.{i}.b.b", (co,), "bias", 0.01)]
    m += [("conv_out.w", (1, c[-1], cd.conv_k), "bf16", 1.0 / np.sqrt(c[-1] * cd.conv_k)),
          ("conv_out.b", (1,), "bias", 0.01)]
    # the encoder mirrors the decoder: stage j runs at the channels and the
    # stride of decoder stage n - 1 - j, downsampling where that one upsamples
    n = len(cd.strides)
    m += [("enc.conv_in.w", (c[-1], 1, cd.conv_k), "bf16", 1.0 / np.sqrt(cd.conv_k)),
          ("enc.conv_in.b", (c[-1],), "bias", 0.01)]
    for j in range(n):
        ci, co, st = c[n - j], c[n - 1 - j], cd.strides[n - 1 - j]
        m += [(f"enc.res.{j}.a.w", (ci // 2, ci, cd.res_k), "bf16", 1.0 / np.sqrt(ci * cd.res_k)),
              (f"enc.res.{j}.a.b", (ci // 2,), "bias", 0.01),
              (f"enc.res.{j}.b.w", (ci, ci // 2, 1), "bf16", 0.5 / np.sqrt(ci // 2)),
              (f"enc.res.{j}.b.b", (ci,), "bias", 0.01),
              (f"enc.down.{j}.w", (co, ci, 2 * st), "bf16", 1.0 / np.sqrt(2 * st * ci)),
              (f"enc.down.{j}.b", (co,), "bias", 0.01)]
    m += [("enc.conv_out.w", (d, c[0], cd.conv_k), "bf16", 1.0 / np.sqrt(c[0] * cd.conv_k)),
          ("enc.conv_out.b", (d,), "bias", 0.01)]
    for l in range(cd.n_layers):
        m += [(f"enc.layers.{l}.attn_norm", (d,), "alpha", 0.0),
              (f"enc.layers.{l}.wqkv", (3 * d, d), "bf16", 0.02),
              (f"enc.layers.{l}.wo", (d, d), "bf16", 0.02),
              (f"enc.layers.{l}.mlp_norm", (d,), "alpha", 0.0),
              (f"enc.layers.{l}.w_in", (2 * F, d), "bf16", 0.02),
              (f"enc.layers.{l}.w_out", (d, F), "bf16", 0.02)]
    m.append(("enc.out_norm", (d,), "alpha", 0.0))
    return m


def _make_codec_tensor(seed: int, index: int, shape, kind: str, scale: float) -> np.ndarray:
    rng = _rng(seed, 100000 + index)
    if kind == "bf16":
        return _normal_bf16(rng, shape, scale)
    a = rng.standard_normal(shape, dtype=np.float32)
    if kind == "alpha":
        a *= np.float32(0.01)
        a += np.float32(1.0)
    else:
        a *= np.float32(scale)
    return a


def make_codec_weights(cd: CodecDims, seed: int = 0) -> dict:
    """All codec weights, name -> array (uint16 bf16 bits or fp32), each from
    its own child stream."""
    return {name: _make_codec_tensor(seed, i, shp, kind, scale)
            for i, (name, shp, kind, scale) in enumerate(codec_manifest(cd))}


def user_audio(seed: int, n_frames: int, samples: int = 1920) -> np.ndarray:
    """Synthetic 24 kHz user audio, fp32 [n_frames, samples]: a sum of three
    sinusoids at seeded frequencies (80-1000 Hz) and phases, amplitude 0.3
    each, plus N(0, 0.01) noise; speech-like in level and band, not in
    content."""
    rng = _rng(seed)
    t = np.arange(n_frames * samples, dtype=np.float64) / 24000.0
    x = np.zeros_like(t)
    for _ in range(3):
        f, ph = rng.uniform(80.0, 1000.0), rng.uniform(0.0, 2 * np.pi)
        x += 0.3 * np.sin(2 * np.pi * f * t + ph)
    x += rng.normal(0.0, 0.01, t.size)
    return x.astype(np.float32).reshape(n_frames, samples)


def agent_frames(seed: int, n_frames: int, card: int = 2048) -> np.ndarray:
    """i.i.d. uniform agent-audio frames for the codec, int32 [n_frames, 8]."""
    return _rng(seed).integers(0, card, (n_frames, N_AGENT), dtype=np.int32)


# ---------------------------------------------------------------- streams

def user_codes(seed: int, n_ticks: int, card: int = 2048) -> np.ndarray:
    """i.i.d. uniform user codes, int32 [n_ticks, 8]."""
    return _rng(seed).integers(0, card, (n_ticks, N_USER), dtype=np.int32)


def fixed_frame(seed: int, card: int = 2048) -> np.ndarray:
    """One 8-code frame drawn once (stand-in for the silence/sine constant
    frames whose values the pages do not print)."""
    return _rng(seed).integers(0, card, N_USER, dtype=np.int32)


def ring_fill(dm: Dims, seed: int, n: int):
    """Pre-filled ring contents for positions 0..n-1: K then V, each bf16 bits
    [L, n, H, Dh], values N(0,1).  The draws are the stored (post-rotation)
    keys and values."""
    rng = _rng(seed)
    shape = (dm.n_layers, n, dm.n_heads, dm.head_dim)
    k = _normal_bf16(rng, shape, 1.0)
    v = _normal_bf16(rng, shape, 1.0)
    return k, v


def alternating_codes(n_ticks: int, seed_random: int = 1, seed_fixed: int = 2,
                      block: int = 40, card: int = 2048) -> np.ndarray:
    """User codes in alternating blocks: uniform random, then a fixed repeated
    silence-like frame."""
    rnd = user_codes(seed_random, n_ticks, card)
    fix = fixed_frame(seed_fixed, card)
    out = rnd.copy()
    for t in range(n_ticks):
        if (t // block) % 2 == 1:
            out[t] = fix
    return out


def open_schedule(voice_codes: np.ndarray, persona: np.ndarray, silence: np.ndarray,
                  sine: np.ndarray) -> np.ndarray:
    """Forced frames for session open, int32 [n, 17]: voice frames force the
    agent rows, then silence frames, then the persona tokens force the text
    row, then silence again.  Rows 9..16 of every forced frame carry the sine
    placeholder as the user stream.  Unforced rows are FREE."""
    frames = []

    def frame(text=FREE, agent=None):
        f = np.full(N_ROWS, FREE, dtype=np.int32)
        f[0] = text
        if agent is not None:
            f[1:9] = agent
        f[9:17] = sine
        return f

    for v in voice_codes:
        frames.append(frame(agent=v))
    for _ in range(SILENCE_FRAMES):
        frames.append(frame(agent=silence))
    for t in persona:
        frames.append(frame(text=int(t)))
    for _ in range(SILENCE_FRAMES):
        frames.append(frame(agent=silence))
    return np.stack(frames)


def session_open(b: int, text_card: int = 32000, card: int = 2048,
                 n_voice: int = 16, n_persona: int = 64) -> np.ndarray:
    """The session-open forced schedule of slot b (92 frames at the defaults)."""
    voice = _rng(2000 + b).integers(0, card, (n_voice, N_AGENT), dtype=np.int32)
    persona = _rng(3000 + b).integers(0, text_card, n_persona, dtype=np.int32)
    return open_schedule(voice, persona, fixed_frame(2, card), fixed_frame(5, card))


def batch_occupancy(B: int, window: int, seed: int = 4) -> np.ndarray:
    """Per-slot ring occupancy uniform in [0, window]."""
    return _rng(seed).integers(0, window + 1, B, dtype=np.int32)


def elastic_schedule(B: int, n_ticks: int, window: int, p_event: float = 0.01,
                     seed_class: int = 7, seed_event: int = 6):
    """Elastic batch: each slot holds a session; on each tick each slot's
    session leaves and a fresh one joins with probability p_event.

    Returns (sessions, events): sessions is a list of dicts {slot, start_tick,
    fill_n, fill_seed, code_seed}; events[t] lists the slots whose session is
    replaced at the start of tick t (tick 0 opens every slot).  Occupancy
    classes: 25% near-empty n~U[0,32], 50% mid n~U[1000,2000] (clipped to the
    window), 25% full n=window."""
    rc = _rng(seed_class)
    re = _rng(seed_event)
    sessions = []
    events = [[] for _ in range(n_ticks)]

    def new_session(slot, t):
        s = len(sessions)
        c = rc.random()
        if c < 0.25:
            n = int(rc.integers(0, 33))
        elif c < 0.75:
            n = int(rc.integers(1000, 2001))
        else:
            n = window
        n = min(n, window)
        sessions.append(dict(slot=slot, start_tick=t, fill_n=n,
                             fill_seed=20000 + s, code_seed=10000 + s))

    for b in range(B):
        new_session(b, 0)
        events[0].append(b)
    for t in range(1, n_ticks):
        flips = re.random(B) < p_event
        for b in np.nonzero(flips)[0]:
            new_session(int(b), t)
            events[t].append(int(b))
    return sessions, events
