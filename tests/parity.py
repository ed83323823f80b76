"""Comparison helpers for GPU-vs-oracle parity (tests only).

Acceptance: hidden states per layer within rel-L2 1e-2; logits within 5e-2
absolute; greedy tokens identical wherever the oracle's top-2 margin exceeds
1e-2, under teacher-forced streams.  Depformer steps 8..15 (fed the engine's
own user-stream predictions) are compared only up to the first step where a
low-margin prediction legitimately differs."""
import numpy as np

HIDDEN_REL_L2 = 1e-2
LOGIT_ABS = 5e-2
MARGIN = 1e-2


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def margin(logits):
    top2 = np.partition(np.asarray(logits, np.float64), -2)[-2:]
    return float(top2[1] - top2[0])


def oracle_run(oracle, codes, slot=0):
    """Free-running oracle ticks for one slot of a B=1 oracle; returns a list
    of per-tick records (tokens + taps)."""
    recs = []
    for t in range(len(codes)):
        tok = oracle.step(codes[t:t + 1])
        tp = oracle.taps
        recs.append(dict(tokens=tok[slot].copy(), hidden=tp["hidden"][:, slot].copy(),
                         text_logits=tp["text_logits"][slot].copy(), dep_logits=tp["dep_logits"][slot].copy(),
                         chosen=tp["chosen"][slot].copy(), user_pred=tp["user_pred"][slot].copy()))
    return recs


def teacher_frames(recs, codes, schedule=None):
    """Forced frames that replay the oracle's choices: rows 0-8 = the oracle's
    chosen tokens, rows 9-16 = the user codes (or the schedule's rows where a
    schedule frame forces them)."""
    f = np.zeros((len(recs), 17), np.int32)
    for t, r in enumerate(recs):
        f[t, 0:9] = r["chosen"]
        f[t, 9:17] = codes[t] if schedule is None or t >= len(schedule) else schedule[t, 9:17]
    return f


def compare_tick(gpu, ref, t, report, tokens=True):
    """Compare one tick's GPU taps (dict for one slot) with the oracle's
    record; appends stats to report; returns a list of failure strings.
    tokens=False: hidden states and logits only."""
    fails = []
    L1 = ref["hidden"].shape[0]
    worst = 0.0
    for j in range(L1):
        e = rel_l2(gpu["hidden"][j], ref["hidden"][j])
        worst = max(worst, e)
        if e > HIDDEN_REL_L2:
            fails.append(f"tick {t} hidden[{j}] rel-L2 {e:.3e}")
    report.setdefault("hidden_rel_l2", []).append(worst)
    # each layer's own contribution (attention + MLP added to the residual),
    # so that error in a small update cannot hide behind the residual stream
    contrib = max(rel_l2(gpu["hidden"][j + 1] - gpu["hidden"][j], ref["hidden"][j + 1] - ref["hidden"][j])
                  for j in range(L1 - 1))
    report.setdefault("contrib_rel_l2", []).append(contrib)
    d = float(np.abs(gpu["text_logits"] - ref["text_logits"]).max())
    report.setdefault("text_logit_abs", []).append(d)
    if d > LOGIT_ABS:
        fails.append(f"tick {t} text logits max abs {d:.3e}")
    if tokens and margin(ref["text_logits"]) > MARGIN:
        report["tok_checked"] = report.get("tok_checked", 0) + 1
        if gpu["tokens"][0] != ref["tokens"][0]:
            fails.append(f"tick {t} text token {gpu['tokens'][0]} != {ref['tokens'][0]}")
    dl = 0.0
    for k in range(ref["dep_logits"].shape[0]):
        dk = float(np.abs(gpu["dep_logits"][k] - ref["dep_logits"][k]).max())
        dl = max(dl, dk)
        if dk > LOGIT_ABS:
            fails.append(f"tick {t} dep logits step {k} max abs {dk:.3e}")
        g_pred = gpu["tokens"][1 + k] if k < 8 else gpu["user_pred"][k - 8]
        r_pred = ref["tokens"][1 + k] if k < 8 else ref["user_pred"][k - 8]
        if tokens and margin(ref["dep_logits"][k]) > MARGIN:
            report["tok_checked"] = report.get("tok_checked", 0) + 1
            if g_pred != r_pred:
                fails.append(f"tick {t} dep step {k} token {g_pred} != {r_pred}")
        elif g_pred != r_pred and k >= 8:
            break   # later steps are fed this step's (unforced) prediction: inputs differ from here on
    report.setdefault("dep_logit_abs", []).append(dl)
    return fails


def gpu_slot(taps, b):
    return dict(hidden=taps["hidden"][:, b], text_logits=taps["text_logits"][b],
                dep_logits=taps["dep_logits"][b], tokens=taps["tokens"][b],
                user_pred=taps["user_pred"][b], chosen=taps["chosen"][b])
