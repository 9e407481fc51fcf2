"""Write the stored greedy-decode results of the oracle at the full workload sizes.

TEST INFRASTRUCTURE.  This script calls only the oracle and the seeded input
generator; nothing in it comes from the GPU library.  Its output files under
``tests/golden/`` are what the full-workload GPU parity test compares with.

Workloads (the generation loop of the "run.c" page at temperature 0, and the
generation loop of "run.c 逐行解讀" §7 with the prompt forced):

* ``llama7b``     -- the Llama-2-7B-shaped model: token 1 at position 0, then
  2048 greedy steps (positions 0..2047), each step's argmax fed back.
* ``llama70b_8l`` -- eight layers of Llama-2-70B shape: the KV cache is filled
  by 3584 forward steps over seeded uniform tokens (positions 0..3583), then
  the argmax of the last of them starts 512 greedy steps (positions 3584..4095).

For every step p the file keeps the input token, the oracle's argmax, its eight
largest logits with their indices (descending, ties to the lower index) and
max |logit|; the full logit vector is kept at sixteen positions.  A step is a
tie event when the top-2 gap is at most 1e-4 * max |logit| (the parity bar of
one step), since there two correct implementations may pick different tokens.

The run takes hours of CPU time, so it keeps a resumable checkpoint (KV cache
rows and the records so far) in a scratch directory.  Matrix rows and attention
heads may be shared out among threads (``--threads``): every output is the same
sequential sum whatever the count, so the stored values do not depend on it.

    python -m oracle.make_goldens --config llama7b --threads 7 --scratch /tmp/goldens
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

TOPK = 8
REL_TOL = 1e-4
GOLDEN_DIR = os.path.join(_ROOT, "tests", "golden")

WORKLOADS = {
    # name: (number of forced prompt steps, total steps, positions whose full logits are stored)
    "llama7b": (0, 2048, (0, 1, 2, 15, 16, 127, 128, 255, 511, 512, 1023, 1024, 1535, 2000, 2046, 2047)),
    "llama70b_8l": (3584, 4096, (0, 1, 511, 1024, 2047, 2048, 3072, 3583, 3584, 3585, 3600, 3840, 4000, 4094,
                                 4095, 2500)),
}


def source_digest() -> dict:
    """sha256 of every source file the stored values depend on."""
    files = ["oracle/oracle.c", "oracle/oracle.h", "synth/synth.c", "synth/__init__.py"]
    out = {}
    for f in files:
        with open(os.path.join(_ROOT, f), "rb") as fh:
            out[f] = hashlib.sha256(fh.read()).hexdigest()
    return out


def golden_path(name: str) -> str:
    return os.path.join(GOLDEN_DIR, f"greedy_{name}.npz")


def top_k(logits: np.ndarray, k: int = TOPK):
    """Indices and values of the k largest logits, descending, equal values by lower index."""
    order = np.lexsort((np.arange(logits.size), -logits.astype(np.float64)))[:k]
    return order.astype(np.int32), logits[order].astype(np.float32)


def run(name: str, threads: int, scratch: str, checkpoint_every: int = 256) -> str:
    cfg = synth.CONFIGS[name]
    n_forced, n_steps, keep = WORKLOADS[name]
    keep = tuple(sorted(keep))
    digest = source_digest()
    oracle.set_threads(threads)
    t0 = time.time()
    blob = synth.make_blob(cfg)
    print(f"[{name}] blob {blob.nbytes / 1e9:.2f} GB in {time.time() - t0:.1f} s", flush=True)
    prompt = synth.prefill_tokens(cfg, n_forced) if n_forced else np.zeros(0, np.int32)

    tok_in = np.zeros(n_steps, np.int32)
    nxt = np.zeros(n_steps, np.int32)
    top_idx = np.zeros((n_steps, TOPK), np.int32)
    top_val = np.zeros((n_steps, TOPK), np.float32)
    maxabs = np.zeros(n_steps, np.float32)
    kept = np.zeros((len(keep), cfg.vocab_size), np.float32)
    cache = oracle.KVCache(cfg)
    start, elapsed = 0, 0.0

    os.makedirs(scratch, exist_ok=True)
    ck_meta = os.path.join(scratch, f"{name}_ckpt.json")
    ck_data = os.path.join(scratch, f"{name}_ckpt.npz")
    if os.path.exists(ck_meta) and os.path.exists(ck_data):
        meta = json.load(open(ck_meta))
        if meta.get("digest") == digest:
            start, elapsed = int(meta["next_step"]), float(meta["elapsed_s"])
            with np.load(ck_data, allow_pickle=False) as z:
                for arr, key in ((tok_in, "tok_in"), (nxt, "next"), (top_idx, "top_idx"), (top_val, "top_val"),
                                 (maxabs, "maxabs"), (kept, "kept")):
                    arr[...] = z[key]
                cache.k[:, :start] = z["k"]
                cache.v[:, :start] = z["v"]
            print(f"[{name}] resumed at step {start} ({elapsed:.0f} s already spent)", flush=True)
        else:
            print(f"[{name}] checkpoint is from other sources; starting over", flush=True)

    def save_checkpoint(next_step: int, spent: float) -> None:
        tmp = ck_data + ".tmp.npz"
        np.savez(tmp, tok_in=tok_in, next=nxt, top_idx=top_idx, top_val=top_val, maxabs=maxabs, kept=kept,
                 k=cache.k[:, :next_step], v=cache.v[:, :next_step])
        os.replace(tmp, ck_data)
        with open(ck_meta + ".tmp", "w") as fh:
            json.dump({"digest": digest, "next_step": next_step, "elapsed_s": spent}, fh)
        os.replace(ck_meta + ".tmp", ck_meta)

    t_run = time.time() - elapsed
    for p in range(start, n_steps):
        if p == 0:
            tok = int(prompt[0]) if n_forced else 1
        elif p < n_forced:
            tok = int(prompt[p])
        else:
            tok = int(nxt[p - 1])
        tok_in[p] = tok
        logits = oracle.forward(cfg, blob, cache, tok, p)
        nxt[p] = oracle.argmax(logits)
        top_idx[p], top_val[p] = top_k(logits)
        maxabs[p] = np.max(np.abs(logits))
        if p in keep:
            kept[keep.index(p)] = logits
        done = p + 1
        if done % 16 == 0 or done == n_steps:
            rate = (time.time() - t_run) / done
            print(f"[{name}] step {done}/{n_steps}  {rate:.2f} s/step  eta {rate * (n_steps - done) / 60:.0f} min",
                  flush=True)
        if done % checkpoint_every == 0 and done < n_steps:
            save_checkpoint(done, time.time() - t_run)

    gap = top_val[:, 0].astype(np.float64) - top_val[:, 1]
    tie = gap <= REL_TOL * maxabs.astype(np.float64)
    ties = np.flatnonzero(tie)
    meta = {
        "workload": name,
        "config": {f: getattr(cfg, f) for f in ("dim", "hidden_dim", "n_layers", "n_heads", "n_kv_heads",
                                                "vocab_size", "seq_len", "shared_classifier", "seed",
                                                "norm_eps", "rope_theta")},
        "forced_steps": n_forced,
        "steps": n_steps,
        "start_token": 1 if not n_forced else None,
        "tie_rule": "top-2 gap <= 1e-4 * max|logit| of the step",
        "tie_steps": [int(t) for t in ties],
        "first_tie_step": int(ties[0]) if ties.size else None,
        # the first decision a free-running generation depends on is the argmax of the last forced step
        "first_greedy_tie_step": next((int(t) for t in ties if t >= max(n_forced - 1, 0)), None),
        "sources_sha256": digest,
        "oracle_threads": threads,
        "oracle_seconds": round(time.time() - t_run, 1),
        "host": platform.processor() or platform.machine(),
        "written_by": "oracle/make_goldens.py",
    }
    os.makedirs(GOLDEN_DIR, exist_ok=True)
    out = golden_path(name)
    tmp = out + ".tmp.npz"
    np.savez(tmp, tok_in=tok_in, next=nxt, top_idx=top_idx, top_val=top_val, maxabs=maxabs,
             logit_pos=np.asarray(keep, np.int32), logits=kept, meta=np.array(json.dumps(meta)))
    os.replace(tmp, out)
    print(f"[{name}] wrote {out}: {n_steps} steps, tie steps {meta['tie_steps']}, "
          f"{meta['oracle_seconds']:.0f} s", flush=True)
    for f in (ck_meta, ck_data):
        if os.path.exists(f):
            os.remove(f)
    return out


def load(name: str):
    """The stored run as a dict of arrays plus ``meta`` (a dict)."""
    with np.load(golden_path(name), allow_pickle=False) as z:
        d = {k: z[k] for k in z.files}
    d["meta"] = json.loads(str(d["meta"]))
    return d


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--config", choices=sorted(WORKLOADS), action="append", required=True)
    ap.add_argument("--threads", type=int, default=1)
    ap.add_argument("--scratch", default=os.path.join("/tmp", "ld_goldens"))
    a = ap.parse_args()
    for name in a.config:
        run(name, a.threads, a.scratch)


if __name__ == "__main__":
    main()
