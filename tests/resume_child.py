"""Child process for the signal-driven resume test (not collected by pytest).

usage: resume_child.py DIR WORKLOAD N TOTAL_STEPS USR1_AT TERM_AT [sync|async [EVERY STALL_AT]]

Resumes from the newest step file in DIR (or starts fresh), then runs updates
until TOTAL_STEPS. It sends itself SIGUSR1 after update USR1_AT and SIGTERM
after update TERM_AT (0 = never), the way an operator or a supervising proxy
would; the checkpointer writes step files on both and exits on SIGTERM, and
every EVERY updates (0 = only on signals). After update STALL_AT (0 = never)
it finishes its device work and any write in flight, prints "stalled", and
waits on the host to be killed (the parent's stand-in for a crash).
Prints one line per event so the parent can follow what happened.
"""
import os
import signal
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import resumable_checkpoint_state_amd as rcs  # noqa: E402
import workloads  # noqa: E402


def main():
    d, name, n, total, usr1_at, term_at = sys.argv[1], sys.argv[2], *map(int, sys.argv[3:7])
    async_write = len(sys.argv) > 7 and sys.argv[7] == "async"
    every = int(sys.argv[8]) if len(sys.argv) > 8 else 0
    stall_at = int(sys.argv[9]) if len(sys.argv) > 9 else 0
    wl = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.init_params(wl, device=dev, n=n)
    m, v = workloads.zeros_like_state(n, device=dev)
    ck = rcs.StepFileCheckpointer(d, n, every=every, keep=3, async_write=async_write)
    start = ck.resume(w, m, v)
    print(f"child: resumed at step {start}", flush=True)
    g = torch.empty(n, device=dev)
    for t in range(start + 1, total + 1):
        workloads.grads(wl, t, device=dev, n=n, out=g)
        rcs.adamw_clip_step(w, g, m, v, t, wl.lr, wl.wd, wl.clip)
        if t == usr1_at:
            os.kill(os.getpid(), signal.SIGUSR1)
        if t == term_at:
            os.kill(os.getpid(), signal.SIGTERM)
        if ck.after_step(t, w, m, v):
            print(f"child: SIGTERM after step {t}, wrote {ck.written[-1]}", flush=True)
            return 0
        if t == stall_at:
            torch.cuda.synchronize()
            ck.flush()
            print(f"child: stalled after step {t}", flush=True)
            time.sleep(600)
            return 1
    ck.save(total, w, m, v, wait=True)
    print(f"child: finished {total}, wrote {ck.written[-1]}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
