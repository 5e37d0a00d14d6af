"""CPU model of the forward scan's split-sequence hand-off (race detection
for the one place where workgroups communicate).

tests/split_model/handoff_model.cpp re-implements the protocol with
std::thread workers in place of workgroups: chunk tickets from 8 per-XCD
queues (each chunk-major over a contiguous range of channel groups; a worker
takes from its own XCD's queue, else from the next ones), a relaxed flag
load with an acquire fence after the
wait, a release fence before the flag store, the bounded wait that sets the
error word and poisons the chunk with NaN when it gives up, random delays at
every step, and fewer workers than chunks (a workgroup takes new work only
after finishing its chunk, as on a device shared with other work). The
program checks every chunk's inclusive state bit for bit against the
sequential composition."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "split_model", "handoff_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("handoff") / "handoff_model")
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-pthread", "-Wall", "-Werror", SRC, "-o", exe])
    return exe


def run(model, order, nbg, nchunks, workers, seed, spin, lost=-1):
    res = subprocess.run([model, order, str(nbg), str(nchunks), str(workers), str(seed), str(spin), str(lost)],
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert res.returncode == 0, res.stdout
    fields = dict(kv.split("=") for kv in res.stdout.split()[1:])
    return {k: (int(v) if v.lstrip("-").isdigit() else v) for k, v in fields.items()}


# Ticket order: every chunk is taken once and every wait ends, with any
# number of workers (down to one, i.e. no two chunks ever resident together),
# under random delays, and also when every worker reports the same XCD (the
# other queues are then reached only by the fallback).
@pytest.mark.parametrize("order", ["ticket", "skew"])
@pytest.mark.parametrize("workers", [1, 2, 5, 16, 64])
@pytest.mark.parametrize("nbg,nchunks", [(16, 6), (8, 24), (3, 7), (128, 6), (20, 5)])
def test_ticket_order_never_gives_up(model, order, workers, nbg, nchunks):
    for seed in range(3):
        r = run(model, order, nbg, nchunks, workers, seed, 10 ** 9)
        assert r["gave_up"] == 0 and r["err"] == 0 and r["nan_chunks"] == 0
        assert r["waits"] == nbg * (nchunks - 1)


# The fixed block order of a launch without tickets depends on every
# workgroup being resident: with one worker a chunk waits for a predecessor
# that nobody is running, and only the bounded wait ends it.
def test_fixed_block_order_needs_every_block_resident(model):
    r = run(model, "static", 16, 6, 1, 0, 2000)
    assert r["gave_up"] > 0 and r["err"] == 1 and r["nan_chunks"] > 0


# A lost chunk (never hands its state on): the waits after it give up, the
# error word is set, and exactly the later chunks of that group are NaN
# (checked inside the model); nothing hangs.
@pytest.mark.parametrize("lost", [0, 2, 4])
def test_lost_chunk_poisons_only_the_later_chunks(model, lost):
    nbg, nchunks = 8, 6
    r = run(model, "ticket", nbg, nchunks, 8, lost, 20000, lost=lost)
    assert r["err"] == 1
    assert r["nan_chunks"] == nbg * (nchunks - 1 - lost)
