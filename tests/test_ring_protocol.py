"""Host-side model of the bf16 state pass's LDS ring (kda_state_pass_ring32).

The kernel's loader and compute wavefronts meet at one workgroup barrier per
step; correctness rests on three counting facts that the GPU tests cannot
show directly (a violation would be a race, seen only now and then):

  * both roles execute the same number of barriers for every T;
  * the compute wave reads pair n from its slot only after the barrier that
    follows the loader's write of pair n, and the loader does not write the
    slot again before the compute wave's read of pair n is behind a barrier;
  * each loader keeps at most 63 vector loads in flight at a commit (the
    wait counter's range);
  * the V wavefront (four slices per workgroup) runs the loaders' loop, so
    the loaders' counts hold for it;
  * with the output wavefront (one slice per workgroup, dk = 128), it reads
    each pair's slot in the same step as the compute wave, and the compute
    wave's operands for it, left in an exchange buffer by step parity, only
    after the barrier that ends their write and before they are rewritten.

The constants are read from the kernel source, so a change to the slot or
loader count is checked here as well. The model follows the kernel's loops
step by step: epochs are the intervals between consecutive barriers."""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "linear_attention_recurrence_11_amd", "csrc",
                   "kda_chunk.hip")


def ring_constants(dk, spw=1):
    text = open(SRC).read()
    geom = text[text.index("struct Ring32Geom"):]
    geom = geom[:geom.index("};")]
    rec = re.search(r"kRec = DK == 128 \? (\d+) : (\d+);", geom)
    k_rec = int(rec.group(1) if dk == 128 else rec.group(2))
    k_slots = int(re.search(r"kSlots = (\d+);", geom).group(1))
    k_loaders = int(re.search(r"kLoaders = (\d+);", geom).group(1))
    max_stages = int(re.search(r"kStagesRaw > (\d+) \? \d+ : kStagesRaw", geom).group(1))
    # the V loader adds two loads per slice of the workgroup (SPW slices)
    per_slice = int(re.search(r"kStagesRaw = 1 \+ 63 / \(kUnitsPer \+ (\d+) \* SPW\)", geom).group(1))
    v_loads = per_slice * spw
    v_pitch = int(re.search(r"kVPitch = (\d+);", geom).group(1))
    units = k_rec // 1024
    per = (units + k_loaders - 1) // k_loaders
    stages = min(max_stages, 1 + 63 // (per + v_loads))
    return dict(slots=k_slots, loaders=k_loaders, units=units, per=per, stages=stages,
                v_loads=v_loads, slot_bytes=k_rec + spw * 2 * 16 * v_pitch)


def simulate(T, slots, stages):
    """Replay both roles' loops for a sequence of T tokens. Returns the loader's
    and the compute wave's barrier counts and, per pair, the epoch of its
    write and of its read, and the epoch of the next write to the same slot."""
    kR, kS = slots, stages
    NPR = (T + 31) // 32
    NPS = (NPR + kS - 1) // kS * kS
    writes = {}        # pair -> epoch of its commit to LDS
    slot_writes = {}   # slot -> list of (epoch, pair)
    issued = set()

    # loader: prologue (epoch 0), then one commit + issue per step
    epoch = 0
    for c in range(kS):
        issued.add(c)
    for c in range(kR - 1):
        assert c in issued
        writes.setdefault(c, epoch)
        slot_writes.setdefault(c % kR, []).append((epoch, c))
        issued.add(c + kS)
    loader_barriers = 1
    epoch = 1
    for n in range(0, NPS, kS):
        for k in range(kS):
            c = n + k + kR - 1
            assert c in issued, "commit of a pair whose loads were never issued"
            writes.setdefault(c, epoch)
            slot_writes.setdefault(c % kR, []).append((epoch, c))
            issued.add(c + kS)
            loader_barriers += 1
            epoch += 1

    # compute: barrier 0, one read per step, then padding barriers
    reads = {}
    compute_barriers = 1
    epoch = 1
    for n in range(NPR):
        reads[n] = epoch
        compute_barriers += 1
        epoch += 1
    compute_barriers += NPS - NPR
    return loader_barriers, compute_barriers, writes, reads, slot_writes, NPR


SPWS = [1, 2, 4]   # slices per workgroup the launcher instantiates


@pytest.mark.parametrize("spw", SPWS)
@pytest.mark.parametrize("dk", [128, 64])
def test_constants_fit_the_wait_counter_and_lds(dk, spw):
    c = ring_constants(dk, spw)
    # the loader that also loads V keeps per + v_loads loads per pair in flight
    assert (c["stages"] - 1) * (c["per"] + c["v_loads"]) <= 63
    assert c["per"] * c["loaders"] >= c["units"]
    assert c["slots"] * c["slot_bytes"] <= 160 * 1024
    assert c["slots"] >= 2 and c["stages"] >= 1


@pytest.mark.parametrize("spw", SPWS)
@pytest.mark.parametrize("dk", [128, 64])
def test_barriers_match_and_slots_never_race(dk, spw):
    # every compute wavefront of the workgroup runs the compute loop, so the
    # counts below hold for each of them
    c = ring_constants(dk, spw)
    for T in list(range(1, 700)) + [1023, 1024, 1025, 4095, 4096, 4097, 65536, 65537]:
        lb, cb, writes, reads, slot_writes, NPR = simulate(T, c["slots"], c["stages"])
        assert lb == cb, "barrier counts differ at T=%d" % T
        for n in range(NPR):
            assert n in writes, "pair %d read but never written (T=%d)" % (n, T)
            # the write epoch ends at a barrier no later than the read's start
            assert writes[n] + 1 <= reads[n], "pair %d read before its write completed" % n
            # the next write into the same slot starts after the read's barrier
            later = [e for e, p in slot_writes[n % c["slots"]] if p > n]
            if later:
                assert min(later) >= reads[n] + 1, "slot of pair %d rewritten during its read" % n


@pytest.mark.parametrize("slots", [3, 4, 5])
def test_protocol_holds_for_other_ring_sizes(slots):
    # the sweep's other sizes: the same invariants (the stage count is that of dk = 128)
    stages = ring_constants(128)["stages"]
    for T in range(1, 400):
        lb, cb, writes, reads, slot_writes, NPR = simulate(T, slots, stages)
        assert lb == cb
        for n in range(NPR):
            assert writes[n] + 1 <= reads[n]
            later = [e for e, p in slot_writes[n % slots] if p > n]
            if later:
                assert min(later) >= reads[n] + 1


def test_a_one_slot_ring_would_race():
    # the check has teeth: with a single slot the loader writes each pair in
    # the same epoch as the compute wave reads it, and the model reports it
    stages = ring_constants(128)["stages"]
    with pytest.raises(AssertionError):
        for T in range(33, 200):
            lb, cb, writes, reads, slot_writes, NPR = simulate(T, 1, stages)
            for n in range(NPR):
                assert writes[n] + 1 <= reads[n]
                later = [e for e, p in slot_writes[n % 1] if p > n]
                if later:
                    assert min(later) >= reads[n] + 1


def test_launcher_instantiates_the_modelled_slice_counts():
    text = open(SRC).read()
    launch = text[text.index("switch (choose_slices_per_wg("):]
    launch = launch[:launch.index("}")]
    found = sorted(int(x) for x in re.findall(r"launch_ring32_pair<OutT, DK, (\d+), MODE>", launch))
    assert found == SPWS


def split_constants():
    text = open(SRC).read()
    x = text[text.index("struct Ring32Split"):]
    x = x[:x.index("};")]
    on = re.search(r"kOn = DK == (\d+) && SPW == (\d+) && MODE == kPassOutputs && !SCALED;", x)
    nbuf = int(re.search(r"kXStage = kOn \? (\d+) \* kXPair : 0;", x).group(1))
    per = re.search(r"kXPair = \(DK / (\d+) \+ (\d+)\) \* 1024;", x)
    dk = int(on.group(1))
    return dict(dk=dk, spw=int(on.group(2)), buffers=nbuf,
                pair_bytes=(dk // int(per.group(1)) + int(per.group(2))) * 1024)


def simulate_output_wave(T, slots, stages, buffers):
    """The output wavefront's loop beside the compute wave's: returns its
    barrier count, the epoch of its read of each pair's slot, and per pair
    the epochs of the exchange buffer's write (compute wave) and read."""
    kS = stages
    NPR = (T + 31) // 32
    NPS = (NPR + kS - 1) // kS * kS
    slot_reads, x_reads = {}, {}
    x_writes = {}                       # buffer -> list of (epoch, pair)
    for n in range(NPR):                # the compute wave writes pair n in step n
        x_writes.setdefault(n % buffers, []).append((n + 1, n))
    barriers = 1
    epoch = 1
    for n in range(NPR + 1):
        if n < NPR:
            slot_reads[n] = epoch
        if n > 0:
            x_reads[n - 1] = epoch
        if n < NPR:
            barriers += 1
            epoch += 1
    barriers += NPS - NPR
    return barriers, slot_reads, x_reads, x_writes, NPR


def _check_output_wave(T, c, buffers):
    lb, cb, writes, reads, slot_writes, NPR = simulate(T, c["slots"], c["stages"])
    ob, slot_reads, x_reads, x_writes, _ = simulate_output_wave(T, c["slots"], c["stages"], buffers)
    assert ob == lb, "output wavefront barrier count differs at T=%d" % T
    for n in range(NPR):
        assert slot_reads[n] == reads[n], "output wavefront reads pair %d in another step" % n
        wr = [e for e, p in x_writes[n % buffers] if p == n][0]
        assert wr + 1 <= x_reads[n], "operands of pair %d read before their write completed" % n
        later = [e for e, p in x_writes[n % buffers] if p > n]
        if later:
            assert min(later) >= x_reads[n] + 1, "exchange buffer of pair %d rewritten during its read" % n


def test_output_wavefront_barriers_and_exchange_never_race():
    x = split_constants()
    c = ring_constants(x["dk"], x["spw"])
    assert c["slots"] * c["slot_bytes"] + x["buffers"] * x["pair_bytes"] <= 160 * 1024
    for T in list(range(1, 700)) + [1023, 1024, 1025, 4095, 4096, 4097, 65536, 65537]:
        _check_output_wave(T, c, x["buffers"])


def test_a_single_exchange_buffer_would_race():
    c = ring_constants(128, 1)
    with pytest.raises(AssertionError):
        for T in range(65, 200):
            _check_output_wave(T, c, 1)


SKELETON = re.compile(r"for \(int c = 0; c < kS; \+\+c\) issue\(|for \(int c = 0; c < kR - 1; \+\+c\) \{|"
                      r"commit\(st\[c % kS\], c\);|issue\(st\[c % kS\], c \+ kS\);|ring_barrier\(\);|"
                      r"for \(int64_t n = 0; n < NPS; n \+= kS\) \{|for \(int k = 0; k < kS; \+\+k\) \{|"
                      r"const int64_t c = n \+ k \+ kR - 1;|commit\(st\[\(k \+ kR - 1\) % kS\], c\);|"
                      r"issue\(st\[\(k \+ kR - 1\) % kS\], c \+ kS\);|return;")


def _block(text, marker):
    i = text.index(marker)
    j = text.index("return;", i)
    return text[i:j + len("return;")]


def test_v_wavefront_runs_the_loaders_loop():
    # the barrier and slot facts above are modelled on the loaders' loop; the
    # V wavefront must step through the same prologue, commits, issues and
    # barriers in the same order
    text = open(SRC).read()
    loaders = SKELETON.findall(_block(text, "// ---------------- loaders ----------------"))
    vwave = SKELETON.findall(_block(text, "// ---------------- V (four slices per workgroup) ----------------"))
    assert loaders.count("ring_barrier();") == 2 and loaders == vwave
