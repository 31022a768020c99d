"""Host-only checks of the C-ABI library (no GPU needed, no compute calls).

* every function ``include/somaopt.h`` declares is exported by libsomaopt.so;
* the planner behind ``somaopt_debug_plan`` drops frozen tensors, covers every
  trainable element exactly once per pass (owned elements only in the norm
  pass), keeps vector bodies aligned, and bounds workgroup sizes;
* descriptor validation returns SOMAOPT_E_INVALID with a message.
"""
import os
import re

import numpy as np
import pytest

from tensor_optimizer_step_amd import somaopt as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "somaopt.h")

pytestmark = pytest.mark.skipif(not os.path.exists(S.LIB_PATH),
                                reason="libsomaopt.so not built (python -m tensor_optimizer_step_amd.build)")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(somaopt_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_exported():
    lib = S.load()
    names = header_functions()
    assert len(names) >= 14
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(S.SIGNATURES), "binding signatures differ from the header"


def test_version_and_error_string():
    assert "gfx950" in S.version()
    assert isinstance(S.last_error(), str)


# ------------------------------------------------------------------ planner

BASE = 1 << 40   # fake device addresses: the planner never dereferences them


def _rows(sizes, dtypes=None, trainable=None, owner=None, misalign=None, groups=None):
    """Lay p, m, v, g of every tensor out in separate fake arenas."""
    rows, off = [], [BASE, BASE * 2, BASE * 3, BASE * 4]
    n = len(sizes)
    dtypes = dtypes or [S.F32] * n
    trainable = trainable or [1] * n
    owner = owner or [1] * n
    misalign = misalign or [(0, 0, 0, 0)] * n
    groups = groups or [0] * n
    for i, sz in enumerate(sizes):
        gsz = 2 if dtypes[i] == S.BF16 else 4
        mis = misalign[i]
        ptr = [off[0] + 4 * mis[0], off[1] + 4 * mis[1], off[2] + 4 * mis[2], off[3] + gsz * mis[3]]
        rows.append((ptr[0], ptr[3], ptr[1], ptr[2], sz, dtypes[i], groups[i], trainable[i], owner[i]))
        for k in range(3):
            off[k] += (4 * (sz + 16) + 511) // 256 * 256
        off[3] += (gsz * (sz + 16) + 511) // 256 * 256
    return rows


def _check_cover(rows, segs, pass_, chunk):
    covered = {}
    for s in segs:
        covered.setdefault(s.tensor, []).append(s)
        assert s.numel == s.head + s.nvec * s.vec_elems + s.tail
        assert s.numel <= chunk
        if s.vec_elems:
            r = rows[s.tensor]
            gsz = 2 if r[5] == S.BF16 else 4
            start = s.offset + s.head
            if pass_ == 2:
                for ptr, esz in ((r[0], 4), (r[2], 4), (r[3], 4), (r[1], gsz)):
                    assert (ptr + esz * start) % (esz * 4) == 0
            else:
                assert (r[1] + gsz * start) % 16 == 0
                assert s.vec_elems == 16 // gsz
    for i, r in enumerate(rows):
        want = r[7] == 1 and r[4] > 0 and (pass_ == 2 or r[8] == 1)
        if not want:
            assert i not in covered
            continue
        parts = sorted(covered[i], key=lambda s: s.offset)
        pos = 0
        for s in parts:
            assert s.offset == pos
            pos += s.numel
        assert pos == r[4]
    blocks = sorted({s.block for s in segs})
    assert blocks == list(range(len(blocks)))


@pytest.mark.parametrize("pass_", [1, 2])
def test_plan_covers_every_element_once(pass_):
    rng = np.random.default_rng(5)
    n = 300
    sizes = list(rng.integers(0, 20000, size=n))
    sizes[:5] = [0, 1, 3, 7, 65536 * 3 + 5]
    dt = [S.BF16 if x else S.F32 for x in rng.integers(0, 2, size=n)]
    tr = [int(x) for x in rng.random(n) > 0.3]
    ow = [int(x) for x in rng.random(n) > 0.2]
    mis = [tuple(int(x) for x in rng.integers(0, 4, size=4)) for _ in range(n)]
    mis[:50] = [(0, 0, 0, 0)] * 50
    rows = _rows(sizes, dt, tr, ow, mis)
    segs, info = S.debug_plan(rows, 1, pass_, 4096, 2048)
    chunk = 4096 if pass_ == 1 else 2048
    _check_cover(rows, segs, pass_, chunk)
    assert info.trainable_numel == sum(s for s, t in zip(sizes, tr) if t)
    assert info.owned_numel == sum(s for s, t, o in zip(sizes, tr, ow) if t and o)
    assert info.n_trainable == sum(tr)
    # workgroup cost bound
    cost = 1024   # per-segment packing cost of the planner
    per_block = {}
    for s in segs:
        per_block[s.block] = per_block.get(s.block, 0) + s.numel + cost
    assert max(per_block.values()) <= chunk + cost


def test_plan_aligned_tensors_use_vectors():
    rows = _rows([1000, 4096, 13], [S.F32, S.BF16, S.F32])
    segs, info = S.debug_plan(rows, 1, 2, 0, 4096)
    assert info.scalar_segments == 0
    assert all(s.vec_elems == 4 for s in segs)
    assert segs[0].head == 0 and segs[0].nvec == 250 and segs[0].tail == 0
    assert segs[2].nvec == 3 and segs[2].tail == 1


def test_plan_incompatible_alignment_falls_back_to_scalar():
    # p is offset by one element relative to m: no common aligned start
    rows = _rows([1000], misalign=[(1, 0, 0, 0)])
    segs, info = S.debug_plan(rows, 1, 2, 0, 0)
    assert info.scalar_segments == len(segs) >= 1
    assert sum(s.numel for s in segs) == 1000
    # a common offset is absorbed by a scalar head
    rows = _rows([1000], misalign=[(1, 1, 1, 1)])
    segs, _ = S.debug_plan(rows, 1, 2, 0, 0)
    assert segs[0].head == 3 and segs[0].vec_elems == 4


def test_plan_frozen_and_not_owned():
    rows = _rows([100, 200, 300], trainable=[1, 0, 1], owner=[1, 1, 0])
    rows[1] = (0, 0, 0, 0, 200, S.F32, 0, 0, 1)     # frozen: NULL pointers are fine
    s1, info = S.debug_plan(rows, 1, 1, 0, 0)
    assert {s.tensor for s in s1} == {0}
    s2, _ = S.debug_plan(rows, 1, 2, 0, 0)
    assert {s.tensor for s in s2} == {0, 2}
    assert info.n_trainable == 2 and info.owned_numel == 100 and info.trainable_numel == 400


def test_plan_many_small_tensors_pack_into_few_blocks():
    sizes = list(np.random.default_rng(1).integers(1, 4097, size=2000))
    rows = _rows(sizes)
    # norm pass: 1,024 elements charged per segment, budget chunk + 1,024
    segs, info = S.debug_plan(rows, 1, 1, 8192, 0)
    assert info.pass1_blocks < len(sizes) / 2
    assert info.pass1_segments == len(sizes)
    # update pass: 4,096 charged per segment -- small tensors pack in pairs at most
    # under a chunk of 8,192, and one per workgroup under the default 4,096
    segs, info = S.debug_plan(rows, 1, 2, 0, 8192)
    assert len(sizes) / 3 < info.pass2_blocks < len(sizes)
    assert info.pass2_segments == len(sizes)
    blocks = {}
    for sg in segs:
        blocks[sg.block] = blocks.get(sg.block, 0) + sg.numel + 4096
    assert max(blocks.values()) <= 8192 + 4096
    segs, info = S.debug_plan(rows, 1, 2, 0, 0)
    assert info.pass2_blocks == len(sizes)


def test_chunks_stay_within_32_bit_buffer_offsets():
    """Every pass addresses a segment's vector body through a buffer resource
    with 32-bit byte sizes and offsets: a requested chunk of 2^30 elements is
    lowered to 2^26 for the norm pass as for the update pass, so no segment's
    body reaches 2^31 bytes (at 2^30 fp32 elements it would be 2^32 bytes,
    which wraps to 0 and would silently read zeros)."""
    n = (1 << 29) + 12345
    rows = _rows([n, 1000], dtypes=[S.F32, S.BF16])
    for pass_ in (1, 2):
        segs, info = S.debug_plan(rows, 1, pass_, 1 << 30, 1 << 30)
        assert info.pass1_chunk == 1 << 26 and info.pass2_chunk == 1 << 26
        assert max(sg.numel for sg in segs) <= 1 << 26
        assert max(16 * sg.nvec for sg in segs) < 1 << 31
        # the segments still tile every element of every tensor
        covered = {}
        for sg in segs:
            covered[sg.tensor] = covered.get(sg.tensor, 0) + sg.numel
        assert covered == {0: n, 1: 1000}


def test_occupancy_follows_the_table_shape():
    """Large tensors (full-length segments) get the streaming plan: 6 norm-pass
    workgroups per CU, and update-pass segments of 2048 elements at 4 per CU;
    a table of many small tensors, whose workgroups walk several short
    segments, keeps 4096-element update segments at 4 per CU and no norm-pass
    limit.  An explicit update chunk is used as given."""
    big = _rows([1 << 20] * 4 + [1024] * 3, dtypes=[S.BF16] * 7)
    segs, info = S.debug_plan(big, 1, 2)
    assert (info.pass1_wg_per_cu, info.pass2_wg_per_cu, info.pass2_chunk) == (6, 4, 2048)
    assert max(sg.numel for sg in segs) == 2048 and info.pass2_blocks == 4 * 512 + 3
    rng = np.random.default_rng(3)
    small = _rows([int(x) for x in rng.integers(1, 4097, size=2000)])
    _, info = S.debug_plan(small, 1, 2)
    assert (info.pass1_wg_per_cu, info.pass2_wg_per_cu, info.pass2_chunk) == (0, 4, 4096)
    # half of the elements in full segments is still a streaming table
    mixed = _rows([8192 * 8] + [100] * 600)
    _, info = S.debug_plan(mixed, 1, 2)
    assert (info.pass2_wg_per_cu, info.pass2_chunk) == (4, 2048)
    # an explicit chunk is not re-planned
    _, info = S.debug_plan(big, 1, 2, 0, 4096)
    assert (info.pass2_chunk, info.pass2_blocks) == (4096, 4 * 256 + 3)


def test_update_pass_launch_split():
    """An update pass above 262144 workgroups is split into launches of equal
    size; at or below it stays one launch; an empty pass has none."""
    _, info = S.debug_plan(_rows([262144 * 2048], dtypes=[S.BF16]), 1, 2)
    assert (info.pass2_blocks, info.pass2_launches) == (262144, 1)
    _, info = S.debug_plan(_rows([262144 * 2048 + 1], dtypes=[S.BF16]), 1, 2)
    assert (info.pass2_blocks, info.pass2_launches) == (262145, 2)
    _, info = S.debug_plan(_rows([100 * 2048] * 5), 1, 2)
    assert (info.pass2_blocks, info.pass2_launches) == (500, 1)
    _, info = S.debug_plan([], 1, 2)
    assert info.pass2_launches == 0


def test_plan_empty_table():
    segs, info = S.debug_plan([], 1, 2)
    assert segs == [] and info.trainable_numel == 0


@pytest.mark.parametrize("bad,needle", [
    (dict(numel=-1), "numel"),
    (dict(group=3), "group"),
    (dict(grad_dtype=7), "dtype"),
    (dict(param=0), "NULL"),
    (dict(grad=BASE * 4 + 2, grad_dtype=0), "aligned"),
    (dict(trainable=2), "trainable"),
    (dict(owner=5), "owner"),
])
def test_validation_errors(bad, needle):
    rows = _rows([64, 64])
    r = dict(zip(["param", "grad", "exp_avg", "exp_avg_sq", "numel", "grad_dtype", "group",
                  "trainable", "owner"], rows[1]))
    r.update(bad)
    rows[1] = tuple(r.values())
    with pytest.raises(S.SomaoptError) as ei:
        S.debug_plan(rows, 2, 2)
    assert ei.value.code == S.E_INVALID
    assert needle in str(ei.value)


def test_working_copy_alignment_and_validation():
    rows = _rows([1000, 333], [S.BF16, S.F16])
    lp = BASE * 5
    # working copies aligned with p: vector path kept; misaligned by one element:
    # the head absorbs it only if all buffers agree, else scalar fallback
    r0 = rows[0] + (lp, S.BF16)
    r1 = rows[1] + (lp + 4096, S.F16)
    segs, info = S.debug_plan([r0, r1], 1, 2)
    assert info.scalar_segments == 0
    r1b = rows[1] + (lp + 4096 + 2, S.F16)
    segs, info = S.debug_plan([r0, r1b], 1, 2)
    assert info.scalar_segments == 1 and sum(s.numel for s in segs if s.tensor == 1) == 333
    with pytest.raises(S.SomaoptError, match="lowp_dtype"):
        S.debug_plan([rows[0] + (lp, S.F32)], 1, 2)
    with pytest.raises(S.SomaoptError, match="reserved"):
        S.debug_plan([rows[0] + (lp, S.BF16, 7)], 1, 2)
    with pytest.raises(S.SomaoptError, match="aligned"):
        S.debug_plan([rows[0] + (lp + 1, S.BF16)], 1, 2)
    # a working copy may not overlap any other written buffer or a gradient
    with pytest.raises(S.SomaoptError, match="overlap"):
        S.debug_plan([rows[0] + (rows[0][2], S.BF16)], 1, 2)
    with pytest.raises(S.SomaoptError, match="overlap"):
        S.debug_plan([rows[0] + (rows[0][1], S.BF16)], 1, 2)


def test_fp16_gradients_plan_like_bf16():
    rows = _rows([4096, 4097], [S.F16, S.BF16])
    s1, _ = S.debug_plan(rows, 1, 1)
    assert all(s.vec_elems == 8 for s in s1)
    assert [s.nvec for s in s1] == [512, 512] and s1[1].tail == 1


def test_validation_overlaps():
    rows = _rows([64, 64])
    # p of tensor 1 aliases m of tensor 0
    r = list(rows[1]); r[0] = rows[0][2] + 16; rows[1] = tuple(r)
    with pytest.raises(S.SomaoptError, match="overlap"):
        S.debug_plan(rows, 1, 2)
    # a gradient inside a weight buffer
    rows = _rows([64, 64])
    r = list(rows[1]); r[1] = rows[0][0]; rows[1] = tuple(r)
    with pytest.raises(S.SomaoptError, match="overlap"):
        S.debug_plan(rows, 1, 2)
    # two tensors sharing one read-only gradient are allowed
    rows = _rows([64, 64])
    r = list(rows[1]); r[1] = rows[0][1]; rows[1] = tuple(r)
    S.debug_plan(rows, 1, 2)


def test_validation_n_groups():
    with pytest.raises(S.SomaoptError):
        S.debug_plan(_rows([4]), 0, 2)
    with pytest.raises(S.SomaoptError):
        S.debug_plan(_rows([4]), S.MAX_GROUPS + 1, 2)


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    bench = os.path.join(ROOT, "bench.py")
    r = subprocess.run([sys.executable, bench, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_traffic_record_needs_same_kernel_and_split(tmp_path, monkeypatch):
    """The bench reports counted HBM traffic only from a record taken on the
    current kernel source with the same number of update launches per pass."""
    import json
    import sys
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    rec = {"kernel_sha256_16": bench.kernel_hash(), "launches_per_pass": 13, "hbm_bytes_per_pass": 12345}
    (tmp_path / "traffic_pass2_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w", 13) == 12345
    assert bench.load_traffic("w", 1) is None
    assert bench.load_traffic("missing", 13) is None
    rec["kernel_sha256_16"] = "0" * 16
    (tmp_path / "traffic_pass2_w.json").write_text(json.dumps(rec))
    assert bench.load_traffic("w", 13) is None
    # records from before the split carry one launch per pass implicitly
    old = {"kernel_sha256_16": bench.kernel_hash(), "hbm_bytes_per_launch": 777}
    (tmp_path / "traffic_pass2_old.json").write_text(json.dumps(old))
    assert bench.load_traffic("old", 1) == 777
    assert bench.load_traffic("old", 2) is None


def test_noalloc_init_refuses_tables_beyond_its_scratch():
    """The no-allocation build counts its device bytes before touching any
    device: a table that needs more than the 32 MiB scratch array is refused
    with both sizes in the message (fake, never dereferenced addresses)."""
    lib = S.load()
    rows = [(1 << 40, 2 << 40, 3 << 40, 4 << 40, 1 << 31, S.F32, 0, 1, 1)]
    descs = S.make_descs(rows)
    groups = S.make_groups([dict(lr=1e-3, weight_decay=0.0, beta1=0.9, beta2=0.999, eps=1e-8)])
    h = S.ctypes.c_void_p()
    rc = lib.somaopt_init_tensor_table_noalloc(descs, 1, groups, 1, 1.0, 1.0, 0, None, S.ctypes.byref(h))
    assert rc == S.E_INVALID and not h.value
    msg = S.last_error()
    assert "bytes of device scratch" in msg and "33554432" in msg, msg


def test_bench_cpu_baseline_runs_the_oracle_on_the_host_pool():
    """The bench's CPU baseline: the oracle's whole step (sum of squares, clip
    coefficient, update of every element) timed on a pool of host threads; the
    line reports the threads it used and what the sample was."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    from tensor_optimizer_step_amd import workloads as W
    wl = W.tiny()
    cores, model = bench.cpu_pool()
    rec = bench.cpu_baseline_workload(wl, 0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "param-elements/s"
    assert rec["cores"] == cores >= 1 and rec["value"] > 0
    assert f"first {wl.n_tensors} tensors of tiny ({wl.trainable_numel} elements)" in rec["sample"]
    assert model in rec["sample"]
