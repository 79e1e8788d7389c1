"""The forward pass's work split, checked on the host (no GPU): every launch the plan
can make keeps its buffer-descriptor spans and 32-bit byte offsets in range, and
shapes beyond those limits are refused with SSCAN_ERR_UNSUPPORTED.

The kernels read x and delta and write y through raw buffer descriptors whose record
count is at most 2^31 - 1 bytes and whose offsets are 32-bit.  The segment kernels
walk one segment's token rows through one descriptor and prefetch up to 2 * 8 rows
past its end; the lockstep kernel walks a run and prefetches up to one chunk
(16 waves x 16 tokens) plus 8 rows ahead of a run start."""
import pytest

MAX_DESC = 2**31 - 1
MAX_ITEMS = 2**32 - 1
PREFETCH_ROWS = 16        # segment kernels: 2 * the 8-token prefetch group
LOCK_REACH_ROWS = 256 + 8  # lockstep: a chunk plus one prefetch group


@pytest.fixture(scope="module")
def sscan():
    from tests.test_abi import _build_module
    hb = _build_module()
    import os
    if not os.path.exists(hb.LIB):
        hb.build()
    import selective_state_space_77_amd as s
    return s


SHAPES = [
    # (batch, seqlen, dim, N, io)
    (1, 256, 16, 4, "f32"),              # tiny
    (8, 2048, 1536, 16, "f32"),          # 130M width
    (4, 8192, 4096, 16, "bf16"),         # 1.4B width (benchmarked)
    (1, 2**20, 2048, 16, "bf16"),        # 2^20 tokens
    (1, 2**20, 12160, 16, "f32"),        # 190 tiles: segment path with ~2.3 GB segments unbounded
    (1, 2**21, 12160, 16, "bf16"),
    (1, 65536, 65536, 16, "f32"),        # 1024 tiles, 256 KiB token rows
    (1, 65536, 65536, 16, "bf16"),
    (1, 2**27, 64, 16, "bf16"),          # one tile, 2^27 tokens
    (3, 10**6, 1000, 5, "f32"),
    (1, 1, 2**22, 16, "f32"),            # lockstep rejected by its row reach: segment path
    (1, 100, 2**24, 1, "bf16"),
    (2**16, 1, 4096, 16, "bf16"),        # 2^22 tiles: lockstep launch too wide -> segment path
    (256, 1000, 64, 16, "f32"),
    (1, 7, 100000, 2, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}_L{}_d{}_N{}_{}".format(*s))
def test_plan_keeps_every_offset_in_range(sscan, shape):
    batch, L, dim, N, io = shape
    es = 2 if io == "bf16" else 4
    rowb = dim * es
    p = sscan.forward_plan(batch, L, dim, N, io)
    tiles = batch * ((dim + 63) // 64)
    assert p["tiles"] == tiles
    # the segments cover the sequence exactly
    S, sl = p["segments"], p["seg_len"]
    assert S >= 1 and sl >= 1
    assert (S - 1) * sl < L <= S * sl
    nt = 1 if N <= 1 else 2 if N <= 2 else 4 if N <= 4 else 8 if N <= 8 else 16
    staged = batch * L * 2 * nt * 4  # B/(n+1) and C rows, fp32
    if p["kernel"] == "lockstep":
        # one workgroup per tile walks the whole sequence chunk by chunk
        assert S == 1 and sl == L
        assert tiles >= 192
        assert p["chunk_tokens"] == 256
        assert LOCK_REACH_ROWS * rowb <= MAX_DESC
        assert tiles * 1024 <= MAX_ITEMS
        assert L < 2**31
        # no segment aggregates on this path: staged rows + tile flags only
        assert staged <= p["scratch_bytes"] <= staged + 4 * tiles + 512
    else:
        assert p["kernel"] == "segment"
        assert p["chunk_tokens"] == 0
        # a segment's rows fit one descriptor and no prefetched offset wraps past 2^32
        assert sl * rowb <= MAX_DESC
        assert (sl + PREFETCH_ROWS) * rowb < 2**32
        assert S * tiles * 64 <= MAX_ITEMS
        assert p["scratch_bytes"] >= staged + S * batch * dim * (1 + nt) * 4


def test_named_workloads_take_the_expected_kernels(sscan):
    assert sscan.forward_plan(4, 8192, 4096, 16, "bf16")["kernel"] == "lockstep"
    assert sscan.forward_plan(8, 2048, 1536, 16, "f32")["kernel"] == "lockstep"
    long1m = sscan.forward_plan(1, 2**20, 2048, 16, "bf16")
    assert long1m["kernel"] == "segment" and long1m["tiles"] == 32


def test_forced_segment_counts(sscan, monkeypatch):
    """SSCAN_FORCE_SEGMENTS=n takes the segment path with n segments (at most one per
    token, at least what the descriptor bound needs); unset or 0, the plan is automatic."""
    for n in (1, 7, 33, 300):
        monkeypatch.setenv("SSCAN_FORCE_SEGMENTS", str(n))
        p = sscan.forward_plan(3, 3000, 4096, 16, "f32")
        assert p["kernel"] == "segment" and p["segments"] == n, (n, p)
        assert (p["segments"] - 1) * p["seg_len"] < 3000 <= p["segments"] * p["seg_len"]
    monkeypatch.setenv("SSCAN_FORCE_SEGMENTS", "5000")
    assert sscan.forward_plan(1, 100, 64, 16, "f32")["segments"] == 100   # one per token at most
    monkeypatch.setenv("SSCAN_FORCE_SEGMENTS", "1")
    p = sscan.forward_plan(1, 2**20, 12160, 16, "f32")                    # the descriptor bound wins
    assert p["segments"] >= 23 and p["seg_len"] * 12160 * 4 <= MAX_DESC
    monkeypatch.setenv("SSCAN_FORCE_SEGMENTS", "0")
    assert sscan.forward_plan(4, 8192, 4096, 16, "bf16")["kernel"] == "lockstep"


def test_the_previously_unbounded_segment_shapes_are_now_split_finer(sscan):
    # 190 tiles: ~22 segments by occupancy alone, which would give 2.3 GB segments
    p = sscan.forward_plan(1, 2**20, 12160, 16, "f32")
    assert p["kernel"] == "segment"
    assert p["seg_len"] * 12160 * 4 <= MAX_DESC
    assert p["segments"] >= 23


@pytest.mark.parametrize("dim,io", [(2**25, "f32"), (2**26, "bf16"), (2**27, "f32")])
def test_rows_too_wide_for_32_bit_offsets_are_refused(sscan, dim, io):
    with pytest.raises(sscan.SScanError) as e:
        sscan.forward_plan(1, 4, dim, 16, io)
    assert e.value.status == -3
    assert "dim too large" in str(e.value)


def test_forward_refuses_the_same_shape_before_touching_memory(sscan):
    # fake, never-dereferenced addresses: the refusal comes from planning
    lib = sscan.lib
    n = 1 << 30
    rc = lib.sscan_forward(0x1000, 0x1000 + n, 0x3000, 0x4000, 0x5000, None, 0x1000 + 4 * n, None,
                           1, 1, 2**25, 1, 0, None)
    assert rc == -3


def test_plan_argument_errors(sscan):
    with pytest.raises(sscan.SScanError):
        sscan.forward_plan(1, 4, 8, 17, "f32")
    with pytest.raises(sscan.SScanError):
        sscan.forward_plan(-1, 4, 8, 4, "f32")
    assert sscan.lib.sscan_forward_plan(1, 4, 8, 4, 0, None) == -1
