"""C-ABI checks that need no GPU: exported symbols, host-only calls (block
allocation, table validation) and argument errors that every entry point
reports before it would touch a device."""
import ctypes as C
import os

import numpy as np
import pytest

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import _abi
from oracle import paging


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_attention_17_amd import build
        build.build()
    return pkv.load()


def test_library_exports_every_header_function(lib):
    names = pkv.header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.SIGNATURES), "binding and header disagree"


def test_status_strings(lib):
    for code in range(8):
        assert pkv.pkv_status_str(code)
    assert pkv.pkv_status_str(99) == "unknown status"
    assert pkv.pkv_abi_version() >> 16 == 1


def test_workspace_and_partition_sizes(lib):
    # streaming kernel: two regions (launches chained over a step's layers
    # alternate) of two records per CU (at most 512 CUs), then the plan the
    # first chained launch stores for the others (16 + 257 x 4 + 256 x 4 +
    # 256 x 2 + 512 x 2 = 3,604 bytes, rounded up to 256)
    plan = 3840
    stream = 2 * 2 * 512 * 32 * 68 * 4 + plan
    assert pkv.pkv_decode_workspace_bytes(1, 32, 8, 64, 17, 0) == stream
    ps = pkv.pkv_decode_partition_size(64, 8, 4096)
    assert ps % 16 == 0 and ps >= 64
    P = -(-4096 // ps)
    up = lambda x: -(-x // 256) * 256  # noqa: E731

    def expect(B, nq, nkv, P):
        # the larger of: per-partition outputs + (max, sum), and the streaming records
        return max(up(B * nq * P * 64 * 4) + up(B * nq * P * 2 * 4), 2 * 2 * 512 * nq * 68 * 4 + plan)
    assert pkv.pkv_decode_workspace_bytes(64, 32, 8, 64, 4096, 0) == expect(64, 32, 8, P)
    assert pkv.pkv_decode_workspace_bytes(2, 32, 8, 64, 100, 16) == expect(2, 32, 8, 7)
    assert pkv.pkv_decode_workspace_bytes(2, 32, 8, 32, 100, 16) == 0       # unsupported head_dim


FAKE = 1 << 20          # an aligned non-null "device" address; never dereferenced on these paths


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=64, bt=FAKE, stride=4, rows=1, mb=4, sid=None, ctx=FAKE,
             batch=1, maxctx=17, nq=32, nkv=8, d=64, scale=0.125, ps=0, ws=None, wsb=0)
    a.update(kw)
    return lib.pkv_paged_attn_decode(a["out"], a["q"], a["k"], a["v"], a["nb"], a["bt"], a["stride"], a["rows"],
                                     a["mb"], a["sid"], a["ctx"], None, a["batch"], a["maxctx"], a["nq"], a["nkv"],
                                     a["d"], a["scale"], a["ps"], a["ws"], a["wsb"], None)


def test_decode_argument_errors_before_launch(lib):
    assert _decode(lib, d=128) == _abi.PKV_ERR_UNSUPPORTED
    assert _decode(lib, nq=24, nkv=8) == _abi.PKV_ERR_UNSUPPORTED        # ratio 3
    assert _decode(lib, nq=30, nkv=8) == _abi.PKV_ERR_INVALID_ARG        # not divisible
    assert _decode(lib, out=None) == _abi.PKV_ERR_NULL
    assert _decode(lib, q=FAKE + 2) == _abi.PKV_ERR_MISALIGNED
    assert _decode(lib, ctx=FAKE + 2) == _abi.PKV_ERR_MISALIGNED
    assert _decode(lib, ps=24) == _abi.PKV_ERR_INVALID_ARG               # not a multiple of 16
    assert _decode(lib, stride=2) == _abi.PKV_ERR_INVALID_ARG            # row stride shorter than the row
    assert _decode(lib, batch=-1) == _abi.PKV_ERR_INVALID_ARG
    assert _decode(lib, scale=float("nan")) == _abi.PKV_ERR_INVALID_ARG
    assert _decode(lib, scale=0.0) == _abi.PKV_ERR_INVALID_ARG
    assert _decode(lib, scale=-0.125) == _abi.PKV_ERR_INVALID_ARG
    assert _decode(lib, batch=0) == _abi.PKV_OK                          # empty batch: nothing to do
    # a context needing 2 partitions of 16 with no workspace
    assert _decode(lib, ps=16, maxctx=17) == _abi.PKV_ERR_CAPACITY
    assert _decode(lib, ps=16, maxctx=17, ws=FAKE, wsb=100) == _abi.PKV_ERR_CAPACITY


def test_other_entry_points_argument_errors(lib):
    E = _abi
    assert lib.pkv_rope_decode(FAKE, FAKE, FAKE, 4, 32, 8, 32, FAKE, 100, None) == E.PKV_ERR_UNSUPPORTED
    assert lib.pkv_rope_decode(None, FAKE, FAKE, 4, 32, 8, 64, FAKE, 100, None) == E.PKV_ERR_NULL
    assert lib.pkv_rope_decode(FAKE, FAKE, FAKE, 0, 32, 8, 64, FAKE, 100, None) == E.PKV_OK
    assert lib.pkv_rope_table_init(FAKE, 0, 64, 5e5, 32, 1, 4, 8192, None) == E.PKV_ERR_INVALID_ARG
    assert lib.pkv_rope_table_init(FAKE, 10, 64, 5e5, 32, 4, 1, 8192, None) == E.PKV_ERR_INVALID_ARG
    assert lib.pkv_paged_kv_append(FAKE, FAKE, 8, FAKE, FAKE, FAKE, 4, 1, 4, FAKE, FAKE, 3, 8, 32, None) \
        == E.PKV_ERR_UNSUPPORTED
    assert lib.pkv_paged_kv_append(FAKE, None, 8, FAKE, FAKE, FAKE, 4, 1, 4, FAKE, FAKE, 3, 8, 64, None) \
        == E.PKV_ERR_NULL
    assert lib.pkv_paged_kv_append(FAKE, FAKE + 8, 8, FAKE, FAKE, FAKE, 4, 1, 4, FAKE, FAKE, 3, 8, 64, None) \
        == E.PKV_ERR_MISALIGNED
    assert lib.pkv_paged_gather(FAKE, FAKE, FAKE, FAKE, 8, FAKE, 4, 4, 0, 65, 8, 64, None) == E.PKV_ERR_CAPACITY
    assert lib.pkv_paged_attn_prefill(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 8, FAKE, 4, 1, 4, 1, 10, 10,
                                      32, 8, 48, 0.125, None, None, None) == E.PKV_ERR_UNSUPPORTED
    assert lib.pkv_paged_attn_prefill(FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 8, FAKE, 4, 1, 4, 1, 10, 10,
                                      32, 8, 64, 0.125, None, None, None) == E.PKV_ERR_NULL
    # the masked scores are -inf: a scale of 0, below 0 or not finite would
    # turn them into NaN or +inf, so it is refused
    for bad in (0.0, -0.125, float("inf"), float("nan")):
        assert lib.pkv_paged_attn_prefill(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 8, FAKE, 4, 1, 4, 1, 10, 10,
                                          32, 8, 64, bad, None, None, None) == E.PKV_ERR_INVALID_ARG
    # fused decode: same checks plus its own inputs
    assert lib.pkv_paged_decode_fused(FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, None, 1, 17,
                                      32, 8, 64, FAKE, 100, 0.125, 0, None, 0, None) == E.PKV_ERR_NULL
    assert lib.pkv_paged_decode_fused(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, None, 1, 17,
                                      32, 8, 64, FAKE, 0, 0.125, 0, None, 0, None) == E.PKV_ERR_INVALID_ARG
    assert lib.pkv_paged_decode_fused(FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, None, 1,
                                      17, 32, 8, 64, FAKE, 100, 0.125, 0, None, 0, None) == E.PKV_ERR_MISALIGNED
    assert lib.pkv_decode_workspace_init(FAKE + 4, 64, None) == E.PKV_ERR_MISALIGNED
    assert lib.pkv_decode_workspace_init(None, 64, None) == E.PKV_ERR_NULL
    assert lib.pkv_decode_workspace_init(None, 0, None) == E.PKV_OK
    offs = np.array([0], np.int32)
    assert lib.pkv_block_table_patch(FAKE + 2, 10, offs.ctypes.data, offs.ctypes.data, 1, None) \
        == E.PKV_ERR_MISALIGNED
    assert lib.pkv_block_table_patch(FAKE, 10, offs.ctypes.data, offs.ctypes.data, 0, None) == E.PKV_OK



def test_layer_sizes_and_argument_errors(lib):
    E = _abi
    # K-split partials: splits x rows x features x 4 bytes, the most splits
    # (a power of two) that keep the workgroups (tiles x 64-row blocks x
    # splits) within 256, each split whole 128-wide slices but the last;
    # shapes that would split with K <= 4096 take the narrow-tile kernel,
    # which needs no partials
    assert pkv.pkv_linear_workspace_bytes(64, 2048, 8192) == 8 * 64 * 2048 * 4
    assert pkv.pkv_linear_workspace_bytes(64, 3072, 2048) == 0        # would split 4 ways: narrow tiles
    assert pkv.pkv_linear_workspace_bytes(1, 512, 2048) == 0          # would split 16 ways: narrow tiles
    assert pkv.pkv_linear_workspace_bytes(1, 512, 4104) == 17 * 1 * 512 * 4   # K above 4096: 256-wide ranges, 17
    assert pkv.pkv_linear_workspace_bytes(64, 16384, 2048) == 0       # 256 tiles: no split
    assert pkv.pkv_linear_workspace_bytes(65, 2048, 8192) == 4 * 65 * 2048 * 4   # two row blocks
    assert pkv.pkv_linear_workspace_bytes(64, 2048, 8008) == 8 * 64 * 2048 * 4   # last K range shorter
    assert pkv.pkv_linear_workspace_bytes(64, 100, 2048) == 0         # features % 8: not taken
    assert pkv.pkv_linear_workspace_bytes(64, 2048, 2044) == 0        # K % 8: not taken
    # layer scratch: the eight activations, then the largest partials (the
    # 2048-wide products at 8 splits, 4 MiB = 2 Mi bf16 elements)
    acts = 64 * (2048 * 2 + 2048 * 2 + 512 * 2 + 8192 * 3)
    assert pkv.pkv_decode_layer_scratch_elems(64, 2048, 8192, 32, 8) == acts + 4 * 64 * 2048 * 8 // 2
    assert pkv.pkv_decode_layer_scratch_elems(0, 2048, 8192, 32, 8) == 0
    # pkv_linear: checks before any launch
    assert lib.pkv_linear(FAKE, FAKE, FAKE, -1, 64, 128, 0, None, 0, None) == E.PKV_ERR_INVALID_ARG
    assert lib.pkv_linear(FAKE, FAKE, FAKE, 0, 64, 128, 0, None, 0, None) == E.PKV_OK
    assert lib.pkv_linear(None, FAKE, FAKE, 4, 64, 128, 0, None, 0, None) == E.PKV_ERR_NULL
    assert lib.pkv_linear(FAKE, FAKE + 8, FAKE, 4, 64, 128, 0, None, 0, None) == E.PKV_ERR_MISALIGNED
    assert lib.pkv_linear(FAKE, FAKE, FAKE, 4, 64, 128, 0, FAKE + 4, 64, None) == E.PKV_ERR_MISALIGNED
    assert lib.pkv_linear(FAKE, FAKE, FAKE, 4, 60, 128, 0, None, 0, None) == E.PKV_ERR_UNSUPPORTED
    assert lib.pkv_linear(FAKE, FAKE, FAKE, 4, 64, 100, 0, None, 0, None) == E.PKV_ERR_UNSUPPORTED
    # the layer calls: a null weight, a short scratch, the multi-layer call's own arguments
    lw = _abi.LayerWeights(*([FAKE] * 8))
    lw_null = _abi.LayerWeights(*([FAKE] * 7 + [None]))
    need = pkv.pkv_decode_layer_scratch_elems(4, 2048, 8192, 32, 8)

    def layer(w, scratch_elems, kp=FAKE, ctx=FAKE, cos=FAKE, max_pos=100, max_ctx=17, ws=FAKE, wsb=1 << 20,
              nq=32, nkv=8):
        return lib.pkv_decode_layer(FAKE, C.byref(w), 2048, 8192, FAKE, scratch_elems, kp, FAKE, 8, FAKE, 4, 4, 2,
                                    None, ctx, None, 4, max_ctx, nq, nkv, cos, max_pos, 0.125, 1e-5, ws, wsb, None)
    assert layer(lw_null, need) == E.PKV_ERR_NULL
    assert layer(lw, need - 1) == E.PKV_ERR_CAPACITY
    # the attention's own arguments, found before the layer's first launch
    assert layer(lw, need, kp=None) == E.PKV_ERR_NULL
    assert layer(lw, need, ctx=None) == E.PKV_ERR_NULL
    assert layer(lw, need, cos=None) == E.PKV_ERR_NULL
    assert layer(lw, need, max_pos=0) == E.PKV_ERR_INVALID_ARG
    assert layer(lw, need, nq=24, nkv=8) == E.PKV_ERR_UNSUPPORTED
    # contexts of up to 5,000 tokens split into partitions need partials
    assert layer(lw, need, max_ctx=5000, ws=None, wsb=0) == E.PKV_ERR_CAPACITY
    assert layer(lw, need, max_ctx=5000, wsb=1024) == E.PKV_ERR_CAPACITY

    def layers(arr, n, scratch_elems=need, bt=FAKE):
        return lib.pkv_decode_layers(FAKE, arr, n, 2048, 8192, FAKE, scratch_elems, FAKE, FAKE, 8, bt, 8, 4, 4, 2,
                                     None, FAKE, None, 4, 17, 32, 8, FAKE, 100, 0.125, 1e-5, FAKE, 1 << 20, None)
    two = (_abi.LayerWeights * 2)(lw, lw_null)
    assert layers(two, -1) == E.PKV_ERR_INVALID_ARG
    assert layers(two, 0) == E.PKV_OK
    assert layers(None, 2) == E.PKV_ERR_NULL
    assert layers(two, 2, bt=None) == E.PKV_ERR_NULL
    assert layers(two, 2) == E.PKV_ERR_NULL                   # the second layer's null weight, found before any launch
    assert layers((_abi.LayerWeights * 1)(lw), 1, scratch_elems=need - 1) == E.PKV_ERR_CAPACITY

def test_noalloc_decode_argument_errors_before_launch(lib):
    """The allocation-free decode call reports argument errors, and partials
    beyond its device array, before it touches a device (fake pointers)."""
    E = _abi

    def call(batch=4, maxctx=17, nq=32, nkv=8, d=64, out=FAKE, cos=FAKE, max_pos=100):
        return lib.pkv_paged_decode_fused_noalloc(out, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 4, 4, 2, None, FAKE,
                                                  None, batch, maxctx, nq, nkv, d, cos, max_pos, 0.125, 0, None)
    assert call(batch=0) == E.PKV_OK
    assert call(d=128) == E.PKV_ERR_UNSUPPORTED
    assert call(out=None) == E.PKV_ERR_NULL
    assert call(cos=None) == E.PKV_ERR_NULL
    assert call(max_pos=0) == E.PKV_ERR_INVALID_ARG
    # 64 rows of up to a million tokens on the per-partition kernels: the
    # partials (about 528 MB) exceed the array
    need = pkv.pkv_decode_workspace_bytes(64, 32, 8, 64, 1_000_000, 0)
    assert need > _abi.NOALLOC_SCRATCH_BYTES
    assert call(batch=64, maxctx=1_000_000) == E.PKV_ERR_CAPACITY


def test_two_half_step_host_errors_change_nothing(lib):
    """The host half of the replayed step checks everything before it
    changes anything (same rules as pkv_decode_step), and the device half
    rejects a staging area written for other sizes before any launch."""
    E = _abi
    L, slots, mb = 2, 3, 4
    assert lib.pkv_decode_step_staging_bytes(L, 0, slots) == 0
    assert lib.pkv_decode_step_staging_bytes(L, 257, 300) == 0
    nbytes = lib.pkv_decode_step_staging_bytes(L, 2, slots)
    assert nbytes % 4 == 0 and nbytes > 4 * (4 + slots + 4 + 2 * 2 * L)
    bt = np.full((slots, L, mb), -1, np.int32)
    bt[:, :, 0] = np.arange(slots * L, dtype=np.int32).reshape(slots, L)
    free = np.arange(10, 14, dtype=np.int32)
    cached = np.array([16, 5, 16], np.int32)        # slots 0 and 2 open a block per layer
    stage = np.zeros(nbytes // 4, np.int32)

    def host(sids, n_free):
        nf = C.c_int(n_free)
        sids = np.asarray(sids, np.int32)
        rc = lib.pkv_decode_step_host(L, bt.ctypes.data, slots, mb, free.ctypes.data, C.byref(nf),
                                      cached.ctypes.data, sids.ctypes.data, len(sids), stage.ctypes.data)
        return rc, nf.value

    before = (bt.copy(), cached.copy(), free.copy(), stage.copy())
    assert host([0, 0], 4) == (E.PKV_ERR_INVALID_ARG, 4)        # a slot twice
    assert host([0, 3], 4) == (E.PKV_ERR_INVALID_ARG, 4)        # no such slot
    assert host([0, 2], 3) == (E.PKV_ERR_CAPACITY, 3)           # four blocks needed, three free
    cached[1] = mb * 16
    assert host([1, 0], 4) == (E.PKV_ERR_CAPACITY, 4)           # the table row is full
    cached[1] = 5
    for a, b in zip((bt, cached, free, stage), before):
        np.testing.assert_array_equal(a, b)
    rc, nf = host([2, 0], 4)
    if rc == E.PKV_OK:                                          # a device to plan for
        assert nf == 0 and list(cached) == [17, 5, 17]
        assert stage[0] == 4 and list(stage[1:4]) == [2, L, slots]
    else:                                                       # no device: nothing changed
        assert rc == E.PKV_ERR_UNSUPPORTED and nf == 4
        for a, b in zip((bt, cached, free, stage), before):
            np.testing.assert_array_equal(a, b)
    # device half: staging written for another batch size, null and misaligned staging
    stage[1:4] = [3, L, slots]
    ptrs = (C.c_void_p * L)(FAKE, FAKE)

    def device(stage_host, stage_dev):
        return lib.pkv_decode_step_device(L, ptrs, ptrs, ptrs, ptrs, FAKE, FAKE, 64, FAKE, slots, mb, FAKE, 2, 32,
                                          8, 64, FAKE, 100, 0.125, stage_host, stage_dev, FAKE, 1 << 20, None)
    assert device(stage.ctypes.data, FAKE) == E.PKV_ERR_INVALID_ARG
    assert device(None, FAKE) == E.PKV_ERR_NULL
    assert device(stage.ctypes.data, FAKE + 4) == E.PKV_ERR_MISALIGNED


# ------------------------------------------------------- block allocation --

def test_blocks_assign_walk_is_valid_every_step(lib):
    """Drive many decode steps of ragged sequences; every step's allocation
    must satisfy the oracle's validity rules and the tables must end up
    covering exactly each sequence's tokens with distinct blocks."""
    rng = np.random.default_rng(7)
    n_slots, layers, mb, nb = 6, 3, 20, 400
    bt = np.full((n_slots, layers, mb), -1, np.int32)
    free = rng.permutation(nb).astype(np.int32)
    n_free = nb
    cached = np.zeros(n_slots, np.int32)
    for step in range(120):
        active = np.sort(rng.choice(n_slots, size=rng.integers(1, n_slots + 1), replace=False)).astype(np.int32)
        active = active[cached[active] < mb * 16]
        pos = cached[active].copy()
        for layer in range(layers):
            view = bt[:, layer, :]
            before = view.copy()
            free_before = free[:n_free].copy()
            n_free, off, val = pkv.pkv_blocks_assign(view, free, n_free, active, pos)
            assert paging.allocation_problems(before, view, free_before, free[:n_free], active, pos) == []
            # the patch list replays the change
            replay = before.ravel().copy()
            flat_stride = view.strides[0] // 4
            for o, v in zip(off, val):
                s, j = divmod(int(o), flat_stride)
                replay[s * mb + j] = v
            np.testing.assert_array_equal(replay.reshape(view.shape), view)
        cached[active] += 1
    used = bt[bt >= 0]
    assert len(np.unique(used)) == len(used)
    for s in range(n_slots):
        for layer in range(layers):
            nblk = -(-int(cached[s]) // 16)
            assert (bt[s, layer, :nblk] >= 0).all() and (bt[s, layer, nblk:] == -1).all()
    st, _, _ = pkv.pkv_check_block_table(np.ascontiguousarray(bt[:, 0, :]), None, cached, nb)
    assert st == 0


def test_blocks_assign_is_all_or_nothing(lib):
    bt = np.full((3, 4), -1, np.int32)
    free = np.array([9, 8], np.int32)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.pkv_blocks_assign(bt, free, 2, np.array([0, 1, 2], np.int32), np.array([0, 0, 0], np.int32))
    assert e.value.status == _abi.PKV_ERR_CAPACITY
    assert (bt == -1).all() and list(free) == [9, 8]
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.pkv_blocks_assign(bt, free, 2, np.array([0], np.int32), np.array([64], np.int32))   # past the row
    assert e.value.status == _abi.PKV_ERR_CAPACITY
    # two tokens of one chunk (a prefill chunk) take one block
    n_free, off, val = pkv.pkv_blocks_assign(bt, free, 2, np.array([1, 1], np.int32), np.array([3, 4], np.int32))
    assert n_free == 1 and list(val) == [8] and bt[1, 0] == 8


def test_blocks_release_returns_blocks(lib):
    bt = np.full((2, 5), -1, np.int32)
    bt[1, :3] = [4, 7, 1]
    free = np.zeros(10, np.int32)
    free[:2] = [0, 2]
    n_free, off, val = pkv.pkv_blocks_release(bt, 1, free, 2)
    assert n_free == 5 and sorted(free[:5]) == [0, 1, 2, 4, 7]
    assert (bt == -1).all() and list(val) == [-1, -1, -1] and list(off) == [5, 6, 7]


def test_check_block_table_reports_first_problem(lib):
    bt = np.array([[3, 5, -1, -1], [0, 1, 2, -1], [7, -1, -1, -1]], np.int32)
    ctx = np.array([20, 40, 16], np.int32)
    assert pkv.pkv_check_block_table(bt, None, ctx, 8)[0] == 0
    assert pkv.pkv_check_block_table(bt, None, np.array([33, 40, 16], np.int32), 8) == (5, 0, 2)   # -1 inside
    assert pkv.pkv_check_block_table(bt, None, ctx, 7) == (5, 2, 0)                                # id >= NB
    bt2 = bt.copy()
    bt2[2, 0] = 5
    assert pkv.pkv_check_block_table(bt2, None, ctx, 8) == (5, 2, 0)                               # shared
    assert pkv.pkv_check_block_table(bt, None, np.array([20, 80, 16], np.int32), 8) == (5, 1, -1)  # too long
    assert pkv.pkv_check_block_table(bt, np.array([2, 9], np.int32), ctx, 8) == (5, 1, -2)         # bad slot
    assert pkv.pkv_check_block_table(bt, np.array([1, 1, 0], np.int32), ctx, 8)[0] == 0            # repeat ok
    # a strided [slots][layers][max_blocks] view, layer 1
    bt3 = np.full((3, 2, 4), -1, np.int32)
    bt3[:, 1, :] = bt
    assert pkv.pkv_check_block_table(bt3[:, 1, :], None, ctx, 8)[0] == 0


def test_paged_read_probe_argument_errors(lib):
    E = _abi
    lens = np.array([17, 40], np.int32)

    def call(k=FAKE, sink=FAKE, d=64, batch=2, rl=lens.ctypes.data, stride=4, sid=None):
        return lib.pkv_paged_read_probe(k, FAKE, 64, FAKE, stride, 2, 4, sid, rl, batch, 8, d, sink, None)
    assert call(batch=0) == E.PKV_OK
    assert call(d=128) == E.PKV_ERR_UNSUPPORTED
    assert call(k=None) == E.PKV_ERR_NULL
    assert call(rl=None) == E.PKV_ERR_NULL
    assert call(sink=FAKE + 2) == E.PKV_ERR_MISALIGNED
    assert call(stride=3) == E.PKV_ERR_INVALID_ARG
    assert call(batch=3) == E.PKV_ERR_INVALID_ARG      # more rows than the table without slot ids


def test_device_errors_argument_errors(lib):
    assert lib.pkv_device_errors(None, 0, None) == _abi.PKV_ERR_NULL


def test_read_probe_argument_errors(lib):
    E = _abi
    assert lib.pkv_hbm_read_probe(None, 0, None, None) == E.PKV_OK
    assert lib.pkv_hbm_read_probe(None, 64, FAKE, None) == E.PKV_ERR_NULL
    assert lib.pkv_hbm_read_probe(FAKE, 64, None, None) == E.PKV_ERR_NULL
    assert lib.pkv_hbm_read_probe(FAKE + 4, 64, FAKE, None) == E.PKV_ERR_MISALIGNED
    assert lib.pkv_hbm_read_probe(FAKE, 60, FAKE, None) == E.PKV_ERR_MISALIGNED
    # the weight-stream probe: shape rules before pointers, nothing launched
    assert lib.pkv_weight_read_probe(FAKE, 0, 2048, 1, FAKE, None) == E.PKV_ERR_INVALID_ARG
    assert lib.pkv_weight_read_probe(FAKE, 64, 2048, 3, FAKE, None) == E.PKV_ERR_INVALID_ARG
    assert lib.pkv_weight_read_probe(FAKE, 24, 2048, 1, FAKE, None) == E.PKV_ERR_UNSUPPORTED    # n % 16
    assert lib.pkv_weight_read_probe(FAKE, 64, 384, 2, FAKE, None) == E.PKV_ERR_UNSUPPORTED     # k % 256
    assert lib.pkv_weight_read_probe(None, 64, 2048, 1, FAKE, None) == E.PKV_ERR_NULL
    assert lib.pkv_weight_read_probe(FAKE, 64, 2048, 1, None, None) == E.PKV_ERR_NULL
    assert lib.pkv_weight_read_probe(FAKE + 4, 64, 2048, 1, FAKE, None) == E.PKV_ERR_MISALIGNED


def test_load_shares_torch_hip_runtime():
    """Loaded before anything imports torch, the library must still end up on
    the HIP runtime torch brings (one libamdhip64 in the process): with two,
    torch's streams and allocations are foreign to this library's kernels."""
    import subprocess
    import sys
    code = (
        "import sys, paged_kv_attention_17_amd as p\n"
        "assert 'torch' not in sys.modules\n"
        "p.load()\n"
        "import torch\n"
        "maps = open('/proc/self/maps').read().split('\\n')\n"
        "libs = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
        "print(libs)\n"
        "assert len(libs) == 1, libs\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_kv_read_policy_setting(lib):
    """The K/V read policy: STREAM by default, REUSE settable, anything else
    refused with nothing changed."""
    E = _abi
    assert lib.pkv_kv_read_policy() == E.PKV_KV_READ_STREAM
    try:
        assert lib.pkv_set_kv_read_policy(E.PKV_KV_READ_REUSE) == E.PKV_OK
        assert lib.pkv_kv_read_policy() == E.PKV_KV_READ_REUSE
        for bad in (0, 3, -1):
            assert lib.pkv_set_kv_read_policy(bad) == E.PKV_ERR_INVALID_ARG
            assert lib.pkv_kv_read_policy() == E.PKV_KV_READ_REUSE
    finally:
        assert lib.pkv_set_kv_read_policy(E.PKV_KV_READ_STREAM) == E.PKV_OK
    assert lib.pkv_kv_read_policy() == E.PKV_KV_READ_STREAM
