"""The C-ABI library loads without a GPU, exports every declared entry point,
and rejects bad configurations on the host before any launch."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "replayssm.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(replay_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def B():
    from hybrid_model_ssm_replay_amd import binding
    binding.load_library()
    return binding


def test_every_declared_symbol_is_exported_and_bound(B):
    lib = B.load_library()
    names = _declared()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
        assert n in B.EXPORTS, n


def test_struct_sizes_match(B):
    import ctypes
    lib = B.load_library()
    for i, st in enumerate((B.replay_config, B.replay_buffers, B.replay_record, B.replay_ctx, B.replay_ring_view)):
        assert lib.replay_abi_sizeof(i) == ctypes.sizeof(st)


@pytest.mark.parametrize("args", [
    (0, 0, 4, 1, 16, 16, 4),       # batch 0
    (0, 2, 4, 3, 16, 16, 4),       # heads not a multiple of groups
    (0, 2, 4, 1, 20, 16, 4),       # head_dim not a multiple of 16
    (0, 2, 4, 1, 16, 24, 4),       # unsupported state_dim
    (0, 2, 4, 1, 16, 16, 0),       # window 0
    (0, 2, 4, 1, 16, 16, 17),      # window above 16
    (1, 2, 4, 2, 16, 16, 4),       # GDN with groups != heads
    (2, 2, 4, 4, 16, 16, 4),       # unknown kind
])
def test_bad_configs_rejected(B, args):
    cfg = B.make_config(*args)
    assert B.replay_validate_config(cfg) == B.EINVAL
    assert B.replay_ckpt_bytes(cfg) == 0 and B.replay_ring_bytes(cfg) == 0


def test_draft_bound(B):
    assert B.replay_validate_config(B.make_config(0, 2, 4, 1, 16, 16, 4, max_draft=5)) == B.EINVAL
    assert B.replay_validate_config(B.make_config(0, 2, 4, 1, 16, 16, 4, max_draft=4)) == B.OK


def test_sizes(B):
    cfg = B.make_config(0, 256, 128, 8, 64, 128, 16, 8)
    assert B.replay_ckpt_bytes(cfg) == 256 * 128 * 64 * 128 * 4
    assert B.replay_pointer_words(cfg) == 4 * 256
    ring = 256 * 128 * 16 * 64 * 4 + 256 * 8 * 32 * 128 * 4 + 256 * 128 * 16 * 4
    assert B.replay_ring_bytes(cfg) == ring


def test_sizes_bf16_records(B):
    """bf16 records halve the ring's record vector fields (Mamba-2 x, B; GDN k and,
    with a separate read copy, v); scalars, pseudo-values and the state do not change."""
    cfg = B.make_config(0, 256, 128, 8, 64, 128, 16, 8, flags=B.FLAG_BF16_RECORDS)
    assert B.replay_validate_config(cfg) == B.OK
    assert B.replay_ckpt_bytes(cfg) == 256 * 128 * 64 * 128 * 4
    assert B.replay_ring_bytes(cfg) == 256 * 128 * 16 * 64 * 2 + 256 * 8 * 32 * 128 * 2 + 256 * 128 * 16 * 4
    g = B.make_config(1, 64, 32, 32, 128, 128, 16, 4, B.FMT_F32, B.FMT_F4E2M1_B16, flags=B.FLAG_BF16_RECORDS)
    k, u, sc, v = 64 * 32 * 16 * 128 * 2, 64 * 32 * 16 * 128 * 4, 64 * 32 * 16 * 4, 64 * 32 * 16 * 128 * 2
    assert B.replay_ring_bytes(g) == k + u + 2 * sc + v


def test_sizes_records_in_ring(B):
    """The zero-copy ring has 2L slots per field (the Mamba-2 B field has 2L anyway)."""
    cfg = B.make_config(0, 256, 128, 8, 64, 128, 16, 8, flags=B.FLAG_RECORDS_IN_RING)
    assert B.replay_ring_bytes(cfg) == 256 * 128 * 32 * 64 * 4 + 256 * 8 * 32 * 128 * 4 + 256 * 128 * 32 * 4
    g = B.make_config(1, 4, 2, 2, 64, 32, 8, 8, flags=B.FLAG_RECORDS_IN_RING)
    k, u, sc = 4 * 2 * 16 * 32 * 4, 4 * 2 * 16 * 64 * 4, 4 * 2 * 16 * 4
    a256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    assert B.replay_ring_bytes(g) == a256(k) + a256(u) + 2 * a256(sc)


def test_unknown_flag_rejected(B):
    assert B.replay_validate_config(B.make_config(0, 2, 4, 1, 16, 16, 4, flags=0x8)) == B.EINVAL


def test_calls_reject_uninitialised_context(B):
    ctx = B.replay_ctx()
    rec = B.make_record(16, 16, 16, 16)
    with pytest.raises(B.ReplayError):
        B.replay_step(ctx, rec, 16, 0)
    with pytest.raises(B.ReplayError):
        B.replay_commit(ctx, 16, 0)
    with pytest.raises(B.ReplayError):
        B.replay_hbm_probe(16, 16, 15, 0, 0)


def test_low_precision_format_pairs(B):
    """Format pairs: split precision (F32 / FP16-SR / e4m3 checkpoint with an e2m1
    read copy) and one shared low-precision copy, for both families at
    state_dim 128; the two-axis read copy for GDN only; the decay skip and
    zero-copy append stay float32-only for Mamba-2, and the decay skip is
    float32-only for both families."""
    F = (B.FMT_F32, B.FMT_F16_SR, B.FMT_F8E4M3, B.FMT_F4E2M1_B16)
    split = [(c, B.FMT_F4E2M1_B16) for c in F[:3]] + [(c, c) for c in F[1:]]
    for cf, rf in split:
        assert B.replay_validate_config(B.make_config(0, 2, 8, 2, 64, 128, 16, 4, cf, rf)) == B.OK
        assert B.replay_validate_config(B.make_config(1, 2, 8, 8, 128, 128, 16, 4, cf, rf)) == B.OK
    assert B.replay_validate_config(B.make_config(1, 2, 8, 8, 128, 128, 16, 4, B.FMT_F32, B.FMT_F4E2M1_CS)) == B.OK
    ns = B.ENOTSUP
    assert B.replay_validate_config(B.make_config(0, 2, 8, 2, 64, 128, 16, 4, B.FMT_F32, B.FMT_F4E2M1_CS)) == ns
    assert B.replay_validate_config(B.make_config(0, 2, 8, 2, 64, 64, 16, 4, B.FMT_F32, B.FMT_F4E2M1_B16)) == ns
    assert B.replay_validate_config(B.make_config(0, 2, 8, 2, 32, 128, 16, 4, B.FMT_F32, B.FMT_F4E2M1_B16)) == ns
    assert B.replay_validate_config(B.make_config(1, 2, 8, 8, 128, 128, 16, 4, flags=B.FLAG_DECAY_SKIP)) == B.OK
    assert B.replay_validate_config(B.make_config(1, 2, 8, 8, 128, 128, 16, 4, B.FMT_F32, B.FMT_F4E2M1_B16,
                                                  flags=B.FLAG_DECAY_SKIP)) == ns
    for fl in (B.FLAG_DECAY_SKIP, B.FLAG_RECORDS_IN_RING):
        assert B.replay_validate_config(B.make_config(0, 2, 8, 2, 64, 128, 16, 4, B.FMT_F32, B.FMT_F4E2M1_B16,
                                                      flags=fl)) == ns
    assert B.replay_validate_config(B.make_config(0, 2, 8, 2, 64, 128, 16, 4, B.FMT_F32, B.FMT_F16_SR)) == ns
    # sizes: e2m1 codes then, at the next 256 bytes, one e4m3 scale per 16 elements
    cfg = B.make_config(0, 256, 128, 8, 64, 128, 16, 4, B.FMT_F32, B.FMT_F4E2M1_B16)
    n = 256 * 128 * 64 * 128
    assert B.replay_ckpt_bytes(cfg) == 4 * n
    assert B.replay_read_copy_bytes(cfg) == (n // 2 + 255) // 256 * 256 + n // 16
