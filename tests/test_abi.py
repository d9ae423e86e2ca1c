"""The C-ABI library loads, exports every entry point include/moe.h declares, and
rejects bad arguments on the host before anything is enqueued (no GPU needed: the
fake pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

B = pytest.importorskip("mixture_experts_layer_plan_amd.binding")


@pytest.fixture(scope="module")
def lib():
    try:
        return B.lib()
    except B.MoeLibraryMissing as e:
        pytest.fail(str(e))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.exported_names()) == names


def test_status_strings(lib):
    for c in range(7):
        assert B.moe_status_str(c)


FAKE = 0x10000          # 16-byte aligned, never dereferenced
BAD = 0x10004           # misaligned


def s_(**kw):
    d = dict(T=64, H=256, I=128, E=8, k=2, I_shared=0, T_minibatch=0)
    d.update(kw)
    return B.shape(**d)


def rc_route(s, logits=FAKE, idx=FAKE, w=FAKE):
    return B.lib().moe_route(ctypes.byref(s), logits, idx, w, None)


def test_shape_checks(lib):
    assert rc_route(s_(k=0)) == 2
    assert rc_route(s_(k=9)) == 2          # k > E
    assert rc_route(s_(E=0)) == 2
    assert rc_route(s_(E=1025)) == 2
    assert rc_route(s_(T=-1)) == 2
    assert rc_route(s_(H=200)) == 2
    assert rc_route(s_(T=2 ** 28, k=8)) == 2   # T*k >= 2^31


def test_null_and_alignment(lib):
    assert rc_route(s_(), logits=None) == 1
    assert rc_route(s_(), idx=BAD) == 3
    assert lib.moe_route(None, FAKE, FAKE, FAKE, None) == 1


def fwd_rc(s, ws_bytes, **over):
    a = dict(plan=FAKE, x=FAKE, w=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, sg=None, su=None, sd=None,
             y=FAKE, saved=FAKE, ws=FAKE)
    a.update(over)
    return B.lib().moe_forward_bf16(ctypes.byref(s), a["plan"], a["x"], a["w"], a["wg"], a["wu"],
                                    a["wd"], a["sg"], a["su"], a["sd"], a["y"], a["saved"], a["ws"],
                                    ws_bytes, None)


def test_forward_checks_before_enqueue(lib):
    s = s_()
    need = B.moe_workspace_bytes(s, B.MOE_BF16, False)
    assert need > 0
    assert fwd_rc(s, need - 1) == 4                       # workspace too small
    assert fwd_rc(s, need, wg=None) == 1
    assert fwd_rc(s, need, y=BAD) == 3
    assert fwd_rc(s_(I=100), need) == 2
    assert fwd_rc(s_(I_shared=128), need) == 1            # shared weights missing
    assert fwd_rc(s_(T_minibatch=32), need) == 5          # minibatching: MXFP8 path only


def test_layout_functions(lib):
    s = s_(T=300, k=4, E=16)
    L = B.moe_plan_layout_of(s)
    assert L.tile_m == 128 and L.chunk_pairs == 512
    assert L.n_chunks == (300 * 4 + 511) // 512
    assert L.max_tiles >= 300 * 4 // 128 + 16
    assert L.wtile_m == 256 and L.max_wtiles >= 300 * 4 // 256 + 16
    offs = [L.counts, L.offsets, L.src_token, L.src_slot, L.pos, L.tiles, L.n_tiles, L.err_flag,
            L.active, L.n_active, L.tile_first, L.wtiles, L.n_wtiles, L.scratch]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert B.moe_plan_bytes(s) == L.total_bytes >= L.scratch + 4 * (L.n_chunks * 16 + L.n_chunks)
    R, I, H = 1200, 128, 256
    assert B.moe_saved_bytes(s, B.MOE_BF16) >= R * 2 * I * 4
    assert B.moe_saved_bytes(s, B.MOE_F32) >= R * 2 * I * 4
    assert B.moe_workspace_bytes(s, B.MOE_BF16, True) >= R * (2 * I + I + H) * 2
    assert B.moe_plan_bytes(s_(E=0)) == 0


def test_mx_rejects_shapes_whose_offsets_overflow(lib):
    """MXFP8 calls refuse shapes whose 32-bit row offsets would overflow: one
    minibatch of T*k rows of H = 7168 bytes reaches 2^31 at T = 37450 with k = 8."""
    ok = s_(T=8192, H=7168, I=2048, E=256, k=8, T_minibatch=2048)
    assert B.moe_workspace_bytes(ok, B.MOE_MXFP8, True) > 0
    big = s_(T=37450, H=7168, I=2048, E=256, k=8, T_minibatch=0)
    assert B.moe_workspace_bytes(big, B.MOE_MXFP8, True) == 0
    assert B.moe_saved_bytes(big, B.MOE_MXFP8) == 0
    rc = B.lib().moe_forward_mxfp8(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, None, None, None,
                                   FAKE, FAKE, FAKE, 1 << 40, None)
    assert rc == 5
    # in minibatches of 8192 tokens the same T fits
    assert B.moe_workspace_bytes(s_(T=37450, H=7168, I=2048, E=256, k=8, T_minibatch=8192),
                                 B.MOE_MXFP8, True) > 0


def test_router_gemm_needs_fp32_buffers():
    from mixture_experts_layer_plan_amd import LayerBuffers
    with pytest.raises(ValueError):
        LayerBuffers(8, 256, 128, 4, 2, dtype="bf16", router_gemm=True, device="cpu")


def test_replay_flag_shrinks_saved_activations(lib):
    kept = s_(T=300, T_minibatch=128)
    rep = s_(T=300, T_minibatch=128, flags=B.MOE_REPLAY)
    R_mb, I = 128 * 2, 128
    assert B.moe_saved_bytes(kept, B.MOE_MXFP8) - B.moe_saved_bytes(rep, B.MOE_MXFP8) == \
        2 * R_mb * 2 * I * 4                    # two of three minibatches' Z not kept
    assert B.moe_workspace_bytes(rep, B.MOE_MXFP8, True) > B.moe_workspace_bytes(kept, B.MOE_MXFP8, True)
    # one minibatch: nothing to replay
    assert B.moe_saved_bytes(s_(T=300, flags=B.MOE_REPLAY), B.MOE_MXFP8) == \
        B.moe_saved_bytes(s_(T=300), B.MOE_MXFP8)
    assert B.moe_saved_bytes(s_(flags=4), B.MOE_MXFP8) == 0   # unknown flag bits
    assert rc_route(s_(flags=8)) == 2
