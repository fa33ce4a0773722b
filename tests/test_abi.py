"""libdiffattn C ABI on the CPU: the library loads, exports every declared symbol,
and rejects invalid arguments on the host before any HIP call is made."""
import ctypes
import os
import re

import pytest

from differential_attention_v2_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from differential_attention_v2_amd import build_lib
        build_lib.build()
    return bd.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"diffattn_prefill_fwd", "diffattn_decode_fwd", "diffattn_decode_workspace_bytes",
            "diffattn_decode_num_splits", "diffattn_v1_lambda", "diffattn_status_string",
            "diffattn_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in bd._SIGNATURES, f"binding lacks {n}"


def test_version_and_status_strings(lib):
    assert bd.diffattn_version() == 100
    for st in range(5):
        assert bd.status_string(st)
    assert bd.status_string(99) == "unknown status"


# a fake, 256-byte aligned "device" address: never dereferenced, every call
# below fails validation on another argument first
P = 0x7F0000000000


def _prefill(**kw):
    a = dict(q=P, k=P, v=P, lam=P, out=P, B=1, T=16, Hq=8, Hkv=2, d=128, causal=1, dtype=0, flags=0,
             rms_eps=1e-5, stream=None)
    a.update(kw)
    return bd.diffattn_prefill_fwd(**a)


def _decode(**kw):
    a = dict(q=P, k_cache=P, v_cache=P, lam=P, out=P, B=2, L=100, Hq=8, Hkv=2, d=128, dtype=0, flags=0,
             rms_eps=1e-5, num_splits=0, workspace=None, workspace_bytes=0, stream=None)
    a.update(kw)
    return bd.diffattn_decode_fwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(out=None), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(lam=None), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(k=P + 8), bd.DIFFATTN_ERR_INVALID_ARG),          # not 16-byte aligned
    (dict(lam=P + 2), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(B=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(T=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(T=-5), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=2), bd.DIFFATTN_ERR_INVALID_ARG),      # Hq not a multiple of 2*Hkv
    (dict(Hq=8, Hkv=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(d=96), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(d=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(Hq=36, Hkv=2), bd.DIFFATTN_ERR_UNSUPPORTED),     # G = 9 pairs per KV head
    (dict(dtype=7), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(flags=0x4), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(flags=1, rms_eps=0.0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(flags=1, rms_eps=float("nan")), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(B=1 << 20, T=1 << 20), bd.DIFFATTN_ERR_INVALID_ARG),   # element count overflow
])
def test_prefill_rejects(lib, kw, status):
    assert _prefill(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(v_cache=P + 4), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(L=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(num_splits=-1), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(d=32), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(Hq=10, Hkv=2), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(flags=1, rms_eps=-1.0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(workspace=None, workspace_bytes=1 << 30), bd.DIFFATTN_ERR_WORKSPACE),
    (dict(workspace=P, workspace_bytes=16), bd.DIFFATTN_ERR_WORKSPACE),
    (dict(workspace=P + 8, workspace_bytes=1 << 30), bd.DIFFATTN_ERR_WORKSPACE),
])
def test_decode_rejects(lib, kw, status):
    assert _decode(**kw) == status


def test_v1_lambda_rejects(lib):
    assert bd.diffattn_v1_lambda(None, P, P, P, 0.8, P, 4, 128, 1, None) == bd.DIFFATTN_ERR_INVALID_ARG
    assert bd.diffattn_v1_lambda(P, P, P, P, 0.8, P, 0, 128, 1, None) == bd.DIFFATTN_ERR_INVALID_ARG
    assert bd.diffattn_v1_lambda(P, P, P, P, float("inf"), P, 4, 128, 1, None) == bd.DIFFATTN_ERR_INVALID_ARG


def test_decode_split_plan(lib):
    # B*Hkv (b, KV head) units are split so that ~512 waves (two per CU) stream the cache
    assert bd.diffattn_decode_num_splits(64, 8192, 64, 8, 128) == 1
    assert bd.diffattn_decode_num_splits(8, 131072, 64, 8, 128) == 8
    assert bd.diffattn_decode_num_splits(16, 8192, 64, 8, 128) == 4
    assert bd.diffattn_decode_num_splits(512, 1000, 64, 8, 128) == 1
    assert bd.diffattn_decode_num_splits(1, 1, 2, 1, 64) == 1
    assert bd.diffattn_decode_num_splits(1, 100, 2, 1, 64) == 4       # ceil(100/32) ranges of 32
    assert bd.diffattn_decode_num_splits(1, 100, 3, 1, 64) == 0       # invalid heads
    rec = 128 + 4
    assert bd.diffattn_decode_workspace_bytes(64, 8192, 64, 8, 128, 0) == 64 * 64 * 1 * rec * 4
    assert bd.diffattn_decode_workspace_bytes(8, 131072, 64, 8, 128, 0) == 8 * 64 * 8 * rec * 4
    assert bd.diffattn_decode_workspace_bytes(64, 8192, 64, 8, 128, 8) == 64 * 64 * 8 * rec * 4
    # explicit split counts are clamped to the number of 32-key blocks and never leave a range empty
    assert bd.diffattn_decode_workspace_bytes(1, 100, 2, 1, 64, 1000) == 1 * 2 * 4 * (64 + 4) * 4
    assert bd.diffattn_decode_workspace_bytes(1, 100, 2, 1, 64, 3) == 1 * 2 * 2 * (64 + 4) * 4   # chunk 64 -> 2
    assert bd.diffattn_decode_workspace_bytes(0, 100, 2, 1, 64, 0) == 0


def test_binding_refuses_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(bd, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        bd.load_library(str(tmp_path / "nope.so"))


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "differential_attention_v2_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), f
                assert "diffattn_oracle" not in text, f


def _train(**kw):
    a = dict(q=P, k=P, v=P, lam=P, out=P, o2=P, lse=P, B=1, T=16, Hq=8, Hkv=2, d=128, causal=1, stream=None)
    a.update(kw)
    return bd.diffattn_prefill_fwd_train(**a)


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, lam=P, out=P, o2=P, lse=P, dout=P, dq=P, dk=P, dv=P, dlam=P, B=1, T=16, Hq=8, Hkv=2,
             d=128, causal=1, workspace=P, workspace_bytes=1 << 20, stream=None)
    a.update(kw)
    return bd.diffattn_prefill_bwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(o2=None), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(lse=None), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(o2=P + 8), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(lse=P + 2), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(T=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(d=96), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=2), bd.DIFFATTN_ERR_INVALID_ARG),
])
def test_train_forward_rejects(lib, kw, status):
    assert _train(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dout=None), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(dq=P + 8), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(dlam=None), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(lse=P + 1), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(B=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(d=32), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(Hq=36, Hkv=2), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(workspace=None), bd.DIFFATTN_ERR_WORKSPACE),
    (dict(workspace_bytes=1024), bd.DIFFATTN_ERR_WORKSPACE),
    (dict(workspace=P + 4), bd.DIFFATTN_ERR_WORKSPACE),
])
def test_backward_rejects(lib, kw, status):
    assert _bwd(**kw) == status


def test_backward_workspace_bytes(lib):
    # per-pair row statistics [B][P][5][T rounded up to 32] + fp32 dK and dV accumulators
    assert bd.diffattn_prefill_bwd_workspace_bytes(1, 4096, 64, 8, 128) == (32 * 5 * 4096 + 2 * 4096 * 8 * 128) * 4
    assert bd.diffattn_prefill_bwd_workspace_bytes(2, 100, 8, 2, 64) == (2 * 4 * 5 * 128 + 2 * 2 * 100 * 2 * 64) * 4
    assert bd.diffattn_prefill_bwd_workspace_bytes(1, 100, 6, 2, 64) == 0
    assert bd.diffattn_prefill_bwd_workspace_bytes(0, 100, 8, 2, 64) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(H=30, Hkv=8), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(H=136, Hkv=8), bd.DIFFATTN_ERR_UNSUPPORTED),     # 17 heads per KV head
    (dict(d=96), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(L=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(out=P + 8), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(workspace_bytes=64), bd.DIFFATTN_ERR_WORKSPACE),
])
def test_compare_decodes_reject(lib, kw, status):
    a = dict(q=P, k_cache=P, v_cache=P, out=P, B=2, L=100, H=32, Hkv=8, d=128, num_splits=0, workspace=P,
             workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    assert bd.diffattn_decode_standard(**a) == status
    a2 = dict(a, lam=P, flags=0, rms_eps=1e-5)
    assert bd.diffattn_decode_v1_layout(**a2) == status


def test_v1_layout_needs_lambda(lib):
    assert bd.diffattn_decode_v1_layout(P, P, P, None, P, 2, 100, 32, 8, 128, 0, 1e-5, 0, P, 1 << 30,
                                        None) == bd.DIFFATTN_ERR_INVALID_ARG


def test_compare_workspace_bytes(lib):
    # two record arrays (one per V1 branch) of [B, H, S, d + 4] fp32, S from the decode plan
    S = bd.diffattn_decode_num_splits(64, 8192, 64, 8, 128)
    assert bd.diffattn_decode_compare_workspace_bytes(64, 8192, 32, 8, 128, 0) == 2 * 64 * 32 * S * 132 * 4
    assert bd.diffattn_decode_compare_workspace_bytes(2, 100, 30, 8, 128, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=1000), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(P=24), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(P=80), bd.DIFFATTN_ERR_UNSUPPORTED),
    (dict(rows=0), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(x=P + 8), bd.DIFFATTN_ERR_INVALID_ARG),
    (dict(lambda_out=None), bd.DIFFATTN_ERR_INVALID_ARG),
])
def test_lambda_proj_rejects(lib, kw, status):
    a = dict(x=P, w_lambda=P, lambda_out=P, rows=16, d_model=4096, P=32, stream=None)
    a.update(kw)
    assert bd.diffattn_lambda_proj(**a) == status


def test_output_proj_rejects(lib):
    assert bd.diffattn_output_proj(P, P, P, 16, 48, 64, None) == bd.DIFFATTN_ERR_UNSUPPORTED   # k steps of 32
    assert bd.diffattn_output_proj(P, P, P, 16, 64, 60, None) == bd.DIFFATTN_ERR_UNSUPPORTED   # 16-byte columns
    assert bd.diffattn_output_proj(P, P, None, 16, 64, 64, None) == bd.DIFFATTN_ERR_INVALID_ARG
    assert bd.diffattn_output_proj(P, P + 2, P, 16, 64, 64, None) == bd.DIFFATTN_ERR_INVALID_ARG
    assert bd.diffattn_output_proj(P, P, P, 0, 64, 64, None) == bd.DIFFATTN_ERR_INVALID_ARG


def test_varlen_workspace_bytes(lib):
    # max of the per-(b, KV head) split records and the even-split records + plan
    split = 64 * 64 * 1 * 132 * 4                   # S = 1 key range per (b, KV head)
    flat = 64 * (64 + 64) * 132 * 4 + (64 + 2) * 4  # 512 / 8 = 64 ranges per KV head
    assert bd.diffattn_decode_varlen_workspace_bytes(64, 8192, 64, 8, 128, 0) == max(split, flat)
    assert bd.diffattn_decode_varlen_workspace_bytes(64, 8192, 62, 8, 128, 0) == 0


# Tile rows are addressed with 32-bit per-lane byte offsets from a 64-bit base:
# head counts whose 64-token stride would pass 2^31 bytes are refused on the host.
@pytest.mark.parametrize("Hq,Hkv,d", [(65536, 32768, 128), (131072, 65536, 64), (1 << 20, 1 << 17, 128)])
def test_wide_token_rows_rejected(lib, Hq, Hkv, d):
    assert _prefill(B=1, T=1, Hq=Hq, Hkv=Hkv, d=d) == bd.DIFFATTN_ERR_UNSUPPORTED
    assert _decode(B=1, L=1, Hq=Hq, Hkv=Hkv, d=d) == bd.DIFFATTN_ERR_UNSUPPORTED
    assert _train(B=1, T=1, Hq=Hq, Hkv=Hkv, d=d) == bd.DIFFATTN_ERR_UNSUPPORTED
    assert _bwd(B=1, T=1, Hq=Hq, Hkv=Hkv, d=d) == bd.DIFFATTN_ERR_UNSUPPORTED
    assert bd.diffattn_decode_workspace_bytes(1, 1, Hq, Hkv, d, 0) == 0
    assert bd.diffattn_decode_standard(P, P, P, P, 1, 1, Hq, Hq // 8, d, 0, P, 1 << 30,
                                       None) == bd.DIFFATTN_ERR_UNSUPPORTED


def test_widest_supported_token_row_passes_validation(lib):
    # Hq*d = 2^22 is the largest accepted width: the call gets past the head check
    # and fails on the missing workspace instead (nothing is launched)
    assert _decode(B=1, L=1, Hq=32768, Hkv=4096, d=128) == bd.DIFFATTN_ERR_WORKSPACE


def test_backward_sequence_limit(lib):
    assert _bwd(B=1, T=(1 << 26) + 1, Hq=2, Hkv=1, d=64) == bd.DIFFATTN_ERR_UNSUPPORTED


def test_lambda_proj_model_dim_limit(lib):
    assert bd.diffattn_lambda_proj(P, P, P, 16, (1 << 24) + 512, 32, None) == bd.DIFFATTN_ERR_UNSUPPORTED


def test_noalloc_decode_validation(lib):
    """The decode entry point without a workspace validates on the host like the
    workspace one and refuses problems whose records exceed its fixed array."""
    text = open(HEADER).read()
    m = re.search(r"#define DIFFATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == bd.DIFFATTN_NOALLOC_SCRATCH_BYTES

    def call(**kw):
        a = dict(q=P, k_cache=P, v_cache=P, lam=P, out=P, B=2, L=100, Hq=8, Hkv=2, d=128, dtype=0, flags=0,
                 rms_eps=1e-5, num_splits=0, stream=None)
        a.update(kw)
        return bd.diffattn_decode_fwd_noalloc(**a)

    assert call(B=0) == bd.DIFFATTN_ERR_INVALID_ARG
    assert call(q=None) == bd.DIFFATTN_ERR_INVALID_ARG
    assert call(out=P + 8) == bd.DIFFATTN_ERR_INVALID_ARG
    assert call(d=96) == bd.DIFFATTN_ERR_UNSUPPORTED
    assert call(flags=1, rms_eps=0.0) == bd.DIFFATTN_ERR_INVALID_ARG
    # 64 x 64 heads x 64 ranges x (128 + 4) floats = 138 MB of records > 32 MiB
    assert call(B=64, L=8192, Hq=64, Hkv=8, num_splits=64) == bd.DIFFATTN_ERR_WORKSPACE
