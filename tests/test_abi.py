"""The C ABI without a GPU: the library loads, exports every symbol that
include/qattn.h declares, and rejects every invalid argument with its status
before any HIP call (so no call here reaches the device)."""

import ctypes
import os
import re
import subprocess

import pytest

import bit_quantized_attention_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qattn.h")

OK, NULL, SHAPE, ALIGN, UNSUP, ARG = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qa.LIB_PATH):
        pytest.fail("libqattn.so is not built (run python -m bit_quantized_attention_amd.build)")
    return qa.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qattn_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"qattn_smooth_quant", "qattn_block_mask", "qattn_fwd"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", qa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(qattn_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for s in range(8):
        assert len(qa.qattn_status_str(s)) > 0
    assert qa.qattn_status_str(99) == "unknown status"
    assert "gfx950" in qa.qattn_version()


def _p(**kw):
    base = dict(B=1, Hq=4, Hkv=2, N=256, d=128, dtype=1, causal=1)
    base.update(kw)
    return qa.qattn_problem_t(**base)


# aligned, non-null fake addresses: validation must fail before they are used
A = 1 << 20


def _sq(p, **over):
    args = dict(q=A, k=A, q_i8=A, q_scale=A, k_i8=A, k_scale=A, k_mean=A, q_pool=None,
                k_pool=None, workspace=A, workspace_bytes=1 << 30)
    args.update(over)
    return qa.qattn_smooth_quant(p, args["q"], args["k"], args["q_i8"], args["q_scale"],
                                 args["k_i8"], args["k_scale"], args["k_mean"], args["q_pool"],
                                 args["k_pool"], args["workspace"], args["workspace_bytes"],
                                 stream=0, check=False)


def _bm(p, **over):
    args = dict(qp=A, kp=A, num=1, den=10, mk=1000, idx=A, cnt=A, ws=A, wsb=1 << 30)
    args.update(over)
    return qa.qattn_block_mask(p, args["qp"], args["kp"], args["num"], args["den"], args["mk"],
                               args["idx"], args["cnt"], args["ws"], args["wsb"], stream=0,
                               check=False)


def _fw(p, **over):
    args = dict(qi=A, qs=A, ki=A, kscl=A, v=A, idx=None, cnt=None, mk=0, o=A, lse=None)
    args.update(over)
    return qa.qattn_fwd(p, args["qi"], args["qs"], args["ki"], args["kscl"], args["v"],
                        args["idx"], args["cnt"], args["mk"], args["o"], args["lse"], stream=0,
                        check=False)


def _fp(p, **over):
    args = dict(qi=A, qs=A, ki=A, kscl=A, q=A, k=A, km=A, v=A, idx=A, cnt=A, mk=8, o=A, lse=None)
    args.update(over)
    return qa.qattn_fwd_promoted(p, args["qi"], args["qs"], args["ki"], args["kscl"], args["q"],
                                 args["k"], args["km"], args["v"], args["idx"], args["cnt"],
                                 args["mk"], args["o"], args["lse"], stream=0, check=False)


def _f4(p, **over):
    args = dict(q=A, k=A, km=A, v=A, idx=A, cnt=A, mk=8, o=A, lse=None, ws=A, wsb=1 << 40)
    args.update(over)
    return qa.qattn_fwd_promoted_fp4(p, args["q"], args["k"], args["km"], args["v"], args["idx"],
                                     args["cnt"], args["mk"], args["o"], args["lse"], args["ws"],
                                     args["wsb"], stream=0, check=False)


def _pm(p, **over):
    args = dict(idx=A, cnt=A, mk=8, nv=4, ns=4, oidx=A + (1 << 24), ocnt=A + (2 << 24), omk=16,
                lines=A + (3 << 24))
    args.update(over)
    return qa.qattn_block_mask_patterns(p, args["idx"], args["cnt"], args["mk"], args["nv"],
                                        args["ns"], args["oidx"], args["ocnt"], args["omk"],
                                        args["lines"], stream=0, check=False)


def _he(p, **over):
    args = dict(qi=A, qs=A, ki=A, kscl=A, q=A, k=A, km=A, thr=0.02, err=A, hi=None)
    args.update(over)
    return qa.qattn_head_error(p, args["qi"], args["qs"], args["ki"], args["kscl"], args["q"],
                               args["k"], args["km"], args["thr"], args["err"], args["hi"],
                               stream=0, check=False)


def _fa(p, **over):
    args = dict(qi=A, qs=A, ki=A, kscl=A, q=A, k=A, km=A, v=A, hi=A, o=A, lse=None)
    args.update(over)
    return qa.qattn_fwd_adaptive(p, args["qi"], args["qs"], args["ki"], args["kscl"], args["q"],
                                 args["k"], args["km"], args["v"], args["hi"], args["o"],
                                 args["lse"], stream=0, check=False)


def _lb(p, **over):
    args = dict(q=A, k=A, km=A, num=1, den=10, mk=1000, idx=A, cnt=A, sc=None, ws=A, wsb=1 << 40)
    args.update(over)
    return qa.qattn_block_mask_lowbit(p, args["q"], args["k"], args["km"], args["num"], args["den"],
                                      args["mk"], args["idx"], args["cnt"], args["sc"], args["ws"],
                                      args["wsb"], stream=0, check=False)


def _ss(p, **over):
    args = dict(qp=A, ki=A, ks=A, th=1.0, mk=512, idx=A, cnt=A)
    args.update(over)
    return qa.qattn_stripe_select(p, args["qp"], args["ki"], args["ks"], args["th"], args["mk"],
                                  args["idx"], args["cnt"], stream=0, check=False)


def _fs(p, **over):
    args = dict(qi=A, qs=A, ki=A, kscl=A, v=A, idx=A, cnt=A, mk=512, o=A, lse=None)
    args.update(over)
    return qa.qattn_fwd_stripes(p, args["qi"], args["qs"], args["ki"], args["kscl"], args["v"],
                                args["idx"], args["cnt"], args["mk"], args["o"], args["lse"],
                                stream=0, check=False)


def _sn(p, **over):
    args = dict(q=A, k=A, q_i8=A, q_scale=A, k_i8=A, k_scale=A, k_mean=A, q_pool=None,
                k_pool=None)
    args.update(over)
    return qa.qattn_smooth_quant_noalloc(p, args["q"], args["k"], args["q_i8"], args["q_scale"],
                                         args["k_i8"], args["k_scale"], args["k_mean"],
                                         args["q_pool"], args["k_pool"], stream=0, check=False)


@pytest.mark.parametrize("call", [_sq, _sn, _bm, _fw, _fp, _he, _fa, _lb, _ss, _fs])
def test_problem_validation(lib, call):
    assert call(_p(B=0)) == SHAPE
    assert call(_p(Hq=0)) == SHAPE
    assert call(_p(N=-128)) == SHAPE
    assert call(_p(Hq=6, Hkv=4)) == SHAPE
    assert call(_p(d=96)) == UNSUP
    assert call(_p(d=256)) == UNSUP
    assert call(_p(N=200)) == UNSUP          # N not a multiple of 128 (a ragged tail)
    assert call(_p(dtype=2)) == UNSUP
    assert call(_p(causal=2)) == ARG


def test_null_problem(lib):
    st = lib.qattn_fwd(None, A, A, A, A, A, None, None, 0, A, None, None)
    assert st == NULL
    assert lib.qattn_workspace_bytes(None) == 0
    assert lib.qattn_max_keep(None, 1, 10) == -1


def test_smooth_quant_arguments(lib):
    p = _p()
    for name in ["q", "k", "q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "workspace"]:
        assert _sq(p, **{name: None}) == NULL, name
    for name in ["q", "k", "q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "workspace"]:
        assert _sq(p, **{name: A + 8}) == ALIGN, name
    assert _sq(p, q_pool=A + 4) == ALIGN
    assert _sq(p, k_pool=A + 2) == ALIGN
    need = qa.qattn_workspace_bytes(p)
    assert need > 0
    assert _sq(p, workspace_bytes=need - 1) == ARG


def test_smooth_quant_noalloc_arguments(lib):
    p = _p()
    for name in ["q", "k", "q_i8", "q_scale", "k_i8", "k_scale", "k_mean"]:
        assert _sn(p, **{name: None}) == NULL, name
        assert _sn(p, **{name: A + 8}) == ALIGN, name
    assert _sn(p, q_pool=A + 4) == ALIGN
    # partial sums of B * Hkv * ceil(N/128) * d * 16 bytes must fit the static
    # 16 MiB array: here 2 * 4097 * 128 * 16 bytes do not
    need = 2 * ((524288 + 128) // 128) * 128 * 16
    assert need > qa.NOALLOC_SCRATCH_BYTES
    assert _sn(_p(N=524288 + 128)) == 7  # QATTN_ERR_SCRATCH
    assert "scratch" in qa.qattn_status_str(7)


def test_block_mask_arguments(lib):
    p = _p(N=1024)
    for name in ["qp", "kp", "idx", "cnt", "ws"]:
        assert _bm(p, **{name: None}) == NULL, name
        assert _bm(p, **{name: A + 4}) == ALIGN, name
    assert _bm(p, num=-1) == ARG
    assert _bm(p, den=0) == ARG
    assert _bm(p, num=11, den=10) == ARG
    mk = qa.qattn_max_keep(p, 1, 10)
    assert mk == min(16, 3 + 2)
    assert _bm(p, mk=mk - 1) == ARG
    assert _bm(p, wsb=qa.qattn_workspace_bytes(p) - 1) == ARG
    assert _bm(_p(N=131072 + 128)) == UNSUP


def test_fwd_arguments(lib):
    p = _p()
    for name in ["qi", "qs", "ki", "kscl", "v", "o"]:
        assert _fw(p, **{name: None}) == NULL, name
        assert _fw(p, **{name: A + 8}) == ALIGN, name
    assert _fw(p, lse=A + 4) == ALIGN
    assert _fw(p, idx=A) == ARG           # kv_idx without kv_cnt
    assert _fw(p, cnt=A) == ARG
    assert _fw(p, idx=A, cnt=A, mk=0) == ARG
    # a kept list indexes at most 2048 blocks of 64 keys; dense has no such limit
    assert _fw(_p(N=131072 + 128), idx=A, cnt=A, mk=16) == UNSUP
    assert _fw(_p(N=(1 << 21) + 128), idx=A, cnt=A, mk=16) == UNSUP


def test_fwd_promoted_arguments(lib):
    p = _p()
    names = ["qi", "qs", "ki", "kscl", "q", "k", "km", "v", "idx", "cnt", "o"]
    for name in names:
        assert _fp(p, **{name: None}) == NULL, name
        assert _fp(p, **{name: A + 8}) == ALIGN, name
    assert _fp(p, lse=A + 4) == ALIGN
    assert _fp(p, mk=0) == ARG
    assert _fp(p, mk=2049) == ARG
    assert _fp(_p(N=131072 + 128)) == UNSUP


def test_fwd_promoted_fp4_arguments(lib):
    p = _p(N=1024)
    for name in ["q", "k", "km", "v", "idx", "cnt", "o", "ws"]:
        assert _f4(p, **{name: None}) == NULL, name
        assert _f4(p, **{name: A + 8}) == ALIGN, name
    assert _f4(p, lse=A + 4) == ALIGN
    assert _f4(p, mk=0) == ARG
    assert _f4(p, mk=2049) == ARG
    # the workspace holds the MX FP4 codes (the low-bit mask's layout)
    assert _f4(p, wsb=qa.qattn_lowbit_workspace_bytes(p) - 4 * 8 * 16 * 4 - 1) == ARG
    assert _f4(_p(N=131072 + 128)) == UNSUP


def test_block_mask_patterns_arguments(lib):
    p = _p(N=1024)   # 16 key blocks
    for name in ["idx", "cnt", "oidx", "ocnt", "lines"]:
        assert _pm(p, **{name: None}) == NULL, name
        assert _pm(p, **{name: (A + 4) if name in ("idx", "cnt") else _pm_addr(name) + 4}) == ALIGN
    # no line asked for: lines may be NULL (not called with valid arguments
    # here: every other check must fail first)
    assert _pm(p, nv=0, ns=0, lines=None, omk=7) == ARG
    assert _pm(p, nv=-1) == ARG
    assert _pm(p, ns=qa.MAX_PATTERN_LINES + 1) == ARG
    assert _pm(p, mk=0) == ARG
    assert _pm(p, omk=15) == ARG            # below max_keep + n_vertical + n_slash
    assert _pm(_p(N=256), mk=3, omk=3) == ARG   # 4 key blocks: at least 4
    # an output overlapping an input
    assert _pm(p, oidx=A + 64) == ARG
    assert _pm(p, ocnt=A) == ARG
    assert _pm(_p(N=131072 + 128)) == UNSUP


def _pm_addr(name):
    return {"oidx": A + (1 << 24), "ocnt": A + (2 << 24), "lines": A + (3 << 24)}[name]


def test_head_error_arguments(lib):
    p = _p()
    for name in ["qi", "qs", "ki", "kscl", "q", "k", "km", "err"]:
        assert _he(p, **{name: None}) == NULL, name
        assert _he(p, **{name: A + 8}) == ALIGN, name
    assert _he(p, hi=A + 4) == ALIGN
    assert _he(p, thr=-1.0) == ARG
    assert _he(p, thr=float("nan")) == ARG
    assert _he(p, thr=float("inf")) == ARG


def test_fwd_adaptive_arguments(lib):
    p = _p()
    for name in ["qi", "qs", "ki", "kscl", "q", "k", "km", "v", "hi", "o"]:
        assert _fa(p, **{name: None}) == NULL, name
        assert _fa(p, **{name: A + 8}) == ALIGN, name
    assert _fa(p, lse=A + 4) == ALIGN
    assert _fa(_p(N=131072 + 128)) == UNSUP


def test_block_mask_lowbit_arguments(lib):
    p = _p(N=1024)
    for name in ["q", "k", "km", "idx", "cnt", "ws"]:
        assert _lb(p, **{name: None}) == NULL, name
        assert _lb(p, **{name: A + 4}) == ALIGN, name
    assert _lb(p, sc=A + 4) == ALIGN
    assert _lb(p, num=-1) == ARG
    assert _lb(p, den=0) == ARG
    assert _lb(p, mk=qa.qattn_max_keep(p, 1, 10) - 1) == ARG
    need = qa.qattn_lowbit_workspace_bytes(p)
    assert _lb(p, wsb=need - 1) == ARG
    assert _lb(_p(N=131072 + 128)) == UNSUP
    # FP4 codes and exponents of Q (4 heads) and K (2 heads), 256-byte aligned,
    # plus the block scores
    n_q, n_k = 4 * 1024, 2 * 1024
    assert need == (n_q * 64 + n_q * 4 + n_k * 64 + n_k * 4) + 4 * 8 * 16 * 4


def test_stripe_arguments(lib):
    p = _p(N=1024)
    for name in ["qp", "ki", "ks", "idx", "cnt"]:
        assert _ss(p, **{name: None}) == NULL, name
        assert _ss(p, **{name: A + 4}) == ALIGN, name
    assert _ss(p, th=float("nan")) == ARG
    assert _ss(p, mk=191) == ARG
    assert _ss(p, mk=3073) == ARG
    assert _ss(_p(N=65536 + 128)) == UNSUP
    for name in ["qi", "qs", "ki", "kscl", "v", "idx", "cnt", "o"]:
        assert _fs(p, **{name: None}) == NULL, name
        assert _fs(p, **{name: A + 8}) == ALIGN, name
    assert _fs(p, lse=A + 4) == ALIGN
    assert _fs(p, mk=0) == ARG
    assert _fs(p, mk=3073) == ARG
    assert _fs(_p(N=65536 + 128)) == UNSUP


def test_max_keep_and_workspace_sizes(lib):
    p = _p(N=32768, Hq=32, Hkv=8)
    assert qa.qattn_max_keep(p, 1, 10) == 55
    assert qa.qattn_max_keep(p, 1, 1) == 512
    assert qa.qattn_max_keep(p, 0, 1) == 3
    assert qa.qattn_max_keep(p, 2, 1) == -1
    ws = qa.qattn_workspace_bytes(p)
    # K partial sums: 8 heads x 256 chunks x 128 channels x 16 bytes; mask codes:
    # (32*256 + 8*512) pooled vectors x (128 + 4) bytes
    assert ws == max(8 * 256 * 128 * 16, (32 * 256 + 8 * 512) * 132)


def test_binding_has_the_c_names():
    for n in ["qattn_smooth_quant", "qattn_block_mask", "qattn_fwd", "qattn_fwd_promoted",
              "qattn_fwd_promoted_fp4", "qattn_smooth_quant_noalloc", "qattn_block_mask_patterns",
              "qattn_head_error", "qattn_fwd_adaptive", "qattn_block_mask_lowbit",
              "qattn_lowbit_workspace_bytes", "qattn_stripe_select", "qattn_fwd_stripes",
              "qattn_workspace_bytes", "qattn_max_keep",
              "qattn_status_str", "qattn_version"]:
        assert callable(getattr(qa, n))


def test_load_fails_loudly_without_library(tmp_path):
    saved = qa._lib
    try:
        qa._lib = None
        with pytest.raises(ImportError):
            qa.load(str(tmp_path / "missing.so"))
    finally:
        qa._lib = saved


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(QATTN_[A-Z_]+)\s+(\d+)", text))
    assert int(defs["QATTN_Q_BLOCK"]) == qa.Q_BLOCK
    assert int(defs["QATTN_K_BLOCK"]) == qa.K_BLOCK
    assert int(defs["QATTN_KV_TILE"]) == qa.KV_TILE
    assert int(defs["QATTN_SOFTMAX_REF_THRESHOLD"]) == qa.SOFTMAX_REF_THRESHOLD
    assert "#define QATTN_NOALLOC_SCRATCH_BYTES (16u << 20)" in text
    assert qa.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert int(defs["QATTN_MAX_PATTERN_LINES"]) == qa.MAX_PATTERN_LINES
