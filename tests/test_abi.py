"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ft.h")


def _lib():
    from bit_quantized_lora_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        from bit_quantized_lora_amd import build
        build.build()
    return L


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ft_status|size_t|const char\*)\s+(ft_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("ft_quant_block16", "ft_lowrank_fused", "ft_linear_fwd", "ft_linear_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    lib = L.lib()
    missing = [n for n in _declared() if getattr(lib, n, None) is None]
    assert not missing, missing
    # the Python binding knows every declared function
    assert set(_declared()) <= set(L._SIGS)


def test_status_strings():
    lib = _lib().lib()
    for s in range(7):
        assert lib.ft_status_str(s)
    assert b"unknown" in lib.ft_status_str(99)


def test_quant_argument_validation():
    L = _lib(); lib = L.lib()
    p = ctypes.c_void_p(16 * 1024)   # never dereferenced: validation fails or nothing launches
    assert lib.ft_quant_block16(p, 15, 16, 16, 0, p, None, p, None, None) == L.FT_ESHAPE
    assert lib.ft_quant_block16(p, 16, 16, 8, 0, p, None, p, None, None) == L.FT_ESHAPE      # ldx < cols
    assert lib.ft_quant_block16(p, 16, 16, 16, 7, p, None, p, None, None) == L.FT_EINVAL     # bad mode
    assert lib.ft_quant_block16(p, 16, 16, 16, 0, None, None, p, None, None) == L.FT_EINVAL  # no codes out
    assert lib.ft_quant_block16(None, 16, 16, 16, 0, p, None, p, None, None) == L.FT_EINVAL
    assert lib.ft_quant_block16(ctypes.c_void_p(16 * 1024 + 4), 16, 16, 16, 0, p, None, p, None, None) == L.FT_EALIGN
    assert lib.ft_quant_block16(p, 16, 16, 20, 0, p, None, p, None, None) == L.FT_EALIGN    # row pitch
    assert lib.ft_quant_block16(None, 0, 16, 16, 0, None, None, None, None, None) == L.FT_OK  # empty


def test_lowrank_argument_validation():
    L = _lib(); lib = L.lib()
    p = ctypes.c_void_p(16 * 1024)
    assert lib.ft_lowrank_fused(p, 16, 16, 16, p, 8, p, 16, p, None, 0, None) == L.FT_ESHAPE    # rank % 16
    assert lib.ft_lowrank_fused(p, 16, 16, 16, p, 96, p, 48, p, None, 0, None) == L.FT_ESHAPE   # rho > 128
    assert lib.ft_lowrank_fused(p, 17, 16, 16, p, 16, p, 16, p, None, 0, None) == L.FT_ESHAPE
    assert lib.ft_lowrank_fused(p, 0, 16, 16, p, 16, p, 16, p, None, 0, None) == L.FT_OK         # empty
    big_ws = lib.ft_lowrank_workspace(4608, 12288, 48)
    assert big_ws > 0
    assert lib.ft_lowrank_fused(p, 4608, 12288, 12288, p, 32, p, 16, p, None, 0, None) == L.FT_EINVAL
    assert lib.ft_lowrank_fused(p, 4608, 12288, 12288, p, 32, p, 16, p, p, 16, None) == L.FT_ESPACE


def test_linear_argument_validation():
    L = _lib(); lib = L.lib()
    p = ctypes.c_void_p(16 * 1024)
    # f32 block scales: the 4-bit GEMM applies power-of-two scales only
    assert lib.ft_linear_fwd(16, 16, 16, 1, p, p, p, p, p, p, 16, p, 16, p, 0, None) == L.FT_ENOTSUP
    assert lib.ft_linear_fwd(16, 16, 24, 0, p, p, p, p, p, p, 16, p, 16, p, 0, None) == L.FT_ESHAPE
    assert lib.ft_linear_fwd(16, 16, 16, 0, p, p, p, p, p, p, 16, p, 16, p, 5, None) == L.FT_EINVAL
    assert lib.ft_linear_fwd(16, 16, 16, 0, None, p, p, p, p, p, 16, p, 16, p, 0, None) == L.FT_EINVAL
    assert lib.ft_linear_fwd(0, 16, 16, 0, None, None, None, None, None, None, 16, None, 16, None, 0, None) == L.FT_OK
    # 512 tokens: the dX GEMM splits its reduction, so the backward needs a workspace
    ws = lib.ft_linear_bwd_workspace(512, 9216, 3072, 32)
    assert ws > 0
    args = [512, 9216, 3072, 0, p, p, p, p, p, p, 32, p, 32, p, p, p, p, 0, p, p]
    assert lib.ft_linear_bwd(*args, p, 16, None) == L.FT_ESPACE
    assert lib.ft_linear_bwd(*args, None, 0, None) == L.FT_EINVAL


def test_linear_fwd_gelu_argument_validation():
    L = _lib(); lib = L.lib()
    p = ctypes.c_void_p(16 * 1024)
    ok = [16, 16, 16, 0, p, p, p, p, p, p, 16, p, 16, p, p, p, p, None]
    bad_mode = list(ok); bad_mode[3] = 1
    assert lib.ft_linear_fwd_gelu(*bad_mode) == L.FT_ENOTSUP                 # f32 scales
    bad_k = list(ok); bad_k[2] = 24
    assert lib.ft_linear_fwd_gelu(*bad_k) == L.FT_ESHAPE
    no_h = list(ok); no_h[14] = None
    assert lib.ft_linear_fwd_gelu(*no_h) == L.FT_EINVAL                      # H missing
    no_codes = list(ok); no_codes[15] = None
    assert lib.ft_linear_fwd_gelu(*no_codes) == L.FT_EINVAL
    odd = list(ok); odd[16] = ctypes.c_void_p(16 * 1024 + 8)
    assert lib.ft_linear_fwd_gelu(*odd) == L.FT_EALIGN
    empty = [0, 16, 16, 0] + [None] * 6 + [16, None, 16, None, None, None, None, None]
    assert lib.ft_linear_fwd_gelu(*empty) == L.FT_OK


def test_precision_variant_argument_validation():
    L = _lib(); lib = L.lib()
    p = ctypes.c_void_p(16 * 1024)
    #      M   N   K   X  rq rs T  L2 rs  B  r   Y  ydt stream
    fwd = [16, 16, 16, p, p, p, p, p, 16, p, 16, p, 0, None]
    bad = list(fwd); bad[12] = 7
    assert lib.ft_linear_fwd_a16(*bad) == L.FT_EINVAL                        # unknown output type
    bad = list(fwd); bad[1] = 24
    assert lib.ft_linear_fwd_a16(*bad) == L.FT_ESHAPE
    bad = list(fwd); bad[8] = 128
    assert lib.ft_linear_fwd_a16(*bad) == L.FT_ESHAPE                        # rs + r > 128
    bad = list(fwd); bad[3] = None
    assert lib.ft_linear_fwd_a16(*bad) == L.FT_EINVAL                        # X missing
    bad = list(fwd); bad[3] = ctypes.c_void_p(16 * 1024 + 8)
    assert lib.ft_linear_fwd_a16(*bad) == L.FT_EALIGN
    assert lib.ft_linear_fwd_a16(0, 16, 16, None, None, None, None, None, 16, None, 16, None, 0, None) == L.FT_OK
    ws = int(lib.ft_linear_bwd_workspace(16, 16, 16, 16))
    #      M   N   K   G  rqc rsc V  L1t rs At r   X  T  dX dxdt dAt dB ws  bytes stream
    bwd = [16, 16, 16, p, p, p, p, p, 16, p, 16, p, p, p, 0, p, p, p, ws, None]
    bad = list(bwd); bad[18] = ws - 1
    assert lib.ft_linear_bwd_g16(*bad) == L.FT_ESPACE
    bad = list(bwd); bad[17] = None
    assert lib.ft_linear_bwd_g16(*bad) == L.FT_EINVAL                        # workspace missing
    bad = list(bwd); bad[3] = None
    assert lib.ft_linear_bwd_g16(*bad) == L.FT_EINVAL                        # G missing
    bad = list(bwd); bad[2] = 40
    assert lib.ft_linear_bwd_g16(*bad) == L.FT_ESHAPE
    bad = list(bwd); bad[13] = ctypes.c_void_p(16 * 1024 + 4)
    assert lib.ft_linear_bwd_g16(*bad) == L.FT_EALIGN


def test_group_granularity_argument_validation():
    L = _lib(); lib = L.lib()
    p = ctypes.c_void_p(16 * 1024)
    assert lib.ft_quant_group(p, 16, 32, 32, 8, p, p, None) == L.FT_EINVAL            # group 8
    assert lib.ft_quant_group(p, 16, 48, 48, 32, p, p, None) == L.FT_ESHAPE           # cols % 32
    assert lib.ft_quant_group(p, 16, 32, 24, 16, p, p, None) == L.FT_ESHAPE           # ldx < cols
    assert lib.ft_quant_group(p, 0, 32, 32, 16, None, None, None) == L.FT_OK
    assert lib.ft_requant_group_t(p, p, 48, 64, 32, p, p, None) == L.FT_ESHAPE        # rows % 32
    assert lib.ft_requant_group_t(p, p, 32, 64, 16, None, p, None) == L.FT_EINVAL
    #      M   N    K    g  xq xs rq rs T  L2 rs  B  r   Y  ydt stream
    fwd = [16, 128, 128, 16, p, p, p, p, p, p, 16, p, 16, p, 0, None]
    bad = list(fwd); bad[2] = 144
    assert lib.ft_linear_fwd_grp(*bad) == L.FT_ENOTSUP                                 # K % 128
    bad = list(fwd); bad[3] = 64
    assert lib.ft_linear_fwd_grp(*bad) == L.FT_EINVAL
    bad = list(fwd); bad[5] = None
    assert lib.ft_linear_fwd_grp(*bad) == L.FT_EINVAL
    ws = int(lib.ft_linear_bwd_workspace(16, 128, 128, 16))
    bwd = [16, 144, 128, 32, p, p, p, p, p, p, 16, p, 16, p, p, p, p, 0, p, p, p, ws, None]
    assert lib.ft_linear_bwd_grp(*bwd) == L.FT_ENOTSUP                                 # N % 128


def test_gelu_argument_validation():
    L = _lib(); lib = L.lib()
    p = ctypes.c_void_p(16 * 1024)
    assert lib.ft_gelu_fwd(p, 12, p, None) == L.FT_ESHAPE
    assert lib.ft_gelu_bwd(p, p, 12, p, None) == L.FT_ESHAPE
    assert lib.ft_gelu_fwd(p, 0, p, None) == L.FT_OK
    assert lib.ft_gelu_fwd(None, 16, p, None) == L.FT_EINVAL


def test_noalloc_backward_rejects_requests_beyond_its_scratch():
    """ft_linear_bwd_noalloc refuses a backward whose reduction partials exceed its
    fixed scratch, before touching the device."""
    L = _lib(); lib = L.lib()
    M, N, K, r = 1 << 20, 1 << 14, 1 << 12, 64
    assert lib.ft_linear_bwd_workspace(M, N, K, r) > L.FT_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(16 * 1024)   # never dereferenced
    st = lib.ft_linear_bwd_noalloc(M, N, K, 0, p, p, p, p, p, p, 64, p, r, p, p, p, p, 0, p, p, None)
    assert st == L.FT_ESPACE
    # every config of the method fits
    for (M, N, K, r) in ((18432, 9216, 3072, 64), (4608, 12288, 3072, 16), (4096, 3072, 12288, 32)):
        assert lib.ft_linear_bwd_workspace(M, N, K, r) <= L.FT_NOALLOC_SCRATCH_BYTES


def test_lowrank_plan_layouts_fit_two_workgroups_per_cu():
    """ft_lowrank_plan (the one-pass quantize + projection's launch) validates its
    arguments, gives the step's two passes the 64-row, whole-line-load layout, and
    for every rank keeps two workgroups per CU (at most 80 KB of LDS each, of a
    CU's 160 KB), chooses whole-line loads exactly where their 32 KB of staging
    still fits, covers the reduction with its splits, and stays within the
    workspace ft_lowrank_workspace sizes (no GPU needed)."""
    L = _lib(); lib = L.lib()
    plan = (ctypes.c_int32 * 5)()
    pp = ctypes.addressof(plan)
    assert lib.ft_lowrank_plan(4608, 3072, 48, None) == L.FT_EINVAL
    assert lib.ft_lowrank_plan(4600, 3072, 48, pp) == L.FT_ESHAPE
    assert lib.ft_lowrank_plan(4608, 3072, 40, pp) == L.FT_ESHAPE
    assert lib.ft_lowrank_plan(4608, 3072, 144, pp) == L.FT_ESHAPE
    assert lib.ft_lowrank_plan(0, 3072, 48, pp) == L.FT_OK and list(plan) == [0] * 5
    # the MLP-up step: X pass [4608 x 3072] and G pass [4608 x 12288] at rank 48
    assert lib.ft_lowrank_plan(4608, 3072, 48, pp) == L.FT_OK
    assert (plan[0], plan[1], plan[2], plan[3]) == (64, 1, 6, 2)
    assert lib.ft_lowrank_plan(4608, 12288, 48, pp) == L.FT_OK
    assert (plan[0], plan[1], plan[2], plan[3]) == (64, 1, 7, 7)
    stage, weights = 4 * 8192, lambda rho, wc: 2 * rho * 256 * wc
    for rho in range(0, 129, 16):
        for M in (16, 400, 4096, 4608, 18432):
            for K in (16, 1296, 3072, 12288):
                assert lib.ft_lowrank_plan(M, K, rho, pp) == L.FT_OK
                rows, lines, splits, cps, lds = list(plan)
                wc = 2 if rows == 64 else 1
                assert rows in (64, 128) and lds <= 80 * 1024, (rho, M, K, list(plan))
                # whole-line loads wherever the staging fits, column groups first
                fits2, fits1 = weights(rho, 2) + stage <= 80 * 1024, weights(rho, 1) + stage <= 80 * 1024
                assert lines == int(fits2 or fits1) and (rows == 64) == fits2, (rho, list(plan))
                assert lds >= weights(rho, wc) + (stage if lines else 0)
                chunk = 128 * wc
                nchunks = -(-K // chunk)
                assert splits * cps >= nchunks > (splits - 1) * cps, (rho, M, K, list(plan))
                if splits > 1 and rho:
                    assert lib.ft_lowrank_workspace(M, K, rho) >= splits * M * rho * 4


def test_backward_plan_query():
    """ft_linear_bwd_plan validates its arguments and describes a launch: the
    dX GEMM's tile and splits, the adapter workgroups of the same launch and
    their token ranges (no GPU needed: the plan uses the CU count, 256 without
    a device)."""
    L = _lib(); lib = L.lib()
    plan = (ctypes.c_int32 * 5)()
    assert lib.ft_linear_bwd_plan(4608, 12288, 3072, 16, 1, None) == L.FT_EINVAL
    assert lib.ft_linear_bwd_plan(4608, 12288, 3000, 16, 1, ctypes.addressof(plan)) == L.FT_ESHAPE
    assert lib.ft_linear_bwd_plan(4608, 12288, 3072, 24, 1, ctypes.addressof(plan)) == L.FT_ESHAPE
    assert lib.ft_linear_bwd_plan(4608, 12288, 3072, 16, 1, ctypes.addressof(plan)) == L.FT_OK
    assert plan[3] > 0 and plan[4] >= 1                      # adapter workgroups in the GEMM launch
    assert lib.ft_linear_bwd_plan(4608, 12288, 3072, 96, 1, ctypes.addressof(plan)) == L.FT_OK
    assert plan[3] == 0                                      # r > 64: side stream


def test_backward_workspace_covers_every_launch_plan():
    """The one workspace size of the backward covers what ft_linear_bwd_plan
    says the launch writes there, for shapes across the planner's branches
    (one-round GEMMs with the adapter workgroups beside them, multi-round ones
    with them after, the small tile with split reductions, ragged sizes) and
    ranks of one and two rank tiles, with and without dB: the adapter
    workgroups' token-range partials first (their largest size over both dB
    settings, 256-byte aligned), then the dX GEMM's split partials."""
    L = _lib(); lib = L.lib()
    a256 = lambda n: (n + 255) // 256 * 256
    plan = (ctypes.c_int32 * 5)()
    checked = 0
    for M in (256, 400, 512, 528, 4096, 4608, 16384, 18432):
        for (N, K) in ((3072, 3072), (12288, 3072), (3072, 12288), (9216, 3072), (1040, 1152), (1024, 4096),
                       (384, 4624)):
            for r in (16, 32, 48, 64):
                ws = lib.ft_linear_bwd_workspace(M, N, K, r)
                plans = {}
                for with_db in (1, 0):
                    assert lib.ft_linear_bwd_plan(M, N, K, r, with_db, ctypes.addressof(plan)) == L.FT_OK
                    plans[with_db] = tuple(plan)
                adapt = [p[4] * r * (K + (N if db else 0)) * 4 if p[3] > 0 and p[4] > 1 else 0
                         for db, p in plans.items()]
                for db, p in plans.items():
                    gemm = p[2] * M * K * 4 if p[2] > 1 else 0
                    need = (a256(max(adapt)) if p[3] > 0 else 0) + gemm
                    assert need <= ws, f"M={M} N={N} K={K} r={r} dB={db}: plan {p} needs {need} > {ws}"
                    checked += 1
    assert checked == 8 * 7 * 4 * 2
