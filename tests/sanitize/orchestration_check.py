"""Drive the host orchestration of every entry point through the host-only
sanitizer build of the library (launchers stubbed, see launch_stubs.cpp).

Each call passes validation and runs the planning, workspace carving and
launch sequence to the end; the stubs never touch the fake device addresses,
so AddressSanitizer and UndefinedBehaviorSanitizer see only host-side work.
Run by tests/test_host_sanitize.py with QV_LIBRARY pointing at that build;
never against the real library (it would launch kernels on fake addresses)."""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import resolution_vit_vision_amd as qv  # noqa: E402
from resolution_vit_vision_amd import _abi  # noqa: E402
from resolution_vit_vision_amd.encoder import MergerConfig, VisionConfig  # noqa: E402


def main() -> int:
    if "stub" not in os.path.basename(os.environ.get("QV_LIBRARY", "")):
        print("refusing to run: QV_LIBRARY must name the stubbed sanitizer build")
        return 2
    L = qv.lib()
    dev = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x7f0000000000)          # 256-byte aligned fake workspace
    workloads = [wl for wl in synth.WORKLOADS.values()]
    runs = 0
    for wl in workloads:
        grids = [(-(-f // 2), h // 14, w // 14) for (h, w, f) in wl.images]
        g = np.ascontiguousarray(np.asarray(grids, np.int32).reshape(-1, 3))
        variants = [dict(window=0, weights="dtype"), dict(window=8, weights="dtype"), dict(window=10, weights="dtype")]
        if wl.dtype == "bf16":
            variants.append(dict(window=0, weights="int8"))
            variants.append(dict(window=8, weights="int8"))
        for v in variants:
            cfg = VisionConfig(depth=wl.depth, dtype=wl.dtype, patch_dim=1176, ld=1176, window=v["window"],
                               full_blocks=(0,) if v["window"] else (), weights=v["weights"])
            c = cfg.c()
            nbytes = ctypes.c_size_t()
            _abi.check(L.qv_vision_workspace_size(ctypes.byref(c), g.ctypes.data, len(g), ctypes.byref(nbytes)))
            blocks = (_abi.BlockW * wl.depth)(*[_abi.BlockW(*([0x20000] * 12 + [0x30000] * 4))
                                                for _ in range(wl.depth)])
            w = _abi.VisionW(0x40000, None, blocks)
            _abi.check(L.qv_vision_forward(ctypes.byref(c), ctypes.byref(w), dev, g.ctypes.data, len(g), dev, dev,
                                           ws, nbytes.value, None))
            st = L.qv_vision_forward_noalloc(ctypes.byref(c), ctypes.byref(w), dev, g.ctypes.data, len(g), dev, dev,
                                             None)
            assert st == (_abi.QV_OK if nbytes.value <= _abi.QV_SCRATCH_BYTES else _abi.QV_ERR_WORKSPACE), st
            runs += 2
        n = int((g[:, 0].astype(np.int64) * g[:, 1] * g[:, 2]).sum())
        mc = MergerConfig(out_dim=wl.out_dim, dtype=wl.dtype).c()
        mb = ctypes.c_size_t()
        _abi.check(L.qv_merge_workspace_size(ctypes.byref(mc), n, ctypes.byref(mb)))
        mw = _abi.MergerW(*([0x50000] * 6))
        _abi.check(L.qv_patch_merge(ctypes.byref(mc), ctypes.byref(mw), dev, n, dev, ws, mb.value, None))
        imgs = (_abi.Image * len(grids))(*[_abi.Image(0, f, 3, h, w, 0) for (h, w, f) in wl.images])
        for fold in ((False, True) if all(f == 1 for (_, _, f) in wl.images) else (False,)):
            opts = qv.patch_opts(fold=fold, normalize=fold)
            ld = qv.patch_width(3, fold)
            _abi.check(L.qv_patchify_ex(dev, imgs, len(grids), g.ctypes.data, None, ctypes.byref(opts), dev,
                                        _abi.QV_BF16, ld, None))
        runs += 3
    _abi.check(L.qv_fold_patch_weight(dev, 1280, 3, 14, 2, 1176, dev, 592, _abi.QV_BF16, None))
    _abi.check(L.qv_quantize_i8(dev, 3840, 1280, 1280, _abi.QV_BF16, dev, dev, None))
    print(f"orchestration_check: {runs} entry-point calls ran to completion")
    return 0


if __name__ == "__main__":
    sys.exit(main())
