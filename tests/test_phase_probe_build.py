"""The phase-timing build (linear_attention_lightning_amd/phase_probe.py) still
compiles, and only it exports the record entry points: the library proper
compiles the marks to nothing (CPU only; the build cross-compiles for gfx950)."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NAMES = ("lightning_attn_phase_probe_copy", "lightning_attn_phase_probe_copy_local",
         "lightning_attn_phase_probe_clear")


@pytest.mark.slow
def test_phase_probe_build_exports_its_entry_points():
    from linear_attention_lightning_amd import phase_probe
    path = phase_probe.build()
    lib = ctypes.CDLL(path)
    for n in NAMES:
        assert hasattr(lib, n), n
    main = ctypes.CDLL(os.path.join(ROOT, "linear_attention_lightning_amd", "liblightning_attn.so"))
    for n in NAMES:
        assert not hasattr(main, n), n
