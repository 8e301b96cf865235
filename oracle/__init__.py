"""CPU oracle for the routed-MoE expert layer with 2-bit routed experts.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may.  It shares no code with the HIP library
(``bit_quantized_routed_amd``); the two meet only through the seeded inputs of
``synthetic``.

Parts:
  formats  -- block layouts, the reference quantizers (plain C in
              ``quant_ref.c``, loaded through ctypes) and dequantization
              (numpy, exact fp32).
  moe_ref  -- router (fp64 logits, top-k, normalised sigmoid weights),
              grouping (offsets / perm / inv), the SwiGLU expert FFN and the
              routing-weighted combine, all in fp64.

Every function is pinned by ``tests/test_oracle_*.py`` against values and
properties fixed independently of it (hand-computed blocks, closed forms,
invariants, brute force on tiny inputs, library routines).
"""
import os
import subprocess
import ctypes

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liboracle_quant.so")
_lib = None


def build_oracle_lib() -> str:
    """Compile quant_ref.c with gcc (strict IEEE fp32: no contraction)."""
    os.makedirs(_BUILD, exist_ok=True)
    src = os.path.join(_HERE, "quant_ref.c")
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    """The loaded reference-quantizer library (built on first use if absent)."""
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "quant_ref.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
            build_oracle_lib()
        L = ctypes.CDLL(_LIB_PATH)
        L.ref_quant_rows.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.ref_quant_rows.restype = ctypes.c_int
        L.ref_f32_to_f16_bits.argtypes = [ctypes.c_float]
        L.ref_f32_to_f16_bits.restype = ctypes.c_uint16
        L.ref_f16_bits_to_f32.argtypes = [ctypes.c_uint16]
        L.ref_f16_bits_to_f32.restype = ctypes.c_float
        _lib = L
    return _lib
