"""CPU oracle for the PARO W4A8 linear hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the ``rotated_w4a8_group_amd``
package, its C-ABI library or its kernels) may import, call or link this package; only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg use it.

It is a plain, slow, obviously-correct restatement of what the method computes, written
from the page "ParoQuant (PARO) W4A8 on gfx1201 — engineering log" (sections "Format" and
"Design"), with no blocking, fusion or reordering beyond what that text states:

* ``e4m3``     — OCP E4M3FN decode table and round-to-nearest-even saturating encoder.
* ``awq``      — AWQ nibble unpack of ``qweight`` / ``qzeros``.
* ``records``  — Givens pair records (channel pair + f16 cos/sin) from ``pairs``/``theta``.
* ``prologue`` — channel scale, 8 rotation layers, per-(token, group) amax, e4m3 encode,
  code-domain row-sums, emulated step by step in IEEE binary32.
* ``gemm``     — the same-codes reference GEMM, exact per group in fp64.
* ``tokquant`` — the per-token activation-scale prologue and GEMM.
* ``int8``     — the per-group int8 activation prologue and GEMM.
* ``int5``     — the int5 bit-plane weight unpack and GEMM.
* ``producer`` — the fused residual add + RMSNorm + rotate + quant producer.

Every function is pinned by ``tests/test_oracle_*.py`` against values that do not come
from the oracle itself (closed forms, library routines, exact rationals, brute force).
"""
from . import e4m3, awq, records, prologue, gemm, tokquant, int8, int5, producer  # noqa: F401

__all__ = ["e4m3", "awq", "records", "prologue", "gemm", "tokquant", "int8", "int5", "producer"]
