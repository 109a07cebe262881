"""CPU oracle (test infrastructure only; never imported by the product path).

ref  -- NumPy float64 definitions, exact-rational scans, brute force.
cpu  -- ctypes wrapper of the plain-C float64 recurrence and the float32
        replay of the blocked scan order (oracle/ref_cpu.c).
"""
