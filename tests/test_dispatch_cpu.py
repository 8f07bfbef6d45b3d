"""The chain launcher reaches a compiled kernel for every size the entry
points accept. Host only: in the launcher's dry-run mode the kernel is
selected exactly as for a launch and nothing is launched, so a size for which
no template instance exists (the launcher's hipErrorInvalidValue paths:
rank slices, list lengths, staged rows, stage counts, one or two workgroups
per CU, the pruned form's budgets) fails here without a GPU."""
import ctypes

import dspark_block_drafter_amd as dsp

BS = sorted(set(list(range(1, 70)) + [95, 96, 97, 127, 128, 129, 255, 256, 257, 511, 512, 513,
                                       1000, 1023, 1024, 1025, 2047, 2048, 4095, 4096]))
VS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257,
      511, 512, 513, 1000, 1023, 1024, 1025, 4095, 4096, 4097, 32768, 65535, 65536, 151936, 248320,
      262144, 1 << 20, (1 << 20) + 3]
RS = list(range(0, 257, 8)) + [4, 264]   # the last two are rejected by the argument checks


def _arr(xs):
    return (ctypes.c_int * len(xs))(*xs)


def test_chain_dispatch_covers_every_accepted_size():
    lib = dsp.load_library()
    walk = lib.dspark_internal_chain_dispatch_walk
    walk.restype = ctypes.c_long
    bad = (ctypes.c_int * 5)()
    checked = ctypes.c_long(0)
    n = walk(_arr(BS), len(BS), _arr(VS), len(VS), _arr(RS), len(RS), bad, ctypes.byref(checked))
    assert n == 0, (f"{n} accepted sizes reach no compiled chain kernel; first (B, V, r, top_k, "
                    f"bounded) = {tuple(bad)}")
    # every (B, V, r <= 256 in steps of 8, top_k <= min(V, 16), bounded) the checks accept
    want = sum(2 * min(V, 16) * 33 for B in BS for V in VS)
    assert checked.value == want, (checked.value, want)
