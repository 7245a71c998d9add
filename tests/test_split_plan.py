"""Host logic of the decode FFN's K split (csrc/split_plan.h), compiled with
g++ on the CPU: the busiest-CU model against brute force over every CU, the
chosen parts against every feasible alternative, and the decisions the rule
makes on the layers it was measured on."""
import os
import random
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4_group_quantized_amd", "csrc")

CUS = 256
MAX_PARTS = 8
MIN_BYTES = 48 << 10
COST_BYTES = 160 << 10

DRIVER = r"""
#include "split_plan.h"
#include <cstdio>
#include <cstring>
using namespace moe;
int main() {
  // constants first, then one answer per input line
  std::printf("%d %d %lld %lld\n", kCus, kMaxParts, (long long)kSplitMinBytes,
              (long long)kSplitCostBytes);
  char op[16];
  while (std::scanf("%15s", op) == 1) {
    if (!std::strcmp(op, "busiest")) {
      long long ns, sb, nr, rb; int slots;
      if (std::scanf("%lld %lld %lld %lld %d", &ns, &sb, &nr, &rb, &slots) != 5) return 1;
      std::printf("%lld\n", (long long)busiest_cu(ns, sb, nr, rb, slots));
    } else if (!std::strcmp(op, "parts")) {
      long long nr, rb, ns, sb; int max_rp, max_sp, slots, rp, sp;
      if (std::scanf("%lld %lld %d %lld %lld %d %d", &nr, &rb, &max_rp, &ns, &sb, &max_sp,
                     &slots) != 7) return 1;
      split_parts(nr, rb, max_rp, ns, sb, max_sp, slots, &rp, &sp);
      std::printf("%d %d\n", rp, sp);
    } else {
      return 1;
    }
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def plan(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    d = tmp_path_factory.mktemp("split_plan")
    src, exe = d / "driver.cpp", d / "driver"
    src.write_text(DRIVER)
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, str(src), "-o",
                    str(exe)], check=True)

    def run(lines):
        r = subprocess.run([str(exe)], input="\n".join(lines) + "\n", capture_output=True,
                           text=True, check=True)
        out = r.stdout.split("\n")
        consts = tuple(int(v) for v in out[0].split())
        return consts, [tuple(int(v) for v in ln.split()) for ln in out[1:1 + len(lines)]]
    return run


def brute_busiest(ns, sb, nr, rb, slots):
    """Blocks 0 .. ns-1 of sb bytes, then nr of rb bytes; block b on CU b % 256
    in dispatch round b // 256 (at most `slots` rounds): the largest CU load."""
    load = [0] * CUS
    for b in range(ns + nr):
        assert b < slots * CUS
        load[b % CUS] += sb if b < ns else rb
    return max(load)


def test_constants(plan):
    consts, _ = plan([])
    assert consts == (CUS, MAX_PARTS, MIN_BYTES, COST_BYTES)


@pytest.mark.parametrize("seed", [0, 1])
def test_busiest_cu_against_brute_force(plan, seed):
    """Evaluated only where a CU's load can change, busiest_cu still finds the
    maximum over all 256 CUs: random block counts across one to four dispatch
    rounds, and the edge cases (no blocks of one kind, exactly full rounds)."""
    rng = random.Random(seed)
    cases = [(0, 0, 0, 0, 3), (256, 5, 0, 0, 3), (0, 0, 768, 7, 3), (768, 2, 0, 9, 3),
             (1, 100, 1023, 3, 4), (255, 1, 1, 1000, 1), (257, 10, 255, 20, 2)]
    for _ in range(600):
        slots = rng.randint(1, 4)
        n = rng.randint(0, slots * CUS)
        ns = rng.randint(0, n)
        cases.append((ns, rng.randint(1, 1 << 20), n - ns, rng.randint(1, 1 << 20), slots))
    _, got = plan([f"busiest {ns} {sb} {nr} {rb} {s}" for ns, sb, nr, rb, s in cases])
    for c, (g,) in zip(cases, got):
        assert g == brute_busiest(*c), c


def feasible(nr, rb, max_rp, ns, sb, max_sp, slots, r, q):
    if nr * r + ns * q > slots * CUS:
        return False
    if r > 1 and rb // r < MIN_BYTES:
        return False
    if q > 1 and sb // q < MIN_BYTES:
        return False
    return 1 <= r <= min(max_rp, MAX_PARTS) and 1 <= q <= min(max_sp if ns else 1, MAX_PARTS)


def cost(nr, rb, ns, sb, slots, r, q):
    c = brute_busiest(ns * q, sb // q if ns else 0, nr * r, rb // r, slots)
    return c if (r, q) == (1, 1) else c + COST_BYTES


@pytest.mark.parametrize("seed", [0, 1])
def test_split_parts_is_the_cheapest_feasible_choice(plan, seed):
    """The parts returned are feasible (one round of slots, blocks of at least
    48 KB, at most 8 parts and the caller's maxima) and no feasible choice has
    a smaller busiest-CU load plus the split's fixed cost; batches that do not
    fit one round unsplit stay whole."""
    rng = random.Random(100 + seed)
    cases = []
    for _ in range(120):
        slots = rng.choice([3, 4])
        nr = rng.randint(0, 500)
        ns = rng.choice([0, rng.randint(1, 300)])
        cases.append((nr, rng.randint(16 << 10, 4 << 20), rng.randint(1, 32), ns,
                      rng.randint(16 << 10, 1 << 20), rng.randint(1, 8), slots))
    _, got = plan([f"parts {a} {b} {c} {d} {e} {f} {g}" for a, b, c, d, e, f, g in cases])
    for (nr, rb, max_rp, ns, sb, max_sp, slots), (r, q) in zip(cases, got):
        if nr + ns > slots * CUS:
            assert (r, q) == (1, 1)
            continue
        args = (nr, rb, max_rp, ns, sb, max_sp, slots)
        assert (r, q) == (1, 1) or feasible(*args, r, q), (args, r, q)
        mine = cost(nr, rb, ns, sb, slots, r, q)
        for rr in range(1, MAX_PARTS + 1):
            for qq in range(1, MAX_PARTS + 1):
                if feasible(*args, rr, qq):
                    assert mine <= cost(nr, rb, ns, sb, slots, rr, qq), (args, (r, q), (rr, qq))


def test_decisions_on_the_measured_layers(plan):
    """One token: on the 288-expert layer (H 4096, F 1536, fp16 shared expert
    of 1536) gate/up splits 3 ways per routed and 2 per shared item, the down
    launch stays whole; on the coarse 16-expert layer (H 12288, F 65536, top-4)
    gate/up stays whole (4096 items, more than one round) and down splits in
    2.  Item bytes are codes + fp16 scales of 128-column groups."""
    def item(rows, K):
        return rows * (K // 2 + K // 128 * 2)
    lines = [
        # 288-expert layer, gate/up: 8 experts x 24 items of 64 + 64 rows; 96 shared items
        f"parts {8 * 24} {item(128, 4096)} {4096 // 256} 96 {16 * 2 * 4096 * 2} {4096 // 1024} 3",
        # 288-expert layer, down: 8 experts x 32 items of 128 rows; 256 shared items
        f"parts {8 * 32} {item(128, 1536)} {1536 // 256} 256 {16 * 1536 * 2} {1536 // 1024} 3",
        # coarse layer, gate/up and down at one token (4 experts, no shared expert)
        f"parts {4 * 1024} {item(128, 12288)} {12288 // 256} 0 0 0 3",
        f"parts {4 * 96} {item(128, 65536)} {65536 // 256} 0 0 0 3",
    ]
    _, got = plan(lines)
    assert got == [(3, 2), (1, 1), (1, 1), (2, 1)]
