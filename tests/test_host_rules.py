"""Host-side shape rules of the launchers (csrc/host_rules.h), compiled with the system C++
compiler and checked on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RULES = os.path.join(ROOT, "block_diffusion_drafter_draft_amd", "csrc", "host_rules.h")


def test_resid_norm_fusion_predicate(tmp_path):
    """The split-K reduction fuses the next RMSNorm only for rows one 1,024-thread workgroup
    covers with whole four-float vectors, stored densely: up to 8,192 columns, a multiple of 4,
    row stride equal to the width.  Wider, ragged or strided rows fall back to the plain
    reduction plus a separate norm."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    cases = [(4096, 4096, 1), (8192, 8192, 1), (8196, 8196, 0), (16384, 16384, 0),
             (4094, 4094, 0), (4, 4, 1), (0, 0, 0), (-4, -4, 0), (4096, 4160, 0),
             (2880, 2880, 1), (3584, 3584, 1)]
    src = [f'#include "{RULES}"', "#include <cstdio>", "int main() {"]
    src.append("  static_assert(dbd::kResidNormMaxCols == 8192, \"coverage\");")
    for n, ld, _ in cases:
        src.append(f'  std::printf("%d\\n", (int)dbd::resid_norm_fits({n}, {ld}));')
    src.append("  return 0;\n}")
    f = tmp_path / "probe.cpp"
    f.write_text("\n".join(src))
    exe = tmp_path / "probe"
    subprocess.run([cxx, "-std=c++17", str(f), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert [int(x) for x in out] == [c[2] for c in cases]


ATTN_SCHEDULE_PROBE = r'''
#include "RULES"
#include <cstdio>
#include <cstdint>
#include <set>
#include <vector>

// Brute-force check of the balanced attention schedule for one set of key counts: the active
// workgroup count P is at most the launched one and at most T; the ranges cut [0, T) into P
// consecutive non-empty pieces; the owner of every chunk is the workgroup whose range
// holds it; the per-sequence workgroup runs that the plan kernel walks give every workgroup
// exactly one start, equal to its range's first chunk; the bisection finds every chunk's
// sequence; launched workgroups and ranges map one to one; the partial slots of all (workgroup, segment) pieces are distinct and below
// P + segments.
static int check(const std::vector<int>& keys, int hd, int kvh, int rows, int launched) {
  const int kch = dbd::attn_chunk_keys(hd), segs = kvh * dbd::attn_row_blocks(rows);
  const int N = (int)keys.size();
  std::vector<int64_t> pref(N + 1, 0);
  for (int n = 0; n < N; ++n) pref[n + 1] = pref[n] + (keys[n] > 0 ? (keys[n] + kch - 1) / kch : 0);
  const int64_t T = pref[N] * segs;
  if (T == 0) return 0;
  const int P = (int)dbd::attn_active_workgroups(launched, T);
  if (P < 1 || P > launched || P > T) return 10;
  // chunk -> (sequence, segment) by walking
  std::vector<int> cseq(T), cseg(T), cchunk(T);
  for (int n = 0; n < N; ++n) {
    const int64_t cn = pref[n + 1] - pref[n];
    for (int s = 0; s < segs; ++s)
      for (int64_t c = 0; c < cn; ++c) {
        const int64_t x = pref[n] * segs + s * cn + c;
        cseq[x] = n; cseg[x] = s; cchunk[x] = (int)c;
      }
  }
  int64_t prev = 0;
  for (int j = 0; j <= P; ++j) {
    const int64_t lo = dbd::attn_range_lo(j, T, P);
    if (lo < prev || (j == 0 && lo != 0) || (j == P && lo != T)) return 1;
    if (j > 0 && lo == prev) return 11;       // an empty range
    prev = lo;
  }
  std::vector<int> pref32(pref.begin(), pref.end());
  for (int64_t x = 0; x < T; ++x) {
    if (dbd::attn_seq_of_chunk(pref32.data(), N, segs, x) != cseq[x]) return 9;
    const int64_t w = dbd::attn_range_owner(x, T, P);
    if (w < 0 || w >= P) return 2;
    if (!(dbd::attn_range_lo(w, T, P) <= x && x < dbd::attn_range_lo(w + 1, T, P))) return 3;
  }
  std::vector<int> starts(P, 0);
  for (int n = 0; n < N; ++n) {
    const int64_t c = pref[n + 1] - pref[n];
    if (c == 0) continue;
    const int64_t S = pref[n] * segs, E = S + c * segs;
    for (int64_t j = dbd::attn_first_range_from(S, T, P); j < dbd::attn_first_range_from(E, T, P); ++j) {
      const int64_t x = dbd::attn_range_lo(j, T, P);
      if (x < S || x >= E) return 4;
      const int64_t off = x - S;
      if (cseq[x] != n || cseg[x] != (int)(off / c) || cchunk[x] != (int)(off % c)) return 5;
      ++starts[j];
    }
  }
  for (int j = 0; j < P; ++j) if (starts[j] != 1) return 6;
  // launched workgroup <-> range: a bijection on [0, launched), ranges [0, P) on P workgroups
  std::vector<int> seen(launched, 0);
  for (int bid = 0; bid < launched; ++bid) {
    const int j = dbd::attn_range_of_bid(bid, launched, P);
    if (j < 0 || j >= launched || seen[j]++) return 12;
    if (dbd::attn_bid_of_range(j, launched, P) != bid) return 13;
  }
  std::set<int64_t> slots;
  for (int j = 0; j < P; ++j) {
    int64_t last = -1;
    for (int64_t x = dbd::attn_range_lo(j, T, P); x < dbd::attn_range_lo(j + 1, T, P); ++x) {
      const int64_t s = (int64_t)cseq[x] * segs + cseg[x];
      if (s == last) continue;
      last = s;
      const int64_t slot = dbd::attn_partial_slot(j, s);
      if (slot < 0 || slot >= dbd::attn_partial_slots(P, (int64_t)N * segs)) return 7;
      if (!slots.insert(slot).second) return 8;
    }
  }
  return 0;
}

int main() {
  unsigned st = 12345u;
  auto rnd = [&](int m) { st = st * 1103515245u + 12345u; return (int)((st >> 8) % (unsigned)m); };
  int bad = 0, cases = 0;
  const int Ps[] = {1, 2, 3, 7, 8, 64, 512, 1000, 4096, 24};
  for (int t = 0; t < 300; ++t) {
    const int N = 1 + rnd(40);
    std::vector<int> keys(N);
    for (auto& k : keys) k = rnd(5) == 0 ? 0 : 1 + rnd(3000);
    const int hd = rnd(2) ? 128 : 64, kvh = 1 + rnd(8), rows = 1 + rnd(300);
    const int P = Ps[t % 10];
    const int rc = check(keys, hd, kvh, rows, P);
    ++cases;
    if (rc) { ++bad; std::printf("case %d: error %d\n", t, rc); }
  }
  std::printf("%d %d\n", cases, bad);
  return bad != 0;
}
'''


def test_attention_schedule_partitions_and_slots(tmp_path):
    """The balanced attention's chunk ranges, owners, plan starts and partial slots, checked by
    brute force over 300 random sets of context lengths (some sequences empty), head sizes 64 and
    128, 1-8 kv heads, 1-300 query rows and 1-4,096 workgroups (more workgroups than chunks
    included)."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    f = tmp_path / "sched.cpp"
    f.write_text(ATTN_SCHEDULE_PROBE.replace("RULES", RULES))
    exe = tmp_path / "sched"
    subprocess.run([cxx, "-std=c++17", "-O2", str(f), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert r.stdout.split()[-2:] == ["300", "0"]
