// Host check of the grouped GEMM's streaming plan (csrc/gemm_plan.h): replays,
// for one wave, the loads, waits, barriers and LDS reads of gemm_body in their
// program order, and checks
//  (a) at every vmcnt wait, the loads the sub-iteration reads (its weight
//      sub-block and, at even sub-iterations, its K block's activations) are
//      older than the `count` youngest loads (loads complete in issue order);
//  (b) every read finds in its stage the load it expects (no later load into
//      the stage was issued before the read);
//  (c) a load into a stage that several waves read (activation stages; with 8
//      waves also weight stages) comes after a barrier that follows this
//      wave's last read of the stage's previous contents (every wave runs the
//      same sequence, so all of them have read it by then);
//  (d) counts stay below 64 (the vmcnt field).
// Prints one line per failure and "ok <cases>" at the end.
#include <cstdio>
#include <vector>

#include "gemm_plan.h"

using namespace moe::plan;

namespace {

enum Kind { A_LOAD, B_LOAD };

struct Event {
  enum Type { ISSUE, WAIT, BARRIER, READ } type;
  Kind kind;
  long idx;   // block (A) or sub-block (B) index; negative or past the end = dummy
  int stage;
  int loads;  // ISSUE: loads in the group
  int count;  // WAIT: vmcnt
  long need_b, need_a;  // WAIT: sub-block and K block needed (-1: none)
};

int mod(long v, int m) { return (int)(((v % m) + m) % m); }

std::vector<Event> replay(int W, int NA, int NB, int NRH, int KBL, long nkb, int ce, int co) {
  std::vector<Event> ev;
  auto issue_a = [&](long k) { ev.push_back({Event::ISSUE, A_LOAD, k, mod(k, NA), NRH, 0, -1, -1}); };
  auto issue_b = [&](long v) { ev.push_back({Event::ISSUE, B_LOAD, v, mod(v, NB), KBL, 0, -1, -1}); };
  auto wait = [&](int c, long nb, long na) { ev.push_back({Event::WAIT, B_LOAD, 0, 0, 0, c, nb, na}); };
  auto bar = [&]() { ev.push_back({Event::BARRIER, B_LOAD, 0, 0, 0, 0, -1, -1}); };
  auto read = [&](Kind k, long i, int st) { ev.push_back({Event::READ, k, i, st, 0, 0, -1, -1}); };
  const long lead = (NB - 1) > 2 * (NA - 1) ? (NB - 1) : 2 * (NA - 1);
  for (long q = -lead; q < 0; ++q) {
    const long ub = q + NB - 1;
    const bool even = (q & 1) == 0;
    if (W == 8) {
      if (even) issue_a(q / 2 + NA - 1);
      issue_b(ub);
    } else {
      issue_b(ub);
      if (even) issue_a(q / 2 + NA - 1);
    }
  }
  for (long kb = 0; kb < nkb; ++kb) {
    const long u0 = 2 * kb, u1 = 2 * kb + 1;
    if (W == 4) {
      issue_b(u0 + NB - 1);
      wait(ce, u0, kb);
      bar();
      issue_a(kb + NA - 1);
      read(A_LOAD, kb, mod(kb, NA));
      read(B_LOAD, u0, mod(u0, NB));
      issue_b(u1 + NB - 1);
      wait(co, u1, -1);
      read(A_LOAD, kb, mod(kb, NA));  // the second sub-block may read A again
      read(B_LOAD, u1, mod(u1, NB));
    } else {
      wait(ce, u0, kb);
      bar();
      issue_a(kb + NA - 1);
      issue_b(u0 + NB - 1);
      read(A_LOAD, kb, mod(kb, NA));
      read(B_LOAD, u0, mod(u0, NB));
      wait(co, u1, -1);
      bar();
      issue_b(u1 + NB - 1);
      read(A_LOAD, kb, mod(kb, NA));
      read(B_LOAD, u1, mod(u1, NB));
    }
  }
  return ev;
}

int check_v(bool verbose, int W, int NR, int NA, int NB, int NRH, int KBL, long nkb, int ce, int co) {
  const std::vector<Event> ev = replay(W, NA, NB, NRH, KBL, nkb, ce, co);
  int bad = 0;
  auto fail = [&](const char* what, long i) {
    if (verbose && bad < 3)
      std::printf("FAIL W=%d NR=%d NRH=%d nkb=%ld: %s (index %ld)\n", W, NR, NRH, nkb, what, i);
    ++bad;
  };
  if (ce >= 64 || co >= 64) fail("vmcnt count out of range", ce > co ? ce : co);
  // loads issued so far, in order: (kind, idx) per load
  std::vector<std::pair<int, long>> issued;
  // last issue event per stage, last read event per stage, barrier positions
  std::vector<long> last_issue_a(NA, -1), last_issue_b(NB, -1);
  std::vector<long> last_read_a(NA, -1), last_read_b(NB, -1);
  long last_barrier = -1;
  for (long e = 0; e < (long)ev.size(); ++e) {
    const Event& x = ev[e];
    switch (x.type) {
      case Event::ISSUE: {
        const bool shared = x.kind == A_LOAD || W == 8;
        const long prev_read = x.kind == A_LOAD ? last_read_a[x.stage] : last_read_b[x.stage];
        if (shared && prev_read >= 0 && !(last_barrier > prev_read)) fail("stage refilled before a barrier", x.idx);
        for (int l = 0; l < x.loads; ++l) issued.push_back({x.kind, x.idx});
        (x.kind == A_LOAD ? last_issue_a[x.stage] : last_issue_b[x.stage]) = e;
        break;
      }
      case Event::WAIT: {
        // loads that may still be in flight: the `count` youngest
        const long done = (long)issued.size() - x.count;
        auto landed = [&](int kind, long idx) {
          long last = -1;
          for (long i = 0; i < (long)issued.size(); ++i)
            if (issued[i].first == kind && issued[i].second == idx) last = i;
          return last >= 0 && last < done;
        };
        if (!landed(B_LOAD, x.need_b)) fail("weight sub-block not landed at its wait", x.need_b);
        if (x.need_a >= 0 && NRH > 0 && !landed(A_LOAD, x.need_a)) fail("activations not landed at their wait", x.need_a);
        break;
      }
      case Event::BARRIER:
        last_barrier = e;
        break;
      case Event::READ: {
        const long li = x.kind == A_LOAD ? last_issue_a[x.stage] : last_issue_b[x.stage];
        if (x.kind == B_LOAD || NRH > 0) {
          if (li < 0 || ev[li].idx != x.idx) fail("stage holds another block when read", x.idx);
        }
        (x.kind == A_LOAD ? last_read_a[x.stage] : last_read_b[x.stage]) = e;
        break;
      }
    }
  }
  return bad;
}

int check(int W, int NR, int NA, int NB, int NRH, int KBL, long nkb, int ce, int co) {
  return check_v(true, W, NR, NA, NB, NRH, KBL, nkb, ce, co);
}
int check_silent(int W, int NA, int NB, int NRH, int KBL, long nkb, int ce, int co) {
  return check_v(false, W, 0, NA, NB, NRH, KBL, nkb, ce, co);
}

// The counts must pass, and be tight: one more at even or at odd sub-iterations
// lets a read through before its data (checked on a long K, where the steady
// state is reached).  Exception: a wave without activation loads (8 waves,
// one row block) still waits at even sub-iterations as if it had them, which
// is safe but not tight.
int check_tight(int W, int NR, int NA, int NB, int NRH, int KBL, long nkb, int ce, int co) {
  int bad = check(W, NR, NA, NB, NRH, KBL, nkb, ce, co);
  if (nkb >= 16) {
    if (NRH > 0 && check_silent(W, NA, NB, NRH, KBL, nkb, ce + 1, co) == 0) {
      std::printf("FAIL W=%d NR=%d NRH=%d: even count %d is not tight\n", W, NR, NRH, ce);
      ++bad;
    }
    if (check_silent(W, NA, NB, NRH, KBL, nkb, ce, co + 1) == 0) {
      std::printf("FAIL W=%d NR=%d NRH=%d: odd count %d is not tight\n", W, NR, NRH, co);
      ++bad;
    }
  }
  return bad;
}

template <int NR, int LDS = kLdsMax>
int check_nr(long nkb) {
  constexpr int NA = Ring<NR, LDS>::kNA, NB = Ring<NR, LDS>::kNB;
  int bad = 0;
  // 4 waves: a wave owns all NR row blocks, 4 weight loads per sub-block
  bad += check_tight(4, NR, NA, NB, NR, 4, nkb, wait_count<4, NA, NB, NR, 4>(true),
                     wait_count<4, NA, NB, NR, 4>(false));
  // 8 waves: the two waves of a pair own ceil(NR/2) and floor(NR/2) blocks
  constexpr int H0 = (NR + 1) / 2, H1 = NR / 2;
  bad += check_tight(8, NR, NA, NB, H0, 2, nkb, wait_count<8, NA, NB, H0, 2>(true),
                     wait_count<8, NA, NB, H0, 2>(false));
  bad += check_tight(8, NR, NA, NB, H1, 2, nkb, wait_count<8, NA, NB, H1, 2>(true),
                     wait_count<8, NA, NB, H1, 2>(false));
  return bad;
}

}  // namespace

int main() {
  int bad = 0, cases = 0;
  for (long nkb : {1L, 2L, 3L, 4L, 5L, 7L, 16L, 32L, 112L}) {
    bad += check_nr<1>(nkb) + check_nr<2>(nkb) + check_nr<3>(nkb) + check_nr<4>(nkb) +
           check_nr<5>(nkb) + check_nr<6>(nkb) + check_nr<7>(nkb) + check_nr<8>(nkb);
    // the half-LDS plans of tiles that share a CU two by two (up to 4 row blocks)
    bad += check_nr<1, kLdsHalf>(nkb) + check_nr<2, kLdsHalf>(nkb) +
           check_nr<3, kLdsHalf>(nkb) + check_nr<4, kLdsHalf>(nkb);
    cases += 12 * 3;
  }
  if (bad) {
    std::printf("%d failures\n", bad);
    return 1;
  }
  std::printf("ok %d\n", cases);
  return 0;
}
