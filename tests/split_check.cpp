// Host check of the streaming kernels' token splits (block_causal_linear_phi_amd/csrc/split.h).
//
// For many shapes and device sizes, the forward's plan (plan_forward_splits)
// is walked the way the kernels walk it -- each workgroup g takes positions
// [g L, min((g + 1) L, total)) as segments from segment_at, the reduction
// writes one piece per segment at slot g + block, the scan reads a block's
// pieces at block_first_slot .. block_last_slot, and the folded prefix
// counts arrivals with `arrives` -- and the following are checked:
//   - every token of every block is taken by exactly one segment (reduction
//     and output pass alike), and segments never leave their block;
//   - the grids stay within the occupancy bounds they were planned for;
//   - every piece's slot lies in the workspace (the largest reduction grid
//     plus one slot a block) and in its block's slot range, and every slot
//     the scan reads for a block holds a piece of that block;
//   - with the folded prefix, each sequence receives exactly one arrival from
//     each workgroup seq_first_wg .. seq_last_wg;
//   - a split that align_split cut block by block has no range that crosses a
//     block boundary (what it is for).
// Prints "ok <shapes>" and exits 0, or prints the first failure and exits 1.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

// SPLIT_H: the header under test (tests/test_split_host.py also builds this
// file against altered copies of it, each of which must fail)
#ifndef SPLIT_H
#define SPLIT_H "../block_causal_linear_phi_amd/csrc/split.h"
#endif
#include SPLIT_H

namespace {

constexpr long long kRedWorkgroupsMax = 1024;  // the library's bound on the reduction grid

int failures = 0;

void fail(const char* what, long long BH, int nb, int Nb, long long a, long long b) {
  if (failures++ < 10)
    std::printf("FAIL %s: BH=%lld nb=%d Nb=%d (%lld, %lld)\n", what, BH, nb, Nb, a, b);
}

// Walks split sp over G workgroups; with pieces, checks the reduction's
// slots and, with fold, the arrivals.  Returns the number of workgroups whose
// range holds tokens of more than one block.
long long walk(const SplitArgs& sp, int G, long long BH, int nb, int Nb, long long max_wg, bool pieces, bool fold) {
  const long long blocks = BH * nb;
  if (G < 1 || G > max_wg) fail("grid bound", BH, nb, Nb, G, max_wg);
  if (sp.Nbp < Nb) fail("padded block shorter than the block", BH, nb, Nb, sp.Nbp, Nb);
  if (sp.total != blocks * sp.Nbp) fail("total", BH, nb, Nb, sp.total, blocks * sp.Nbp);
  if ((long long)G * sp.L < sp.total || (long long)(G - 1) * sp.L >= sp.total)
    fail("grid is not ceil(total / L)", BH, nb, Nb, G, sp.L);
  // next uncovered token of each block (segments of one block come in order)
  std::vector<int> next(blocks, 0);
  const long long slots = kRedWorkgroupsMax + blocks;
  std::vector<long long> owner(pieces ? slots : 0, -1);
  std::vector<long long> arrivals(fold ? BH : 0, 0);
  long long crossing = 0;
  for (long long g = 0; g < G; ++g) {
    const long long g0 = g * sp.L;
    const long long g1 = split_min(g0 + sp.L, sp.total);
    long long pos = g0;
    int with_tokens = 0;
    do {
      const Segment s = segment_at(pos, g1, sp, Nb);
      with_tokens += s.js < s.je;
      if (s.bhc < 0 || s.bhc >= blocks || s.end <= pos || s.end > (s.bhc + 1) * (long long)sp.Nbp ||
          s.js < 0 || s.je > Nb) {
        fail("segment leaves its block", BH, nb, Nb, g, pos);
        break;  // the rest of this range cannot be walked
      }
      if (s.js < s.je) {
        if (s.js != next[s.bhc]) fail("tokens skipped or taken twice", BH, nb, Nb, s.bhc, s.js);
        next[s.bhc] = s.je;
      }
      if (pieces) {
        const long long slot = g + s.bhc;
        if (slot >= slots) fail("slot past the workspace", BH, nb, Nb, slot, slots);
        else {
          if (owner[slot] != -1) fail("slot written twice", BH, nb, Nb, slot, owner[slot]);
          owner[slot] = s.bhc;
        }
        if (slot < block_first_slot(s.bhc, sp.Nbp, sp.L) || slot > block_last_slot(s.bhc, sp.Nbp, sp.L))
          fail("slot outside its block's range", BH, nb, Nb, slot, s.bhc);
      }
      if (fold) {
        const long long bh = s.bhc / nb;
        if (arrives(s.end, g1, bh, nb, sp.Nbp)) {
          if (g < seq_first_wg(bh, nb, sp.Nbp, sp.L) || g > seq_last_wg(bh, nb, sp.Nbp, sp.L))
            fail("arrival from a workgroup outside the sequence", BH, nb, Nb, g, bh);
          ++arrivals[bh];
        }
      }
      pos = s.end;
    } while (pos < g1);
    crossing += with_tokens > 1;
  }
  for (long long b = 0; b < blocks; ++b)
    if (next[b] != Nb) fail("block not fully covered", BH, nb, Nb, b, next[b]);
  if (pieces) {
    for (long long b = 0; b < blocks; ++b)
      for (long long s = block_first_slot(b, sp.Nbp, sp.L); s <= block_last_slot(b, sp.Nbp, sp.L); ++s)
        if (s >= slots || owner[s] != b) fail("the scan reads a slot without this block's piece", BH, nb, Nb, b, s);
  }
  if (fold) {
    for (long long bh = 0; bh < BH; ++bh) {
      const long long want = seq_last_wg(bh, nb, sp.Nbp, sp.L) - seq_first_wg(bh, nb, sp.Nbp, sp.L) + 1;
      if (arrivals[bh] != want) fail("arrivals", BH, nb, Nb, arrivals[bh], want);
    }
  }
  return crossing;
}

struct Device {
  long long r_max, a_max, cus;
};

int check_shape(long long BH, int nb, int Nb, const Device& dv) {
  const long long blocks = BH * nb;
  const long long total = blocks * Nb;
  SplitArgs red, app;
  int G_red = 0, G_app = 0;
  plan_forward_splits(total, blocks, Nb, dv.r_max, dv.a_max, dv.cus, &red, &G_red, &app, &G_app);
  // the reduction's split before alignment: aligned iff align_split changed it
  int G0 = 0;
  const SplitArgs red0 = make_split(total, dv.r_max, &G0, Nb);
  const bool aligned = red.L != red0.L || red.Nbp != Nb;
  const long long crossing = walk(red, G_red, BH, nb, Nb, dv.r_max, true, nb >= 32);
  if (aligned && crossing) fail("aligned split with ranges crossing a block", BH, nb, Nb, crossing, G_red);
  walk(app, G_app, BH, nb, Nb, dv.a_max, false, false);
  return 1;
}

}  // namespace

int main() {
  std::setvbuf(stdout, nullptr, _IONBF, 0);
  // (reduction workgroups that fit, output-pass workgroups that fit, CUs):
  // MI355X (one reduction and three output workgroups a CU), fp32 shapes with
  // more of each, and smaller and larger devices
  const Device devices[] = {{256, 768, 256}, {512, 1024, 256}, {304, 912, 304}, {64, 192, 64}, {1024, 4096, 512}};
  const long long bhs[] = {1, 2, 3, 4, 8, 16, 32, 64};
  const int nbs[] = {1, 2, 3, 7, 20, 32, 33, 80};
  const int Nbs[] = {1, 15, 64, 100, 255, 256, 292, 293, 700, 2001, 4680, 10800, 20000};
  int shapes = 0;
  for (const Device& dv : devices)
    for (long long BH : bhs)
      for (int nb : nbs)
        for (int Nb : Nbs) shapes += check_shape(BH, nb, Nb, dv);
  std::mt19937_64 rng(20261204);
  for (int i = 0; i < 4000; ++i) {
    const Device& dv = devices[rng() % 5];
    const long long BH = 1 + (long long)(rng() % 48);
    const int nb = 1 + (int)(rng() % 90);
    const int Nb = 1 + (int)(rng() % 12000);
    shapes += check_shape(BH, nb, Nb, dv);
  }
  if (failures) {
    std::printf("%d failures over %d shapes\n", failures, shapes);
    return 1;
  }
  std::printf("ok %d\n", shapes);
  return 0;
}
