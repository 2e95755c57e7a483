// split.h -- how the streaming kernels cut the flattened token axis into
// workgroup ranges, and where the reduction's per-block pieces go.  Plain
// C++ (no HIP headers): the segment and slot helpers are constexpr, so the
// kernels call them as device code and host tests compile this header alone.
#ifndef SVA_SPLIT_H
#define SVA_SPLIT_H

// The B*H sequences' blocks laid end to end: block bhc (sequence bhc / nb,
// block bhc % nb) holds positions [bhc * Nbp, bhc * Nbp + Nb) of the
// flattened axis; positions Nb .. Nbp - 1 of it hold no token.  Workgroup g
// takes positions [g * L, min((g + 1) * L, total)).
struct SplitArgs {
  long long total;  // flattened positions: blocks * Nbp
  long long L;      // positions per workgroup
  int Nbp;          // a block's length on the flattened axis: Nb, or Nb padded up to a multiple of L
};

constexpr long long kMinTokensPerWG = 256;  // a workgroup's least share of tokens
constexpr long long kAlignSlack = 512;      // see align_split

constexpr long long split_min(long long a, long long b) { return a < b ? a : b; }

// A workgroup's segment that starts at position pos (its range ends at g1):
// block bhc, the segment's end on the flattened axis, and the block-local
// token range [js, je) (js >= je: positions past the block's last token).
struct Segment {
  long long bhc, end;
  int js, je;
};
constexpr Segment segment_at(long long pos, long long g1, const SplitArgs& sp, int Nb) {
  const long long bhc = pos / sp.Nbp;
  const long long end = split_min(g1, (bhc + 1) * (long long)sp.Nbp);
  const int jend = (int)(end - bhc * sp.Nbp);
  return Segment{bhc, end, (int)(pos - bhc * sp.Nbp), jend < Nb ? jend : Nb};
}

// First and last slot of the pieces of block bhc: the piece of workgroup g
// sits at slot g + bhc, so one block's pieces are contiguous (a slot between
// two blocks is unused when a range ends exactly at a block boundary).
constexpr long long block_first_slot(long long bhc, int Nbp, long long L) { return (bhc * Nbp) / L + bhc; }
constexpr long long block_last_slot(long long bhc, int Nbp, long long L) {
  return (bhc * Nbp + Nbp - 1) / L + bhc;
}

// The folded prefix's arrivals: the workgroups holding positions of
// sequence bh are first .. last (seq_first_wg, seq_last_wg); each counts one
// arrival, at its segment that ends the sequence or ends its own range.
constexpr long long seq_end_pos(long long bh, int nb, int Nbp) { return (bh + 1) * nb * (long long)Nbp; }
constexpr long long seq_first_wg(long long bh, int nb, int Nbp, long long L) { return bh * nb * (long long)Nbp / L; }
constexpr long long seq_last_wg(long long bh, int nb, int Nbp, long long L) { return (seq_end_pos(bh, nb, Nbp) - 1) / L; }
constexpr bool arrives(long long seg_end, long long g1, long long bh, int nb, int Nbp) {
  return seg_end >= g1 || seg_end == seq_end_pos(bh, nb, Nbp);
}

// Equal contiguous ranges of the unpadded axis, as many as target_wg (or
// fewer, so that each range has at least kMinTokensPerWG tokens).
inline SplitArgs make_split(long long total, long long target_wg, int* G_out, int Nb) {
  long long G = target_wg;
  const long long g_min_tokens = (total + kMinTokensPerWG - 1) / kMinTokensPerWG;
  if (G > g_min_tokens) G = g_min_tokens;
  if (G < 1) G = 1;
  SplitArgs s;
  s.total = total;
  s.L = (total + G - 1) / G;
  s.Nbp = Nb;
  G = (total + s.L - 1) / s.L;
  *G_out = (int)G;
  return s;
}

// The split of make_split with every range inside one block, when that takes
// at most max_wg workgroups: each of the `blocks` blocks is cut into J equal
// ranges of Lb <= L tokens (its length padded to J * Lb on the flattened
// axis).  A range that crosses a block boundary costs its workgroup a second
// setup (the new block's operands, RoPE rows) and epilogue; on a grid of one
// round that workgroup finishes last.  With `fewer`, when that J needs more
// workgroups than fit, one range fewer per block is taken if it lengthens a
// range by at most kAlignSlack tokens: fewer workgroups, none crossing (480p
// reduction: 224 workgroups of 2,340 tokens instead of 256 of 2,048, 111 of
// which crossed; 27.8 -> 26.4 us).  Splits of several blocks per range stay
// as they are.
inline void align_split(SplitArgs* s, int* G_out, long long blocks, int Nb, long long max_wg, bool fewer = false) {
  if (s->L >= Nb) return;
  long long J = (Nb + s->L - 1) / s->L;
  if (blocks * J > max_wg) {
    if (!fewer) return;
    J = Nb / s->L;
    if (J < 1 || blocks * J > max_wg || (Nb + J - 1) / J > s->L + kAlignSlack) return;
  }
  const long long Lb = (Nb + J - 1) / J;
  s->L = Lb;
  s->Nbp = (int)(J * Lb);
  s->total = blocks * s->Nbp;
  *G_out = (int)(blocks * J);
}

// The forward's two splits, from the workgroups of each kernel that fit at
// once (r_max: reduction, a_max: output pass) and the CU count.  When the
// output pass's minimum of tokens per workgroup, not occupancy, bounds its
// grid (one block of a few thousand tokens per sequence), a multiple of the
// CU count gives every CU the same number of workgroups (304 workgroups on
// 256 CUs left 48 CUs with twice the work of the rest).
inline void plan_forward_splits(long long total, long long blocks, int Nb, long long r_max, long long a_max,
                                long long cus, SplitArgs* red, int* G_red, SplitArgs* app, int* G_app) {
  long long a_target = a_max;
  const long long a_tok = total / kMinTokensPerWG;
  if (a_tok < a_target) a_target = a_tok >= cus ? a_tok / cus * cus : a_tok;
  *red = make_split(total, r_max, G_red, Nb);
  *app = make_split(total, a_target > 0 ? a_target : 1, G_app, Nb);
  align_split(red, G_red, blocks, Nb, r_max, true);
  align_split(app, G_app, blocks, Nb, a_max);
}

#endif  // SVA_SPLIT_H
