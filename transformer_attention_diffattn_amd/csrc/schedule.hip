// Host-side choice between the two persistent schedules of the causal
// bf16 prefill (prefill.hip): a model of how each deals the work items to
// the workgroups, and the rule that picks one.  Plain C++ (no device code),
// so that host tests can build it on its own.

namespace diffattn {

// Host model of the two causal schedules of prefill_bf16_kernel (its
// item_at): the largest workgroup total over the mean, an item costing its
// query tile's key count plus about one tile's worth of fixed work (in
// units of query tiles).
static double schedule_spread(int G, int BH, int n_qtiles, bool xcd) {
  const long long n_items = (long long)n_qtiles * BH;
  const long long R_all = n_items / G;
  const bool tail3 = n_items == R_all * G && (R_all & 1) && R_all >= 3 && !(G & 1);
  const long long R3 = R_all - 3;
  auto perm = [](int k, int v, int n) {
    const int h = n / 2, w = v + h - 1;
    return k == 1 ? (w >= n ? w - n : w) : v < h ? n - 1 - 2 * v : v == h ? 0 : 2 * n - 2 * v;
  };
  auto tail_pos = [&](int k, int g) {
    return G % 16 == 0 ? 8 * perm(k, g / 8, G / 8) + perm(k, g % 8, 8) : perm(k, g, G);
  };
  double worst = 0.0, sum = 0.0;
  for (int g = 0; g < G; ++g) {
    double tot = 0.0;
    for (long long r = 0;; ++r) {
      long long i;
      if (xcd) {
        const int W = G / 8;
        const int pos = (r & 1) ? G - 1 - g : g;  // XCD pos % 8, tile pos / 8 of the chunk
        const long long c = r * 8 + pos % 8;
        if (c >= n_items / W) break;
        const long long kk = c / BH;
        i = (kk * W + pos / 8) * BH + (c - kk * BH);
      } else {
        const int alt = (G % BH == 0) ? ((G / BH - 1 - g / BH) * BH + g % BH) : (G - 1 - g);
        int x = (r & 1) ? alt : g;
        if (tail3 && r > R3) x = tail_pos((int)(r - R3), g);
        i = r * G + x;
        if (i >= n_items) break;
      }
      tot += (double)(n_qtiles - i / BH) + 1.0;  // items run longest first
    }
    worst = tot > worst ? tot : worst;
    sum += tot;
  }
  return sum > 0.0 ? worst / (sum / G) : 1.0;
}

// The per-XCD schedule of long causal sequences: a grid of 8 equal XCD shares whose
// W workgroups each take whole chunks of W query tiles of one head (at least
// four chunks per head, so that chunk lengths differ little), unless the
// grid is already a multiple of B*H (then each head keeps its workgroup
// positions, and so its XCD, anyway).  Where whole chunks leave the
// workgroups' totals uneven (an odd number of rounds or a partial last
// one), it runs only while its spread exceeds the item-wise schedule's by
// less than its shared key streams save, taken as 7% per 128 query tiles
// and at most 12% (measured on MI355X: 5-9% at 16K tokens, 8-11% at 32K).
bool prefill_xcd_schedule(long long grid, int BH, int n_qtiles) {
  if (grid % 8 != 0 || grid % BH == 0) return false;
  const long long W = grid / 8;
  if (n_qtiles % W != 0 || n_qtiles < 4 * W) return false;
  const long long n_items = (long long)n_qtiles * BH;
  if (n_items % grid == 0 && (n_items / grid) % 2 == 0) return true;  // even whole rounds: balanced
  if (n_items / grid > 64) return true;  // one round's spread is small against so many (and the model costs)
  const double margin = n_qtiles >= 220 ? 0.12 : 0.07 * (double)n_qtiles / 128.0;
  return schedule_spread((int)grid, BH, n_qtiles, true) <= schedule_spread((int)grid, BH, n_qtiles, false) + margin;
}

}  // namespace diffattn
