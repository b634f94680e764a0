// DMA schedule arithmetic of the tiled TQ2 kernel, kept free of HIP so that
// host tests can compile it and replay the issue order.
//
// Per iteration (stage s = 4 rd + ch of round rd) a wave issues, after the
// stage barrier: at ch = wch the weight/scale DMA of round rd + WD (w_issue
// instructions; wch = 1 with two weight slots, 0 with one, whose slot is free
// once round rd's weights are in registers at ch = 3 of the round before),
// then the activation DMA of stage s + XS - 1 (kper instructions).  Before
// the kernel loop it issues the weight DMA of rounds 0 .. WD - 1, then the
// activation DMA of stages 0 .. XS - 2.
#pragma once

namespace tq {

struct RingPlan {
  int xs;  // activation stages in the LDS ring (XS - 1 in flight)
  int wd;  // rounds of weights/scales in the LDS ring
};

// Weight issue stage within a round (see above).
constexpr int w_issue_ch(int wd) { return wd == 1 ? 0 : 1; }

// The deepest ring that fits budget bytes, given the bytes of one activation
// stage and of one round of weights and scales.  xs <= 4 wd - w_issue_ch(wd)
// keeps the weights of round rd + 1 older than the activation DMA of stage
// 4 rd + 3, the stage that reads them.  A fourth activation stage is worth
// more than a second weight slot (N = 8192: M = 128 33.6 -> 31.8 us, M = 256
// 67.3 -> 63.0, M = 32 17.7 -> 17.1; unchanged at N = 28672).
constexpr RingPlan ring_plan(int stage_bytes, int round_bytes, int budget) {
  const int cand[6][2] = {{6, 2}, {5, 2}, {4, 2}, {4, 1}, {3, 2}, {3, 1}};
  for (const auto& c : cand)
    if (c[0] * stage_bytes + c[1] * round_bytes <= budget) return RingPlan{c[0], c[1]};
  return RingPlan{3, 1};
}

// First stage of a round (ch) at whose wait the weights of the next round
// have landed: they were issued at ch = wch of round rd + 1 - wd, and the wait
// of stage s covers every DMA issued up to iteration s - xs + 1.
constexpr int w_ready_ch(int xs, int wd) {
  const int c = 4 * (1 - wd) + w_issue_ch(wd) + xs - 1;
  return c < 0 ? 0 : c;
}

// Instructions a wave may leave outstanding at the wait of stage s = 4 rd + ch
// such that stage s's activation DMA (and round rd + 1's weights at ch = 3)
// have landed: the activation DMAs of the xs - 2 stages after stage s, plus
// the weight DMA of every iteration t = s - xs + 2 .. s - 1 with t % 4 = wch
// (the iteration that issued stage s's DMA issued its weights first).  In
// round 0 only iterations t >= 0 count: stage s's DMA may be a prologue one,
// and the prologue's weight DMAs precede all.  xs <= 6.
constexpr int vm_younger(int xs, int kper, int w_issue, int ch, bool round0, int wch) {
  int n = (xs - 2) * kper;
  for (int j = 1; j <= xs - 2; ++j) {
    const int t = ch - j;  // iteration, relative to the round's first
    if (round0 && t < 0) continue;
    if ((t % 4 + 4) % 4 == wch) n += w_issue;
  }
  return n;
}

}  // namespace tq
