// DMA schedule arithmetic of the tiled TQ2 kernel, kept free of HIP so that
// host tests can compile it and replay the issue order.
//
// Per iteration (stage s = 4 rd + ch of round rd) a wave issues, after the
// stage barrier: at ch = 1 the weight/scale DMA of round rd + WD (w_issue
// instructions), then the activation DMA of stage s + XS - 1 (kper
// instructions).  Before the kernel loop it issues the weight DMA of rounds
// 0 .. WD - 1, then the activation DMA of stages 0 .. XS - 2.
#pragma once

namespace tq {

struct RingPlan {
  int xs;  // activation stages in the LDS ring (XS - 1 in flight)
  int wd;  // rounds of weights/scales in the LDS ring
};

// The deepest ring that fits budget bytes, given the bytes of one activation
// stage and of one round of weights and scales.  xs <= 4 wd - 1 keeps the
// weights of round rd + 1 older than the activation DMA of stage 4 rd + 3,
// the stage that reads them.
constexpr RingPlan ring_plan(int stage_bytes, int round_bytes, int budget) {
  const int cand[5][2] = {{6, 2}, {5, 2}, {4, 2}, {3, 2}, {3, 1}};
  for (const auto& c : cand)
    if (c[0] * stage_bytes + c[1] * round_bytes <= budget) return RingPlan{c[0], c[1]};
  return RingPlan{3, 1};
}

// Instructions a wave may leave outstanding at the wait of stage ch of a round
// such that stage s's activation DMA (and round rd + 1's weights at ch = 3)
// have landed: the activation DMAs of the xs - 2 stages after stage s, plus
// the weight DMA of every ch = 1 iteration that came after stage s's DMA.  From
// round 1 on those are the ch = 1 iterations among the xs - 2 before (xs <= 6).
// In round 0 stage s's DMA is a prologue one (or iteration 0's) whenever
// s - xs + 1 < 1, and the only weight DMA after it is iteration 1's, once
// iteration 1 is past (s >= 2); the prologue's weight DMAs precede all.
constexpr int vm_younger(int xs, int kper, int w_issue, int ch, bool round0) {
  int n = (xs - 2) * kper;
  if (round0) return n + ((ch - xs + 1 < 1 && ch >= 2) ? w_issue : 0);
  for (int j = 1; j <= xs - 2; ++j)
    if (((ch - j) % 4 + 4) % 4 == 1) n += w_issue;
  return n;
}

}  // namespace tq
