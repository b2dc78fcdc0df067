// guard.hip -- the adaptive speculation guard (host code only).  Drafting
// pays only while the accepted drafts save more than their verification's
// extra expert loads cost; the pages turn drafting off adaptively for the
// cold-cache case (colibrì README, "Implemented features", native MTP item;
// "Quick start": DRAFT=n).  Per mode, an exponentially weighted average of
// the step cost and a slower one of the tokens per step, whose ratio
// estimates the cost per token; the cheaper mode runs, the other is probed
// periodically.
#include <cmath>

#include "coli_moe.h"


extern "C" {

coli_status coli_spec_guard_init(coli_spec_guard *g, int32_t max_draft, int32_t probe_every,
                                 float ema, float margin) {
  if (!g || max_draft < 1 || probe_every < 2 || !(ema > 0.0f && ema <= 1.0f) ||
      !(margin >= 0.0f) || !std::isfinite(margin))
    return COLI_ERR_INVALID_ARG;
  g->max_draft = max_draft;
  g->probe_every = probe_every;
  g->ema = ema;
  g->margin = margin;
  g->cost_draft = -1.0;
  g->cost_plain = -1.0;
  for (int m = 0; m < 2; ++m) {
    g->sum_cost[m] = 0.0;
    g->sum_tokens[m] = 0.0;
  }
  g->next_draft = max_draft;
  g->since_probe = 0;
  g->steps = 0;
  g->draft_steps = 0;
  g->tokens = 0;
  return COLI_OK;
}

int32_t coli_spec_guard_step(coli_spec_guard *g, int32_t drafted, int32_t accepted,
                             double cost) {
  if (!g || g->max_draft < 1 || g->probe_every < 2 || drafted < 0 || drafted > g->max_draft ||
      accepted < 0 || accepted > drafted || !(cost >= 0.0) || !std::isfinite(cost))
    return -1;
  const int produced = 1 + accepted;
  const int m = drafted > 0 ? 1 : 0;
  // the first sample sets both averages; the tokens' average moves slower
  const bool first = !(g->sum_tokens[m] > 0.0);
  const double w = first ? 1.0 : (double)g->ema;
  const double wn = first ? 1.0 : 0.4 * (double)g->ema;
  g->sum_cost[m] = (1.0 - w) * g->sum_cost[m] + w * cost;
  g->sum_tokens[m] = (1.0 - wn) * g->sum_tokens[m] + wn * produced;
  (m ? g->cost_draft : g->cost_plain) = g->sum_cost[m] / g->sum_tokens[m];
  g->steps += 1;
  g->tokens += produced;
  if (drafted > 0) g->draft_steps += 1;

  // the mode the estimates prefer; with one unmeasured, keep drafting on
  // (the engine's default) until the first probe has measured plain decode
  bool draft = true;
  if (g->cost_draft >= 0.0 && g->cost_plain >= 0.0)
    draft = g->cost_draft <= g->cost_plain * (1.0 + (double)g->margin);
  g->since_probe += 1;
  if (g->since_probe >= g->probe_every) {
    draft = !draft;  // one step in the other mode keeps its estimate current
    g->since_probe = 0;
  }
  g->next_draft = draft ? g->max_draft : 0;
  return g->next_draft;
}

}  // extern "C"
