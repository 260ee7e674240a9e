// Test-only planner overrides (include/st_testing.h).  The planners read the
// installed plan; its defaults are the planners' own choices.
#include "st_internal.h"
#include "st_testing.h"

namespace {
st::TestingPlan g_plan;
}

const st::TestingPlan& st::testing_plan() { return g_plan; }

extern "C" int st_testing_set_plan(const st_testing_plan* p) {
  if (!p) {
    g_plan = st::TestingPlan{};
    return ST_OK;
  }
  if (p->attn_shape < -1 || p->attn_shape > 6 || p->attn_target_wg < 0 ||
      p->attn_split_keys < 0 || p->linear_ksplit < 0 ||
      (p->linear_stages != 0 && p->linear_stages != 4 && p->linear_stages != 8) ||
      p->attn_balance < 0 || p->attn_balance > 2 || p->step_serial < 0 || p->step_serial > 1)
    return ST_E_INVALID;
  g_plan = st::TestingPlan{p->attn_shape,    p->attn_target_wg, p->attn_split_keys,
                           p->linear_ksplit, p->linear_stages,  p->attn_balance,
                           p->step_serial};
  return ST_OK;
}
