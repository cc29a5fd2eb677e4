// governor.cpp -- the speculation cost governor (host C++).
//
// Speculation must never make decoding slower, so a measurement policy sits
// beside the verify loop: it times speculative steps against plain steps at
// run time, parks drafting while it loses and probes again with backoff
// (TensorSharp speculative decoding page, protocol section and the governor
// paragraphs of the small-batch section).  The rules, as the page states
// them and as they are read here:
//   - A probe is a run of speculative steps, each timed as milliseconds per
//     committed token, against the plain steps' milliseconds per token.  A
//     full probe is eight steps; after a losing verdict the re-probe is three.
//   - Four measured speculative steps in a row that accept nothing end a probe
//     early as a loss.  A step that ran the speculative path and drafted
//     nothing (a matchless n-gram lookup) is a speculative sample of one
//     token.
//   - A loss parks drafting: 32 steps first, doubling on every further loss up
//     to 256.  A win restores the first park length and the full probe.
//   - While a win holds, every speculative step is timed; the hold ends as a
//     loss as soon as the last eight speculative steps average a loss against
//     the plain baseline, and every 64 held steps three plain steps refresh the
//     baseline.
//   - Parked steps feed the plain baseline, except the first step after
//     speculation, which pays the switch.
//   - A new request caps what is left of a park at the first park length and
//     forgets the backoff; a loss already seen keeps the re-probe short.
// Readings where the page leaves a number open: the plain baseline is the
// mean milliseconds per token of the last 16 plain samples; a fresh governor
// (and every probe that finds no baseline) first measures three plain steps;
// a verdict compares total time over total tokens of the probe's samples;
// "the last eight average a loss" compares the eight samples' total time per
// token with the baseline the same way.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <new>

#include "../../include/specv.h"

namespace {

enum GovState { G_BASELINE = 0, G_PROBE = 1, G_HOLD = 2, G_PARKED = 3 };

struct Sample {
  double s;
  int tokens;
};

double per_token(const std::deque<Sample>& v, size_t last) {
  double t = 0.0;
  long n = 0;
  const size_t from = v.size() > last ? v.size() - last : 0;
  for (size_t i = from; i < v.size(); ++i) {
    t += v[i].s;
    n += v[i].tokens;
  }
  return n > 0 ? t / (double)n : 0.0;
}

}  // namespace

struct spec_governor {
  spec_governor_params p;
  int state = G_BASELINE;
  int left = 0;             // steps left in the current baseline run, probe or park
  int park_len = 0;         // the next park's length
  bool lost_once = false;   // a loss was seen: re-probes are the short ones
  bool skip_next_plain = false;  // the first plain step after speculation pays the switch
  int zero_run = 0;         // consecutive speculative steps that accepted nothing
  int held = 0;             // steps since the hold began or was last refreshed
  int after_baseline = G_PROBE;  // where a baseline run continues
  std::deque<Sample> plain;  // the plain baseline samples (last 16 kept)
  std::deque<Sample> spec;   // this probe's or hold's speculative samples
  spec_governor_stats st;
};

namespace {

constexpr size_t kPlainWindow = 16;

void start_probe(spec_governor* g) {
  g->spec.clear();
  g->zero_run = 0;
  if (g->plain.empty()) {  // nothing to compare against yet: measure plain steps first
    g->state = G_BASELINE;
    g->left = g->p.probe_plain;
    g->after_baseline = G_PROBE;
    return;
  }
  g->state = G_PROBE;
  g->left = g->lost_once ? g->p.probe_spec_short : g->p.probe_spec;
  g->st.probes++;
}

void park(spec_governor* g) {
  g->st.losses++;
  g->lost_once = true;
  g->state = G_PARKED;
  g->left = g->park_len;
  g->park_len = std::min(2 * g->park_len, g->p.park_max);
  g->spec.clear();
  g->skip_next_plain = true;
}

void win(spec_governor* g) {
  g->st.wins++;
  g->lost_once = false;
  g->park_len = g->p.park_first;
  g->state = G_HOLD;
  g->held = 0;
  g->spec.clear();
}

}  // namespace

extern "C" {

int spec_governor_create(const spec_governor_params* params, spec_governor** out) {
  if (!out) return SPEC_EINVAL;
  *out = nullptr;
  spec_governor_params p;
  if (params) {
    p = *params;
  } else {
    p.probe_spec = 8;
    p.probe_spec_short = 3;
    p.probe_plain = 3;
    p.park_first = 32;
    p.park_max = 256;
    p.zero_accept_exit = 4;
    p.hold_window = 8;
    p.hold_refresh = 64;
  }
  if (p.probe_spec < 1 || p.probe_spec_short < 1 || p.probe_plain < 1 || p.park_first < 1 ||
      p.park_max < p.park_first || p.zero_accept_exit < 1 || p.hold_window < 1 || p.hold_refresh < 1)
    return SPEC_EINVAL;
  spec_governor* g = new (std::nothrow) spec_governor;
  if (!g) return SPEC_ECAPACITY;
  g->p = p;
  memset(&g->st, 0, sizeof(g->st));
  g->park_len = p.park_first;
  start_probe(g);
  *out = g;
  return SPEC_OK;
}

int spec_governor_destroy(spec_governor* g) {
  delete g;
  return SPEC_OK;
}

int spec_governor_should_draft(spec_governor* g) {
  if (!g) return SPEC_EINVAL;
  return (g->state == G_PROBE || g->state == G_HOLD) ? 1 : 0;
}

int spec_governor_record(spec_governor* g, int speculative, int committed, int accepted, double seconds) {
  if (!g || committed < 1 || accepted < 0 || !(seconds >= 0.0)) return SPEC_EINVAL;
  if ((speculative != 0) != (spec_governor_should_draft(g) == 1))
    return SPEC_ESTATE;  // the step did not follow the governor's decision
  const Sample smp{seconds, committed};
  if (!speculative) {
    if (g->skip_next_plain) {
      g->skip_next_plain = false;
    } else {
      g->plain.push_back(smp);
      if (g->plain.size() > kPlainWindow) g->plain.pop_front();
      g->st.plain_samples++;
    }
    if (g->state == G_PARKED) g->st.parked_steps++;
    if (--g->left > 0) return SPEC_OK;
    if (g->state == G_BASELINE && g->after_baseline == G_HOLD) {
      g->state = G_HOLD;  // a refresh of the hold's baseline: back to holding
      g->held = 0;
      return SPEC_OK;
    }
    start_probe(g);
    return SPEC_OK;
  }
  g->st.spec_steps++;
  g->spec.push_back(smp);
  g->zero_run = accepted == 0 ? g->zero_run + 1 : 0;
  const double base = per_token(g->plain, kPlainWindow);
  if (g->state == G_PROBE) {
    if (g->zero_run >= g->p.zero_accept_exit) {
      park(g);
      return SPEC_OK;
    }
    if (--g->left > 0) return SPEC_OK;
    if (per_token(g->spec, g->spec.size()) < base) win(g);
    else park(g);
    return SPEC_OK;
  }
  // holding a win
  if ((int)g->spec.size() >= g->p.hold_window &&
      per_token(g->spec, (size_t)g->p.hold_window) >= base) {
    park(g);
    return SPEC_OK;
  }
  while ((int)g->spec.size() > g->p.hold_window) g->spec.pop_front();
  if (++g->held >= g->p.hold_refresh) {
    g->state = G_BASELINE;  // three plain steps refresh the baseline, all of them samples
    g->left = g->p.probe_plain;
    g->after_baseline = G_HOLD;
    g->skip_next_plain = false;
  }
  return SPEC_OK;
}

int spec_governor_new_request(spec_governor* g) {
  if (!g) return SPEC_EINVAL;
  g->park_len = g->p.park_first;
  if (g->state == G_PARKED && g->left > g->p.park_first) g->left = g->p.park_first;
  return SPEC_OK;
}

int spec_governor_get_stats(spec_governor* g, spec_governor_stats* out) {
  if (!g || !out) return SPEC_EINVAL;
  *out = g->st;
  out->state = g->state;
  out->plain_ms_per_token = 1e3 * per_token(g->plain, kPlainWindow);
  out->spec_ms_per_token = 1e3 * per_token(g->spec, g->spec.size());
  return SPEC_OK;
}

}  // extern "C"
