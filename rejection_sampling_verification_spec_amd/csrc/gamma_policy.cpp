// gamma_policy.cpp -- host-side policies that choose the next draft length
// (gamma) from the accepted counts the verify step returns.  No GPU code; the
// caller owns the policy state (sv_gamma_policy) and the library keeps none.
//
// Policies, from the page "投機的デコーディングとは：同時リクエストが多いと遅くなる理由"
// (section vLLM は利用者が書く表で、SGLang は実行中に観測した受理の長さで先読み数を変える)
// and the page "LLM推測デコーディング最適化実踐" (section 動的推測戦略):
//   SV_GAMMA_BY_BATCH    a user table of draft lengths per range of concurrent
//                        requests (the documented example: 1-64 -> 3,
//                        65-128 -> 1, 129-512 -> 0), looked up at every step;
//   SV_GAMMA_EMA         per batch-size bucket, an exponential moving average of
//                        the accepted length; next length = round(average) + 1
//                        clamped to [min, max] of the candidate lengths (default
//                        candidates 1, 3, 7); batches of 32 or more use 1;
//   SV_GAMMA_RATE_WINDOW the mean acceptance rate over the last 100 steps;
//                        above 0.85 the length grows by one (up to 8), below 0.65
//                        it shrinks by one (down to 2); it starts at 5.
#include <math.h>
#include <string.h>

#include "specverify.h"

namespace {

int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

int ema_bucket(const sv_gamma_policy *p, int batch) {
  for (int i = 0; i < p->n_buckets; ++i)
    if (batch <= p->bucket_max_batch[i]) return i;
  return -1;
}

}  // namespace

extern "C" {

int spec_gamma_policy_init(sv_gamma_policy *p, int kind) {
  if (!p) return SV_EINVAL;
  memset(p, 0, sizeof *p);
  p->kind = kind;
  switch (kind) {
    case SV_GAMMA_BY_BATCH:
      p->n_ranges = 3;
      p->range_max_batch[0] = 64;
      p->range_gamma[0] = 3;
      p->range_max_batch[1] = 128;
      p->range_gamma[1] = 1;
      p->range_max_batch[2] = 512;
      p->range_gamma[2] = 0;
      return SV_OK;
    case SV_GAMMA_EMA: {
      static const int bounds[] = {1, 2, 4, 8, 16, 31};
      p->n_buckets = 6;
      for (int i = 0; i < 6; ++i) p->bucket_max_batch[i] = bounds[i];
      p->ema_weight = 0.2;
      p->steps_min = 1;
      p->steps_max = 7;
      p->fixed_from_batch = 32;
      p->fixed_steps = 1;
      return SV_OK;
    }
    case SV_GAMMA_RATE_WINDOW:
      p->window = 100;
      p->raise_above = 0.85;
      p->lower_below = 0.65;
      p->gamma_min = 2;
      p->gamma_max = 8;
      p->gamma_current = 5;
      return SV_OK;
    default:
      return SV_EINVAL;
  }
}

int spec_gamma_next(const sv_gamma_policy *p, int batch) {
  if (!p || batch < 1) return SV_EINVAL;
  switch (p->kind) {
    case SV_GAMMA_BY_BATCH: {
      if (p->n_ranges < 1 || p->n_ranges > SV_GAMMA_POLICY_SLOTS) return SV_EINVAL;
      for (int i = 0; i < p->n_ranges; ++i)
        if (batch <= p->range_max_batch[i]) return p->range_gamma[i];
      return p->range_gamma[p->n_ranges - 1];  // past the table: its last entry
    }
    case SV_GAMMA_EMA: {
      if (batch >= p->fixed_from_batch) return p->fixed_steps;
      const int k = ema_bucket(p, batch);
      if (k < 0 || p->ema_count[k] == 0) return p->steps_max;  // nothing observed yet
      return clampi(static_cast<int>(lround(p->ema[k])) + 1, p->steps_min, p->steps_max);
    }
    case SV_GAMMA_RATE_WINDOW:
      return p->gamma_current;
    default:
      return SV_EINVAL;
  }
}

int spec_gamma_observe(sv_gamma_policy *p, const int32_t *accepted_count, int B, int gamma_used) {
  if (!p || !accepted_count || B < 1 || gamma_used < 0) return SV_EINVAL;
  double sum = 0.0;
  for (int b = 0; b < B; ++b) sum += accepted_count[b];
  const double mean = sum / B;
  switch (p->kind) {
    case SV_GAMMA_BY_BATCH:
      return SV_OK;  // the table does not learn
    case SV_GAMMA_EMA: {
      if (B >= p->fixed_from_batch) return SV_OK;
      const int k = ema_bucket(p, B);
      if (k < 0) return SV_OK;
      p->ema[k] = p->ema_count[k] == 0 ? mean : (1.0 - p->ema_weight) * p->ema[k] + p->ema_weight * mean;
      p->ema_count[k] += 1;
      return SV_OK;
    }
    case SV_GAMMA_RATE_WINDOW: {
      if (gamma_used == 0) return SV_OK;  // no drafts, no rate
      if (p->window < 1 || p->window > SV_GAMMA_WINDOW_MAX) return SV_EINVAL;
      const double rate = mean / gamma_used;
      p->history[p->hist_pos] = rate;
      p->hist_pos = (p->hist_pos + 1) % p->window;
      if (p->hist_len < p->window) p->hist_len += 1;
      double avg = 0.0;  // mean over the stored window, oldest first
      for (int i = 0; i < p->hist_len; ++i) {
        const int idx = (p->hist_pos - p->hist_len + i + p->window) % p->window;
        avg += p->history[idx];
      }
      avg /= p->hist_len;
      if (avg > p->raise_above) p->gamma_current = clampi(p->gamma_current + 1, p->gamma_min, p->gamma_max);
      else if (avg < p->lower_below) p->gamma_current = clampi(p->gamma_current - 1, p->gamma_min, p->gamma_max);
      return SV_OK;
    }
    default:
      return SV_EINVAL;
  }
}

}  // extern "C"
