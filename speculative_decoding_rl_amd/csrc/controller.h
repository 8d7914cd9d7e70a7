// Roofline SD on/off toggle and acceptance-aware draft length (host only).
//
// EfficientRollout, "关键模块" item 2: decode latency is modelled with a
// roofline; speculation is turned on only when the shrinking active batch
// leaves decode memory-bound (idle compute absorbs the parallel verify), and
// off when a large batch is compute-bound.  "局限": the compute/memory
// boundary is calibrated per GPU.  Item 3: the draft length follows the recent
// acceptance rate.  TLT reading notes section 2: enable below an active-request
// threshold and choose draft depth per batch size.  History Tree Dynamic RL
// section 2.2: EMA coefficient 0.3, switch margin 1.02.
//
// Model (gamma = 0 is autoregressive decoding, so one argmax covers the toggle
// and the draft length):
//   E[n](a, g)   = (1 - a^(g+1)) / (1 - a)
//   T(bytes, fl) = t_fwd + (rows - 1) t_row + max(bytes / BW, fl / FLOPS),
//   rows = B (AR, draft) or B (g+1) (verify), t_row = t_row_draft / t_row_target:
//   what the GPU's forwards take beyond the roofline per further row
//   AR:     bytes = wb P + B C kvb + B kvb + 4 B V,   fl = 2 P B + 4 B C hq hd L
//   draft:  bytes = bq P + B C kvb + B kvb + 4 B V,   fl = 2 P B + 4 B C hq hd L
//   verify: bytes = wb P + B C kvb + B (g+1) kvb + 4 B (g+1) V,
//           fl = 2 P B (g+1) + 4 B (g+1) C hq hd L
//   score(0) = B / T_AR,  score(g) = B E[n] / (g T_draft + T_verify)
// pick the argmax over {0} U [g_min, g_max] (ties to the smaller g) and keep
// the current choice unless the best beats it by the margin.
#pragma once

#include <algorithm>
#include <cmath>

namespace er {

struct CostModel {
  int n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  double w_bytes, q_bytes, kv_bytes_el;
  double bw, flops, t_fwd;
  double t_row_draft = 0.0, t_row_target = 0.0;

  double p_lin() const {
    const double d = d_model, hq = n_q_heads, hkv = n_kv_heads, hd = head_dim, F = ffn;
    const double per = d * (hq + 2 * hkv) * hd + hq * hd * d + 2 * F * d + F * d;
    return n_layers * per + (double)vocab * d;
  }
  double kvb() const { return (double)n_layers * 2 * n_kv_heads * head_dim * kv_bytes_el; }
};

inline double expected_tokens(double alpha, int gamma) {
  if (gamma <= 0) return 1.0;
  if (alpha >= 1.0) return gamma + 1.0;
  return (1.0 - std::pow(alpha, gamma + 1)) / (1.0 - alpha);
}

inline double fwd_time(const CostModel& m, double bytes, double fl, double extra) {
  return m.t_fwd + extra + std::max(bytes / m.bw, fl / m.flops);
}

inline double ar_time(const CostModel& m, int B, double C) {
  const double P = m.p_lin(), kvb = m.kvb();
  const double by = m.w_bytes * P + B * C * kvb + B * kvb + (double)B * m.vocab * 4.0;
  const double fl = 2.0 * P * B + 4.0 * B * C * m.n_q_heads * m.head_dim * m.n_layers;
  return fwd_time(m, by, fl, m.t_row_target * (B - 1));
}

inline double sd_time(const CostModel& m, int B, double C, int g) {
  const double P = m.p_lin(), kvb = m.kvb();
  const double att = 4.0 * C * m.n_q_heads * m.head_dim * m.n_layers;
  const double d_by = m.q_bytes * P + B * C * kvb + B * kvb + (double)B * m.vocab * 4.0;
  const double d_fl = 2.0 * P * B + B * att;
  const double v_by = m.w_bytes * P + B * C * kvb + (double)B * (g + 1) * kvb + (double)B * (g + 1) * m.vocab * 4.0;
  const double v_fl = 2.0 * P * B * (g + 1) + (double)B * (g + 1) * att;
  return g * fwd_time(m, d_by, d_fl, m.t_row_draft * (B - 1)) +
         fwd_time(m, v_by, v_fl, m.t_row_target * ((double)B * (g + 1) - 1));
}

inline double score(const CostModel& m, int B, double C, double alpha, int g) {
  if (g == 0) return B / ar_time(m, B, C);
  return B * expected_tokens(alpha, g) / sd_time(m, B, C, g);
}

// g_lo..g_hi is the speculative range; allow_ar adds g = 0.
inline int choose(const CostModel& m, int B, double C, double alpha, int g_lo, int g_hi, bool allow_ar, int current,
                  double margin) {
  int best = -1;
  double best_s = -1.0;
  auto consider = [&](int g) {
    const double s = score(m, B, C, alpha, g);
    if (s > best_s) { best = g; best_s = s; }
  };
  if (allow_ar) consider(0);
  for (int g = g_lo; g <= g_hi; ++g) consider(g);
  const bool cur_ok = (current == 0 && allow_ar) || (current >= g_lo && current <= g_hi);
  if (cur_ok && current != best && best_s <= margin * score(m, B, C, alpha, current)) return current;
  return best;
}

// Trials-based acceptance of one step: trials = a + 1 after a rejection, g
// after a full acceptance.
struct AlphaAcc {
  long num = 0, den = 0;
  void add(int accepted, int gamma) {
    num += accepted;
    den += accepted < gamma ? accepted + 1 : gamma;
  }
  double value() const { return den > 0 ? (double)num / (double)den : 0.0; }
};

inline double ema(double prev, double sample, double beta) { return (1.0 - beta) * prev + beta * sample; }

// Acceptance probes of the roofline policy.  The acceptance estimate only
// moves on speculative steps; while the policy keeps choosing AR in a regime
// where the initial estimate would make speculation pay, every probe_every-th
// consecutive AR choice becomes one speculative step (the recorded choice stays
// AR).  The gap starts at kProbeFirst and doubles, up to kProbeMax, after each
// probe; a speculative choice resets it.  The pages do not say how the
// estimate is refreshed while speculation is off; this is the reading used.
constexpr int kProbeFirst = 32;
constexpr int kProbeMax = 1024;

struct PlanState {
  int choice = -1;       // last recorded choice (0 = AR), -1 none yet
  int ar_streak = 0;     // consecutive AR choices since the last probe or speculative choice
  int probe_every = 0;   // current gap (0: kProbeFirst)
};

// One step of the roofline policy (allow_ar: the roofline toggle may choose
// AR; false forces speculation).  Returns the gamma to run (0 = AR).
inline int plan_step(const CostModel& m, PlanState& s, bool allow_ar, int B, double C, double alpha_ema,
                     double alpha_init, int g_lo, int g_hi, double margin) {
  const int g = choose(m, B, C, alpha_ema, g_lo, g_hi, allow_ar, s.choice, margin);
  s.choice = g;
  if (g > 0 || !allow_ar) {
    s.ar_streak = 0;
    if (g > 0) s.probe_every = kProbeFirst;
    return g;
  }
  if (s.probe_every <= 0) s.probe_every = kProbeFirst;
  if (++s.ar_streak < s.probe_every) return 0;
  s.ar_streak = 0;
  if (choose(m, B, C, alpha_init, g_lo, g_hi, true, -1, 1.0) == 0) return 0;
  s.probe_every = std::min(2 * s.probe_every, kProbeMax);
  return choose(m, B, C, alpha_ema, g_lo, g_hi, false, -1, 1.0);
}

}  // namespace er
