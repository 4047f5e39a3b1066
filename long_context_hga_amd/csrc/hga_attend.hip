// hga_attend: exact softmax attention over the selected token K/V.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 4: after
// routing, the output is standard softmax attention over the exact token
// K/V of the selected set; no summary value enters it.
//
// Two launches per call: a split kernel on the matrix cores (hga_decode.hip
// for 1..15 query tokens, hga_prefill.hip for 16..64) writes one partial
// (running max m in log2 units, sum l, unnormalised o) per split of 8
// selected groups, query row and head; the merge kernel below combines the
// splits of each (sequence, KV head, query token) exactly (log-sum-exp) and
// writes the fp32 output and the natural-log LSE.
#include "hga_attend_common.h"

namespace hga {

// Merge of the splits of one query row (sequence, KV head, query token,
// head): exact log-sum-exp combination of the partial (m, l, o) of every
// non-empty split.  grid = B*Hkv*lq*Hg workgroups of one wave; lane t owns
// D/64 consecutive outputs and issues all its loads (every split's m, l and
// o values) before using any.
template <int D, int HG>
__global__ __launch_bounds__(64) void attend_combine_kernel(AttendArgs args) {
  constexpr int EPL = D / 64;  // outputs per lane
  using OV = typename std::conditional<EPL == 2, float2, float>::type;
  const KCfg& c = args.cfg;
  const AttendLaunch& a = args.a;
  // every kernel argument used below, read at once (one scalar round trip;
  // rec_splits, not used here, keeps whole the 16-byte argument load it shares
  // with max_sel: left dead, its register was reused by a later load, which
  // then had to wait for the first)
  asm volatile("" ::"s"(c.lists), "s"(c.hq), "s"(c.n_sink), "s"(c.n_local), "s"(a.lq),
               "s"(a.max_sel), "s"(a.part_sel), "s"(a.two_part), "s"(args.n_splits), "s"(a.part),
               "s"(a.out), "s"(a.lse), "s"(a.q_pos0), "s"(a.n_sel), "s"(a.rec_splits));
  const int lane = threadIdx.x;
  const int hh = blockIdx.x % HG, ut = blockIdx.x / HG;  // ut = unit * lq + tq
  const int unit = ut / a.lq, tq = ut % a.lq;
  const int b = unit / c.lists, h = unit % c.lists;
  const size_t orow = ((size_t)(b * c.hq + h * HG + hh) * a.lq + tq) * D + lane * EPL;
  // every split's (m, l, o) is read before the list length is known
  // (splits that did not run are read but not used)
  const float* pbase = a.part + (size_t)ut * args.n_splits * part_floats<D, HG>();
  float pm[kMaxSplits], pl[kMaxSplits];
  OV po[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    if (sp < args.n_splits) {  // uniform
      const float* pp = pbase + (size_t)sp * part_floats<D, HG>();
      pm[sp] = pp[hh];
      pl[sp] = pp[HG + hh];
      po[sp] = *reinterpret_cast<const OV*>(pp + part_head<HG>() + hh * D + lane * EPL);
    }
  }
  const int pos0 = a.q_pos0[b];
  const int n_sel = a.n_sel[unit];

  bool bad = n_sel < 0 || n_sel > a.max_sel || pos0 < 0 || (pos0 % kChunk) + a.lq > kChunk;
  ListParts lp{0, 0, 0};
  if (!bad) {
    lp = list_parts(n_sel, pos0 + a.lq - 1, pos0, c.n_sink, c.n_local);
    // a two-part list longer than the record layout holds (not one hga_route
    // writes) is reported, not truncated
    bad = lp.n_routed < 0 || records_active(a, lp, n_sel) > args.n_splits;
  }
  const size_t lrow = (size_t)(b * c.hq + h * HG + hh) * a.lq + tq;
  if (bad) {
    const float nan = __builtin_nanf("");
    if constexpr (EPL == 2) *reinterpret_cast<float2*>(a.out + orow) = make_float2(nan, nan);
    else a.out[orow] = nan;
    if (a.lse && lane == 0) a.lse[lrow] = nan;
    return;
  }
  const int n_act = records_active(a, lp, n_sel);
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < n_act) M = fmaxf(M, pm[sp]);
  float L = 0.f, ax = 0.f, ay = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
      if (sp < n_act) {
        const float wgt = exp2f(pm[sp] - M);
        L = fmaf(wgt, pl[sp], L);
        if constexpr (EPL == 2) {
          ax = fmaf(wgt, po[sp].x, ax);
          ay = fmaf(wgt, po[sp].y, ay);
        } else {
          ax = fmaf(wgt, po[sp], ax);
        }
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if constexpr (EPL == 2) *reinterpret_cast<float2*>(a.out + orow) = make_float2(ax * inv, ay * inv);
  else a.out[orow] = ax * inv;
  if (a.lse && lane == 0)
    a.lse[lrow] = L > 0.f ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

size_t attend_ws_bytes(const KCfg& cfg, int B, int lq, int max_sel) {
  const int n_splits = (max_sel + kSplitGroups - 1) / kSplitGroups;
  const int pf = ((2 * cfg.lhg + 3) / 4 * 4) + cfg.lhg * cfg.d;
  return (size_t)B * cfg.lists * lq * n_splits * pf * sizeof(float);
}

template <int D>
static void launch_combine_d(const AttendArgs& x, dim3 grid, hipStream_t st) {
  switch (x.cfg.lhg) {
    case 1: hipLaunchKernelGGL((attend_combine_kernel<D, 1>), grid, dim3(64), 0, st, x); break;
    case 2: hipLaunchKernelGGL((attend_combine_kernel<D, 2>), grid, dim3(64), 0, st, x); break;
    case 4: hipLaunchKernelGGL((attend_combine_kernel<D, 4>), grid, dim3(64), 0, st, x); break;
    default: hipLaunchKernelGGL((attend_combine_kernel<D, 8>), grid, dim3(64), 0, st, x); break;
  }
}

static void launch_combine(const AttendArgs& x, hipStream_t st) {
  const dim3 grid(x.a.B * x.cfg.lists * x.a.lq * x.cfg.lhg);
  if (x.cfg.d == 128) launch_combine_d<128>(x, grid, st);
  else launch_combine_d<64>(x, grid, st);
}

static AttendArgs attend_args(const KCfg& cfg, const AttendLaunch& a) {
  AttendArgs x;
  x.cfg = cfg;
  x.a = a;
  x.grid_splits = (a.max_sel + kSplitGroups - 1) / kSplitGroups;
  x.n_splits = a.rec_splits > 0 ? a.rec_splits : x.grid_splits;
  return x;
}

hipError_t launch_attend_split(const KCfg& cfg, const AttendLaunch& a, hipStream_t st) {
  const AttendArgs x = attend_args(cfg, a);
  if (a.lq >= kPrefillMinLq) launch_prefill(x, st);
  else launch_decode(x, st);
  return hipGetLastError();
}

hipError_t launch_tiered_front(const KCfg& cfg, const AttendLaunch& win, const GatherArgs& g,
                               int n_items, hipStream_t st) {
  const AttendArgs x = attend_args(cfg, win);
  // the window part holds at most the sink, local and current chunks' groups
  const int max_win = (cfg.n_sink + cfg.n_local + 1) * kGroups;
  const int ws = (max_win + kSplitGroups - 1) / kSplitGroups;
  launch_tier_front(x, ws < x.grid_splits ? ws : x.grid_splits, g, n_items, st);
  return hipGetLastError();
}

hipError_t launch_attend_merge(const KCfg& cfg, const AttendLaunch& a, hipStream_t st) {
  launch_combine(attend_args(cfg, a), st);
  return hipGetLastError();
}

hipError_t launch_attend(const KCfg& cfg, const AttendLaunch& a, hipStream_t st) {
  const AttendArgs x = attend_args(cfg, a);
  if (a.lq >= kPrefillMinLq) launch_prefill(x, st);
  else launch_decode(x, st);
  launch_combine(x, st);
  return hipGetLastError();
}

}  // namespace hga
