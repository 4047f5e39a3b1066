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

// Merge of the splits of one (sequence, KV head, query token): exact
// log-sum-exp combination of the partial (m, l, o) of every non-empty split.
// grid = B*Hkv*lq workgroups of 256 threads; thread t owns 4 consecutive
// outputs (head t*4/D), and issues all its loads (every split's m, l and
// 4 o values) before using any.
template <int D, int HG>
__global__ __launch_bounds__(256) void attend_combine_kernel(AttendArgs args) {
  const KCfg& c = args.cfg;
  const AttendLaunch& a = args.a;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / a.lq, tq = blockIdx.x % a.lq;
  const int b = unit / c.hkv, h = unit % c.hkv;
  const size_t orow0 = ((size_t)(b * c.hq + h * HG) * a.lq + tq) * D;  // head hh: + hh*lq*D
  const int i0 = 4 * tid;  // first output of this thread
  const int hh = i0 / D, e = i0 % D;
  const bool mine = i0 < HG * D;
  // every split's (m, l, 4 o values) of this thread's head is read before the
  // list length is known (splits that did not run are read but not used)
  const int ic = mine ? i0 : 0;
  const int hc = mine ? hh : 0;
  const float* pbase = a.part + (size_t)(unit * a.lq + tq) * args.n_splits * part_floats<D, HG>();
  float pm[kMaxSplits], pl[kMaxSplits];
  float4 po[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    if (sp < args.n_splits) {  // uniform
      const float* pp = pbase + (size_t)sp * part_floats<D, HG>();
      pm[sp] = pp[hc];
      pl[sp] = pp[HG + hc];
      po[sp] = *reinterpret_cast<const float4*>(pp + part_head<HG>() + ic);
    }
  }
  const int pos0 = a.q_pos0[b];
  const int n_sel = a.n_sel[unit];

  bool bad = n_sel < 0 || n_sel > a.max_sel || pos0 < 0 || (pos0 % kChunk) + a.lq > kChunk;
  ListParts lp{0, 0, 0};
  if (!bad) {
    lp = list_parts(n_sel, pos0 + a.lq - 1, pos0, c.n_sink, c.n_local);
    bad = lp.n_routed < 0;
  }
  if (bad) {
    if (mine) {
      const float nan = __builtin_nanf("");
      *reinterpret_cast<float4*>(a.out + orow0 + (size_t)hh * a.lq * D + e) = make_float4(nan, nan, nan, nan);
      if (a.lse && e == 0) a.lse[(size_t)(b * c.hq + h * HG + hh) * a.lq + tq] = nan;
    }
    return;
  }
  if (!mine) return;
  const int n_part = part_count(a.part_sel, lp, n_sel);
  const int n_act = (n_part + kSplitGroups - 1) / kSplitGroups;
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < n_act) M = fmaxf(M, pm[sp]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
      if (sp < n_act) {
        const float wgt = exp2f(pm[sp] - M);
        L = fmaf(wgt, pl[sp], L);
        acc.x = fmaf(wgt, po[sp].x, acc.x);
        acc.y = fmaf(wgt, po[sp].y, acc.y);
        acc.z = fmaf(wgt, po[sp].z, acc.z);
        acc.w = fmaf(wgt, po[sp].w, acc.w);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(a.out + orow0 + (size_t)hh * a.lq * D + e) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse && e == 0)
    a.lse[(size_t)(b * c.hq + h * HG + hh) * a.lq + tq] =
        L > 0.f ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

size_t attend_ws_bytes(const KCfg& cfg, int B, int lq, int max_sel) {
  const int n_splits = (max_sel + kSplitGroups - 1) / kSplitGroups;
  const int pf = ((2 * cfg.hg + 3) / 4 * 4) + cfg.hg * cfg.d;
  return (size_t)B * cfg.hkv * lq * n_splits * pf * sizeof(float);
}

template <int D>
static void launch_combine_d(const AttendArgs& x, dim3 grid, hipStream_t st) {
  switch (x.cfg.hg) {
    case 1: hipLaunchKernelGGL((attend_combine_kernel<D, 1>), grid, dim3(256), 0, st, x); break;
    case 2: hipLaunchKernelGGL((attend_combine_kernel<D, 2>), grid, dim3(256), 0, st, x); break;
    case 4: hipLaunchKernelGGL((attend_combine_kernel<D, 4>), grid, dim3(256), 0, st, x); break;
    default: hipLaunchKernelGGL((attend_combine_kernel<D, 8>), grid, dim3(256), 0, st, x); break;
  }
}

static void launch_combine(const AttendArgs& x, hipStream_t st) {
  const dim3 grid(x.a.B * x.cfg.hkv * x.a.lq);
  if (x.cfg.d == 128) launch_combine_d<128>(x, grid, st);
  else launch_combine_d<64>(x, grid, st);
}

hipError_t launch_attend(const KCfg& cfg, const AttendLaunch& a, hipStream_t st) {
  AttendArgs x;
  x.cfg = cfg;
  x.a = a;
  x.n_splits = (a.max_sel + kSplitGroups - 1) / kSplitGroups;
  if (a.lq >= kPrefillMinLq) launch_prefill(x, st);
  else launch_decode(x, st);
  launch_combine(x, st);
  return hipGetLastError();
}

}  // namespace hga
