// Exact top-k of fp64 scores on one wave or one 256-thread workgroup, in the
// order (score descending, index ascending); shared by the routing (level-1
// and level-2 selection) and the warm tier (least recently used slots).
#pragma once

#include "hga_internal.h"

namespace hga {

// Top-k by one wave, no barriers: the k best of s[0..n) (LDS, fp64; order
// score descending, index ascending) are written ascending by index to out
// (LDS); returns min(k, n).  hist (256 ints), bl and win (n ints each) are
// LDS scratch.  A 256-bin histogram between the min and max score finds the
// bin holding the k-th largest score; every score in a higher bin is kept,
// and the boundary bin is resolved exactly by rank counting.  Counts use a
// DPP scan and ballot / mbcnt.
//   n <= 1024: scores stay in registers (element i in slot i / 64 of lane
//   i % 64); longer lists stream from LDS in the same passes.
struct TopkScratch {
  int* hist;  // 256
  int* bl;    // boundary members, by index
  int* win;   // 1 if the boundary member at that list position is kept
};

__device__ __forceinline__ int topk_bin(double x, double mn, double scale) {
  const double f = (x - mn) * scale;
  const int b = f >= 0.0 ? (int)f : 0;  // monotone in x; NaN -> 0
  return b > 255 ? 255 : b;
}

// Boundary bin and how many of its members are kept, from the histogram.
__device__ __forceinline__ void topk_cut(const int* hist, int k, int* bs, int* need) {
  const int lane = threadIdx.x & 63;
  const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
            h3 = hist[4 * lane + 3];
  const int local = h0 + h1 + h2 + h3;
  const int pre = wave_incl_scan(local);
  const int total = __builtin_amdgcn_readlane(pre, 63);
  const int suf = total - pre + local;  // scores in bins >= 4*lane
  const int above = suf - local;
  int bs_l, ab_l;
  const int c3 = above + h3, c2 = c3 + h2, c1 = c2 + h1;
  if (c3 >= k) { bs_l = 4 * lane + 3; ab_l = above; }
  else if (c2 >= k) { bs_l = 4 * lane + 2; ab_l = c3; }
  else if (c1 >= k) { bs_l = 4 * lane + 1; ab_l = c2; }
  else { bs_l = 4 * lane; ab_l = c1; }
  const int src = __ffsll((long long)__ballot(above < k && k <= suf)) - 1;
  *bs = __builtin_amdgcn_readlane(bs_l, src);
  *need = k - __builtin_amdgcn_readlane(ab_l, src);
}

// Ranks the nb boundary members; win[t] = 1 for the `need` best.
__device__ __forceinline__ void topk_rank(const double* s, int nb, int need, const int* bl, int* win) {
  const int lane = threadIdx.x & 63;
  for (int t = lane; t < nb; t += 64) {
    const int i = bl[t];
    const double si = s[i];
    int r = 0;
    for (int u = 0; u < nb; ++u) {
      const int jx = bl[u];
      const double sj = s[jx];
      r += (sj > si) || (sj == si && jx < i);
    }
    win[t] = r < need;
  }
}

__device__ int wave_topk(const double* s, int n, int k, int* out, const TopkScratch& sc) {
  constexpr int SL = 16;
  const int lane = threadIdx.x & 63;
  if (k <= 0) return 0;
  if (k >= n) {
    for (int i = lane; i < n; i += 64) out[i] = i;
    return n;
  }
  for (int j = 0; j < 4; ++j) sc.hist[4 * lane + j] = 0;
  int cnt = 0;
  if (n <= 64 * SL) {
    double x[SL];
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      const int i = 64 * j + lane;
      x[j] = s[i < n ? i : n - 1];
    }
    double mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      const bool v = 64 * j + lane < n;
      mn = fmin(mn, v ? x[j] : INFINITY);
      mx = fmax(mx, v ? x[j] : -INFINITY);
    }
    mn = wave_ext_d<false>(mn);
    mx = wave_ext_d<true>(mx);
    const double scale = mx > mn ? 256.0 / (mx - mn) : 0.0;
    int bins[SL];
#pragma unroll
    for (int j = 0; j < SL; ++j) bins[j] = 64 * j + lane < n ? topk_bin(x[j], mn, scale) : -1;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < SL; ++j)
      if (bins[j] >= 0) atomicAdd(&sc.hist[bins[j]], 1);
    __builtin_amdgcn_wave_barrier();
    int bs, need;
    topk_cut(sc.hist, k, &bs, &need);
    int nb = 0, bpos[SL];
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      const unsigned long long m = __ballot(bins[j] == bs);
      bpos[j] = nb + lanes_below(m);
      if (bins[j] == bs) sc.bl[bpos[j]] = 64 * j + lane;
      nb += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    topk_rank(s, nb, need, sc.bl, sc.win);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      const bool keep = bins[j] > bs || (bins[j] == bs && sc.win[bpos[j]]);
      const unsigned long long m = __ballot(keep);
      if (keep) out[cnt + lanes_below(m)] = 64 * j + lane;
      cnt += __popcll(m);
    }
  } else {
    double mn = INFINITY, mx = -INFINITY;
    for (int i = lane; i < n; i += 64) {
      mn = fmin(mn, s[i]);
      mx = fmax(mx, s[i]);
    }
    mn = wave_ext_d<false>(mn);
    mx = wave_ext_d<true>(mx);
    const double scale = mx > mn ? 256.0 / (mx - mn) : 0.0;
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < n; i += 64) atomicAdd(&sc.hist[topk_bin(s[i], mn, scale)], 1);
    __builtin_amdgcn_wave_barrier();
    int bs, need;
    topk_cut(sc.hist, k, &bs, &need);
    int nb = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const bool e = i < n && topk_bin(s[i], mn, scale) == bs;
      const unsigned long long m = __ballot(e);
      if (e) sc.bl[nb + lanes_below(m)] = i;
      nb += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    topk_rank(s, nb, need, sc.bl, sc.win);
    __builtin_amdgcn_wave_barrier();
    int seen = 0;  // boundary members met so far, in index order
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const int bi = i < n ? topk_bin(s[i], mn, scale) : -1;
      const unsigned long long mb = __ballot(bi == bs);
      const bool keep = bi > bs || (bi == bs && sc.win[seen + lanes_below(mb)]);
      seen += __popcll(mb);
      const unsigned long long m = __ballot(keep);
      if (keep) out[cnt + lanes_below(m)] = i;
      cnt += __popcll(m);
    }
  }
  return cnt;
}

// Top-k by a whole 256-thread workgroup (n <= 1024, all threads call it with
// the same arguments): the k best of s[0..n) (LDS, fp64; order score
// descending, index ascending) are written ascending by index to out (LDS);
// returns min(k, n) in every thread.  Thread t owns elements 4t..4t+3, so
// the kept indices come out in order from one exclusive scan of per-thread
// counts.  Same histogram / cut / boundary-rank steps as wave_topk, with a
// quarter of the elements per lane.  Scratch: hist (256 ints), bl (n ints),
// red (8 doubles), ints (8 ints).
//
// Every barrier is a round of LDS latency for the whole workgroup, so the
// range of the scores is not reduced here: the threads that write s call
// topk_publish before the barrier that publishes s, which also clears the
// histogram.  The boundary bin is then found by every wave from the same
// histogram, with no barrier between the count and the cut.
struct BlockTopkScratch {
  int* hist;
  int* bl;
  double* red;
  int* ints;
};

// Called by all 256 threads before the barrier that publishes the scores:
// mn / mx are the min and max of the scores this thread wrote (+inf / -inf if
// none).
__device__ __forceinline__ void topk_publish(double mn, double mx, const BlockTopkScratch& sc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  mn = wave_ext_d<false>(mn);
  mx = wave_ext_d<true>(mx);
  if (lane == 0) {
    sc.red[wave] = mn;
    sc.red[4 + wave] = mx;
  }
  sc.hist[tid] = 0;
  if (tid == 0) sc.ints[2] = 0;  // boundary members collected
}

__device__ int block_topk(const double* s, int n, int k, int* out, const BlockTopkScratch& sc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (k <= 0) return 0;
  if (k >= n) {
    for (int i = tid; i < n; i += 256) out[i] = i;
    __syncthreads();
    return n;
  }
  double x[4];
  bool v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * tid + e;
    v[e] = i < n;
    x[e] = s[v[e] ? i : n - 1];
  }
  const double mn = fmin(fmin(sc.red[0], sc.red[1]), fmin(sc.red[2], sc.red[3]));
  const double mx = fmax(fmax(sc.red[4], sc.red[5]), fmax(sc.red[6], sc.red[7]));
  const double scale = mx > mn ? 256.0 / (mx - mn) : 0.0;
  int bin[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bin[e] = v[e] ? topk_bin(x[e], mn, scale) : -1;
    if (bin[e] >= 0) atomicAdd(&sc.hist[bin[e]], 1);
  }
  __syncthreads();
  int bs, need;
  topk_cut(sc.hist, k, &bs, &need);  // the same result in every wave
  const int nb = sc.hist[bs];
  int keep = 0;  // bit e: element 4t+e kept
#pragma unroll
  for (int e = 0; e < 4; ++e) keep |= (bin[e] > bs ? 1 : 0) << e;
  if (nb == need) {  // the whole boundary bin is kept
#pragma unroll
    for (int e = 0; e < 4; ++e) keep |= (bin[e] == bs ? 1 : 0) << e;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (bin[e] == bs) sc.bl[atomicAdd(&sc.ints[2], 1)] = 4 * tid + e;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (bin[e] == bs) {
        const int i = 4 * tid + e;
        int r = 0;
        for (int u = 0; u < nb; u += 4) {  // 4 members per round of LDS reads
          int j[4];
          double sj[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) j[q] = sc.bl[u + q < nb ? u + q : nb - 1];
#pragma unroll
          for (int q = 0; q < 4; ++q) sj[q] = s[j[q]];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            r += (u + q < nb) && ((sj[q] > x[e]) || (sj[q] == x[e] && j[q] < i));
        }
        keep |= (r < need ? 1 : 0) << e;
      }
    }
  }
  // kept indices in ascending order: exclusive scan of per-thread counts
  const int cnt = __popc(keep);
  const int incl = wave_incl_scan(cnt);
  if (lane == 63) sc.ints[4 + wave] = incl;
  __syncthreads();
  int off = incl - cnt;
  for (int w = 0; w < wave; ++w) off += sc.ints[4 + w];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (keep & (1 << e)) out[off++] = 4 * tid + e;
  __syncthreads();
  return k;
}

// ---------------------------------------------------------------------------
// Histogram selection with member slots (the routing's fast selection).
// Scores are binned into kSelBins fine bins between their min and max (a
// monotone map), counted in LDS, and each fine bin records the indices of
// its first kSelSlots members.  The bin bs of the k-th best is found by one
// wave in two short scans (the group of 16 bins holding it, from the lane
// sums of 16 counts each, then its 16 bins); every element in a higher bin is
// kept, and when bs holds more members than the `need` it contributes, they
// are ranked exactly (score descending, index ascending) among the members
// its slots list (or, when the bin overflowed its slots, among all members).
// LDS atomics are the costly step here (they run at a fraction of the LDS
// rate), so each element takes exactly one: its fine count, whose return
// value is its slot.
constexpr int kSelBins = 1024;
constexpr int kSelSlots = 4;

struct SelHist {
  int* fine;  // kSelBins counts, 16-byte aligned
  int* slot;  // kSelBins * kSelSlots member indices, 16-byte aligned
};

template <int NB>
__device__ __forceinline__ int topk_bin_n(double x, double mn, double scale) {
  const double f = (x - mn) * scale;
  const int b = f >= 0.0 ? (int)f : 0;  // monotone in x; NaN -> 0
  return b > NB - 1 ? NB - 1 : b;
}

// Zeroes the counts; threads t = 0, step, 2 step, ... of the caller share it.
__device__ __forceinline__ void sel_clear(const SelHist& h, int t, int step) {
  for (int i = t; i < kSelBins; i += step) h.fine[i] = 0;
}

// The bin bs of the k-th best (count(bins > bs) < k <= count(bins >= bs)),
// need = k - count(bins > bs) and nb = count(bs), from complete counts; run
// by a whole wave (every lane gets the result).  1 <= k <= total.
__device__ __forceinline__ void sel_cut(const SelHist& h, int k, int* bs, int* need, int* nb) {
  static_assert(kSelBins == 64 * 16, "16 bins per lane");
  const int lane = threadIdx.x & 63;
  // lane l sums bins 16 l .. 16 l + 15 (four 16-byte reads)
  const int4* f4 = reinterpret_cast<const int4*>(h.fine + 16 * lane);
  int cc = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int4 v = f4[u];
    cc += (v.x + v.y) + (v.z + v.w);
  }
  const int pre = wave_incl_scan(cc);
  const int total = __builtin_amdgcn_readlane(pre, 63);
  const int suf = total - pre + cc;  // count in bins >= 16 lane
  const int above = suf - cc;        // count in bins >= 16 (lane + 1)
  const int C = __ffsll((long long)__ballot(above < k && k <= suf)) - 1;
  const int above_c = __builtin_amdgcn_readlane(above, C);
  // the 16 bins of C, highest first: lane l of each 16-lane row holds
  // bin 16 C + 15 - l; a row-local inclusive scan counts bins >= it in C
  const int fl = lane & 15;
  const int fc = h.fine[16 * C + 15 - fl];
  int f = fc;
  f += __builtin_amdgcn_update_dpp(0, f, 0x111, 0xF, 0xF, true);
  f += __builtin_amdgcn_update_dpp(0, f, 0x112, 0xF, 0xF, true);
  f += __builtin_amdgcn_update_dpp(0, f, 0x114, 0xF, 0xF, true);
  f += __builtin_amdgcn_update_dpp(0, f, 0x118, 0xF, 0xF, true);
  const int L = __ffsll((long long)(__ballot(above_c + f >= k) & 0xFFFFull)) - 1;
  const int fL = __builtin_amdgcn_readlane(f, L), cL = __builtin_amdgcn_readlane(fc, L);
  *bs = 16 * C + 15 - L;
  *need = k - (above_c + fL - cL);
  *nb = cL;
}

// The slot-listed members of the boundary bin bs (nb <= kSelSlots of them,
// nb >= 1) and their scores, read once for all of a thread's elements: one
// 16-byte slot read, then the nb score reads together (absent slots repeat
// member 0).  vals: scores by element (LDS).
struct SlotMembers {
  int m[kSelSlots];
  double v[kSelSlots];
};
__device__ __forceinline__ SlotMembers sel_slot_members(const SelHist& h, int bs, int nb,
                                                        const double* vals) {
  static_assert(kSelSlots == 4, "one 16-byte slot read");
  const int4 ms = *reinterpret_cast<const int4*>(h.slot + bs * kSelSlots);
  SlotMembers r;
  r.m[0] = ms.x;
  r.m[1] = nb > 1 ? ms.y : ms.x;
  r.m[2] = nb > 2 ? ms.z : ms.x;
  r.m[3] = nb > 3 ? ms.w : ms.x;
#pragma unroll
  for (int u = 0; u < kSelSlots; ++u) r.v[u] = vals[r.m[u]];
  return r;
}

// Rank of element (i, x) of the boundary bin among those members: the
// members scoring higher, or equal with a lower index.
__device__ __forceinline__ int sel_rank_slots(const SlotMembers& sm, int nb, int i, double x) {
  int r = 0;
#pragma unroll
  for (int u = 0; u < kSelSlots; ++u)
    r += (u < nb) && ((sm.v[u] > x) || (sm.v[u] == x && sm.m[u] < i));
  return r;
}

// One level of the selection, run by all 256 threads of the workgroup (the
// routing calls it for both levels, so the second call runs from a warm
// instruction cache).  Thread t holds up to ne (1..4, uniform) elements: x[e]
// with element index id[e] (< 0: no element; elements ne..3 must be absent).  Of the n elements the k best
// are kept (1 <= k < n); mn / mx bound the scores.  The counts (fine) are
// zero on entry (the caller clears them a barrier earlier); slot receives
// the member slots; vals must already hold every element's score at its
// index (the boundary ranking reads it after this routine's barrier); bl /
// nbl (nbl zero on entry) collect the members of a boundary bin that
// overflowed its slots.  Returns bit e set iff element e is kept.
__device__ __noinline__ uint32_t sel_level(double x0, double x1, double x2, double x3, int i0,
                                           int i1, int i2, int i3, int ne, int k, double mn,
                                           double mx, int* fine, int* slot, const double* vals,
                                           int* bl, int* nbl) {
  const SelHist h{fine, slot};  // by pointer: a struct argument would go through scratch
  const double x[4] = {x0, x1, x2, x3};
  const int id[4] = {i0, i1, i2, i3};
  // a monotone map to bins (the scale needs no more than fp32)
  const double scale = mx > mn ? (double)((float)kSelBins / (float)(mx - mn)) : 0.0;
  // the counts of the ne elements go out before any of their results is
  // waited for; an absent element among them adds 0 to a count of its own
  int bin[4], at[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bin[e] = id[e] >= 0 ? topk_bin_n<kSelBins>(x[e], mn, scale) : -1;
    at[e] = kSelSlots;
    if (e < ne)  // uniform
      at[e] = atomicAdd(&h.fine[bin[e] >= 0 ? bin[e] : (4 * threadIdx.x + e) % kSelBins],
                        id[e] >= 0 ? 1 : 0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (id[e] >= 0 && at[e] < kSelSlots) h.slot[bin[e] * kSelSlots + at[e]] = id[e];
  __syncthreads();
  int bs, need, nb;
  sel_cut(h, k, &bs, &need, &nb);
  uint32_t keep = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) keep |= (bin[e] > bs || (bin[e] == bs && nb == need) ? 1u : 0u) << e;
  if (nb == need) return keep;  // uniform
  if (nb <= kSelSlots) {
    const SlotMembers sm = sel_slot_members(h, bs, nb, vals);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (bin[e] == bs && sel_rank_slots(sm, nb, id[e], x[e]) < need) keep |= 1u << e;
    return keep;
  }
  // more members than slots (uniform): collect them all, then rank
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (bin[e] == bs) bl[atomicAdd(nbl, 1)] = id[e];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (bin[e] != bs) continue;
    int r = 0;
    for (int u = 0; u < nb; ++u) {
      const int m = bl[u];
      const double v = vals[m];
      r += (v > x[e]) || (v == x[e] && m < id[e]);
    }
    if (r < need) keep |= 1u << e;
  }
  return keep;
}

}  // namespace hga
