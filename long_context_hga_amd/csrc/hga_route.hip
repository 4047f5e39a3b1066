// Two-level chunk -> group routing with the deterministic visibility windows.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 2: the current
// query scores a compact table of chunk key summaries (level 1), then the
// group key summaries inside the chosen chunks (level 2); the current chunk,
// the first sink chunks and the most recent local chunks are always visible.
//
// One launch per call.  grid = (tiles of 64 candidate chunks, Hkv, B):
//   1. every workgroup forms the pooled routing query qbar (mean over the
//      KV head's query heads and query tokens of RoPE(q, position), fp64);
//   2. it scores its tile: one 512-byte summary row per chunk, 32 lanes x
//      float4, fp64 dot and cross-lane sum, fp64 score to the workspace;
//   3. the last workgroup of the (sequence, KV head) to arrive selects the
//      level-1 top-k, scores the level-2 groups of the kept chunks, selects
//      the level-2 top-k and writes the ascending group list.
// Top-k: a 256-bin histogram between the min and max score finds the bin
// holding the k-th largest score; every score in a higher bin is kept, and
// the boundary bin is resolved exactly by rank counting with the order
// (score descending, id ascending).  Scores stay fp64 throughout, so the
// kept set equals the fp64 reference wherever its score gap exceeds the
// error of the fp32-stored summaries.
#include "hga_internal.h"

namespace hga {

constexpr int kTile = 64;

struct RouteArgs {
  KCfg cfg;
  RouteLaunch r;
  int n_tiles;
  int max_cand;
};

struct RouteShared {
  double qbar[128];
  double red[8];
  int hist[256];
  int scan[8];
  int bstar, need, bcount, flag;
};

__device__ __forceinline__ double wave_max_d(double x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmax(x, shfl_xor_d(x, m));
  return x;
}
__device__ __forceinline__ double wave_min_d(double x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmin(x, shfl_xor_d(x, m));
  return x;
}

// Flags the k best of s[0..n) (score desc, index asc).  All 256 threads.
__device__ void topk_flags(const double* s, int n, int k, unsigned char* flag, int* blist,
                           RouteShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (k >= n || k <= 0) {
    for (int i = tid; i < n; i += 256) flag[i] = k > 0;
    __syncthreads();
    return;
  }
  double mn = INFINITY, mx = -INFINITY;
  for (int i = tid; i < n; i += 256) {
    mn = fmin(mn, s[i]);
    mx = fmax(mx, s[i]);
  }
  mn = wave_min_d(mn);
  mx = wave_max_d(mx);
  if (lane == 0) {
    sh.red[wave] = mn;
    sh.red[4 + wave] = mx;
  }
  sh.hist[tid] = 0;
  if (tid == 0) sh.bcount = 0;
  __syncthreads();
  mn = fmin(fmin(sh.red[0], sh.red[1]), fmin(sh.red[2], sh.red[3]));
  mx = fmax(fmax(sh.red[4], sh.red[5]), fmax(sh.red[6], sh.red[7]));
  const double scale = mx > mn ? 256.0 / (mx - mn) : 0.0;
  auto bin = [&](double x) {
    double f = (x - mn) * scale;
    int b = f >= 0.0 ? (int)f : 0;  // monotone in x; NaN -> 0
    return b > 255 ? 255 : b;
  };
  for (int i = tid; i < n; i += 256) atomicAdd(&sh.hist[bin(s[i])], 1);
  __syncthreads();
  if (wave == 0) {
    const int h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1];
    const int h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
    const int local = h0 + h1 + h2 + h3;
    int suf = local;  // count in bins >= 4*lane
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += o;
    }
    const int above = suf - local;
    if (above < k && k <= suf) {
      const int c3 = above + h3, c2 = c3 + h2, c1 = c2 + h1;
      int bs, ab;
      if (c3 >= k) { bs = 4 * lane + 3; ab = above; }
      else if (c2 >= k) { bs = 4 * lane + 2; ab = c3; }
      else if (c1 >= k) { bs = 4 * lane + 1; ab = c2; }
      else { bs = 4 * lane; ab = c1; }
      sh.bstar = bs;
      sh.need = k - ab;
    }
  }
  __syncthreads();
  const int bs = sh.bstar, need = sh.need;
  for (int i = tid; i < n; i += 256) {
    const int bi = bin(s[i]);
    flag[i] = bi > bs;
    if (bi == bs) blist[atomicAdd(&sh.bcount, 1)] = i;
  }
  __syncthreads();
  const int m = sh.bcount;
  for (int t = tid; t < m; t += 256) {
    const int i = blist[t];
    const double si = s[i];
    int r = 0;
    for (int u = 0; u < m; ++u) {
      const int jx = blist[u];
      const double sj = s[jx];
      r += (sj > si) || (sj == si && jx < i);
    }
    if (r < need) flag[i] = 1;
  }
  __syncthreads();
}

// Ordered compaction: out[rank] = i for every flagged i, ascending.  Returns
// the count (in every thread).
__device__ int compact_ordered(const unsigned char* flag, int n, int* out, RouteShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + 255) / 256;
  const int b0 = tid * per, b1 = min(n, b0 + per);
  int cnt = 0;
  for (int i = b0; i < b1; ++i) cnt += flag[i];
  int inc = cnt;  // inclusive wave scan
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) sh.scan[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += sh.scan[w];
  const int total = sh.scan[0] + sh.scan[1] + sh.scan[2] + sh.scan[3];
  int pos = base + inc - cnt;
  for (int i = b0; i < b1; ++i)
    if (flag[i]) out[pos++] = i;
  __syncthreads();
  return total;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  constexpr int P = D / 2;
  constexpr int S = 256 / P;
  constexpr int LPR = D / 4;          // lanes per summary row (float4 each)
  constexpr int RPI = 64 / LPR;       // rows per wave instruction
  constexpr int ITER = (kTile / 4) / RPI;
  using T = typename std::conditional<BF16, uint16_t, float>::type;

  __shared__ RouteShared sh;
  __shared__ double qpart[S][P][2];
  extern __shared__ double dyn[];

  const KCfg& c = a.cfg;
  const RouteLaunch& r = a.r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int unit = b * c.hkv + h;
  const int pos0 = r.q_pos0[b];
  const int lq = r.lq;
  const int ct = pos0 / kChunk;
  const Windows w = windows_of(ct, c.n_sink, c.n_local);
  const int n_cand = w.cand_hi - w.cand_lo;
  const bool valid = pos0 >= 0 && (pos0 % kChunk) + lq <= kChunk && w.cand_hi <= r.max_chunks &&
                     n_cand <= a.max_cand;
  if (!valid) {  // uniform over the unit: nobody arrives, the counter stays 0
    if (blockIdx.x == 0 && tid == 0) r.n_sel[unit] = -1;
    return;
  }

  // ---- 1. pooled routing query (fp64)
  {
    const int j = tid % P, sl = tid / P;
    double qa = 0.0, qb = 0.0;
    const T* q = static_cast<const T*>(r.q);
    for (int t = sl; t < lq; t += S) {
      double cs, sn;
      rope_cs((double)(pos0 + t), c.omega[j], &cs, &sn);
      for (int hh = 0; hh < c.hg; ++hh) {
        const size_t row = ((size_t)(b * c.hq + h * c.hg + hh) * lq + t) * D;
        double x, y;
        if constexpr (BF16) {
          x = bf16_to_f(q[row + j]);
          y = bf16_to_f(q[row + j + P]);
        } else {
          x = q[row + j];
          y = q[row + j + P];
        }
        qa += x * cs - y * sn;
        qb += x * sn + y * cs;
      }
    }
    qpart[sl][j][0] = qa;
    qpart[sl][j][1] = qb;
    __syncthreads();
    if (sl == 0) {
      for (int u = 1; u < S; ++u) {
        qa += qpart[u][j][0];
        qb += qpart[u][j][1];
      }
      const double inv = 1.0 / (double)(c.hg * lq);
      sh.qbar[j] = qa * inv;
      sh.qbar[j + P] = qb * inv;
    }
    __syncthreads();
  }

  // ---- 2. level-1 scores of this tile
  const int col = lane % LPR, rin = lane / LPR;
  double qv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) qv[e] = sh.qbar[4 * col + e];
  double* scores = r.scores + (size_t)unit * a.max_cand;
  {
    const int tile0 = blockIdx.x * kTile;
    float4 buf[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int idx = tile0 + wave * (kTile / 4) + it * RPI + rin;
      const int cc = w.cand_lo + idx;
      buf[it] = idx < n_cand ? *reinterpret_cast<const float4*>(
                                   r.chunk_sum + ((size_t)unit * r.max_chunks + cc) * D + 4 * col)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int idx = tile0 + wave * (kTile / 4) + it * RPI + rin;
      double d = (double)buf[it].x * qv[0];
      d = fma((double)buf[it].y, qv[1], d);
      d = fma((double)buf[it].z, qv[2], d);
      d = fma((double)buf[it].w, qv[3], d);
      for (int m = LPR / 2; m >= 1; m >>= 1) d += shfl_xor_d(d, m);
      if (col == 0 && idx < n_cand) {
        const double sc = d * c.inv_sqrt_d;
        scores[idx] = sc;
        if (r.chunk_scores) r.chunk_scores[(size_t)unit * r.max_chunks + w.cand_lo + idx] = sc;
      }
    }
  }

  if (!arrive_last(r.counters + unit, a.n_tiles, &sh.flag)) return;

  // ---- 3. selection (last workgroup of the unit)
  const int n2max = c.topk_c * kGroups;
  const int nmax = a.max_cand > n2max ? a.max_cand : n2max;
  double* s_lds = dyn;
  int* blist = reinterpret_cast<int*>(s_lds + nmax);
  int* sel1 = blist + nmax;
  unsigned char* flag = reinterpret_cast<unsigned char*>(sel1 + nmax);

  for (int i = tid; i < n_cand; i += 256) s_lds[i] = scores[i];
  __syncthreads();
  topk_flags(s_lds, n_cand, c.topk_c, flag, blist, sh);
  const int k1 = compact_ordered(flag, n_cand, sel1, sh);  // candidate indices, ascending

  // level 2: score the G groups of each kept chunk
  const int n2 = k1 * kGroups;
  {
    constexpr int RPP = 256 / LPR;   // rows per pass
    constexpr int U = 8;             // passes in flight
    const int rsub = tid / LPR;
    for (int base = 0; base < n2; base += RPP * U) {
      float4 buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * RPP + rsub;
        if (i < n2) {
          const int gid = (w.cand_lo + sel1[i / kGroups]) * kGroups + i % kGroups;
          buf[u] = *reinterpret_cast<const float4*>(
              r.group_sum + ((size_t)unit * r.max_chunks * kGroups + gid) * D + 4 * col);
        } else {
          buf[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * RPP + rsub;
        double d = (double)buf[u].x * qv[0];
        d = fma((double)buf[u].y, qv[1], d);
        d = fma((double)buf[u].z, qv[2], d);
        d = fma((double)buf[u].w, qv[3], d);
        for (int m = LPR / 2; m >= 1; m >>= 1) d += shfl_xor_d(d, m);
        if (col == 0 && i < n2) s_lds[i] = d * c.inv_sqrt_d;
      }
    }
  }
  __syncthreads();
  topk_flags(s_lds, n2, c.topk_g, flag, blist, sh);
  const int k2 = compact_ordered(flag, n2, blist, sh);  // level-2 indices, ascending = gid order

  // ---- 4. the list: sink | routed | local | current
  const int last = pos0 + lq - 1;
  const int n_head = w.sink_end * kGroups;
  const int n_local = (ct - w.local_begin) * kGroups;
  const int n_cur = last / kGroupTokens - ct * kGroups + 1;
  const int n_sel = n_head + k2 + n_local + n_cur;
  int* out = r.sel + (size_t)unit * r.max_sel;
  for (int i = tid; i < n_sel; i += 256) {
    int gid;
    if (i < n_head) {
      gid = i;
    } else if (i < n_head + k2) {
      const int x = blist[i - n_head];
      gid = (w.cand_lo + sel1[x / kGroups]) * kGroups + x % kGroups;
    } else {
      gid = w.local_begin * kGroups + (i - n_head - k2);
    }
    out[i] = gid;
  }
  if (tid == 0) r.n_sel[unit] = n_sel;
}

size_t route_ws_bytes(const KCfg& cfg, int B, int max_chunks) {
  const int max_cand = max_chunks > cfg.n_sink ? max_chunks - cfg.n_sink : 1;
  return (size_t)B * cfg.hkv * max_cand * sizeof(double);
}

hipError_t launch_route(const KCfg& cfg, const RouteLaunch& r, hipStream_t st) {
  RouteArgs a;
  a.cfg = cfg;
  a.r = r;
  a.max_cand = r.max_chunks > cfg.n_sink ? r.max_chunks - cfg.n_sink : 1;
  a.n_tiles = (a.max_cand + kTile - 1) / kTile;
  const int n2max = cfg.topk_c * kGroups;
  const int nmax = a.max_cand > n2max ? a.max_cand : n2max;
  const size_t lds = (size_t)nmax * (sizeof(double) + 2 * sizeof(int) + 1);
  dim3 grid(a.n_tiles, cfg.hkv, r.B);
  const bool bf = cfg.dtype == HGA_BF16;
  if (cfg.d == 128) {
    if (bf) hipLaunchKernelGGL((route_kernel<128, true>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((route_kernel<128, false>), grid, dim3(256), lds, st, a);
  } else {
    if (bf) hipLaunchKernelGGL((route_kernel<64, true>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((route_kernel<64, false>), grid, dim3(256), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace hga
