// Two-level chunk -> group routing with the deterministic visibility windows.
//
// HGA technical summary (gist.science), "Kernmechanisme" item 2: the current
// query scores a compact table of chunk key summaries (level 1), then the
// group key summaries inside the chosen chunks (level 2); the current chunk,
// the first sink chunks and the most recent local chunks are always visible.
//
// Two launches per call.
//  route_tiles: grid = (tiles of 64 candidate chunks, Hkv, B), 256 threads.
//    Each workgroup forms the pooled routing query qbar (mean over the KV
//    head's query heads and query tokens of RoPE(q, position), fp64) and
//    scores its tile: a 512-byte summary row is read by 8 lanes (4 x 16 B
//    each, one wave instruction covering 8 rows), fp64 dot, fp64 DPP sum over
//    the 8 lanes, fp64 score to the workspace.  Tile 0 also stores qbar.
//  route_select: one workgroup per (sequence, KV head).  Level-1 top-k over
//    the scores, level-2 scores of the G groups of every kept chunk (all row
//    loads in flight at once), level-2 top-k, and the ascending group list.
//    The kernel boundary makes the first launch's scores visible to the
//    second with plain loads.
// Top-k: a 256-bin histogram between the min and max score finds the bin
// holding the k-th largest score; every score in a higher bin is kept, and
// the boundary bin is resolved exactly by rank counting with the order
// (score descending, id ascending).  Scores stay fp64 throughout, so the
// kept set equals the fp64 reference wherever its score gap exceeds the
// error of the fp32-stored summaries.
#include "hga_internal.h"

namespace hga {

constexpr int kTile = 64;       // candidate chunks per tile workgroup
constexpr int kLanesPerRow = 8; // lanes per summary row

struct RouteArgs {
  KCfg cfg;
  RouteLaunch r;
  int max_cand;
};

__device__ __forceinline__ double wave_max_d(double x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmax(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ double wave_min_d(double x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmin(x, __shfl_xor(x, m, 64));
  return x;
}

struct SelShared {
  double red[8];
  int hist[256];
  int scan[8];
  int bstar, need, bcount;
};

// Flags the k best of s[0..n) (score desc, index asc).  All 256 threads.
__device__ void topk_flags(const double* s, int n, int k, unsigned char* flag, int* blist,
                           SelShared& sh) {
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
__device__ int compact_ordered(const unsigned char* flag, int n, int* out, SelShared& sh) {
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

// Position and candidate range of a unit; false if the query position is
// unusable (negative, query tokens spanning two chunks, or candidates whose
// summaries lie beyond the table).
__device__ __forceinline__ bool route_geometry(const KCfg& c, const RouteLaunch& r, int max_cand,
                                               int b, int* pos0, Windows* w) {
  *pos0 = r.q_pos0[b];
  *w = windows_of(*pos0 / kChunk, c.n_sink, c.n_local);
  return *pos0 >= 0 && (*pos0 % kChunk) + r.lq <= kChunk && w->cand_hi <= r.max_chunks &&
         w->cand_hi - w->cand_lo <= max_cand;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void route_tiles_kernel(RouteArgs a) {
  constexpr int P = D / 2;
  constexpr int S = 256 / P;                 // query-token slices
  constexpr int NV = D / 32;                 // float4 per lane per row
  constexpr int RPI = 64 / kLanesPerRow;     // rows per wave instruction
  constexpr int ITER = (kTile / 4) / RPI;    // row passes per wave
  using T = typename std::conditional<BF16, uint16_t, float>::type;

  __shared__ double qpart[S][P][2];
  __shared__ double qbar[D];

  const KCfg& c = a.cfg;
  const RouteLaunch& r = a.r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int unit = b * c.hkv + h;
  const int lq = r.lq;
  int pos0;
  Windows w;
  if (!route_geometry(c, r, a.max_cand, b, &pos0, &w)) return;  // route_select reports it
  const int n_cand = w.cand_hi - w.cand_lo;
  const int tile0 = blockIdx.x * kTile;
  if (tile0 >= n_cand && blockIdx.x != 0) return;  // tile 0 always stores qbar

  // ---- loads: this thread's raw query pairs (first query token of its
  // slice) first, then the tile's summary rows.  Rows past the candidates
  // are read from a clamped in-range row (so every load issues together) and
  // ignored.
  const int j = tid % P, sl = tid / P;
  const T* q = static_cast<const T*>(r.q);
  const double wj = c.omega[j];
  T xa[8], xb[8];
  {
    const int t0 = sl < lq ? sl : lq - 1;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      const int hc = hh < c.hg ? hh : c.hg - 1;
      const size_t row = ((size_t)(b * c.hq + h * c.hg + hc) * lq + t0) * D;
      xa[hh] = q[row + j];
      xb[hh] = q[row + j + P];
    }
  }
  const int sub = lane % kLanesPerRow, rin = lane / kLanesPerRow;
  float4 buf[ITER][NV];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    int idx = tile0 + wave * (kTile / 4) + it * RPI + rin;
    idx = idx < n_cand ? w.cand_lo + idx : (n_cand > 0 ? w.cand_hi - 1 : 0);
    const float4* rowp =
        reinterpret_cast<const float4*>(r.chunk_sum + ((size_t)unit * r.max_chunks + idx) * D);
#pragma unroll
    for (int v = 0; v < NV; ++v) buf[it][v] = rowp[v * kLanesPerRow + sub];
  }

  // ---- pooled routing query (fp64): thread (j, slice) rotates pair j of
  // every query head of this KV head for the query tokens of its slice
  {
    double qa = 0.0, qb = 0.0;
    for (int t = sl; t < lq; t += S) {
      if (t != sl) {  // later query tokens (prefill): load them here
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
          const int hc = hh < c.hg ? hh : c.hg - 1;
          const size_t row = ((size_t)(b * c.hq + h * c.hg + hc) * lq + t) * D;
          xa[hh] = q[row + j];
          xb[hh] = q[row + j + P];
        }
      }
      double cs, sn;
      rope_cs((double)(pos0 + t), wj, &cs, &sn);
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) {
        if (hh < c.hg) {
          double x, y;
          if constexpr (BF16) {
            x = bf16_to_f(xa[hh]);
            y = bf16_to_f(xb[hh]);
          } else {
            x = xa[hh];
            y = xb[hh];
          }
          qa += x * cs - y * sn;
          qb += x * sn + y * cs;
        }
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
      qbar[j] = qa * inv;
      qbar[j + P] = qb * inv;
      if (blockIdx.x == 0) {
        r.qbar[(size_t)unit * D + j] = qa * inv;
        r.qbar[(size_t)unit * D + j + P] = qb * inv;
      }
    }
    __syncthreads();
  }

  // ---- level-1 scores of this tile
#pragma unroll
  for (int it = 0; it < ITER; ++it)
#pragma unroll
    for (int v = 0; v < NV; ++v) hold(buf[it][v]);
  double qv[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[v][e] = qbar[4 * (v * kLanesPerRow + sub) + e];
  double* scores = r.scores + (size_t)unit * a.max_cand;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = tile0 + wave * (kTile / 4) + it * RPI + rin;
    double d = 0.0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      d = fma((double)buf[it][v].x, qv[v][0], d);
      d = fma((double)buf[it][v].y, qv[v][1], d);
      d = fma((double)buf[it][v].z, qv[v][2], d);
      d = fma((double)buf[it][v].w, qv[v][3], d);
    }
    d = group8_sum_d(d);
    if (sub == 0 && idx < n_cand) {
      const double sc = d * c.inv_sqrt_d;
      scores[idx] = sc;
      if (r.chunk_scores) r.chunk_scores[(size_t)unit * r.max_chunks + w.cand_lo + idx] = sc;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a) {
  constexpr int NV = D / 32;
  constexpr int RPP = 256 / kLanesPerRow;  // rows per pass of the workgroup
  constexpr int U = 8;                     // passes in flight
  __shared__ SelShared sh;
  extern __shared__ double dyn[];

  const KCfg& c = a.cfg;
  const RouteLaunch& r = a.r;
  const int tid = threadIdx.x, lane = tid & 63;
  const int h = blockIdx.x, b = blockIdx.y;
  const int unit = b * c.hkv + h;
  int pos0;
  Windows w;
  if (!route_geometry(c, r, a.max_cand, b, &pos0, &w)) {
    if (tid == 0) r.n_sel[unit] = -1;
    return;
  }
  const int n_cand = w.cand_hi - w.cand_lo;
  const int ct = pos0 / kChunk;

  const int n2max = c.topk_c * kGroups;
  const int nmax = a.max_cand > n2max ? a.max_cand : n2max;
  double* s_lds = dyn;
  int* blist = reinterpret_cast<int*>(s_lds + nmax);
  int* sel1 = blist + nmax;
  unsigned char* flag = reinterpret_cast<unsigned char*>(sel1 + nmax);

  // qbar slice of this lane (for level 2) and the level-1 scores: all loads
  // first
  const int sub = lane % kLanesPerRow;
  double qv[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      qv[v][e] = r.qbar[(size_t)unit * D + 4 * (v * kLanesPerRow + sub) + e];
  const double* scores = r.scores + (size_t)unit * a.max_cand;
  for (int i0 = 0; i0 < n_cand; i0 += 4 * 256) {
    double v4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 256 + tid;
      v4[u] = scores[i < n_cand ? i : n_cand - 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < n_cand) s_lds[i] = v4[u];
    }
  }
  __syncthreads();
  topk_flags(s_lds, n_cand, c.topk_c, flag, blist, sh);
  const int k1 = compact_ordered(flag, n_cand, sel1, sh);  // candidate indices, ascending

  // level 2: the G groups of each kept chunk
  const int n2 = k1 * kGroups;
  const int rsub = tid / kLanesPerRow;
  for (int base = 0; base < n2; base += RPP * U) {
    float4 gb[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int i = base + u * RPP + rsub;
      i = i < n2 ? i : n2 - 1;  // clamped: every load issues, extras ignored
      const int gid = (w.cand_lo + sel1[i / kGroups]) * kGroups + i % kGroups;
      const float4* rowp = reinterpret_cast<const float4*>(
          r.group_sum + ((size_t)unit * r.max_chunks * kGroups + gid) * D);
#pragma unroll
      for (int v = 0; v < NV; ++v) gb[u][v] = rowp[v * kLanesPerRow + sub];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * RPP + rsub;
      double d = 0.0;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        d = fma((double)gb[u][v].x, qv[v][0], d);
        d = fma((double)gb[u][v].y, qv[v][1], d);
        d = fma((double)gb[u][v].z, qv[v][2], d);
        d = fma((double)gb[u][v].w, qv[v][3], d);
      }
      d = group8_sum_d(d);
      if (sub == 0 && i < n2) s_lds[i] = d * c.inv_sqrt_d;
    }
  }
  __syncthreads();
  topk_flags(s_lds, n2, c.topk_g, flag, blist, sh);
  const int k2 = compact_ordered(flag, n2, blist, sh);  // level-2 indices, ascending = gid order

  // the list: sink | routed | local | current
  const int last = pos0 + r.lq - 1;
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

static int max_cand_of(const KCfg& cfg, int max_chunks) {
  return max_chunks > cfg.n_sink ? max_chunks - cfg.n_sink : 1;
}

size_t route_ws_bytes(const KCfg& cfg, int B, int max_chunks) {
  return (size_t)B * cfg.hkv * (max_cand_of(cfg, max_chunks) + cfg.d) * sizeof(double);
}

size_t route_select_lds(const KCfg& cfg, int max_chunks) {
  const int max_cand = max_cand_of(cfg, max_chunks);
  const int n2 = cfg.topk_c * kGroups;
  return (size_t)(max_cand > n2 ? max_cand : n2) * (sizeof(double) + 2 * sizeof(int) + 1);
}

hipError_t launch_route(const KCfg& cfg, const RouteLaunch& r, hipStream_t st) {
  RouteArgs a;
  a.cfg = cfg;
  a.r = r;
  a.max_cand = max_cand_of(cfg, r.max_chunks);
  const int n_tiles = (a.max_cand + kTile - 1) / kTile;
  const size_t lds = route_select_lds(cfg, r.max_chunks);
  dim3 grid(n_tiles, cfg.hkv, r.B);
  dim3 sgrid(cfg.hkv, r.B);
  const bool bf = cfg.dtype == HGA_BF16;
  if (cfg.d == 128) {
    if (bf) hipLaunchKernelGGL((route_tiles_kernel<128, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((route_tiles_kernel<128, false>), grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((route_select_kernel<128>), sgrid, dim3(256), lds, st, a);
  } else {
    if (bf) hipLaunchKernelGGL((route_tiles_kernel<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((route_tiles_kernel<64, false>), grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((route_select_kernel<64>), sgrid, dim3(256), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace hga
