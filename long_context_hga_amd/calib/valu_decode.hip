// Calibration kernel for the benchmark (not part of the HGA path): the
// decode attention split on the vector ALUs, for comparison with the
// matrix-core split kernel of the library on the same lists.
//
// Shape: head_dim 128, 8 query heads per KV head (grouped-query attention),
// bf16 pool, one query token per sequence.  grid = (splits of 8 listed
// groups, KV heads, sequences), 256 threads; wave w owns list slots
// 8 split + 2w, +1 (32 tokens).  A 256-byte key row is read by 16 lanes, 16
// bytes each, so a wave instruction reads 4 rows; every K and V load of a
// wave is issued before any is used.  Each lane keeps the rotated query of
// all 8 heads for its 8 dims (64 floats) and forms 8 partial dot products
// per row; the 8 lanes of a half-row reduce-scatter them with DPP so that
// each lane ends with the logit of one head (head = lane % 8, permuted per
// register slot so that every step is a plain DPP add), one exp2 per lane
// and token, and the 8 probabilities are gathered back with 7 DPP moves for
// P V.  The four row groups of a wave merge with permlane swaps, the four
// waves through LDS, into one partial (m, l, o) per head and split, in the
// library's partial layout; a second kernel merges the splits.  V is read
// from row-major token rows (the same 4 KiB per group and tensor as the
// library's transposed group blocks).  Keys after the query position are
// masked and their V zeroed.
#include "hga_attend_common.h"

namespace hga {
namespace {

constexpr int kD = 128, kHg = 8;
constexpr int kLpr = kD / 8;            // lanes per token row
constexpr int kRps = 64 / kLpr;         // rows per wave instruction
constexpr int kSteps = kGroupTokens / kRps;
constexpr int kRows = 2 * kSteps;       // row loads per lane (two groups)
constexpr int kRec = 16 + kHg * kD;     // floats per partial record: m[8], l[8], o[8][128]
constexpr int kDppRor8 = 0x128;
constexpr int kDppXor3 = 0x1B;
// register slot k of a lane with head i (i = lane % 8) holds head i ^ kMask[k]
__device__ constexpr int kMask[8] = {0, 1, 2, 3, 7, 6, 5, 4};

struct ValuArgs {
  const uint16_t* q;   // [B][Hq][D] raw bf16
  const int* pos0;     // [B]
  const uint16_t* k;   // [B][Hkv][cap][D] rotated bf16 pool rows
  const uint16_t* v;   // [B][Hkv][cap][D] bf16 value rows
  const int* sel;      // [B][Hkv][max_sel]
  const int* n_sel;    // [B][Hkv]
  float* part;         // [B][Hkv][splits][kRec]
  float* out;          // [B][Hq][D]
  int cap, max_sel, hq, hkv, splits;
  float qscale_log2;   // log2(e) / sqrt(D)
  double omega[kD / 2];
};

// x of this lane's head -> p[k] = x of head (lane % 8) ^ kMask[k]
__device__ __forceinline__ void gather8(float x, float* p) {
  p[0] = x;
  p[1] = dpp_f<kDppXor1>(x);
  p[2] = dpp_f<kDppXor2>(x);
  p[3] = dpp_f<kDppXor3>(x);
  p[4] = dpp_f<kDppHalfMirror>(x);
  p[5] = dpp_f<kDppXor1>(p[4]);
  p[6] = dpp_f<kDppXor2>(p[4]);
  p[7] = dpp_f<kDppXor3>(p[4]);
}

__device__ __forceinline__ void unpack8(uint4 r, float* f) {
  f[0] = bf16lo(r.x); f[1] = bf16hi(r.x);
  f[2] = bf16lo(r.y); f[3] = bf16hi(r.y);
  f[4] = bf16lo(r.z); f[5] = bf16hi(r.z);
  f[6] = bf16lo(r.w); f[7] = bf16hi(r.w);
}

__global__ __launch_bounds__(256) void valu_decode_split(ValuArgs a) {
  __shared__ float qs[kHg][kD];
  __shared__ float mw[4][kHg];
  __shared__ float obuf[4][kHg][kD];
  __shared__ float lbuf[4][kHg];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int unit = b * a.hkv + h;
  const int pos = a.pos0[b];
  const int n_sel = a.n_sel[unit];
  const int v0 = split * kSplitGroups;
  if (n_sel <= 0 || n_sel > a.max_sel || v0 >= n_sel) return;  // the merge reads splits < ceil(n_sel / 8) only
  const int* sel = a.sel + (size_t)unit * a.max_sel;
  const int sub = lane % kLpr, row = lane / kLpr;
  int gpos[2];
  uint4 kr[kRows], vr[kRows];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int v = v0 + 2 * wave + g;
    int gid = sel[v < n_sel ? v : v0];
    gpos[g] = (v < n_sel && gid >= 0 && gid < a.cap / kGroupTokens) ? gid * kGroupTokens : -1;
    gid = gpos[g] < 0 ? 0 : gid;
    const size_t base = ((size_t)unit * a.cap + (size_t)gid * kGroupTokens) * kD;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const size_t e = base + (size_t)(st * kRps + row) * kD + sub * 8;
      kr[g * kSteps + st] = *reinterpret_cast<const uint4*>(a.k + e);
      vr[g * kSteps + st] = *reinterpret_cast<const uint4*>(a.v + e);
    }
  }
  // rotated, pre-scaled query of the 8 heads at the query position: fp64
  // angle as a fraction of a turn, hardware sin / cos of the reduced turn
  if (tid < kD / 2) {
    const int j = tid;
    const double turns = (double)pos * (a.omega[j] * 0.15915494309189533577);
    const float fr = (float)(turns - rint(turns));
    const float cs = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
#pragma unroll
    for (int hh = 0; hh < kHg; ++hh) {
      const size_t qrow = (size_t)(b * a.hq + h * kHg + hh) * kD;
      const float x = bf16_to_f(a.q[qrow + j]), y = bf16_to_f(a.q[qrow + j + kD / 2]);
      qs[hh][j] = (x * cs - y * sn) * a.qscale_log2;
      qs[hh][j + kD / 2] = (x * sn + y * cs) * a.qscale_log2;
    }
  }
  __syncthreads();

  const int hi = sub & 7;  // this lane's head
  float q[8][8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) q[k][i] = qs[hi ^ kMask[k]][sub * 8 + i];
  float m = -INFINITY, l = 0.f, o[8][8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[k][i] = 0.f;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (gpos[g] < 0) continue;  // wave-uniform
    float lg[kSteps];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      float kf[8];
      unpack8(kr[g * kSteps + st], kf);
      float acc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float t = q[k][0] * kf[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) t = fmaf(q[k][i], kf[i], t);
        acc[k] = t;
      }
      // reduce-scatter over the 16 lanes of the row: each lane keeps its head
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] += dpp_f<kDppRor8>(acc[k]);
      float r4[4], r2[2];
#pragma unroll
      for (int k = 0; k < 4; ++k) r4[k] = acc[k] + dpp_f<kDppHalfMirror>(acc[4 + k]);
#pragma unroll
      for (int k = 0; k < 2; ++k) r2[k] = r4[k] + dpp_f<kDppXor2>(r4[2 + k]);
      const float logit = r2[0] + dpp_f<kDppXor1>(r2[1]);
      lg[st] = (gpos[g] + st * kRps + row <= pos) ? logit : -INFINITY;
    }
    float mx = m;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) mx = fmaxf(mx, lg[st]);
    if (__ballot(mx > m) != 0ull) {
      const float al = mx == -INFINITY ? 1.f : exp2f(m - mx);
      float a8[8];
      gather8(al, a8);
      l *= al;
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[k][i] *= a8[k];
      m = mx;
    }
    const float mref = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const float pw = exp2f(lg[st] - mref);
      l += pw;
      float p8[8], vf[8];
      gather8(pw, p8);
      unpack8(vr[g * kSteps + st], vf);
      if (gpos[g] + st * kRps + row > pos) {  // a row not yet written may hold NaN
#pragma unroll
        for (int i = 0; i < 8; ++i) vf[i] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[k][i] = fmaf(p8[k], vf[i], o[k][i]);
    }
  }
  // the four row groups of the wave, then the four waves
  const float mrow = rows_max(m);
  if (lane < 8) mw[wave][lane] = mrow;
  __syncthreads();
  const float M = fmaxf(fmaxf(mw[0][hi], mw[1][hi]), fmaxf(mw[2][hi], mw[3][hi]));
  const float f = M == -INFINITY ? 0.f : exp2f(m - M);
  float f8[8];
  gather8(f, f8);
  l = rows_sum(l * f);
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[k][i] = rows_sum(o[k][i] * f8[k]);
  if (lane < kLpr) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) obuf[wave][hi ^ kMask[k]][sub * 8 + i] = o[k][i];
    if (lane < 8) lbuf[wave][hi] = l;
  }
  __syncthreads();
  float* rec = a.part + ((size_t)unit * a.splits + split) * kRec;
  {
    const int hh = tid / 32, d0 = (tid % 32) * 4;  // 8 heads x 128 dims over 256 threads
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s.x += obuf[w][hh][d0];
      s.y += obuf[w][hh][d0 + 1];
      s.z += obuf[w][hh][d0 + 2];
      s.w += obuf[w][hh][d0 + 3];
    }
    *reinterpret_cast<float4*>(rec + 16 + hh * kD + d0) = s;
  }
  if (tid < kHg) {
    rec[tid] = fmaxf(fmaxf(mw[0][tid], mw[1][tid]), fmaxf(mw[2][tid], mw[3][tid]));
    rec[kHg + tid] = lbuf[0][tid] + lbuf[1][tid] + lbuf[2][tid] + lbuf[3][tid];
  }
}

// One wave per (unit, head): the exact merge of the unit's splits, every
// split's (m, l, o) loaded before any is used.
__global__ __launch_bounds__(64) void valu_decode_merge(ValuArgs a) {
  const int lane = threadIdx.x;
  const int hh = blockIdx.x % kHg, unit = blockIdx.x / kHg;
  const int b = unit / a.hkv, h = unit % a.hkv;
  const int n_sel = a.n_sel[unit];
  const int ns = (n_sel > 0 && n_sel <= a.max_sel) ? (n_sel + kSplitGroups - 1) / kSplitGroups : 0;
  float pm[kMaxSplits], pl[kMaxSplits];
  float2 po[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < ns) {  // uniform
      const float* rec = a.part + ((size_t)unit * a.splits + s) * kRec;
      pm[s] = rec[hh];
      pl[s] = rec[kHg + hh];
      po[s] = *reinterpret_cast<const float2*>(rec + 16 + hh * kD + 2 * lane);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < ns) M = fmaxf(M, pm[s]);
  float L = 0.f, ox = 0.f, oy = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      if (s < ns) {
        const float w = exp2f(pm[s] - M);
        L = fmaf(w, pl[s], L);
        ox = fmaf(w, po[s].x, ox);
        oy = fmaf(w, po[s].y, oy);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float2*>(a.out + (size_t)(b * a.hq + h * kHg + hh) * kD + 2 * lane) =
      make_float2(ox * inv, oy * inv);
}

}  // namespace
}  // namespace hga

// Decode attention of B sequences over their lists on the vector ALUs (the
// shape above; cap a multiple of 16, max_sel <= 256): the split kernel, then
// the merge, on `stream`.  part holds B * hkv * ceil(max_sel / 8) records of
// 1040 floats.  Returns 0, or -1 for an unsupported argument, or the HIP
// error of the launches.
extern "C" int hga_calib_valu_decode(const void* q, const int* pos0, const void* k_pool,
                                     const void* v_rows, int cap, const int* sel, const int* n_sel,
                                     int max_sel, int B, int hq, int hkv, const double* omega,
                                     float qscale_log2, float* part, float* out, void* stream) {
  using namespace hga;
  if (!q || !pos0 || !k_pool || !v_rows || !sel || !n_sel || !part || !out || !omega || B <= 0 ||
      cap <= 0 || cap % kGroupTokens != 0 || max_sel <= 0 || max_sel > kMaxSplits * kSplitGroups ||
      hkv <= 0 || hq != hkv * kHg)
    return -1;
  ValuArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.pos0 = pos0;
  a.k = static_cast<const uint16_t*>(k_pool);
  a.v = static_cast<const uint16_t*>(v_rows);
  a.sel = sel;
  a.n_sel = n_sel;
  a.part = part;
  a.out = out;
  a.cap = cap;
  a.max_sel = max_sel;
  a.hq = hq;
  a.hkv = hkv;
  a.splits = (max_sel + kSplitGroups - 1) / kSplitGroups;
  a.qscale_log2 = qscale_log2;
  for (int j = 0; j < kD / 2; ++j) a.omega[j] = omega[j];
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(valu_decode_split, dim3(a.splits, hkv, B), dim3(256), 0, st, a);
  hipLaunchKernelGGL(valu_decode_merge, dim3(B * hkv * kHg), dim3(64), 0, st, a);
  return (int)hipGetLastError();
}
