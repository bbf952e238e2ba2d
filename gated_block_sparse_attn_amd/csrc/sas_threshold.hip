// Gate activation, Top-K threshold and selector-score gradient kernels.
//
// SAS paper (arXiv 2609.13141): Sec. 4.1 Eq. 4 (current block keeps a unit
// gate), Sec. 4.2.2 Eq. 6 (log g_m = s_m - LSE(s) over the historical blocks;
// the sigmoid and raw-logit activations of Sec. 4.1 / Tab. 1 as switches),
// Sec. 4.3 Alg. 1 and App. E (Top-K realised as a per-query threshold on the
// gate, no sort), App. D.3 and Eq. 8 (softmax backward to the scores under
// the sparse scope).
//
// One wavefront owns one row (b, h_kv, i) of the [C, C] score table: the
// row's historical scores (m < i) are staged in LDS once and every pass
// (max, sum, log-gate write, radix select, compaction) reads them from there;
// the radix select keeps a 256-bin histogram per wavefront in LDS.
// Both kernels are HBM-bound: they read and write the score-table rows once.
#include <math.h>

#include "../../include/sas.h"
#include "sas_internal.h"

namespace sas {
namespace {

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Order-preserving map of fp32 bit patterns to unsigned integers:
// a < b (as finite floats, -0 canonicalised to +0)  <=>  key(a) < key(b).
__device__ __forceinline__ uint32_t f2key(float x) {
  const uint32_t b = __float_as_uint(x);
  return b ^ ((b >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float(k ^ ((k >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}

__device__ __forceinline__ int popc64(unsigned long long m) { return __popcll(m); }

// lanes below the current one whose bit is set in mask
__device__ __forceinline__ int rank_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ void __launch_bounds__(256) threshold_kernel(const float* __restrict__ scores,
                                                        float* __restrict__ log_gate,
                                                        float* __restrict__ tau,
                                                        int32_t* __restrict__ sel_idx,
                                                        int32_t* __restrict__ sel_cnt,
                                                        int32_t* __restrict__ d_status,
                                                        long long rows, int C, int K, int cap,
                                                        int act, const int32_t* __restrict__ lens,
                                                        const int32_t* __restrict__ cu,
                                                        long long T, int Hs, int N) {
  extern __shared__ float s_lds[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const long long row = (long long)blockIdx.x * nw + w;
  if (row >= rows) return;  // whole wavefront leaves; no workgroup barrier follows
  const int i = (int)(row % C);
  const float* srow = scores + row * (long long)C;
  float* s = s_lds + (size_t)w * (C + 256);   // this wavefront's row
  int* hist = (int*)(s + C);                  // and its 256-bin histogram

  // Stage the historical scores (four loads in flight per lane); +0.0f turns
  // -0 into +0 so that the integer keys order exactly like the fp32
  // comparison used for the selected set.
  float mx = -INFINITY;
  for (int m0 = 0; m0 < i; m0 += 256) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int m = m0 + u * 64 + lane;
      x[u] = m < i ? srow[m] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int m = m0 + u * 64 + lane;
      if (m < i) {
        s[m] = x[u] + 0.0f;
        mx = fmaxf(mx, x[u]);
      }
    }
  }
  mx = wave_max_f(mx);

  // LSE over the historical blocks (Eq. 6): fp32 exponentials of values <= 0,
  // accumulated in fp64 so the normaliser does not drift with long rows.
  double lse = 0.0;
  if (i > 0 && act == SAS_GATE_SOFTMAX) {
    double acc = 0.0;
    for (int m = lane; m < i; m += 64) acc += (double)expf(s[m] - mx);
    acc = wave_sum_d(acc);
    lse = (double)mx + log(acc);
  }

  // log_gate row: log phi(s) for historical blocks (softmax: s - LSE;
  // sigmoid: log sigmoid(s) = -log(1 + exp(-s)), evaluated without overflow;
  // raw: s), 0 for the current block (unit gate, Eq. 4), -inf above the
  // diagonal.
  float* lrow = log_gate + row * (long long)C;
  for (int m = lane; m < C; m += 64) {
    float val;
    if (m < i) {
      const float x = s[m];
      if (act == SAS_GATE_SOFTMAX) val = (float)((double)x - lse);
      else if (act == SAS_GATE_SIGMOID) val = x >= 0.0f ? -log1pf(expf(-x)) : x - log1pf(expf(x));
      else val = x;
    } else if (m == i) val = 0.0f;
    else val = -INFINITY;
    lrow[m] = val;
  }

  // Variable-length batch: a row past the sequence's last block holds no
  // query and selects nothing.
  bool empty = false;
  if (lens != nullptr || cu != nullptr) {
    const int b = (int)(row / ((long long)Hs * C));
    int n;
    if (cu != nullptr) {   // packed batch: offsets clamped into [0, T] like the attention kernels
      const long long s0 = min(max((long long)cu[b], 0LL), T);
      const long long s1 = min(max((long long)cu[b + 1], s0), T);
      n = (int)min(s1 - s0, (long long)N);
    } else {
      n = min(max(lens[b], 0), N);
    }
    const int blk = N / C;
    empty = i >= (n + blk - 1) / blk;
  }

  // Threshold: the K-th largest historical score (radix select over the
  // order-preserving integer keys, no sort), eight bits per pass from the
  // most significant end: a 256-bin histogram of the keys that match the
  // digits found so far, then the digit d where the count of keys with a
  // larger digit is < krem <= that count plus bin d.
  float t;
  if (empty) {
    t = INFINITY;
  } else if (K >= i) {
    t = -INFINITY;
  } else if (K == 0) {
    t = INFINITY;
  } else {
    uint32_t prefix = 0u, known = 0u;
    int krem = K;   // rank of the wanted key among those matching prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) hist[q * 64 + lane] = 0;
      for (int m = lane; m < i; m += 64) {
        const uint32_t key = f2key(s[m]);
        if ((key & known) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      // lane l holds bins 255 - 4 l - q (q = 0..3): descending digit order
      int c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = hist[255 - 4 * lane - q];
      const int local = c[0] + c[1] + c[2] + c[3];
      int incl = local;   // inclusive scan over the lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const int excl = incl - local;
      const bool hit = excl < krem && krem <= incl;
      int dig = 0, above = excl;
      if (hit) {
        int q = 0;
        while (above + c[q] < krem) above += c[q++];
        dig = 255 - 4 * lane - q;
      }
      const unsigned long long hm = __ballot(hit);
      const int src = __builtin_ctzll(hm);   // exactly one lane hits (1 <= krem <= count)
      dig = __shfl(dig, src, 64);
      above = __shfl(above, src, 64);
      prefix |= (uint32_t)dig << shift;
      known |= 255u << shift;
      krem -= above;
    }
    t = key2f(prefix);
  }

  // Compact {m < i : s_m >= t} in ascending order.
  int32_t* out = sel_idx + row * (long long)cap;
  int base = 0;
  for (int m0 = 0; m0 < i; m0 += 64) {
    const int m = m0 + lane;
    const bool p = !empty && (m < i) && (s[m < i ? m : 0] >= t);
    const unsigned long long mask = __ballot(p);
    if (p) {
      const int pos = base + rank_below(mask);
      if (pos < cap) out[pos] = m;
    }
    base += popc64(mask);
  }
  for (int pos = base + lane; pos < cap; pos += 64) out[pos] = -1;
  if (lane == 0) {
    sel_cnt[row] = base;
    tau[row] = t;
    if (base > cap && d_status != nullptr) *d_status = SAS_E_CAPACITY;
  }
}

// dscores[i, m] = dLogG[i, m] - g[i, m] * sum_{l < i} dLogG[i, l] for m < i, else 0.
// This is App. D.3's ds_m = g_m (dg_m - sum_l g_l dg_l) with dLogG = g * dg,
// and dg = 0 on unselected blocks (sparse scope, Eq. 8).  Sigmoid gates
// depend on their own score only: ds_m = g_m (1 - g_m) dg_m = (1 - g_m) dLogG_m;
// raw logits: ds_m = dLogG_m.  Hard gates (straight-through estimator): the
// table holds dg itself for every historical block (full scope), so
// ds_m = g_m (dg_m - sum_l g_l dg_l).
//
// One wavefront per gate row.  fill (sel_idx given; soft gates): the
// key-major pass wrote dLogG only at the row's selected blocks, so the values
// of the other entries are not used and are written here as 0; the selected
// ones are marked in a per-row LDS bit mask, and the softmax sum gathers them
// from the row's selection list.
constexpr int kDsRows = 4;                 // gate rows per workgroup
constexpr int kDsMaxWords = 8192 / 32;     // bit mask words of the longest row
__global__ void __launch_bounds__(64 * kDsRows) dscores_kernel(
    float* __restrict__ dlg, const float* __restrict__ lg, float* __restrict__ ds, long long rows,
    int C, int act, int hard, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, int cap) {
  __shared__ uint32_t s_sel[kDsRows][kDsMaxWords];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * kDsRows + wv;
  const bool live = row < rows;
  const bool fill = sel_idx != nullptr && !hard;
  const bool masked = fill;   // only the selected entries are valid
  const int i = live ? (int)(row % C) : 0;
  float* drow = dlg + (live ? row : 0) * (long long)C;
  const float* grow = lg + (live ? row : 0) * (long long)C;
  float* orow = ds + (live ? row : 0) * (long long)C;
  float tot = 0.0f;
  if (masked) {   // every wavefront reaches both barriers
    const int nw = (C + 31) / 32;
    for (int x = lane; x < nw; x += 64) s_sel[wv][x] = 0u;
    __syncthreads();
    if (live) {
      const int cnt = min(sel_cnt[row], cap);
      const int32_t* sr = sel_idx + row * (long long)cap;
      for (int e = lane; e < cnt; e += 64) {
        const int m = sr[e];
        atomicOr(&s_sel[wv][m >> 5], 1u << (m & 31));
        if (act == SAS_GATE_SOFTMAX) tot += drow[m];   // the row's sum over its selected blocks
      }
    }
    __syncthreads();
    if (act == SAS_GATE_SOFTMAX) tot = wave_sum_f(tot);
  }
  if (!live) return;
  if (hard) {   // dlog_gate holds dg of every historical block: g (dg - sum g dg)
    for (int m = lane; m < i; m += 64) tot += expf(grow[m]) * drow[m];
    tot = wave_sum_f(tot);
  } else if (act == SAS_GATE_SOFTMAX && !masked) {
    for (int m = lane; m < i; m += 64) tot += drow[m];
    tot = wave_sum_f(tot);
  }
  // entry m: dLogG value raw (the load is in the row whatever m is; values of
  // unwritten entries are not used) and log gate lgm -> (dLogG, dscores)
  auto entry = [&](int m, float raw, float lgm, float& d, float& o) {
    const bool valid = m < i && (!masked || ((s_sel[wv][m >> 5] >> (m & 31)) & 1u) != 0u);
    d = valid ? raw : 0.0f;
    o = 0.0f;
    if (m < i) {
      if (hard) o = expf(lgm) * (d - tot);
      else if (act == SAS_GATE_SOFTMAX) o = d - expf(lgm) * tot;
      else if (act == SAS_GATE_SIGMOID) o = d * (1.0f - expf(lgm));
      else o = d;
    }
  };
  const bool vec = (C & 3) == 0 && (((uintptr_t)dlg | (uintptr_t)lg | (uintptr_t)ds) & 15) == 0;
  if (vec) {   // 16-byte pieces (every row then starts 16-byte aligned)
    for (int m0 = 4 * lane; m0 < C; m0 += 256) {
      const float4 r = *(const float4*)(drow + m0);
      const float4 gl = *(const float4*)(grow + m0);
      float4 dv, ov;
      entry(m0, r.x, gl.x, dv.x, ov.x);
      entry(m0 + 1, r.y, gl.y, dv.y, ov.y);
      entry(m0 + 2, r.z, gl.z, dv.z, ov.z);
      entry(m0 + 3, r.w, gl.w, dv.w, ov.w);
      if (fill) *(float4*)(drow + m0) = dv;
      *(float4*)(orow + m0) = ov;
    }
  } else {
    for (int m = lane; m < C; m += 64) {
      float d, o;
      entry(m, drow[m], grow[m], d, o);
      if (fill) drow[m] = d;
      orow[m] = o;
    }
  }
}

}  // namespace

hipError_t launch_threshold(const Shape& s, const float* scores, float* log_gate, float* tau,
                            int32_t* sel_idx, int32_t* sel_cnt, int32_t* d_status,
                            hipStream_t st) {
  const long long rows = (long long)s.B * s.Hs * s.C;
  const int nw = (s.C <= 2048) ? 4 : 1;   // at most 34 KB of LDS per workgroup (C <= 8192)
  const size_t lds = (size_t)nw * (s.C + 256) * sizeof(float);
  const long long grid = (rows + nw - 1) / nw;
  hipLaunchKernelGGL(threshold_kernel, dim3((unsigned)grid), dim3(64 * nw), lds, st, scores,
                     log_gate, tau, sel_idx, sel_cnt, d_status, rows, s.C, s.K, s.cap, s.act,
                     s.lens, s.cu, s.T, s.Hs, s.N);
  return hipGetLastError();
}

hipError_t launch_dscores(const Shape& s, float* dlog_gate, const float* log_gate,
                          float* dscores, const int32_t* sel_idx, const int32_t* sel_cnt,
                          hipStream_t st) {
  const long long rows = (long long)s.B * s.Hs * s.C;
  const long long grid = (rows + kDsRows - 1) / kDsRows;
  hipLaunchKernelGGL(dscores_kernel, dim3((unsigned)grid), dim3(64 * kDsRows), 0, st, dlog_gate,
                     log_gate, dscores, rows, s.C, s.act, s.hard, sel_idx, sel_cnt, s.cap);
  return hipGetLastError();
}

}  // namespace sas
