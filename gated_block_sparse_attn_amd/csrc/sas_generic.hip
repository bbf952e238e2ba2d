// Vector-ALU gated block-sparse attention, forward and backward, for every
// supported (dtype, head_dim, block) combination.  The bf16 / D = 128 /
// b = 64 shape normally runs on the matrix-core kernels instead; this path
// covers fp32 tensors, D = 64 and blocks of 16 or 32 tokens, with the same
// semantics:
//
//  forward  (SAS Sec. 4.3 Eq. 9, App. E Alg. 3): per query block the current
//           block (causal, bias 0) and the selected historical blocks (bias
//           log g), streamed tile by tile with an online softmax in base 2;
//           with the outer gate position (Sec. 4.1, Tab. 1 row 3) the logits
//           carry no bias and the block's value rows are scaled by g; with
//           hard Top-K gates (Eq. 7, Tab. 1 row 8) the selected blocks carry
//           unit gates and the dropped blocks' gate gradients come from
//           ste_dropped_kernel;
//  backward (App. E Alg. 4): P recomputed from LSE, dS = P (dP - Delta);
//           query-major pass: dQ = scale dS K with Delta = rowsum(O dO), and
//           the row sum of P dP (Delta without the rounding of O); key-major
//           pass, with that Delta: dK = scale dS^T Q, dV = P^T dO and
//           dLogG = block sums of dS.
//
// One thread owns one query row (forward, dQ pass) or one key row (dK/dV
// pass); K/V tiles are staged in LDS as fp32.
#include <math.h>

#include <type_traits>

#include "sas_internal.h"

namespace sas {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return (float)(*p); }
template <typename T>
__device__ __forceinline__ void st(T* p, float x) { *p = (T)x; }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

struct GenArgs {
  const void* q; const void* k; const void* v; const void* o; const void* d_o;
  const float* lse; const float* lg; const int32_t* sel_idx; const int32_t* sel_cnt;
  void* out; float* lse_out; void* dq; void* dk; void* dv; float* dlg; float* delta;
  int Hq, Hkv, G, N, C, cap;
  int Hs, Gs;   // score heads (rows of the gate tables) and query heads per score head
  int o_fp32;   // o is stored as float32 (else as T)
  int outer;    // gates scale the value rows after the softmax (else log g bias)
  int hard;     // hard Top-K gates (straight-through estimator): unit gates
  const int32_t* lens;   // valid tokens per sequence (nullptr: all N)
  const int32_t* cu;     // packed layout: sequence b holds tokens cu[b] .. cu[b+1]-1
                         // of [T, H, D] tensors (nullptr: padded [B, H, N, D])
  long long T;           // packed layout: total tokens
  float c2;     // sm_scale * log2(e)
  float scale;  // sm_scale
};

// First token (packed layout) and number of valid tokens of sequence b,
// clamped so that every row stays inside the tensors: 0 <= start,
// start + n <= T, 0 <= n <= N.
struct Seq {
  long long start;
  int n;
};
__device__ __forceinline__ Seq seq_of(const GenArgs& a, int b) {
  if (a.cu != nullptr) {
    const long long s0 = min(max((long long)a.cu[b], 0LL), a.T);
    const long long s1 = min(max((long long)a.cu[b + 1], s0), a.T);
    return {s0, (int)min(s1 - s0, (long long)a.N)};
  }
  return {0, a.lens == nullptr ? a.N : min(max(a.lens[b], 0), a.N)};
}
// Row (in rows of D elements) of token n of sequence b, head h of H heads:
// padded [B, H, N, D] or packed [T, H, D].
__device__ __forceinline__ long long row_of(const GenArgs& a, int b, const Seq& sq, int h, int H,
                                            int n) {
  return a.cu != nullptr ? (sq.start + n) * H + h : ((long long)b * H + h) * a.N + n;
}
// Index of token n of sequence b, query head h, in LSE and Delta: padded
// [B, Hq, N] or packed [Hq, T].
__device__ __forceinline__ long long stat_of(const GenArgs& a, int b, const Seq& sq, int h, int n) {
  return a.cu != nullptr ? (long long)h * a.T + sq.start + n : ((long long)b * a.Hq + h) * a.N + n;
}

// Index of token n of sequence b, query head h, in the workspace's Delta
// array: padded order [B, Hq, N] in every layout (the matrix-core kernels
// use the same order, so either path's Delta serves the dropped-block pass).
__device__ __forceinline__ long long ws_of(const GenArgs& a, int b, int h, int n) {
  return ((long long)b * a.Hq + h) * a.N + n;
}

// Stage the BLK rows of key block kb of (sequence b, kv head hk) of a K or V
// tensor into LDS as fp32.  In the packed layout rows past the sequence's
// end read as zero (they belong to the next sequence or lie past the tensor);
// they are never attended.
template <typename T, int D, int BLK>
__device__ __forceinline__ void stage_block(float* dst, const void* base, const GenArgs& a, int b,
                                            const Seq& sq, int hk, int kb) {
  const bool packed = a.cu != nullptr;
  const T* src = (const T*)base + row_of(a, b, sq, hk, a.Hkv, kb * BLK) * D;
  const long long stride = packed ? (long long)a.Hkv * D : D;   // elements from token to token
  const int nvalid = packed ? min(BLK, max(sq.n - kb * BLK, 0)) : BLK;
  for (int e = threadIdx.x; e < BLK * D; e += blockDim.x) {
    const int r = e / D, c = e - r * D;
    dst[e] = r < nvalid ? ld(src + r * stride + c) : 0.0f;
  }
}

template <typename T, int D, int BLK>
__global__ void __launch_bounds__(64) fwd_generic_kernel(GenArgs a) {
  extern __shared__ float smem[];
  float* ks = smem;
  float* vs = smem + BLK * D;
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const int bb = bh / a.Hq, h = bh % a.Hq, hk = h / a.G;
  const int t = threadIdx.x;
  const Seq sq = seq_of(a, bb);
  const int nb = sq.n;
  const bool active = t < BLK && i * BLK + t < nb;   // padding rows stay inactive
  const bool any = i * BLK < nb;                      // block holds a valid row (uniform)
  const long long row = ((long long)bb * a.Hs + h / a.Gs) * a.C + i;   // this head's gate row
  const int cnt = min(a.sel_cnt[row], a.cap);
  const int32_t* sel = a.sel_idx + row * a.cap;
  const long long qr = row_of(a, bb, sq, h, a.Hq, i * BLK + t);   // dereferenced when active
  const T* qrow = (const T*)a.q + qr * D;

  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = active ? ld(qrow + d) * a.c2 : 0.0f;
    acc[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int tile = 0; any && tile <= cnt; ++tile) {
    const int kb = tile == 0 ? i : sel[tile - 1];
    const float lgv = (tile == 0 || a.hard) ? 0.0f : a.lg[row * a.C + kb] * kLog2e;
    const float beta = a.outer ? 0.0f : lgv;           // bias of the logits
    const float gv = a.outer ? exp2f(lgv) : 1.0f;      // factor of the value rows
    __syncthreads();
    stage_block<T, D, BLK>(ks, a.k, a, bb, sq, hk, kb);
    stage_block<T, D, BLK>(vs, a.v, a, bb, sq, hk, kb);
    __syncthreads();
    if (active) {
      // per-key online softmax update (this path favours simplicity)
#pragma unroll 1
      for (int u = 0; u < BLK; ++u) {
        if (tile == 0 && u > t) break;   // causal inside the current block
        float x = beta;
#pragma unroll
        for (int d = 0; d < D; ++d) x += q[d] * ks[u * D + d];
        const float mnew = fmaxf(m, x);
        const float corr = exp2f(m - mnew);
        const float p = exp2f(x - mnew);
        l = l * corr + p;
        const float pv = p * gv;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = acc[d] * corr + pv * vs[u * D + d];
        m = mnew;
      }
    }
  }
  // padded layout: padding rows get o = 0, lse = 0; packed: only valid rows
  // exist (the rows after a sequence belong to the next one)
  if (a.cu != nullptr ? active : t < BLK) {
    const float inv = active ? 1.0f / l : 0.0f;
    if (a.o_fp32) {
      float* orow = (float*)a.out + qr * D;
#pragma unroll
      for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
    } else {
      T* orow = (T*)a.out + qr * D;
#pragma unroll
      for (int d = 0; d < D; ++d) st(orow + d, acc[d] * inv);
    }
    a.lse_out[stat_of(a, bb, sq, h, i * BLK + t)] = active ? (m + log2f(l)) * kLn2 : 0.0f;
  }
}

// Query-major backward: dQ, and Delta = sum of P dP over each query row.
template <typename T, int D, int BLK>
__global__ void __launch_bounds__(64) bwd_q_generic_kernel(GenArgs a) {
  extern __shared__ float smem[];
  float* ks = smem;
  float* vs = smem + BLK * D;
  const int i = blockIdx.x;
  const int bhk = blockIdx.y;
  const int bb = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int t = threadIdx.x;
  const Seq sq = seq_of(a, bb);
  const int nb = sq.n;
  const bool active = t < BLK && i * BLK + t < nb;   // padding rows: dq = 0, Delta = 0
  const bool any = i * BLK < nb;

  for (int hl = 0; hl < a.G; ++hl) {
    const int h = hk * a.G + hl;
    const long long row = ((long long)bb * a.Hs + h / a.Gs) * a.C + i;   // this head's gate row
    const int cnt = min(a.sel_cnt[row], a.cap);
    const int32_t* sel = a.sel_idx + row * a.cap;
    const long long qr = row_of(a, bb, sq, h, a.Hq, i * BLK + t);   // q / o / dO / dq row
    const long long qs = stat_of(a, bb, sq, h, i * BLK + t);        // LSE / Delta entry
    float q[D], dov[D], dq[D];
    float delta = 0.0f, lse2 = 0.0f, dx = 0.0f;
    if (active) {
      const T* qrow = (const T*)a.q + qr * D;
      const T* drow = (const T*)a.d_o + qr * D;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        q[d] = ld(qrow + d);
        dov[d] = ld(drow + d);
        const float od = a.o_fp32 ? ((const float*)a.o)[qr * D + d] : ld((const T*)a.o + qr * D + d);
        delta += od * dov[d];
        dq[d] = 0.0f;
      }
      lse2 = a.lse[qs] * kLog2e;
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d) { q[d] = 0.0f; dov[d] = 0.0f; dq[d] = 0.0f; }
    }
    for (int tile = 0; any && tile <= cnt; ++tile) {
      const int kb = tile == 0 ? i : sel[tile - 1];
      const float lgv = (tile == 0 || a.hard) ? 0.0f : a.lg[row * a.C + kb] * kLog2e;
      const float beta = a.outer ? 0.0f : lgv;
      const float gv = a.outer ? exp2f(lgv) : 1.0f;   // outer: dP = g dO . v
      __syncthreads();
      stage_block<T, D, BLK>(ks, a.k, a, bb, sq, hk, kb);
      stage_block<T, D, BLK>(vs, a.v, a, bb, sq, hk, kb);
      __syncthreads();
      if (active) {
#pragma unroll 1
        for (int u = 0; u < BLK; ++u) {
          if (tile == 0 && u > t) break;
          float x = 0.0f, dp = 0.0f;
#pragma unroll
          for (int d = 0; d < D; ++d) {
            x += q[d] * ks[u * D + d];
            dp += dov[d] * vs[u * D + d];
          }
          dp *= gv;
          const float p = exp2f(x * a.c2 + beta - lse2);
          const float ds = p * (dp - delta);
          dx += p * dp;
#pragma unroll
          for (int d = 0; d < D; ++d) dq[d] += ds * ks[u * D + d];
        }
      }
    }
    if (a.cu != nullptr ? active : t < BLK) {
      a.delta[ws_of(a, bb, h, i * BLK + t)] = dx;
      T* dqrow = (T*)a.dq + qr * D;
#pragma unroll
      for (int d = 0; d < D; ++d) st(dqrow + d, dq[d] * a.scale);
    }
  }
}

// Key-major backward: dK and dV of one key block j, over every query block
// that attends it (the diagonal block and each later block that selected it)
// and every query head of the kv group, and column j of the dLogG table of
// each score head of the group (every entry written: the dS sum of a
// selecting block i > j over the score head's query heads, else 0; one
// wavefront, fixed summation order).
template <typename T, int D, int BLK>
__global__ void __launch_bounds__(64) bwd_kv_generic_kernel(GenArgs a) {
  extern __shared__ float smem[];
  float* ks = smem;
  float* vs = smem + BLK * D;
  const int j = blockIdx.x;
  const int bhk = blockIdx.y;
  const int bb = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int u = threadIdx.x;
  const bool active = u < BLK;
  const Seq sq = seq_of(a, bb);
  const int nb = sq.n;
  stage_block<T, D, BLK>(ks, a.k, a, bb, sq, hk, j);
  stage_block<T, D, BLK>(vs, a.v, a, bb, sq, hk, j);
  __syncthreads();
  float dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { dk[d] = 0.0f; dv[d] = 0.0f; }
  const int ns = a.G / a.Gs;   // score heads of this kv group
  for (int si = 0; si < ns; ++si) {
    const long long rb = ((long long)bb * a.Hs + hk * ns + si) * a.C;
    for (int i = u; i <= j && i < a.C; i += blockDim.x) a.dlg[(rb + i) * a.C + j] = 0.0f;
  }
  for (int i = j; i < a.C; ++i)
  for (int si = 0; si < ns; ++si) {
    const long long rowbase = ((long long)bb * a.Hs + hk * ns + si) * a.C;
    float beta = 0.0f;
    if (i != j) {
      // is j in the ascending selected list of row i?  (binary search)
      const int cnt = min(a.sel_cnt[rowbase + i], a.cap);
      const int32_t* sel = a.sel_idx + (rowbase + i) * a.cap;
      int lo = 0, hi = cnt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sel[mid] < j) lo = mid + 1; else hi = mid;
      }
      if (lo >= cnt || sel[lo] != j) {
        if (u == 0) a.dlg[(rowbase + i) * a.C + j] = 0.0f;
        continue;
      }
      beta = a.hard ? 0.0f : a.lg[(rowbase + i) * a.C + j] * kLog2e;
    }
    // outer: no bias; dP = g dO . v, dV = g P^T dO, dLogG = sum of P dP
    const float gv = a.outer ? exp2f(beta) : 1.0f;
    if (a.outer) beta = 0.0f;
    float gsum = 0.0f;
    for (int hl = 0; hl < a.Gs; ++hl) {
      const int h = (hk * ns + si) * a.Gs + hl;
#pragma unroll 1
      for (int tq = 0; tq < BLK; ++tq) {
        if (!active || (i == j && u > tq) || i * BLK + tq >= nb) continue;   // padding queries
        const long long qr = row_of(a, bb, sq, h, a.Hq, i * BLK + tq);
        const long long qs = stat_of(a, bb, sq, h, i * BLK + tq);
        const T* qrow = (const T*)a.q + qr * D;
        const T* drow = (const T*)a.d_o + qr * D;
        float x = 0.0f, dp = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          x += ld(qrow + d) * ks[u * D + d];
          dp += ld(drow + d) * vs[u * D + d];
        }
        dp *= gv;
        const float p = exp2f(x * a.c2 + beta - a.lse[qs] * kLog2e);
        const float ds = p * (dp - a.delta[ws_of(a, bb, h, i * BLK + tq)]);
        gsum += a.outer ? p * dp : ds;
        const float pg = p * gv;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          dv[d] += pg * ld(drow + d);
          dk[d] += ds * ld(qrow + d);
        }
      }
    }
    if (i != j) {
      gsum = wave_sum(gsum);
      if (u == 0) a.dlg[(rowbase + i) * a.C + j] = gsum;
    }
  }
  // padded layout: every row of the block (padding keys get 0); packed: only
  // the sequence's own rows
  if (active && (a.cu == nullptr || j * BLK + u < nb)) {
    const long long r = row_of(a, bb, sq, hk, a.Hkv, j * BLK + u);
    T* dkrow = (T*)a.dk + r * D;
    T* dvrow = (T*)a.dv + r * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      st(dkrow + d, dk[d] * a.scale);
      st(dvrow + d, dv[d]);
    }
  }
}

// Hard Top-K gates with the straight-through estimator (Sec. 4.1 "Ranking
// preservation", Eq. 7): the gate gradient of every dropped historical block
// m of query block i is the attention mass its tokens would receive under the
// selected set's normaliser, exp(z - lse), times (dP - Delta), summed over
// the block's tokens, the query block's rows and the query heads of the
// score head.  One wavefront per gate row (b, score head, i); dropped blocks
// are found by walking the ascending selected list; fixed summation order.
template <typename T, int D, int BLK>
__global__ void __launch_bounds__(64) ste_dropped_kernel(GenArgs a) {
  extern __shared__ float smem[];
  float* ks = smem;
  float* vs = smem + BLK * D;
  const int i = blockIdx.x;
  const int bs = blockIdx.y;
  const int bb = bs / a.Hs, sh = bs % a.Hs;
  const int hk = sh * a.Gs / a.G;
  const int t = threadIdx.x;
  const Seq sq = seq_of(a, bb);
  const int nb = sq.n;
  if (i * BLK >= nb) return;   // no query in this block: its row stays 0 (key pass)
  const bool active = t < BLK && i * BLK + t < nb;
  const long long row = ((long long)bb * a.Hs + sh) * a.C + i;
  const int cnt = min(a.sel_cnt[row], a.cap);
  const int32_t* sel = a.sel_idx + row * a.cap;
  int e = 0;
  for (int m = 0; m < i; ++m) {
    while (e < cnt && sel[e] < m) ++e;
    if (e < cnt && sel[e] == m) continue;   // selected: its dS sum comes from the kv pass
    __syncthreads();
    stage_block<T, D, BLK>(ks, a.k, a, bb, sq, hk, m);
    stage_block<T, D, BLK>(vs, a.v, a, bb, sq, hk, m);
    __syncthreads();
    float acc = 0.0f;
    for (int hl = 0; hl < a.Gs; ++hl) {
      if (!active) continue;
      const int h = sh * a.Gs + hl;
      const long long qr = row_of(a, bb, sq, h, a.Hq, i * BLK + t);
      const long long qs = stat_of(a, bb, sq, h, i * BLK + t);
      const T* qrow = (const T*)a.q + qr * D;
      const T* drow = (const T*)a.d_o + qr * D;
      const float lse2 = a.lse[qs] * kLog2e;
      const float delta = a.delta[ws_of(a, bb, h, i * BLK + t)];
#pragma unroll 1
      for (int u = 0; u < BLK; ++u) {
        float x = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; ++d) {
          x += ld(qrow + d) * ks[u * D + d];
          dp += ld(drow + d) * vs[u * D + d];
        }
        acc += exp2f(x * a.c2 - lse2) * (dp - delta);
      }
    }
    acc = wave_sum(acc);
    if (t == 0) a.dlg[row * a.C + m] = acc;
  }
}

GenArgs make_args(const Shape& s) {
  GenArgs a{};
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.G; a.N = s.N; a.C = s.C; a.cap = s.cap;
  a.Hs = s.Hs; a.Gs = s.Hq / s.Hs;
  a.o_fp32 = s.o_fp32;
  a.outer = s.outer;
  a.hard = s.hard;
  a.lens = s.lens;
  a.cu = s.cu;
  a.T = s.T;
  a.c2 = s.scale * kLog2e;
  a.scale = s.scale;
  return a;
}

template <typename T, int D, int BLK>
hipError_t fwd_launch(const GenArgs& a, const Shape& s, hipStream_t st) {
  const size_t lds = 2 * BLK * D * sizeof(float);
  hipLaunchKernelGGL((fwd_generic_kernel<T, D, BLK>), dim3(s.C, s.B * s.Hq), dim3(64), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D, int BLK>
hipError_t bwd_q_launch(const GenArgs& a, const Shape& s, hipStream_t st) {
  const size_t lds = 2 * BLK * D * sizeof(float);
  hipLaunchKernelGGL((bwd_q_generic_kernel<T, D, BLK>), dim3(s.C, s.B * s.Hkv), dim3(64), lds, st,
                     a);
  return hipGetLastError();
}

template <typename T, int D, int BLK>
hipError_t bwd_kv_launch(const GenArgs& a, const Shape& s, hipStream_t st) {
  const size_t lds = 2 * BLK * D * sizeof(float);
  hipLaunchKernelGGL((bwd_kv_generic_kernel<T, D, BLK>), dim3(s.C, s.B * s.Hkv), dim3(64), lds,
                     st, a);
  return hipGetLastError();
}

// Dispatch over (dtype, D, blk).
template <typename Fn>
hipError_t dispatch(const Shape& s, Fn&& fn) {
  if (s.fp32) {
    if (s.D == 64) {
      if (s.blk == 16) return fn((float*)nullptr, std::integral_constant<int, 64>{}, std::integral_constant<int, 16>{});
      if (s.blk == 32) return fn((float*)nullptr, std::integral_constant<int, 64>{}, std::integral_constant<int, 32>{});
      return fn((float*)nullptr, std::integral_constant<int, 64>{}, std::integral_constant<int, 64>{});
    }
    if (s.blk == 16) return fn((float*)nullptr, std::integral_constant<int, 128>{}, std::integral_constant<int, 16>{});
    if (s.blk == 32) return fn((float*)nullptr, std::integral_constant<int, 128>{}, std::integral_constant<int, 32>{});
    return fn((float*)nullptr, std::integral_constant<int, 128>{}, std::integral_constant<int, 64>{});
  }
  if (s.D == 64) {
    if (s.blk == 16) return fn((__bf16*)nullptr, std::integral_constant<int, 64>{}, std::integral_constant<int, 16>{});
    if (s.blk == 32) return fn((__bf16*)nullptr, std::integral_constant<int, 64>{}, std::integral_constant<int, 32>{});
    return fn((__bf16*)nullptr, std::integral_constant<int, 64>{}, std::integral_constant<int, 64>{});
  }
  if (s.blk == 16) return fn((__bf16*)nullptr, std::integral_constant<int, 128>{}, std::integral_constant<int, 16>{});
  if (s.blk == 32) return fn((__bf16*)nullptr, std::integral_constant<int, 128>{}, std::integral_constant<int, 32>{});
  return fn((__bf16*)nullptr, std::integral_constant<int, 128>{}, std::integral_constant<int, 64>{});
}

}  // namespace

hipError_t launch_fwd_generic(const Shape& s, const void* q, const void* k, const void* v,
                              const float* log_gate, const int32_t* sel_idx,
                              const int32_t* sel_cnt, void* o, float* lse, hipStream_t st) {
  GenArgs a = make_args(s);
  a.q = q; a.k = k; a.v = v; a.lg = log_gate; a.sel_idx = sel_idx; a.sel_cnt = sel_cnt;
  a.out = o; a.lse_out = lse;
  return dispatch(s, [&](auto tp, auto dc, auto bc) {
    using T = std::remove_pointer_t<decltype(tp)>;
    return fwd_launch<T, decltype(dc)::value, decltype(bc)::value>(a, s, st);
  });
}

GenArgs bwd_args(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl) {
  GenArgs a = make_args(s);
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.d_o = p.d_o; a.lse = p.lse; a.lg = p.log_gate;
  a.sel_idx = p.sel_idx; a.sel_cnt = p.sel_cnt; a.dq = p.dq; a.dk = p.dk; a.dv = p.dv;
  a.dlg = p.dlog_gate;
  a.delta = (float*)(ws + wl.delta);
  return a;
}

hipError_t launch_bwd_dq_generic(const Shape& s, const BwdPtrs& p, char* ws,
                                 const BwdWorkspace& wl, hipStream_t st) {
  const GenArgs a = bwd_args(s, p, ws, wl);
  hipError_t e = dispatch(s, [&](auto tp, auto dc, auto bc) {
    using T = std::remove_pointer_t<decltype(tp)>;
    return bwd_q_launch<T, decltype(dc)::value, decltype(bc)::value>(a, s, st);
  });
  return e;
}

// Gate gradients of the dropped blocks of hard Top-K gates (any path: the
// workspace's Delta array has the same layout on both).
hipError_t launch_ste_dropped(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl,
                              hipStream_t st) {
  const GenArgs a = bwd_args(s, p, ws, wl);
  return dispatch(s, [&](auto tp, auto dc, auto bc) {
    using T = std::remove_pointer_t<decltype(tp)>;
    constexpr int D = decltype(dc)::value, BLK = decltype(bc)::value;
    const size_t lds = 2 * BLK * D * sizeof(float);
    hipLaunchKernelGGL((ste_dropped_kernel<T, D, BLK>), dim3(s.C, s.B * s.Hs), dim3(64), lds, st,
                       a);
    return hipGetLastError();
  });
}

hipError_t launch_bwd_dkdv_generic(const Shape& s, const BwdPtrs& p, char* ws,
                                   const BwdWorkspace& wl, hipStream_t st) {
  const GenArgs a = bwd_args(s, p, ws, wl);
  hipError_t e = dispatch(s, [&](auto tp, auto dc, auto bc) {
    using T = std::remove_pointer_t<decltype(tp)>;
    return bwd_kv_launch<T, decltype(dc)::value, decltype(bc)::value>(a, s, st);
  });
  if (e == hipSuccess && s.hard) e = launch_ste_dropped(s, p, ws, wl, st);
  if (e != hipSuccess || p.dscores == nullptr) return e;
  return launch_dscores(s, p.dlog_gate, p.log_gate, p.dscores, nullptr, nullptr, st);
}

}  // namespace sas
