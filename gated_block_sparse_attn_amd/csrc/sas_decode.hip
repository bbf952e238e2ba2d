// Sparse decode: one new query token per sequence attends its current block
// and the Top-K blocks chosen from the selector scores, gathered from a paged
// KV cache.
//
// SAS paper (arXiv 2609.13141): Sec. 4.3 Alg. 2 (inference step: I =
// Top-K(s, K), S = B0 u U_{m in I} B_m, o = softmax(q K_S^T) V_S, no gates);
// Sec. 5.1 "Inference implementation" (per-query-group selection with GQA,
// only the selected KV blocks are gathered from the paged cache, batched
// decoding); Sec. 6.3 / Fig. 7(c) (Top-K ranking dominates the step at long
// context, so the selection gets a workgroup per row).
//
// Kernels:
//   decode_select_kernel   one workgroup per (sequence, kv head): holds the
//                          row's historical scores as order-preserving
//                          integer keys in registers, bounds the K-th
//                          largest from below by the group maxima (a value
//                          histogram when that bound does not narrow it
//                          enough), finds it exactly among the few keys
//                          above the bound, then compacts {m : key >= tau}
//                          in ascending order.
//   decode_attn_kernel     one workgroup per (sequence, kv head, tile): tile
//                          0 is the current block (tokens up to the query),
//                          tile t >= 1 the (t-1)-th selected block.  The K / V
//                          block is read once from its page (shared by the G
//                          query heads of the group), scores and the tile's
//                          softmax statistics go to a workspace partial.
//   decode_combine_kernel  one wavefront per (sequence, query head): merges
//                          the partials in tile order (deterministic).
// All three are memory-bound: HBM bytes are the selected K / V blocks.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "../../include/sas.h"
#include "sas_internal.h"

namespace sas {
namespace {

__device__ __forceinline__ uint32_t f2key(float x) {
  const uint32_t b = __float_as_uint(x);
  return b ^ ((b >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float(k ^ ((k >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}
__device__ __forceinline__ int rank_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Current block of a sequence of n tokens (query at position n - 1), with n
// clamped into [1, cmax * blk]; *bad is set when n was out of range.
__device__ __forceinline__ int current_block(int n, int blk, int cmax, int* nn, bool* bad) {
  int v = n;
  if (v < 1 || v > cmax * blk) {
    *bad = true;
    v = v < 1 ? 1 : cmax * blk;
  }
  *nn = v;
  return (v - 1) / blk;
}

// Per (sequence, kv head) row: the threshold T is the K-th largest of the c_s
// historical scores, over order-preserving integer keys held in registers
// (thread t holds blocks t KPT .. t KPT + KPT - 1).  The row is cut into 128
// groups of consecutive threads.  When K <= 128, T is at least the K-th
// largest group maximum (K groups each hold a key at or above it), so every
// key >= T lies in that maximum's bin of a 256-bin histogram of the group
// maxima (bins linear in the score between the row's minimum and maximum) or
// above it -- usually a few keys beyond K.  Those keys go to an LDS list and
// each finds its rank among the others; the one with fewer than K above it
// and at least K at or above it is T.  Without such a bound, or when the
// list overflows (dense ties), 256-bin histograms of the remaining keys
// (linear in the score, then in the integer key) narrow the range level by
// level until it fits the list.  Then the ascending compaction
// {m < c_s : key_m >= T} from a scan of per-thread counts.
constexpr int kSelMaxThreads = 1024;   // 256 for rows of up to 1024 blocks, 1024 otherwise
constexpr int kSelGroups = 128;
constexpr int kSelBins = 256;
constexpr int kSelCand = 256;          // keys the exact search takes

// DPP lane exchanges (rows of 16 lanes): quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror, row_shr:n, row_bcast:15 / :31
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}
// max over aligned groups of S lanes (S = 2, 8 or 16), in every lane
template <int S>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  v = max(v, dpp<0xB1>(v, v));
  if (S >= 4) v = max(v, dpp<0x4E>(v, v));
  if (S >= 8) v = max(v, dpp<0x141>(v, v));
  if (S >= 16) v = max(v, dpp<0x140>(v, v));
  return v;
}
__device__ __forceinline__ uint32_t row_min(uint32_t v) {
  v = min(v, dpp<0xB1>(v, v));
  v = min(v, dpp<0x4E>(v, v));
  v = min(v, dpp<0x141>(v, v));
  return min(v, dpp<0x140>(v, v));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = row_min(v);
  const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return min(a, b);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = group_max<16>(v);
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_incl_scan(int v) {
  uint32_t u = (uint32_t)v;
  u += dpp<0x111>(0u, u);
  u += dpp<0x112>(0u, u);
  u += dpp<0x114>(0u, u);
  u += dpp<0x118>(0u, u);
  u += dpp<0x142, 0xA>(0u, u);
  u += dpp<0x143, 0xC>(0u, u);
  return (int)u;
}

// 256 bins over the keys in [lo, hi], non-decreasing in the key: linear in
// the score when allowed and the range is finite and resolvable in fp32,
// else 2^sh-wide key bins
struct KeyBins {
  uint32_t lo;
  float flo, scale;
  int sh;
  bool byval;
  __device__ KeyBins(uint32_t lo_, uint32_t hi, bool by_value) : lo(lo_) {
    flo = key2f(lo);
    const float span = key2f(hi) - flo;
    scale = kSelBins / span;
    byval = by_value && isfinite(flo) && isfinite(span) && isfinite(scale) && scale > 0.0f;
    sh = hi == lo ? 0 : max(0, 24 - __builtin_clz(hi - lo));   // (hi - lo) >> sh < 256
  }
  __device__ int operator()(uint32_t k) const {
    if (byval) return min((int)((key2f(k) - flo) * scale), kSelBins - 1);
    return (int)((k - lo) >> sh);
  }
};

template <int KPT>
__global__ void __launch_bounds__(kSelMaxThreads) decode_select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    float* __restrict__ tau, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
    int32_t* __restrict__ d_status, int Hkv, int cmax, int blk, int K, int cap) {
  __shared__ int s_hist[kSelBins];
  __shared__ __align__(16) uint32_t s_cand[kSelCand];
  __shared__ uint32_t s_gmax[kSelGroups];
  __shared__ int s_wsum[kSelMaxThreads / 64];
  __shared__ int s_pick[3];                    // boundary bin, keys above it, keys in it
  __shared__ uint32_t s_ext[2];                // boundary-bin key range (row maximum first)
  __shared__ int s_ncand;
  __shared__ uint32_t s_t;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int nw = nthr >> 6;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const long long row = blockIdx.x;            // b * Hkv + h
  const int b = (int)(row / Hkv);
  int n;
  bool bad = false;
  const int c = current_block(seq_lens[b], blk, cmax, &n, &bad);
  const float* srow = scores + row * (long long)cmax;
  const int m0 = tid * KPT;
  // the loads do not wait for the length: every m < cmax is in the row
  float raw[KPT];
  if (KPT % 4 == 0 && (cmax & 3) == 0 && ((uintptr_t)srow & 15) == 0) {
#pragma unroll
    for (int j = 0; j < KPT / 4; ++j) {
      const float4 v = m0 + 4 * j < cmax ? *(const float4*)(srow + m0 + 4 * j)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
      raw[4 * j] = v.x; raw[4 * j + 1] = v.y; raw[4 * j + 2] = v.z; raw[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int x = 0; x < KPT; ++x) raw[x] = m0 + x < cmax ? srow[m0 + x] : 0.f;
  }
  const int nv = min(max(c - m0, 0), KPT);     // historical blocks this thread holds
  uint32_t key[KPT];
#pragma unroll
  for (int x = 0; x < KPT; ++x) key[x] = x < nv ? f2key(raw[x] + 0.0f) : 0u;   // -0 -> +0

  uint32_t tkey;   // select m iff key >= tkey; none when K == 0
  bool none = false;
  if (K >= c) {
    tkey = 0u;
  } else if (K == 0) {
    tkey = 0xFFFFFFFFu;
    none = true;
  } else {
    // group maxima: groups of nthr / 128 threads (2 or 8)
    uint32_t hi = 0u;
#pragma unroll
    for (int x = 0; x < KPT; ++x)
      if (x < nv) hi = max(hi, key[x]);
    const int gs = nthr / kSelGroups;
    const uint32_t gm = gs == 8 ? group_max<8>(hi) : group_max<2>(hi);
    if ((lane & (gs - 1)) == 0) s_gmax[tid / gs] = gm;
    for (int i = tid; i < kSelBins; i += nthr) s_hist[i] = 0;
    if (tid == 0) s_ncand = 0;
    __syncthreads();
    if (w == 0) {
      // groups holding at least one historical block; their maxima span the row's keys' top
      const int ng = min(kSelGroups, (c + gs * KPT - 1) / (gs * KPT));
      const bool v0 = lane < ng, v1 = lane + 64 < ng;
      const uint32_t g0 = s_gmax[lane], g1 = s_gmax[lane + 64];
      const uint32_t ghi = wave_max_u32(max(v0 ? g0 : 0u, v1 ? g1 : 0u));
      uint32_t l0 = 0u;
      if (K <= ng) {
        // T is at least the K-th largest group maximum, so at least the
        // smallest group maximum in that maximum's bin or above
        const uint32_t glo = wave_min_u32(min(v0 ? g0 : 0xFFFFFFFFu, v1 ? g1 : 0xFFFFFFFFu));
        const KeyBins bins(glo, ghi, true);
        const int b0 = v0 ? bins(g0) : -1, b1 = v1 ? bins(g1) : -1;
        if (v0) atomicAdd(&s_hist[b0], 1);
        if (v1) atomicAdd(&s_hist[b1], 1);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
        // lane l holds bins 255 - 4l .. 252 - 4l (descending); the inclusive
        // scan over lanes counts the maxima in bins >= 252 - 4l
        int v4[4], v = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) { v4[x] = s_hist[kSelBins - 1 - 4 * lane - x]; v += v4[x]; }
        const int incl = wave_incl_scan(v);
        const int L = __builtin_ctzll(__ballot(incl >= K));   // K <= ng: some lane hits
        int cum = incl - v, x = 0;
        while (x < 3 && cum + v4[x] < K) cum += v4[x++];
        const int blo = __builtin_amdgcn_readlane(kSelBins - 1 - 4 * lane - x, L);
        l0 = wave_min_u32(min(v0 && b0 >= blo ? g0 : 0xFFFFFFFFu, v1 && b1 >= blo ? g1 : 0xFFFFFFFFu));
      }
      if (lane == 0) { s_t = l0; s_ext[1] = ghi; }
    }
    __syncthreads();
    const uint32_t l0 = s_t;       // every key >= T is >= l0
    uint32_t rhi = s_ext[1];       // the row's largest key
    // keys >= l0 into the list (when they fit)
    unsigned long long bits[KPT];
    int tot = 0;
#pragma unroll
    for (int x = 0; x < KPT; ++x) {
      bits[x] = __ballot(x < nv && key[x] >= l0);
      tot += __popcll(bits[x]);
    }
    int base = 0;
    if (lane == 0 && tot > 0) base = atomicAdd(&s_ncand, tot);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int x = 0; x < KPT; ++x) {
      if ((bits[x] >> lane) & 1ull) {
        const int pos = base + rank_below(bits[x]);
        if (pos < kSelCand) s_cand[pos] = key[x];
      }
      base += __popcll(bits[x]);
    }
    for (int i = tid; i < kSelBins; i += nthr) s_hist[i] = 0;
    __syncthreads();
    {
      int nb = s_ncand;
      int kk = K;
      uint32_t rlo = l0;
      bool fits = nb <= kSelCand;
      for (int level = 0; !fits && rlo != rhi; ++level) {
        // keys in [rlo, rhi] (more than the list holds) rank kk-th among
        // themselves; bins linear in the score at the first level only
        const KeyBins bin_of(rlo, rhi, level == 0);
#pragma unroll
        for (int x = 0; x < KPT; ++x)
          if (x < nv && key[x] >= rlo && key[x] <= rhi) atomicAdd(&s_hist[bin_of(key[x])], 1);
        __syncthreads();
        if (w == 0) {
          // lane l holds bins 255 - 4l .. 252 - 4l (descending); the
          // inclusive scan over lanes counts the keys in bins >= 252 - 4l
          int v4[4], v = 0;
#pragma unroll
          for (int x = 0; x < 4; ++x) { v4[x] = s_hist[kSelBins - 1 - 4 * lane - x]; v += v4[x]; }
          const int incl = wave_incl_scan(v);
          const unsigned long long hit = __ballot(incl >= kk);
          const int L = __builtin_ctzll(hit);  // kk <= keys in range, so some lane hits
          if (lane == L) {
            int cum = incl - v;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              if (cum + v4[x] >= kk) {
                s_pick[0] = kSelBins - 1 - 4 * lane - x;
                s_pick[1] = cum;
                s_pick[2] = v4[x];
                break;
              }
              cum += v4[x];
            }
          }
          if (lane == 0) { s_ext[0] = 0xFFFFFFFFu; s_ext[1] = 0u; s_ncand = 0; }
        }
        __syncthreads();
        const int bsel = s_pick[0];
        kk -= s_pick[1];
        nb = s_pick[2];
        fits = nb <= kSelCand;
        // the boundary bin's keys: their range, and the keys themselves when
        // the list holds them all
        uint32_t cl = 0xFFFFFFFFu, ch = 0u;
#pragma unroll
        for (int x = 0; x < KPT; ++x) {
          const uint32_t k = key[x];
          const bool in = x < nv && k >= rlo && k <= rhi && bin_of(k) == bsel;
          if (in) { cl = min(cl, k); ch = max(ch, k); }
          if (fits) {
            const unsigned long long bb = __ballot(in);
            if (bb != 0ull) {
              const int first = __builtin_ctzll(bb);
              int bs = 0;
              if (lane == first) bs = atomicAdd(&s_ncand, __popcll(bb));
              bs = __builtin_amdgcn_readlane(bs, first);
              if (in) s_cand[bs + rank_below(bb)] = k;
            }
          }
        }
        cl = wave_min_u32(cl);
        ch = wave_max_u32(ch);
        if (lane == 0 && ch >= cl) { atomicMin(&s_ext[0], cl); atomicMax(&s_ext[1], ch); }
        for (int i = tid; i < kSelBins; i += nthr) s_hist[i] = 0;
        __syncthreads();
        rlo = s_ext[0];
        rhi = s_ext[1];
      }
      if (rlo == rhi) {
        tkey = rlo;
      } else {
        // the list holds every key in [rlo, rhi] (nb of them); the kk-th
        // largest is the entry with fewer than kk entries above it and at
        // least kk at or above it
        if (tid < nb) {
          const uint32_t ci = s_cand[tid];
          int gt = 0, ge = 0;
          const uint4* c4 = (const uint4*)s_cand;
          int j = 0;
          for (; j + 16 <= nb; j += 16) {   // four 16-byte reads in flight
            uint4 q[4];
#pragma unroll
            for (int y = 0; y < 4; ++y) q[y] = c4[(j >> 2) + y];
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              gt += (q[y].x > ci) + (q[y].y > ci) + (q[y].z > ci) + (q[y].w > ci);
              ge += (q[y].x >= ci) + (q[y].y >= ci) + (q[y].z >= ci) + (q[y].w >= ci);
            }
          }
          for (; j + 4 <= nb; j += 4) {
            const uint4 q = c4[j >> 2];
            gt += (q.x > ci) + (q.y > ci) + (q.z > ci) + (q.w > ci);
            ge += (q.x >= ci) + (q.y >= ci) + (q.z >= ci) + (q.w >= ci);
          }
          for (; j < nb; ++j) {
            const uint32_t q = s_cand[j];
            gt += q > ci;
            ge += q >= ci;
          }
          if (gt < kk && kk <= ge) s_t = ci;   // every such entry holds the same key
        }
        __syncthreads();
        tkey = s_t;
      }
    }
  }

  // ascending compaction: the output position of thread tid's selected
  // blocks is the number selected by lower threads plus its own earlier ones
  int mine = 0;
#pragma unroll
  for (int x = 0; x < KPT; ++x) mine += (!none && x < nv && key[x] >= tkey) ? 1 : 0;
  const int incl = wave_incl_scan(mine);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  // lane y < nw holds wave y's count; their scan gives this wave's offset
  // and the total
  const int wc = lane < nw ? s_wsum[lane] : 0;
  const int wincl = wave_incl_scan(wc);
  const int total = __builtin_amdgcn_readlane(wincl, 63);
  int pos = incl - mine + (w > 0 ? __builtin_amdgcn_readlane(wincl, w - 1) : 0);
  int32_t* out = sel_idx + row * (long long)cap;
#pragma unroll
  for (int x = 0; x < KPT; ++x) {
    if (!none && x < nv && key[x] >= tkey) {
      if (pos < cap) out[pos] = m0 + x;
      ++pos;
    }
  }
  for (int p = total + tid; p < cap; p += nthr) out[p] = -1;
  if (tid == 0) {
    sel_cnt[row] = total;
    if (tau != nullptr) tau[row] = (K >= c) ? -INFINITY : (none ? INFINITY : key2f(tkey));
    if (d_status != nullptr) {
      if (bad) *d_status = SAS_E_INVALID;
      else if (total > cap) *d_status = SAS_E_CAPACITY;
    }
  }
}

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return (float)(*p); }

// 16-byte chunk of T values -> float
template <typename T> struct Chunk;
template <> struct Chunk<__bf16> {
  static constexpr int N = 8;
  __device__ static void get(const uint4& u, float* f) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    const bf16x8 v = __builtin_bit_cast(bf16x8, u);
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] = (float)v[x];
  }
};
template <> struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void get(const uint4& u, float* f) {
    const float4 v = __builtin_bit_cast(float4, u);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
};
// two consecutive T values -> float
__device__ __forceinline__ float2 get2(const __bf16* p) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = *(const bf16x2*)p;
  return make_float2((float)v[0], (float)v[1]);
}
__device__ __forceinline__ float2 get2(const float* p) { return *(const float2*)p; }

struct DecArgs {
  const void* q; const void* kp; const void* vp; const int32_t* bt; const int32_t* seq_lens;
  const int32_t* sel_idx; const int32_t* sel_cnt; void* o; float* lse; float* part;
  int32_t* d_status;
  int Hq, Hkv, G, cmax, pool, cap, T;
  float c2;   // sm_scale * log2(e)
};

constexpr int kAttnThreads = 256;

// LDS bytes of one decode_attn_kernel workgroup: K and V blocks in the input
// type, the G scaled queries and the G x BLK probabilities in fp32.
template <typename T, int D, int BLK>
constexpr size_t attn_lds(int G) {
  return 2 * (size_t)BLK * D * sizeof(T) + sizeof(float) * ((size_t)G * D + (size_t)G * BLK);
}

template <typename T, int D, int BLK>
__global__ void __launch_bounds__(kAttnThreads) decode_attn_kernel(DecArgs a) {
  constexpr int EPC = Chunk<T>::N;       // elements per 16-byte chunk
  constexpr int NCH = D / EPC;           // chunks per row
  constexpr int SWM = NCH < 16 ? NCH - 1 : 15;
  extern __shared__ uint4 smem4[];
  uint4* ks = smem4;                     // BLK x NCH chunks; chunk c of row r at c ^ (r & SWM)
  uint4* vs = ks + BLK * NCH;            // BLK x NCH chunks, row-major
  float* qs = (float*)(vs + BLK * NCH);  // G x D, pre-scaled by c2
  float* ps = qs + a.G * D;              // G x BLK
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;             // b * Hkv + hk
  const int t = blockIdx.y;              // 0: current block, t >= 1: selected entry t - 1
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.G;
  int n;
  bool bad = false;
  const int c = current_block(a.seq_lens[b], BLK, a.cmax, &n, &bad);
  const int cnt = min(max(a.sel_cnt[bh], 0), a.cap);
  float* part = a.part + ((long long)bh * a.T + t) * G * (D + 2);

  int blkid = c, nkeys = n - c * BLK;
  if (t > 0) {
    if (t > cnt) {   // no such tile: empty partial
      for (int hh = tid; hh < G; hh += kAttnThreads) {
        part[hh * (D + 2) + D] = -INFINITY;
        part[hh * (D + 2) + D + 1] = 0.0f;
      }
      return;
    }
    blkid = a.sel_idx[(long long)bh * a.cap + t - 1];
    nkeys = BLK;
    if (blkid < 0 || blkid >= c) {   // not a historical block: flag, attend nothing
      bad = true;
      nkeys = 0;
      blkid = 0;
    }
  }
  int page = a.bt[(long long)b * a.cmax + blkid];
  if (page < 0 || page >= a.pool) {
    bad = true;
    page = 0;
    nkeys = 0;
  }
  if (bad && tid == 0 && a.d_status != nullptr) *a.d_status = SAS_E_INVALID;

  // stage the K / V block (16-byte chunks) and the scaled queries
  const uint4* kg = (const uint4*)((const T*)a.kp + (((long long)page * a.Hkv + hk) * BLK) * D);
  const uint4* vg = (const uint4*)((const T*)a.vp + (((long long)page * a.Hkv + hk) * BLK) * D);
  constexpr int TOTAL = BLK * NCH;
  constexpr bool EVEN = TOTAL % kAttnThreads == 0;
  constexpr int PER = (TOTAL + kAttnThreads - 1) / kAttnThreads;   // chunks per thread
  uint4 kr[PER], vr[PER];
#pragma unroll
  for (int x = 0; x < PER; ++x) {   // every load issued before the first LDS store
    const int ch = tid + x * kAttnThreads;
    kr[x] = make_uint4(0u, 0u, 0u, 0u);
    vr[x] = kr[x];
    if (EVEN || ch < TOTAL) {
      kr[x] = kg[ch];
      vr[x] = vg[ch];
    }
  }
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    const int ch = tid + x * kAttnThreads;
    if (EVEN || ch < TOTAL) {
      const int r = ch / NCH, cc = ch % NCH;
      ks[r * NCH + (cc ^ (r & SWM))] = kr[x];
      vs[ch] = vr[x];
    }
  }
  const T* qg = (const T*)a.q + ((long long)b * a.Hq + hk * G) * D;
  for (int e = tid; e < G * D; e += kAttnThreads) qs[e] = ld(qg + e) * a.c2;
  __syncthreads();

  // scores (log2 units) and the tile's softmax statistics: pair (hh, kk),
  // kk fastest, so each head's BLK keys are one aligned segment of a wavefront
  for (int pr0 = 0; pr0 < G * BLK; pr0 += kAttnThreads) {
    const int pr = pr0 + tid;
    const int hh = pr / BLK, kk = pr % BLK;
    float z = -INFINITY;
    if (hh < G && kk < nkeys) {
      float acc = 0.0f;
#pragma unroll 4
      for (int cc = 0; cc < NCH; ++cc) {
        float kf[EPC];
        Chunk<T>::get(ks[kk * NCH + (cc ^ (kk & SWM))], kf);
        const float* qp = qs + hh * D + cc * EPC;
#pragma unroll
        for (int x = 0; x < EPC; ++x) acc = fmaf(qp[x], kf[x], acc);
      }
      z = acc;
    }
    float mx = z;
#pragma unroll
    for (int o = BLK / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float p = (mx == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z - mx);
    float l = p;
#pragma unroll
    for (int o = BLK / 2; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
    if (hh < G) {
      ps[hh * BLK + kk] = p;
      if (kk == 0) {
        part[hh * (D + 2) + D] = mx;
        part[hh * (D + 2) + D + 1] = l;
      }
    }
  }
  __syncthreads();

  // unnormalised output of the tile: acc[hh][d] = sum_kk p[hh][kk] v[kk][d]
  const T* vrow = (const T*)vs;
  for (int e = tid; e < G * (D / 2); e += kAttnThreads) {
    const int hh = e / (D / 2), d = (e % (D / 2)) * 2;
    float o0 = 0.0f, o1 = 0.0f;
    for (int kk = 0; kk < nkeys; ++kk) {
      const float p = ps[hh * BLK + kk];
      const float2 v2 = get2(vrow + kk * D + d);
      o0 = fmaf(p, v2.x, o0);
      o1 = fmaf(p, v2.y, o1);
    }
    part[hh * (D + 2) + d] = o0;
    part[hh * (D + 2) + d + 1] = o1;
  }
}

// ---- matrix-core tile kernel (bf16, D = 128, b = 64, G <= 32) ----
// One wavefront per (sequence, kv head, tile), the same partials as
// decode_attn_kernel.  The G query heads are the columns of two 32x32x16
// MFMA products: S^T = K Q^T (A: key rows of the block, read straight from
// the page; B: the heads' queries, columns >= G zero) and O^T = V^T P^T (A:
// transposed reads of the V block staged in LDS; B: the bf16 probabilities,
// whose accumulator layout already is the B operand's).  Each head's 64
// scores sit in one column, i.e. in lanes h and h + 32.
typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 dbf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 dbf16x2 __attribute__((ext_vector_type(2)));
typedef float df32x16 __attribute__((ext_vector_type(16)));
typedef float df32x4 __attribute__((ext_vector_type(4)));
typedef float df32x2 __attribute__((ext_vector_type(2)));
constexpr int kMD = 128, kMB = 64;

// element offset of 16-byte chunk c of row r in the staged V block
__device__ __forceinline__ int dswz(int r, int c) { return r * kMD + ((c ^ slot16(r)) << 3); }
// gfx950 transposed LDS read: within each 16-lane group, lane u gets element
// u % 4 of the 8-byte chunks addressed by lanes u / 4 + 4x (x = 0..3)
__device__ __forceinline__ dbf16x4 dread_tr(const __bf16* p) {
  typedef __attribute__((address_space(3))) dbf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}
// v_mfma_f32_32x32x16_bf16: lane l (g = l / 32): A row l % 32, k = 8 g .. +7;
// B column l % 32, same k; C column l % 32, rows 8 (jj / 4) + 4 g + jj % 4
__device__ __forceinline__ df32x16 dmfma(dbf16x8 a, dbf16x8 b, df32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// max / sum over the lanes l and l ^ 32 (the two lanes of a C column)
__device__ __forceinline__ float dmax2(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float dsum2(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ void __launch_bounds__(64) decode_attn_mfma_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 vs[kMB * kMD];
  const int lane = threadIdx.x;
  const int g = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x;             // b * Hkv + hk
  const int t = blockIdx.y;              // 0: current block, t >= 1: selected entry t - 1
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.G;
  int n;
  bool bad = false;
  const int c = current_block(a.seq_lens[b], kMB, a.cmax, &n, &bad);
  const int cnt = min(max(a.sel_cnt[bh], 0), a.cap);
  float* part = a.part + ((long long)bh * a.T + t) * G * (kMD + 2);

  int blkid = c, nkeys = n - c * kMB;
  if (t > 0) {
    if (t > cnt) {   // no such tile: empty partial
      if (lane < G) {
        part[lane * (kMD + 2) + kMD] = -INFINITY;
        part[lane * (kMD + 2) + kMD + 1] = 0.0f;
      }
      return;
    }
    blkid = a.sel_idx[(long long)bh * a.cap + t - 1];
    nkeys = kMB;
    if (blkid < 0 || blkid >= c) {   // not a historical block: flag, attend nothing
      bad = true;
      nkeys = 0;
      blkid = 0;
    }
  }
  int page = a.bt[(long long)b * a.cmax + blkid];
  if (page < 0 || page >= a.pool) {
    bad = true;
    page = 0;
    nkeys = 0;
  }
  if (bad && lane == 0 && a.d_status != nullptr) *a.d_status = SAS_E_INVALID;

  const __bf16* kg = (const __bf16*)a.kp + (((long long)page * a.Hkv + hk) * kMB) * kMD;
  const __bf16* vg = (const __bf16*)a.vp + (((long long)page * a.Hkv + hk) * kMB) * kMD;
  // V block -> LDS: 16 asynchronous copies of 1 KB (rows 4 s .. 4 s + 3), each
  // lane fetching the chunk that its LDS slot holds under the swizzle
#pragma unroll
  for (int sg = 0; sg < 16; ++sg) {
    const int row = sg * 4 + (lane >> 4);
    const int ch = (lane & 15) ^ slot16(row);
    dma16(vg + row * kMD + ch * 8, lds_addr(vs + sg * 512));
  }
  // K rows (A operand): key kh * 32 + l32, dims ks * 16 + 8 g .. +7
  dbf16x8 ka[2][8];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      ka[kh][ks] = *(const dbf16x8*)(kg + (kh * 32 + l32) * kMD + ks * 16 + g * 8);
  // queries (B operand): head l32 of the group, dims ks * 16 + 8 g .. +7
  dbf16x8 qf[8];
  const __bf16* qg = (const __bf16*)a.q + ((long long)b * a.Hq + hk * G + min(l32, G - 1)) * kMD;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qf[ks] = *(const dbf16x8*)(qg + ks * 16 + g * 8);
    if (l32 >= G) qf[ks] = dbf16x8{};
  }
  // S^T of the two 32-key halves
  df32x16 sc[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    sc[kh] = df32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sc[kh] = dmfma(ka[kh][ks], qf[ks], sc[kh]);
  }
  // the head's softmax statistics over the tile (log2 units; keys past the
  // query are masked)
  float mx = -INFINITY;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int key = kh * 32 + 8 * (jj >> 2) + 4 * g + (jj & 3);
      const float z = key < nkeys ? sc[kh][jj] * a.c2 : -INFINITY;
      sc[kh][jj] = z;
      mx = fmaxf(mx, z);
    }
  mx = dmax2(mx);
  float l = 0.0f;
  dbf16x8 pb[2][2];   // [half][16-key slice]: B operand of O^T
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int jj = 0; jj < 16; jj += 2) {
      df32x2 pp;
      pp[0] = mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[kh][jj] - mx);
      pp[1] = mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[kh][jj + 1] - mx);
      l += pp[0] + pp[1];
      const dbf16x2 h2 = __builtin_convertvector(pp, dbf16x2);
      pb[kh][jj >> 3][jj & 7] = h2[0];
      pb[kh][jj >> 3][(jj & 7) + 1] = h2[1];
    }
  l = dsum2(l);
  // O^T = V^T P^T: head-dim tiles dt, A fragments (dims dt * 32 + l32, keys
  // 16 sl + {4 g .. 4 g + 3, 8 + 4 g .. 8 + 4 g + 3}) by transposed reads
  const int u = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the V copies (and loads) landed
  __syncthreads();
  df32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    oacc[dt] = df32x16{};
    const int o0 = dswz(g * 4 + (u >> 2), dt * 4 + dhalf * 2 + ((u >> 1) & 1)) + (u & 1) * 4;
    const int o1 = dswz(g * 4 + (u >> 2) + 8, dt * 4 + dhalf * 2 + ((u >> 1) & 1)) + (u & 1) * 4;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const __bf16* vp = vs + (kh * 32 + sl * 16) * kMD;
        const dbf16x8 va = __builtin_shufflevector(dread_tr(vp + o0), dread_tr(vp + o1),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
        oacc[dt] = dmfma(va, pb[kh][sl], oacc[dt]);
      }
  }
  // partial of head l32: unnormalised output (dims dt * 32 + 8 q4 + 4 g .. +3), max, sum
  if (l32 < G) {
    float* ph = part + l32 * (kMD + 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int y = 0; y < 4; ++y) ph[dt * 32 + q4 * 8 + g * 4 + y] = oacc[dt][q4 * 4 + y];
    if (g == 0) {
      ph[kMD] = mx;
      ph[kMD + 1] = l;
    }
  }
}

// merge the tile partials of one (sequence, query head): wavefront w takes
// tiles w, w + 4, ..., loads up to kCombBatch of them at once (one memory
// round trip) and folds them in tile order into a running (max, sum,
// output) with the online-softmax rescale; the four wavefronts' results are
// then rescaled to the common max and added in wave order (deterministic).
constexpr int kCombWaves = 4;
constexpr int kCombBatch = 16;

template <typename T, int D>
__global__ void __launch_bounds__(64 * kCombWaves) decode_combine_kernel(DecArgs a) {
  constexpr int PER = D / 64;   // output values per lane
  __shared__ float s_red[kCombWaves][D + 2];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int bq = blockIdx.x;                  // b * Hq + h
  const int b = bq / a.Hq, h = bq % a.Hq;
  const int hk = h / a.G, hh = h % a.G;
  const int bh = b * a.Hkv + hk;
  const int cnt_raw = a.sel_cnt[bh];
  const float* p0 = a.part + (long long)bh * a.T * a.G * (D + 2) + hh * (D + 2);
  const long long stride = (long long)a.G * (D + 2);
  float mw = -INFINITY, lw = 0.0f;
  float acc[PER];
#pragma unroll
  for (int x = 0; x < PER; ++x) acc[x] = 0.0f;
  // this wavefront's tiles: w + kCombWaves * j.  The first batch is read for
  // every tile slot (all T slots lie in the buffer) together with the
  // count, so that one memory latency serves both; slots past the count are
  // skipped below (their O was never written).
  auto fold = [&](float m, float l, const float (&ov)[PER]) {
    const float mn = fmaxf(mw, m);
    const float so = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mn);
    const float sn = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    lw = lw * so + l * sn;
#pragma unroll
    for (int x = 0; x < PER; ++x) acc[x] = acc[x] * so + ov[x] * sn;
    mw = mn;
  };
  const int nw_cap = a.T > w ? (a.T - w + kCombWaves - 1) / kCombWaves : 0;
  const int n0 = min(kCombBatch, nw_cap);
  {
    float mt[kCombBatch], lt[kCombBatch], ot[kCombBatch][PER];
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      if (j < n0) {
        const float* pt = p0 + (long long)(w + kCombWaves * j) * stride;
        mt[j] = pt[D];
        lt[j] = pt[D + 1];
#pragma unroll
        for (int x = 0; x < PER; ++x) ot[j][x] = pt[x * 64 + lane];
      }
    }
    const int nt = min(max(cnt_raw, 0), a.cap) + 1;
    const int nw = nt > w ? (nt - w + kCombWaves - 1) / kCombWaves : 0;
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j)
      if (j < min(n0, nw)) fold(mt[j], lt[j], ot[j]);
  }
  const int nt = min(max(cnt_raw, 0), a.cap) + 1;
  const int nw = nt > w ? (nt - w + kCombWaves - 1) / kCombWaves : 0;
  for (int j0 = kCombBatch; j0 < nw; j0 += kCombBatch) {
    const int n = min(kCombBatch, nw - j0);
    float mt[kCombBatch], lt[kCombBatch], ot[kCombBatch][PER];
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      if (j < n) {
        const float* pt = p0 + (long long)(w + kCombWaves * (j0 + j)) * stride;
        mt[j] = pt[D];
        lt[j] = pt[D + 1];
#pragma unroll
        for (int x = 0; x < PER; ++x) ot[j][x] = pt[x * 64 + lane];
      }
    }
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j)
      if (j < n) fold(mt[j], lt[j], ot[j]);
  }
#pragma unroll
  for (int x = 0; x < PER; ++x) s_red[w][x * 64 + lane] = acc[x];
  if (lane == 0) {
    s_red[w][D] = mw;
    s_red[w][D + 1] = lw;
  }
  __syncthreads();
  if (w != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int y = 0; y < kCombWaves; ++y) M = fmaxf(M, s_red[y][D]);
  float sy[kCombWaves], Lt = 0.0f;
#pragma unroll
  for (int y = 0; y < kCombWaves; ++y) {
    const float m = s_red[y][D];
    sy[y] = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    Lt += s_red[y][D + 1] * sy[y];
  }
  const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
  T* op = (T*)a.o + (long long)bq * D;
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    float v = 0.0f;
#pragma unroll
    for (int y = 0; y < kCombWaves; ++y) v += s_red[y][x * 64 + lane] * sy[y];
    op[x * 64 + lane] = (T)(v * inv);
  }
  if (lane == 0) a.lse[bq] = (M + log2f(Lt)) * kLn2;
}

template <typename T, int D, int BLK>
hipError_t launch_attn(const DecArgs& a, int B, hipStream_t st) {
  if (std::is_same<T, __bf16>::value && D == kMD && BLK == kMB && a.G <= 32) {
    hipLaunchKernelGGL(decode_attn_mfma_kernel, dim3((unsigned)(B * a.Hkv), (unsigned)a.T), dim3(64),
                       0, st, a);
  } else {
    const size_t lds = attn_lds<T, D, BLK>(a.G);
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute((const void*)&decode_attn_kernel<T, D, BLK>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_attn_kernel<T, D, BLK>), dim3((unsigned)(B * a.Hkv), (unsigned)a.T),
                       dim3(kAttnThreads), lds, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(B * a.Hq)), dim3(64 * kCombWaves),
                     0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attn_d(const DecArgs& a, int B, int blk, hipStream_t st) {
  if (blk == 16) return launch_attn<T, D, 16>(a, B, st);
  if (blk == 32) return launch_attn<T, D, 32>(a, B, st);
  return launch_attn<T, D, 64>(a, B, st);
}

}  // namespace

// ---------------------------------------------------------------------------
// fixed scratch of the allocation-free decode entry point
// ---------------------------------------------------------------------------
// The tile partials of sas_decode_attn_noalloc live in this array instead of
// a caller workspace.  Each device holds its own copy (from the library's
// code-object load until the process ends).  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is looked
// up once per device with hipGetSymbolAddress and only that address is
// handed to kernels.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {   // first use on this device (it is current)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t decode_attn_lds_bytes(const DecodeShape& s) {
  const size_t el = s.fp32 ? 4 : 2;
  return 2 * (size_t)s.blk * s.D * el + sizeof(float) * ((size_t)s.G * s.D + (size_t)s.G * s.blk);
}

hipError_t launch_decode_select(const DecodeShape& s, const float* scores, const int32_t* seq_lens,
                                float* tau, int32_t* sel_idx, int32_t* sel_cnt, int32_t* d_status,
                                hipStream_t st) {
  // 256 threads up to 1024 blocks, else 1024; KPT = keys per thread, a power of two
  const int nthr = s.cmax > 1024 ? kSelMaxThreads : 256;
  int kpt = 1;
  while (kpt * nthr < s.cmax) kpt *= 2;
  if (kpt > 16) return hipErrorInvalidValue;   // rows of at most 16384 blocks
  void (*kern)(const float*, const int32_t*, float*, int32_t*, int32_t*, int32_t*, int, int, int,
               int, int) = kpt == 1   ? decode_select_kernel<1>
                           : kpt == 2 ? decode_select_kernel<2>
                           : kpt == 4 ? decode_select_kernel<4>
                           : kpt == 8 ? decode_select_kernel<8>
                                      : decode_select_kernel<16>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(s.B * s.Hkv)), dim3(nthr), 0, st, scores, seq_lens,
                     tau, sel_idx, sel_cnt, d_status, s.Hkv, s.cmax, s.blk, s.K, s.cap);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const DecodeShape& s, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* sel_idx,
                              const int32_t* sel_cnt, void* o, float* lse, float* part,
                              int32_t* d_status, hipStream_t st) {
  DecArgs a{};
  a.q = q; a.kp = k_pool; a.vp = v_pool; a.bt = block_table; a.seq_lens = seq_lens;
  a.sel_idx = sel_idx; a.sel_cnt = sel_cnt; a.o = o; a.lse = lse; a.part = part;
  a.d_status = d_status;
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.G; a.cmax = s.cmax; a.pool = s.pool; a.cap = s.cap;
  a.T = s.cap + 1;
  a.c2 = s.scale * kLog2e;
  if (s.fp32) {
    return s.D == 64 ? launch_attn_d<float, 64>(a, s.B, s.blk, st)
                     : launch_attn_d<float, 128>(a, s.B, s.blk, st);
  }
  return s.D == 64 ? launch_attn_d<__bf16, 64>(a, s.B, s.blk, st)
                   : launch_attn_d<__bf16, 128>(a, s.B, s.blk, st);
}

}  // namespace sas
